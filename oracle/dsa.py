"""DSA sparse decode: indexer scores, top-k token selection, MLA decode over the selected slots.

Test infrastructure only (see the package docstring).

Sources:
* "vLLM KV Cache Layout 可视化", section on two caches sharing one block table: DeepSeek's sparse
  attention keeps, next to the MLA cache, an indexer cache in which the lightning indexer stores one
  index key per token (128 B FP8 key + 4 B FP32 scale), used to pick a sparse top-k set of tokens;
  both caches follow the same token sequence and share one block table.
* "deep dive into vLLM 05", §3.3: MLA attends in latent space (oracle.attention.mla_decode).
* "vLLM KV Cache Layout 可视化", section "kernel 那一侧": a slot is block * block_size + position.

Readings (the pages name the indexer and the top-k selection but give neither formula; the
scoring below is the published lightning indexer of DeepSeek's sparse attention):
* A decode token carries H index queries q_j (128 bf16 values each) and H float32 head weights w_j.
  Cached token t has the dequantized index key k_t = codes_t * scale_t. Its index score is
      I_t = sum_j w_j * max(q_j . k_t, 0).
* The selection keeps the top_k tokens of highest score; among equal scores the earlier position
  wins. With top_k >= the context every token is kept. Selected positions are listed in ascending
  order, and each is handed to the attention as its slot through the block table.
* The sparse decode is the MLA decode over the selected slots only (one softmax over them). A slot
  outside [0, num_blocks * block_size) contributes nothing; no valid slot gives an output of 0.
"""

from __future__ import annotations

import numpy as np

from .attention import gather_rows, mla_parse_rows, MLA_LATENT
from .numerics import bf16_bits_to_f64, e4m3_bytes_to_f64, f32le_bytes_to_f64
from .paging import CacheView, address, slot_of, split_slot

INDEX_DIM = 128
INDEX_ROW = 132


def index_keys(rows: np.ndarray) -> np.ndarray:
    """Indexer rows uint8 [n, 132] -> dequantized keys float64 [n, 128] (code times the row's scale)."""
    rows = np.asarray(rows, dtype=np.uint8)
    codes = e4m3_bytes_to_f64(rows[:, :INDEX_DIM])
    scale = f32le_bytes_to_f64(rows[:, INDEX_DIM:INDEX_ROW])   # [n, 1]
    return codes * scale


def index_scores_of_rows(q_bits, weights, rows: np.ndarray) -> np.ndarray:
    """I_t = sum_j w_j max(q_j . k_t, 0) for the given indexer rows. q [H, 128] bf16 bits, w [H] float32."""
    q = bf16_bits_to_f64(np.asarray(q_bits, dtype=np.uint16))            # [H, 128]
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)          # [H]
    logits = index_keys(rows) @ q.T                                       # [n, H]
    return np.maximum(logits, 0.0) @ w


def indexer_scores(q_bits, weights, image: np.ndarray, view: CacheView, layer: int, table_row, num_tokens: int,
                   block_size: int) -> np.ndarray:
    """Index scores of positions 0..num_tokens-1 of one sequence, read through its block table."""
    rows = gather_rows(image, view, layer, table_row, num_tokens, block_size)
    return index_scores_of_rows(q_bits, weights, rows)


def topk_positions(scores, top_k: int) -> np.ndarray:
    """The top_k highest scores' positions (earlier position first among equal scores), ascending."""
    n = len(scores)
    if top_k >= n:
        return np.arange(n, dtype=np.int64)
    ranked = sorted(range(n), key=lambda t: (-float(scores[t]), t))
    return np.sort(np.array(ranked[:top_k], dtype=np.int64))


def slots_of_positions(table_row, positions, block_size: int) -> np.ndarray:
    """Slot of each position through the sequence's block table."""
    return np.array([slot_of(table_row, int(t), block_size) for t in positions], dtype=np.int64)


def sparse_mla_decode(q_bits, image: np.ndarray, view: CacheView, layer: int, slot_lists, block_size: int,
                      num_blocks: int, scale: float, select=None) -> np.ndarray:
    """MLA decode of sequence b over the rows at slot_lists[b]. q [B, Hq, 576] bf16 bits -> float64 [B, Hq, 512].

    s_t = scale * (q_lat . c_t + q_rope . r_t) over the valid selected slots t, out = sum_t p_t c_t.
    """
    q = bf16_bits_to_f64(np.asarray(q_bits))
    B, Hq, _ = q.shape
    out = np.zeros((B, Hq, MLA_LATENT)) if select is None else np.full((B, Hq, MLA_LATENT), np.nan)
    for b in (range(B) if select is None else select):
        slots = [int(s) for s in slot_lists[b] if 0 <= int(s) < num_blocks * block_size]
        if not slots:
            out[b] = 0.0
            continue
        rows = np.empty((len(slots), view.row_bytes), dtype=np.uint8)
        for i, s in enumerate(slots):
            blk, pos = split_slot(s, block_size)
            a = address(view, layer, blk, pos)
            rows[i] = image[a:a + view.row_bytes]
        latent, rope = mla_parse_rows(rows)
        s_t = scale * (q[b, :, :MLA_LATENT] @ latent.T + q[b, :, MLA_LATENT:] @ rope.T)   # [Hq, n]
        p = np.exp(s_t - s_t.max(axis=1, keepdims=True))
        out[b] = (p @ latent) / p.sum(axis=1, keepdims=True)
    return out

"""Attention over a block-paged KV cache, in float64, by definition.

What is computed: for each query vector q and the rows it may see,
out = softmax(scale * K q) V, with one whole-row softmax in float64. This is
the same formula whether the rows are read contiguously or block by block.

Sources:
* "deep dive into vLLM 05", §2 (read path): for each block in the request's
  block table, take that physical block's K and V, score the query against
  K, then softmax the scores and weight V. The kernel sees only the table.
* "KV Cache 与推理服务内存管理", paged_attention pseudocode: look up the
  physical id of every logical block, read K and V, accumulate.
* "vLLM 技术内幕", §2.1: keys are read block by block and values are
  accumulated per block. The online and partitioned forms are exact
  rearrangements of the whole-row softmax used here.
* "deep dive into vLLM 05", §3.2: grouped queries. Consecutive query heads
  share one K/V head, so head h reads KV head h // (Hq / Hkv).
* "deep dive into vLLM 05", §3.3: MLA stores only the latent and attends in
  latent space once W_uk is folded into the query.
* "vLLM KV Cache Layout 可视化", section on two caches sharing one block
  table: an MLA row is 512 B FP8 latent + 16 B scale + 128 B BF16 RoPE.
* "vLLM 技术内幕", §3.2: a long prompt is cut into chunks, and each chunk
  attends causally to what is already cached.

Readings where the pages are silent:
* The score accumulation is written as ``scores += Q @ K_block^T``. It is
  read as concatenating each block's scores along the token axis.
* The caller writes the current token before attending, so a context length
  includes it.
* A context of length 0 gives an output of 0.
* MLA byte order: [0, 512) e4m3 latent; [512, 528) four float32 scales,
  scale k covering latent values [128k, 128k + 128); [528, 656) 64 bf16
  RoPE values; little-endian.
* MLA scores use [latent | rope] (576 dims). The value is the dequantized
  512-dim latent only.
* FP8 dense caches ("deep dive into vLLM 05" §3.4: quantize on write,
  dequantize on read, FP8 the safest format): one OCP E4M3 byte per value and
  one float32 scale per cache (K and V each); the value is code * scale. The
  query and output stay bf16.
"""

from __future__ import annotations

import numpy as np

from .numerics import bits_to_f64, bf16_bits_to_f64, e4m3_bytes_to_f64, f32le_bytes_to_f64, u16le_bytes
from .paging import CacheView, address


# --------------------------------------------------------------------------
# Gather through the block table
# --------------------------------------------------------------------------

def gather_rows(image: np.ndarray, view: CacheView, layer: int, table_row, num_tokens: int,
                block_size: int) -> np.ndarray:
    """Rows of tokens 0..num_tokens-1 in logical order, each read at its view address. uint8 [n, row]."""
    n = int(num_tokens)
    out = np.empty((n, view.row_bytes), dtype=np.uint8)
    for j in range(-(-n // block_size)):
        phys = int(table_row[j])
        count = min(block_size, n - j * block_size)
        start = address(view, layer, phys, 0)
        page = image[start:start + count * view.row_bytes]
        out[j * block_size:j * block_size + count] = page.reshape(count, view.row_bytes)
    return out


def dense_heads(rows: np.ndarray, dtype: str, num_kv_heads: int, head_dim: int, scale: float = 1.0) -> np.ndarray:
    """Decode dense NHD rows into float64 [n, Hkv, D].

    dtype "f16" / "bf16": 16-bit values. dtype "e4m3": one OCP E4M3 byte per value, times the cache's
    float32 ``scale`` (dequantize-on-read, "deep dive into vLLM 05" §3.4).
    """
    if dtype == "e4m3":
        codes = rows[:, :num_kv_heads * head_dim]
        return (e4m3_bytes_to_f64(codes) * float(scale)).reshape(len(rows), num_kv_heads, head_dim)
    words = u16le_bytes(rows[:, :num_kv_heads * head_dim * 2])
    return bits_to_f64(words, dtype).reshape(len(rows), num_kv_heads, head_dim)


def softmax_attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query vector, whole-row, float64."""
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = scale * (K @ q)
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


# --------------------------------------------------------------------------
# Dense decode: one query token per sequence
# --------------------------------------------------------------------------

def paged_decode(q_bits, dtype: str, k_image: np.ndarray, k_view: CacheView, v_image: np.ndarray,
                 v_view: CacheView, layer: int, block_tables, context_lens, block_size: int,
                 num_kv_heads: int, head_dim: int, scale: float, select=None, kv_dtype: str | None = None,
                 k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Paged decode. q [B, Hq, D] stored bits of type ``dtype``. Returns float64 [B, Hq, D].

    ``select`` is an optional list of (seq, q_head) pairs; only those outputs
    are computed and the rest are NaN. ``kv_dtype`` (default: ``dtype``) is the
    cache's type; for "e4m3" the K and V values are the codes times ``k_scale``
    and ``v_scale``.
    """
    kv_dtype = kv_dtype or dtype
    q = bits_to_f64(q_bits, dtype)
    B, Hq, D = q.shape
    g = Hq // num_kv_heads
    out = np.full((B, Hq, D), np.nan) if select is not None else np.zeros((B, Hq, D))
    want = {}
    for b, h in (select if select is not None else [(b, h) for b in range(B) for h in range(Hq)]):
        want.setdefault(int(b), []).append(int(h))
    for b, heads in want.items():
        n = int(context_lens[b])
        K = dense_heads(gather_rows(k_image, k_view, layer, block_tables[b], n, block_size), kv_dtype,
                        num_kv_heads, head_dim, k_scale)
        V = dense_heads(gather_rows(v_image, v_view, layer, block_tables[b], n, block_size), kv_dtype,
                        num_kv_heads, head_dim, v_scale)
        for h in heads:
            kvh = h // g
            out[b, h] = softmax_attend(q[b, h], K[:, kvh, :], V[:, kvh, :], scale)
    return out


# --------------------------------------------------------------------------
# Causal chunk over paged context (varlen; decodes are chunks of length 1)
# --------------------------------------------------------------------------

def chunk_prefill(q_bits, dtype: str, k_image: np.ndarray, k_view: CacheView, v_image: np.ndarray,
                  v_view: CacheView, layer: int, block_tables, seq_lens, query_start_loc,
                  block_size: int, num_kv_heads: int, head_dim: int, scale: float,
                  select_rows=None) -> np.ndarray:
    """Query i of sequence b sits at absolute position a = seq_len - qlen + i and sees tokens [0, a].

    q [total_q, Hq, D] stored bits. Returns float64 [total_q, Hq, D]. With
    ``select_rows`` (a set of query-row indices), only those rows are
    computed and the others are NaN.
    """
    q = bits_to_f64(q_bits, dtype)
    T, Hq, D = q.shape
    g = Hq // num_kv_heads
    out = np.zeros((T, Hq, D)) if select_rows is None else np.full((T, Hq, D), np.nan)
    for b in range(len(seq_lens)):
        q0, q1 = int(query_start_loc[b]), int(query_start_loc[b + 1])
        rows = [r for r in range(q0, q1) if select_rows is None or r in select_rows]
        if not rows:
            continue
        n, qlen = int(seq_lens[b]), q1 - q0
        K = dense_heads(gather_rows(k_image, k_view, layer, block_tables[b], n, block_size), dtype,
                        num_kv_heads, head_dim)
        V = dense_heads(gather_rows(v_image, v_view, layer, block_tables[b], n, block_size), dtype,
                        num_kv_heads, head_dim)
        for r in rows:
            a = n - qlen + (r - q0)          # absolute position of this query token
            for h in range(Hq):
                kvh = h // g
                out[r, h] = softmax_attend(q[r, h], K[:a + 1, kvh, :], V[:a + 1, kvh, :], scale)
    return out


# --------------------------------------------------------------------------
# MLA latent decode over packed 656-byte rows
# --------------------------------------------------------------------------

MLA_LATENT, MLA_GROUP, MLA_ROPE = 512, 128, 64


def mla_parse_rows(rows: np.ndarray):
    """[n, 656] bytes -> (latent float64 [n, 512] already scaled, rope float64 [n, 64])."""
    rows = np.asarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    raw = e4m3_bytes_to_f64(rows[:, :MLA_LATENT])                          # [n, 512]
    scales = f32le_bytes_to_f64(rows[:, MLA_LATENT:MLA_LATENT + 16])        # [n, 4]
    latent = raw * np.repeat(scales, MLA_GROUP, axis=1)                     # element j uses scale j // 128
    rope = bf16_bits_to_f64(u16le_bytes(rows[:, MLA_LATENT + 16:MLA_LATENT + 16 + 2 * MLA_ROPE]))
    return latent, rope.reshape(n, MLA_ROPE)


def mla_decode(q_bits, image: np.ndarray, view: CacheView, layer: int, block_tables, context_lens,
               block_size: int, scale: float, select=None) -> np.ndarray:
    """MLA decode. q [B, Hq, 576] bf16 bits (latent part first, then rope). Returns float64 [B, Hq, 512].

    s_t = scale * (q_lat . c_t + q_rope . r_t), and out = sum_t p_t c_t, with
    softmax weights p. ``select`` is an optional list of sequence indices.
    """
    q = bf16_bits_to_f64(q_bits)
    B, Hq, _ = q.shape
    out = np.zeros((B, Hq, MLA_LATENT)) if select is None else np.full((B, Hq, MLA_LATENT), np.nan)
    for b in (range(B) if select is None else select):
        n = int(context_lens[b])
        if n == 0:
            out[b] = 0.0
            continue
        latent, rope = mla_parse_rows(gather_rows(image, view, layer, block_tables[b], n, block_size))
        s = scale * (q[b, :, :MLA_LATENT] @ latent.T + q[b, :, MLA_LATENT:] @ rope.T)   # [Hq, n]
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[b] = (p @ latent) / p.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# Split-context partitions and their log-sum-exp merge
# --------------------------------------------------------------------------

def partition_partials(scores: np.ndarray, V: np.ndarray, partition_tokens: int):
    """Per partition p of tokens [p*P, (p+1)*P): m_p = max s, l_p = sum e^(s-m_p), acc_p = sum e^(s-m_p) v."""
    ms, ls, accs = [], [], []
    for start in range(0, len(scores), partition_tokens):
        s = scores[start:start + partition_tokens]
        m = s.max()
        e = np.exp(s - m)
        ms.append(m)
        ls.append(e.sum())
        accs.append(e @ V[start:start + partition_tokens])
    return np.array(ms), np.array(ls), np.array(accs)


def merge_partitions(ms: np.ndarray, ls: np.ndarray, accs: np.ndarray) -> np.ndarray:
    """out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p, with M = max_p m_p."""
    M = ms.max()
    w = np.exp(ms - M)
    return (w @ accs) / (w @ ls)

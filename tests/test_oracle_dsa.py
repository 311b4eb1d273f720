"""Pins for oracle.dsa: indexer scores, top-k selection, sparse MLA decode.

The index keys are checked against torch's float8_e4m3fn decoding (a library conversion). Scores
are checked against closed forms (one-hot keys, where each score is a hand-computed sum of clipped
query entries) and against brute force in plain Python loops on a tiny case; the selection against
NumPy's lexsort on tie-heavy scores; the sparse decode against the dense MLA decode (itself pinned
against torch's attention) over a cache that holds exactly the selected rows, and against the
closed form of a single selected row. "vLLM KV Cache Layout 可视化" (section "kernel 那一侧") fixes the
slot of token 130 at block size 64 with block_table[2] = 5: 322.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import dsa as D
from oracle import paging as P
from oracle import quant as Q
import workloads


def bf16_bits(x) -> np.ndarray:
    return torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def index_row(codes, scale) -> np.ndarray:
    r = np.zeros(132, dtype=np.uint8)
    r[:128] = codes
    r[128:132] = np.array([scale], dtype="<f4").view(np.uint8)
    return r


def test_index_keys_match_torch_fp8_decoding():
    rows = workloads.draw_indexer_rows(3, 50).numpy()
    rows[0, 128:132] = np.array([0.0], dtype="<f4").view(np.uint8)      # zero scale
    got = D.index_keys(rows)
    t = torch.from_numpy(rows)
    codes = t[:, :128].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    scale = t[:, 128:132].contiguous().view(torch.float32).to(torch.float64)
    np.testing.assert_array_equal(got, (codes * scale).numpy())


def test_one_hot_keys_closed_form():
    # Token t's key is one code of value 1.0 (e4m3 0x38) at dim d_t, times scale s_t, so its score is
    # s_t * sum_j w_j * max(q_j[d_t], 0). Query entries and weights are small exact binary fractions.
    H = 3
    w = np.array([0.5, -2.0, 1.25], dtype=np.float32)
    q = np.zeros((H, 128), dtype=np.float32)
    q[:, 0] = [1.0, -2.0, 3.0]
    q[:, 5] = [-1.0, -0.5, -4.0]
    q[:, 7] = [2.0, 0.25, 0.0]
    q[:, 127] = [0.0, 1.5, -1.0]
    dims = [0, 5, 7, 127, 9]
    scales = [1.0, 2.0, 0.5, 4.0, 3.0]
    rows = []
    for d, s in zip(dims, scales):
        c = np.zeros(128, dtype=np.uint8)
        c[d] = 0x38
        rows.append(index_row(c, s))
    got = D.index_scores_of_rows(bf16_bits(q), w, np.stack(rows))
    # dim 0: 0.5*1 + (-2)*0 + 1.25*3 = 4.25;  dim 5: every entry clipped -> 0
    # dim 7: 0.5*2 + (-2)*0.25 + 0 = 0.5, times 0.5;  dim 127: -2*1.5 = -3, times 4;  dim 9: 0
    np.testing.assert_array_equal(got, [4.25, 0.0, 0.25, -12.0, 0.0])


def test_scores_brute_force_tiny():
    rng = np.random.default_rng(4)
    H, n = 4, 6
    q = bf16_bits(rng.standard_normal((H, 128)))
    w = rng.standard_normal(H).astype(np.float32)
    rows = workloads.draw_indexer_rows(11, n).numpy()
    got = D.index_scores_of_rows(q, w, rows)
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(torch.float64).tolist()
    for t in range(n):
        codes = torch.from_numpy(rows[t, :128].copy()).view(torch.float8_e4m3fn).to(torch.float64).tolist()
        s = float(np.frombuffer(rows[t, 128:132].tobytes(), dtype="<f4")[0])
        total = 0.0
        for j in range(H):
            dot = 0.0
            for d in range(128):
                dot += qf[j][d] * codes[d] * s
            total += float(w[j]) * (dot if dot > 0 else 0.0)
        assert got[t] == pytest.approx(total, rel=1e-12, abs=1e-12)


def test_scores_read_through_the_block_table_are_placement_invariant():
    # The same logical rows under two different block tables (block-outer dual cache, layer 1).
    rng = np.random.Generator(np.random.PCG64(8))
    bs, nb, n = 64, 10, 300
    views, block = P.block_outer_views([("mla", 656, 2), ("indexer", 132, 2)], bs)
    rows = workloads.draw_indexer_rows(21, n).numpy()
    q = bf16_bits(rng.standard_normal((8, 128)))
    w = rng.standard_normal(8).astype(np.float32)
    ref = D.index_scores_of_rows(q, w, rows)
    for seed in (1, 2):
        table, _ = workloads.allocate_block_tables(np.random.Generator(np.random.PCG64(seed)), [n], bs, nb)
        image = np.zeros(nb * block, dtype=np.uint8)
        for t in range(n):
            a = P.address(views["indexer"], 1, table[0][t // bs], t % bs)
            image[a:a + 132] = rows[t]
        got = D.indexer_scores(q, w, image, views["indexer"], 1, table[0], n, bs)
        np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("n,k", [(50, 7), (300, 64), (64, 64), (10, 20), (1, 1), (200, 1)])
def test_topk_matches_lexsort(n, k):
    rng = np.random.default_rng(n * 31 + k)
    scores = rng.integers(-4, 5, size=n).astype(np.float64) * 0.5       # many ties
    got = D.topk_positions(scores, k)
    order = np.lexsort((np.arange(n), -scores))                        # by score desc, then position
    np.testing.assert_array_equal(got, np.sort(order[:min(k, n)]))


def test_topk_ties_prefer_earlier_positions():
    scores = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.0])
    assert D.topk_positions(scores, 1).tolist() == [1]
    assert D.topk_positions(scores, 3).tolist() == [1, 2, 3]
    assert D.topk_positions(scores, 4).tolist() == [1, 2, 3, 4]
    assert D.topk_positions(np.zeros(5), 2).tolist() == [0, 1]


def test_slot_of_token_130_from_page():
    assert D.slots_of_positions([7, 1, 5], [130], 64).tolist() == [322]


def _mla_case(rng, ctx, bs, nb, hq):
    views, block = P.block_outer_views([("mla", 656, 2), ("indexer", 132, 2)], bs)
    tables, _ = workloads.allocate_block_tables(rng, ctx, bs, nb)
    image = np.zeros(nb * block, dtype=np.uint8)
    rows = [workloads.draw_mla_rows(500 + b, n).numpy() for b, n in enumerate(ctx)]
    for b, r in enumerate(rows):
        for t in range(len(r)):
            a = P.address(views["mla"], 1, tables[b][t // bs], t % bs)
            image[a:a + 656] = r[t]
    q = bf16_bits(rng.standard_normal((len(ctx), hq, 576)))
    return image, views["mla"], tables, rows, q


def test_sparse_decode_over_every_position_is_the_dense_decode():
    rng = np.random.Generator(np.random.PCG64(12))
    bs, nb, ctx = 64, 12, [1, 90, 200]
    image, view, tables, _, q = _mla_case(rng, ctx, bs, nb, 16)
    slots = [D.slots_of_positions(tables[b], range(n), bs) for b, n in enumerate(ctx)]
    got = D.sparse_mla_decode(q, image, view, 1, slots, bs, nb, 0.05)
    ref = A.mla_decode(q, image, view, 1, tables, ctx, bs, 0.05)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_sparse_decode_equals_dense_decode_over_only_the_selected_rows():
    rng = np.random.Generator(np.random.PCG64(13))
    bs, nb, ctx = 64, 12, [150, 260]
    image, view, tables, rows, q = _mla_case(rng, ctx, bs, nb, 16)
    picks = [np.sort(rng.choice(n, size=k, replace=False)) for n, k in zip(ctx, (40, 77))]
    slots = [D.slots_of_positions(tables[b], picks[b], bs) for b in range(2)]
    got = D.sparse_mla_decode(q, image, view, 1, slots, bs, nb, 0.05)
    # A fresh cache holding exactly the selected rows, contiguous from block 0 (layer 0).
    sub_rows = [rows[b][picks[b]] for b in range(2)]
    sub_tables = np.array([[0, 1], [2, 3]], dtype=np.int32)
    sub_image = np.zeros(4 * bs * 656, dtype=np.uint8)
    sub_view = P.CacheView(0, 0, bs * 656, 656)
    for b in range(2):
        for t in range(len(sub_rows[b])):
            a = P.address(sub_view, 0, sub_tables[b][t // bs], t % bs)
            sub_image[a:a + 656] = sub_rows[b][t]
    ref = A.mla_decode(q, sub_image, sub_view, 0, sub_tables, [40, 77], bs, 0.05)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # The order of the slots does not matter; invalid slots contribute nothing.
    shuffled = [np.concatenate([rng.permutation(s), [-1, nb * bs, 10 ** 9]]) for s in slots]
    np.testing.assert_allclose(D.sparse_mla_decode(q, image, view, 1, shuffled, bs, nb, 0.05), got,
                               rtol=0, atol=1e-12)


def test_single_selected_row_returns_its_latent():
    rng = np.random.Generator(np.random.PCG64(14))
    bs, nb, ctx = 64, 6, [70]
    image, view, tables, rows, q = _mla_case(rng, ctx, bs, nb, 16)
    slot = D.slots_of_positions(tables[0], [33], bs)
    got = D.sparse_mla_decode(q, image, view, 1, [slot], bs, nb, 0.05)
    r = torch.from_numpy(rows[0][33:34])
    lat = r[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64).reshape(4, 128)
    sc = r[:, 512:528].contiguous().view(torch.float32).to(torch.float64).reshape(4, 1)
    np.testing.assert_array_equal(got[0], np.broadcast_to((lat * sc).reshape(512).numpy(), (16, 512)))
    assert not D.sparse_mla_decode(q, image, view, 1, [[-1, -5]], bs, nb, 0.05).any()

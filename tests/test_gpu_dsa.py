"""GPU parity of the DSA sparse path: indexer scores, top-k selection, sparse MLA decode.

The dual cache is written by pa_reshape_and_cache and checked byte for byte against the oracle's
image, as in the MLA tests (unwritten bytes stay 0xFF: NaN as e4m3 codes and as float32 scales, so
a stray read shows). Then:

* scores: each context position's score against the oracle's float64 score, within
  2^-14 * M_t, where M_t = scale_t * sum_j |w_j| * sum_d |q_jd * code_td| bounds every term of the
  sum (fp32 accumulation of exact bf16 products over 128 dims and up to 64 heads);
* selection: bit-exact against the oracle's top-k applied to the kernel's own fp32 scores (the
  decision taken in the kernel's precision), and valid against the oracle's scores: no unselected
  score exceeds a selected one by more than their tolerances;
* slots: bit-exact against the block-table slot of each selected position;
* sparse decode: against the oracle's MLA decode over the same slots, within the 3e-2 MLA bound.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
import workloads
from oracle import dsa as D
from oracle import numerics as N
from oracle import paging as P
from helpers import MLA_ATOL, MLA_RTOL, assert_close, bits_np, dev, image_of
from test_gpu_mla import mla_desc, populate, to_pa, views

pytestmark = pytest.mark.gpu

SCORE_REL = 2.0 ** -14
SENTINEL = 0x7FFFFFFF


def magnitude(q_bits, w, rows):
    """M_t = |scale_t| * sum_j |w_j| * sum_d |q_jd| |code_td| for indexer rows [n, 132]."""
    q = np.abs(N.bf16_bits_to_f64(np.asarray(q_bits, dtype=np.uint16)))
    codes = np.abs(N.e4m3_bytes_to_f64(rows[:, :128]))
    sc = np.abs(N.f32le_bytes_to_f64(rows[:, 128:132]))[:, 0]
    return sc * ((codes @ q.T) @ np.abs(np.asarray(w, dtype=np.float64)))


def run_topk(case, img, layer, top_k, q_index=None, weights=None, max_ctx=None):
    _, idx_v, _ = views(case.block_size)
    B = len(case.context_lens)
    max_ctx = max(1, int(case.context_lens.max())) if max_ctx is None else max_ctx
    q_index = case.q_index if q_index is None else q_index
    weights = case.index_weights if weights is None else weights
    scores = torch.full((B, max_ctx + 3), float("nan"), dtype=torch.float32, device="cuda")
    pos = torch.full((B, top_k), SENTINEL, dtype=torch.int32, device="cuda")
    slots = torch.full_like(pos, SENTINEL)
    lens = torch.full((B,), SENTINEL, dtype=torch.int32, device="cuda")
    pa.pa_indexer_topk(pos, slots, lens, scores, dev(q_index), dev(weights), img, to_pa(idx_v), layer,
                       dev(case.block_tables), dev(case.context_lens), max_ctx, case.block_size, case.num_blocks)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), pos.cpu().numpy(), slots.cpu().numpy(), lens.cpu().numpy()


def check_topk(case, host, layer, top_k, res, q_index=None, weights=None, seqs=None):
    """Scores against the oracle, selection exact on the kernel's scores and valid on the oracle's."""
    scores, pos, slots, lens = res
    _, idx_v, _ = views(case.block_size)
    q_index = bits_np(case.q_index if q_index is None else q_index)
    weights = (case.index_weights if weights is None else weights).cpu().numpy()
    bs = case.block_size
    for b in (range(len(case.context_lens)) if seqs is None else seqs):
        n = int(case.context_lens[b])
        k = min(n, top_k)
        assert lens[b] == k, (b, lens[b], k)
        g = scores[b, :n].astype(np.float64)
        assert np.isnan(scores[b, n:]).all(), f"seq {b}: scores written past the context"
        rows = np.stack([host[a:a + 132] for a in (P.address(idx_v, layer, case.block_tables[b][t // bs], t % bs)
                                                   for t in range(n))]) if n else np.zeros((0, 132), np.uint8)
        if n:
            want = D.index_scores_of_rows(q_index[b], weights[b], rows)
            tol = SCORE_REL * magnitude(q_index[b], weights[b], rows) + 1e-30
            err = np.abs(g - want)
            assert np.isfinite(g).all() and (err <= tol).all(), \
                f"seq {b}: score error {err.max():.3e} (bound at worst {tol[np.argmax(err - tol)]:.3e})"
        sel = D.topk_positions(g, top_k)
        assert np.array_equal(pos[b, :k], sel), f"seq {b}: selection differs from top-k of the kernel's scores"
        assert (pos[b, k:] == -1).all() and (slots[b, k:] == -1).all()
        assert np.array_equal(slots[b, :k], D.slots_of_positions(case.block_tables[b], sel, bs))
        if n > top_k:
            mask = np.zeros(n, dtype=bool)
            mask[sel] = True
            assert (want[mask] + tol[mask]).min() >= (want[~mask] - tol[~mask]).max(), f"seq {b}: invalid top-k"


def sparse_decode(case, img, layer, slots, counts, max_count, partition_size=0):
    desc = mla_desc(case, img, layer, partition_size)
    B = len(case.context_lens)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max(1, max_count))), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, case.num_q_heads, 512), -1, dtype=torch.int16, device="cuda")
    pa.pa_mla_sparse_decode(out, dev(case.q), img, dev(slots), dev(counts), max_count, case.scale, desc, ws)
    torch.cuda.synchronize()
    return out.view(torch.bfloat16).double().cpu().numpy()


def dsa_case(seed, ctx, hq, bs, index_heads=64):
    need = sum(P.blocks_needed(n, bs) for n in ctx)
    case = workloads.make_mla_case(seed=seed, context_lens=ctx, num_blocks=need + 3, num_q_heads=hq, block_size=bs)
    case.q_index, case.index_weights = workloads.draw_index_queries(seed + 1, len(ctx), index_heads)
    img, host = populate(case)
    assert np.array_equal(image_of(img), host), "dual-cache bytes differ from the oracle's reshape_and_cache"
    return case, img, host


# index heads, query heads, block size, contexts, top_k, decode partition (0: balanced)
SHAPES = [
    (64, 16, 64, [0, 1, 15, 16, 17, 100, 640, 1000], 64, 0),
    (16, 32, 16, [5, 300, 33, 2], 16, 64),
    (32, 64, 64, [2000, 1], 128, 0),
    (48, 16, 128, [700, 129, 0, 64], 100, 96),
    (64, 128, 64, [50, 60], 2048, 0),            # top_k above every context: everything selected
    (64, 16, 256, [1023, 1024, 1025], 512, 32),
]


@pytest.mark.parametrize("H,hq,bs,ctx,top_k,part", SHAPES)
def test_indexer_topk_and_sparse_decode(H, hq, bs, ctx, top_k, part):
    case, img, host = dsa_case(4000 + H + hq + bs, ctx, hq, bs, H)
    mla_v, _, _ = views(bs)
    for layer in (1, 0):
        res = run_topk(case, img, layer, top_k)
        check_topk(case, host, layer, top_k, res)
        _, _, slots, lens = res
        got = sparse_decode(case, img, layer, slots, lens, top_k, part)
        want = D.sparse_mla_decode(bits_np(case.q), host, mla_v, layer, [slots[b, :lens[b]] for b in range(len(ctx))],
                                   bs, case.num_blocks, case.scale)
        assert_close(got, want, MLA_ATOL, MLA_RTOL, f"sparse decode layer {layer}")


def test_ties_take_the_earliest_positions():
    # Five distinct indexer rows repeated over every position: scores tie exactly, in groups.
    ctx = [300, 77, 1000]
    case = workloads.make_mla_case(seed=4100, context_lens=ctx, num_blocks=sum(P.blocks_needed(n, 64) for n in ctx) + 2,
                                   num_q_heads=16)
    case.q_index, case.index_weights = workloads.draw_index_queries(4101, 3, 64)
    for layer in range(2):
        base = case.idx_rows[layer][:5].clone()
        case.idx_rows[layer] = base[torch.arange(len(case.idx_rows[layer])) % 5]
        case.step_idx_rows[layer] = base[torch.arange(3) % 5]
    img, host = populate(case)
    assert np.array_equal(image_of(img), host)
    res = run_topk(case, img, 1, 50)
    check_topk(case, host, 1, 50, res)
    # Zero head weights: every score is 0, so the first top_k positions are selected.
    zero = torch.zeros_like(case.index_weights)
    res = run_topk(case, img, 1, 64, weights=zero)
    check_topk(case, host, 1, 64, res, weights=zero)
    assert (res[0][:, :64][np.isfinite(res[0][:, :64])] == 0).all()
    assert np.array_equal(res[1][0, :64], np.arange(64))


def test_every_code_and_extreme_scales():
    # Indexer rows whose codes run through all 254 finite e4m3 values, with scales from 0 and a
    # subnormal float32 up to large values: the exact widening of every code and the scale product.
    ctx = [260, 40]
    case = workloads.make_mla_case(seed=4200, context_lens=ctx, num_blocks=8, num_q_heads=16)
    case.q_index, case.index_weights = workloads.draw_index_queries(4201, 2, 32)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    scales = np.array([1.0, 0.0, 2.0 ** -140, 3.5e-3, 7.0, 1.0e20], dtype=np.float32)
    for layer in range(2):
        rows = case.idx_rows[layer].numpy().copy()
        for t in range(len(rows)):
            rows[t, :128] = finite[(np.arange(128) + 37 * t) % len(finite)]
            rows[t, 128:132] = scales[t % len(scales):t % len(scales) + 1].view(np.uint8)
        case.idx_rows[layer] = torch.from_numpy(rows)
    img, host = populate(case)
    assert np.array_equal(image_of(img), host)
    for top_k in (7, 300):
        res = run_topk(case, img, 0, top_k)
        check_topk(case, host, 0, top_k, res)


def test_long_context_past_the_lds_cache():
    # 40000 scores do not fit the 32768-entry LDS copy: the selection passes re-read them from memory.
    ctx = [40000, 3000]
    case, img, host = dsa_case(4300, ctx, 16, 64, 16)
    res = run_topk(case, img, 1, 2048)
    check_topk(case, host, 1, 2048, res)


def test_sparse_decode_given_slots():
    # Hand-made slot lists: unsorted, duplicated, invalid (-1, past the pool), counts 0..100.
    ctx = [300, 200, 90, 40]
    case, img, host = dsa_case(4400, ctx, 64, 64)
    mla_v, _, _ = views()
    rng = np.random.default_rng(9)
    nslots = case.num_blocks * 64
    counts = np.array([100, 33, 0, 31], dtype=np.int32)
    stride = 128
    slots = np.full((4, stride), -1, dtype=np.int32)
    for b, c in enumerate(counts):
        picks = rng.integers(0, ctx[b], size=c)
        s = D.slots_of_positions(case.block_tables[b], picks, 64).astype(np.int32)
        if c > 10:
            s[3], s[7] = -1, nslots + 5      # invalid entries: no token
            s[9] = s[2]                      # a duplicated row counts twice
        slots[b, :c] = s
    for part in (0, 64):
        got = sparse_decode(case, img, 1, slots, counts, stride, part)
        want = D.sparse_mla_decode(bits_np(case.q), host, mla_v, 1, [slots[b, :counts[b]] for b in range(4)], 64,
                                   case.num_blocks, case.scale)
        assert_close(got, want, MLA_ATOL, MLA_RTOL, f"given slots P={part}")
    assert (got[2] == 0).all()               # no slot: output 0


def seq_rows(case, layer, which):
    """Generator rows of every sequence in position order (not read back from the device)."""
    pop = case.mla_rows[layer] if which == "mla" else case.idx_rows[layer]
    step = case.step_mla_rows[layer] if which == "mla" else case.step_idx_rows[layer]
    out, off = [], 0
    for b, n in enumerate(case.context_lens):
        n = int(n)
        m = max(n - 1, 0)
        rows = torch.cat([pop[off:off + m], step[b:b + 1]]) if n else pop[:0]
        off += m
        out.append(rows)
    return out


def test_full_size_dsa_sparse_sampled():
    """64 seqs, ctx U[1024, 8192], 64 index heads, top 2048, 128 query heads; layer 1."""
    case = workloads.make_mla_case(device="cuda")
    img, _ = populate(case, with_oracle=False)
    layer, top_k, bs = 1, case.top_k, case.block_size
    scores, pos, slots, lens = run_topk(case, img, layer, top_k)
    qi = bits_np(case.q_index)
    w = case.index_weights.cpu().numpy()
    idx_rows = seq_rows(case, layer, "idx")
    rng = np.random.default_rng(11)
    sampled = sorted(set(rng.choice(64, size=4, replace=False).tolist()) | {int(np.argmax(case.context_lens))})
    for b in range(64):
        n = int(case.context_lens[b])
        g = scores[b, :n].astype(np.float64)
        sel = D.topk_positions(g, top_k)
        assert lens[b] == min(n, top_k) and np.array_equal(pos[b, :lens[b]], sel), f"seq {b}"
        assert np.array_equal(slots[b, :lens[b]], D.slots_of_positions(case.block_tables[b], sel, bs))
        if b in sampled:
            rows = idx_rows[b].cpu().numpy()
            want = D.index_scores_of_rows(qi[b], w[b], rows)
            tol = SCORE_REL * magnitude(qi[b], w[b], rows) + 1e-30
            assert (np.abs(g - want) <= tol).all(), f"seq {b}: scores"
            mask = np.zeros(n, dtype=bool)
            mask[sel] = True
            assert (want[mask] + tol[mask]).min() >= (want[~mask] - tol[~mask]).max(), f"seq {b}: invalid top-k"
    mla_rows = seq_rows(case, layer, "mla")
    q_plain = case.q
    # The second pass scales the queries by 6 so each head's softmax over the 2048 selected rows
    # concentrates and the outputs reach |o| ~ 0.3-1, where the 3e-2 tolerance discriminates.
    for gain in (1.0, 6.0):
        case.q = q_plain if gain == 1.0 else (q_plain.view(torch.bfloat16).float() * gain).to(
            torch.bfloat16).view(torch.int16)
        got = sparse_decode(case, img, layer, slots, lens, top_k)
        assert np.isfinite(got).all()
        q = bits_np(case.q)
        for b in sampled:
            # A compact image of the sequence's rows in position order (block j = positions 64j..),
            # addressed by position: the oracle reads generator rows, not the device cache.
            n = int(case.context_lens[b])
            rows = mla_rows[b].cpu().numpy()
            nb = P.blocks_needed(n, bs)
            image = np.zeros(nb * bs * 656, dtype=np.uint8)
            image[:n * 656] = rows.reshape(-1)
            view = P.CacheView(0, 0, bs * 656, 656)
            want = D.sparse_mla_decode(q[b:b + 1], image, view, 0, [pos[b, :lens[b]]], bs, nb, case.scale)
            assert_close(got[b], want[0], MLA_ATOL, MLA_RTOL, f"gain {gain} seq {b} (ctx {n})")
            if gain != 1.0 and b == sampled[0]:
                # An all-zero output, or scores without RoPE, would fail this check.
                q_nr = q[b:b + 1].copy()
                q_nr[..., 512:] = 0
                want_nr = D.sparse_mla_decode(q_nr, image, view, 0, [pos[b, :lens[b]]], bs, nb, case.scale)
                bound = MLA_ATOL + MLA_RTOL * np.abs(want[0])
                assert (np.abs(want[0]) > bound).mean() > 0.9
                assert (np.abs(want_nr[0] - want[0]) > bound).mean() > 0.6


def test_many_sequences_and_uncached_block_ids():
    # 300 sequences (five 64-sequence passes of the sparse decode's unit search) with short and empty contexts,
    # and one 40,000-token sequence at block size 16, whose 2500 block ids exceed the selection
    # kernel's LDS copy (slots are then looked up in memory).
    rng = np.random.default_rng(21)
    ctx = rng.integers(0, 90, size=300).tolist()
    case, img, host = dsa_case(4500, ctx, 16, 16, 16)
    mla_v, _, _ = views(16)
    res = run_topk(case, img, 1, 24)
    check_topk(case, host, 1, 24, res)
    _, _, slots, lens = res
    got = sparse_decode(case, img, 1, slots, lens, 24)
    want = D.sparse_mla_decode(bits_np(case.q), host, mla_v, 1, [slots[b, :lens[b]] for b in range(len(ctx))], 16,
                               case.num_blocks, case.scale)
    assert_close(got, want, MLA_ATOL, MLA_RTOL, "300 sequences")
    long_case, long_img, long_host = dsa_case(4600, [40000], 16, 16, 16)
    res = run_topk(long_case, long_img, 0, 1000)
    check_topk(long_case, long_host, 0, 1000, res)

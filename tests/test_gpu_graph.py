"""The hot path under HIP graph capture: every entry point launches its kernels on the caller's
stream, allocates nothing and records no memset, so a serving loop can capture a decode step once
and replay it.

Each case runs one step eagerly, captures the same step (torch.cuda.graph) and replays it three
times; before every replay the output is overwritten with 0xFFFF (NaN in fp16 and bf16), and
between replays the eager step runs again, so the replays are checked against the program's own
eager work. Every replay must give the eager output bit for bit: the kernels are the same and
their results do not depend on timing. The eager outputs themselves are what the parity tests of
each path check against the oracle; here they are also spot-checked to be finite.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
import workloads
from oracle import paging as P
from helpers import dev, poison_tails
import test_gpu_dsa as DSA
import test_gpu_fp8 as F8
import test_gpu_mla as M

pytestmark = pytest.mark.gpu

REPLAYS = 3


def replays_match_eager(step, outs):
    """Capture `step` (which writes every tensor in `outs`) and check REPLAYS replays against it."""
    step()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"replay {i}: output {k} differs from the eager step"
        step()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o, r), f"eager step after replay {i}: output {k} differs"
    return refs


def finite_bf16_or_f16(t, dtype):
    x = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).float()
    return bool(torch.isfinite(x).all())


# dtype, Hq, Hkv, contexts, partition (a few partitions per row, so the merge kernel runs too)
DENSE = [
    ("f16", 8, 8, [1, 17, 130, 300, 1000], 64),      # vector kernel
    ("bf16", 32, 8, [2, 33, 500, 1200], 128),        # matrix-core kernel (groups of 4)
]


@pytest.mark.parametrize("dtype,Hq,Hkv,ctx,part", DENSE)
def test_graph_write_and_decode(dtype, Hq, Hkv, ctx, part):
    need = sum(P.blocks_needed(n, 16) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=7100 + Hq, context_lens=ctx, num_blocks=need + 3, num_q_heads=Hq,
                                     num_kv_heads=Hkv, dtype=dtype)
    kh, vh = case.k_pool.clone(), case.v_pool.clone()
    poison_tails(kh, case.block_tables, case.context_lens, 16, dtype)
    poison_tails(vh, case.block_tables, case.context_lens, 16, dtype)
    kd, vd = dev(kh), dev(vh)
    view = pa.dense_view(16, Hkv, 128)
    B, max_ctx = case.num_seqs, int(case.context_lens.max())
    desc = pa.dense_desc(dtype, Hq, Hkv, 128, 16, case.num_blocks, kd.numel() * 2, vd.numel() * 2, part)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, 128, dtype=torch.int16, device="cuda")
    q, bt, lens = dev(case.q), dev(case.block_tables), dev(case.context_lens)
    new_k, new_v, slots = dev(case.new_k), dev(case.new_v), dev(case.new_slots)

    def step():
        pa.pa_reshape_and_cache(new_k, slots, kd, view, 0, 16, case.num_blocks, v=new_v, v_cache=vd, v_view=view)
        pa.pa_decode(out, q, kd, vd, bt, lens, max_ctx, case.scale, desc, ws)

    ref, = replays_match_eager(step, [out])
    assert finite_bf16_or_f16(ref, dtype)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8)])
def test_graph_quantize_and_fp8_decode(Hq, Hkv):
    """FP8 cache: the step quantizes the new tokens on write, then decodes (vector and matrix-core kernels)."""
    ctx = [3, 90, 700, 1300]
    need = sum(P.blocks_needed(n, 16) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=7200 + Hq, context_lens=ctx, num_blocks=need + 3, num_q_heads=Hq,
                                     num_kv_heads=Hkv, dtype="bf16")
    k8, v8 = F8.quantize_pool(case)
    F8.poison(k8, v8, case)
    view8 = pa.dense_view(16, Hkv, 128, 1)
    B, max_ctx = case.num_seqs, int(case.context_lens.max())
    desc = pa.dense_desc("fp8", Hq, Hkv, 128, 16, case.num_blocks, k8.numel(), v8.numel(), 128,
                         k_scale=F8.K_SCALE, v_scale=F8.V_SCALE)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, 128, dtype=torch.int16, device="cuda")
    q, bt, lens = dev(case.q), dev(case.block_tables), dev(case.context_lens)
    new_k = dev(case.new_k).reshape(B, Hkv * 128)
    new_v = dev(case.new_v).reshape(B, Hkv * 128)
    slots = dev(case.new_slots)

    def step():
        pa.pa_quantize_and_cache(new_k, slots, k8, view8, 0, 16, case.num_blocks, F8.K_SCALE, v=new_v, v_cache=v8,
                                 v_view=view8, v_scale=F8.V_SCALE)
        pa.pa_decode(out, q, k8, v8, bt, lens, max_ctx, case.scale, desc, ws)

    ref, = replays_match_eager(step, [out])
    assert finite_bf16_or_f16(ref, "bf16")


def test_graph_mla_decode():
    """MLA latent decode with fixed work-group ranges of 64 tokens, so most sequences are merged."""
    ctx = [40, 300, 1, 900, 64]
    need = sum(P.blocks_needed(n, M.BS) for n in ctx)
    case = workloads.make_mla_case(seed=7300, context_lens=ctx, num_blocks=need + 1, num_q_heads=128)
    img, _ = M.populate(case, with_oracle=False)
    desc = M.mla_desc(case, img, 0, partition_size=64)
    B, max_ctx = len(ctx), max(ctx)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, 128, 512, dtype=torch.int16, device="cuda")
    q, bt, lens = dev(case.q), dev(case.block_tables), dev(case.context_lens)

    def step():
        pa.pa_decode(out, q, img, None, bt, lens, max_ctx, case.scale, desc, ws)

    ref, = replays_match_eager(step, [out])
    assert finite_bf16_or_f16(ref, "bf16")


def test_graph_dsa_sparse_step():
    """Indexer scores, top-k selection and the sparse MLA decode over the selection, as one step."""
    ctx = [5, 300, 1100, 64]
    top_k = 128
    case, img, _ = DSA.dsa_case(7400, ctx, 64, 64)
    _, idx_v, _ = M.views(64)
    B, max_ctx = len(ctx), max(ctx)
    scores = torch.empty((B, max_ctx), dtype=torch.float32, device="cuda")
    pos = torch.empty((B, top_k), dtype=torch.int32, device="cuda")
    slots = torch.empty_like(pos)
    counts = torch.empty((B,), dtype=torch.int32, device="cuda")
    desc = M.mla_desc(case, img, 1)
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, top_k)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, 64, 512, dtype=torch.int16, device="cuda")
    qi, w, q = dev(case.q_index), dev(case.index_weights), dev(case.q)
    bt, lens = dev(case.block_tables), dev(case.context_lens)

    def step():
        pa.pa_indexer_topk(pos, slots, counts, scores, qi, w, img, M.to_pa(idx_v), 1, bt, lens, max_ctx, 64,
                           case.num_blocks)
        pa.pa_mla_sparse_decode(out, q, img, slots, counts, top_k, case.scale, desc, ws)

    ref_pos, ref_slots, ref_counts, ref_out = replays_match_eager(step, [pos, slots, counts, out])
    assert np.array_equal(ref_counts.cpu().numpy(), np.minimum(ctx, top_k))
    assert finite_bf16_or_f16(ref_out, "bf16")


def test_graph_mixed_chunk_call():
    """One chunked-prefill call: chunk rows and decode rows (a partition merge for the long decode)."""
    seq_lens, query_lens = [700, 40, 1500, 90], [1, 40, 1, 64]
    need = sum(P.blocks_needed(n, 16) for n in seq_lens)
    case = workloads.make_chunk_case(seed=7500, seq_lens=seq_lens, query_lens=query_lens, num_blocks=need + 3,
                                     num_q_heads=32, num_kv_heads=8, dtype="bf16", block_size=16)
    kd, vd = dev(case.k_pool), dev(case.v_pool)
    desc = pa.dense_desc("bf16", 32, 8, 128, 16, case.num_blocks, kd.numel() * 2, vd.numel() * 2, 256)
    S, max_q, max_s = len(seq_lens), max(query_lens), max(seq_lens)
    ws = torch.empty(max(16, pa.pa_prefill_workspace_bytes(desc, S, case.total_q, max_q, max_s)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((case.total_q, 32, 128), dtype=torch.int16, device="cuda")
    q, bt, sl, qsl = dev(case.q), dev(case.block_tables), dev(case.seq_lens), dev(case.query_start_loc)

    def step():
        pa.pa_prefill_chunk(out, q, kd, vd, bt, sl, qsl, max_q, max_s, case.scale, desc, ws)

    ref, = replays_match_eager(step, [out])
    assert finite_bf16_or_f16(ref, "bf16")


def test_graph_decode_no_alloc():
    """pa_decode_no_alloc, the entry point meant for callers that capture: its scratch is static."""
    ctx = [9, 250, 1000]
    need = sum(P.blocks_needed(n, 16) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=7600, context_lens=ctx, num_blocks=need + 3, num_q_heads=32,
                                     num_kv_heads=8, dtype="bf16")
    kd, vd = dev(case.k_pool), dev(case.v_pool)
    B, max_ctx = case.num_seqs, max(ctx)
    desc = pa.dense_desc("bf16", 32, 8, 128, 16, case.num_blocks, kd.numel() * 2, vd.numel() * 2, 64)
    out = torch.empty(B, 32, 128, dtype=torch.int16, device="cuda")
    q, bt, lens = dev(case.q), dev(case.block_tables), dev(case.context_lens)

    def step():
        pa.pa_decode_no_alloc(out, q, kd, vd, bt, lens, max_ctx, case.scale, desc)

    ref, = replays_match_eager(step, [out])
    assert finite_bf16_or_f16(ref, "bf16")

"""pa_decode_no_alloc (static scratch, no allocation) against pa_decode and the oracle.

Each case runs two calls in a row through the C ABI, the second with a smaller input, and checks
that both outputs equal pa_decode's bit for bit (the same kernels) and match the oracle within the
decode tolerances. The scratch keeps the previous call's partials, so the second call also shows
that stale contents do not leak into a result.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
import workloads
from oracle import attention as A
from oracle import paging as P
from helpers import (DENSE_ATOL, DENSE_RTOL, MLA_ATOL, MLA_RTOL, assert_close, bits_np, dev, image_of,
                     out_to_f64, poison_tails)
import test_gpu_mla as M

pytestmark = pytest.mark.gpu


def dense_pair(case, part):
    kd, vd = case.k_pool.clone(), case.v_pool.clone()
    poison_tails(kd, case.block_tables, case.context_lens, case.block_size, case.dtype)
    poison_tails(vd, case.block_tables, case.context_lens, case.block_size, case.dtype)
    kd, vd = dev(kd), dev(vd)
    B, max_ctx = case.num_seqs, int(case.context_lens.max())
    desc = pa.dense_desc(case.dtype, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size,
                         case.num_blocks, kd.numel() * 2, vd.numel() * 2, part)
    need = pa.pa_decode_workspace_bytes(desc, B, max_ctx)
    assert 0 < need <= pa._lib.PA_STATIC_SCRATCH_BYTES, "the case must use the scratch"
    q, bt, lens = dev(case.q), dev(case.block_tables), dev(case.context_lens)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref_out = torch.empty(B, case.num_q_heads, case.head_dim, dtype=torch.int16, device="cuda")
    pa.pa_decode(ref_out, q, kd, vd, bt, lens, max_ctx, case.scale, desc, ws)
    out = torch.full_like(ref_out, -1)
    pa.pa_decode_no_alloc(out, q, kd, vd, bt, lens, max_ctx, case.scale, desc)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "pa_decode_no_alloc differs from pa_decode"
    row = case.row_bytes
    ov = P.CacheView(0, 0, case.block_size * row, row)
    want = A.paged_decode(bits_np(case.q), case.dtype, image_of(kd), ov, image_of(vd), ov, 0, case.block_tables,
                          case.context_lens, case.block_size, case.num_kv_heads, case.head_dim, case.scale)
    assert_close(out_to_f64(out, case.dtype), want, DENSE_ATOL, DENSE_RTOL, "no-alloc decode")


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f16", 8, 8), ("bf16", 32, 8)])
def test_no_alloc_dense_two_calls(dtype, Hq, Hkv):
    big = [3000, 1, 700, 0, 1500, 129, 2047, 16]
    small = [900, 2, 300]
    for i, ctx in enumerate((big, small)):
        need = sum(P.blocks_needed(n, 16) for n in ctx)
        case = workloads.make_dense_case("tiny", seed=6100 + 10 * i + Hq, context_lens=ctx, num_blocks=need + 4,
                                         num_q_heads=Hq, num_kv_heads=Hkv, dtype=dtype)
        dense_pair(case, 128)


def test_no_alloc_mla_two_calls():
    for i, (ctx, hq) in enumerate((([1, 600, 2000, 0, 65, 1300], 64), ([40, 500], 32))):
        need = sum(P.blocks_needed(n, M.BS) for n in ctx)
        case = workloads.make_mla_case(seed=6200 + i, context_lens=ctx, num_blocks=need + 2, num_q_heads=hq)
        img, host = M.populate(case)
        desc = M.mla_desc(case, img, 1, 64)
        B, max_ctx = len(ctx), max(ctx)
        need_ws = pa.pa_decode_workspace_bytes(desc, B, max_ctx)
        assert 0 < need_ws <= pa._lib.PA_STATIC_SCRATCH_BYTES
        ref_out = M.mla_decode_gpu(case, img, 1, 64)
        out = torch.full_like(ref_out, -1)
        pa.pa_decode_no_alloc(out, dev(case.q), img, None, dev(case.block_tables), dev(case.context_lens), max_ctx,
                              case.scale, desc)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), "pa_decode_no_alloc differs from pa_decode (MLA)"
        mla_v, _, _ = M.views()
        want = A.mla_decode(bits_np(case.q), host, mla_v, 1, case.block_tables, case.context_lens, M.BS, case.scale)
        assert_close(out.view(torch.bfloat16).double().cpu().numpy(), want, MLA_ATOL, MLA_RTOL, "no-alloc MLA")


def test_no_alloc_rejects_a_call_beyond_the_scratch():
    case = workloads.make_dense_case("tiny", seed=6300, context_lens=[5], num_blocks=4)
    desc = pa.dense_desc("f16", 8, 8, 128, 16, 4, case.k_pool.numel() * 2, case.v_pool.numel() * 2, 16)
    kd, vd = dev(case.k_pool), dev(case.v_pool)
    B, max_ctx = 9000, 16 * 64
    assert pa.pa_decode_workspace_bytes(desc, B, max_ctx) > pa._lib.PA_STATIC_SCRATCH_BYTES
    out = torch.empty(B, 8, 128, dtype=torch.int16, device="cuda")
    q = torch.zeros(B, 8, 128, dtype=torch.int16, device="cuda")
    bt = torch.zeros(B, 64, dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    with pytest.raises(pa.PagedAttentionError) as e:
        pa.pa_decode_no_alloc(out, q, kd, vd, bt, lens, max_ctx, case.scale, desc)
    assert e.value.status == pa._lib.PA_ERR_SCRATCH_LIMIT

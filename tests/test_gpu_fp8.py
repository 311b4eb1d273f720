"""GPU parity of the dense FP8 cache: quantize-on-write (pa_quantize_and_cache) and decode over it.

"deep dive into vLLM 05" §3.4: quantize on write, dequantize on read, FP8 the safest format. Each
case quantizes a whole 16-bit pool through pa_quantize_and_cache (every slot in order), checks every
byte against the oracle's quantization, NaN-poisons the rows past each context and the unused
blocks (E4M3 code 0x7F), then decodes with bf16 queries and compares with the oracle's float64
decode of the same bytes (codes times the cache scales) at the dense tolerance. Groups of 2..16
query heads at head_dim 128 run on the matrix cores, the other shapes on the FP8 vector kernel.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
import workloads
from oracle import attention as A
from oracle import paging as P
from oracle import quant as Q
from helpers import DENSE_ATOL, DENSE_RTOL, assert_close, bits_np, dev, image_of

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 2.0 ** -5, 0.02


def quantize_pool(case, src_dtype="bf16"):
    """fp8 pools [nb, bs, Hkv, D] (device uint8) written by pa_quantize_and_cache from the case's pools."""
    nb, bs, hkv, d = case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim
    tdt = torch.bfloat16 if src_dtype == "bf16" else torch.float16
    rows = []
    for pool in (case.k_pool, case.v_pool):
        x = pool.view(tdt).float()
        x = torch.nan_to_num(x, nan=0.0)                 # the unused-block NaNs are not valid inputs
        rows.append(x.to(tdt).reshape(nb * bs, hkv * d).contiguous())
    view = pa.dense_view(bs, hkv, d, 1)
    k8 = torch.full((nb, bs, hkv, d), 0xA5, dtype=torch.uint8, device="cuda")
    v8 = torch.full_like(k8, 0xA5)
    slots = torch.arange(nb * bs, dtype=torch.int64, device="cuda")
    pa.pa_quantize_and_cache(rows[0].cuda(), slots, k8, view, 0, bs, nb, K_SCALE, src_dtype=src_dtype,
                             v=rows[1].cuda(), v_cache=v8, v_view=view, v_scale=V_SCALE)
    torch.cuda.synchronize()
    for r, img, s in ((rows[0], k8, K_SCALE), (rows[1], v8, V_SCALE)):
        want = Q.dense_fp8_rows(r.view(torch.int16).numpy().view(np.uint16), src_dtype, np.float32(s))
        assert np.array_equal(image_of(img).reshape(nb * bs, hkv * d), want), "fp8 cache bytes differ"
    return k8, v8


def poison(k8, v8, case):
    """0x7F (E4M3 NaN) in every row no sequence may read."""
    bs = case.block_size
    used = np.zeros((case.num_blocks, bs), dtype=bool)
    for b, n in enumerate(case.context_lens):
        for t in range(int(n)):
            used[int(case.block_tables[b, t // bs]), t % bs] = True
    mask = torch.from_numpy(~used).cuda()
    k8[mask] = 0x7F
    v8[mask] = 0x7F


def decode(case, k8, v8, part, select=None):
    B, hq, d = case.num_seqs, case.num_q_heads, case.head_dim
    desc = pa.dense_desc("fp8", hq, case.num_kv_heads, d, case.block_size, case.num_blocks, k8.numel(), v8.numel(),
                         part, k_scale=K_SCALE, v_scale=V_SCALE)
    max_ctx = max(1, int(case.context_lens.max()))
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(desc, B, max_ctx)), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, hq, d, dtype=torch.int16, device="cuda")
    pa.pa_decode(out, dev(case.q), k8, v8, dev(case.block_tables), dev(case.context_lens), max_ctx, case.scale, desc, ws)
    torch.cuda.synchronize()
    view8 = P.CacheView(0, 0, case.block_size * case.num_kv_heads * d, case.num_kv_heads * d)
    want = A.paged_decode(bits_np(case.q), "bf16", image_of(k8), view8, image_of(v8), view8, 0, case.block_tables,
                          case.context_lens, case.block_size, case.num_kv_heads, d, case.scale, select=select,
                          kv_dtype="e4m3", k_scale=K_SCALE, v_scale=V_SCALE)
    got = out.view(torch.bfloat16).to(torch.float64).cpu().numpy()
    if select is not None:
        idx = tuple(np.array(select).T)
        got, want = got[idx], want[idx]
    assert_close(got, want, DENSE_ATOL, DENSE_RTOL, "fp8 decode")


SHAPES = [
    # Hq, Hkv, D, bs, contexts, partition
    (8, 8, 128, 16, [1, 17, 130, 300], 0),
    (40, 40, 128, 16, [5, 600, 1500], 0),
    (32, 8, 128, 16, [1, 15, 16, 17, 511, 512, 513, 2000], 0),
    (16, 8, 64, 16, [5, 64, 700], 128),
    (8, 4, 256, 16, [9, 257, 900], 0),
    (8, 1, 128, 64, [63, 64, 65, 3000], 0),
    (4, 4, 128, 32, [0, 31, 33, 1000], 64),
    (8, 8, 64, 16, [2, 3, 5], 0),
    (32, 2, 128, 16, [7, 300, 1100], 0),      # group 16, matrix cores
    (24, 8, 128, 16, [2, 3, 4, 5, 33], 0),    # group 3, matrix cores, short rows
    (8, 2, 128, 16, [1100, 2100, 1, 0], 16),  # more than 64 and 128 partials per row, matrix cores
    (4, 4, 128, 16, [1300, 3, 1025], 16),     # more than 64 partials, vector kernel
    # head_dim 64 and 256, four and eight query heads per K/V head (eight: two waves of four each)
    (32, 8, 64, 16, [3, 100, 900], 0),
    (16, 2, 64, 16, [2, 70, 1200], 128),
    (16, 4, 256, 16, [5, 300, 800], 0),
    (16, 2, 256, 32, [9, 200, 1100], 64),
    # block size 128, matrix-core and vector kernels
    (16, 4, 128, 128, [127, 128, 129, 900, 0], 0),
    (4, 4, 128, 128, [1, 255, 2000], 256),
]


@pytest.mark.parametrize("Hq,Hkv,D,bs,ctx,part", SHAPES)
def test_fp8_write_and_decode(Hq, Hkv, D, bs, ctx, part):
    need = sum(P.blocks_needed(n, bs) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=5000 + Hq + D + bs, context_lens=ctx, num_blocks=need + 5,
                                     num_q_heads=Hq, num_kv_heads=Hkv, block_size=bs, dtype="bf16", head_dim=D)
    k8, v8 = quantize_pool(case)
    poison(k8, v8, case)
    decode(case, k8, v8, part)


@pytest.mark.parametrize("Hq,Hkv,num_seqs", [(2, 2, 350), (8, 2, 520)])
def test_fp8_many_sequences(Hq, Hkv, num_seqs):
    """More than 256 sequences (the work search re-reads the partition counts), empty and 1-token rows."""
    rng = np.random.default_rng(num_seqs)
    ctx = rng.integers(0, 900, size=num_seqs)
    ctx[[0, num_seqs - 1]] = 0
    ctx[[1, 260, num_seqs - 2]] = 1
    need = sum(P.blocks_needed(int(n), 16) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=5600 + num_seqs, context_lens=ctx.tolist(), num_blocks=need + 5,
                                     num_q_heads=Hq, num_kv_heads=Hkv, dtype="bf16")
    k8, v8 = quantize_pool(case)
    poison(k8, v8, case)
    decode(case, k8, v8, 0)


def test_fp8_write_from_f16_sources():
    case = workloads.make_dense_case("tiny", seed=77, context_lens=[40, 3], num_blocks=8, num_q_heads=8,
                                     num_kv_heads=8, dtype="f16")
    quantize_pool(case, "f16")


def test_full_size_13b_shape_fp8_sampled():
    # The 13B-shaped decode (64 sequences, ctx U[128, 2048], 40/40 heads of 128, 12288 blocks of 16) with
    # its K/V quantized to FP8; checked on sampled (sequence, head) outputs.
    case = workloads.make_dense_case("mha13b", device="cuda")
    case.dtype = "bf16"
    case.k_pool = case.k_pool.view(torch.float16).to(torch.bfloat16).view(torch.int16)
    case.v_pool = case.v_pool.view(torch.float16).to(torch.bfloat16).view(torch.int16)
    case.q = case.q.view(torch.float16).to(torch.bfloat16).view(torch.int16)
    nb, bs, hkv, d = case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim
    view = pa.dense_view(bs, hkv, d, 1)
    k8 = torch.empty((nb, bs, hkv, d), dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)
    slots = torch.arange(nb * bs, dtype=torch.int64, device="cuda")
    ksrc = torch.nan_to_num(case.k_pool.view(torch.bfloat16), nan=0.0).reshape(nb * bs, hkv * d)
    vsrc = torch.nan_to_num(case.v_pool.view(torch.bfloat16), nan=0.0).reshape(nb * bs, hkv * d)
    pa.pa_quantize_and_cache(ksrc, slots, k8, view, 0, bs, nb, K_SCALE, v=vsrc, v_cache=v8, v_view=view,
                             v_scale=V_SCALE)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    select = [(int(b), int(h)) for b, h in zip(rng.integers(0, case.num_seqs, 12), rng.integers(0, 40, 12))]
    decode(case, k8, v8, 0, select=select)


def test_full_size_gqa_copied_prefix_fp8_sampled():
    # The GQA-8 batch (256 sequences, a 2000-token prompt copied into each sequence's own blocks plus
    # lognormal suffixes, 32/8 heads of 128, bf16) with its K/V quantized to FP8: the matrix-core FP8
    # decode at the bench's full size and library-chosen partitions; sampled (sequence, head) outputs.
    case = workloads.make_dense_case("gqa_prefix", device="cuda", copied_prefix=True)
    assert case.dtype == "bf16"
    nb, bs, hkv, d = case.num_blocks, case.block_size, case.num_kv_heads, case.head_dim
    view = pa.dense_view(bs, hkv, d, 1)
    k8 = torch.empty((nb, bs, hkv, d), dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)
    slots = torch.arange(nb * bs, dtype=torch.int64, device="cuda")
    ksrc = torch.nan_to_num(case.k_pool.view(torch.bfloat16), nan=0.0).reshape(nb * bs, hkv * d)
    vsrc = torch.nan_to_num(case.v_pool.view(torch.bfloat16), nan=0.0).reshape(nb * bs, hkv * d)
    pa.pa_quantize_and_cache(ksrc, slots, k8, view, 0, bs, nb, K_SCALE, v=vsrc, v_cache=v8, v_view=view,
                             v_scale=V_SCALE)
    torch.cuda.synchronize()
    del ksrc, vsrc
    case.k_pool = case.v_pool = None
    rng = np.random.default_rng(4)
    select = [(int(b), int(h)) for b, h in zip(rng.integers(0, case.num_seqs, 12),
                                               rng.integers(0, case.num_q_heads, 12))]
    select.append((int(np.argmax(case.context_lens)), case.num_q_heads - 1))
    decode(case, k8, v8, 0, select=select)

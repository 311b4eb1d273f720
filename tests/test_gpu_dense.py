"""GPU parity of the dense path: pa_reshape_and_cache (bit-exact) and pa_decode (tolerance) vs the oracle.

Inputs are seeded synthetic draws from ``workloads``. Bytes past each context
in the last block are NaN-poisoned, as are unused blocks, so any stray read
shows up as a non-finite output.
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_130_amd as pa
import workloads
from oracle import attention as A
from oracle import cache_write as W
from oracle import paging as P
from helpers import (DENSE_ATOL, DENSE_RTOL, assert_close, bits_np, compact_seq_image, dev, image_of,
                     out_to_f64, poison_tails)

pytestmark = pytest.mark.gpu


def oracle_view(case):
    row = case.row_bytes
    return P.CacheView(offset=0, layer_stride=0, block_stride=case.block_size * row, row_bytes=row)


def run_case(case, partition_size=0, check_write=True):
    """Write each sequence's last token with pa_reshape_and_cache, then pa_decode; compare both to the oracle."""
    k_host, v_host = case.k_pool.clone(), case.v_pool.clone()
    poison_tails(k_host, case.block_tables, case.context_lens, case.block_size, case.dtype)
    poison_tails(v_host, case.block_tables, case.context_lens, case.block_size, case.dtype)
    kd, vd = dev(k_host), dev(v_host)
    view = pa.dense_view(case.block_size, case.num_kv_heads, case.head_dim)
    slots = dev(case.new_slots)
    pa.pa_reshape_and_cache(dev(case.new_k), slots, kd, view, 0, case.block_size, case.num_blocks,
                            v=dev(case.new_v), v_cache=vd, v_view=view)
    ov = oracle_view(case)
    B = case.num_seqs
    k_img = W.reshape_and_cache(image_of(k_host), image_of(case.new_k).reshape(B, -1), case.new_slots, ov, 0,
                                case.block_size)
    v_img = W.reshape_and_cache(image_of(v_host), image_of(case.new_v).reshape(B, -1), case.new_slots, ov, 0,
                                case.block_size)
    torch.cuda.synchronize()
    if check_write:
        assert np.array_equal(image_of(kd), k_img), "K cache bytes differ after reshape_and_cache"
        assert np.array_equal(image_of(vd), v_img), "V cache bytes differ after reshape_and_cache"
    out = decode_gpu(case, kd, vd, partition_size)
    ref = A.paged_decode(bits_np(case.q), case.dtype, k_img, ov, v_img, ov, 0, case.block_tables,
                         case.context_lens, case.block_size, case.num_kv_heads, case.head_dim, case.scale)
    assert_close(out_to_f64(out, case.dtype), ref, DENSE_ATOL, DENSE_RTOL, f"decode P={partition_size}")
    return out, kd, vd


def decode_gpu(case, kd, vd, partition_size=0, tables=None, max_ctx=None):
    B = case.num_seqs
    tables = case.block_tables if tables is None else tables
    max_ctx = int(case.context_lens.max()) if max_ctx is None else max_ctx
    desc = pa.dense_desc(case.dtype, case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size,
                         case.num_blocks, kd.numel() * 2, vd.numel() * 2, partition_size)
    ws_bytes = pa.pa_decode_workspace_bytes(desc, B, max_ctx)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, case.num_q_heads, case.head_dim, dtype=torch.int16, device="cuda")
    pa.pa_decode(out, dev(case.q), kd, vd, dev(tables), dev(case.context_lens), max_ctx, case.scale, desc, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("partition_size", [0, 16, 64, 128, 512, 1024])
def test_tiny_workload_write_and_decode(partition_size):
    """4 sequences {1, 17, 130, 300}, 8/8 heads of 128, fp16, block size 16, 64 blocks."""
    run_case(workloads.make_dense_case("tiny"), partition_size)


SHAPES = [
    # dtype, Hq, Hkv, D, bs, contexts, partition
    ("bf16", 32, 8, 128, 16, [1, 15, 16, 17, 511, 512, 513, 2000], 0),
    ("f16", 16, 8, 128, 16, [2, 33, 100, 1500], 256),
    ("bf16", 64, 8, 128, 16, [7, 300, 1100], 0),
    ("f16", 8, 8, 64, 16, [5, 64, 700], 128),
    ("bf16", 8, 4, 256, 16, [9, 257, 900], 0),
    ("f16", 8, 8, 128, 32, [31, 32, 33, 1000], 64),
    ("bf16", 32, 8, 128, 64, [63, 64, 65, 3000], 0),
    ("f16", 4, 4, 128, 16, [0, 3000, 5, 1024, 1025], 1024),
    ("bf16", 4, 1, 128, 16, [1, 1000], 0),
    ("f16", 8, 1, 128, 256, [255, 256, 257, 3000], 0),
    # few tokens per row: the softmax weights are not averaged out, so their rounding shows
    ("bf16", 32, 8, 128, 16, [2, 3, 4, 5, 6, 7, 8, 9], 0),
    ("bf16", 8, 8, 128, 16, [2, 3, 4, 5], 0),
    ("bf16", 8, 8, 64, 16, [2, 3, 5], 0),
    # partitions of 16 tokens: more than 64 (and more than 128) partials per row to merge
    ("bf16", 8, 2, 128, 16, [1100, 2100, 3, 0], 16),
    ("f16", 4, 4, 128, 16, [1300, 2, 1025], 16),
    ("bf16", 4, 4, 256, 16, [1040, 17], 16),
    # head_dim 64 and 256 with four and eight query heads per K/V head (eight: two waves of four
    # read each K/V head)
    ("bf16", 32, 8, 64, 16, [3, 100, 900], 0),
    ("f16", 64, 8, 64, 16, [2, 70, 1200], 128),
    ("bf16", 16, 4, 256, 16, [5, 300, 800], 0),
    ("f16", 16, 2, 256, 32, [9, 200, 1100], 256),
    # block size 128, both kernels
    ("bf16", 16, 4, 128, 128, [127, 128, 129, 900, 0], 0),
    ("f16", 4, 4, 128, 128, [1, 255, 2000], 256),
]


@pytest.mark.parametrize("dtype,Hq,Hkv,D,bs,ctx,part", SHAPES)
def test_decode_shapes(dtype, Hq, Hkv, D, bs, ctx, part):
    need = sum(P.blocks_needed(n, bs) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=4000 + Hq + D + bs, context_lens=ctx, num_blocks=need + 7,
                                     num_q_heads=Hq, num_kv_heads=Hkv, block_size=bs, dtype=dtype, head_dim=D)
    run_case(case, part)


# partition_size far above every context (2^20 tokens). The library uses at most 64 blocks per
# partition: at block size 256 every context here (up to 16,384 tokens) is one partition, so no
# workspace and no merge; at block size 16 the long contexts are cut at 1,024 tokens.
UNBOUNDED = [
    # dtype, Hq, Hkv, bs, contexts, single partition
    ("f16", 4, 4, 256, [16000, 5, 257, 9000], True),    # vector kernel
    ("bf16", 8, 2, 256, [12000, 700, 1], True),         # matrix-core kernel
    ("bf16", 8, 8, 16, [3000, 40], False),
]


@pytest.mark.parametrize("dtype,Hq,Hkv,bs,ctx,single", UNBOUNDED)
def test_partition_beyond_every_context(dtype, Hq, Hkv, bs, ctx, single):
    need = sum(P.blocks_needed(n, bs) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=4500 + Hq + bs, context_lens=ctx, num_blocks=need + 3,
                                     num_q_heads=Hq, num_kv_heads=Hkv, block_size=bs, dtype=dtype)
    part = 1 << 20
    desc = pa.dense_desc(dtype, Hq, Hkv, 128, bs, case.num_blocks, case.k_pool.numel() * 2,
                         case.v_pool.numel() * 2, part)
    assert (pa.pa_decode_workspace_bytes(desc, case.num_seqs, max(ctx)) == 0) == single
    run_case(case, part, check_write=False)


def test_decode_is_deterministic_and_invariant_to_block_relabelling():
    ctx = [700, 33, 1600, 1]
    case = workloads.make_dense_case("tiny", seed=77, context_lens=ctx, num_blocks=200, num_q_heads=32,
                                     num_kv_heads=8, dtype="bf16")
    out1, kd, vd = run_case(case, 256)
    out2 = decode_gpu(case, kd, vd, 256)
    assert torch.equal(out1, out2), "two identical calls differ"
    rng = np.random.default_rng(5)
    pi = rng.permutation(case.num_blocks)
    pit = torch.as_tensor(pi, device="cuda")
    k2, v2 = torch.empty_like(kd), torch.empty_like(vd)
    k2[pit] = kd
    v2[pit] = vd
    t2 = case.block_tables.copy()
    m = t2 != workloads.INT32_PAD
    t2[m] = pi[t2[m]]
    out3 = decode_gpu(case, k2, v2, 256, tables=t2)
    assert torch.equal(out1, out3), "output changed under a relabelling of physical blocks"


def test_shared_prefix_equals_copied_prefix_bitwise():
    bs, prefix = 16, 160
    ctx = [prefix + 3, prefix + 90, prefix + 1, prefix + 400]
    rng = np.random.Generator(np.random.PCG64(31))
    shared, _ = workloads.allocate_block_tables(rng, ctx, bs, 200, shared_prefix_blocks=prefix // bs)
    copied = shared.copy()
    used = set(shared[shared != workloads.INT32_PAD].tolist())
    free = [b for b in range(200) if b not in used]
    kd = dev(workloads.draw_bits(41, (200, bs, 8, 128), "bf16"))
    vd = dev(workloads.draw_bits(42, (200, bs, 8, 128), "bf16"))
    for b in range(1, len(ctx)):
        for j in range(prefix // bs):
            nbk = free.pop()
            kd[nbk] = kd[int(shared[b, j])]
            vd[nbk] = vd[int(shared[b, j])]
            copied[b, j] = nbk
    case = workloads.DenseCase(name="prefix", dtype="bf16", block_size=bs, num_blocks=200, num_q_heads=32,
                               num_kv_heads=8, head_dim=128, scale=1 / math.sqrt(128),
                               context_lens=np.asarray(ctx, dtype=np.int32), block_tables=shared, seed=0)
    case.q = workloads.draw_bits(43, (len(ctx), 32, 128), "bf16")
    a = decode_gpu(case, kd, vd, 128)
    b = decode_gpu(case, kd, vd, 128, tables=copied)
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,Hq,Hkv,num_seqs,part", [
    ("f16", 2, 2, 400, 0),      # vector kernel
    ("bf16", 8, 2, 300, 128),   # matrix-core kernel (group 4)
    ("bf16", 16, 1, 600, 0),    # matrix-core kernel (group 16)
])
def test_decode_many_sequences(dtype, Hq, Hkv, num_seqs, part):
    """More than 256 sequences: the work search re-reads the partition counts from memory.

    Contexts are drawn in [0, 1200] with empty and one-token sequences forced in, so items of every
    partition index exist beside sequences with a single (or an empty) item.
    """
    rng = np.random.default_rng(num_seqs + Hq)
    ctx = rng.integers(0, 1201, size=num_seqs)
    ctx[[0, 7, num_seqs - 1]] = 0
    ctx[[1, 130, 257, num_seqs - 2]] = 1
    ctx[[2, 299]] = 1200
    need = sum(P.blocks_needed(int(n), 16) for n in ctx)
    case = workloads.make_dense_case("tiny", seed=4500 + num_seqs, context_lens=ctx.tolist(), num_blocks=need + 9,
                                     num_q_heads=Hq, num_kv_heads=Hkv, dtype=dtype)
    run_case(case, part)


# --------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the bench times (library-chosen
# partition), checked on sampled (sequence, head) outputs.
# --------------------------------------------------------------------------

def sampled_full_size(case, n_samples, seed):
    kd, vd = case.k_pool, case.v_pool            # already on the device
    poison_tails(kd, case.block_tables, case.context_lens, case.block_size, case.dtype)
    poison_tails(vd, case.block_tables, case.context_lens, case.block_size, case.dtype)
    out = decode_gpu(case, kd, vd, 0)
    got = out_to_f64(out, case.dtype)
    rng = np.random.default_rng(seed)
    seqs = sorted(set(rng.choice(case.num_seqs, size=min(n_samples, case.num_seqs), replace=False).tolist())
                  | {int(np.argmax(case.context_lens)), int(np.argmin(case.context_lens))})
    ov = oracle_view(case)
    q = bits_np(case.q)
    for s in seqs:
        n = int(case.context_lens[s])
        k_img, tbl = compact_seq_image(kd, case.block_tables[s], n, case.block_size)
        v_img, _ = compact_seq_image(vd, case.block_tables[s], n, case.block_size)
        heads = sorted(set(rng.choice(case.num_q_heads, size=4, replace=False).tolist()) | {0, case.num_q_heads - 1})
        ref = A.paged_decode(q[s:s + 1], case.dtype, k_img, ov, v_img, ov, 0, tbl[None, :], [n], case.block_size,
                             case.num_kv_heads, case.head_dim, case.scale, select=[(0, h) for h in heads])
        assert_close(got[s, heads], ref[0, heads], DENSE_ATOL, DENSE_RTOL, f"seq {s} (ctx {n})")
    assert np.isfinite(got).all()


def test_full_size_mha13b_sampled():
    """13B-shaped MHA decode: 64 seqs, ctx U[128, 2048], 40/40 heads, fp16, 12288-block pool."""
    sampled_full_size(workloads.make_dense_case("mha13b", device="cuda"), 12, 1)


def test_full_size_gqa_shared_prefix_sampled():
    """256 seqs sharing a 2000-token prompt plus lognormal suffixes, 32/8 heads, bf16."""
    sampled_full_size(workloads.make_dense_case("gqa_prefix", device="cuda"), 12, 2)


def test_full_size_gqa_copied_prefix_sampled():
    """The same batch with each sequence's 125 prompt blocks copied to private blocks (the timed variant)."""
    sampled_full_size(workloads.make_dense_case("gqa_prefix", device="cuda", copied_prefix=True), 12, 3)


def test_full_size_long_context_decode_sampled():
    """8 decodes at 32768 tokens, 32/8 heads, bf16, split-context partitions of 512."""
    case = workloads.make_dense_case("tiny", seed=1304, context_lens=[32768] * 8, num_blocks=17408,
                                     num_q_heads=32, num_kv_heads=8, dtype="bf16", device="cuda")
    kd, vd = case.k_pool, case.v_pool
    out = decode_gpu(case, kd, vd, 512)
    got = out_to_f64(out, "bf16")
    ov = oracle_view(case)
    q = bits_np(case.q)
    for s in (0, 5):
        k_img, tbl = compact_seq_image(kd, case.block_tables[s], 32768, 16)
        v_img, _ = compact_seq_image(vd, case.block_tables[s], 32768, 16)
        heads = [0, 3, 4, 17, 31]
        ref = A.paged_decode(q[s:s + 1], "bf16", k_img, ov, v_img, ov, 0, tbl[None, :], [32768], 16, 8, 128,
                             case.scale, select=[(0, h) for h in heads])
        assert_close(got[s, heads], ref[0, heads], DENSE_ATOL, DENSE_RTOL, f"seq {s}")

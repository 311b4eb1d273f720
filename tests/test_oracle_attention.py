"""Pins for oracle.attention: brute force, closed forms, invariances, and library routines.

Brute force here means torch's scaled_dot_product_attention in float64 on
the logically ordered (unpaged) K/V. Those tensors are placed into the pool
by the test itself, block by block, so the oracle's gather is checked
against an independent placement.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import numerics as N
from oracle import paging as P
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(rng, shape, dtype):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    t = x.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def build_paged(rng, ctx, Hkv, D, bs, nb, dtype, poison=True):
    """Logical per-sequence K/V bits, placed into a pool through seeded block tables."""
    tables, _ = workloads.allocate_block_tables(rng, ctx, bs, nb)
    nan = np.uint16(0x7E00 if dtype == "f16" else 0x7FC0)
    kpool = np.full((nb, bs, Hkv, D), nan if poison else 0, dtype=np.uint16)
    vpool = kpool.copy()
    K, V = [], []
    for b, n in enumerate(ctx):
        k = bits(rng, (n, Hkv, D), dtype)
        v = bits(rng, (n, Hkv, D), dtype)
        K.append(k)
        V.append(v)
        for j in range(P.blocks_needed(n, bs)):
            c = min(bs, n - j * bs)
            kpool[tables[b, j], :c] = k[j * bs:j * bs + c]
            vpool[tables[b, j], :c] = v[j * bs:j * bs + c]
    return tables, kpool, vpool, K, V


def dense_view(bs, Hkv, D):
    row = P.dense_row_bytes(Hkv, D, 2)
    return P.CacheView(offset=0, layer_stride=0, block_stride=bs * row, row_bytes=row)


def img(pool):
    return np.ascontiguousarray(pool).view(np.uint8).reshape(-1)


def sdpa(q, k, v, scale, causal=False):
    """torch SDPA (float64, CPU). q [Hq, Lq, D], k/v [Hq, Lk, D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale, is_causal=causal)[0].numpy()


@pytest.mark.parametrize("dtype,Hq,Hkv", [("f16", 8, 8), ("bf16", 32, 8), ("bf16", 6, 2), ("f16", 4, 1)])
def test_decode_matches_bruteforce_contiguous(dtype, Hq, Hkv):
    rng = np.random.Generator(np.random.PCG64(100 + Hq))
    D, bs, nb = 64, 16, 64
    ctx = [1, 17, 130, 300]
    tables, kpool, vpool, K, V = build_paged(rng, ctx, Hkv, D, bs, nb, dtype)
    q = bits(rng, (len(ctx), Hq, D), dtype)
    scale = 1 / math.sqrt(D)
    view = dense_view(bs, Hkv, D)
    out = A.paged_decode(q, dtype, img(kpool), view, img(vpool), view, 0, tables, ctx, bs, Hkv, D, scale)
    qf = N.bits_to_f64(q, dtype)
    g = Hq // Hkv
    for b, n in enumerate(ctx):
        kf = np.repeat(N.bits_to_f64(K[b], dtype).transpose(1, 0, 2), g, axis=0)   # [Hq, n, D]
        vf = np.repeat(N.bits_to_f64(V[b], dtype).transpose(1, 0, 2), g, axis=0)
        ref = sdpa(qf[b][:, None, :], kf, vf, scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_context_one_returns_v0_and_zero_context_returns_zero():
    rng = np.random.Generator(np.random.PCG64(3))
    D, bs, nb, Hkv = 32, 16, 8, 2
    tables, kpool, vpool, K, V = build_paged(rng, [1, 0], Hkv, D, bs, nb, "f16")
    q = bits(rng, (2, 4, D), "f16")
    view = dense_view(bs, Hkv, D)
    out = A.paged_decode(q, "f16", img(kpool), view, img(vpool), view, 0, tables, [1, 0], bs, Hkv, D, 0.3)
    v0 = N.f16_bits_to_f64(V[0][0])                 # [Hkv, D]
    assert np.array_equal(out[0], np.repeat(v0, 2, axis=0))
    assert np.array_equal(out[1], np.zeros((4, D)))


def test_equal_keys_give_mean_of_values():
    rng = np.random.Generator(np.random.PCG64(4))
    D, bs, nb, Hkv, n = 16, 16, 16, 1, 77
    tables, kpool, vpool, K, V = build_paged(rng, [n], Hkv, D, bs, nb, "bf16")
    for j in range(P.blocks_needed(n, bs)):         # overwrite every key with the same row
        kpool[tables[0, j]] = K[0][0]
    q = bits(rng, (1, 3, D), "bf16")
    view = dense_view(bs, Hkv, D)
    out = A.paged_decode(q, "bf16", img(kpool), view, img(vpool), view, 0, tables, [n], bs, Hkv, D, 0.5)
    mean = N.bf16_bits_to_f64(V[0]).mean(axis=0)[0]
    for h in range(3):
        np.testing.assert_allclose(out[0, h], mean, rtol=0, atol=1e-14)


def test_head_grouping_matches_page():
    g = json.load(open(os.path.join(GOLDEN, "head_grouping.json")))
    D, bs = 8, 16
    for kind in ("mha", "gqa", "mqa"):
        Hq, Hkv = g["num_q_heads"], g[kind]["num_kv_heads"]
        rng = np.random.Generator(np.random.PCG64(9))
        tables, kpool, vpool, K, V = build_paged(rng, [1], Hkv, D, bs, 4, "f16")
        q = bits(rng, (1, Hq, D), "f16")
        view = dense_view(bs, Hkv, D)
        out = A.paged_decode(q, "f16", img(kpool), view, img(vpool), view, 0, tables, [1], bs, Hkv, D, 1.0)
        v0 = N.f16_bits_to_f64(V[0][0])
        for kvh, members in enumerate(g[kind]["groups"]):
            for h1 in members:                       # page labels are 1-based
                assert np.array_equal(out[0, h1 - 1], v0[kvh])


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.Generator(np.random.PCG64(12))
    D, bs, nb, Hq, Hkv = 32, 16, 64, 8, 2
    ctx = [50, 129]
    tables, kpool, vpool, _, _ = build_paged(rng, ctx, Hkv, D, bs, nb, "f16")
    q = bits(rng, (2, Hq, D), "f16")
    rep_k = np.repeat(kpool, Hq // Hkv, axis=2)
    rep_v = np.repeat(vpool, Hq // Hkv, axis=2)
    a = A.paged_decode(q, "f16", img(kpool), dense_view(bs, Hkv, D), img(vpool), dense_view(bs, Hkv, D),
                       0, tables, ctx, bs, Hkv, D, 0.2)
    b = A.paged_decode(q, "f16", img(rep_k), dense_view(bs, Hq, D), img(rep_v), dense_view(bs, Hq, D),
                       0, tables, ctx, bs, Hq, D, 0.2)
    assert np.array_equal(a, b)


def test_physical_block_permutation_invariance():
    rng = np.random.Generator(np.random.PCG64(13))
    D, bs, nb, Hkv = 32, 16, 48, 4
    ctx = [33, 200, 7]
    tables, kpool, vpool, _, _ = build_paged(rng, ctx, Hkv, D, bs, nb, "bf16")
    q = bits(rng, (3, 8, D), "bf16")
    view = dense_view(bs, Hkv, D)
    out1 = A.paged_decode(q, "bf16", img(kpool), view, img(vpool), view, 0, tables, ctx, bs, Hkv, D, 0.1)
    pi = rng.permutation(nb)
    k2, v2 = np.empty_like(kpool), np.empty_like(vpool)
    k2[pi] = kpool
    v2[pi] = vpool
    t2 = tables.copy()
    m = t2 != workloads.INT32_PAD
    t2[m] = pi[t2[m]]
    out2 = A.paged_decode(q, "bf16", img(k2), view, img(v2), view, 0, t2, ctx, bs, Hkv, D, 0.1)
    assert np.array_equal(out1, out2)


def test_shared_prefix_equals_copied_prefix():
    rng = np.random.Generator(np.random.PCG64(14))
    D, bs, Hkv, prefix = 16, 16, 2, 48
    ctx = [prefix + 5, prefix + 40, prefix + 1]
    shared_tables, _ = workloads.allocate_block_tables(rng, ctx, bs, 64, shared_prefix_blocks=prefix // bs)
    kpool = bits(rng, (64, bs, Hkv, D), "f16")
    vpool = bits(rng, (64, bs, Hkv, D), "f16")
    copied = shared_tables.copy()
    free = sorted(set(range(64)) - set(shared_tables[shared_tables != workloads.INT32_PAD].tolist()))
    kc, vc = kpool.copy(), vpool.copy()
    for b in range(1, len(ctx)):                    # give sequences 1.. private byte copies of the prefix
        for j in range(prefix // bs):
            nbk = free.pop()
            kc[nbk], vc[nbk] = kpool[shared_tables[b, j]], vpool[shared_tables[b, j]]
            copied[b, j] = nbk
    q = bits(rng, (3, 4, D), "f16")
    view = dense_view(bs, Hkv, D)
    a = A.paged_decode(q, "f16", img(kpool), view, img(vpool), view, 0, shared_tables, ctx, bs, Hkv, D, 0.25)
    b = A.paged_decode(q, "f16", img(kc), view, img(vc), view, 0, copied, ctx, bs, Hkv, D, 0.25)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("part", [1, 3, 16, 32, 512, 10 ** 6])
def test_partition_merge_identity(part):
    rng = np.random.Generator(np.random.PCG64(part % 1000))
    n, D = 1000, 24
    s = rng.standard_normal(n) * 4
    V = rng.standard_normal((n, D))
    whole = np.exp(s - s.max()) @ V / np.exp(s - s.max()).sum()
    ms, ls, accs = A.partition_partials(s, V, part)
    assert len(ms) == -(-n // part)
    np.testing.assert_allclose(A.merge_partitions(ms, ls, accs), whole, rtol=0, atol=1e-12)


def test_chunk_rows_match_decode_causal_and_unchunked():
    rng = np.random.Generator(np.random.PCG64(15))
    D, bs, nb, Hq, Hkv, dt = 32, 16, 64, 4, 2, "bf16"
    total = 70
    tables, kpool, vpool, K, V = build_paged(rng, [total], Hkv, D, bs, nb, dt)
    view = dense_view(bs, Hkv, D)
    q_all = bits(rng, (total, Hq, D), dt)
    scale = 0.2
    # Unchunked causal pass over all 70 tokens (prior context 0) = SDPA causal.
    one = A.chunk_prefill(q_all, dt, img(kpool), view, img(vpool), view, 0, tables, [total], [0, total], bs,
                          Hkv, D, scale)
    kf = np.repeat(N.bits_to_f64(K[0], dt).transpose(1, 0, 2), Hq // Hkv, axis=0)
    vf = np.repeat(N.bits_to_f64(V[0], dt).transpose(1, 0, 2), Hq // Hkv, axis=0)
    qf = N.bits_to_f64(q_all, dt).transpose(1, 0, 2)
    ref = sdpa(qf, kf, vf, scale, causal=True).transpose(1, 0, 2)
    np.testing.assert_allclose(one, ref, rtol=0, atol=1e-12)
    # Chunked: 40 tokens, then 30 over the cached 40, in one varlen call as two "sequences".
    t2 = np.vstack([tables, tables])
    two = A.chunk_prefill(q_all, dt, img(kpool), view, img(vpool), view, 0, t2, [40, total], [0, 40, total],
                          bs, Hkv, D, scale)
    assert np.array_equal(two, one)
    # The last row of a chunk equals decode at the same total length.
    dec = A.paged_decode(q_all[total - 1:total], dt, img(kpool), view, img(vpool), view, 0, tables, [total],
                         bs, Hkv, D, scale)
    np.testing.assert_array_equal(one[total - 1], dec[0])


def _mla_image(rows_per_seq, tables, bs, nb, layer=0):
    views, block = P.block_outer_views([("mla", 656, 2), ("indexer", 132, 2)], bs)
    image = np.zeros(nb * block, dtype=np.uint8)
    for b, rows in enumerate(rows_per_seq):     # placement by the test, block by block
        for pos in range(len(rows)):
            a = P.address(views["mla"], layer, tables[b][pos // bs], pos % bs)
            image[a:a + 656] = rows[pos]
    return image, views["mla"]


def test_mla_matches_bruteforce_with_library_fp8_decode():
    rng = np.random.Generator(np.random.PCG64(16))
    bs, nb, Hq = 64, 12, 16
    ctx = [1, 70, 200]
    tables, _ = workloads.allocate_block_tables(rng, ctx, bs, nb)
    rows = [workloads.draw_mla_rows(1000 + b, n).numpy() for b, n in enumerate(ctx)]
    image, view = _mla_image(rows, tables, bs, nb, layer=1)
    q = bits(rng, (3, Hq, 576), "bf16")
    scale = 1 / math.sqrt(576)
    out = A.mla_decode(q, image, view, 1, tables, ctx, bs, scale)
    for b, n in enumerate(ctx):
        r = torch.from_numpy(rows[b])
        lat = r[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
        sc = r[:, 512:528].contiguous().view(torch.float32).to(torch.float64)        # [n, 4]
        c = (lat.reshape(n, 4, 128) * sc[:, :, None]).reshape(n, 512)
        rope = r[:, 528:656].contiguous().view(torch.bfloat16).to(torch.float64)
        kk = torch.cat([c, rope], dim=1)                                           # [n, 576]
        qf = torch.from_numpy(q[b].view(np.int16)).view(torch.bfloat16).to(torch.float64)
        ref = torch.nn.functional.scaled_dot_product_attention(
            qf[:, None, :], kk[None].expand(Hq, n, 576), c[None].expand(Hq, n, 512), scale=scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


def test_mla_with_unit_scales_and_zero_rope_is_mqa_decode():
    rng = np.random.Generator(np.random.PCG64(17))
    bs, nb, Hq = 64, 8, 8
    ctx = [90, 5]
    tables, _ = workloads.allocate_block_tables(rng, ctx, bs, nb)
    rows, kv_bits = [], []
    for n in ctx:
        codes = rng.integers(0, 256, size=(n, 512), dtype=np.uint8)
        codes[(codes & 0x7F) == 0x7F] = 0x3C        # no NaN codes
        r = np.zeros((n, 656), dtype=np.uint8)
        r[:, :512] = codes
        r[:, 512:528] = np.ones((n, 4), dtype="<f4").view(np.uint8)
        rows.append(r)
        # the same values as bf16 bits (exact), via torch's library conversion
        kv_bits.append(torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.bfloat16)
                       .view(torch.int16).numpy().view(np.uint16))
    image, view = _mla_image(rows, tables, bs, nb)
    q = bits(rng, (2, Hq, 576), "bf16")
    q[:, :, 512:] = 0
    out = A.mla_decode(q, image, view, 0, tables, ctx, bs, 0.05)
    pool = np.zeros((nb, bs, 1, 512), dtype=np.uint16)
    for b, n in enumerate(ctx):
        for pos in range(n):
            pool[tables[b][pos // bs], pos % bs, 0] = kv_bits[b][pos]
    dv = dense_view(bs, 1, 512)
    ref = A.paged_decode(np.ascontiguousarray(q[:, :, :512]), "bf16", img(pool), dv, img(pool), dv, 0, tables,
                         ctx, bs, 1, 512, 0.05)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_fp8_cache_decode_equals_bf16_decode_of_the_dequantized_values():
    # With scales that are powers of two, code * scale is exactly representable in bf16 (E4M3 values
    # carry 4 significant bits). So an FP8 cache and a bf16 cache holding the dequantized values must
    # give the same float64 decode: this pins the FP8 read path (codes, scales, and where each scale
    # applies) against the plain dense path.
    from oracle import numerics as N
    import torch
    rng = np.random.Generator(np.random.PCG64(17))
    bs, nb, hkv, hq, d = 16, 24, 2, 4, 64
    row8, row16 = hkv * d, hkv * d * 2
    k_codes = rng.integers(0, 256, size=nb * bs * row8, dtype=np.uint8)
    v_codes = rng.integers(0, 256, size=nb * bs * row8, dtype=np.uint8)
    for c in (k_codes, v_codes):
        c[(c & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    ks, vs = 2.0 ** -3, 2.0 ** 2
    to_bf16 = lambda codes, s: torch.from_numpy(N.e4m3_bytes_to_f64(codes) * s).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint8)
    k16, v16 = to_bf16(k_codes, ks), to_bf16(v_codes, vs)
    assert np.array_equal(N.bf16_bits_to_f64(k16.view(np.uint16)), N.e4m3_bytes_to_f64(k_codes) * ks)
    view8 = P.CacheView(0, 0, bs * row8, row8)
    view16 = P.CacheView(0, 0, bs * row16, row16)
    tables = rng.permutation(nb).reshape(3, 8).astype(np.int64)
    ctx = [1, 50, 128]
    q = torch.randn(3, hq, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)
    a = A.paged_decode(q, "bf16", k_codes, view8, v_codes, view8, 0, tables, ctx, bs, hkv, d, 0.125,
                       kv_dtype="e4m3", k_scale=ks, v_scale=vs)
    b = A.paged_decode(q, "bf16", k16, view16, v16, view16, 0, tables, ctx, bs, hkv, d, 0.125)
    assert np.array_equal(a, b)

"""Pins for oracle.quant: quantize-on-write of the DSA dual cache rows.

The encoder is checked against torch's float8_e4m3fn cast (a library
conversion to the same OCP format, round to nearest even) on every finite
value, every midpoint between neighbours and random values. The group recipe
(scale = amax / 448, codes of x / scale) is checked against the same recipe
written with torch float32 operations. The row layout is checked against the
byte counts of "vLLM KV Cache Layout 可视化" (656 B MLA rows: 512 B FP8 latent,
16 B scale, 128 B BF16 RoPE; 132 B indexer rows: 128 B FP8 key, 4 B FP32
scale), and the dequantized values against the format's error bound.
"""

import numpy as np
import pytest
import torch

from oracle import numerics as N
from oracle import paging as P
from oracle import quant as Q
from oracle.cache_write import reshape_and_cache


def torch_e4m3(x64: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x64, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def finite_values():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    return codes, N.E4M3_TABLE[codes]


def test_every_finite_code_encodes_to_itself():
    codes, vals = finite_values()
    assert np.array_equal(Q.e4m3_encode(vals), codes.astype(np.uint8))


def test_midpoints_round_to_even_like_torch():
    _, vals = finite_values()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2            # exactly representable in float32
    got = Q.e4m3_encode(np.concatenate([mids, -mids]))
    ref = torch_e4m3(np.concatenate([mids, -mids]))
    assert np.array_equal(got, ref)
    # spot checks from the definition: 0.5 * 2^-9 ties to 0 (even), 1.5 * 2^-9 ties to 2 * 2^-9
    assert Q.e4m3_encode([2.0 ** -10, 3 * 2.0 ** -10]).tolist() == [0x00, 0x02]


def test_random_values_match_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-463.0, 463.0, 200000), rng.normal(0, 1e-2, 50000),
                        rng.normal(0, 2.0 ** -8, 50000)]).astype(np.float32).astype(np.float64)
    assert np.array_equal(Q.e4m3_encode(x), torch_e4m3(x))


def test_saturation_reading():
    # 448 < |q| < 464 rounds to 448 under round-to-nearest; at and above 464 the reading saturates.
    got = Q.e4m3_encode([448.0, 455.0, 463.99, 464.0, 470.0, 1.0e6, -464.0, -1.0e6])
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert Q.e4m3_encode([-0.0, -1e-9]).tolist() == [0x80, 0x80]


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)


def torch_group(bits: np.ndarray):
    """The group recipe in torch float32: scale = amax / 448, codes = e4m3(x / scale)."""
    x = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).to(torch.float32)
    amax = x.abs().max()
    scale = amax / torch.tensor(448.0, dtype=torch.float32)
    codes = (x / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, np.float32(scale.item())


@pytest.mark.parametrize("kind", ["normal", "wide", "tiny", "one_hot", "negative_max", "huge"])
def test_group_recipe_matches_torch(kind):
    g = torch.Generator().manual_seed(11)
    x = torch.randn(128, generator=g)
    if kind == "wide":
        x = x * torch.pow(10.0, torch.randint(-6, 6, (128,), generator=g).float())
    elif kind == "tiny":
        x = x * 1e-30
    elif kind == "one_hot":
        x = torch.zeros(128)
        x[17] = 3.0
    elif kind == "negative_max":
        x[5] = -50.0
    elif kind == "huge":
        x = x * 1e30
    bits = bf16_bits(x)
    codes, scale = Q.quantize_group(bits)
    ref_codes, ref_scale = torch_group(bits)
    assert np.float32(scale).view(np.uint32) == np.float32(ref_scale).view(np.uint32)
    assert np.array_equal(codes, ref_codes)


def test_zero_group_reading():
    codes, scale = Q.quantize_group(np.zeros(128, dtype=np.uint16))
    assert scale == 0 and not codes.any()


def test_dequantized_error_bound():
    # Normal E4M3 values carry 3 mantissa bits: nearest rounding errs by at most 2^-4 of the value's
    # binade, and values below the smallest normal by half the subnormal step 2^-10. In units of the
    # group's scale: |code * scale - x| <= max(2^-4 |x|, 2^-10 scale) + float32 rounding.
    g = torch.Generator().manual_seed(3)
    for _ in range(20):
        bits = bf16_bits(torch.randn(128, generator=g) * 5)
        codes, scale = Q.quantize_group(bits)
        x = N.bf16_bits_to_f64(bits)
        deq = N.e4m3_bytes_to_f64(codes) * float(scale)
        bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * float(scale)) * (1 + 1e-6) + 1e-30
        assert np.all(np.abs(deq - x) <= bound)
        assert np.max(np.abs(N.e4m3_bytes_to_f64(codes))) == 448.0   # the group maximum maps to 448


def test_row_layout_matches_page_byte_counts():
    g = torch.Generator().manual_seed(5)
    lat = bf16_bits(torch.randn(512, generator=g))
    rope = bf16_bits(torch.randn(64, generator=g))
    key = bf16_bits(torch.randn(128, generator=g))
    row = Q.mla_row(lat, rope)
    assert row.shape == (656,) and 512 + 16 + 128 == 656
    for k in range(4):
        codes, scale = torch_group(lat[128 * k:128 * (k + 1)])
        assert np.array_equal(row[128 * k:128 * (k + 1)], codes)
        assert row[512 + 4 * k:516 + 4 * k].view("<f4")[0] == scale
    assert np.array_equal(row[528:656].view("<u2"), rope)
    irow = Q.indexer_row(key)
    assert irow.shape == (132,) and 128 + 4 == 132
    codes, scale = torch_group(key)
    assert np.array_equal(irow[:128], codes) and irow[128:132].view("<f4")[0] == scale


def test_quantize_and_cache_scatters_like_reshape_and_cache():
    # The dual cache of the page at block size 16 and 8 blocks, block-outer: MLA L0 | MLA L1 | IDX L0 | IDX L1.
    bs, nb = 16, 8
    pm, pi = bs * 656, bs * 132
    block = 2 * pm + 2 * pi
    mla_v = P.CacheView(0, pm, block, 656)
    idx_v = P.CacheView(2 * pm, pi, block, 132)
    image = np.full(nb * block, 0xA5, dtype=np.uint8)
    g = torch.Generator().manual_seed(9)
    T = 10
    lat = bf16_bits(torch.randn(T, 512, generator=g))
    rope = bf16_bits(torch.randn(T, 64, generator=g))
    key = bf16_bits(torch.randn(T, 128, generator=g))
    slots = np.array([5, 17, -1, 100, 3, 127, 64, -1, 90, 31], dtype=np.int64)
    got = Q.quantize_and_cache(image, lat, rope, key, slots, mla_v, idx_v, 1, bs)
    rows = np.stack([Q.mla_row(lat[t], rope[t]) for t in range(T)])
    irows = np.stack([Q.indexer_row(key[t]) for t in range(T)])
    ref = reshape_and_cache(reshape_and_cache(image, rows, slots, mla_v, 1, bs), irows, slots, idx_v, 1, bs)
    assert np.array_equal(got, ref)
    # layer 0 and every unaddressed byte keep the sentinel
    touched = np.zeros(image.size, dtype=bool)
    for s in slots[slots >= 0]:
        b, pos = P.split_slot(int(s), bs)
        a = P.address(mla_v, 1, b, pos)
        touched[a:a + 656] = True
        a = P.address(idx_v, 1, b, pos)
        touched[a:a + 132] = True
    assert (got[~touched] == 0xA5).all()
    only_mla = Q.quantize_and_cache(image, lat, rope, None, slots, mla_v, None, 1, bs)
    assert np.array_equal(only_mla, reshape_and_cache(image, rows, slots, mla_v, 1, bs))


@pytest.mark.parametrize("src", ["bf16", "f16"])
def test_dense_fp8_rows_match_torch(src):
    # The dense recipe with a per-cache scale, written with torch float32 operations: x / scale, clamped
    # to the format's range (the reading saturates), cast to float8_e4m3fn.
    g = torch.Generator().manual_seed(13)
    x = torch.randn(64, 256, generator=g) * 3
    x[0, :8] = torch.tensor([1e4, -1e4, 500.0, -470.0, 0.0, -0.0, 1e-6, -1e-6])   # saturating, zero, tiny
    tdt = torch.bfloat16 if src == "bf16" else torch.float16
    bits = x.to(tdt).view(torch.int16).numpy().view(np.uint16)
    scale = np.float32(0.0625)
    got = Q.dense_fp8_rows(bits, src, scale)
    xf = torch.from_numpy(bits.astype(np.int16)).view(tdt).to(torch.float32)
    ref = (xf / torch.tensor(scale)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)

"""Quantize-on-write of the DSA dual cache rows, as bytes (test infrastructure only).

Sources:
* "deep dive into vLLM 05", §3.4 (KV cache quantization): the cache may be
  stored at low precision by quantizing when it is written and dequantizing
  when it is read; finer scale groups are more accurate and carry more
  metadata; FP8 is the safest format in practice.
* "vLLM KV Cache Layout 可视化", section on two caches sharing one block
  table: an MLA row is 512 B of FP8 latent, 16 B of scale and 128 B of BF16
  RoPE (656 B per token); an indexer row is 128 B of FP8 key and a 4 B FP32
  scale (132 B per token).

Readings (the pages give the row formats but not the scale recipe):
* Inputs are bf16: the 512-value latent, the 64-value RoPE part and the
  128-value indexer key of each token.
* The 16 B of MLA scale are four little-endian float32 values; scale k covers
  latent values [128k, 128k + 128). The indexer row has one scale for its 128
  values.
* scale = amax / 448 in float32 (448 is the largest finite E4M3 value), with
  amax the largest magnitude in the group; each value is stored as the OCP
  E4M3 code nearest to x / scale (float32 division), ties to the even
  mantissa, with the quotient's sign (a negative value that rounds to zero is
  stored as -0). A quotient at or above 464 (half-way to the next,
  unrepresented, step) saturates to 448 instead of becoming NaN.
* A group of zeros stores scale 0 and zero codes.
* Inputs are finite; non-finite inputs give unspecified rows.

The rows are then scattered through slot_mapping exactly as by
``cache_write.reshape_and_cache``.
"""

from __future__ import annotations

import numpy as np

from .cache_write import reshape_and_cache
from .numerics import E4M3_TABLE, bf16_bits_to_f64
from .paging import CacheView

E4M3_MAX = 448.0
# Positive finite E4M3 values in increasing order, with their codes (0x00 .. 0x7E).
_POS_CODES = np.arange(0x00, 0x7F)
_POS_VALUES = E4M3_TABLE[_POS_CODES]
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_encode(q) -> np.ndarray:
    """Nearest OCP E4M3 code to each finite value of ``q``, ties to the even mantissa, saturating at 448.

    Written from the definition: among the representable values, take the one
    at the smallest distance from |q|; on a tie take the code whose lowest
    mantissa bit is 0; copy the sign bit (so -0.0 and negative values that
    round to zero give 0x80). Values at or above 464 map to 448.
    """
    q = np.asarray(q, dtype=np.float64)
    a = np.abs(q)
    hi = np.searchsorted(_POS_VALUES, a, side="left").clip(1, len(_POS_VALUES) - 1)
    lo = hi - 1
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((_POS_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a <= _POS_VALUES[0], 0, code)         # exact zero
    code = np.where(a >= 464.0, 0x7E, code)                # beyond the last step: saturate
    return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def quantize_group(values_bf16_bits) -> tuple[np.ndarray, np.float32]:
    """One scale group: bf16 bits [n] -> (e4m3 codes [n], float32 scale)."""
    x = bf16_bits_to_f64(values_bf16_bits).astype(np.float32)  # exact
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / np.float32(E4M3_MAX))            # float32 division, correctly rounded
    if scale == 0:
        return np.zeros(x.shape, dtype=np.uint8), np.float32(0)
    q = (x / scale).astype(np.float32)                          # float32 division per value
    return e4m3_encode(q.astype(np.float64)), scale


def mla_row(latent_bits, rope_bits) -> np.ndarray:
    """bf16 latent [512] + bf16 rope [64] (bit patterns) -> packed 656-byte MLA row."""
    latent_bits = np.asarray(latent_bits, dtype=np.uint16)
    rope_bits = np.asarray(rope_bits, dtype=np.uint16)
    assert latent_bits.shape == (512,) and rope_bits.shape == (64,)
    row = np.zeros(656, dtype=np.uint8)
    scales = np.zeros(4, dtype="<f4")
    for k in range(4):
        codes, scales[k] = quantize_group(latent_bits[128 * k:128 * (k + 1)])
        row[128 * k:128 * (k + 1)] = codes
    row[512:528] = scales.view(np.uint8)
    row[528:656] = rope_bits.astype("<u2").view(np.uint8)
    return row


def indexer_row(key_bits) -> np.ndarray:
    """bf16 key [128] (bit patterns) -> packed 132-byte indexer row."""
    key_bits = np.asarray(key_bits, dtype=np.uint16)
    assert key_bits.shape == (128,)
    codes, scale = quantize_group(key_bits)
    row = np.zeros(132, dtype=np.uint8)
    row[:128] = codes
    row[128:132] = np.array([scale], dtype="<f4").view(np.uint8)
    return row


def quantize_and_cache(image: np.ndarray, latent_bits, rope_bits, index_bits, slot_mapping,
                       mla_view: CacheView, index_view: CacheView | None, layer: int,
                       block_size: int) -> np.ndarray:
    """Quantize every token's rows and scatter them; ``index_bits`` None writes only the MLA view.

    ``image`` is the byte image of one allocation that holds both views (the DSA
    dual cache); a copy is returned.
    """
    latent_bits = np.asarray(latent_bits, dtype=np.uint16)
    rope_bits = np.asarray(rope_bits, dtype=np.uint16)
    T = latent_bits.shape[0]
    mla_rows = np.stack([mla_row(latent_bits[t], rope_bits[t]) for t in range(T)]) if T else \
        np.zeros((0, 656), dtype=np.uint8)
    out = reshape_and_cache(image, mla_rows, slot_mapping, mla_view, layer, block_size)
    if index_bits is not None:
        index_bits = np.asarray(index_bits, dtype=np.uint16)
        idx_rows = np.stack([indexer_row(index_bits[t]) for t in range(T)]) if T else \
            np.zeros((0, 132), dtype=np.uint8)
        out = reshape_and_cache(out, idx_rows, slot_mapping, index_view, layer, block_size)
    return out


def dense_fp8_rows(src_bits, src_dtype: str, scale) -> np.ndarray:
    """Dense rows for an FP8 cache: 16-bit values [n, m] (stored bits) -> E4M3 codes [n, m].

    Reading for the dense FP8 cache ("deep dive into vLLM 05" §3.4 names quantize-on-write and FP8; the
    granularity is left open): one float32 scale per cache, given by the caller; each value is stored
    as the E4M3 code nearest to the float32 quotient x / scale, saturating at 448.
    """
    from .numerics import bits_to_f64
    x = bits_to_f64(np.asarray(src_bits, dtype=np.uint16), src_dtype).astype(np.float32)  # exact
    q = (x / np.float32(scale)).astype(np.float32)                                      # float32 division
    return e4m3_encode(q.astype(np.float64))

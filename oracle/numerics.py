"""Exact decoding of stored number formats into float64.

fp16 and bf16 convert exactly into float64. So does every finite OCP E4M3
code. The e4m3 table is built from the OCP 8-bit floating point
specification's definition of E4M3: layout S.EEEE.MMM with exponent bias 7,
no infinities, and NaN only for S.1111.111. The fp8 format comes from the
"vLLM KV Cache Layout 可视化" page, section on two caches sharing one block
table: 512 B of FP8 latent per MLA row and 128 B of FP8 key per indexer row.
"""

from __future__ import annotations

import numpy as np


def f16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16/int16) to float64, exactly."""
    b = np.ascontiguousarray(np.asarray(bits)).astype(np.uint16, copy=False)
    return b.view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns to float64: the 16 bits are the top half of a binary32."""
    b = np.ascontiguousarray(np.asarray(bits)).astype(np.uint16, copy=False)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns quieten; still NaN
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bits_to_f64(bits, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(dtype)


def _e4m3_value(code: int) -> float:
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)          # subnormal: 0.MMM x 2^(1-bias)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)        # normal: 1.MMM x 2^(E-bias)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_bytes_to_f64(codes) -> np.ndarray:
    """OCP E4M3 byte codes to float64 via the 256-entry table."""
    return E4M3_TABLE[np.asarray(codes).astype(np.uint8)]


def f32le_bytes_to_f64(raw) -> np.ndarray:
    """Little-endian binary32 values stored as bytes ([..., 4k] uint8) to float64 [..., k]."""
    r = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    return r.view("<f4").astype(np.float64)


def u16le_bytes(raw) -> np.ndarray:
    """Little-endian 16-bit words stored as bytes to uint16."""
    r = np.ascontiguousarray(np.asarray(raw, dtype=np.uint8))
    return r.view("<u2")

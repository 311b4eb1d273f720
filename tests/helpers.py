"""Shared test plumbing: tolerance checks, byte images, tail poisoning, device upload."""

from __future__ import annotations

import numpy as np
import torch

from oracle import paging as P
import workloads

# Tolerances: |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise.
DENSE_ATOL, DENSE_RTOL = 2e-3, 1e-2   # fp16 / bf16 inputs, fp32 accumulation
MLA_ATOL, MLA_RTOL = 3e-2, 3e-2       # fp8-dequantised MLA latent


def assert_close(got: np.ndarray, want: np.ndarray, atol: float, rtol: float, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(want).all(), "oracle produced non-finite values"
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} want {want[i]!r} (max abs err {err.max():.3e})")


def out_to_f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16).to(torch.float64).cpu().numpy()


def image_of(t: torch.Tensor) -> np.ndarray:
    """Bytes of a tensor (any device) as a flat numpy uint8 array."""
    return t.detach().contiguous().view(torch.uint8).reshape(-1).cpu().numpy()


def bits_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().view(np.uint16)


def poison_tails(pool: torch.Tensor, tables: np.ndarray, context_lens, block_size: int, dtype: str):
    """NaN-fill positions past each sequence's context in its last block (in place)."""
    nan = workloads.f16_nan_bits() if dtype == "f16" else workloads.bf16_nan_bits()
    for b, n in enumerate(context_lens):
        n = int(n)
        if n == 0 or n % block_size == 0:
            continue
        lb, off = P.logical_block_and_offset(n, block_size)
        pool[int(tables[b, lb]), off:] = nan


def compact_seq_image(pool: torch.Tensor, table_row, num_tokens: int, block_size: int):
    """Copy one sequence's blocks out of a (device) pool; returns (image uint8, relabelled table row)."""
    nblk = P.blocks_needed(num_tokens, block_size)
    ids = torch.as_tensor(np.asarray(table_row[:nblk], dtype=np.int64), device=pool.device)
    sub = pool.index_select(0, ids)
    return image_of(sub), np.arange(nblk, dtype=np.int64)


def dev(x, device="cuda"):
    if isinstance(x, np.ndarray):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return x.to(device)

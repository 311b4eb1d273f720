"""ctypes binding of libpa.so (include/pa.h): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels. This module
turns torch tensors into device pointers and sizes, and turns the caller's
descriptors into the C structs. If the library is missing it raises at
import time; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK = 0
PA_ERR_NULL_POINTER = 1
PA_ERR_INVALID_ARGUMENT = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_MISALIGNED = 4
PA_ERR_VIEW_OUT_OF_RANGE = 5
PA_ERR_WORKSPACE = 6
PA_ERR_HIP = 7
PA_ERR_SCRATCH_LIMIT = 8

PA_STATIC_SCRATCH_BYTES = 64 << 20  # pa_decode_no_alloc's static scratch per GPU

PA_KV_F16 = 0
PA_KV_BF16 = 1
PA_KV_MLA656_E4M3 = 2
PA_KV_FP8_E4M3 = 3

EXPORTS = ("pa_abi_version", "pa_status_string", "pa_last_hip_error", "pa_reshape_and_cache", "pa_quantize_and_cache_mla",
           "pa_copy_blocks", "pa_quantize_and_cache",
           "pa_decode_workspace_bytes", "pa_decode", "pa_prefill_workspace_bytes", "pa_prefill_chunk",
           "pa_indexer_topk", "pa_mla_sparse_decode", "pa_decode_no_alloc")


class pa_cache_view(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("layer_stride", ctypes.c_int64), ("block_stride", ctypes.c_int64),
                ("row_bytes", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class pa_attn_desc(ctypes.Structure):
    _fields_ = [("kv_format", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("qk_dim", ctypes.c_int32), ("v_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("layer", ctypes.c_int32), ("partition_size", ctypes.c_int32), ("num_blocks", ctypes.c_int64),
                ("k_view", pa_cache_view), ("v_view", pa_cache_view), ("k_cache_bytes", ctypes.c_int64),
                ("v_cache_bytes", ctypes.c_int64), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class PagedAttentionError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = f"{fn} failed: {status_string(status)} (status {status})"
        if status == PA_ERR_HIP:
            msg += f", hipError {_lib.pa_last_hip_error()}"
        super().__init__(msg)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_kv_cache_130_amd/build.py`")
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7). Loading torch first
    # makes libpa.so bind to that runtime, so the streams and device memory torch hands over belong to
    # the runtime that launches the kernels. Loading libpa.so first would pull a second runtime into the
    # process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    V = pa_cache_view
    sig = {
        "pa_abi_version": (I32, []),
        "pa_status_string": (ctypes.c_char_p, [I32]),
        "pa_last_hip_error": (I32, []),
        "pa_reshape_and_cache": (I32, [P, I64, P, I64, P, I32, P, I64, V, P, I64, V, I32, I32, I64, P]),
        "pa_quantize_and_cache_mla": (I32, [P, I64, P, I64, P, I64, P, I32, P, I64, V, P, I64, V, I32, I32, I64,
                                            P]),
        "pa_copy_blocks": (I32, [P, I64, V, P, I64, V, P, I32, I32, I32, I64, P]),
        "pa_quantize_and_cache": (I32, [P, I64, P, I64, I32, ctypes.c_float, ctypes.c_float, P, I32, P, I64, V, P, I64,
                                        V, I32, I32, I64, P]),
        "pa_decode_workspace_bytes": (SZ, [ctypes.POINTER(pa_attn_desc), I32, I32]),
        "pa_decode": (I32, [P, P, P, P, P, I32, P, I32, I32, ctypes.c_float, ctypes.POINTER(pa_attn_desc), P, SZ,
                            P]),
        "pa_decode_no_alloc": (I32, [P, P, P, P, P, I32, P, I32, I32, ctypes.c_float, ctypes.POINTER(pa_attn_desc),
                                     P]),
        "pa_prefill_workspace_bytes": (SZ, [ctypes.POINTER(pa_attn_desc), I32, I32, I32, I32]),
        "pa_prefill_chunk": (I32, [P, P, P, P, P, I32, P, P, I32, I32, I32, I32, ctypes.c_float,
                                   ctypes.POINTER(pa_attn_desc), P, SZ, P]),
        "pa_indexer_topk": (I32, [P, P, P, I32, P, I64, P, P, I32, P, I64, V, I32, P, I32, P, I32, I32, I32, I64, P]),
        "pa_mla_sparse_decode": (I32, [P, P, P, P, I32, P, I32, I32, ctypes.c_float, ctypes.POINTER(pa_attn_desc), P,
                                       SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def abi_version() -> int:
    return _lib.pa_abi_version()


def status_string(status: int) -> str:
    return _lib.pa_status_string(int(status)).decode()


# --------------------------------------------------------------------------
# Python-side descriptions
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class CacheView:
    offset: int
    layer_stride: int
    block_stride: int
    row_bytes: int

    def c(self) -> pa_cache_view:
        return pa_cache_view(self.offset, self.layer_stride, self.block_stride, self.row_bytes, 0)


@dataclass
class AttnDesc:
    kv_format: int
    num_q_heads: int
    num_kv_heads: int
    qk_dim: int
    v_dim: int
    block_size: int
    num_blocks: int
    k_view: CacheView
    v_view: CacheView | None = None
    k_cache_bytes: int = 0
    v_cache_bytes: int = 0
    layer: int = 0
    partition_size: int = 0
    k_scale: float = 1.0
    v_scale: float = 1.0

    def c(self) -> pa_attn_desc:
        vv = self.v_view.c() if self.v_view is not None else pa_cache_view(0, 0, 0, 0, 0)
        return pa_attn_desc(self.kv_format, self.num_q_heads, self.num_kv_heads, self.qk_dim, self.v_dim,
                            self.block_size, self.layer, self.partition_size, self.num_blocks, self.k_view.c(), vv,
                            self.k_cache_bytes, self.v_cache_bytes, self.k_scale, self.v_scale)


def dense_view(block_size: int, num_kv_heads: int, head_dim: int, elem_bytes: int = 2) -> CacheView:
    """View of a [num_blocks, block_size, num_kv_heads, head_dim] per-layer cache tensor."""
    row = num_kv_heads * head_dim * elem_bytes
    return CacheView(offset=0, layer_stride=0, block_stride=block_size * row, row_bytes=row)


def dense_desc(dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int, num_blocks: int,
               k_cache_bytes: int, v_cache_bytes: int, partition_size: int = 0, k_scale: float = 1.0,
               v_scale: float = 1.0) -> AttnDesc:
    """dtype "f16" / "bf16" (16-bit caches) or "fp8" (E4M3 caches with k_scale / v_scale, bf16 queries)."""
    fmt = {"f16": PA_KV_F16, "bf16": PA_KV_BF16, "fp8": PA_KV_FP8_E4M3}[dtype]
    v = dense_view(block_size, num_kv_heads, head_dim, 1 if dtype == "fp8" else 2)
    return AttnDesc(kv_format=fmt, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, qk_dim=head_dim, v_dim=head_dim, block_size=block_size,
                    num_blocks=num_blocks, k_view=v, v_view=v, k_cache_bytes=k_cache_bytes,
                    v_cache_bytes=v_cache_bytes, partition_size=partition_size, k_scale=k_scale, v_scale=v_scale)


# --------------------------------------------------------------------------
# Calls (names follow the C entry points)
# --------------------------------------------------------------------------

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn: str, status: int):
    if status != PA_OK:
        raise PagedAttentionError(fn, status)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _require_device(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("pa_* calls take device tensors")


def pa_reshape_and_cache(k, slot_mapping, k_cache, k_view: CacheView, layer: int, block_size: int,
                         num_blocks: int, v=None, v_cache=None, v_view: CacheView | None = None, stream=None):
    """Scatter rows of k (and v) into the cache views; rows are k[t] viewed as bytes (k.stride(0) pitch)."""
    _require_device(k, slot_mapping, k_cache, v, v_cache)
    if slot_mapping.dtype.itemsize != 8 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    T = slot_mapping.numel()
    kp = k.stride(0) * k.element_size() if k.dim() > 0 and k.shape[0] > 1 else k_view.row_bytes
    vp = (v.stride(0) * v.element_size() if v.dim() > 0 and v.shape[0] > 1 else v_view.row_bytes) if v is not None else 0
    for name, src, pitch, view in (("k", k, kp, k_view), ("v", v, vp, v_view)):
        if src is None:
            continue
        if not src.is_contiguous() or src.shape[0] < T or _nbytes(src) < (T - 1) * pitch + view.row_bytes:
            raise ValueError(f"{name} must be contiguous with at least num_tokens rows of row_bytes bytes")
    vv = v_view.c() if v_view is not None else pa_cache_view(0, 0, 0, 0, 0)
    st = _lib.pa_reshape_and_cache(_ptr(k), kp, _ptr(v), vp, _ptr(slot_mapping), T, _ptr(k_cache), _nbytes(k_cache),
                                   k_view.c(), _ptr(v_cache), _nbytes(v_cache) if v_cache is not None else 0, vv,
                                   layer, block_size, num_blocks, _stream(stream))
    _check("pa_reshape_and_cache", st)


def pa_quantize_and_cache_mla(latent, rope, slot_mapping, mla_cache, mla_view: CacheView, layer: int,
                              block_size: int, num_blocks: int, index_key=None, index_cache=None,
                              index_view: CacheView | None = None, stream=None):
    """Quantize bf16 latent [T, 512] + RoPE [T, 64] (and indexer key [T, 128]) into the fp8 dual-cache rows."""
    _require_device(latent, rope, slot_mapping, mla_cache, index_key, index_cache)
    if slot_mapping.dtype.itemsize != 8 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    T = slot_mapping.numel()

    def pitch(x, cols):
        if x.dim() != 2 or x.shape[1] != cols or x.element_size() != 2 or x.stride(1) != 1 or x.shape[0] < T:
            raise ValueError(f"expected a [>= {T}, {cols}] 16-bit tensor with unit column stride")
        return x.stride(0) * 2
    lp, rp = pitch(latent, 512), pitch(rope, 64)
    ip = pitch(index_key, 128) if index_key is not None else 0
    iv = index_view.c() if index_view is not None else pa_cache_view(0, 0, 0, 0, 0)
    st = _lib.pa_quantize_and_cache_mla(_ptr(latent), lp, _ptr(rope), rp, _ptr(index_key), ip, _ptr(slot_mapping), T,
                                        _ptr(mla_cache), _nbytes(mla_cache), mla_view.c(), _ptr(index_cache),
                                        _nbytes(index_cache) if index_cache is not None else 0, iv, layer,
                                        block_size, num_blocks, _stream(stream))
    _check("pa_quantize_and_cache_mla", st)


def pa_quantize_and_cache(k, slot_mapping, k_cache, k_view: CacheView, layer: int, block_size: int, num_blocks: int,
                          k_scale: float, src_dtype: str = "bf16", v=None, v_cache=None, v_view: CacheView | None = None,
                          v_scale: float = 1.0, stream=None):
    """Quantize 16-bit K (and V) rows [T, Hkv*D] into FP8 E4M3 cache views (value = code * scale)."""
    _require_device(k, slot_mapping, k_cache, v, v_cache)
    if slot_mapping.dtype.itemsize != 8 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be a contiguous int64 tensor")
    T = slot_mapping.numel()

    def pitch(x, view):
        if x.dim() != 2 or x.element_size() != 2 or x.stride(1) != 1 or x.shape[0] < T or x.shape[1] != view.row_bytes:
            raise ValueError(f"expected a [>= {T}, {view.row_bytes}] 16-bit tensor with unit column stride")
        return x.stride(0) * 2
    kp = pitch(k, k_view)
    vp = pitch(v, v_view) if v is not None else 0
    vv = v_view.c() if v_view is not None else pa_cache_view(0, 0, 0, 0, 0)
    fmt = PA_KV_F16 if src_dtype == "f16" else PA_KV_BF16
    st = _lib.pa_quantize_and_cache(_ptr(k), kp, _ptr(v), vp, fmt, float(k_scale), float(v_scale), _ptr(slot_mapping),
                                    T, _ptr(k_cache), _nbytes(k_cache), k_view.c(), _ptr(v_cache),
                                    _nbytes(v_cache) if v_cache is not None else 0, vv, layer, block_size, num_blocks,
                                    _stream(stream))
    _check("pa_quantize_and_cache", st)


def pa_copy_blocks(block_pairs, k_cache, k_view: CacheView, num_layers: int, block_size: int, num_blocks: int,
                   v_cache=None, v_view: CacheView | None = None, stream=None):
    """Copy each (src, dst) block pair's pages (all num_layers layers) in the K (and V) view."""
    _require_device(block_pairs, k_cache, v_cache)
    if block_pairs.dtype.itemsize != 8 or not block_pairs.is_contiguous() or block_pairs.dim() != 2 \
            or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be a contiguous int64 [n, 2] tensor")
    vv = v_view.c() if v_view is not None else pa_cache_view(0, 0, 0, 0, 0)
    st = _lib.pa_copy_blocks(_ptr(k_cache), _nbytes(k_cache), k_view.c(), _ptr(v_cache),
                             _nbytes(v_cache) if v_cache is not None else 0, vv, _ptr(block_pairs),
                             block_pairs.shape[0], num_layers, block_size, num_blocks, _stream(stream))
    _check("pa_copy_blocks", st)


def pa_decode_workspace_bytes(desc: AttnDesc, num_seqs: int, max_context_len: int) -> int:
    d = desc.c()
    return int(_lib.pa_decode_workspace_bytes(ctypes.byref(d), num_seqs, max_context_len))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int, scale: float,
              desc: AttnDesc, workspace=None, stream=None):
    _require_device(out, q, k_cache, v_cache, block_tables, context_lens, workspace)
    for name, t in (("out", out), ("q", q), ("block_tables", block_tables), ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    d = desc.c()
    B = context_lens.numel()
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = _lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                        block_tables.shape[1], _ptr(context_lens), B, int(max_context_len), float(scale),
                        ctypes.byref(d), _ptr(workspace), ws_bytes, _stream(stream))
    _check("pa_decode", st)


def pa_decode_no_alloc(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len: int, scale: float,
                       desc: AttnDesc, stream=None):
    _require_device(out, q, k_cache, v_cache, block_tables, context_lens)
    for name, t in (("out", out), ("q", q), ("block_tables", block_tables), ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    d = desc.c()
    st = _lib.pa_decode_no_alloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                 block_tables.shape[1], _ptr(context_lens), context_lens.numel(),
                                 int(max_context_len), float(scale), ctypes.byref(d), _stream(stream))
    _check("pa_decode_no_alloc", st)


def pa_prefill_workspace_bytes(desc: AttnDesc, num_seqs: int, total_q: int, max_query_len: int,
                               max_seq_len: int) -> int:
    d = desc.c()
    return int(_lib.pa_prefill_workspace_bytes(ctypes.byref(d), num_seqs, total_q, max_query_len, max_seq_len))


def pa_prefill_chunk(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, max_query_len: int,
                     max_seq_len: int, scale: float, desc: AttnDesc, workspace=None, stream=None):
    _require_device(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc, workspace)
    d = desc.c()
    S = seq_lens.numel()
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = _lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                               block_tables.shape[1], _ptr(seq_lens), _ptr(query_start_loc), S, q.shape[0],
                               int(max_query_len), int(max_seq_len), float(scale), ctypes.byref(d), _ptr(workspace),
                               ws_bytes, _stream(stream))
    _check("pa_prefill_chunk", st)


def pa_indexer_topk(topk_positions, topk_slots, topk_lens, scores, q_index, head_weights, index_cache,
                    index_view: CacheView, layer: int, block_tables, context_lens, max_context_len: int,
                    block_size: int, num_blocks: int, stream=None):
    """Indexer scores (written into scores [B, >= max_context_len] float32) and each sequence's top-k.

    topk_positions / topk_slots: int32 [B, top_k]; topk_lens int32 [B]; q_index bf16 [B, H, 128];
    head_weights float32 [B, H].
    """
    _require_device(topk_positions, topk_slots, topk_lens, scores, q_index, head_weights, index_cache, block_tables,
                    context_lens)
    for name, t in (("topk_positions", topk_positions), ("topk_slots", topk_slots), ("topk_lens", topk_lens),
                    ("q_index", q_index), ("head_weights", head_weights), ("block_tables", block_tables),
                    ("context_lens", context_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scores.dim() != 2 or scores.stride(1) != 1 or scores.element_size() != 4:
        raise ValueError("scores must be a float32 [B, n] tensor with unit column stride")
    B = context_lens.numel()
    top_k = topk_positions.shape[1]
    if topk_slots.shape[1] != top_k or q_index.shape[0] < B or q_index.shape[-1] != 128:
        raise ValueError("inconsistent shapes")
    st = _lib.pa_indexer_topk(_ptr(topk_positions), _ptr(topk_slots), _ptr(topk_lens), top_k, _ptr(scores),
                              scores.stride(0), _ptr(q_index), _ptr(head_weights), q_index.shape[1],
                              _ptr(index_cache), _nbytes(index_cache), index_view.c(), layer, _ptr(block_tables),
                              block_tables.shape[1], _ptr(context_lens), B, int(max_context_len), block_size,
                              num_blocks, _stream(stream))
    _check("pa_indexer_topk", st)


def pa_mla_sparse_decode(out, q, kv_cache, slots, slot_counts, max_count: int, scale: float, desc: AttnDesc,
                         workspace=None, stream=None):
    """MLA decode of sequence b over the rows at slots[b, :slot_counts[b]] (int32 slots [B, n])."""
    _require_device(out, q, kv_cache, slots, slot_counts, workspace)
    for name, t in (("out", out), ("q", q), ("slots", slots), ("slot_counts", slot_counts)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    d = desc.c()
    B = slot_counts.numel()
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = _lib.pa_mla_sparse_decode(_ptr(out), _ptr(q), _ptr(kv_cache), _ptr(slots), slots.shape[1],
                                   _ptr(slot_counts), B, int(max_count), float(scale), ctypes.byref(d),
                                   _ptr(workspace), ws_bytes, _stream(stream))
    _check("pa_mla_sparse_decode", st)

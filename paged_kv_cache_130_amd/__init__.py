"""MI355X-native paged-KV-cache attention: HIP kernels for gfx950 behind the C ABI of include/pa.h.

The package holds the kernels (csrc/), the in-tree build (build.py) and a
ctypes binding (_lib.py) whose functions carry the C entry points' names.
Importing it loads libpa.so; a missing library raises ImportError.
"""

from ._lib import (  # noqa: F401
    AttnDesc,
    CacheView,
    PagedAttentionError,
    PA_KV_BF16,
    PA_KV_F16,
    PA_KV_FP8_E4M3,
    PA_KV_MLA656_E4M3,
    abi_version,
    dense_desc,
    dense_view,
    pa_copy_blocks,
    pa_decode,
    pa_decode_no_alloc,
    pa_decode_workspace_bytes,
    pa_indexer_topk,
    pa_mla_sparse_decode,
    pa_prefill_chunk,
    pa_prefill_workspace_bytes,
    pa_quantize_and_cache,
    pa_quantize_and_cache_mla,
    pa_reshape_and_cache,
    status_string,
)

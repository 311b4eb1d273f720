// reshape_and_cache: scatter new K/V rows into paged cache views through slot_mapping.
//
// Page "vLLM KV Cache Layout 可视化", kernel section: the write kernel receives only its
// layer's view (offset and layer already folded into the start address). It splits each slot
// into block = slot / block_size and position = slot % block_size, and writes the row at
// start + block*block_stride + position*row width. Several views (the DSA MLA and indexer
// caches) take the same slot_mapping and land at different addresses.
//
// The copy is bit-exact: rows move as 16-byte or 4-byte words. One wave copies one row, so a
// work-group of 4 waves covers 4 tokens of one view; blockIdx.y selects the view.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
    const int view = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= p.num_tokens) return;
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) return;  // padding token, or out of range: no write
    int64_t block, pos;
    if (p.num_slots <= 0x7FFFFFFF) {
        const uint32_t s32 = (uint32_t)slot;
        block = s32 / (uint32_t)p.block_size;
        pos = s32 - (uint32_t)block * (uint32_t)p.block_size;
    } else {
        block = slot / p.block_size;
        pos = slot - block * p.block_size;
    }
    const int row = p.row_bytes[view];
    char* dst = p.dst[view] + block * p.block_stride[view] + pos * (int64_t)row;
    const char* src = p.src[view] + (int64_t)t * p.pitch[view];
    if (p.vec16[view]) {
        const int n = row >> 4;
        for (int i = lane; i < n; i += 64)
            reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else {
        const int n = row >> 2;
        for (int i = lane; i < n; i += 64)
            reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
    }
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
    if (p.num_tokens <= 0) return hipSuccess;
    dim3 grid((p.num_tokens + 3) / 4, p.num_views);
    hipLaunchKernelGGL(cache_write_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

// Host side of the C ABI in include/pa.h: argument validation, kernel selection, launch.
// Every check runs before anything is enqueued; no call reads device memory on the host.

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/pa.h"
#include "pa_internal.h"

// Scratch of pa_decode_no_alloc: the split-context partials of its kernels, one copy per GPU,
// held until the process ends. Host code must not use this name as a device address (it names a
// host-side stand-in); it uses the per-device address from hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[PA_STATIC_SCRATCH_BYTES];

namespace {

thread_local int32_t g_last_hip_error = 0;

int32_t hip_status(hipError_t e) {
    if (e == hipSuccess) return PA_OK;
    g_last_hip_error = (int32_t)e;
    return PA_ERR_HIP;
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }
bool aligned(int64_t v, int64_t a) { return (v & (a - 1)) == 0; }

// A view is well formed when its fields are non-negative, its rows are non-empty, one block's rows
// fit in a block stride (so blocks do not overlap), and every row of `layer` for blocks
// [0, num_blocks) lies inside [0, cache_bytes).
int32_t check_view(const pa_cache_view& v, int32_t layer, int64_t num_blocks, int32_t block_size,
                   int64_t cache_bytes) {
    if (v.reserved != 0 || v.offset < 0 || v.layer_stride < 0 || v.block_stride < 0 || v.row_bytes <= 0)
        return PA_ERR_INVALID_ARGUMENT;
    if (layer < 0 || num_blocks <= 0 || block_size <= 0 || cache_bytes <= 0) return PA_ERR_INVALID_ARGUMENT;
    const __int128 page = (__int128)block_size * v.row_bytes;
    if (num_blocks > 1 && page > v.block_stride) return PA_ERR_INVALID_ARGUMENT;
    const __int128 end = (__int128)v.offset + (__int128)layer * v.layer_stride +
                         (__int128)(num_blocks - 1) * v.block_stride + page;
    if (end > cache_bytes) return PA_ERR_VIEW_OUT_OF_RANGE;
    return PA_OK;
}

bool view_aligned(const pa_cache_view& v, int32_t layer, int64_t a) {
    return aligned(v.offset, a) && aligned((int64_t)layer * v.layer_stride, a) && aligned(v.block_stride, a) &&
           aligned((int64_t)v.row_bytes, a);
}

constexpr int32_t kMaxBlockSize = 256;
// Decode waves resident at once on an MI355X (256 CUs x 4 SIMDs x 2 waves of the decode kernels).
constexpr int64_t kResidentWaves = 2048;

// Block sizes are powers of two from 16 to 256, so that token -> (block, row) is a shift and a mask.
bool block_size_ok(int32_t bs) { return bs >= 16 && bs <= kMaxBlockSize && (bs & (bs - 1)) == 0; }

int32_t log2_int(int32_t v) {
    int32_t r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

// Tokens per split-context partition. A requested size is a multiple of block_size; partitions are
// capped at 64 blocks, because a partition's block ids are held one per lane of a wave.
//
// The automatic size (partition_size 0), rounded to whole blocks, counts the call's work items as
// num_kv_heads * num_seqs * ceil(max_context_len / P) (an upper bound): 1024 tokens when that is at
// least 4 items per resident wave, else the largest of 768, 512 and 256 giving at least one item per
// resident wave, else 256. Large partitions mean fewer item starts and fewer partials to merge; the
// work list runs the short partial partitions last, so they leave no ragged end as long as the
// items are several times the waves. (Measured on one MI355X: the 2000-token-prompt GQA-8 batch
// runs at 70.0 / 74.4 / 75.1% of HBM with partitions of 512 / 768 / 1024, the 13B MHA batch at
// 78.1 / 78.8 / 75.9%.) It depends only on host-known sizes, so the workspace query and the call
// agree on every device.
int32_t effective_partition(const pa_attn_desc& d, int32_t num_seqs, int32_t max_context_len) {
    const int32_t bs = d.block_size;
    const int32_t cap = 64 * bs;
    auto whole_blocks = [&](int64_t t) {
        int64_t P = t < bs ? bs : t - t % bs;
        return (int32_t)(P > cap ? cap : P);
    };
    if (d.partition_size > 0) return whole_blocks(d.partition_size);
    const int64_t pairs = (int64_t)(d.num_kv_heads > 0 ? d.num_kv_heads : 1) * (num_seqs > 0 ? num_seqs : 1);
    auto items = [&](int32_t P) { return pairs * (((int64_t)max_context_len + P - 1) / P); };
    if (items(whole_blocks(1024)) >= 4 * kResidentWaves) return whole_blocks(1024);
    for (int64_t t : {768, 512}) {
        const int32_t P = whole_blocks(t);
        if (items(P) >= kResidentWaves) return P;
    }
    return whole_blocks(256);
}

// Wave items per stored K/V head in the vector decode kernels: eight query heads per K/V head at
// head_dim 64 or 256 take two waves of four (decode_dense.hip, decode_fp8.hip).
int64_t kv_waves(const pa_attn_desc& d) {
    return (d.qk_dim != 128 && d.num_q_heads == 8 * d.num_kv_heads) ? 2 : 1;
}

int32_t check_dense_desc(const pa_attn_desc& d) {
    if (d.kv_format != PA_KV_F16 && d.kv_format != PA_KV_BF16 && d.kv_format != PA_KV_FP8_E4M3)
        return PA_ERR_UNSUPPORTED;
    const bool fp8 = d.kv_format == PA_KV_FP8_E4M3;
    if (fp8 && !(std::isfinite(d.k_scale) && d.k_scale > 0.f && std::isfinite(d.v_scale) && d.v_scale > 0.f))
        return PA_ERR_INVALID_ARGUMENT;
    if (d.num_q_heads <= 0 || d.num_kv_heads <= 0 || d.num_q_heads % d.num_kv_heads != 0)
        return PA_ERR_INVALID_ARGUMENT;
    if (d.qk_dim != d.v_dim) return PA_ERR_INVALID_ARGUMENT;
    if (d.qk_dim != 64 && d.qk_dim != 128 && d.qk_dim != 256) return PA_ERR_UNSUPPORTED;
    // Group sizes: any of 1..16 at head_dim 128 (matrix-core kernel for 2..16); 1, 2, 4 or 8 otherwise.
    const int32_t g = d.num_q_heads / d.num_kv_heads;
    const bool g_ok = d.qk_dim == 128 ? (g >= 1 && g <= 16) : (g == 1 || g == 2 || g == 4 || g == 8);
    if (!g_ok) return PA_ERR_UNSUPPORTED;
    if (!block_size_ok(d.block_size)) return PA_ERR_UNSUPPORTED;
    if (d.partition_size < 0 || (d.partition_size > 0 && d.partition_size % d.block_size != 0))
        return PA_ERR_INVALID_ARGUMENT;
    const int64_t row = (int64_t)d.num_kv_heads * d.qk_dim * (fp8 ? 1 : 2);
    if (d.k_view.row_bytes != row || d.v_view.row_bytes != row) return PA_ERR_INVALID_ARGUMENT;
    int32_t st = check_view(d.k_view, d.layer, d.num_blocks, d.block_size, d.k_cache_bytes);
    if (st != PA_OK) return st;
    st = check_view(d.v_view, d.layer, d.num_blocks, d.block_size, d.v_cache_bytes);
    if (st != PA_OK) return st;
    if (!view_aligned(d.k_view, d.layer, 16) || !view_aligned(d.v_view, d.layer, 16)) return PA_ERR_MISALIGNED;
    if (d.num_blocks > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;  // block ids are int32
    return PA_OK;
}

constexpr int32_t kMlaRowBytes = 656;  // 512 e4m3 latent + 4 float32 scales + 64 bf16 RoPE
constexpr int32_t kIndexRowBytes = 132;  // 128 e4m3 key values + 1 float32 scale
constexpr int32_t kMlaUnit = 32;       // tokens per MLA work unit

int32_t check_mla_desc(const pa_attn_desc& d) {
    if (d.num_kv_heads != 1 || d.qk_dim != 576 || d.v_dim != 512) return PA_ERR_INVALID_ARGUMENT;
    if (d.num_q_heads <= 0 || d.num_q_heads % 16 != 0) return PA_ERR_UNSUPPORTED;
    if (!block_size_ok(d.block_size)) return PA_ERR_UNSUPPORTED;
    if (d.partition_size < 0 || d.partition_size % kMlaUnit != 0) return PA_ERR_INVALID_ARGUMENT;
    if (d.k_view.row_bytes != kMlaRowBytes) return PA_ERR_INVALID_ARGUMENT;
    const int32_t st = check_view(d.k_view, d.layer, d.num_blocks, d.block_size, d.k_cache_bytes);
    if (st != PA_OK) return st;
    if (!view_aligned(d.k_view, d.layer, 16)) return PA_ERR_MISALIGNED;
    if (d.num_blocks > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

// Compute units of the current device (cached per device; 1 if the query fails).
int32_t device_cus() {
    static std::atomic<int32_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 1;
    if (dev >= 0 && dev < 64) {
        const int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// MLA work split: heads per work-group, work-groups along the unit stream, and the partial slots
// (num_seqs + num_wgs) the workspace holds. The grid is sized from the host bound on the units
// (num_seqs * ceil(max_context_len / 32)); the kernel computes the exact split from context_lens.
struct MlaLayout {
    int32_t heads_per_wg;
    int32_t groups;
    int32_t num_wgs;
    int32_t units_per_wg;  // 0: balanced over num_wgs
    int64_t slots;
};

bool mla_layout(const pa_attn_desc& d, int32_t num_seqs, int32_t max_context_len, MlaLayout& L) {
    const int32_t hq = d.num_q_heads;
    L.heads_per_wg = hq % 64 == 0 ? 64 : hq % 32 == 0 ? 32 : 16;
    L.groups = hq / L.heads_per_wg;
    const int64_t units_max = std::max<int64_t>(1, (int64_t)num_seqs * ((max_context_len + kMlaUnit - 1) / kMlaUnit));
    int64_t wgs;
    if (d.partition_size > 0) {
        L.units_per_wg = d.partition_size / kMlaUnit;
        wgs = (units_max + L.units_per_wg - 1) / L.units_per_wg;
    } else {
        L.units_per_wg = 0;
        wgs = std::min<int64_t>(std::max(1, device_cus() / L.groups), units_max);
    }
    if (units_max + L.units_per_wg + wgs > 0x7FFFFFFFLL || L.groups > 65535) return false;
    L.num_wgs = (int32_t)wgs;
    L.slots = (int64_t)num_seqs + wgs;
    return true;
}

size_t mla_decode_ws(const MlaLayout& L, int32_t num_q_heads, int32_t num_seqs) {
    return (size_t)L.slots * num_q_heads * (512 * sizeof(uint16_t) + 2 * sizeof(float)) +
           (size_t)num_seqs * 2 * sizeof(int32_t);
}

// Device address of `scratch` on the device that runs `stream`, resolved once per device (with that
// device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

int32_t static_scratch(void* stream, void** addr) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e);
    int dev = cur;
    if (stream != nullptr) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
        if (e != hipSuccess) return hip_status(e);
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (dev != cur) {
                const hipError_t e2 = hipSetDevice(cur);
                if (e == hipSuccess) e = e2;
            }
            if (e != hipSuccess || p == nullptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol);
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return PA_OK;
}

// The workspace of a decode call: the caller's (checked against `need`), or, for
// pa_decode_no_alloc, the static scratch of the stream's device (need <= PA_STATIC_SCRATCH_BYTES).
// Runs after every other argument check, so a rejected call never touches the device.
int32_t take_workspace(size_t need, bool no_alloc, void* stream, void*& workspace, size_t& workspace_bytes) {
    if (no_alloc) {
        workspace = nullptr;
        workspace_bytes = 0;
        if (need == 0) return PA_OK;
        if (need > PA_STATIC_SCRATCH_BYTES) return PA_ERR_SCRATCH_LIMIT;
        workspace_bytes = PA_STATIC_SCRATCH_BYTES;
        return static_scratch(stream, &workspace);
    }
    if (need == 0) return PA_OK;
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return PA_ERR_MISALIGNED;
    return PA_OK;
}

// The MLA decode, dense (through block_tables) or sparse (through slots); the descriptor and the
// common pointers are already checked.
int32_t mla_decode_call(void* out, const void* q, const void* k_cache, const int32_t* block_tables,
                        int32_t bt_stride, const int32_t* slots, int64_t slot_stride, const int32_t* lens,
                        int32_t num_seqs, int32_t max_len, float scale, const pa_attn_desc& d, void* workspace,
                        size_t workspace_bytes, bool no_alloc, void* stream) {
    MlaLayout L;
    if (!mla_layout(d, num_seqs, max_len, L)) return PA_ERR_UNSUPPORTED;
    const size_t need = mla_decode_ws(L, d.num_q_heads, num_seqs);
    const int32_t st = take_workspace(need, no_alloc, stream, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    pa::MlaDecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.out = out;
    p.q = q;
    p.kv = static_cast<const char*>(k_cache) + d.k_view.offset + (int64_t)d.layer * d.k_view.layer_stride;
    p.block_tables = block_tables;
    p.context_lens = lens;
    // Workspace: bf16 partial outputs [slots, Hq, 512], then fp32 (m, l) [slots, Hq, 2], then the
    // sequences' first and last work-groups.
    p.part_acc = static_cast<uint16_t*>(workspace);
    p.part_ml = reinterpret_cast<float*>(p.part_acc + L.slots * d.num_q_heads * 512);
    p.seq_meta = reinterpret_cast<int32_t*>(p.part_ml + L.slots * d.num_q_heads * 2);
    p.block_stride = d.k_view.block_stride;
    p.num_blocks = d.num_blocks;
    p.bt_stride = bt_stride;
    p.num_seqs = num_seqs;
    p.num_q_heads = d.num_q_heads;
    p.heads_per_wg = L.heads_per_wg;
    p.block_size = d.block_size;
    p.block_size_log2 = log2_int(d.block_size);
    p.max_context_len = max_len;
    p.num_wgs = L.num_wgs;
    p.units_per_wg = L.units_per_wg;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.slots = slots;
    p.slot_stride = slot_stride;
    p.num_slots = d.num_blocks * d.block_size;
    return hip_status(pa::launch_decode_mla(p, static_cast<hipStream_t>(stream)));
}

size_t dense_decode_ws(const pa_attn_desc& d, int32_t num_seqs, int32_t max_context_len) {
    const int32_t P = effective_partition(d, num_seqs, max_context_len);
    const int64_t parts = ((int64_t)max_context_len + P - 1) / P;
    if (parts <= 1 || num_seqs <= 0) return 0;
    const int64_t n = (int64_t)num_seqs * d.num_q_heads * parts;
    return (size_t)(n * 2 + n * d.v_dim) * sizeof(float);
}

}  // namespace

extern "C" {

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_string(int32_t s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_NULL_POINTER: return "null pointer";
        case PA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported format or shape";
        case PA_ERR_MISALIGNED: return "misaligned pointer, stride or row width";
        case PA_ERR_VIEW_OUT_OF_RANGE: return "cache view reaches past the allocation";
        case PA_ERR_WORKSPACE: return "workspace missing or too small";
        case PA_ERR_HIP: return "HIP launch failed";
        case PA_ERR_SCRATCH_LIMIT: return "call needs more than the library's static scratch";
        default: return "unknown status";
    }
}

int32_t pa_last_hip_error(void) { return g_last_hip_error; }

int32_t pa_reshape_and_cache(const void* k, int64_t k_pitch, const void* v, int64_t v_pitch,
                             const int64_t* slot_mapping, int32_t num_tokens, void* k_cache, int64_t k_cache_bytes,
                             pa_cache_view k_view, void* v_cache, int64_t v_cache_bytes, pa_cache_view v_view,
                             int32_t layer, int32_t block_size, int64_t num_blocks, void* stream) {
    if (num_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return PA_OK;
    if (!k || !slot_mapping || !k_cache) return PA_ERR_NULL_POINTER;
    if (v && !v_cache) return PA_ERR_NULL_POINTER;
    if (block_size <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_blocks > INT64_MAX / block_size) return PA_ERR_INVALID_ARGUMENT;
    const int nviews = v ? 2 : 1;
    const void* src[2] = {k, v};
    const int64_t pitch[2] = {k_pitch, v_pitch};
    void* base[2] = {k_cache, v_cache};
    const int64_t bytes[2] = {k_cache_bytes, v_cache_bytes};
    const pa_cache_view* view[2] = {&k_view, &v_view};
    pa::CacheWriteParams p;
    std::memset(&p, 0, sizeof(p));
    for (int i = 0; i < nviews; ++i) {
        int32_t st = check_view(*view[i], layer, num_blocks, block_size, bytes[i]);
        if (st != PA_OK) return st;
        if (pitch[i] < view[i]->row_bytes) return PA_ERR_INVALID_ARGUMENT;
        const bool a4 = aligned(src[i], 4) && aligned(base[i], 4) && aligned(pitch[i], 4) &&
                        view_aligned(*view[i], layer, 4);
        if (!a4) return PA_ERR_MISALIGNED;
        const bool a16 = aligned(src[i], 16) && aligned(base[i], 16) && aligned(pitch[i], 16) &&
                         view_aligned(*view[i], layer, 16);
        p.src[i] = static_cast<const char*>(src[i]);
        p.pitch[i] = pitch[i];
        p.dst[i] = static_cast<char*>(base[i]) + view[i]->offset + (int64_t)layer * view[i]->layer_stride;
        p.block_stride[i] = view[i]->block_stride;
        p.row_bytes[i] = view[i]->row_bytes;
        p.vec16[i] = a16 ? 1 : 0;
    }
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_views = nviews;
    p.block_size = block_size;
    p.num_slots = num_blocks * block_size;
    return hip_status(pa::launch_cache_write(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_quantize_and_cache_mla(const void* latent, int64_t latent_pitch, const void* rope, int64_t rope_pitch,
                                  const void* index_key, int64_t index_pitch, const int64_t* slot_mapping,
                                  int32_t num_tokens, void* mla_cache, int64_t mla_cache_bytes, pa_cache_view mla_view,
                                  void* index_cache, int64_t index_cache_bytes, pa_cache_view index_view,
                                  int32_t layer, int32_t block_size, int64_t num_blocks, void* stream) {
    if (num_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return PA_OK;
    if (!latent || !rope || !slot_mapping || !mla_cache) return PA_ERR_NULL_POINTER;
    if (index_key && !index_cache) return PA_ERR_NULL_POINTER;
    if (block_size <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_blocks > INT64_MAX / block_size) return PA_ERR_INVALID_ARGUMENT;
    if (mla_view.row_bytes != kMlaRowBytes) return PA_ERR_INVALID_ARGUMENT;
    if (latent_pitch < 512 * 2 || rope_pitch < 64 * 2) return PA_ERR_INVALID_ARGUMENT;
    int32_t st = check_view(mla_view, layer, num_blocks, block_size, mla_cache_bytes);
    if (st != PA_OK) return st;
    if (!aligned(latent, 16) || !aligned(rope, 16) || !aligned(latent_pitch, 16) || !aligned(rope_pitch, 16) ||
        !aligned(mla_cache, 16) || !view_aligned(mla_view, layer, 16))
        return PA_ERR_MISALIGNED;
    pa::QuantWriteParams p;
    std::memset(&p, 0, sizeof(p));
    if (index_key) {
        if (index_view.row_bytes != kIndexRowBytes) return PA_ERR_INVALID_ARGUMENT;
        if (index_pitch < 128 * 2) return PA_ERR_INVALID_ARGUMENT;
        st = check_view(index_view, layer, num_blocks, block_size, index_cache_bytes);
        if (st != PA_OK) return st;
        if (!aligned(index_key, 16) || !aligned(index_pitch, 16) || !aligned(index_cache, 4) ||
            !view_aligned(index_view, layer, 4))
            return PA_ERR_MISALIGNED;
        p.index_key = static_cast<const char*>(index_key);
        p.index_pitch = index_pitch;
        p.idx_dst = static_cast<char*>(index_cache) + index_view.offset + (int64_t)layer * index_view.layer_stride;
        p.idx_block_stride = index_view.block_stride;
    }
    p.latent = static_cast<const char*>(latent);
    p.latent_pitch = latent_pitch;
    p.rope = static_cast<const char*>(rope);
    p.rope_pitch = rope_pitch;
    p.slots = slot_mapping;
    p.mla_dst = static_cast<char*>(mla_cache) + mla_view.offset + (int64_t)layer * mla_view.layer_stride;
    p.mla_block_stride = mla_view.block_stride;
    p.num_slots = num_blocks * block_size;
    p.num_tokens = num_tokens;
    p.block_size = block_size;
    return hip_status(pa::launch_quant_cache_write(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_quantize_and_cache(const void* k, int64_t k_pitch, const void* v, int64_t v_pitch, int32_t src_format,
                              float k_scale, float v_scale, const int64_t* slot_mapping, int32_t num_tokens,
                              void* k_cache, int64_t k_cache_bytes, pa_cache_view k_view, void* v_cache,
                              int64_t v_cache_bytes, pa_cache_view v_view, int32_t layer, int32_t block_size,
                              int64_t num_blocks, void* stream) {
    if (num_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return PA_OK;
    if (!k || !slot_mapping || !k_cache) return PA_ERR_NULL_POINTER;
    if (v && !v_cache) return PA_ERR_NULL_POINTER;
    if (src_format != PA_KV_F16 && src_format != PA_KV_BF16) return PA_ERR_UNSUPPORTED;
    if (block_size <= 0 || num_blocks <= 0 || num_blocks > INT64_MAX / block_size) return PA_ERR_INVALID_ARGUMENT;
    const int nviews = v ? 2 : 1;
    const void* src[2] = {k, v};
    const int64_t pitch[2] = {k_pitch, v_pitch};
    void* base[2] = {k_cache, v_cache};
    const int64_t bytes[2] = {k_cache_bytes, v_cache_bytes};
    const pa_cache_view* view[2] = {&k_view, &v_view};
    const float scale[2] = {k_scale, v_scale};
    pa::QuantDenseParams p;
    std::memset(&p, 0, sizeof(p));
    for (int i = 0; i < nviews; ++i) {
        if (!std::isfinite(scale[i]) || !(scale[i] > 0.f)) return PA_ERR_INVALID_ARGUMENT;
        int32_t st = check_view(*view[i], layer, num_blocks, block_size, bytes[i]);
        if (st != PA_OK) return st;
        if (view[i]->row_bytes != k_view.row_bytes || view[i]->row_bytes % 8 != 0) return PA_ERR_INVALID_ARGUMENT;
        if (pitch[i] < 2 * (int64_t)view[i]->row_bytes) return PA_ERR_INVALID_ARGUMENT;
        if (!aligned(src[i], 16) || !aligned(pitch[i], 16) || !aligned(base[i], 8) || !view_aligned(*view[i], layer, 8))
            return PA_ERR_MISALIGNED;
        p.src[i] = static_cast<const char*>(src[i]);
        p.pitch[i] = pitch[i];
        p.dst[i] = static_cast<char*>(base[i]) + view[i]->offset + (int64_t)layer * view[i]->layer_stride;
        p.block_stride[i] = view[i]->block_stride;
        p.scale[i] = scale[i];
        p.inv_scale[i] = 1.0f / scale[i];  // IEEE float division on the host: correctly rounded
    }
    p.slots = slot_mapping;
    p.num_slots = num_blocks * block_size;
    p.row_values = k_view.row_bytes;
    p.num_tokens = num_tokens;
    p.num_views = nviews;
    p.block_size = block_size;
    p.src_f16 = src_format == PA_KV_F16;
    return hip_status(pa::launch_quant_dense_write(p, static_cast<hipStream_t>(stream)));
}

int32_t pa_copy_blocks(void* k_cache, int64_t k_cache_bytes, pa_cache_view k_view, void* v_cache,
                       int64_t v_cache_bytes, pa_cache_view v_view, const int64_t* block_pairs, int32_t num_pairs,
                       int32_t num_layers, int32_t block_size, int64_t num_blocks, void* stream) {
    if (num_pairs < 0 || num_layers < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_pairs == 0 || num_layers == 0) return PA_OK;
    if (!k_cache || !block_pairs) return PA_ERR_NULL_POINTER;
    if (block_size <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARGUMENT;
    if ((int64_t)num_pairs * num_layers > 0x7FFFFFFFLL) return PA_ERR_UNSUPPORTED;
    if (!aligned(block_pairs, 8)) return PA_ERR_MISALIGNED;
    void* base[2] = {k_cache, v_cache};
    const int64_t bytes[2] = {k_cache_bytes, v_cache_bytes};
    const pa_cache_view* view[2] = {&k_view, &v_view};
    const int nviews = v_cache ? 2 : 1;
    pa::BlockCopyParams p;
    std::memset(&p, 0, sizeof(p));
    for (int i = 0; i < nviews; ++i) {
        // The last layer's pages must lie inside the allocation.
        int32_t st = check_view(*view[i], num_layers - 1, num_blocks, block_size, bytes[i]);
        if (st != PA_OK) return st;
        if (!aligned(base[i], 4) || !view_aligned(*view[i], 0, 4) || !aligned(view[i]->layer_stride, 4))
            return PA_ERR_MISALIGNED;
        p.base[i] = static_cast<char*>(base[i]) + view[i]->offset;
        p.layer_stride[i] = view[i]->layer_stride;
        p.block_stride[i] = view[i]->block_stride;
        p.page_bytes[i] = (int64_t)block_size * view[i]->row_bytes;
        p.vec16[i] = aligned(base[i], 16) && view_aligned(*view[i], 0, 16) && aligned(view[i]->layer_stride, 16);
    }
    p.pairs = block_pairs;
    p.num_blocks = num_blocks;
    p.num_pairs = num_pairs;
    p.num_layers = num_layers;
    p.num_views = nviews;
    return hip_status(pa::launch_block_copy(p, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_workspace_bytes(const pa_attn_desc* desc, int32_t num_seqs, int32_t max_context_len) {
    if (!desc || num_seqs <= 0 || max_context_len <= 0) return 0;
    if (desc->kv_format == PA_KV_F16 || desc->kv_format == PA_KV_BF16 || desc->kv_format == PA_KV_FP8_E4M3) {
        if (!block_size_ok(desc->block_size)) return 0;
        return dense_decode_ws(*desc, num_seqs, max_context_len);
    }
    if (desc->kv_format == PA_KV_MLA656_E4M3) {
        if (check_mla_desc(*desc) != PA_OK) return 0;
        MlaLayout L;
        if (!mla_layout(*desc, num_seqs, max_context_len, L)) return 0;
        return mla_decode_ws(L, desc->num_q_heads, num_seqs);
    }
    return 0;
}

}  // extern "C"

namespace {

// pa_decode and pa_decode_no_alloc: every argument check, then the workspace (the caller's or the
// static scratch), then the launches.
int32_t decode_entry(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_context_len, float scale, const pa_attn_desc* desc, void* workspace,
                     size_t workspace_bytes, bool no_alloc, void* stream) {
    if (!desc) return PA_ERR_NULL_POINTER;
    if (num_seqs < 0 || max_context_len < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !k_cache || !block_tables || !context_lens) return PA_ERR_NULL_POINTER;
    if (bt_stride <= 0 || !std::isfinite(scale) || scale < 0.f) return PA_ERR_INVALID_ARGUMENT;
    const pa_attn_desc& d = *desc;
    const bool mla = d.kv_format == PA_KV_MLA656_E4M3;
    int32_t st = mla ? check_mla_desc(d) : check_dense_desc(d);
    if (st != PA_OK) return st;
    if (!mla && !v_cache) return PA_ERR_NULL_POINTER;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || (!mla && !aligned(v_cache, 16)) ||
        !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return PA_ERR_MISALIGNED;
    if (mla)
        return mla_decode_call(out, q, k_cache, block_tables, bt_stride, nullptr, 0, context_lens, num_seqs,
                               max_context_len, scale, d, workspace, workspace_bytes, no_alloc, stream);
    const int32_t P = effective_partition(d, num_seqs, max_context_len);
    const int64_t max_parts64 = ((int64_t)max_context_len + P - 1) / P;
    const int32_t max_parts = max_parts64 < 1 ? 1 : (int32_t)max_parts64;
    if ((int64_t)d.num_kv_heads * kv_waves(d) * num_seqs * max_parts > 0x7FFFFFFFLL - 64) return PA_ERR_UNSUPPORTED;
    const size_t need = dense_decode_ws(d, num_seqs, max_context_len);
    st = take_workspace(need, no_alloc, stream, workspace, workspace_bytes);
    if (st != PA_OK) return st;

    pa::DenseDecodeParams p;
    std::memset(&p, 0, sizeof(p));
    p.out = out;
    p.q = q;
    p.k = static_cast<const char*>(k_cache) + d.k_view.offset + (int64_t)d.layer * d.k_view.layer_stride;
    p.v = static_cast<const char*>(v_cache) + d.v_view.offset + (int64_t)d.layer * d.v_view.layer_stride;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    const int64_t n = (int64_t)num_seqs * d.num_q_heads * max_parts;
    p.part_ml = need > 0 ? static_cast<float*>(workspace) : nullptr;
    p.part_acc = need > 0 ? static_cast<float*>(workspace) + 2 * n : nullptr;
    p.k_block_stride = d.k_view.block_stride;
    p.v_block_stride = d.v_view.block_stride;
    p.num_blocks = d.num_blocks;
    p.k_row_bytes = d.k_view.row_bytes;
    p.v_row_bytes = d.v_view.row_bytes;
    p.bt_stride = bt_stride;
    p.num_seqs = num_seqs;
    p.num_q_heads = d.num_q_heads;
    p.num_kv_heads = d.num_kv_heads;
    p.block_size = d.block_size;
    p.tiles_per_block_log2 = log2_int(d.block_size / 16);
    p.partition_tokens = P;
    p.max_parts = max_parts;
    p.max_context_len = max_context_len;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.is_bf16 = d.kv_format != PA_KV_F16;  // FP8 rows take bf16 queries and outputs
    p.head_dim = d.v_dim;
    p.group = d.num_q_heads / d.num_kv_heads;
    p.kv_fp8 = d.kv_format == PA_KV_FP8_E4M3;
    p.v_scale = p.kv_fp8 ? d.v_scale : 1.f;
    if (p.kv_fp8) p.scale_log2 = scale * d.k_scale * 1.4426950408889634f;
    return hip_status(pa::launch_decode_dense(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int32_t pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                  int32_t bt_stride, const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                  float scale, const pa_attn_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
    return decode_entry(out, q, k_cache, v_cache, block_tables, bt_stride, context_lens, num_seqs, max_context_len,
                        scale, desc, workspace, workspace_bytes, false, stream);
}

int32_t pa_decode_no_alloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                           int32_t num_seqs, int32_t max_context_len, float scale, const pa_attn_desc* desc,
                           void* stream) {
    return decode_entry(out, q, k_cache, v_cache, block_tables, bt_stride, context_lens, num_seqs, max_context_len,
                        scale, desc, nullptr, 0, true, stream);
}

size_t pa_prefill_workspace_bytes(const pa_attn_desc* desc, int32_t num_seqs, int32_t total_q,
                                  int32_t max_query_len, int32_t max_seq_len) {
    (void)total_q;
    (void)max_query_len;
    if (!desc || num_seqs <= 0 || max_seq_len <= 0) return 0;
    if (desc->kv_format != PA_KV_F16 && desc->kv_format != PA_KV_BF16) return 0;
    if (!block_size_ok(desc->block_size)) return 0;
    // The decode rows (query length 1) of the call use split-context partials.
    return dense_decode_ws(*desc, num_seqs, max_seq_len);
}

int32_t pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t total_q, int32_t max_query_len,
                         int32_t max_seq_len, float scale, const pa_attn_desc* desc, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!desc) return PA_ERR_NULL_POINTER;
    if (num_seqs < 0 || total_q < 0 || max_query_len < 0 || max_seq_len < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0 || total_q == 0) return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc)
        return PA_ERR_NULL_POINTER;
    if (bt_stride <= 0 || !std::isfinite(scale) || scale < 0.f) return PA_ERR_INVALID_ARGUMENT;
    const pa_attn_desc& d = *desc;
    if (d.kv_format == PA_KV_MLA656_E4M3 || d.kv_format == PA_KV_FP8_E4M3) return PA_ERR_UNSUPPORTED;
    int32_t st = check_dense_desc(d);
    if (st != PA_OK) return st;
    if (d.qk_dim != 128) return PA_ERR_UNSUPPORTED;  // causal chunks are implemented for head_dim 128
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(query_start_loc, 4))
        return PA_ERR_MISALIGNED;
    const size_t need = dense_decode_ws(d, num_seqs, max_seq_len);
    st = take_workspace(need, false, stream, workspace, workspace_bytes);
    if (st != PA_OK) return st;
    const int32_t P = effective_partition(d, num_seqs, max_seq_len);
    const int64_t max_parts64 = ((int64_t)max_seq_len + P - 1) / P;
    const int32_t max_parts = max_parts64 < 1 ? 1 : (int32_t)max_parts64;
    if ((int64_t)d.num_kv_heads * kv_waves(d) * num_seqs * max_parts > 0x7FFFFFFFLL - 64) return PA_ERR_UNSUPPORTED;
    if ((int64_t)total_q * d.num_q_heads > 0x7FFFFFFFLL / 2) return PA_ERR_UNSUPPORTED;

    const char* kb = static_cast<const char*>(k_cache) + d.k_view.offset + (int64_t)d.layer * d.k_view.layer_stride;
    const char* vb = static_cast<const char*>(v_cache) + d.v_view.offset + (int64_t)d.layer * d.v_view.layer_stride;

    // 1) Decode rows (query length 1): split-context decode over their whole context.
    pa::DenseDecodeParams dp;
    std::memset(&dp, 0, sizeof(dp));
    dp.out = out;
    dp.q = q;
    dp.k = kb;
    dp.v = vb;
    dp.block_tables = block_tables;
    dp.context_lens = seq_lens;
    dp.query_start_loc = query_start_loc;
    const int64_t n = (int64_t)num_seqs * d.num_q_heads * max_parts;
    dp.part_ml = need > 0 ? static_cast<float*>(workspace) : nullptr;
    dp.part_acc = need > 0 ? static_cast<float*>(workspace) + 2 * n : nullptr;
    dp.k_block_stride = d.k_view.block_stride;
    dp.v_block_stride = d.v_view.block_stride;
    dp.num_blocks = d.num_blocks;
    dp.k_row_bytes = d.k_view.row_bytes;
    dp.v_row_bytes = d.v_view.row_bytes;
    dp.bt_stride = bt_stride;
    dp.num_seqs = num_seqs;
    dp.num_q_heads = d.num_q_heads;
    dp.num_kv_heads = d.num_kv_heads;
    dp.block_size = d.block_size;
    dp.tiles_per_block_log2 = log2_int(d.block_size / 16);
    dp.partition_tokens = P;
    dp.max_parts = max_parts;
    dp.max_context_len = max_seq_len;
    dp.scale_log2 = scale * 1.4426950408889634f;
    dp.is_bf16 = d.kv_format == PA_KV_BF16;
    dp.head_dim = d.qk_dim;
    dp.group = d.num_q_heads / d.num_kv_heads;

    // 2) Chunk rows (query length >= 2): causal attention over the paged context.
    pa::PrefillParams pp;
    std::memset(&pp, 0, sizeof(pp));
    pp.out = out;
    pp.q = q;
    pp.k = kb;
    pp.v = vb;
    pp.block_tables = block_tables;
    pp.seq_lens = seq_lens;
    pp.query_start_loc = query_start_loc;
    pp.k_block_stride = d.k_view.block_stride;
    pp.v_block_stride = d.v_view.block_stride;
    pp.num_blocks = d.num_blocks;
    pp.k_row_bytes = d.k_view.row_bytes;
    pp.v_row_bytes = d.v_view.row_bytes;
    pp.bt_stride = bt_stride;
    pp.num_seqs = num_seqs;
    pp.num_q_heads = d.num_q_heads;
    pp.num_kv_heads = d.num_kv_heads;
    pp.block_size = d.block_size;
    pp.tiles_per_block_log2 = log2_int(d.block_size / 16);
    pp.max_seq_len = max_seq_len;
    pp.max_query_len = max_query_len;
    pp.scale_log2 = dp.scale_log2;
    pp.is_bf16 = dp.is_bf16;
    pp.group = dp.group;
    pp.rows_per_item = 128;
    pp.total_q = total_q;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // Grouped heads at head_dim 128 decode on the matrix cores: one launch takes both kinds of rows.
    if (max_query_len >= 2 && d.qk_dim == 128 && dp.group >= 2) return hip_status(pa::launch_mixed_chunk(pp, dp, s));
    st = hip_status(pa::launch_decode_dense(dp, s));
    if (st != PA_OK || max_query_len < 2) return st;
    return hip_status(pa::launch_prefill_chunk(pp, s));
}

int32_t pa_mla_sparse_decode(void* out, const void* q, const void* kv_cache, const int32_t* slots, int32_t slot_stride,
                             const int32_t* slot_counts, int32_t num_seqs, int32_t max_count, float scale,
                             const pa_attn_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
    if (!desc) return PA_ERR_NULL_POINTER;
    if (num_seqs < 0 || max_count < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return PA_OK;
    if (!out || !q || !kv_cache || !slots || !slot_counts) return PA_ERR_NULL_POINTER;
    if (slot_stride <= 0 || !std::isfinite(scale) || scale < 0.f) return PA_ERR_INVALID_ARGUMENT;
    const pa_attn_desc& d = *desc;
    if (d.kv_format != PA_KV_MLA656_E4M3) return PA_ERR_UNSUPPORTED;
    const int32_t st = check_mla_desc(d);
    if (st != PA_OK) return st;
    if (d.num_blocks * d.block_size > 0x7FFFFFFFLL) return PA_ERR_UNSUPPORTED;  // slots are int32
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(kv_cache, 16) || !aligned(slots, 4) ||
        !aligned(slot_counts, 4))
        return PA_ERR_MISALIGNED;
    return mla_decode_call(out, q, kv_cache, nullptr, 0, slots, slot_stride, slot_counts, num_seqs,
                           std::min(max_count, slot_stride), scale, d, workspace, workspace_bytes, false, stream);
}

int32_t pa_indexer_topk(int32_t* topk_positions, int32_t* topk_slots, int32_t* topk_lens, int32_t top_k, float* scores,
                        int64_t score_stride, const void* q_index, const float* head_weights, int32_t num_index_heads,
                        const void* index_cache, int64_t index_cache_bytes, pa_cache_view index_view, int32_t layer,
                        const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                        int32_t num_seqs, int32_t max_context_len, int32_t block_size, int64_t num_blocks,
                        void* stream) {
    if (num_seqs < 0 || max_context_len < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_seqs == 0) return PA_OK;
    if (!topk_positions || !topk_slots || !topk_lens || !scores || !q_index || !head_weights || !index_cache ||
        !block_tables || !context_lens)
        return PA_ERR_NULL_POINTER;
    if (top_k <= 0 || bt_stride <= 0 || score_stride < std::max(1, max_context_len)) return PA_ERR_INVALID_ARGUMENT;
    if (num_index_heads != 16 && num_index_heads != 32 && num_index_heads != 48 && num_index_heads != 64)
        return PA_ERR_UNSUPPORTED;
    if (!block_size_ok(block_size)) return PA_ERR_UNSUPPORTED;
    if (index_view.row_bytes != kIndexRowBytes) return PA_ERR_INVALID_ARGUMENT;
    const int32_t st = check_view(index_view, layer, num_blocks, block_size, index_cache_bytes);
    if (st != PA_OK) return st;
    if (num_blocks * block_size > 0x7FFFFFFFLL) return PA_ERR_UNSUPPORTED;  // slots are int32
    if ((int64_t)num_seqs * top_k > 0x7FFFFFFFLL || (int64_t)num_seqs > 0x7FFFFFFFLL / 64) return PA_ERR_UNSUPPORTED;
    if (!aligned(q_index, 16) || !aligned(index_cache, 16) || !view_aligned(index_view, layer, 4) ||
        !aligned(index_view.offset, 16) || !aligned((int64_t)layer * index_view.layer_stride, 16) ||
        !aligned(index_view.block_stride, 16) ||
        !aligned(head_weights, 4) || !aligned(scores, 4) || !aligned(topk_positions, 4) ||
        !aligned(topk_slots, 4) || !aligned(topk_lens, 4) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
        return PA_ERR_MISALIGNED;
    pa::IndexerParams p;
    std::memset(&p, 0, sizeof(p));
    p.idx = static_cast<const char*>(index_cache) + index_view.offset + (int64_t)layer * index_view.layer_stride;
    p.q = static_cast<const uint16_t*>(q_index);
    p.w = head_weights;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.scores = scores;
    p.topk_pos = topk_positions;
    p.topk_slots = topk_slots;
    p.topk_lens = topk_lens;
    p.score_stride = score_stride;
    p.block_stride = index_view.block_stride;
    p.num_blocks = num_blocks;
    p.bt_stride = bt_stride;
    p.num_seqs = num_seqs;
    p.num_heads = num_index_heads;
    p.block_size = block_size;
    p.block_size_log2 = log2_int(block_size);
    p.max_context_len = max_context_len;
    p.top_k = top_k;
    if ((int64_t)num_seqs * ((max_context_len + 511) / 512) > 0x7FFFFFFFLL) return PA_ERR_UNSUPPORTED;
    return hip_status(pa::launch_indexer_topk(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

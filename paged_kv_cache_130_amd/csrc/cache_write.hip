// reshape_and_cache: scatter new K/V rows into paged cache views through slot_mapping.
//
// Page "vLLM KV Cache Layout 可视化", kernel section: the write kernel receives only its
// layer's view (offset and layer already folded into the start address). It splits each slot
// into block = slot / block_size and position = slot % block_size, and writes the row at
// start + block*block_stride + position*row width. Several views (the DSA MLA and indexer
// caches) take the same slot_mapping and land at different addresses.
//
// The copy is bit-exact: rows move as 16-byte or 4-byte words. The words of all tokens of one view
// form one flat run (token-major); a wave moves one chunk of it, at most 64 x B words touching at
// most 64 tokens, issuing every load of the chunk before its first store. Each lane splits the slot
// of one token of the chunk into block and position and forms that token's destination row; the
// lanes storing a word fetch their token's row address with a cross-lane permute. Source rows are read
// once (nontemporal loads); the stores go through the cache, which merges the parts of a 128-byte
// line that neighbouring rows (656 or 132 bytes, not line-aligned) share before it reaches HBM (with
// nontemporal stores the DSA populate ran at 54% of HBM instead of 69%). blockIdx.y selects the view.

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef unsigned int cw_u32x4 __attribute__((ext_vector_type(4)));

// Words each lane moves per chunk: 8 x 16 bytes or 16 x 4 bytes (8 KB or 4 KB per wave).
template <typename Word>
constexpr int copy_batch() { return sizeof(Word) == 16 ? 8 : 16; }

// Words per chunk for rows of n words: 64 x B, but at most 63 x n so that a chunk touches at most
// 64 tokens (one per lane).
template <typename Word>
__host__ __device__ inline uint32_t chunk_words(uint32_t n) {
    const uint32_t full = 64u * copy_batch<Word>();
    return full < 63u * n ? full : 63u * n;
}

template <typename Word>
__device__ __forceinline__ Word load_nt(const char* ptr) {
    if constexpr (sizeof(Word) == 16) {
        const cw_u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const cw_u32x4*>(ptr));
        return make_uint4(a.x, a.y, a.z, a.w);
    } else {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ptr));
    }
}

template <typename Word>
__device__ __forceinline__ void store_nt(char* ptr, const Word& v) {
    if constexpr (sizeof(Word) == 16) {
        const cw_u32x4 a = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(a, reinterpret_cast<cw_u32x4*>(ptr));
    } else if constexpr (sizeof(Word) == 8) {
        typedef unsigned int u32x2_nt __attribute__((ext_vector_type(2)));
        const u32x2_nt a = {v.x, v.y};
        __builtin_nontemporal_store(a, reinterpret_cast<u32x2_nt*>(ptr));
    } else {
        __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(ptr));
    }
}

template <typename Word>
__device__ __forceinline__ void copy_chunk(const CacheWriteParams& p, int view, int64_t chunk, int lane) {
    constexpr int B = copy_batch<Word>();
    const int row = p.row_bytes[view];
    const uint32_t n = (uint32_t)row / sizeof(Word);  // words per row
    const uint32_t cw = chunk_words<Word>(n);
    const int64_t total = (int64_t)p.num_tokens * n;
    const int64_t j0 = chunk * cw;
    if (j0 >= total) return;
    const uint32_t cnt = (uint32_t)min((int64_t)cw, total - j0);
    const int64_t tok0 = j0 / n;                       // wave-uniform
    const uint32_t w0 = (uint32_t)(j0 - tok0 * n);
    const int ntok = (int)((w0 + cnt + n - 1) / n);    // tokens the chunk touches (<= 64)
    const char* src = p.src[view] + tok0 * p.pitch[view];
    const int64_t pitch = p.pitch[view];
    const float rcp_n = 1.f / (float)n;

    // Lane i: the slot of token tok0 + i, loaded beside the words.
    const int64_t my_slot = lane < ntok ? p.slots[tok0 + lane] : -1;

    Word v[B];
    uint32_t tk[B], wd[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const uint32_t jj = 64u * u + (uint32_t)lane;
        if (jj < cnt) {
            const uint32_t x = w0 + jj;                // < 64 B + n: exact in float
            uint32_t t = (uint32_t)((float)x * rcp_n);
            if (t * n > x) --t;
            else if ((t + 1) * n <= x) ++t;
            tk[u] = t;
            wd[u] = x - t * n;
            v[u] = load_nt<Word>(src + (int64_t)t * pitch + (int64_t)wd[u] * sizeof(Word));
        } else {
            tk[u] = 0;
            wd[u] = 0;
        }
    }
    // Destination row of token tok0 + lane (0 for padding and out-of-range slots).
    uint64_t my_dst = 0;
    if (lane < ntok && my_slot >= 0 && my_slot < p.num_slots) {
        const int64_t block = my_slot / p.block_size;
        my_dst = (uint64_t)(p.dst[view] + block * p.block_stride[view] + (my_slot - block * p.block_size) * (int64_t)row);
    }
    const uint32_t dlo = (uint32_t)my_dst, dhi = (uint32_t)(my_dst >> 32);
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const uint32_t jj = 64u * u + (uint32_t)lane;
        const uint64_t d = (uint64_t)(uint32_t)__shfl((int)dlo, (int)tk[u]) |
                           ((uint64_t)(uint32_t)__shfl((int)dhi, (int)tk[u]) << 32);
        if (jj < cnt && d != 0) *reinterpret_cast<Word*>(reinterpret_cast<char*>(d) + (int64_t)wd[u] * sizeof(Word)) = v[u];
    }
}

}  // namespace

__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
    const int view = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * 4 + wave;
    if (p.vec16[view]) copy_chunk<uint4>(p, view, chunk, lane);
    else copy_chunk<uint32_t>(p, view, chunk, lane);
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
    if (p.num_tokens <= 0) return hipSuccess;
    int64_t chunks = 0;
    for (int v = 0; v < p.num_views; ++v) {
        const uint32_t n = (uint32_t)(p.row_bytes[v] / (p.vec16[v] ? 16 : 4));
        const uint32_t cw = p.vec16[v] ? chunk_words<uint4>(n) : chunk_words<uint32_t>(n);
        const int64_t c = ((int64_t)p.num_tokens * n + cw - 1) / cw;
        chunks = c > chunks ? c : chunks;
    }
    const int64_t wgs = (chunks + 3) / 4;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    dim3 grid((unsigned)wgs, p.num_views);
    hipLaunchKernelGGL(cache_write_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantize-on-write for the DSA dual cache.
//
// "deep dive into vLLM 05" §3.4: the cache can be quantized as it is written and dequantized as it
// is read, FP8 being the safest format; finer scale groups are more accurate. "vLLM KV Cache Layout
// 可视化" (two caches sharing one block table) fixes the rows: 512 B FP8 latent + 16 B scale + 128 B
// BF16 RoPE per MLA token, 128 B FP8 key + 4 B FP32 scale per indexer token. Per group of 128 values
// (4 latent groups, 1 indexer group): scale = amax / 448 in float32, and each value is stored as the
// OCP E4M3 code nearest to x / scale (float32 division), ties to the even mantissa, saturating at
// 448; a group of zeros stores scale 0 and zero codes.
//
// A 16-lane DPP row holds one group (8 values per lane, 16 bytes of bf16), so the group maximum is a
// 4-step row reduction. blockIdx.y = 0 writes MLA rows: a wave takes several tokens in turn, its 4
// DPP rows being the 4 groups of a token (lanes 0..7 also move the 128 RoPE bytes unchanged);
// blockIdx.y = 1 writes indexer rows, 4 tokens per step (one token per DPP row). The quotient is clamped to +-448 and converted by
// v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even): after the clamp every quotient lies inside the
// format's range, where that conversion is exactly the nearest-even rounding the rows are defined by
// (quotients between 448 and 464 round to 448 either way).
// ---------------------------------------------------------------------------

namespace {

// Largest magnitude over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_mov<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_mov<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
    return x;
}

// 16 bytes of bf16 -> 8 fp32 values (exact), the largest magnitude among them. The source is read
// once (nontemporal).
__device__ __forceinline__ float load_bf16x8(const char* src, float (&x)[8]) {
    const uint4 v = load_nt<uint4>(src);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
    }
    return amax;
}

// Codes of 8 values of one group given the group's scale; a zero scale (all-zero group) gives zero
// codes.
//
// The quotients x / scale must be the correctly rounded float32 ones. One correctly rounded division
// gives y = 1 / scale for the group; then per value q0 = x * y is within one unit in the last place
// of x / scale, the remainder x - q0 * scale is exact in one fma, and q0 + remainder * y (one more
// fma) is the correctly rounded quotient (Markstein's correction for round-to-nearest, valid while
// nothing overflows; the quotients here are at most 448 in magnitude, and results too small for
// normal float32 are far below the smallest E4M3 step, so they encode as zero either way). A scale
// below the smallest normal float32 (a group whose largest value is below about 5e-36) would make
// 1 / scale overflow; such groups divide each value directly.
__device__ __forceinline__ uint2 quantize8(const float (&x)[8], float scale) {
    uint32_t w[2] = {0u, 0u};
    if (scale > 0.f) {
        const bool normal = scale >= 1.17549435e-38f;
        const float y = __fdiv_rn(1.f, normal ? scale : 1.f);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float q[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float qq;
                if (normal) {
                    const float q0 = x[4 * h + i] * y;
                    const float rem = __builtin_fmaf(-q0, scale, x[4 * h + i]);
                    qq = __builtin_fmaf(rem, y, q0);
                } else {
                    qq = __fdiv_rn(x[4 * h + i], scale);
                }
                q[i] = fminf(fmaxf(qq, -448.f), 448.f);
            }
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
            w[h] = (uint32_t)v;
        }
    }
    return make_uint2(w[0], w[1]);
}

}  // namespace

// Tokens per wave: every load of a wave's tokens is issued before the first is used, so each wave
// keeps several rows in flight instead of one. Sources are read once (nontemporal loads); the
// stores go through the cache, which merges the parts of the 128-byte lines that neighbouring
// rows share (656- and 132-byte rows are not line-aligned). Measured on the DSA batch (bf16 in,
// both views out): 54% of HBM with nontemporal stores, 69% with cached stores.
constexpr int kQuantTokensPerWave = 4;

__global__ __launch_bounds__(256) void quant_cache_write_kernel(QuantWriteParams p) {
    constexpr int TPW = kQuantTokensPerWave;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int w = blockIdx.x * 4 + wave;
    if (blockIdx.y == 0) {
        // MLA rows of tokens TPW*w .. +TPW-1: lane l quantizes latent values 8l .. 8l+7 (group l / 16).
        const int t0 = TPW * w;
        if (t0 >= p.num_tokens) return;
        int64_t slot[TPW];
        float x[TPW][8], amax[TPW];
        uint4 rope[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int t = min(t0 + i, p.num_tokens - 1);
            slot[i] = t0 + i < p.num_tokens ? p.slots[t] : -1;
            amax[i] = load_bf16x8(p.latent + (int64_t)t * p.latent_pitch + 16 * lane, x[i]);
            if (lane < 8) rope[i] = load_nt<uint4>(p.rope + (int64_t)t * p.rope_pitch + 16 * lane);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const float scale = __fdiv_rn(row16_max(amax[i]), 448.f);
            const uint2 codes = quantize8(x[i], scale);
            if (slot[i] < 0 || slot[i] >= p.num_slots) continue;  // padding token, or out of range: no write
            const int64_t block = slot[i] / p.block_size;
            const int64_t pos = slot[i] - block * p.block_size;
            char* row = p.mla_dst + block * p.mla_block_stride + pos * 656;
            *reinterpret_cast<uint2*>(row + 8 * lane) = codes;
            if ((lane & 15) == 0) *reinterpret_cast<float*>(row + 512 + 4 * (lane >> 4)) = scale;
            if (lane < 8) *reinterpret_cast<uint4*>(row + 528 + 16 * lane) = rope[i];
        }
    } else {
        // Indexer rows of tokens 4*TPW*w .. +4*TPW-1: in step i, lane l quantizes key values 8 (l % 16)
        // .. +7 of token 4*TPW*w + 4i + l / 16 (one token per 16-lane row).
        const int t0 = 4 * TPW * w;
        if (t0 >= p.num_tokens) return;  // wave-uniform
        const int c = lane & 15;
        int64_t slot[TPW];
        float k[TPW][8], amax[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tt = t0 + 4 * i + (lane >> 4);
            const int t = min(tt, p.num_tokens - 1);
            slot[i] = tt < p.num_tokens ? p.slots[t] : -1;
            amax[i] = load_bf16x8(p.index_key + (int64_t)t * p.index_pitch + 16 * c, k[i]);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const float scale = __fdiv_rn(row16_max(amax[i]), 448.f);  // every lane of the row takes part
            const uint2 codes = quantize8(k[i], scale);
            if (slot[i] < 0 || slot[i] >= p.num_slots) continue;
            const int64_t block = slot[i] / p.block_size;
            const int64_t pos = slot[i] - block * p.block_size;
            char* row = p.idx_dst + block * p.idx_block_stride + pos * 132;  // only 4-byte aligned
            reinterpret_cast<uint32_t*>(row)[2 * c] = codes.x;
            reinterpret_cast<uint32_t*>(row)[2 * c + 1] = codes.y;
            if (c == 0) reinterpret_cast<uint32_t*>(row)[32] = __float_as_uint(scale);
        }
    }
}

hipError_t launch_quant_cache_write(const QuantWriteParams& p, hipStream_t stream) {
    if (p.num_tokens <= 0) return hipSuccess;
    // x: work-groups of the MLA part (4 waves of kQuantTokensPerWave tokens), which is more than the
    // indexer part needs (4 times as many tokens per wave); y: 0 = MLA rows, 1 = indexer rows.
    const int per_wg = 4 * kQuantTokensPerWave;
    const dim3 grid((p.num_tokens + per_wg - 1) / per_wg, p.index_key != nullptr ? 2 : 1);
    hipLaunchKernelGGL(quant_cache_write_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Block copy for copy-on-write.
//
// "vLLM 技术内幕" §2.2: a sequence about to write into a block whose reference count is above 1 gets
// a new physical block and the contents are copied; the count and the allocation are the block
// manager's. Here is the copy: one work-group per (pair, layer) and view moves the page (block_size
// rows, contiguous in every view of "vLLM KV Cache Layout 可视化") in batches of 4 words per thread.
// Block ids outside [0, num_blocks) skip the pair.
// ---------------------------------------------------------------------------

template <typename Word>
__device__ __forceinline__ void copy_page(const char* src, char* dst, int64_t bytes) {
    constexpr int U = 4;
    const int64_t n = bytes / (int64_t)sizeof(Word);
    const Word* s = reinterpret_cast<const Word*>(src);
    Word* d = reinterpret_cast<Word*>(dst);
    for (int64_t base = 0; base < n; base += 256 * U) {
        Word v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 256 * u + threadIdx.x;
            if (i < n) v[u] = s[i];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + 256 * u + threadIdx.x;
            if (i < n) d[i] = v[u];
        }
    }
}

__global__ __launch_bounds__(256) void block_copy_kernel(BlockCopyParams p) {
    const int view = blockIdx.y;
    const int pair = blockIdx.x / p.num_layers;
    const int layer = blockIdx.x - pair * p.num_layers;
    const int64_t src = p.pairs[2 * pair], dst = p.pairs[2 * pair + 1];
    if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks) return;
    const char* s = p.base[view] + layer * p.layer_stride[view] + src * p.block_stride[view];
    char* d = p.base[view] + layer * p.layer_stride[view] + dst * p.block_stride[view];
    if (p.vec16[view]) copy_page<uint4>(s, d, p.page_bytes[view]);
    else copy_page<uint32_t>(s, d, p.page_bytes[view]);
}

hipError_t launch_block_copy(const BlockCopyParams& p, hipStream_t stream) {
    if (p.num_pairs <= 0 || p.num_layers <= 0) return hipSuccess;
    const dim3 grid((unsigned)((int64_t)p.num_pairs * p.num_layers), p.num_views);
    hipLaunchKernelGGL(block_copy_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantize-on-write of dense rows into an FP8 cache.
//
// "deep dive into vLLM 05" §3.4: quantize on write, FP8. Every 16-bit value x of a row is stored as
// the E4M3 code nearest to the float32 quotient x / scale (one scale per cache), ties to even,
// saturating at 448. A wave takes the rows of 4 tokens as one run of 8-value units (16 bytes in,
// 8 bytes out), loading a batch of units per lane before storing any; the quotients use the same
// one-division-per-scale method as the DSA rows.
// ---------------------------------------------------------------------------

namespace {

// 8 16-bit values -> 8 fp32 values (exact).
template <bool F16>
__device__ __forceinline__ void x16x8_to_f32(const uint4& v, float (&x)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (F16) {
            x[2 * i] = (float)__builtin_bit_cast(f16x2, w[i]).x;
            x[2 * i + 1] = (float)__builtin_bit_cast(f16x2, w[i]).y;
        } else {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}

// Codes of 8 values for a fixed scale with its correctly rounded reciprocal (see quantize8).
__device__ __forceinline__ uint2 quantize8_fixed(const float (&x)[8], float scale, float y) {
    const bool normal = scale >= 1.17549435e-38f;
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float qq;
            if (normal) {
                const float q0 = x[4 * h + i] * y;
                qq = __builtin_fmaf(__builtin_fmaf(-q0, scale, x[4 * h + i]), y, q0);
            } else {
                qq = __fdiv_rn(x[4 * h + i], scale);
            }
            q[i] = fminf(fmaxf(qq, -448.f), 448.f);
        }
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], v, true);
        w[h] = (uint32_t)v;
    }
    return make_uint2(w[0], w[1]);
}

// A wave quantizes one chunk of the flat run of 8-value units of all tokens (at most 512 units,
// touching at most 64 tokens), loading every unit of the chunk before storing the first code word;
// destination rows as in copy_chunk.
template <bool F16>
__device__ __forceinline__ void quant_chunk(const QuantDenseParams& p, int view, int64_t chunk, int lane) {
    constexpr int B = 8;
    const uint32_t n = (uint32_t)p.row_values / 8;  // 8-value units per row
    const uint32_t cw = min(64u * B, 63u * n);
    const int64_t total = (int64_t)p.num_tokens * n;
    const int64_t j0 = chunk * cw;
    if (j0 >= total) return;
    const uint32_t cnt = (uint32_t)min((int64_t)cw, total - j0);
    const int64_t tok0 = j0 / n;
    const uint32_t w0 = (uint32_t)(j0 - tok0 * n);
    const int ntok = (int)((w0 + cnt + n - 1) / n);
    const char* src = p.src[view] + tok0 * p.pitch[view];
    const int64_t pitch = p.pitch[view];
    const float rcp_n = 1.f / (float)n;
    const float scale = p.scale[view], y = p.inv_scale[view];
    const int64_t my_slot = lane < ntok ? p.slots[tok0 + lane] : -1;

    uint4 v[B];
    uint32_t tk[B], wd[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const uint32_t jj = 64u * u + (uint32_t)lane;
        if (jj < cnt) {
            const uint32_t x = w0 + jj;
            uint32_t t = (uint32_t)((float)x * rcp_n);
            if (t * n > x) --t;
            else if ((t + 1) * n <= x) ++t;
            tk[u] = t;
            wd[u] = x - t * n;
            v[u] = load_nt<uint4>(src + (int64_t)t * pitch + (int64_t)wd[u] * 16);
        } else {
            tk[u] = 0;
            wd[u] = 0;
        }
    }
    uint64_t my_dst = 0;
    if (lane < ntok && my_slot >= 0 && my_slot < p.num_slots) {
        const int64_t block = my_slot / p.block_size;
        my_dst = (uint64_t)(p.dst[view] + block * p.block_stride[view] +
                            (my_slot - block * p.block_size) * (int64_t)p.row_values);
    }
    const uint32_t dlo = (uint32_t)my_dst, dhi = (uint32_t)(my_dst >> 32);
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const uint32_t jj = 64u * u + (uint32_t)lane;
        const uint64_t d = (uint64_t)(uint32_t)__shfl((int)dlo, (int)tk[u]) |
                           ((uint64_t)(uint32_t)__shfl((int)dhi, (int)tk[u]) << 32);
        if (jj < cnt && d != 0) {
            float x[8];
            x16x8_to_f32<F16>(v[u], x);
            const uint2 codes = quantize8_fixed(x, scale, y);
            typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t c2 = {codes.x, codes.y};
            __builtin_nontemporal_store(c2, reinterpret_cast<u32x2_t*>(reinterpret_cast<char*>(d) + (int64_t)wd[u] * 8));
        }
    }
}

}  // namespace

__global__ __launch_bounds__(256) void quant_dense_write_kernel(QuantDenseParams p) {
    const int view = blockIdx.y;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * 4 + wave;
    if (p.src_f16) quant_chunk<true>(p, view, chunk, lane);
    else quant_chunk<false>(p, view, chunk, lane);
}

hipError_t launch_quant_dense_write(const QuantDenseParams& p, hipStream_t stream) {
    if (p.num_tokens <= 0) return hipSuccess;
    const uint32_t n = (uint32_t)p.row_values / 8;
    const uint32_t cw = 512u < 63u * n ? 512u : 63u * n;
    const int64_t chunks = ((int64_t)p.num_tokens * n + cw - 1) / cw;
    const int64_t wgs = (chunks + 3) / 4;
    if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
    dim3 grid((unsigned)wgs, p.num_views);
    hipLaunchKernelGGL(quant_dense_write_kernel, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

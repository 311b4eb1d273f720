// MLA latent decode over packed 656-byte rows: many query heads on one latent K/V head.
//
// "deep dive into vLLM 05" §3.3: MLA caches one low-dimensional latent per token; with the
// up-projection folded into the query, attention runs in latent space and the cache is never
// decompressed. "vLLM KV Cache Layout 可视化" (section on two caches sharing one block table) gives
// the row: 512 B of FP8 latent, 16 B of scale, 128 B of BF16 RoPE. The row is read here as 512 e4m3
// latent values, 4 float32 scales (scale k for latent values [128k, 128k+128)) and 64 bf16 RoPE
// values. Scores use [latent | rope] (576 dims); the value is the dequantized 512-dim latent:
//     s_t = scale * (q_lat . (c_t * sc_t) + q_rope . r_t),   out = softmax(s) . (c * sc).
//
// With 128 heads on one latent head the work is a dense contraction: per token 128 x (576 + 512)
// multiply-adds against 656 bytes read, about 425 flop per byte, above the MI355X bf16 ridge
// (2.5 PFLOP/s over 8 TB/s, about 310). So the kernel is laid out for the matrix cores:
//
//  * A work-group owns up to 128 heads (4 waves x 32) and a balanced range of the token stream (all
//    sequences' 32-token units, in order; ranges may cross sequences). Its waves hold their heads'
//    queries (18 k-steps x 2 head tiles, 144 registers) and outputs (32 heads x 512 fp32, 256
//    accumulation registers) for a whole segment, so the only operands streamed are K and V.
//  * Each 32-token unit is copied from HBM straight into LDS (global_load_lds, 16 bytes per lane,
//    four stages in flight), then dequantized once for the whole work-group into a bf16 tile
//    [32 rows x (512 latent * scale | 64 RoPE)]: each e4m3 value is converted exactly to fp32,
//    multiplied by its scale and rounded to bf16. Every wave reads its score (K) and PV (V) operands
//    from that tile; rows are swizzled so the 16-byte operand reads are free of bank conflicts.
//  * Scores S^T = K . Q^T and PV O += P . V run on v_mfma_f32_16x16x32_bf16. The score output
//    registers are directly the PV A operand (token order sigma of mfma_common.h, two 16-token tiles
//    per k=32 step); the V operand is gathered from the tile with v_perm_b32.
//  * Per unit: one barrier; the dequantization of unit u+1 is interleaved with the products of
//    unit u. The softmax is online (lazy reference, as in the dense decode) and a segment that is
//    not a whole sequence writes an fp32 partial merged by mla_merge_kernel (log-sum-exp).

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kRow = 656;                          // bytes per cached token row
constexpr int kScaleOff = 512;                     // 4 x float32
constexpr int kRopeOff = 528;                      // 64 x bf16
constexpr int kUnit = 32;                          // tokens per unit (one step of a work-group)
constexpr int kUnitChunks = kUnit * kRow / 16;     // 1312 chunks of 16 bytes; 41 per row
constexpr int kWindows = (kUnitChunks + 63) / 64;  // one load instruction of a wave fills a 64-chunk window
constexpr int kRawStage = kWindows * 1024;
constexpr int kTileRow = 1152;                     // 576 bf16
constexpr int kTileStage = kUnit * kTileRow;
constexpr int kTile1 = 16 * kTileRow;              // byte offset of the unit's second 16-token tile
constexpr int kLatentChunks = kUnit * 64;          // 16-byte bf16 chunks of dequantized latent per unit
constexpr int kRopeChunks = kUnit * 8;
constexpr int kKSteps = 18;                        // k=32 steps over 576 score dims

// Raw rows arrive in four stages and the dequantized tile has two. They are separate objects rather
// than one indexed array so that the compiler can tell the stage being read from those still being
// filled by the direct-to-LDS loads, and does not wait for all of them.
__shared__ __attribute__((aligned(16))) char s_raw0[kRawStage];
__shared__ __attribute__((aligned(16))) char s_raw1[kRawStage];
__shared__ __attribute__((aligned(16))) char s_raw2[kRawStage];
__shared__ __attribute__((aligned(16))) char s_raw3[kRawStage];
__shared__ __attribute__((aligned(16))) char s_junk[1024];  // target of loads past the last window
__shared__ __attribute__((aligned(16))) char s_tile0[kTileStage];
__shared__ __attribute__((aligned(16))) char s_tile1[kTileStage];

template <int K>
__device__ __forceinline__ char* raw_stage() {
    if constexpr (K == 0) return s_raw0;
    else if constexpr (K == 1) return s_raw1;
    else if constexpr (K == 2) return s_raw2;
    else return s_raw3;
}
template <int K>
__device__ __forceinline__ char* tile_stage() {
    if constexpr (K == 0) return s_tile0;
    else return s_tile1;
}

// 16-byte chunk c of tile row r is stored at chunk c ^ swz(r). The eight rows a group of eight lanes
// reads at once for the score operand (16t + sigma(m), m = 0..7 or 8..15) get distinct swizzles.
// Tile rows are 1152 bytes, a multiple of the 128-byte bank cycle, so unswizzled they would collide.
__device__ __forceinline__ int swz(int r) { return ((r & 1) << 2) | ((r >> 2) & 3); }

// s_waitcnt immediate: wait until at most vm vector-memory operations are outstanding and all LDS
// operations are done (expcnt not waited on).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | ((vm >> 4) << 14); }

__device__ __forceinline__ int mla_ctx(int s, const MlaDecodeParams& p) {
    const int64_t cap = min((int64_t)p.max_context_len, (int64_t)p.bt_stride * p.block_size);
    return (int)max((int64_t)0, min((int64_t)p.context_lens[s], cap));
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Position in the unit stream (all values wave-uniform).
struct Cursor {
    int g;    // unit index in the whole stream
    int s;    // sequence
    int k;    // unit within the sequence
    int nu;   // units of the sequence
    int ctx;  // tokens of the sequence
};

__device__ __forceinline__ void advance(Cursor& c, const MlaDecodeParams& p) {
    ++c.g;
    if (++c.k < c.nu) return;
    c.k = 0;
    do {
        ++c.s;
        c.ctx = c.s < p.num_seqs ? __builtin_amdgcn_readfirstlane(mla_ctx(c.s, p)) : 0;
        c.nu = (c.ctx + kUnit - 1) / kUnit;
    } while (c.nu == 0 && c.s < p.num_seqs);
}

__device__ int total_units(const MlaDecodeParams& p, int lane) {
    int u = 0;
    for (int base = 0; base < p.num_seqs; base += 64) {
        const int s = base + lane;
        u += wave_sum_int(s < p.num_seqs ? (mla_ctx(s, p) + kUnit - 1) / kUnit : 0);
    }
    return __builtin_amdgcn_readfirstlane(u);
}

// Cursor of unit g0 (g0 < total_units).
__device__ Cursor locate(int g0, const MlaDecodeParams& p, int lane) {
    int before = 0;
    for (int base = 0; base < p.num_seqs; base += 64) {
        const int s = base + lane;
        const int ctx = s < p.num_seqs ? mla_ctx(s, p) : 0;
        const int nu = (ctx + kUnit - 1) / kUnit;
        int incl = nu;  // inclusive prefix over the lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl(incl, max(lane - off, 0));
            if (lane >= off) incl += t;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (g0 < before + total) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(before + incl > g0);
            const int ls = __builtin_ctzll(hit);
            Cursor c;
            c.g = g0;
            c.s = base + ls;
            c.ctx = __builtin_amdgcn_readlane(ctx, ls);
            c.nu = __builtin_amdgcn_readlane(nu, ls);
            c.k = g0 - (before + __builtin_amdgcn_readlane(incl, ls) - c.nu);
            return c;
        }
        before += total;
    }
    Cursor c{g0, p.num_seqs, 0, 0, 0};
    return c;
}

// Eight e4m3 bytes, times their row-quarter scale, as eight bf16 (round to nearest even). The
// e4m3 -> fp32 conversion is exact.
__device__ __forceinline__ uint4 dequant8(uint2 b, float sc) {
    const f32x2_t a0 = __builtin_amdgcn_cvt_pk_f32_fp8(b.x, false);
    const f32x2_t a1 = __builtin_amdgcn_cvt_pk_f32_fp8(b.x, true);
    const f32x2_t a2 = __builtin_amdgcn_cvt_pk_f32_fp8(b.y, false);
    const f32x2_t a3 = __builtin_amdgcn_cvt_pk_f32_fp8(b.y, true);
    return make_uint4(pack2<true>(a0.x * sc, a0.y * sc), pack2<true>(a1.x * sc, a1.y * sc),
                      pack2<true>(a2.x * sc, a2.y * sc), pack2<true>(a3.x * sc, a3.y * sc));
}

// Keeps the compiler from moving memory accesses across the hardware barrier next to it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

}  // namespace

// NT: 16-head tiles per wave; NW: waves per work-group (heads_per_wg = 16 * NT * NW).
template <int NT, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mla_kernel(MlaDecodeParams p) {
    constexpr int R = (kWindows + NW - 1) / NW;  // load instructions per lane per unit
    constexpr int kLatentIters = (kLatentChunks + 64 * NW - 1) / (64 * NW);
    constexpr int kRopeIters = (kRopeChunks + 64 * NW - 1) / (64 * NW);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int lane = threadIdx.x & 63;
    int c = lane & 15;
    int g4 = lane >> 4;
    int tid = wave * 64 + lane;
    const int w = blockIdx.x;
    const int Hq = p.num_q_heads;
    const int head0 = blockIdx.y * p.heads_per_wg + wave * 16 * NT;  // first head of this wave

    const int U = total_units(p, lane);
    const int per = p.units_per_wg > 0 ? p.units_per_wg : (U + p.num_wgs - 1) / p.num_wgs;
    const int g_begin = w * per;
    const int g_end = min(U, g_begin + per);
    if (g_begin >= g_end) return;  // the same for every wave of the work-group

    const char* dummy = static_cast<const char*>(p.q);  // in-bounds source of loads that fill nothing used
    const uint32_t nb = (uint32_t)p.num_blocks;
    const float sl2 = p.scale_log2;

    // Per-lane LDS offsets. Score operand (A = K): row 16t + sigma(c), chunk 4ks + g4, swizzled; the
    // swizzled chunk is 8 (ks >> 1) + ((4 (ks & 1)) ^ x) with x = g4 ^ swz(row).
    const int arow = sigma(c);
    const int ax = g4 ^ swz(arow);
    int a_even = arow * kTileRow + (ax << 4);
    int a_odd = arow * kTileRow + ((ax ^ 4) << 4);
    // PV operand (B = V): rows 16t + g4 + 4i, dims 128q + 8c .. +7 (chunk 16q + c, swizzled).
    int vbase[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vbase[i] = (g4 + 4 * i) * kTileRow + ((c ^ (((g4 & 1) << 2) | i)) << 4);

    uint4 qr[NT][kKSteps];
    f32x4_t O[NT][4][8];  // [head tile][latent quarter q][dim 128q + 8c + e]
    float m[NT], l[NT];
    // Unit validity, one slot per raw stage: bits 0..7 valid rows, bit 8 / 9 rows 0..15 / 16..31 in a
    // valid block.
    int info[4];

    Cursor cc = locate(g_begin, p, lane);  // unit being computed
    Cursor cl = cc;                        // next unit to load
    bool seg_from_start = false;           // the current segment began at the sequence's first unit

    // Empty asm statements that tie the queries to vector registers and the outputs to accumulation
    // registers once per step. Without them the register allocator is free to move the queries (an
    // MFMA B operand may come from either file) into the accumulation registers, which pushes the
    // outputs out and costs hundreds of register-to-register copies per step.
    auto pin_outputs = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e) asm volatile("" : "+a"(O[n][q][e]));
    };
    auto pin_registers = [&]() __attribute__((always_inline)) {
        asm volatile("" : "+v"(lane), "+v"(c), "+v"(g4), "+v"(tid), "+v"(a_even), "+v"(a_odd), "+v"(vbase[0]),
                     "+v"(vbase[1]), "+v"(vbase[2]), "+v"(vbase[3]));
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks) {
                u32x4 t = __builtin_bit_cast(u32x4, qr[n][ks]);
                asm volatile("" : "+v"(t));
                qr[n][ks] = __builtin_bit_cast(uint4, t);
            }
        pin_outputs();
    };

    // Copies unit cl into raw stage K, records its validity in info[K], and advances cl.
    auto issue = [&](auto kst) __attribute__((always_inline)) {
        constexpr int K = decltype(kst)::value;
        const bool live = cl.g < g_end;
        int v = 0;
        int64_t off_a = 0, off_b = 0;
        bool ok_a = false, ok_b = false;
        if (live) {
            v = min(kUnit, cl.ctx - cl.k * kUnit);
            const int t0 = cl.k * kUnit;
            const int32_t* bt = p.block_tables + (int64_t)cl.s * p.bt_stride;
            const int lb = t0 >> p.block_size_log2;
            const int pa = bt[lb];
            ok_a = (uint32_t)pa < nb;
            off_a = (int64_t)pa * p.block_stride + (int64_t)(t0 & (p.block_size - 1)) * kRow;
            if (p.block_size < kUnit) {  // block size 16: rows 16..31 are in the next block
                const int pb = v > 16 ? bt[lb + 1] : pa;
                ok_b = (uint32_t)pb < nb;
                off_b = (int64_t)pb * p.block_stride - 16 * kRow;
            } else {
                ok_b = ok_a;
                off_b = off_a;
            }
        }
        info[K] = v | (ok_a ? 0x100 : 0) | (ok_b ? 0x200 : 0);
        char* stage = raw_stage<K>();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int win = r * NW + wave;
            const int kk = win * 64 + lane;  // chunk; row kk / 41, since a row is 41 chunks
            const int row = kk / 41;
            const bool use = kk < v * 41 && (row < 16 ? ok_a : ok_b);
            const char* src = use ? p.kv + (row < 16 ? off_a : off_b) + (int64_t)kk * 16 : dummy;
            char* dst = win < kWindows ? stage + win * 1024 : s_junk;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
        }
        advance(cl, p);
    };

    // Dequantizes latent items [i0, i0 + CNT) (and, if rope, the RoPE chunks) of the unit in raw
    // stage KR (validity vi) into tile stage KT. Branch-free: rows past the valid ones read stale LDS
    // bytes and write zeros.
    auto convert = [&](auto kr, auto kt, int vi, int i0, auto cnt, bool rope) __attribute__((always_inline)) {
        constexpr int KR = decltype(kr)::value;
        constexpr int KT = decltype(kt)::value;
        constexpr int CNT = decltype(cnt)::value;
        const char* raw = raw_stage<KR>();
        char* tile = tile_stage<KT>();
        const int v = vi & 0xFF;
        const bool ok_a = vi & 0x100, ok_b = vi & 0x200;
#pragma unroll
        for (int jj = 0; jj < CNT; ++jj) {
            const int it = i0 + jj;
            const int n = it * 64 * NW + tid;
            if (it < kLatentIters && (kLatentChunks % (64 * NW) == 0 || n < kLatentChunks)) {
                const int r = n >> 6, ch = n & 63;
                const uint2 b8 = *reinterpret_cast<const uint2*>(raw + r * kRow + 8 * ch);
                const float sc = *reinterpret_cast<const float*>(raw + r * kRow + kScaleOff + 4 * (ch >> 4));
                const uint4 d = dequant8(b8, sc);
                const bool keep = r < v && (r < 16 ? ok_a : ok_b);
                *reinterpret_cast<uint4*>(tile + r * kTileRow + ((ch ^ swz(r)) << 4)) =
                    keep ? d : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        if (rope) {
#pragma unroll
            for (int it = 0; it < kRopeIters; ++it) {
                const int n = it * 64 * NW + tid;
                if (kRopeChunks % (64 * NW) == 0 || n < kRopeChunks) {
                    const int r = n >> 3, k8 = n & 7;
                    const uint4 d = *reinterpret_cast<const uint4*>(raw + r * kRow + kRopeOff + 16 * k8);
                    const bool keep = r < v && (r < 16 ? ok_a : ok_b);
                    *reinterpret_cast<uint4*>(tile + r * kTileRow + ((64 + (k8 ^ swz(r))) << 4)) =
                        keep ? d : make_uint4(0u, 0u, 0u, 0u);
                }
            }
        }
    };

    auto begin_segment = [&]() __attribute__((always_inline)) {
        const uint16_t* qs = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)cc.s * Hq + head0 + c) * 576 + 8 * g4;
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int ks = 0; ks < kKSteps; ++ks)
                qr[n][ks] = *reinterpret_cast<const uint4*>(qs + (size_t)n * 16 * 576 + 32 * ks);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            m[n] = kNegInf;
            l[n] = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e) O[n][q][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        pin_outputs();
        seg_from_start = cc.k == 0;
        if (seg_from_start && blockIdx.y == 0 && tid == 0) {
            // This work-group holds the sequence's first unit: record which work-groups it spans.
            p.seq_meta[2 * cc.s] = w;
            p.seq_meta[2 * cc.s + 1] = (cc.g + cc.nu - 1) / per;
        }
    };

    auto end_segment = [&]() __attribute__((always_inline)) {
        const bool whole = seg_from_start && cc.k + 1 == cc.nu;
        float L[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            L[n] = l[n] + __shfl_xor(l[n], 16);
            L[n] += __shfl_xor(L[n], 32);
        }
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int hr = 4 * g4 + j;  // head row of output register j, = the lane holding its (m, l)
                const float Lr = __shfl(L[n], hr);
                const float Mr = __shfl(m[n], hr);
                const int head = head0 + 16 * n + hr;
                if (whole) {
                    const float inv = Lr > 0.f ? 1.f / Lr : 0.f;
                    uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + ((size_t)cc.s * Hq + head) * 512 + 8 * c;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint4*>(o + 128 * q) =
                            make_uint4(pack2<true>(O[n][q][0][j] * inv, O[n][q][1][j] * inv),
                                       pack2<true>(O[n][q][2][j] * inv, O[n][q][3][j] * inv),
                                       pack2<true>(O[n][q][4][j] * inv, O[n][q][5][j] * inv),
                                       pack2<true>(O[n][q][6][j] * inv, O[n][q][7][j] * inv));
                } else {
                    const size_t idx = (size_t)(cc.s + w) * Hq + head;
                    float* a = p.part_acc + idx * 512 + 8 * c;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        *reinterpret_cast<float4*>(a + 128 * q) =
                            make_float4(O[n][q][0][j], O[n][q][1][j], O[n][q][2][j], O[n][q][3][j]);
                        *reinterpret_cast<float4*>(a + 128 * q + 4) =
                            make_float4(O[n][q][4][j], O[n][q][5][j], O[n][q][6][j], O[n][q][7][j]);
                    }
                    if (c == 0) *reinterpret_cast<float2*>(p.part_ml + idx * 2) = make_float2(Mr, Lr);
                }
            }
    };

    // Scores, online softmax and PV of the unit in tile stage KT (validity vi), with the
    // dequantization of the next unit (raw stage KR2 -> tile stage KT2, validity vn) spread over the
    // PV slots. Each slot loads the next slot's LDS operands and then issues its own products; the
    // scheduling barriers keep the compiler from hoisting every operand load to the top, which would
    // need more registers than the queries and outputs leave free.
    auto compute = [&](auto kt, int vi, auto kr2, auto kt2, int vn) __attribute__((always_inline)) {
        constexpr int KT = decltype(kt)::value;
        const char* tile = tile_stage<KT>();
        const int v = vi & 0xFF;
        const bool ok_a = vi & 0x100, ok_b = vi & 0x200;

        // Scores: 36 A operands (t, ks), two per slot.
        constexpr int kSlotsS = kKSteps;  // 2 * 18 operands / 2
        f32x4_t S[2][NT];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int n = 0; n < NT; ++n) S[t][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        uint4 abuf[2][2];
        auto load_a = [&](int slot, uint4 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int x = 2 * slot + h, t = x / kKSteps, ks = x % kKSteps;
                dst[h] = *reinterpret_cast<const uint4*>(tile + ((ks & 1) ? a_odd : a_even) + t * kTile1 +
                                                         (ks >> 1) * 128);
            }
        };
        load_a(0, abuf[0]);
#pragma unroll
        for (int slot = 0; slot < kSlotsS; ++slot) {
            if (slot + 1 < kSlotsS) load_a(slot + 1, abuf[(slot + 1) & 1]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int x = 2 * slot + h, t = x / kKSteps, ks = x % kKSteps;
#pragma unroll
                for (int n = 0; n < NT; ++n) S[t][n] = mfma_k32<true>(abuf[slot & 1][h], qr[n][ks], S[t][n]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // Register j of tile t holds token 16t + g4 + 4j of head column c.
        bool ok[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) ok[t][j] = 16 * t + g4 + 4 * j < v && (t == 0 ? ok_a : ok_b);
        float tmax[NT];
        bool need[NT];
        bool any = false;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float mx = kNegInf;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) mx = ok[t][j] ? fmaxf(mx, S[t][n][j]) : mx;
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            tmax[n] = mx * sl2;
            need[n] = tmax[n] > m[n] + kRescaleSlack;
            any = any || need[n];
        }
        if (__builtin_amdgcn_ballot_w64(any) != 0) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const float mnew = need[n] ? tmax[n] : m[n];
                const float alpha = need[n] ? fast_exp2(m[n] - mnew) : 1.f;
                l[n] *= alpha;
                m[n] = mnew;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float aj = __shfl(alpha, 4 * g4 + j);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int e = 0; e < 8; ++e) O[n][q][e][j] *= aj;
                }
            }
            pin_outputs();
        }
        uint4 A[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float pr[2][4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float ex = fast_exp2(fmaf(S[t][n][j], sl2, -m[n]));
                    pr[t][j] = ok[t][j] ? ex : 0.f;
                    l[n] += pr[t][j];
                }
            A[n] = make_uint4(pack2<true>(pr[0][0], pr[0][1]), pack2<true>(pr[0][2], pr[0][3]),
                              pack2<true>(pr[1][0], pr[1][1]), pack2<true>(pr[1][2], pr[1][3]));
        }

        // PV: one slot per 128-dim latent quarter q. Lane c reads 8 dims (128q + 8c .. +7) of its eight
        // rows; k-slot j of lane group g4 is token g4 + 4j (j < 4) or 16 + g4 + 4(j - 4).
        constexpr int kSlotsP = 4;
        constexpr int kConvPerSlot = (kLatentIters + kSlotsP - 1) / kSlotsP;
        uint4 vbuf[2][2][4];
        auto load_v = [&](int q, uint4 (&dst)[2][4]) __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[t][i] = *reinterpret_cast<const uint4*>(tile + vbase[i] + t * kTile1 + q * 256);
        };
        load_v(0, vbuf[0]);
#pragma unroll
        for (int q = 0; q < kSlotsP; ++q) {
            if (q + 1 < kSlotsP) load_v(q + 1, vbuf[(q + 1) & 1]);
            const uint4 (&V)[2][4] = vbuf[q & 1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t sel = (e & 1) ? kSelHi : kSelLo;
                auto wd = [&](const uint4& x) __attribute__((always_inline)) {
                    return (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
                };
                const uint4 B = make_uint4(__builtin_amdgcn_perm(wd(V[0][1]), wd(V[0][0]), sel),
                                           __builtin_amdgcn_perm(wd(V[0][3]), wd(V[0][2]), sel),
                                           __builtin_amdgcn_perm(wd(V[1][1]), wd(V[1][0]), sel),
                                           __builtin_amdgcn_perm(wd(V[1][3]), wd(V[1][2]), sel));
#pragma unroll
                for (int n = 0; n < NT; ++n) O[n][q][e] = mfma_k32<true>(A[n], B, O[n][q][e]);
            }
            convert(kr2, kt2, vn, q * kConvPerSlot, std::integral_constant<int, kConvPerSlot>{}, q == kSlotsP - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Step of unit u (K = u % 4): wait for unit u+1's rows, start loading unit u+4, compute unit u
    // while dequantizing unit u+1. Returns false when the range is done.
    auto step = [&](auto kst) __attribute__((always_inline)) -> bool {
        constexpr int K = decltype(kst)::value;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * R));  // own loads of unit u+1 are done
        compiler_fence();
        __builtin_amdgcn_s_barrier();                          // everyone's are; step u-1 is finished
        compiler_fence();
        const int cur = info[K];
        const int nxt = info[(K + 1) & 3];
        pin_registers();
        issue(std::integral_constant<int, K>{});
        if (cc.g == g_begin || cc.k == 0) begin_segment();
        compute(std::integral_constant<int, K & 1>{}, cur, std::integral_constant<int, (K + 1) & 3>{},
                std::integral_constant<int, (K + 1) & 1>{}, nxt);
        if (cc.g + 1 == g_end || cc.k + 1 == cc.nu) end_segment();
        advance(cc, p);
        return cc.g < g_end;
    };

    // Prologue: units 0..3 in flight, unit 0 dequantized.
    issue(std::integral_constant<int, 0>{});
    issue(std::integral_constant<int, 1>{});
    issue(std::integral_constant<int, 2>{});
    issue(std::integral_constant<int, 3>{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(3 * R));
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    convert(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, info[0], 0,
            std::integral_constant<int, kLatentIters>{}, true);

    while (true) {
        if (!step(std::integral_constant<int, 0>{})) break;
        if (!step(std::integral_constant<int, 1>{})) break;
        if (!step(std::integral_constant<int, 2>{})) break;
        if (!step(std::integral_constant<int, 3>{})) break;
    }
    // Drain: the loads issued for units past the range still target this work-group's LDS.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
}

// One wave per (sequence, query head): merge the sequence's partials, or write the zero output of
// an empty context.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaDecodeParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;  // = s * Hq + head
    if (item >= p.num_seqs * p.num_q_heads) return;
    const int s = item / p.num_q_heads;
    const int head = item - s * p.num_q_heads;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)item * 512;
    if (__builtin_amdgcn_readfirstlane(mla_ctx(s, p)) == 0) {
        *reinterpret_cast<uint4*>(out + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const int first = __builtin_amdgcn_readfirstlane(p.seq_meta[2 * s]);
    const int last = __builtin_amdgcn_readfirstlane(p.seq_meta[2 * s + 1]);
    if (last <= first) return;  // one segment: written by the decode kernel
    const size_t idx = (size_t)(s + first) * p.num_q_heads + head;
    merge_partials<true, 512>(p.part_ml + idx * 2, (int64_t)p.num_q_heads * 2, p.part_acc + idx * 512,
                              (int64_t)p.num_q_heads * 512, last - first + 1, out);
}

namespace {

template <int NT, int NW>
hipError_t launch_mla_typed(const MlaDecodeParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)p.num_wgs, (unsigned)(p.num_q_heads / p.heads_per_wg));
    hipLaunchKernelGGL((decode_mla_kernel<NT, NW>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mla(const MlaDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    hipError_t e;
    switch (p.heads_per_wg) {
        case 64: e = launch_mla_typed<1, 4>(p, stream); break;
        case 32: e = launch_mla_typed<1, 2>(p, stream); break;
        case 16: e = launch_mla_typed<1, 1>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)p.num_seqs * p.num_q_heads;
    hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

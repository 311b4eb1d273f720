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
//  * A work-group owns up to 64 heads (128 heads take two head groups) and a balanced range of the
//    token stream (all sequences' 32-token units, in order; ranges may cross sequences). Each of its
//    waves owns 16 heads and one half (256 dims) of their outputs: two waves per 16 heads, up to
//    eight waves, two per SIMD. A wave holds its heads' queries (18 k-steps, 72 registers) and its
//    outputs (16 heads x 256 fp32, 64 registers) for a whole segment, so the only operands streamed
//    are K and V. The two waves of a head group split the scores: each computes its own 16-token
//    tile of the unit (18 products) and its probabilities against its own reference, and they trade
//    probabilities and references through LDS (one barrier). Both then take the larger reference
//    and rescale both tiles' probabilities with the same fp32 operations, so they hold bitwise the
//    same 32 probabilities; each runs PV for its 256 dims (16 products). So a wave issues 34 products
//    per unit, the algorithmic count.
//  * Each 32-token unit is copied from HBM straight into LDS (lds_dma, 16 bytes per lane; three raw
//    stages, three units in flight), then widened once per work-group into a bf16 tile
//    [32 rows x (512 latent codes | 64 RoPE)]: every e4m3 code is a bf16 value, so the tile holds
//    the codes exactly, and the unit's 4 x 32 float32 scales go to a small table beside the tile.
//    Every read of a raw stage happens at the start of a step, so the stage takes the next unit's
//    copy right after the score exchange, in the middle of the step. Every wave reads its score (K)
//    and PV (V) operands from the tile; rows are swizzled so the operand reads are free of bank
//    conflicts.
//  * Scores S^T = K . Q^T and PV O += P . V run on v_mfma_f32_16x16x32_bf16. The scale groups stay
//    exact: the latent products of each 128-value group accumulate separately (4 k-steps), and
//    each token's group sum is multiplied by its float32 scale and added in fp32; the RoPE products
//    need no scale. On the value side the scale of token t and group g multiplies the probability:
//    the PV A operand for output dims of group g is bf16(p_t * scale_g[t]). So the only roundings
//    are those of fp32 accumulation and of the bf16 probabilities, as in the dense decode. The score
//    output registers are the PV A operand's token order (sigma of mfma_common.h, two 16-token tiles
//    per k=32 step); the V operand comes from ds_read_b64_tr_b16, which transposes 4 x 4 blocks of
//    16-bit values across the lanes of a 16-lane group.
//  * Per unit: the opening barrier and the exchange barrier; the widening of unit u+1 and all but
//    the first of unit u+4's copy instructions are interleaved with the PV products of unit u, and
//    operands are loaded four products ahead. The
//    softmax is online (lazy reference, as in the dense decode) and a segment that is not a whole
//    sequence writes its own output O / l in bf16 and its (m, l), which mla_merge_kernel weighs
//    (log-sum-exp).

#pragma once

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

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

// Raw rows arrive in three stages and the widened tile has two. They are separate objects rather
// than one indexed array so that the compiler can tell the stage being read from those still being
// filled by the direct-to-LDS loads, and does not wait for all of them.
__shared__ __attribute__((aligned(16))) char s_raw0[kRawStage];
__shared__ __attribute__((aligned(16))) char s_raw1[kRawStage];
__shared__ __attribute__((aligned(16))) char s_raw2[kRawStage];
__shared__ __attribute__((aligned(16))) char s_junk[1024];  // target of loads past the last window
__shared__ __attribute__((aligned(16))) char s_tile0[kTileStage];
__shared__ __attribute__((aligned(16))) char s_tile1[kTileStage];
// Scales of the unit in tile stage 0 / 1: entry 32 g + 8 (r & 3) + 4 (r >> 4) + ((r >> 2) & 3) holds
// scale g of row r, so the 8 rows a lane's score registers hold (16 t + g4 + 4 j) are 8 consecutive
// floats. Rows without a token hold 0.
__shared__ __attribute__((aligned(16))) float s_scale0[4 * kUnit];
__shared__ __attribute__((aligned(16))) float s_scale1[4 * kUnit];
// Sparse form: the slots of unit g (32 used of 64 entries) in table g % 8, copied three units ahead.
__shared__ __attribute__((aligned(16))) int32_t s_slot[8][64];
// Score exchange between the two waves that own the same 16 heads: per wave, the probabilities of
// its 16-token tile for its 16 heads (against its own reference) and that reference per head.
__shared__ __attribute__((aligned(16))) float s_xp[8][16 * 16];
__shared__ __attribute__((aligned(16))) float s_xm[8][16];

template <int K>
__device__ __forceinline__ char* raw_stage() {
    if constexpr (K == 0) return s_raw0;
    else if constexpr (K == 1) return s_raw1;
    else return s_raw2;
}
template <int K>
__device__ __forceinline__ char* tile_stage() {
    if constexpr (K == 0) return s_tile0;
    else return s_tile1;
}
template <int K>
__device__ __forceinline__ float* scale_stage() {
    if constexpr (K == 0) return s_scale0;
    else return s_scale1;
}

// 16-byte chunk c of tile row r is stored at chunk c ^ swz(r). Tile rows are 1152 bytes, a multiple
// of the 128-byte bank cycle, so unswizzled the rows read together would collide. With this swizzle
// the eight rows a group of eight lanes reads for the score operand (16t + sigma(m), m = 0..7 or
// 8..15) get eight different swizzles, and the rows g4 + 4i read for the value operand differ in
// the swizzle's upper two bits.
__device__ __forceinline__ int swz(int r) { return (((r >> 2) & 3) << 1) | (r & 1); }

__device__ __forceinline__ int clamp_ctx(int64_t ctx, const MlaDecodeParams& p) {
    const int64_t row = p.slots != nullptr ? p.slot_stride : (int64_t)p.bt_stride * p.block_size;
    const int64_t cap = min((int64_t)p.max_context_len, row);
    return (int)max((int64_t)0, min(ctx, cap));
}

// Context of sequence s (per lane).
__device__ __forceinline__ int mla_ctx(int s, const MlaDecodeParams& p) { return clamp_ctx(p.context_lens[s], p); }

// Context of sequence s, s wave-uniform.
__device__ __forceinline__ int mla_ctx_uniform(int s, const MlaDecodeParams& p) {
    return clamp_ctx(load_scalar(p.context_lens + s), p);
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
        c.ctx = c.s < p.num_seqs ? mla_ctx_uniform(c.s, p) : 0;
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

// Eight e4m3 codes as eight bf16 values (exact: every e4m3 value is a bf16 value).
__device__ __forceinline__ uint4 codes8(uint2 b) {
    return make_uint4(e4m3x2_bf16<false>(b.x), e4m3x2_bf16<true>(b.x), e4m3x2_bf16<false>(b.y),
                      e4m3x2_bf16<true>(b.y));
}

// Position of row r in the scale table of a unit (see s_scale0).
__device__ __forceinline__ int scale_slot(int r) { return 8 * (r & 3) + 4 * (r >> 4) + ((r >> 2) & 3); }

}  // namespace

// NW: waves per work-group (8, 4 or 2); waves w and w + NW / 2 own the same 16 heads
// (heads_per_wg = 8 * NW) and output dims [0, 256) and [256, 512). A wave needs about 235
// registers, which fit the 256 that two waves per SIMD leave each only when the MFMA accumulators
// are ordinary vector registers: decode_mla.hip is compiled with -mllvm -amdgpu-mfma-vgpr-form.
//
// SPARSE: token i of sequence s is the row at slot slots[s][i], in any block. The slots of a unit are
// copied into LDS (s_slot) along with the rows of the unit four places earlier, so each lane finds
// the row of each of its 16-byte chunks there when it issues the unit's copy; a row whose slot is
// outside the pool, or past the sequence's count, is read from q and masked out.
template <int NW, bool SPARSE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4 > 1 ? 2 : 1, 2)))
void decode_mla_kernel(MlaDecodeParams p) {
    constexpr int R = (kWindows + NW - 1) / NW;  // row-copy instructions per lane per unit
    constexpr int RL = R + (SPARSE ? 1 : 0);     // all copy instructions per lane per unit
    constexpr int kLatentIters = kUnit / NW;     // tile rows each wave dequantizes per unit
    constexpr int kRopeIters = (kRopeChunks + 64 * NW - 1) / (64 * NW);
    static_assert(NW == 2 || NW == 4 || NW == 8, "two to eight waves");
    constexpr int kHeadWaves = NW / 2;
    constexpr int kDimTiles = 16;                // 16-dim output tiles of this wave (256 dims)

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int lane = threadIdx.x & 63;
    int tid = wave * 64 + lane;
    const int w = blockIdx.x;
    const int Hq = p.num_q_heads;
    const int hwave = wave % kHeadWaves;
    const int half = wave / kHeadWaves;  // output dims [256 half, +256)
    const int head0 = blockIdx.y * p.heads_per_wg + hwave * 16;  // first head of this wave

    const int U = total_units(p, lane);
    const int per = p.units_per_wg > 0 ? p.units_per_wg : (U + p.num_wgs - 1) / p.num_wgs;
    const int g_begin = w * per;
    const int g_end = min(U, g_begin + per);
    if (g_begin >= g_end) return;  // the same for every wave of the work-group

    const char* dummy = static_cast<const char*>(p.q);  // in-bounds source of loads that fill nothing used
    const uint32_t nb = (uint32_t)p.num_blocks;
    const float sl2 = p.scale_log2;

    // Per-lane LDS offsets (c = lane % 16, g4 = lane / 16).
    // Score operand (A = K): row 16t + sigma(c), chunk 4ks + g4, swizzled: the physical chunk is
    // 8 (ks >> 1) + ((4 (ks & 1)) ^ x) with x = g4 ^ swz(row).
    int a_even, a_odd;
    // Value operand (B = V), read with ds_read_b64_tr_b16: in each 16-lane block (lane group g4) lane
    // n supplies the address of 4 dims (16dt + 4 (n & 3) .. +3) of row 16t + g4 + 4 (n >> 2), and lane
    // i receives dim 16dt + i of the four rows g4, g4 + 4, g4 + 8, g4 + 12: exactly k-slots 0..3
    // (t = 0) or 4..7 (t = 1) of a 16x16x32 B operand whose column i is dim 16dt + i. The physical
    // chunk of that 8-byte piece is 8 (dt >> 2) + 2 ((dt & 3) ^ j) + (h ^ (g4 & 1)) with j = n >> 2,
    // h = (n >> 1) & 1; trbase[d3] holds everything but the dt >> 2 part, for d3 = dt & 3.
    int trbase[4];
    auto lane_offsets = [&]() __attribute__((always_inline)) {
        const int c = lane & 15, g4 = lane >> 4;
        const int arow = sigma(c);
        const int ax = g4 ^ swz(arow);
        a_even = arow * kTileRow + (ax << 4);
        a_odd = arow * kTileRow + ((ax ^ 4) << 4);
        const int j = c >> 2, h = (c >> 1) & 1;
#pragma unroll
        for (int d3 = 0; d3 < 4; ++d3)
            trbase[d3] = (g4 + 4 * j) * kTileRow + ((2 * (d3 ^ j) + (h ^ (g4 & 1))) << 4) + ((c & 1) << 3);
    };
    lane_offsets();

    uint4 qr[kKSteps];
    f32x4_t O[kDimTiles];  // register j of lane (c, g4): head 4 g4 + j, dim 16 (dt0 + dt) + c
    const int dt0 = half * kDimTiles;
    float m = kNegInf, l = 0.f;
    // Unit validity, bit r set when row r holds a token of the unit; the mask of unit u is kept in
    // info[u % 6] from its copy (step u - 4) to its compute (step u).
    uint32_t info[6];

    Cursor cc = locate(g_begin, p, lane);  // unit being computed
    Cursor cl = cc;                        // next unit to load
    Cursor cs = cc;                        // sparse: next unit whose slot table is copied
    bool seg_from_start = false;           // the current segment began at the sequence's first unit

    // Row copy. Chunk kk of a unit (41 per row) is loaded by lane kk % 64 of wave (kk / 64) % NW in
    // round kk / (64 NW). A lane whose chunk is past the unit's valid rows reloads the last valid
    // chunk into its own LDS slot (a row that is never read); a unit with no valid rows (past the
    // range, or in an invalid block) reads the first 16 bytes of q instead. So every wave issues the
    // same R loads per unit, which the vmcnt accounting relies on.
    int dma_kk[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dma_kk[r] = (r * NW + wave) * 64 + lane;

    // Block ids of unit cl (pre_pb: rows 16..31 when block_size is 16). They are read at the end of
    // a step and waited for by the next step's opening wait, so that no scalar load is outstanding
    // during the products: scalar loads return out of order, so while one is pending every wait for
    // LDS data would have to wait for all of it.
    int pre_pa = 0, pre_pb = 0;
    auto prefetch_ids = [&]() __attribute__((always_inline)) {
        if (!SPARSE && cl.g < g_end) {
            const int t0 = cl.k * kUnit;
            const int32_t* bt = p.block_tables + (int64_t)cl.s * p.bt_stride;
            const int lb = t0 >> p.block_size_log2;
            pre_pa = load_scalar(bt + lb);
            pre_pb = (p.block_size < kUnit && cl.ctx - t0 > 16) ? load_scalar(bt + lb + 1) : pre_pa;
        }
    };

    // Copies unit cl into raw stage K, records its validity in info[K] and advances cl.
    // Slot table of unit cs: wave 0 copies 64 entries (the unit's 32, then the next 32, clamped to the
    // sequence) into s_slot[cs.g % 8]; the other waves issue the same instruction into s_junk, so that
    // every wave counts RL copies per unit.
    auto copy_slot_table = [&]() __attribute__((always_inline)) {
        const int32_t* src = p.slots;
        if (cs.g < g_end) src = p.slots + (int64_t)cs.s * p.slot_stride + min(cs.k * kUnit + lane, cs.ctx - 1);
        lds_dma<4>(src, wave == 0 ? lds_addr(s_slot[0]) + 256 * (cs.g & 7) : lds_addr(s_junk));
        advance(cs, p);
    };

    // The unit whose rows are being copied: its raw stage and where its rows come from (dense: the
    // block bases and last chunks of rows 0..15 and 16..31; sparse: its slot table and valid rows).
    // Inside a step only the first copy instruction goes out with the unit's issue; the other R - 1
    // are spread over the value products, so that the work-group's copies do not all queue at the
    // address units at once (3% of the call). The sparse form reads the slots of all its copy
    // instructions at issue (a read of LDS inside the value products would wait for the prefetched
    // value operands), and spreads them only when there are at most three (eight waves); with fewer
    // waves the copies go out together.
    uint32_t pend_stage = 0;
    const char* pend_a = dummy;
    const char* pend_b = dummy;
    int pend_lim_a = 0, pend_lim_b = 0;
    const int32_t* pend_tab = s_slot[0];
    int pend_v = 0;
    int pend_sl[R];  // sparse, spread copies: the slot of each copy instruction's row, read at issue
    constexpr bool kSpread = !SPARSE || R <= 3;
    auto copy_rows = [&](int r) __attribute__((always_inline)) {
        const int win = r * NW + wave;
        const int kk = dma_kk[r];
        const char* src;
        if constexpr (SPARSE) {
            const int row = kk / 41;  // >= 32 past the unit's last chunk
            const int32_t sl = kSpread ? pend_sl[r] : pend_tab[row & 31];
            const bool ok = row < pend_v && (uint32_t)sl < (uint32_t)p.num_slots;
            src = ok ? p.kv + (int64_t)(sl >> p.block_size_log2) * p.block_stride +
                           (int64_t)(sl & (p.block_size - 1)) * kRow + (kk - row * 41) * 16
                     : dummy;
        } else {
            if (p.block_size >= kUnit) {  // one block holds the unit: one base for all rows
                lds_dma_sv<16>(pend_a, (uint32_t)min(kk, pend_lim_a) * 16u,
                               win < kWindows ? pend_stage + win * 1024 : lds_addr(s_junk));
                return;
            }
            const bool hi = kk >= 16 * 41;
            src = (hi ? pend_b : pend_a) + (int64_t)min(kk, hi ? pend_lim_b : pend_lim_a) * 16;
        }
        lds_dma<16>(src, win < kWindows ? pend_stage + win * 1024 : lds_addr(s_junk));
    };

    auto issue_sparse = [&](auto kst, auto kinf, auto all) __attribute__((always_inline)) {
        constexpr int K = decltype(kst)::value;
        constexpr int KI = decltype(kinf)::value;
        const int v = cl.g < g_end ? min(kUnit, cl.ctx - cl.k * kUnit) : 0;
        const int32_t* tab = s_slot[cl.g & 7];
        const int32_t mine = tab[lane & 31];
        info[KI] = (uint32_t)__builtin_amdgcn_ballot_w64(lane < 32 && lane < v && (uint32_t)mine < (uint32_t)p.num_slots);
        pend_stage = lds_addr(raw_stage<K>());
        pend_tab = tab;
        pend_v = v;
        if constexpr (kSpread) {
#pragma unroll
            for (int r = 0; r < R; ++r) pend_sl[r] = tab[(dma_kk[r] / 41) & 31];
        }
#pragma unroll
        for (int r = 0; r < (decltype(all)::value || !kSpread ? R : 1); ++r) copy_rows(r);
        copy_slot_table();
        advance(cl, p);
    };

    auto issue = [&](auto kst, auto kinf, auto all) __attribute__((always_inline)) {
        constexpr int K = decltype(kst)::value;
        constexpr int KI = decltype(kinf)::value;
        if constexpr (SPARSE) {
            issue_sparse(kst, kinf, all);
            return;
        }
        const bool live = cl.g < g_end;
        int v = 0;
        const char* base_a = dummy;              // rows 0..15 (all rows when block_size >= 32)
        const char* base_b = dummy - 16 * kRow;  // rows 16..31, addressed by chunk kk >= 16 * 41
        int lim_a = 0, lim_b = 16 * 41;
        bool ok_a = false, ok_b = false;
        if (live) {
            v = min(kUnit, cl.ctx - cl.k * kUnit);
            const int t0 = cl.k * kUnit;
            const int pa = pre_pa;
            ok_a = (uint32_t)pa < nb;
            if (p.block_size >= kUnit) {
                ok_b = ok_a;
                if (ok_a) {
                    base_a = p.kv + (int64_t)pa * p.block_stride + (int64_t)(t0 & (p.block_size - 1)) * kRow;
                    lim_a = v * 41 - 1;
                }
            } else {  // block size 16: rows 16..31 are in the next block
                if (ok_a) {
                    base_a = p.kv + (int64_t)pa * p.block_stride;
                    lim_a = min(v, 16) * 41 - 1;
                }
                if (v > 16) {
                    const int pb = pre_pb;
                    ok_b = (uint32_t)pb < nb;
                    if (ok_b) {
                        base_b = p.kv + (int64_t)pb * p.block_stride - 16 * kRow;
                        lim_b = v * 41 - 1;
                    }
                }
            }
        }
        info[KI] = (v >= 32 ? 0xFFFFFFFFu : (1u << v) - 1u) & ((ok_a ? 0xFFFFu : 0u) | (ok_b ? 0xFFFF0000u : 0u));
        pend_stage = lds_addr(raw_stage<K>());
        pend_a = base_a;
        pend_b = base_b;
        pend_lim_a = lim_a;
        pend_lim_b = lim_b;
#pragma unroll
        for (int r = 0; r < (decltype(all)::value ? R : 1); ++r) copy_rows(r);
        advance(cl, p);
    };

    // Dequantization of a unit: raw stage KR (validity vi) -> tile stage KT. Item it is row
    // it * NW + wave (the same for the whole wave), 8 bytes per lane; rows past the valid ones are
    // written as zeros (their stale raw bytes are read but not used) and get a zero scale. conv_load
    // issues the LDS reads of all items; conv_store converts and writes items [i0, i0 + CNT) and, if
    // rope, the RoPE chunks and the scales.
    struct ConvIn {
        uint2 b8[kLatentIters];
        uint4 rope[kRopeIters];
        float4 scl;
    };
    // Every read of the raw stage happens here, so that the stage is free for the next copy once
    // these reads are done.
    auto conv_load = [&](auto kr, ConvIn& in) __attribute__((always_inline)) {
        constexpr int KR = decltype(kr)::value;
        const char* raw = raw_stage<KR>();
        const int conv_raw = wave * kRow + 8 * lane;
#pragma unroll
        for (int it = 0; it < kLatentIters; ++it)
            in.b8[it] = *reinterpret_cast<const uint2*>(raw + conv_raw + it * NW * kRow);
#pragma unroll
        for (int it = 0; it < kRopeIters; ++it) {
            const int n = it * 64 * NW + tid;
            if (kRopeChunks % (64 * NW) == 0 || n < kRopeChunks)
                in.rope[it] = *reinterpret_cast<const uint4*>(raw + (n >> 3) * kRow + kRopeOff + 16 * (n & 7));
        }
        if (tid < kUnit) in.scl = *reinterpret_cast<const float4*>(raw + tid * kRow + kScaleOff);
    };
    auto conv_store = [&](auto kr, auto kt, uint32_t vmask, const ConvIn& in, int i0, auto cnt, bool rope)
        __attribute__((always_inline)) {
        constexpr int KT = decltype(kt)::value;
        constexpr int CNT = decltype(cnt)::value;
        char* tile = tile_stage<KT>();
#pragma unroll
        for (int jj = 0; jj < CNT; ++jj) {
            const int it = i0 + jj;
            if (it < kLatentIters) {
                const int r = it * NW + wave;  // wave-uniform
                // A row without a token is written as zeros (its codes are cleared before they are
                // widened), so that its zero probability meets no NaN from stale bytes.
                const bool keep = (vmask >> r) & 1u;
                *reinterpret_cast<uint4*>(tile + r * kTileRow + ((lane ^ swz(r)) << 4)) =
                    codes8(keep ? in.b8[it] : make_uint2(0u, 0u));
            }
        }
        if (rope) {
#pragma unroll
            for (int it = 0; it < kRopeIters; ++it) {
                const int n = it * 64 * NW + tid;
                if (kRopeChunks % (64 * NW) == 0 || n < kRopeChunks) {
                    const int r = n >> 3, k8 = n & 7;
                    // RoPE values enter only the scores, which are masked for rows without a token.
                    *reinterpret_cast<uint4*>(tile + r * kTileRow + ((64 + (k8 ^ swz(r))) << 4)) = in.rope[it];
                }
            }
            // The unit's scales into the table of tile stage KT (0 for rows without a token).
            if (tid < kUnit) {
                const float4 sv = in.scl;
                const bool keep = (vmask >> tid) & 1u;
                float* st = scale_stage<KT>() + scale_slot(tid);
                st[0] = keep ? sv.x : 0.f;
                st[32] = keep ? sv.y : 0.f;
                st[64] = keep ? sv.z : 0.f;
                st[96] = keep ? sv.w : 0.f;
            }
        }
    };

    // Per-lane offsets pass through an empty asm statement at every step. The LDS objects span
    // 160 KB, beyond the 64 KB immediate offset of the LDS instructions, so each (object, per-lane
    // offset) pair would otherwise become its own long-lived register; recomputing costs one add.
    auto refresh_offsets = [&]() __attribute__((always_inline)) {
        asm volatile("" : "+v"(lane), "+v"(tid), "+v"(a_even), "+v"(a_odd));
        asm volatile("" : "+v"(trbase[0]), "+v"(trbase[1]), "+v"(trbase[2]), "+v"(trbase[3]));
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" : "+v"(dma_kk[r]));
    };

    auto begin_segment = [&]() __attribute__((always_inline)) {
        const uint16_t* qs = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)cc.s * Hq + head0 + (lane & 15)) * 576 +
                             8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < kKSteps; ++ks) qr[ks] = *reinterpret_cast<const uint4*>(qs + 32 * ks);
        // Wait for the queries inside this branch: otherwise the compiler waits for all vector-memory
        // operations where the branch rejoins, which on every step would drain the row prefetch.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        m = kNegInf;
        l = 0.f;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) O[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        seg_from_start = cc.k == 0;
        if (seg_from_start && blockIdx.y == 0 && tid == 0) {
            // This work-group holds the sequence's first unit: record which work-groups it spans.
            p.seq_meta[2 * cc.s] = w;
            p.seq_meta[2 * cc.s + 1] = (cc.g + cc.nu - 1) / per;
        }
    };

    auto end_segment = [&]() __attribute__((always_inline)) {
        const int c = lane & 15, g4 = lane >> 4;
        const bool whole = seg_from_start && cc.k + 1 == cc.nu;
        float L = l + __shfl_xor(l, 16);
        L += __shfl_xor(L, 32);
        // Output register j of a lane is head row 4 g4 + j; lane 4 g4 + j holds that row's (m, L).
        float Lr[4], Mr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            Lr[j] = __shfl(L, 4 * g4 + j);
            Mr[j] = __shfl(m, 4 * g4 + j);
        }
        const size_t row0 = (size_t)cc.s * Hq + head0 + 4 * g4;  // head row of register 0
        // A whole sequence writes its output; a segment of one writes its own normalised output
        // O / L in bf16 (to slot s + w) and its (m, L), which mla_merge_kernel weighs.
        const size_t idx0 = row0 + (size_t)w * Hq;  // slot s + w
        uint16_t* o = whole ? reinterpret_cast<uint16_t*>(p.out) + row0 * 512 + c : p.part_acc + idx0 * 512 + c;
        float inv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) inv[j] = Lr[j] > 0.f ? 1.f / Lr[j] : 0.f;
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[j * 512 + 16 * (dt0 + dt)] = (uint16_t)(pack2<true>(O[dt][j] * inv[j], 0.f) & 0xFFFFu);
            __builtin_amdgcn_sched_barrier(0);  // one tile at a time (see the rescale)
        }
        if (!whole && c == 0 && half == 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float2*>(p.part_ml + (idx0 + j) * 2) = make_float2(Mr[j], Lr[j]);
        }
    };

    // Scores, online softmax and PV of the unit in tile stage KT (validity vi), with the
    // dequantization of the next unit (raw stage KR2 -> tile stage KT2, validity vn) spread over the
    // PV slots. Each slot loads the next slot's LDS operands, then issues its own products; the
    // scheduling barriers keep the compiler from hoisting every operand load to the top, which would
    // need more registers than the queries and outputs leave free.
    auto compute = [&](auto kt, uint32_t vmask, auto kr2, auto kt2, uint32_t vn, auto ki4) __attribute__((always_inline)) {
        constexpr int KT = decltype(kt)::value;
        const char* tile = tile_stage<KT>();
        const float* scl = scale_stage<KT>() + 8 * (lane >> 4);  // this lane's 8 rows, group 0
        const int g4 = lane >> 4;

        // The dequantization of the next unit starts with its LDS reads, whose results are used
        // during PV.
        ConvIn cin;
        conv_load(kr2, cin);

        // Scores of this wave's own 16-token tile (t = half): 18 A operands, loaded kPre products
        // ahead. Order: the two RoPE k-steps (16, 17) into S, then the latent k-steps group by group
        // (g = 0..3: k-steps 4g .. 4g+3) into Sg[g & 1] (one accumulator per group, alternating, so
        // that a group's products run while the previous group's sums are scaled per row and added
        // to S). Register j holds token 16 half + g4 + 4j of head column c.
        constexpr int kPre = 4;
        constexpr int kA = kKSteps;
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        f32x4_t S = zero;
        f32x4_t Sg[2] = {zero, zero};
        auto ks_of = [](int x) constexpr { return x < 2 ? 16 + x : x - 2; };
        const char* atile = tile + half * kTile1;
        auto load_a = [&](int x) __attribute__((always_inline)) {
            const int ks = ks_of(x);
            return *reinterpret_cast<const uint4*>(atile + ((ks & 1) ? a_odd : a_even) + (ks >> 1) * 128);
        };
        uint4 aring[kPre];
#pragma unroll
        for (int i = 0; i < kPre; ++i) aring[i] = load_a(i);
        float4 sg;  // scales of the current group for this lane's rows j
#pragma unroll
        for (int x = 0; x < kA; ++x) {
            const uint4 a = aring[x % kPre];
            if (x + kPre < kA) aring[x % kPre] = load_a(x + kPre);
            if (x < 2) {
                S = mfma_k32<true>(a, qr[ks_of(x)], x == 0 ? zero : S);
            } else {
                const int y = x - 2, g = y >> 2, kk = y & 3;
                if (kk == 0) sg = *reinterpret_cast<const float4*>(scl + 32 * g + 4 * half);
                Sg[g & 1] = mfma_k32<true>(a, qr[ks_of(x)], kk == 0 ? zero : Sg[g & 1]);
                if (kk == 3) {
                    S[0] = fmaf(sg.x, Sg[g & 1][0], S[0]);
                    S[1] = fmaf(sg.y, Sg[g & 1][1], S[1]);
                    S[2] = fmaf(sg.z, Sg[g & 1][2], S[2]);
                    S[3] = fmaf(sg.w, Sg[g & 1][3], S[3]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }

        // Rows past the unit's valid ones (in the last unit of a sequence, or in an invalid block or
        // slot) are masked out.
        bool ok[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ok[jj] = (vmask >> (16 * half + g4 + 4 * jj)) & 1u;
        float mx = kNegInf;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) mx = ok[jj] ? fmaxf(mx, S[jj]) : mx;
        mx = row_max4(mx);
        // This tile's probabilities against the wave's own reference: the running reference m, moved
        // to the tile maximum if that exceeds it by more than kRescaleSlack (so p <= 2^kRescaleSlack).
        const float tmax = mx * sl2;
        const float m_own = tmax > m + kRescaleSlack ? tmax : m;
        float po[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float ex = fast_exp2(fmaf(S[jj], sl2, -m_own));
            po[jj] = ok[jj] ? ex : 0.f;
        }
        // Exchange with the wave that owns the same heads and the other tile: probabilities (token
        // g4 + 4j of the tile, head c at float (g4 + 4j) * 16 + c) and the reference per head.
        float* xo = s_xp[wave];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xo[(g4 + 4 * jj) * 16 + (lane & 15)] = po[jj];
        if (g4 == 0) s_xm[wave][lane] = m_own;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));  // own LDS writes done (copies may stay in flight)
        lds_barrier();
        // Every wave has read the raw stage of the unit it is dequantizing (conv_load, waited for
        // above): the next unit's copy can go there now, in the middle of the step, rather than with
        // every other wave's right after the step's opening barrier.
        issue(kr2, ki4, std::false_type{});
        const int partner = wave < kHeadWaves ? wave + kHeadWaves : wave - kHeadWaves;
        const float* xq = s_xp[partner];
        float pq[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pq[jj] = xq[(g4 + 4 * jj) * 16 + (lane & 15)];
        const float m_par = s_xm[partner][lane & 15];
        // Common reference: the larger of the two (both waves compute the same value, and from it
        // the same factors and probabilities, bit for bit).
        const float m_new = fmaxf(m_own, m_par);
        const float f_own = m_own == m_new ? 1.f : fast_exp2(m_own - m_new);
        const float f_par = m_par == m_new ? 1.f : fast_exp2(m_par - m_new);
        const bool need = m_new > m;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(need) != 0, 0)) {
            const float alpha = need ? fast_exp2(m - m_new) : 1.f;
            l *= alpha;
            const f32x4_t av = {__shfl(alpha, 4 * g4), __shfl(alpha, 4 * g4 + 1), __shfl(alpha, 4 * g4 + 2),
                                __shfl(alpha, 4 * g4 + 3)};
            // One output tile at a time: the scheduling barriers keep the compiler from reading every
            // output into fresh registers at once.
#pragma unroll
            for (int dt = 0; dt < kDimTiles; ++dt) {
                O[dt] *= av;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        m = m_new;
        // Tile 0 and tile 1 probabilities against m, summed into l in that order by both waves.
        float pr[2][4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float a0 = po[jj] * f_own, a1 = pq[jj] * f_par;
            pr[0][jj] = half == 0 ? a0 : a1;
            pr[1][jj] = half == 0 ? a1 : a0;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) l += pr[t][jj];
        // PV A operands: p times the row's scale of each of this wave's two output groups.
        uint4 Ag[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const float* sp = scl + 32 * (2 * half + k);
            const float4 s0 = *reinterpret_cast<const float4*>(sp);
            const float4 s1 = *reinterpret_cast<const float4*>(sp + 4);
            Ag[k] = make_uint4(pack2<true>(pr[0][0] * s0.x, pr[0][1] * s0.y), pack2<true>(pr[0][2] * s0.z, pr[0][3] * s0.w),
                               pack2<true>(pr[1][0] * s1.x, pr[1][1] * s1.y), pack2<true>(pr[1][2] * s1.z, pr[1][3] * s1.w));
        }

        // PV: one 16-dim output tile per product; its B operand is two transposed reads (tile rows
        // 0..15 and 16..31). The dequantization of the next unit is spread over eight groups of four.
        constexpr int kGroups = kLatentIters < 8 ? kLatentIters : 8;
        constexpr int kConvPerGroup = (kLatentIters + kGroups - 1) / kGroups;
        constexpr int kTilesPerGroup = kDimTiles / kGroups;
        const char* vtile = tile + half * (kDimTiles / 4) * 128;  // this wave's output dims
        auto load_b = [&](int dt) __attribute__((always_inline)) {
            const char* base = vtile + trbase[dt & 3] + (dt >> 2) * 128;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)(base));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)(base + kTile1));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            return make_uint4(l2.x, l2.y, h2.x, h2.y);
        };
        uint4 bring[kPre];
#pragma unroll
        for (int i = 0; i < kPre; ++i) bring[i] = load_b(i);
#pragma unroll
        for (int dt = 0; dt < kDimTiles; ++dt) {
            const uint4 bop = bring[dt % kPre];
            if (dt + kPre < kDimTiles) bring[dt % kPre] = load_b(dt + kPre);
            O[dt] = mfma_k32<true>(Ag[dt / (kDimTiles / 2)], bop, O[dt]);
            if constexpr (kSpread) {
#pragma unroll
                for (int r = 1; r < R; ++r)
                    if (dt == (r * kDimTiles) / R) copy_rows(r);  // the rest of the next unit's copies
            }
            if (dt % kTilesPerGroup == kTilesPerGroup - 1)
                conv_store(kr2, kt2, vn, cin, (dt / kTilesPerGroup) * kConvPerGroup,
                           std::integral_constant<int, kConvPerGroup>{}, dt == kDimTiles - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Step of unit u (K = u % 6; raw stage u % 3, tile stage u % 2): wait for unit u+1's rows,
    // compute unit u while dequantizing unit u+1, and (inside compute, once the raw stage of unit u+1
    // is read) start loading unit u+4 into it. Returns false when the range is done.
    auto step = [&](auto kst) __attribute__((always_inline)) -> bool {
        constexpr int K = decltype(kst)::value;
        constexpr int KR = K % 3, KT = K & 1, KR2 = (K + 1) % 3, KT2 = (K + 1) & 1;
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * RL));  // own loads of unit u+1 are done
        compiler_fence();
        __builtin_amdgcn_s_barrier();                          // everyone's are; step u-1 is finished
        compiler_fence();
        const uint32_t cur = info[K];
        const uint32_t nxt = info[(K + 1) % 6];
        refresh_offsets();
        if (__builtin_expect(cc.g == g_begin || cc.k == 0, 0)) begin_segment();
        compute(std::integral_constant<int, KT>{}, cur, std::integral_constant<int, KR2>{},
                std::integral_constant<int, KT2>{}, nxt, std::integral_constant<int, (K + 4) % 6>{});
        if (__builtin_expect(cc.g + 1 == g_end || cc.k + 1 == cc.nu, 0)) end_segment();
        advance(cc, p);
        prefetch_ids();
        return cc.g < g_end;
    };

    // Prologue: units 0..2 in flight, unit 0 dequantized, then unit 3 in flight in its raw stage. The
    // sparse form first copies the slot tables of units 0..2 and waits for them.
    if constexpr (SPARSE) {
#pragma unroll
        for (int i = 0; i < 3; ++i) copy_slot_table();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        lds_barrier();
    }
    prefetch_ids();
    issue(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, std::true_type{});
    prefetch_ids();
    issue(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, std::true_type{});
    prefetch_ids();
    issue(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{}, std::true_type{});
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * RL));
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    {
        ConvIn cin;
        conv_load(std::integral_constant<int, 0>{}, cin);
        conv_store(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, info[0], cin, 0,
                   std::integral_constant<int, kLatentIters>{}, true);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));  // own reads of raw stage 0 are done
    lds_barrier();                                     // everyone's are
    prefetch_ids();
    issue(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{}, std::true_type{});
    prefetch_ids();

    while (true) {
        if (!step(std::integral_constant<int, 0>{})) break;
        if (!step(std::integral_constant<int, 1>{})) break;
        if (!step(std::integral_constant<int, 2>{})) break;
        if (!step(std::integral_constant<int, 3>{})) break;
        if (!step(std::integral_constant<int, 4>{})) break;
        if (!step(std::integral_constant<int, 5>{})) break;
    }
    // Drain: the loads issued for units past the range still target this work-group's LDS.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
}

}  // namespace pa

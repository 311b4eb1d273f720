// Paged decode for grouped-query attention on the matrix cores (head_dim 128, 2..16 query heads per
// K/V head).
//
// What is computed is the same as in decode_dense.hip: for each query head h and its K/V head
// h / G, softmax over the block-table-gathered context, weighted sum of V ("deep dive into vLLM 05"
// §2 and §3.2; "KV Cache 与推理服务内存管理", paged_attention). When several query heads share one
// K/V head, each 16-token tile is a small dense product, [tokens x 128] . [128 x G], followed by
// [G x tokens] . [tokens x 128]. Done on the VALU, the cross-lane reductions and per-head work
// grow with G and dominate the instruction stream. Here both products run as MFMA, and the VALU
// keeps only the softmax bookkeeping.
//
// One wave owns one (K/V head, sequence, partition) item: a 16-row MFMA tile whose rows are the G
// query heads (rows G..15 are zero padding). Per 16-token tile:
//   Scores, S^T = K . Q^T: v_mfma_f32_16x16x32 (4 k-steps over 128 dims). The A operand is K: lane l
//     holds 8 consecutive dims (16 bytes) of token sigma(l%16). The B operand is Q, held in
//     registers for the whole item. Output lane l holds head l%16 and 4 tokens.
//   The M order sigma(m) = m/4 + 4*(m%4) makes lane group g = l/16 hold tokens g, g+4, g+8, g+12,
//   which are the rows its V registers hold. So the probabilities are the A operand of the PV
//   product exactly as they come out of the softmax.
//   PV, O += P . V: v_mfma_f32_16x16x16, one per dim lane-offset e = 0..7, covering dims
//     {8c + e : c = 0..15}. Its B operand (4 tokens of one dim) is two v_perm_b32 of the loaded V rows;
//     the cache layout never has to be transposed.
// The reduction (k) order inside each MFMA is the same for both operands by construction, so the
// exact k layout of the instruction does not matter.
//
// Softmax: lazily moved reference m per head (see decode_common.h), masked tokens get p = 0 and
// their V rows are zeroed, partitions and their merge as in decode_dense.hip.
//
// Device code shared by decode_mfma.hip (the decode kernel) and prefill_mfma.hip (which runs the
// decode rows of a mixed call in the same launch as its chunk rows). Included only by .hip files.

#pragma once

#include <type_traits>

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

template <bool BF16>
__device__ __forceinline__ void mfma_tile_step(const uint4 (&kk)[4], uint4 (&vv)[4], const uint4 (&qb)[4], float& m,
                                               float& l, f32x4_t (&O)[8], int g4, int nvalid, float scale_log2) {
    f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) S = mfma_k32<BF16>(kk[ks], qb[ks], S);
    // S[j]: raw score of this lane's head (l % 16) against token g4 + 4j of the tile.
    bool ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ok[j] = g4 + 4 * j < nvalid;
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = ok[j] ? fmaxf(mx, S[j]) : mx;
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float tmax = mx * scale_log2;
    const bool need = tmax > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float mnew = need ? tmax : m;
        const float alpha = need ? fast_exp2(m - mnew) : 1.f;
        l *= alpha;
        m = mnew;
        // O rows of this lane are heads 4*g4 + j; their factors live in lanes 4*g4 + j.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float a = __shfl(alpha, 4 * g4 + j);
#pragma unroll
            for (int e = 0; e < 8; ++e) O[e][j] *= a;
        }
    }
    float pr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float e = fast_exp2(fmaf(S[j], scale_log2, -m));
        pr[j] = ok[j] ? e : 0.f;
        l += pr[j];
    }
    uint2 A, Alo;
    pack2_split<BF16>(pr[0], pr[1], A.x, Alo.x);
    pack2_split<BF16>(pr[2], pr[3], A.y, Alo.y);
#pragma unroll
    for (int i = 0; i < 4; ++i)  // rows past the context may hold NaN, and 0 * NaN = NaN
        if (!ok[i]) vv[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint2 B = v_operand(vv, e);
        O[e] = mfma_k16<BF16>(A, B, O[e]);
        if constexpr (BF16) O[e] = mfma_k16<BF16>(Alo, B, O[e]);
    }
}

typedef unsigned int u32x2_dm_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes -> 8 bf16 values (exact).
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 w) {
    return make_uint4(e4m3x2_bf16<false>(w.x), e4m3x2_bf16<true>(w.x), e4m3x2_bf16<false>(w.y),
                      e4m3x2_bf16<true>(w.y));
}

__device__ __forceinline__ uint2 load_nt8(const char* ptr) {
    const u32x2_dm_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x2_dm_t*>(ptr));
    return make_uint2(a.x, a.y);
}

}  // namespace

// One wave's work item of the grouped-query decode: item = (partition-major work index) * Hkv + K/V head.
// FP8: E4M3 rows (one byte per value, bf16 queries and outputs). The same operand layouts are
// loaded at half the width (8 bytes per lane instead of 16) and widened to bf16 when used, so the
// products are those of the bf16 path on the exactly dequantized codes; K's scale is in
// scale_log2 and V's multiplies the accumulators at the end.
template <bool BF16, bool FP8 = false>
__device__ __forceinline__ void decode_mfma_wave(const DenseDecodeParams& p, int item) {
    static_assert(!FP8 || BF16, "FP8 rows take bf16 queries");
    using Raw = std::conditional_t<FP8, uint2, uint4>;
    constexpr int kEsz = FP8 ? 1 : 2;  // bytes per cached value
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4;
    const int c = lane & 15;

    const int kvh = item % p.num_kv_heads;
    int s, part;
    int ctx;
    if (!find_work(item / p.num_kv_heads, p, s, part, ctx)) return;

    const int G = p.group;
    const int bs = p.block_size;
    const int P = p.partition_tokens;
    const int nparts = (ctx + P - 1) / P;
    const int hq0 = kvh * G;
    const int qr = query_row(s, p);
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)qr * p.num_q_heads + hq0) * kD;

    if (ctx == 0) {
        for (int h = g4; h < G; h += 4)
            *reinterpret_cast<uint4*>(out + ((size_t)qr * p.num_q_heads + hq0 + h) * kD + c * 8) = make_uint4(0, 0, 0, 0);
        return;
    }
    if (part >= nparts) return;
    const int tb = part * P;
    const int te = min(ctx, tb + P);

    // Q as the B operand of the score MFMA: lane (g4, c) holds head c, dims 32*ks + 8*g4 .. +7 for
    // 16-bit rows. For FP8 rows the k order is permuted so that a lane's K operands of k-steps 2h and
    // 2h+1 are 16 consecutive codes (one 16-byte load): dims 64*(ks/2) + 16*g4 + 8*(ks%2) .. +7. The
    // order of k inside a product is free as long as both operands follow it.
    uint4 qb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int d0 = FP8 ? 64 * (ks >> 1) + 16 * g4 + 8 * (ks & 1) : 32 * ks + 8 * g4;
        qb[ks] = c < G ? *reinterpret_cast<const uint4*>(qrow + c * kD + d0) : make_uint4(0, 0, 0, 0);
    }

    const int tpb_log2 = p.tiles_per_block_log2;
    const int tpb_mask = (1 << tpb_log2) - 1;
    const int lb0 = tb >> (tpb_log2 + 4);
    const int nblk = (te - tb + bs - 1) >> (tpb_log2 + 4);
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const int tbl = lane < nblk ? bt[lb0 + lane] : 0;

    const int64_t krow = p.k_row_bytes, vrow = p.v_row_bytes;
    // K: token sigma(c), dims 8*g4 (+32 per k-step), or for FP8 dims 16*g4 (+64 per 16-byte load);
    // V: token g4 (+4 per load), dims 8*c.
    const uint32_t klane = (uint32_t)(kvh * (kD * kEsz) + (FP8 ? 16 : 8 * kEsz) * g4) + (uint32_t)sigma(c) * (uint32_t)krow;
    const uint32_t vlane = (uint32_t)(kvh * (kD * kEsz) + 8 * kEsz * c) + (uint32_t)g4 * (uint32_t)vrow;
    const uint32_t nb = (uint32_t)p.num_blocks;
    const int ntiles = (te - tb + 15) >> 4;
    const int last = ntiles - 1;
    const char* dummy = reinterpret_cast<const char*>(qrow);

    auto block_of = [&](int j) { return __builtin_amdgcn_readlane(tbl, j >> tpb_log2); };
    auto load = [&](Raw (&kk)[4], Raw (&vv)[4], int j) {
        const bool real = j <= last;
        int phys = block_of(real ? j : last);
        phys = ((uint32_t)phys < nb) ? phys : 0;
        const int64_t row0 = (int64_t)((j & tpb_mask) << 4);
        const char* kt = real ? p.k + (int64_t)phys * p.k_block_stride + row0 * krow : dummy;
        const char* vt = real ? p.v + (int64_t)phys * p.v_block_stride + row0 * vrow : dummy;
        const int64_t kstep = real ? 32 * kEsz : 0, vstep = real ? 4 * vrow : 0;
        const uint32_t ko = real ? klane : 0u, vo = real ? vlane : 0u;
        // K through the cache: an operand load covers a quarter or half of a head's row, so the row's
        // lines are shared by consecutive loads. V (whole head rows per lane group) streams
        // nontemporally.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (FP8) {
                if ((i & 1) == 0) {  // k-steps i and i + 1: one 16-byte load
                    const uint4 w = *reinterpret_cast<const uint4*>(kt + (real ? 64 * (i >> 1) : 0) + ko);
                    kk[i] = make_uint2(w.x, w.y);
                    kk[i + 1] = make_uint2(w.z, w.w);
                }
                vv[i] = load_nt8(vt + i * vstep + vo);
            } else {
                kk[i] = *reinterpret_cast<const uint4*>(kt + i * kstep + ko);
                vv[i] = load_nt16(vt + i * vstep + vo);
            }
        }
    };

    float m = kNegInf, l = 0.f;
    f32x4_t O[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) O[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const Raw (&kk)[4], Raw (&vv)[4], int j) {
        int nvalid = min(16, te - (tb + (j << 4)));
        if ((uint32_t)block_of(j) >= nb) nvalid = 0;
        if constexpr (FP8) {
            uint4 kw[4], vw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kw[i] = e4m3x8_to_bf16(kk[i]);
                vw[i] = e4m3x8_to_bf16(vv[i]);
            }
            mfma_tile_step<true>(kw, vw, qb, m, l, O, g4, nvalid, p.scale_log2);
        } else {
            mfma_tile_step<BF16>(kk, vv, qb, m, l, O, g4, nvalid, p.scale_log2);
        }
    };

    // A ring of kDepth tiles: the loads of the next kDepth - 1 tiles are in flight while one is
    // computed. FP8 tiles are half the bytes, so they keep twice as many in flight.
    constexpr int kDepth = FP8 ? 4 : 2;
    Raw kb[kDepth][4], vb[kDepth][4];
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i) load(kb[i], vb[i], i);
    for (int j = 0; j < ntiles; j += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            load(kb[(u + kDepth - 1) % kDepth], vb[(u + kDepth - 1) % kDepth], j + u + kDepth - 1);
            if (u == 0 || j + u < ntiles) step(kb[u], vb[u], j + u);
        }
    }

    // l summed over the four lane groups gives each head's total; O rows are heads 4*g4 + j.
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int h = 4 * g4 + j;
        const float L = __shfl(l, h);
        const float M = __shfl(m, h);
        if (h >= G) continue;
        if constexpr (FP8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) O[e][j] *= p.v_scale;
        }
        if (nparts == 1) {
            const float inv = 1.f / L;
            uint4 o;
            o.x = pack2<BF16>(O[0][j] * inv, O[1][j] * inv);
            o.y = pack2<BF16>(O[2][j] * inv, O[3][j] * inv);
            o.z = pack2<BF16>(O[4][j] * inv, O[5][j] * inv);
            o.w = pack2<BF16>(O[6][j] * inv, O[7][j] * inv);
            *reinterpret_cast<uint4*>(out + ((size_t)qr * p.num_q_heads + hq0 + h) * kD + c * 8) = o;
        } else {
            const size_t idx = ((size_t)s * p.num_q_heads + hq0 + h) * p.max_parts + part;
            float4* pa = reinterpret_cast<float4*>(p.part_acc + idx * kD + c * 8);
            pa[0] = make_float4(O[0][j], O[1][j], O[2][j], O[3][j]);
            pa[1] = make_float4(O[4][j], O[5][j], O[6][j], O[7][j]);
            if (c == 0) *reinterpret_cast<float2*>(p.part_ml + idx * 2) = make_float2(M, L);
        }
    }
}

}  // namespace pa

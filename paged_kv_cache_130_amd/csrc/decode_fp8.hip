// Paged decode over FP8 (OCP E4M3) dense rows: dequantize-on-read inside the attention kernel.
//
// "deep dive into vLLM 05" §3.4: the KV cache can be stored at low precision (quantize on write) and
// dequantized when read, inside the attention kernel; FP8 is the safest format. A row holds one E4M3
// byte per value, and each cache has one float32 scale (value = code * scale). The attention itself
// is the paged decode of decode_dense.hip ("deep dive into vLLM 05" §2; "KV Cache 与推理服务内存管理",
// paged_attention): block-table gather, scores, online softmax, weighted V, split-context
// partitions merged by decode_reduce_kernel. Queries and outputs are bf16.
//
// Mapping onto CDNA4 (the same work decomposition as the 16-bit vector kernel):
//  * One wave owns one (KV head, sequence, partition) item and all G query heads of that KV head.
//  * A lane holds 16 bytes = 16 values of one row: LPR = D/16 lanes cover a head's row, and one
//    wave-wide 16-byte load covers RPL = 64/LPR rows. Half the bytes of a 16-bit cache per token.
//  * v_cvt_pk_f32_fp8 turns two codes into two exact fp32 values. Every E4M3 value is exactly a
//    bf16 value too (4 significant bits, exponents -9..8), so K goes on as bf16 pairs (two codes per
//    v_cvt_scalef32_pk_bf16_fp8 with scale 1) into
//    v_dot2_f32_bf16 against the bf16 query (exact products, fp32 sums), and V as fp32 into fp32
//    multiply-adds with the fp32 probabilities (no rounding of p).
//  * The scales are applied outside the loops: K's scale is folded into the softmax scale, and V's
//    multiplies the accumulators once per item.

#include "decode_common.h"

namespace pa {

namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct F8Tile {
    static constexpr int LPR = D / 16;    // lanes per head row
    static constexpr int RPL = 64 / LPR;  // rows per wave-wide load
    static constexpr int NL = 16 / RPL;   // loads per 16-token tile
    static_assert(NL >= 1 && RPL * NL == 16, "tile shape");
};

// 4 codes (one dword) -> 4 exact fp32 values.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    o[0] = a.x;
    o[1] = a.y;
    o[2] = b.x;
    o[3] = b.y;
}

// 16 codes -> 8 bf16 pairs (exact).
__device__ __forceinline__ void e4m3x16_to_bf16x2(const uint4& w, uint32_t (&o)[8]) {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = e4m3x2_bf16<false>(ws[i]);
        o[2 * i + 1] = e4m3x2_bf16<true>(ws[i]);
    }
}

template <int D, int G, bool MASK>
__device__ __forceinline__ void f8_tile_step(const uint4 (&kr)[F8Tile<D>::NL], uint4 (&vr)[F8Tile<D>::NL],
                                             const uint32_t (&qr)[G][8], float (&m)[G], float (&l)[G],
                                             float (&acc)[G][16], int r, int nvalid, float scale_log2) {
    using T = F8Tile<D>;
    constexpr int NL = T::NL, RPL = T::RPL, LPR = T::LPR;
    float sc[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        uint32_t kp[8];
        e4m3x16_to_bf16x2(kr[i], kp);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                d0 = dot2acc<true>(qr[g][j], kp[j], d0);
                d1 = dot2acc<true>(qr[g][j + 1], kp[j + 1], d1);
            }
            sc[g][i] = group_sum<LPR>(d0 + d1);
        }
    }
    bool ok[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) ok[i] = !MASK || (r + i * RPL < nvalid);
    bool need_any = false;
    float tmax[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = kNegInf;
#pragma unroll
        for (int i = 0; i < NL; ++i) mx = ok[i] ? fmaxf(mx, sc[g][i]) : mx;
        tmax[g] = mx * scale_log2;  // scale >= 0, so the maximum commutes with the scaling
        need_any |= tmax[g] > m[g] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const bool need = tmax[g] > m[g] + kRescaleSlack;
            const float mnew = need ? tmax[g] : m[g];
            const float alpha = need ? fast_exp2(m[g] - mnew) : 1.f;  // m = -inf gives 0
            l[g] *= alpha;
#pragma unroll
            for (int d = 0; d < 16; ++d) acc[g][d] *= alpha;
            m[g] = mnew;
        }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        // Rows past the context may hold NaN codes, and 0 * NaN = NaN: zero them.
        if (MASK && !ok[i]) vr[i] = make_uint4(0u, 0u, 0u, 0u);
        float v[16];
        e4m3x4_to_f32(vr[i].x, v);
        e4m3x4_to_f32(vr[i].y, v + 4);
        e4m3x4_to_f32(vr[i].z, v + 8);
        e4m3x4_to_f32(vr[i].w, v + 12);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float e = fast_exp2(fmaf(sc[g][i], scale_log2, -m[g]));
            const float pr = ok[i] ? e : 0.f;
            l[g] += pr;
#pragma unroll
            for (int d = 0; d < 16; ++d) acc[g][d] = fmaf(pr, v[d], acc[g][d]);
        }
    }
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(256) void decode_fp8_kernel(DenseDecodeParams p) {
    using T = F8Tile<D>;
    constexpr int LPR = T::LPR, RPL = T::RPL, NL = T::NL;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane / LPR;
    const int c = lane % LPR;

    const int item = blockIdx.x * 4 + wave;
    const int kvh = item % p.num_kv_heads;
    int s, part;
    int ctx;
    if (!find_work(item / p.num_kv_heads, p, s, part, ctx)) return;
    const int bs = p.block_size;
    const int P = p.partition_tokens;
    const int nparts = (ctx + P - 1) / P;
    const int hq0 = kvh * G;
    const int qrow_idx = query_row(s, p);
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);

    if (ctx == 0) {  // empty context: output 0
        if (part == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if ((g % RPL) == r) {
                    uint4* o = reinterpret_cast<uint4*>(out + ((size_t)qrow_idx * p.num_q_heads + hq0 + g) * D + c * 16);
                    o[0] = make_uint4(0, 0, 0, 0);
                    o[1] = make_uint4(0, 0, 0, 0);
                }
        }
        return;
    }
    if (part >= nparts) return;
    const int tb = part * P;
    const int te = min(ctx, tb + P);

    // Query: 16 bf16 values of each of the G heads, as 8 pairs.
    uint32_t qr[G][8];
    const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)qrow_idx * p.num_q_heads + hq0) * D + c * 16;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint4 a = *reinterpret_cast<const uint4*>(qsrc + g * D);
        const uint4 b = *reinterpret_cast<const uint4*>(qsrc + g * D + 8);
        qr[g][0] = a.x; qr[g][1] = a.y; qr[g][2] = a.z; qr[g][3] = a.w;
        qr[g][4] = b.x; qr[g][5] = b.y; qr[g][6] = b.z; qr[g][7] = b.w;
    }

    const int lb0 = tb >> (p.tiles_per_block_log2 + 4);
    const int nblk = (te - tb + bs - 1) >> (p.tiles_per_block_log2 + 4);  // <= 64 by construction
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const int tbl = lane < nblk ? bt[lb0 + lane] : 0;

    const int64_t krow = p.k_row_bytes, vrow = p.v_row_bytes;
    const int kvs = kvh >> p.kv_shift;  // the stored K/V head
    const uint32_t klane = (uint32_t)(kvs * D + c * 16) + (uint32_t)r * (uint32_t)krow;
    const uint32_t vlane = (uint32_t)(kvs * D + c * 16) + (uint32_t)r * (uint32_t)vrow;
    const uint32_t nb = (uint32_t)p.num_blocks;
    const int tpb_log2 = p.tiles_per_block_log2;
    const int tpb_mask = (1 << tpb_log2) - 1;

    float m[G], l[G], acc[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int d = 0; d < 16; ++d) acc[g][d] = 0.f;
    }

    const int ntiles = (te - tb + 15) >> 4;
    const int last = ntiles - 1;
    auto block_of = [&](int j) __attribute__((always_inline)) { return __builtin_amdgcn_readlane(tbl, j >> tpb_log2); };
    // Tile j > last is a dummy: every lane reads the same (cached) bytes of the query row.
    const char* dummy = reinterpret_cast<const char*>(qsrc - c * 16);
    auto load = [&](uint4 (&kk)[NL], uint4 (&vv)[NL], int j) __attribute__((always_inline)) {
        const bool real = j <= last;
        int phys = block_of(real ? j : last);
        phys = ((uint32_t)phys < nb) ? phys : 0;  // an out-of-range id is masked when the tile is used
        const int64_t row0 = (int64_t)((j & tpb_mask) << 4);
        const char* kt = real ? p.k + (int64_t)phys * p.k_block_stride + row0 * krow : dummy;
        const char* vt = real ? p.v + (int64_t)phys * p.v_block_stride + row0 * vrow : dummy;
        const int64_t kstep = real ? (int64_t)RPL * krow : 0, vstep = real ? (int64_t)RPL * vrow : 0;
        const uint32_t ko = real ? klane : 0u, vo = real ? vlane : 0u;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            kk[i] = load_nt16(kt + i * kstep + ko);
            vv[i] = load_nt16(vt + i * vstep + vo);
        }
    };
    auto step = [&](const uint4 (&kk)[NL], uint4 (&vv)[NL], int j) __attribute__((always_inline)) {
        int nvalid = min(16, te - (tb + (j << 4)));
        if ((uint32_t)block_of(j) >= nb) nvalid = 0;
        if (nvalid == 16)
            f8_tile_step<D, G, false>(kk, vv, qr, m, l, acc, r, 16, p.scale_log2);
        else
            f8_tile_step<D, G, true>(kk, vv, qr, m, l, acc, r, nvalid, p.scale_log2);
    };

    // A ring of kDepth tiles: the loads of the next kDepth - 1 tiles are in flight while one is
    // computed (loads past the last tile read the cached dummy row).
    constexpr int kDepth = 2;
    uint4 kb[kDepth][NL], vb[kDepth][NL];
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i) load(kb[i], vb[i], i);
    for (int j = 0; j < ntiles; j += kDepth) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
            load(kb[(u + kDepth - 1) % kDepth], vb[(u + kDepth - 1) % kDepth], j + u + kDepth - 1);
            if (u == 0 || j + u < ntiles) step(kb[u], vb[u], j + u);
        }
    }

    // Merge the RPL row groups of the wave (lanes that differ only in r), then apply V's scale.
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float M = m[g];
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float f = fast_exp2(m[g] - (M == kNegInf ? 0.f : M));
        float L = l[g] * f;
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) L += __shfl_xor(L, off);
#pragma unroll
        for (int d = 0; d < 16; ++d) {
            float a = acc[g][d] * f;
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) a += __shfl_xor(a, off);
            acc[g][d] = a * p.v_scale;
        }
        m[g] = M;
        l[g] = L;
    }

    if (nparts == 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if ((g % RPL) != r) continue;
            const float inv = 1.f / l[g];
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = pack2<true>(acc[g][2 * j] * inv, acc[g][2 * j + 1] * inv);
            uint4* o = reinterpret_cast<uint4*>(out + ((size_t)qrow_idx * p.num_q_heads + hq0 + g) * D + c * 16);
            o[0] = make_uint4(w[0], w[1], w[2], w[3]);
            o[1] = make_uint4(w[4], w[5], w[6], w[7]);
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if ((g % RPL) != r) continue;
            const size_t idx = ((size_t)s * p.num_q_heads + hq0 + g) * p.max_parts + part;
            float4* pa = reinterpret_cast<float4*>(p.part_acc + idx * D + c * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pa[j] = make_float4(acc[g][4 * j], acc[g][4 * j + 1], acc[g][4 * j + 2], acc[g][4 * j + 3]);
            if (c == 0) *reinterpret_cast<float2*>(p.part_ml + idx * 2) = make_float2(m[g], l[g]);
        }
    }
}

namespace {

template <int D, int G>
hipError_t launch_f8(const DenseDecodeParams& p, hipStream_t stream) {
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    hipLaunchKernelGGL((decode_fp8_kernel<D, G>), dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.max_parts <= 1) return e;
    return launch_decode_reduce(p, stream);
}

template <int D>
hipError_t launch_f8_group(const DenseDecodeParams& p, hipStream_t stream) {
    switch (p.group) {
        case 1: return launch_f8<D, 1>(p, stream);
        case 2: return launch_f8<D, 2>(p, stream);
        case 4: return launch_f8<D, 4>(p, stream);
        case 8: {
            // Two waves of four query heads each per K/V head (an eight-head wave would need more
            // than its 512 registers); the host counts these items (kv_waves in api.hip).
            DenseDecodeParams q = p;
            q.num_kv_heads = p.num_kv_heads * 2;
            q.group = 4;
            q.kv_shift = 1;
            return launch_f8<D, 4>(q, stream);
        }
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_fp8(const DenseDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    switch (p.head_dim) {
        case 64: return launch_f8_group<64>(p, stream);
        // Grouped heads at head_dim 128 run on the matrix cores (launch_decode_dense).
        case 128: return p.group == 1 ? launch_f8<128, 1>(p, stream) : hipErrorInvalidValue;
        case 256: return launch_f8_group<256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa

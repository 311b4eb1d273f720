// MLA latent decode over packed 656-byte rows: 128 query heads on one latent K/V head.
//
// "deep dive into vLLM 05" §3.3: MLA caches only a low-dimensional latent per token. With the
// up-projection folded into the query, attention runs in latent space and the cache is never
// decompressed. "vLLM KV Cache Layout 可视化" (section on two caches sharing one block table) gives
// the row: 512 B of FP8 latent, 16 B of scale, 128 B of BF16 RoPE. Here, as in the reading documented
// with the C ABI, the row is 512 e4m3 latent values, 4 float32 scales (scale k for latent values
// [128k, 128k+128)) and 64 bf16 RoPE values. The scores use [latent | rope] (576 dims). The value is
// the dequantized 512-dim latent:
//     s_t = scale * (q_lat . (c_t * sc_t) + q_rope . r_t),   out = sum_t p_t (c_t * sc_t).
//
// Mapping (the operand orders of decode_mfma.hip, see mfma_common.h): one wave owns 16 query heads of
// one sequence and one split-context partition. Per 16-token tile:
//   scores  S^T = K . Q^T on v_mfma_f32_16x16x32_bf16. The A operand is K: lane l holds 8 latent
//           bytes (or 8 RoPE values) of token sigma(l%16), converted e4m3 -> bf16 exactly
//           (v_cvt_scalef32_pk_bf16_fp8 with scale 1). The B operand is Q, from LDS. The four
//           128-dim latent groups accumulate separately and are combined in fp32 with each token's
//           own scales, so the dequantization is exact.
//   PV      O += P . V on v_mfma_f32_16x16x16_bf16, per 128-dim quarter q: A = P scaled by the
//           tokens' scale q, B = two v_perm_b32 of the converted latent bytes (4 tokens x 1 dim).
// Output O (16 heads x 512 dims) lives in 128 accumulator registers. Partitions and their merge are
// those of the dense decode (decode_reduce_kernel at 512 dims).

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

constexpr int kMlaRow = 656;       // bytes per token row
constexpr int kMlaScaleOff = 512;  // 4 x float32
constexpr int kMlaRopeOff = 528;   // 64 x bf16
constexpr int kMlaV = 512;         // latent (value) dims
constexpr int kMlaK = 18;          // k-steps of 32 dims over 576 score dims (16 latent + 2 RoPE)

// Four e4m3 bytes -> four bf16 (exact: every e4m3 value is representable in bf16).
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint2 w) {
    const uint2 a = e4m3x4_to_bf16(w.x), b = e4m3x4_to_bf16(w.y);
    return make_uint4(a.x, a.y, b.x, b.y);
}

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_mla_kernel(DenseDecodeParams p) {
    __shared__ uint4 q_lds[4][kMlaK][64];  // per wave: its 16 heads' query as score B operands

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4;
    const int c = lane & 15;

    const int item = blockIdx.x * 4 + wave;
    const int hg = item % p.num_kv_heads;  // group of 16 query heads
    int s, part;
    if (!find_work(item / p.num_kv_heads, p, s, part)) return;

    const int bs = p.block_size;
    const int ctx = clamp_context(__builtin_amdgcn_readfirstlane(p.context_lens[s]), p);
    const int P = p.partition_tokens;
    const int nparts = (ctx + P - 1) / P;
    const int h0 = hg * 16;
    const int qrow_idx = query_row(s, p);
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);

    if (ctx == 0) {
        for (int h = g4; h < 16; h += 4)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4*>(out + ((size_t)qrow_idx * p.num_q_heads + h0 + h) * kMlaV + 128 * q + 8 * c) =
                    make_uint4(0, 0, 0, 0);
        return;
    }
    if (part >= nparts) return;
    const int tb = part * P;
    const int te = min(ctx, tb + P);

    // Query of head h0 + c, dims 32*ks + 8*g4 .. +7, into this wave's LDS slice.
    const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)qrow_idx * p.num_q_heads + h0 + c) * 576;
#pragma unroll
    for (int ks = 0; ks < kMlaK; ++ks) q_lds[wave][ks][lane] = *reinterpret_cast<const uint4*>(qsrc + 32 * ks + 8 * g4);

    const int tpb_log2 = p.tiles_per_block_log2;
    const int tpb_mask = (1 << tpb_log2) - 1;
    const int lb0 = tb >> (tpb_log2 + 4);
    const int nblk = (te - tb + bs - 1) >> (tpb_log2 + 4);
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const int tbl = lane < nblk ? bt[lb0 + lane] : 0;
    const uint32_t nb = (uint32_t)p.num_blocks;
    const int ntiles = (te - tb + 15) >> 4;
    const float sl2 = p.scale_log2;

    float m = kNegInf, l = 0.f;
    f32x4_t O[4][8];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) O[q][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j < ntiles; ++j) {
        int phys = __builtin_amdgcn_readlane(tbl, j >> tpb_log2);
        const bool bad = (uint32_t)phys >= nb;
        phys = bad ? 0 : phys;
        const int nvalid = bad ? 0 : min(16, te - (tb + (j << 4)));
        const char* tile = p.k + (int64_t)phys * p.k_block_stride + (int64_t)((j & tpb_mask) << 4) * kMlaRow;

        // Scores, one accumulator per 128-dim latent group plus one for RoPE.
        const char* krow = tile + sigma(c) * kMlaRow;
        f32x4_t Sg[4], Sr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            Sg[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k4 = 0; k4 < 4; ++k4) {
                const int ks = 4 * g + k4;
                const uint2 raw = *reinterpret_cast<const uint2*>(krow + 32 * ks + 8 * g4);
                Sg[g] = mfma_k32<true>(e4m3x8_to_bf16(raw), q_lds[wave][ks][lane], Sg[g]);
            }
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const uint4 rope = *reinterpret_cast<const uint4*>(krow + kMlaRopeOff + 64 * k2 + 16 * g4);
            Sr = mfma_k32<true>(rope, q_lds[wave][16 + k2][lane], Sr);
        }
        // Output register jj holds token g4 + 4*jj; its four scales.
        bool ok[4];
        float4 sc[4];
        float S[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            ok[jj] = g4 + 4 * jj < nvalid;
            sc[jj] = *reinterpret_cast<const float4*>(tile + (g4 + 4 * jj) * kMlaRow + kMlaScaleOff);
            if (!ok[jj]) sc[jj] = make_float4(0.f, 0.f, 0.f, 0.f);  // rows past the context may hold NaN
            S[jj] = fmaf(sc[jj].x, Sg[0][jj], fmaf(sc[jj].y, Sg[1][jj], fmaf(sc[jj].z, Sg[2][jj],
                    fmaf(sc[jj].w, Sg[3][jj], Sr[jj]))));
        }
        float mx = kNegInf;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) mx = ok[jj] ? fmaxf(mx, S[jj]) : mx;
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float tmax = mx * sl2;
        const bool need = tmax > m + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float mnew = need ? tmax : m;
            const float alpha = need ? fast_exp2(m - mnew) : 1.f;
            l *= alpha;
            m = mnew;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float a = __shfl(alpha, 4 * g4 + jj);
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 8; ++e) O[q][e][jj] *= a;
            }
        }
        float pr[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float ex = fast_exp2(fmaf(S[jj], sl2, -m));
            pr[jj] = ok[jj] ? ex : 0.f;
            l += pr[jj];
        }
        // PV per latent quarter: P scaled by the tokens' quarter scale; V = converted latent bytes of the
        // four rows g4 + 4i at dims 128q + 8c .. +7.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float s0 = q == 0 ? sc[0].x : q == 1 ? sc[0].y : q == 2 ? sc[0].z : sc[0].w;
            const float s1 = q == 0 ? sc[1].x : q == 1 ? sc[1].y : q == 2 ? sc[1].z : sc[1].w;
            const float s2 = q == 0 ? sc[2].x : q == 1 ? sc[2].y : q == 2 ? sc[2].z : sc[2].w;
            const float s3 = q == 0 ? sc[3].x : q == 1 ? sc[3].y : q == 2 ? sc[3].z : sc[3].w;
            const uint2 A = make_uint2(pack2<true>(pr[0] * s0, pr[1] * s1), pack2<true>(pr[2] * s2, pr[3] * s3));
            uint4 vb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint2 raw = *reinterpret_cast<const uint2*>(tile + (g4 + 4 * i) * kMlaRow + 128 * q + 8 * c);
                vb[i] = ok[i] ? e4m3x8_to_bf16(raw) : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) O[q][e] = mfma_k16<true>(A, v_operand(vb, e), O[q][e]);
        }
    }

    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int h = 4 * g4 + jj;
        const float L = __shfl(l, h);
        const float M = __shfl(m, h);
        if (nparts == 1) {
            const float inv = 1.f / L;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint4 o;
                o.x = pack2<true>(O[q][0][jj] * inv, O[q][1][jj] * inv);
                o.y = pack2<true>(O[q][2][jj] * inv, O[q][3][jj] * inv);
                o.z = pack2<true>(O[q][4][jj] * inv, O[q][5][jj] * inv);
                o.w = pack2<true>(O[q][6][jj] * inv, O[q][7][jj] * inv);
                *reinterpret_cast<uint4*>(out + ((size_t)qrow_idx * p.num_q_heads + h0 + h) * kMlaV + 128 * q + 8 * c) = o;
            }
        } else {
            const size_t idx = ((size_t)s * p.num_q_heads + h0 + h) * p.max_parts + part;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4* pa = reinterpret_cast<float4*>(p.part_acc + idx * kMlaV + 128 * q + 8 * c);
                pa[0] = make_float4(O[q][0][jj], O[q][1][jj], O[q][2][jj], O[q][3][jj]);
                pa[1] = make_float4(O[q][4][jj], O[q][5][jj], O[q][6][jj], O[q][7][jj]);
            }
            if (c == 0) *reinterpret_cast<float2*>(p.part_ml + idx * 2) = make_float2(M, L);
        }
    }
}

hipError_t launch_decode_mla(const DenseDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    const int64_t wgs = (items + 3) / 4;
    hipLaunchKernelGGL(decode_mla_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.max_parts <= 1) return e;
    return launch_decode_reduce(p, stream);
}

}  // namespace pa

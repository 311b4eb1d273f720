// Paged decode over dense fp16 / bf16 KV rows: block-table gather, QK, online softmax, PV,
// split-context partitions and their log-sum-exp merge.
//
// What is computed: page "deep dive into vLLM 05", §2 (read path), and the paged_attention
// pseudocode of "KV Cache 与推理服务内存管理". For every block in the request's block table, read
// the physical block's K and V, score the query against K, softmax, and weight V. The kernel
// knows only the block table. "vLLM 技术内幕" §2.1 adds that keys are read block by block and
// values are accumulated per block; here that is an online softmax. Grouped queries follow
// "deep dive into vLLM 05" §3.2: consecutive query heads share one K/V head.
//
// Mapping onto CDNA4:
//  * One wave owns one (KV head, sequence, partition) item and all G query heads of that KV
//    head, so each K/V row is read from HBM once per group.
//  * A 16-token tile of one KV head is 16 rows of D*2 bytes at the cache's row stride. A lane
//    holds 16 bytes (8 values) of one row. LPR = D/8 lanes cover a row, and one wave-wide 16-byte
//    load covers RPL = 64/LPR consecutive rows, so every load instruction is fully coalesced
//    over whole 64-byte lines.
//  * QK is v_dot2_f32_{f16,bf16} per lane, then a DPP butterfly over the LPR lanes of the row.
//  * Each row group of lanes keeps its own online-softmax state (m, l, acc) over its tokens.
//    The row groups are merged once per partition, so the per-tile work has no cross-row traffic.
//  * The next tile's K and V are loaded into registers while the current tile is computed. The
//    prefetch is unconditional (the last tile reloads itself), so the compiler's wait counts
//    stay exact.
//  * Partition p covers tokens [p*P, (p+1)*P) of the logical sequence; its block ids are read once
//    into one VGPR (lane j = logical block j of the partition) and broadcast with v_readlane.
//  * A sequence with one partition writes its output directly. Otherwise the partition writes
//    (m, l, acc), and decode_reduce_kernel merges them:
//        out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,   M = max_p m_p
//    (scores are kept in the log2 domain: s * scale * log2(e)).

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_inff();

template <bool BF16, int D, int G>
struct Tile {
    static constexpr int LPR = D / 8;     // lanes per row
    static constexpr int RPL = 64 / LPR;  // rows per wave-wide load
    static constexpr int NL = 16 / RPL;   // loads per 16-token tile
};

template <bool BF16, int D, int G, bool MASK>
__device__ __forceinline__ void tile_step(const uint4 (&kr)[Tile<BF16, D, G>::NL],
                                          const uint4 (&vr)[Tile<BF16, D, G>::NL], const uint32_t (&qr)[G][4],
                                          float (&m)[G], float (&l)[G], float (&acc)[G][8], int r, int nvalid,
                                          float scale_log2) {
    using T = Tile<BF16, D, G>;
    constexpr int NL = T::NL, RPL = T::RPL, LPR = T::LPR;
    float sc[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d0 = dot2acc<BF16>(qr[g][0], kr[i].x, 0.f);
            float d1 = dot2acc<BF16>(qr[g][1], kr[i].y, 0.f);
            d0 = dot2acc<BF16>(qr[g][2], kr[i].z, d0);
            d1 = dot2acc<BF16>(qr[g][3], kr[i].w, d1);
            sc[g][i] = group_sum<LPR>(d0 + d1) * scale_log2;
        }
    }
    if constexpr (MASK) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const bool ok = r + i * RPL < nvalid;
#pragma unroll
            for (int g = 0; g < G; ++g) sc[g][i] = ok ? sc[g][i] : kNegInf;
        }
    }
    float pr[G][NL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float mx = m[g];
#pragma unroll
        for (int i = 0; i < NL; ++i) mx = fmaxf(mx, sc[g][i]);
        const float ms = (mx == kNegInf) ? 0.f : mx;
        const float alpha = fast_exp2(m[g] - ms);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            pr[g][i] = fast_exp2(sc[g][i] - ms);
            ps += pr[g][i];
        }
        l[g] = l[g] * alpha + ps;
        m[g] = mx;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const uint32_t w[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        float vf[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            vf[2 * k] = lo_f32<BF16>(w[k]);
            vf[2 * k + 1] = hi_f32<BF16>(w[k]);
        }
        if constexpr (MASK) {
            const bool ok = r + i * RPL < nvalid;
#pragma unroll
            for (int d = 0; d < 8; ++d) vf[d] = ok ? vf[d] : 0.f;  // rows past the context may hold NaN
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[g][d] = fmaf(pr[g][i], vf[d], acc[g][d]);
    }
}

// Context length bounded to [0, min(max_context_len, bt_stride * block_size)], so that no read
// goes past the block table row.
__device__ __forceinline__ int clamp_context(int ctx, const DenseDecodeParams& p) {
    const int64_t cap = min((int64_t)p.max_context_len, (int64_t)p.bt_stride * p.block_size);
    return (int)max((int64_t)0, min((int64_t)ctx, cap));
}

// Walks 16-token tiles inside blocks: (logical block relative to the partition, offset).
struct TileCursor {
    int lb;
    int off;
    __device__ __forceinline__ void advance(int bs) {
        off += 16;
        if (off == bs) {
            off = 0;
            ++lb;
        }
    }
};

}  // namespace

template <bool BF16, int D, int G>
__global__ __launch_bounds__(256) void decode_dense_kernel(DenseDecodeParams p) {
    using T = Tile<BF16, D, G>;
    constexpr int LPR = T::LPR, RPL = T::RPL, NL = T::NL;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int r = lane / LPR;
    const int c = lane % LPR;

    const int item = xcd_linear_block(blockIdx.x, gridDim.x) * 4 + wave;
    const int per_head = p.num_seqs * p.max_parts;
    if (item >= p.num_kv_heads * per_head) return;
    const int kvh = item / per_head;
    const int rem = item - kvh * per_head;
    const int s = rem / p.max_parts;
    const int part = rem - s * p.max_parts;

    const int bs = p.block_size;
    const int ctx = clamp_context(p.context_lens[s], p);
    const int P = p.partition_tokens;
    const int nparts = (ctx + P - 1) / P;
    const int hq0 = kvh * G;  // first query head of this group
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);

    if (ctx == 0) {  // empty context: output 0
        if (part == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if ((g % RPL) == r)
                    *reinterpret_cast<uint4*>(out + ((size_t)s * p.num_q_heads + hq0 + g) * D + c * 8) =
                        make_uint4(0, 0, 0, 0);
        }
        return;
    }
    if (part >= nparts) return;
    const int tb = part * P;
    const int te = min(ctx, tb + P);

    // Query: 8 values of each of the G heads.
    uint32_t qr[G][4];
    const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)s * p.num_q_heads + hq0) * D + c * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint4 v = *reinterpret_cast<const uint4*>(qsrc + g * D);
        qr[g][0] = v.x;
        qr[g][1] = v.y;
        qr[g][2] = v.z;
        qr[g][3] = v.w;
    }

    // Block ids of this partition: lane j holds logical block lb0 + j.
    const int lb0 = tb / bs;
    const int nblk = (te - tb + bs - 1) / bs;  // <= 64 by construction
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const int tbl = lane < nblk ? bt[lb0 + lane] : 0;

    const int64_t krow = p.k_row_bytes, vrow = p.v_row_bytes;
    const char* kbase = p.k + (int64_t)kvh * (D * 2) + c * 16 + r * krow;
    const char* vbase = p.v + (int64_t)kvh * (D * 2) + c * 16 + r * vrow;
    const uint32_t nb = (uint32_t)p.num_blocks;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] = 0.f;
    }

    const int ntiles = (te - tb + 15) >> 4;
    uint4 kA[NL], vA[NL], kB[NL], vB[NL];
    // load cursor runs one tile ahead of the compute cursor (clamped at the last tile)
    TileCursor ld{0, 0}, cp{0, 0};
    int ld_tile = 0;

    auto issue = [&](uint4 (&kk)[NL], uint4 (&vv)[NL]) {
        int phys = __builtin_amdgcn_readlane(tbl, ld.lb);
        phys = ((uint32_t)phys < nb) ? phys : 0;  // out-of-range ids are masked at compute time
        const char* kp = kbase + (int64_t)phys * p.k_block_stride + (int64_t)ld.off * krow;
        const char* vp = vbase + (int64_t)phys * p.v_block_stride + (int64_t)ld.off * vrow;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            kk[i] = *reinterpret_cast<const uint4*>(kp + (int64_t)i * RPL * krow);
            vv[i] = *reinterpret_cast<const uint4*>(vp + (int64_t)i * RPL * vrow);
        }
        if (ld_tile + 1 < ntiles) {
            ld.advance(bs);
            ++ld_tile;
        }
    };
    auto compute = [&](const uint4 (&kk)[NL], const uint4 (&vv)[NL], int tile) {
        const int phys = __builtin_amdgcn_readlane(tbl, cp.lb);
        const int t0 = tb + tile * 16;
        int nvalid = min(16, te - t0);
        if ((uint32_t)phys >= nb) nvalid = 0;
        if (nvalid == 16)
            tile_step<BF16, D, G, false>(kk, vv, qr, m, l, acc, r, 16, p.scale_log2);
        else
            tile_step<BF16, D, G, true>(kk, vv, qr, m, l, acc, r, nvalid, p.scale_log2);
        cp.advance(bs);
    };

    issue(kA, vA);
    int tile = 0;
    for (;;) {
        issue(kB, vB);
        compute(kA, vA, tile);
        if (++tile >= ntiles) break;
        issue(kA, vA);
        compute(kB, vB, tile);
        if (++tile >= ntiles) break;
    }

    // Merge the RPL row groups of the wave.
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
        for (int d = 0; d < 8; ++d) {
            float a = acc[g][d] * f;
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) a += __shfl_xor(a, off);
            acc[g][d] = a;
        }
        m[g] = M;
        l[g] = L;
    }

    if (nparts == 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if ((g % RPL) != r) continue;
            const float inv = 1.f / l[g];
            uint4 o;
            o.x = pack2<BF16>(acc[g][0] * inv, acc[g][1] * inv);
            o.y = pack2<BF16>(acc[g][2] * inv, acc[g][3] * inv);
            o.z = pack2<BF16>(acc[g][4] * inv, acc[g][5] * inv);
            o.w = pack2<BF16>(acc[g][6] * inv, acc[g][7] * inv);
            *reinterpret_cast<uint4*>(out + ((size_t)s * p.num_q_heads + hq0 + g) * D + c * 8) = o;
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if ((g % RPL) != r) continue;
            const size_t idx = ((size_t)s * p.num_q_heads + hq0 + g) * p.max_parts + part;
            float4* pa = reinterpret_cast<float4*>(p.part_acc + idx * D + c * 8);
            pa[0] = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            pa[1] = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
            if (c == 0) *reinterpret_cast<float2*>(p.part_ml + idx * 2) = make_float2(m[g], l[g]);
        }
    }
}

// One wave per (sequence, query head): merge the partition partials of sequences with > 1 partition.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DenseDecodeParams p) {
    constexpr int DPL = D / 64;  // output values per lane
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;  // = s * Hq + head
    if (item >= p.num_seqs * p.num_q_heads) return;
    const int s = item / p.num_q_heads;
    const int ctx = clamp_context(p.context_lens[s], p);
    const int nparts = (ctx + p.partition_tokens - 1) / p.partition_tokens;
    if (nparts <= 1) return;
    const float* ml = p.part_ml + (size_t)item * p.max_parts * 2;
    float M = kNegInf;
    for (int i = lane; i < nparts; i += 64) M = fmaxf(M, ml[2 * i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    for (int i = lane; i < nparts; i += 64) L += fast_exp2(ml[2 * i] - M) * ml[2 * i + 1];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    float a[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) a[k] = 0.f;
    const float* ap = p.part_acc + (size_t)item * p.max_parts * D + lane * DPL;
    for (int i = 0; i < nparts; ++i) {
        const float w = fast_exp2(ml[2 * i] - M);
#pragma unroll
        for (int k = 0; k < DPL; ++k) a[k] = fmaf(w, ap[(size_t)i * D + k], a[k]);
    }
    const float inv = 1.f / L;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)item * D + lane * DPL;
    if constexpr (DPL == 1) {
        out[0] = (uint16_t)(pack2<BF16>(a[0] * inv, 0.f) & 0xFFFFu);
    } else if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(out) = pack2<BF16>(a[0] * inv, a[1] * inv);
    } else {
        *reinterpret_cast<uint2*>(out) = make_uint2(pack2<BF16>(a[0] * inv, a[1] * inv),
                                                    pack2<BF16>(a[2] * inv, a[3] * inv));
    }
}

namespace {

template <bool BF16, int D, int G>
hipError_t launch_typed(const DenseDecodeParams& p, hipStream_t stream) {
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    int64_t wgs = (items + 3) / 4;
    wgs = (wgs + 7) / 8 * 8;
    hipLaunchKernelGGL((decode_dense_kernel<BF16, D, G>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.max_parts <= 1) return e;
    const int64_t red = ((int64_t)p.num_seqs * p.num_q_heads + 3) / 4;
    hipLaunchKernelGGL((decode_reduce_kernel<BF16, D>), dim3((unsigned)red), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_group(const DenseDecodeParams& p, hipStream_t stream) {
    switch (p.group) {
        case 1: return launch_typed<BF16, D, 1>(p, stream);
        case 2: return launch_typed<BF16, D, 2>(p, stream);
        case 4: return launch_typed<BF16, D, 4>(p, stream);
        case 8: return launch_typed<BF16, D, 8>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t launch_dim(const DenseDecodeParams& p, hipStream_t stream) {
    switch (p.head_dim) {
        case 64: return launch_group<BF16, 64>(p, stream);
        case 128: return launch_group<BF16, 128>(p, stream);
        case 256: return launch_group<BF16, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_dense(const DenseDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    return p.is_bf16 ? launch_dim<true>(p, stream) : launch_dim<false>(p, stream);
}

}  // namespace pa

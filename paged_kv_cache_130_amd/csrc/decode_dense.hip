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

#include "decode_common.h"

namespace pa {

namespace {


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
    // Raw scores q.k of this row group's NL tokens, summed over the LPR lanes of the row.
    float sc[G][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d0 = dot2acc<BF16>(qr[g][0], kr[i].x, 0.f);
            float d1 = dot2acc<BF16>(qr[g][1], kr[i].y, 0.f);
            d0 = dot2acc<BF16>(qr[g][2], kr[i].z, d0);
            d1 = dot2acc<BF16>(qr[g][3], kr[i].w, d1);
            sc[g][i] = group_sum<LPR>(d0 + d1);
        }
    }
    bool ok[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) ok[i] = !MASK || (r + i * RPL < nvalid);
    // Move the reference where this tile's maximum is too far above it.
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
            for (int d = 0; d < 8; ++d) acc[g][d] *= alpha;
            m[g] = mnew;
        }
    }
    // p for every (head, token); masked tokens get exactly 0.
    float pr[G][NL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const float e = fast_exp2(fmaf(sc[g][i], scale_log2, -m[g]));
            pr[g][i] = ok[i] ? e : 0.f;
            l[g] += pr[g][i];
        }
    // PV over token pairs with dot2: (v_a[d], v_b[d]) . (p_a, p_b), fp32 accumulation. V words of
    // masked tokens are zeroed first: rows past the context may hold NaN, and 0 * NaN = NaN.
#pragma unroll
    for (int i = 0; i < NL; i += 2) {
        uint32_t wa[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
        uint32_t wb[4] = {vr[i + 1].x, vr[i + 1].y, vr[i + 1].z, vr[i + 1].w};
        if constexpr (MASK) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                wa[k] = ok[i] ? wa[k] : 0u;
                wb[k] = ok[i + 1] ? wb[k] : 0u;
            }
        }
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] = __builtin_amdgcn_perm(wb[k], wa[k], kSelLo);
            hi[k] = __builtin_amdgcn_perm(wb[k], wa[k], kSelHi);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            uint32_t pp, pl;
            pack2_split<BF16>(pr[g][i], pr[g][i + 1], pp, pl);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[g][2 * k] = dot2acc<BF16>(pp, lo[k], acc[g][2 * k]);
                acc[g][2 * k + 1] = dot2acc<BF16>(pp, hi[k], acc[g][2 * k + 1]);
                if constexpr (BF16) {
                    acc[g][2 * k] = dot2acc<BF16>(pl, lo[k], acc[g][2 * k]);
                    acc[g][2 * k + 1] = dot2acc<BF16>(pl, hi[k], acc[g][2 * k + 1]);
                }
            }
        }
    }
}

}  // namespace

template <bool BF16, int D, int G>
__global__ __launch_bounds__(256) void decode_dense_kernel(DenseDecodeParams p) {
    using T = Tile<BF16, D, G>;
    constexpr int LPR = T::LPR, RPL = T::RPL, NL = T::NL;
    // Everything per item is wave-uniform; readfirstlane tells the compiler so, which keeps the
    // item's control flow on scalar registers and the loop free of exec-mask branches.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int r = lane / LPR;
    const int c = lane % LPR;

    // Work list (find_work): full partitions partition-major, then each sequence's partial partition
    // from the longest to the shortest, with the KV head fastest; waves past the end exit at once.
    const int item = blockIdx.x * 4 + wave;
    const int kvh = item % p.num_kv_heads;
    int s, part;
    int ctx;
    if (!find_work(item / p.num_kv_heads, p, s, part, ctx)) return;
    const int bs = p.block_size;
    const int P = p.partition_tokens;
    const int nparts = (ctx + P - 1) / P;
    const int hq0 = kvh * G;  // first query head of this group
    const int qrow_idx = query_row(s, p);
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);

    if (ctx == 0) {  // empty context: output 0
        if (part == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if ((g % RPL) == r)
                    *reinterpret_cast<uint4*>(out + ((size_t)qrow_idx * p.num_q_heads + hq0 + g) * D + c * 8) =
                        make_uint4(0, 0, 0, 0);
        }
        return;
    }
    if (part >= nparts) return;
    const int tb = part * P;
    const int te = min(ctx, tb + P);

    // Query: 8 values of each of the G heads.
    uint32_t qr[G][4];
    const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)qrow_idx * p.num_q_heads + hq0) * D + c * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const uint4 v = *reinterpret_cast<const uint4*>(qsrc + g * D);
        qr[g][0] = v.x;
        qr[g][1] = v.y;
        qr[g][2] = v.z;
        qr[g][3] = v.w;
    }

    // Block ids of this partition: lane j holds logical block lb0 + j.
    const int lb0 = tb >> (p.tiles_per_block_log2 + 4);
    const int nblk = (te - tb + bs - 1) >> (p.tiles_per_block_log2 + 4);  // <= 64 by construction
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const int tbl = lane < nblk ? bt[lb0 + lane] : 0;

    // Per-lane byte offset inside a tile (32-bit) and the uniform per-tile base (64-bit): loads take the
    // scalar-base + vector-offset form.
    const int64_t krow = p.k_row_bytes, vrow = p.v_row_bytes;
    const int kvs = kvh >> p.kv_shift;  // the stored K/V head
    const uint32_t klane = (uint32_t)(kvs * (D * 2) + c * 16) + (uint32_t)r * (uint32_t)krow;
    const uint32_t vlane = (uint32_t)(kvs * (D * 2) + c * 16) + (uint32_t)r * (uint32_t)vrow;
    const uint32_t nb = (uint32_t)p.num_blocks;
    const int tpb_log2 = p.tiles_per_block_log2;  // block_size / 16 is a power of two
    const int tpb_mask = (1 << tpb_log2) - 1;

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] = 0.f;
    }

    const int ntiles = (te - tb + 15) >> 4;
    const int last = ntiles - 1;
    // Tile j of the partition: logical block j >> tpb_log2 of the partition, rows (j & mask)*16 ...
    auto block_of = [&](int j) {
        const int phys = __builtin_amdgcn_readlane(tbl, j >> tpb_log2);
        return phys;
    };
    // Tile j > last is a dummy: every lane reads the same 16 bytes of this item's (cached) query, so
    // the unconditional prefetch after the last tile costs no HBM traffic.
    const char* dummy = reinterpret_cast<const char*>(qsrc - c * 8);
    auto load = [&](uint4 (&kk)[NL], uint4 (&vv)[NL], int j) {
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
    auto step = [&](const uint4 (&kk)[NL], const uint4 (&vv)[NL], int j) {
        int nvalid = min(16, te - (tb + (j << 4)));
        if ((uint32_t)block_of(j) >= nb) nvalid = 0;
        if (nvalid == 16)
            tile_step<BF16, D, G, false>(kk, vv, qr, m, l, acc, r, 16, p.scale_log2);
        else
            tile_step<BF16, D, G, true>(kk, vv, qr, m, l, acc, r, nvalid, p.scale_log2);
    };

    // A ring of kDepth tiles: the loads of the next kDepth - 1 tiles are in flight while one is
    // computed (loads past the last tile read the cached dummy row). Single heads of 128 dims keep
    // three tiles in flight at two waves per SIMD (177 registers): on the 13B-shaped decode that
    // streams about 1% faster than one tile ahead at four waves per SIMD or two at three.
    constexpr int kDepth = (D == 128 && G == 1) ? 4 : 2;
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
            *reinterpret_cast<uint4*>(out + ((size_t)qrow_idx * p.num_q_heads + hq0 + g) * D + c * 8) = o;
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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int item = blockIdx.x * 4 + wave;  // = s * Hq + head
    if (item >= p.num_seqs * p.num_q_heads) return;
    const int s = item / p.num_q_heads;
    const int head = item - s * p.num_q_heads;
    const int nparts = __builtin_amdgcn_readfirstlane(parts_of(s, p));
    if (nparts <= 1) return;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + ((size_t)query_row(s, p) * p.num_q_heads + head) * D;
    merge_partials<BF16, D>(p.part_ml + (size_t)item * p.max_parts * 2, 2, p.part_acc + (size_t)item * p.max_parts * D,
                            D, nparts, out);
}

namespace {

template <bool BF16, int D, int G>
hipError_t launch_typed(const DenseDecodeParams& p, hipStream_t stream) {
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    const int64_t wgs = (items + 3) / 4;
    hipLaunchKernelGGL((decode_dense_kernel<BF16, D, G>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.max_parts <= 1) return e;
    return launch_decode_reduce(p, stream);
}

// Eight query heads per K/V head: two waves of four each read the K/V head (an eight-head wave
// would need more than its 512 registers). The host counts these items (kv_waves in api.hip).
inline DenseDecodeParams split_eight(const DenseDecodeParams& p) {
    DenseDecodeParams q = p;
    q.num_kv_heads = p.num_kv_heads * 2;
    q.group = 4;
    q.kv_shift = 1;
    return q;
}

template <bool BF16, int D>
hipError_t launch_group(const DenseDecodeParams& p, hipStream_t stream) {
    switch (p.group) {
        case 1: return launch_typed<BF16, D, 1>(p, stream);
        case 2: return launch_typed<BF16, D, 2>(p, stream);
        case 4: return launch_typed<BF16, D, 4>(p, stream);
        case 8: return launch_typed<BF16, D, 4>(split_eight(p), stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t launch_dim(const DenseDecodeParams& p, hipStream_t stream) {
    switch (p.head_dim) {
        case 64: return launch_group<BF16, 64>(p, stream);
        // Grouped heads at head_dim 128 run on the matrix cores (launch_decode_dense).
        case 128: return p.group == 1 ? launch_typed<BF16, 128, 1>(p, stream) : hipErrorInvalidValue;
        case 256: return launch_group<BF16, 256>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_reduce(const DenseDecodeParams& p, hipStream_t stream) {
    const int64_t red = ((int64_t)p.num_seqs * p.num_q_heads + 3) / 4;
    if (p.is_bf16) {
        switch (p.head_dim) {
            case 64: hipLaunchKernelGGL((decode_reduce_kernel<true, 64>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
            case 128: hipLaunchKernelGGL((decode_reduce_kernel<true, 128>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
            case 512: hipLaunchKernelGGL((decode_reduce_kernel<true, 512>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
            default: hipLaunchKernelGGL((decode_reduce_kernel<true, 256>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
        }
    } else {
        switch (p.head_dim) {
            case 64: hipLaunchKernelGGL((decode_reduce_kernel<false, 64>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
            case 128: hipLaunchKernelGGL((decode_reduce_kernel<false, 128>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
            default: hipLaunchKernelGGL((decode_reduce_kernel<false, 256>), dim3((unsigned)red), dim3(256), 0, stream, p); break;
        }
    }
    return hipGetLastError();
}

// Grouped heads at head_dim 128 run on the matrix cores (decode_mfma.hip); single heads and the other
// head sizes run on the VALU kernel above.
hipError_t launch_decode_dense(const DenseDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    // Grouped heads at head_dim 128 (16-bit or FP8 rows) run on the matrix cores; the other FP8 shapes
    // on the FP8 vector kernel.
    if (p.head_dim == 128 && p.group >= 2) return launch_decode_mfma(p, stream);
    if (p.kv_fp8) return launch_decode_fp8(p, stream);
    return p.is_bf16 ? launch_dim<true>(p, stream) : launch_dim<false>(p, stream);
}

}  // namespace pa

// DSA sparse path, first half: lightning-indexer scores over the indexer rows of the dual cache, and
// the top-k token selection of every sequence.
//
// "vLLM KV Cache Layout 可视化" (section on two caches sharing one block table): next to the MLA
// cache, DeepSeek's sparse attention keeps an indexer cache in which the lightning indexer stores,
// per token, 128 FP8 key values and one float32 scale (132 bytes); the keys serve to pick a sparse
// top-k set of tokens, and both caches share one block table. The pages give no scoring formula; the
// one computed here is the published lightning indexer's:
//     I_t = sum_j w_j * max(q_j . k_t, 0),   k_t = codes_t * scale_t,
// with H index heads q_j (bf16, 128 dims) and head weights w_j (float32) per decode token. The scales
// quantize-on-write stores are amax / 448 >= 0, for which I_t = scale_t * sum_j w_j max(q_j . codes_t, 0).
//
// Scores. q_j . codes_t for 16 tokens and all H heads is a (16 x 128) by (128 x H) product: it runs
// on v_mfma_f32_16x16x32_bf16, with the e4m3 codes widened exactly to bf16 by the gfx950 convert.
// Per token the kernel reads 132 bytes and does 256 H flops (H = 64: about 124 flop per byte, under
// the bf16 ridge of about 310), so it is bound by HBM. A wave holds one sequence's queries (four
// 16-byte operands per 16 heads) and streams a balanced range of the 16-token units of all sequences,
// three units in flight.
//
// Top-k. One work-group per sequence finds the k-th largest score by a radix select over
// order-preserving 32-bit keys (four 8-bit digit passes, per-wave histograms in LDS), then writes
// the selected positions in ascending order through a work-group prefix scan, taking the scores tied
// at the threshold from the earliest positions, and each position's slot through the block table.

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

constexpr int kIdxRow = 132;   // 128 e4m3 key values + 1 float32 scale
constexpr int kIdxUnit = 16;   // tokens per unit: the rows of one MFMA tile
constexpr int kDepth = 3;      // units in flight per wave

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Rows are 132 bytes, so their 16-byte pieces are only 4-byte aligned.
__device__ __forceinline__ uint4 load16_a4(const char* ptr) {
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(ptr);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Two e4m3 codes (bytes 0, 1 or 2, 3 of w) -> two bf16 (exact: every e4m3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

__device__ __forceinline__ uint4 codes8_bf16(uint32_t lo, uint32_t hi) {
    return make_uint4(e4m3x2_bf16<false>(lo), e4m3x2_bf16<true>(lo), e4m3x2_bf16<false>(hi),
                      e4m3x2_bf16<true>(hi));
}

// Tokens of a sequence, bounded by the host's max_context_len, the block-table row and the score row.
__device__ __forceinline__ int idx_ctx(int64_t ctx, const IndexerParams& p) {
    int64_t cap = min((int64_t)p.max_context_len, (int64_t)p.bt_stride * p.block_size);
    cap = min(cap, p.score_stride);
    return (int)max((int64_t)0, min(ctx, cap));
}

__device__ __forceinline__ int idx_units(int ctx) { return (ctx + kIdxUnit - 1) / kIdxUnit; }

// Position in the stream of 16-token units of all sequences (wave-uniform).
struct IdxCursor {
    int g;    // unit index in the stream
    int s;    // sequence
    int k;    // unit within the sequence
    int nu;   // units of the sequence
    int ctx;  // tokens of the sequence
};

__device__ __forceinline__ void idx_advance(IdxCursor& c, const IndexerParams& p) {
    ++c.g;
    if (++c.k < c.nu) return;
    c.k = 0;
    do {
        ++c.s;
        c.ctx = c.s < p.num_seqs ? idx_ctx(load_scalar(p.context_lens + c.s), p) : 0;
        c.nu = idx_units(c.ctx);
    } while (c.nu == 0 && c.s < p.num_seqs);
}

__device__ int idx_total_units(const IndexerParams& p, int lane) {
    int u = 0;
    for (int base = 0; base < p.num_seqs; base += 64) {
        const int s = base + lane;
        int v = s < p.num_seqs ? idx_units(idx_ctx(p.context_lens[s], p)) : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        u += v;
    }
    return __builtin_amdgcn_readfirstlane(u);
}

// Cursor of unit g0 (g0 < total units).
__device__ IdxCursor idx_locate(int g0, const IndexerParams& p, int lane) {
    int before = 0;
    for (int base = 0; base < p.num_seqs; base += 64) {
        const int s = base + lane;
        const int ctx = s < p.num_seqs ? idx_ctx(p.context_lens[s], p) : 0;
        const int nu = idx_units(ctx);
        int incl = nu;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl(incl, max(lane - off, 0));
            if (lane >= off) incl += t;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (g0 < before + total) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(before + incl > g0);
            const int ls = __builtin_ctzll(hit);
            IdxCursor c;
            c.g = g0;
            c.s = base + ls;
            c.ctx = __builtin_amdgcn_readlane(ctx, ls);
            c.nu = __builtin_amdgcn_readlane(nu, ls);
            c.k = g0 - (before + __builtin_amdgcn_readlane(incl, ls) - c.nu);
            return c;
        }
        before += total;
    }
    IdxCursor c{g0, p.num_seqs, 0, 0, 0};
    return c;
}

// One unit's rows as a lane holds them: lane (c, g4) = (lane % 16, lane / 16) has bytes
// [16 g4, 16 g4 + 16) and [64 + 16 g4, 64 + 16 g4 + 16) of row c, and the scale of row 4 g4 + (c & 3),
// the token whose score it writes.
struct RawUnit {
    uint4 a, b;
    float sc;
    int ok;  // the unit's block id is valid (wave-uniform)
};

}  // namespace

// HT = H / 16 head tiles. Product layout: A = key codes (row = token c), B = queries (column = head
// c of the tile), both with the k slots of lane group g4 at dims {16 g4 .. 16 g4 + 15} (k steps 0, 1)
// and {64 + 16 g4 ..} (k steps 2, 3); output register j of lane (c, g4) is token 4 g4 + j, head c.
template <int HT>
__global__ __launch_bounds__(256) void indexer_score_kernel(IndexerParams p) {
    const int lane = threadIdx.x & 63;
    const int c = lane & 15, g4 = lane >> 4;
    const int wv = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int U = idx_total_units(p, lane);
    const int per = (U + p.num_waves - 1) / p.num_waves;
    const int g0 = wv * per;
    const int g1 = min(U, g0 + per);
    if (g0 >= g1) return;

    const char* dummy = reinterpret_cast<const char*>(p.q);  // in-bounds source of loads past the range
    IdxCursor cl = idx_locate(g0, p, lane);  // next unit to load
    IdxCursor cc = cl;                        // next unit to score

    uint4 qop[HT][4];
    float wt[HT];
    int qseq = -1;
    auto load_queries = [&](int s) __attribute__((always_inline)) {
        const uint16_t* qs = p.q + ((size_t)s * p.num_heads + c) * 128;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                qop[ht][ks] = *reinterpret_cast<const uint4*>(qs + (size_t)ht * 16 * 128 + (ks >> 1) * 64 + 16 * g4 +
                                                              8 * (ks & 1));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) wt[ht] = p.w[(size_t)s * p.num_heads + 16 * ht + c];
        // Wait here, inside the branch: where the branch rejoins the compiler would otherwise wait
        // for every load in flight on every unit.
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        qseq = s;
    };

    // Block id of unit cl, read one unit ahead so that the scalar load's latency is hidden.
    int pre_blk = 0;
    auto fetch_block_id = [&]() __attribute__((always_inline)) {
        if (cl.g < g1)
            pre_blk = load_scalar(p.block_tables + (int64_t)cl.s * p.bt_stride + ((cl.k * kIdxUnit) >> p.block_size_log2));
    };

    // Loads unit cl (a unit past the range reads the queries instead) and advances cl.
    auto load_unit = [&](RawUnit& r) __attribute__((always_inline)) {
        const char* base = dummy;
        const char* sbase = dummy;
        r.ok = 0;
        if (cl.g < g1) {
            const int t0 = cl.k * kIdxUnit;
            const int nv = min(kIdxUnit, cl.ctx - t0);
            if ((uint32_t)pre_blk < (uint32_t)p.num_blocks) {
                const char* unit = p.idx + (int64_t)pre_blk * p.block_stride + (int64_t)(t0 & (p.block_size - 1)) * kIdxRow;
                base = unit + min(c, nv - 1) * kIdxRow;
                sbase = unit + min(4 * g4 + (c & 3), nv - 1) * kIdxRow;
                r.ok = 1;
            }
        }
        r.a = load16_a4(base + 16 * g4);
        r.b = load16_a4(base + 64 + 16 * g4);
        r.sc = *reinterpret_cast<const float*>(sbase + 128);
        idx_advance(cl, p);
        fetch_block_id();
    };

    auto score_unit = [&](const RawUnit& r) __attribute__((always_inline)) {
        if (cc.s != qseq) load_queries(cc.s);
        const int t0 = cc.k * kIdxUnit;
        const int nv = min(kIdxUnit, cc.ctx - t0);
        const uint4 kop[4] = {codes8_bf16(r.a.x, r.a.y), codes8_bf16(r.a.z, r.a.w), codes8_bf16(r.b.x, r.b.y),
                              codes8_bf16(r.b.z, r.b.w)};
        f32x4_t S[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) S[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) S[ht] = mfma_k32<true>(kop[ks], qop[ht][ks], S[ht]);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = fmaf(wt[ht], fmaxf(S[ht][j], 0.f), acc[j]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = group_sum<16>(acc[j]);
        const int jj = c & 3;
        const float tot = jj == 0 ? acc[0] : jj == 1 ? acc[1] : jj == 2 ? acc[2] : acc[3];
        const int t = 4 * g4 + jj;
        if (c < 4 && t < nv) p.scores[(int64_t)cc.s * p.score_stride + t0 + t] = r.ok ? r.sc * tot : kNegInf;
        idx_advance(cc, p);
    };

    fetch_block_id();
    RawUnit r[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth - 1; ++i) load_unit(r[i]);
    bool more = true;
    while (more) {
#pragma unroll
        for (int i = 0; i < kDepth; ++i) {
            if (more) {
                load_unit(r[(i + kDepth - 1) % kDepth]);
                score_unit(r[i]);
                more = cc.g < g1;
            }
        }
    }
}

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkCache = 32768;  // scores of a sequence kept in LDS (128 KB); longer ones re-read

// Order-preserving key: a > b as floats <=> key(a) > key(b) as unsigned (-0 is taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(IndexerParams p) {
    __shared__ float s_sc[kTopkCache];
    __shared__ uint32_t s_hist[kTopkWaves][256];
    __shared__ uint32_t s_tot[256];
    __shared__ int s_pick[2];
    __shared__ int s_wsum[2][kTopkWaves];

    const int s = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = idx_ctx(p.context_lens[s], p);
    const int k = p.top_k;
    int32_t* pos_out = p.topk_pos + (int64_t)s * k;
    int32_t* slot_out = p.topk_slots + (int64_t)s * k;
    const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride;
    const float* src = p.scores + (int64_t)s * p.score_stride;

    // Slot of position t (num_blocks * block_size fits in int32); -1 for an invalid block id.
    auto slot_of = [&](int t) -> int32_t {
        const int32_t b = bt[t >> p.block_size_log2];
        if ((uint32_t)b >= (uint32_t)p.num_blocks) return -1;
        return b * p.block_size + (t & (p.block_size - 1));
    };

    if (tid == 0) p.topk_lens[s] = min(n, k);
    if (n <= k) {  // every token is selected
        for (int i = tid; i < k; i += kTopkThreads) {
            pos_out[i] = i < n ? i : -1;
            slot_out[i] = i < n ? slot_of(i) : -1;
        }
        return;
    }

    const bool cached = n <= kTopkCache;
    if (cached) {
        for (int i = tid; i < n; i += kTopkThreads) s_sc[i] = src[i];
        __syncthreads();
    }
    auto key_at = [&](int i) __attribute__((always_inline)) { return order_key(cached ? s_sc[i] : src[i]); };

    // Radix select: after the pass of digit d, `prefix` holds the top digits of the k-th largest key
    // and `need` how many keys with that prefix still belong to the top k.
    uint32_t prefix = 0, mask = 0;
    int need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < kTopkWaves * 256; i += kTopkThreads) (&s_hist[0][0])[i] = 0u;
        __syncthreads();
        for (int i = tid; i < n; i += kTopkThreads) {
            const uint32_t key = key_at(i);
            if ((key & mask) == prefix) atomicAdd(&s_hist[wave][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            uint32_t t = 0;
#pragma unroll
            for (int w = 0; w < kTopkWaves; ++w) t += s_hist[w][tid];
            s_tot[tid] = t;
        }
        __syncthreads();
        if (wave == 0) {
            // Lane l holds digits 255 - 4l - i (i = 0..3): the digits in descending order.
            uint32_t cnt[4], sum = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cnt[i] = s_tot[255 - 4 * lane - i];
                sum += cnt[i];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t t = __shfl(incl, max(lane - off, 0));
                if (lane >= off) incl += t;
            }
            const uint32_t before = incl - sum;  // keys with a larger digit than this lane's first
            if (before < (uint32_t)need && (uint32_t)need <= incl) {
                uint32_t acc = before;
                bool done = false;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (!done && acc + cnt[i] >= (uint32_t)need) {
                        s_pick[0] = 255 - 4 * lane - i;
                        s_pick[1] = (int)acc;
                        done = true;
                    }
                    acc += cnt[i];
                }
            }
        }
        __syncthreads();
        need -= s_pick[1];
        prefix |= (uint32_t)s_pick[0] << shift;
        mask |= 255u << shift;
        __syncthreads();
    }

    // Selection in position order: keys above the threshold, and the first `need` keys equal to it.
    const uint32_t thr = prefix;
    const uint64_t below = (1ull << lane) - 1ull;
    int run_sel = 0, run_eq = 0;
    for (int base = 0; base < n; base += kTopkThreads) {
        const int i = base + tid;
        const uint32_t key = i < n ? key_at(i) : 0u;
        const bool gt = i < n && key > thr;
        const bool eq = i < n && key == thr;
        const uint64_t em = __builtin_amdgcn_ballot_w64(eq);
        if (lane == 0) s_wsum[0][wave] = __builtin_popcountll(em);
        __syncthreads();
        int eq_rank = run_eq + __builtin_popcountll(em & below), eq_total = 0;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) {
            const int v = s_wsum[0][w];
            eq_rank += w < wave ? v : 0;
            eq_total += v;
        }
        const bool take = gt || (eq && eq_rank < need);
        const uint64_t tm = __builtin_amdgcn_ballot_w64(take);
        if (lane == 0) s_wsum[1][wave] = __builtin_popcountll(tm);
        __syncthreads();
        int out = run_sel + __builtin_popcountll(tm & below), sel_total = 0;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) {
            const int v = s_wsum[1][w];
            out += w < wave ? v : 0;
            sel_total += v;
        }
        if (take && out < k) {  // exactly k are taken; the bound keeps a broken invariant in bounds
            pos_out[out] = i;
            slot_out[out] = slot_of(i);
        }
        run_sel += sel_total;
        run_eq += eq_total;
        __syncthreads();
    }
}

namespace {

template <int HT>
hipError_t launch_scores(const IndexerParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((indexer_score_kernel<HT>), dim3((unsigned)(p.num_waves / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_topk(const IndexerParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    hipError_t e;
    switch (p.num_heads) {
        case 16: e = launch_scores<1>(p, stream); break;
        case 32: e = launch_scores<2>(p, stream); break;
        case 48: e = launch_scores<3>(p, stream); break;
        case 64: e = launch_scores<4>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)p.num_seqs), dim3(kTopkThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

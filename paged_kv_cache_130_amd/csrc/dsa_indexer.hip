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
// the bf16 ridge of about 310), so it is bound by HBM. A work-group takes 512 consecutive tokens of
// one sequence: its four waves share the sequence's queries through LDS (read once from memory) and
// hold them in registers; each wave loads its 128 tokens' rows as eight flat, coalesced 2112-byte
// runs (16 rows each), all in flight at once, and stages each run through LDS to pick out the MFMA
// operands (rows are 132 bytes, so a row's bytes do not line up with the lanes of a flat load).
//
// Top-k. One work-group per sequence finds the k-th largest score by a radix select over
// order-preserving 32-bit keys (three 11/11/10-bit digit passes over a histogram in LDS), then
// writes the selected positions in ascending order through one work-group prefix scan per 8192
// positions, taking the scores tied at the threshold from the earliest positions, and each
// position's slot through the block table.

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

constexpr int kIdxRow = 132;                    // 128 e4m3 key values + 1 float32 scale
constexpr int kIdxUnit = 16;                    // tokens per unit: the rows of one MFMA tile
constexpr int kUnitBytes = kIdxUnit * kIdxRow;  // 2112 = 132 chunks of 16 bytes
constexpr int kUnitChunks = kUnitBytes / 16;
constexpr int kWaveUnits = 8;                   // units per wave (128 tokens)
constexpr int kWgTokens = 4 * kWaveUnits * kIdxUnit;  // 512 tokens per work-group
constexpr int kQRow = 128 * 2 + 16;             // LDS row of one query head (padded against conflicts)

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

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

}  // namespace

// Grid: ceil(max_context_len / 512) work-groups per sequence. HT = H / 16 head tiles. Product layout:
// A = queries (row = head c of the tile), B = key codes (column = token c), both with the k slots of
// lane group g4 at dims {16 g4 .. 16 g4 + 15} (k steps 0, 1) and {64 + 16 g4 ..} (k steps 2, 3);
// output register j of lane (c, g4) is head 16 ht + 4 g4 + j, token c. A lane weighs and sums its 16
// heads, two cross-lane steps add the four lane groups, and lanes 0..15 write tokens 0..15.
template <int HT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void indexer_score_kernel(IndexerParams p) {
    __shared__ __attribute__((aligned(16))) char s_q[HT * 16 * kQRow];
    __shared__ float s_w[HT * 16];
    __shared__ __attribute__((aligned(16))) char s_stage[4][2][3 * 64 * 16];  // three whole load rounds

    const int chunks = (p.max_context_len + kWgTokens - 1) / kWgTokens;
    const int s = blockIdx.x / chunks;
    const int n = idx_ctx(load_scalar(p.context_lens + s), p);
    const int tok0 = (blockIdx.x - s * chunks) * kWgTokens;
    if (tok0 >= n) return;  // the whole work-group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g4 = lane >> 4;

    // This wave's tokens and their block ids (lane u < 8 holds unit u's).
    const int wtok0 = tok0 + wave * kWaveUnits * kIdxUnit;
    const int nunits = min(kWaveUnits, max(0, (n - wtok0 + kIdxUnit - 1) / kIdxUnit));
    int blk = -1;
    if (lane < nunits) blk = p.block_tables[(int64_t)s * p.bt_stride + ((wtok0 + lane * kIdxUnit) >> p.block_size_log2)];

    // Queries and head weights, 16 bytes per thread per round; they go to LDS once the rows' loads
    // are issued.
    const char* qsrc = reinterpret_cast<const char*>(p.q + (size_t)s * p.num_heads * 128);
    u32x4 qv[HT];
#pragma unroll
    for (int r = 0; r < HT; ++r) qv[r] = *reinterpret_cast<const u32x4*>(qsrc + (size_t)(r * 256 + tid) * 16);
    const float wv = tid < HT * 16 ? p.w[(size_t)s * p.num_heads + tid] : 0.f;

    // Issue every unit's flat loads: chunk r * 64 + lane of the unit's 2112 contiguous bytes (a unit
    // never straddles a block). Units past the context or in an invalid block read the queries.
    const char* dummy = qsrc;
    u32x4 raw[kWaveUnits][3];  // a native vector type: a struct copy here would stay in scratch memory
    bool unit_ok[kWaveUnits];
#pragma unroll
    for (int u = 0; u < kWaveUnits; ++u) {
        const int b = __builtin_amdgcn_readlane(blk, u);
        unit_ok[u] = u < nunits && (uint32_t)b < (uint32_t)p.num_blocks;
        const char* base = unit_ok[u] ? p.idx + (int64_t)b * p.block_stride +
                                            (int64_t)((wtok0 + u * kIdxUnit) & (p.block_size - 1)) * kIdxRow
                                      : dummy;
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int ch = min(r * 64 + lane, kUnitChunks - 1);
            raw[u][r] = *reinterpret_cast<const u32x4*>(base + ch * 16);
        }
    }

#pragma unroll
    for (int r = 0; r < HT; ++r) {
        const int ch = r * 256 + tid;  // 16-byte chunk: head ch / 16, dims 8 (ch % 16) ..
        *reinterpret_cast<u32x4*>(s_q + (ch >> 4) * kQRow + (ch & 15) * 16) = qv[r];
    }
    if (tid < HT * 16) s_w[tid] = wv;
    __syncthreads();  // queries and weights in LDS
    uint4 qop[HT][4];
    float wr[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qop[ht][ks] = *reinterpret_cast<const uint4*>(s_q + (16 * ht + c) * kQRow +
                                                          ((ks >> 1) * 64 + 16 * g4 + 8 * (ks & 1)) * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) wr[ht][j] = s_w[16 * ht + 4 * g4 + j];
    }

    // One basic block for all units (the scores are stored after the loop), so that the scheduler can
    // overlap one unit's products with the next one's staging.
    float score[kWaveUnits];
#pragma unroll
    for (int u = 0; u < kWaveUnits; ++u) {
        // Stage the unit's bytes (two buffers, so that one unit's reads overlap the next one's
        // writes), then read row c's key pieces and scale.
        char* stage = s_stage[wave][u & 1];
#pragma unroll
        for (int r = 0; r < 3; ++r) *reinterpret_cast<u32x4*>(stage + (r * 64 + lane) * 16) = raw[u][r];
        const u32x4_a4 a = *reinterpret_cast<const u32x4_a4*>(stage + c * kIdxRow + 16 * g4);
        const u32x4_a4 b = *reinterpret_cast<const u32x4_a4*>(stage + c * kIdxRow + 64 + 16 * g4);
        const float sc = *reinterpret_cast<const float*>(stage + c * kIdxRow + 128);
        const uint4 kop[4] = {codes8_bf16(a.x, a.y), codes8_bf16(a.z, a.w), codes8_bf16(b.x, b.y),
                              codes8_bf16(b.z, b.w)};
        f32x4_t S[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) S[ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) S[ht] = mfma_k32<true>(qop[ht][ks], kop[ks], S[ht]);
        float acc = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc = fmaf(wr[ht][j], fmaxf(S[ht][j], 0.f), acc);
        acc += __shfl_xor(acc, 16);
        acc += __shfl_xor(acc, 32);
        score[u] = unit_ok[u] ? sc * acc : kNegInf;
    }
    if (g4 == 0) {
        float* out = p.scores + (int64_t)s * p.score_stride + wtok0 + c;
#pragma unroll
        for (int u = 0; u < kWaveUnits; ++u)
            if (u < nunits && wtok0 + u * kIdxUnit + c < n) out[u * kIdxUnit] = score[u];
    }
}

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkCache = 32768;  // scores of a sequence kept in LDS (128 KB); longer ones are re-read
constexpr int kBtCache = 2048;     // block ids of a sequence kept in LDS
constexpr int kPer = 8;            // consecutive positions per thread in the selection
constexpr int kSelBlock = kPer * kTopkThreads;
constexpr int kBins = 2048;        // 11-bit digits: bits 31..21, 20..10, then 9..0

// Order-preserving key: a > b as floats <=> key(a) > key(b) as unsigned (-0 is taken as +0).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Work-group barrier for data in LDS: waits for this wave's LDS operations but not for its global
// stores, which __syncthreads would also wait for.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    lds_barrier();
}

// Inclusive prefix sum over the 64 lanes, on the VALU through DPP: shifts by 1, 2, 4 and 8 lanes
// within each 16-lane row, then lane 15 of each row added to the next row and lane 31 to rows 2 and
// 3 (row_bcast:15 and row_bcast:31). A lane without a source adds 0.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
    (void)lane;
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return v;
}

}  // namespace

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(IndexerParams p) {
    __shared__ __attribute__((aligned(16))) float s_sc[kTopkCache];
    __shared__ int32_t s_bt[kBtCache];
    __shared__ uint32_t s_hist[2][kBins];
    __shared__ int s_pick[2];
    __shared__ int s_wsum[kTopkWaves][2];

    const int s = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k = p.top_k;
    int32_t* pos_out = p.topk_pos + (int64_t)s * k;
    int32_t* slot_out = p.topk_slots + (int64_t)s * k;
    const int32_t* bt = p.block_tables + (int64_t)s * p.bt_stride;
    const float* src = p.scores + (int64_t)s * p.score_stride;
    // The first kSelBlock scores and kTopkThreads block ids are read together with the context length
    // rather than after it (from inside the score and table rows; what lies past the context is
    // dropped), so that they arrive in the same round trip to memory.
    float v0[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int i = j * kTopkThreads + tid;
        v0[j] = i < p.score_stride ? src[i] : 0.f;
    }
    const int32_t bt0 = tid < p.bt_stride ? bt[tid] : 0;
    const int n = idx_ctx(p.context_lens[s], p);
    const int nblk = (n + p.block_size - 1) >> p.block_size_log2;
    const bool bt_cached = nblk <= kBtCache;

    // Slot of position t (num_blocks * block_size fits in int32); -1 for an invalid block id.
    auto slot_of = [&](int t) __attribute__((always_inline)) -> int32_t {
        const int j = t >> p.block_size_log2;
        const int32_t b = bt_cached ? s_bt[j] : bt[j];
        if ((uint32_t)b >= (uint32_t)p.num_blocks) return -1;
        return b * p.block_size + (t & (p.block_size - 1));
    };

    if (tid == 0) p.topk_lens[s] = min(n, k);
    if (n <= k) {  // every token is selected
        for (int i = tid; i < k; i += kTopkThreads) {
            int32_t sl = -1;
            if (i < n) {
                const int32_t b = bt[i >> p.block_size_log2];
                sl = (uint32_t)b < (uint32_t)p.num_blocks ? b * p.block_size + (i & (p.block_size - 1)) : -1;
            }
            pos_out[i] = i < n ? i : -1;
            slot_out[i] = sl;
        }
        return;
    }

    // Scores (when they fit) and block ids -> LDS, kPer loads in flight per thread; zero histogram 0.
    const bool cached = n <= kTopkCache;
    if (cached) {
        for (int base = 0; base < n; base += kSelBlock) {
            float v[kPer];
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = base + j * kTopkThreads + tid;
                v[j] = base == 0 ? v0[j] : i < n ? src[i] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = base + j * kTopkThreads + tid;
                if (i < n) s_sc[i] = v[j];
            }
        }
    }
    if (bt_cached)
        for (int j = tid; j < nblk; j += kTopkThreads) s_bt[j] = j < kTopkThreads ? bt0 : bt[j];
    for (int i = tid; i < kBins; i += kTopkThreads) s_hist[0][i] = 0u;
    __syncthreads();

    // Keys of positions base + kPer * tid + j (j < kPer); 0 past n.
    auto keys_at = [&](int base, uint32_t (&key)[kPer]) __attribute__((always_inline)) {
        const int i0 = base + kPer * tid;
        if (cached && i0 + kPer <= n) {
            const float4 a = *reinterpret_cast<const float4*>(s_sc + i0);
            const float4 b = *reinterpret_cast<const float4*>(s_sc + i0 + 4);
            key[0] = order_key(a.x);
            key[1] = order_key(a.y);
            key[2] = order_key(a.z);
            key[3] = order_key(a.w);
            key[4] = order_key(b.x);
            key[5] = order_key(b.y);
            key[6] = order_key(b.z);
            key[7] = order_key(b.w);
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = i0 + j;
                key[j] = order_key(i < n ? (cached ? s_sc[i] : src[i]) : 0.f);
            }
        }
    };

    // Radix select: after each pass, `prefix` holds the top digits of the k-th largest key and
    // `need` how many keys with that prefix still belong to the top k.
    uint32_t prefix = 0, mask = 0;
    int need = k;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const uint32_t dmask = pass == 2 ? 1023u : 2047u;
        uint32_t* hist = s_hist[pass & 1];
        for (int base = 0; base < n; base += kSelBlock) {
            uint32_t key[kPer];
            keys_at(base, key);
#pragma unroll
            for (int j = 0; j < kPer; ++j) {
                const int i = base + kPer * tid + j;
                if (i < n && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
            }
        }
        lds_sync();
        // Thread t holds digits 2047 - 2t and 2046 - 2t (descending); a scan over them gives the keys
        // above each digit, and the digit that holds the need-th key is picked. The other histogram
        // is cleared for the next pass meanwhile.
        const uint32_t c0 = hist[kBins - 1 - 2 * tid], c1 = hist[kBins - 2 - 2 * tid];
        s_hist[(pass + 1) & 1][2 * tid] = 0u;
        s_hist[(pass + 1) & 1][2 * tid + 1] = 0u;
        int incl = wave_incl_scan((int)(c0 + c1), lane);
        if (lane == 63) s_wsum[wave][0] = incl;
        lds_sync();
        // All sixteen wave totals are read at once (a loop bounded by the wave index would wait for
        // each read in turn, and every wave then waits for the last one at the next barrier).
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) {
            const int t = s_wsum[w][0];
            incl += w < wave ? t : 0;
        }
        const uint32_t before = (uint32_t)incl - c0 - c1;  // keys above digit 2047 - 2t
        if (before < (uint32_t)need && (uint32_t)need <= before + c0) {
            s_pick[0] = kBins - 1 - 2 * tid;
            s_pick[1] = (int)before;
        } else if (before + c0 < (uint32_t)need && (uint32_t)need <= (uint32_t)incl) {
            s_pick[0] = kBins - 2 - 2 * tid;
            s_pick[1] = (int)(before + c0);
        }
        lds_sync();
        need -= s_pick[1];
        prefix |= (uint32_t)s_pick[0] << shift;
        mask |= dmask << shift;
    }

    // Selection in position order: keys above the threshold, and the first `need` keys equal to it.
    // A taken position i is output number gt_before(i) + min(eq_before(i), need).
    const uint32_t thr = prefix;
    int run_gt = 0, run_eq = 0;
    for (int base = 0; base < n; base += kSelBlock) {
        uint32_t key[kPer];
        keys_at(base, key);
        int ngt = 0, neq = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const bool in = base + kPer * tid + j < n;
            ngt += in && key[j] > thr;
            neq += in && key[j] == thr;
        }
        const int packed = wave_incl_scan(ngt | (neq << 16), lane);  // both counts <= 512 per wave
        if (lane == 63) s_wsum[wave][1] = packed;
        lds_sync();
        int before = packed - (ngt | (neq << 16)), total = 0;
#pragma unroll
        for (int w = 0; w < kTopkWaves; ++w) {
            const int v = s_wsum[w][1];
            before += w < wave ? v : 0;
            total += v;
        }
        int gt_before = run_gt + (before & 0xFFFF), eq_before = run_eq + (before >> 16);
        run_gt += total & 0xFFFF;
        run_eq += total >> 16;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = base + kPer * tid + j;
            const bool in = i < n;
            const bool gt = in && key[j] > thr, eq = in && key[j] == thr;
            const int out = gt_before + min(eq_before, need);
            if ((gt || (eq && eq_before < need)) && out < k) {  // exactly k are taken; the bound is a guard
                pos_out[out] = i;
                slot_out[out] = slot_of(i);
            }
            gt_before += gt;
            eq_before += eq;
        }
        lds_sync();
    }
}

namespace {

template <int HT>
hipError_t launch_scores(const IndexerParams& p, hipStream_t stream) {
    const int64_t wgs = (int64_t)((p.max_context_len + kWgTokens - 1) / kWgTokens) * p.num_seqs;
    hipLaunchKernelGGL((indexer_score_kernel<HT>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_topk(const IndexerParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    hipError_t e = hipSuccess;
    if (p.max_context_len > 0) {
        switch (p.num_heads) {
            case 16: e = launch_scores<1>(p, stream); break;
            case 32: e = launch_scores<2>(p, stream); break;
            case 48: e = launch_scores<3>(p, stream); break;
            case 64: e = launch_scores<4>(p, stream); break;
            default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)p.num_seqs), dim3(kTopkThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

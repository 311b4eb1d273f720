// Causal query chunks over paged context, on the matrix cores (head_dim 128, 1..16 query heads per
// K/V head).
//
// "vLLM 技术内幕" §3.2: a long prompt is processed in chunks under a per-step token budget, and each
// chunk attends causally to the context already in the cache while decodes run in the same step.
// Query token i of a chunk of length qlen in a sequence of n cached tokens (the chunk included) sits
// at position a = n - qlen + i and attends to tokens [0, a]. The scores, softmax and weighted V are
// those of paged decode ("deep dive into vLLM 05" §2; "KV Cache 与推理服务内存管理",
// paged_attention), for every row of the chunk.
//
// Mapping: the rows of one K/V head are the (position, query head) pairs of the chunk,
// position-major. A work-group owns 128 of them and walks their causal range of the paged context
// in 64-token K/V tiles. Its 8 waves form two groups of 4 (each wave two 16-row tiles of the 128
// rows): group 0 takes the first half of the range's tiles and group 1 the second half, each
// copying its tiles from HBM straight into its own LDS stages (lds_dma; the next tile is in flight
// while one is computed) shared by its 4 waves; at the end group 1 hands its (m, l, O) to group 0
// through LDS and group 0 merges them (log-sum-exp) and writes the rows. The causal ranges of a
// chunk's row blocks grow from one tile to the whole context, so halving the long ones evens out the
// work-groups of a launch. The two waves that share a SIMD belong to different groups, and group 1
// runs its value products one step behind its scores, so that one wave's softmax (VALU) meets the
// other's products (matrix core) rather than its own softmax. Per tile and row
// tile: S^T = K . Q^T on v_mfma_f32_16x16x32 (K from LDS, the rows' queries held in registers as the
// B columns), causal and context masks, lazily rescaled online softmax, and O += P . V on
// v_mfma_f32_16x16x32 with the value operand read through ds_read_b64_tr_b16 (the operand orders of
// mfma_common.h; P in token order sigma is the A operand as it leaves the softmax). For bf16 the
// probabilities go in as hi + lo pairs (pack2_split). Sequences with a single query row are not
// handled here: they are the decode rows of the call and go through the split-context decode.

#include <algorithm>

#include "decode_common.h"
#include "decode_mfma.h"
#include "mfma_common.h"

namespace pa {

namespace {

__device__ __forceinline__ int clamp_i(int v, int lo, int hi) { return max(lo, min(v, hi)); }

// Query length from a sequence's query start and end (0 for single-row sequences, which are decode
// rows).
__device__ __forceinline__ int chunk_len(int qs, int qe, const PrefillParams& p) {
    const int ql = clamp_i(qe - qs, 0, p.max_query_len);
    return ql >= 2 ? ql : 0;
}

// The item of a work-group: its sequence, row block, the sequence's first query row, chunk length
// and context length (as stored; clamped by the caller), all wave-uniform.
struct ChunkItem {
    int s, rb, q0, qlen, n;
};

// Work item w -> (sequence, row block), sequence-major, row blocks in descending order (the last row
// blocks see the longest causal range, so the longest items are dispatched first). The query starts
// and context lengths are read in the same pass, so the item's start waits for one round trip to
// memory instead of two.
__device__ __forceinline__ bool find_chunk_work(int w, const PrefillParams& p, ChunkItem& it) {
    const int lane = threadIdx.x & 63;
    int done = 0;
    for (int base = 0; base < p.num_seqs; base += 64) {
        const int s = base + lane;
        const bool in = s < p.num_seqs;
        const int qs = in ? p.query_start_loc[s] : 0;
        const int qe = in ? p.query_start_loc[s + 1] : 0;
        const int sl = in ? p.seq_lens[s] : 0;
        const int ql = chunk_len(qs, qe, p);
        const int n = (ql * p.group + p.rows_per_item - 1) / p.rows_per_item;
        int incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const int total = __builtin_amdgcn_readlane(incl, 63);
        if (w < done + total) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(done + incl > w);
            const int L = __builtin_ctzll(hit);
            const int before = done + __builtin_amdgcn_readlane(incl - n, L);
            const int cnt = __builtin_amdgcn_readlane(n, L);
            it.s = base + L;
            it.rb = cnt - 1 - (w - before);
            it.q0 = __builtin_amdgcn_readlane(qs, L);
            it.qlen = __builtin_amdgcn_readlane(ql, L);
            it.n = __builtin_amdgcn_readlane(sl, L);
            return true;
        }
        done += total;
    }
    return false;
}

}  // namespace

constexpr int kPT = 64;                    // tokens per K/V tile
constexpr int kPRow = kD * 2;              // bytes of one K/V head row
constexpr int kPStage = kPT * kPRow;       // 16 KB
constexpr int kPRows = 128;                // query rows per work-group
constexpr int kPWaves = 8;                 // waves per chunk work-group: two groups of 4

// K and V tiles: two K stages per wave group ([group][tile] inside each object, as separate objects
// per stage, see decode_mla.h), two V stages for group 0 and three for group 1 (s_pv0 and s_pv1
// hold [group][tile], s_pv2 group 1's third stage): group 1 multiplies a tile's values one step
// after its scores.
__shared__ __attribute__((aligned(16))) char s_pk0[2 * kPStage];
__shared__ __attribute__((aligned(16))) char s_pk1[2 * kPStage];
__shared__ __attribute__((aligned(16))) char s_pv0[2 * kPStage];
__shared__ __attribute__((aligned(16))) char s_pv1[2 * kPStage];
__shared__ __attribute__((aligned(16))) char s_pv2[kPStage];

template <int K>
__device__ __forceinline__ char* pk_stage() {
    if constexpr (K == 0) return s_pk0;
    else return s_pk1;
}
// V stage of the group's tile jrel (its jrel-th step): group 0 alternates two stages, group 1 cycles
// through three.
__device__ __forceinline__ char* pv_stage(int grp, int jrel) {
    if (grp == 0) return (jrel & 1) ? s_pv1 : s_pv0;
    const int r = jrel % 3;
    return r == 0 ? s_pv0 + kPStage : r == 1 ? s_pv1 + kPStage : s_pv2;
}

// Swizzle of the 16-byte chunks of tile row r (256-byte rows, a multiple of the 128-byte bank cycle):
// the rows a group of eight lanes reads together for the score operand (sigma order) and the four
// rows of a transposed value read get different chunks.
__device__ __forceinline__ int pswz(int r) { return (((r >> 2) & 3) << 1) | (r & 1); }

// One work-group's item of the chunk rows (item = (sequence, row block) index * Hkv + K/V head).
template <bool BF16>
__device__ __forceinline__ void prefill_block(const PrefillParams& p, const int item) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0..7
    const int grp = wave >> 2;                                           // tile half of this wave's group
    const int wv = wave & 3;                                             // wave within the group
    const int gtid = threadIdx.x & 255;                                  // thread within the group
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4;
    const int c = lane & 15;

    const int kvh = item % p.num_kv_heads;
    ChunkItem itm;
    if (!find_chunk_work(item / p.num_kv_heads, p, itm)) return;  // the same for the whole work-group
    const int s = itm.s, rb = itm.rb, q0 = itm.q0, qlen = itm.qlen;

    const int G = p.group;
    const int bs = p.block_size;
    const int bs_log2 = p.tiles_per_block_log2 + 4;
    const int64_t ncap = min((int64_t)p.max_seq_len, (int64_t)p.bt_stride * bs);
    const int n = (int)max((int64_t)0, min((int64_t)itm.n, ncap));
    const int R = qlen * G;                                 // rows of this K/V head in this chunk
    const int wg_r0 = rb * kPRows;
    const int wg_rend = min(R, wg_r0 + kPRows);
    const int wg_amax = n - qlen + (wg_rend - 1) / G;      // causal limit of the work-group's last row
    const int r0 = wg_r0 + 32 * wv;                        // this wave's rows
    const int rend = min(wg_rend, r0 + 32);
    const int a_max = r0 < rend ? n - qlen + (rend - 1) / G : -1;
    const int amin = n - qlen + r0 / G;                    // causal limit of this wave's first row
    const int hq0 = kvh * G;
    const int ntiles = wg_amax >= 0 ? wg_amax / kPT + 1 : 0;
    const int wave_tiles = a_max >= 0 ? a_max / kPT + 1 : 0;  // tiles holding this wave's visible tokens
    // Tile halves: group 0 takes tiles [0, mid), group 1 [mid, ntiles); both run mid steps.
    const int mid = (ntiles + 1) >> 1;
    const int jbeg = grp == 0 ? 0 : mid;
    const int jend = grp == 0 ? mid : ntiles;

    // Per row tile: Q of row r0 + 16nt + c as the B operand, and that row's causal limit.
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q);
    uint4 qb[2][4];
    int alim[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        const int r = r0 + 16 * nt + c;
        const bool valid = r < rend;
        const int pos = valid ? r / G : 0;
        const int head = valid ? r - pos * G : 0;
        alim[nt] = valid ? n - qlen + pos : -1;
        const uint16_t* qr = qbase + ((size_t)(q0 + pos) * p.num_q_heads + hq0 + head) * kD;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qb[nt][ks] = valid ? *reinterpret_cast<const uint4*>(qr + 32 * ks + 8 * g4) : make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // queries in, before the copies start

    // Per-lane LDS offsets. Score operand: row 16sub + sigma(c), chunk 4ks + g4 (swizzled).
    int a_off[4];
    {
        const int row = sigma(c);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) a_off[ks] = row * kPRow + (((4 * ks + g4) ^ pswz(row)) << 4);
    }
    // Value operand through ds_read_b64_tr_b16 (see decode_mla.hip): lane c of lane group g4 supplies
    // row 16sub + g4 + 4 (c >> 2), dims 16dt + 4 (c & 3) .. +3.
    int trbase[4];
    {
        const int j = c >> 2, h = (c >> 1) & 1;
#pragma unroll
        for (int d3 = 0; d3 < 4; ++d3)
            trbase[d3] = (g4 + 4 * j) * kPRow + ((2 * (d3 ^ j) + (h ^ (g4 & 1))) << 4) + ((c & 1) << 3);
    }

    // Copies: wave w of a group loads tokens [16w, 16w + 16) of the group's tile, four rows per load
    // instruction: lane i fills LDS chunk i % 16 of row 16w + 4r + i / 16 with global chunk
    // (i % 16) ^ pswz(row).
    const int64_t krow = p.k_row_bytes, vrow = p.v_row_bytes;
    const uint32_t nb = (uint32_t)p.num_blocks;
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const char* dummy = reinterpret_cast<const char*>(qbase);
    int dma_row[4], dma_chunk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        dma_row[r] = 16 * wv + 4 * r + (lane >> 4);
        dma_chunk[r] = (lane & 15) ^ pswz(dma_row[r]);
    }
    // Block id of this wave's 16 tokens of tile j, and whether each 16-token group of the tile holds
    // context tokens in a valid block (bit g).
    auto group_id = [&](int j, int g) __attribute__((always_inline)) {
        const int t = j * kPT + 16 * g;
        return t < n ? load_scalar(bt + (t >> bs_log2)) : -1;
    };
    // Block ids of the next tile to copy, one per 16-token group (-1: past the context). They are
    // only loaded here; the checks that use them wait for the loads in the next step, after its
    // barrier, so the scalar loads' latency is hidden behind the barrier.
    int pre_id[4] = {-1, -1, -1, -1};
    auto prefetch = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g) pre_id[g] = j < jend ? group_id(j, g) : -1;
    };
    int tile_ok[2] = {0, 0};
    auto issue = [&](auto kst, int j) __attribute__((always_inline)) {
        constexpr int K = decltype(kst)::value;
        int pre_ok = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) pre_ok |= ((uint32_t)pre_id[g] < nb ? 1 : 0) << g;
        tile_ok[K] = pre_ok;
        char* ks_ = pk_stage<K>() + grp * kPStage;
        char* vs_ = pv_stage(grp, j - jbeg);
        if (pre_ok & (1 << wv)) {
            const int64_t phys = pre_id[wv];
            const char* kb = p.k + phys * p.k_block_stride + (int64_t)kvh * kPRow;
            const char* vb = p.v + phys * p.v_block_stride + (int64_t)kvh * kPRow;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row_in_block = (j * kPT + dma_row[r]) & (bs - 1);
                const char* ksrc = kb + row_in_block * krow + dma_chunk[r] * 16;
                const char* vsrc = vb + row_in_block * vrow + dma_chunk[r] * 16;
                lds_dma<16>(ksrc, lds_addr(ks_) + (16 * wv + 4 * r) * kPRow);
                lds_dma<16>(vsrc, lds_addr(vs_) + (16 * wv + 4 * r) * kPRow);
            }
        } else {
            // No context tokens here, or an invalid block id: the scores are masked; the value rows
            // are zeroed so that masked probabilities (0) never meet NaN.
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<uint4*>(vs_ + dma_row[r] * kPRow + ((lane & 15) << 4)) = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    (void)dummy;

    float m[2], l[2];
    f32x4_t O[2][8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        m[nt] = kNegInf;
        l[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[nt][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = p.scale_log2;

    // Probabilities of the last scored tile as the A operand of its value product (hi and lo parts).
    uint4 Ahi[2][2], Alo[2][2];
    auto scores = [&](auto kst, int j) __attribute__((always_inline)) {
        constexpr int K = decltype(kst)::value;
        const char* kt = pk_stage<K>() + grp * kPStage;
        const int t0 = j * kPT;
        const int okb = tile_ok[K];

        // Scores for the four 16-token sub-tiles, k-step by k-step over the eight (sub-tile, row tile)
        // accumulators (consecutive products independent); the K operands of the next k-step are
        // read while the current one's products run.
        f32x4_t S[4][2];
        uint4 abuf[2][4];
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) abuf[0][sub] = *reinterpret_cast<const uint4*>(kt + sub * 16 * kPRow + a_off[0]);
#pragma unroll
        for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) S[sub][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks + 1 < 4) {
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
                    abuf[(ks + 1) & 1][sub] = *reinterpret_cast<const uint4*>(kt + sub * 16 * kPRow + a_off[ks + 1]);
            }
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) S[sub][nt] = mfma_k32<BF16>(abuf[ks & 1][sub], qb[nt][ks], S[sub][nt]);
        }

        // Register jj of sub-tile sub holds token t0 + 16 sub + g4 + 4 jj of row c. A tile inside
        // every row's causal range with all four 16-token groups in valid blocks needs no masks (the
        // wave's first row has the shortest range).
        const bool full = okb == 15 && t0 + kPT - 1 <= amin;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            bool ok[4][4];
            float mx = kNegInf;
            if (full) {
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) mx = fmaxf(mx, S[sub][nt][jj]);
            } else {
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int t = t0 + 16 * sub + g4 + 4 * jj;
                        ok[sub][jj] = ((okb >> sub) & 1) && t <= alim[nt];
                        mx = ok[sub][jj] ? fmaxf(mx, S[sub][nt][jj]) : mx;
                    }
            }
            // The reference m is the same in the four lane groups of a row, so a row must move it
            // exactly when one of its lane groups' maxima exceeds it by the slack: the row maxima
            // (two cross-lane steps) are formed only then.
            if (__builtin_amdgcn_ballot_w64(mx * sl2 > m[nt] + kRescaleSlack) != 0) {
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float tmax = mx * sl2;
                const bool need = tmax > m[nt] + kRescaleSlack;
                const float mnew = need ? tmax : m[nt];
                const float alpha = need ? fast_exp2(m[nt] - mnew) : 1.f;
                l[nt] *= alpha;
                m[nt] = mnew;
                const f32x4_t av = {__shfl(alpha, 4 * g4), __shfl(alpha, 4 * g4 + 1), __shfl(alpha, 4 * g4 + 2),
                                    __shfl(alpha, 4 * g4 + 3)};
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) O[nt][dt] *= av;
            }
            float pr[4][4];
#pragma unroll
            for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float ex = fast_exp2(fmaf(S[sub][nt][jj], sl2, -m[nt]));
                    pr[sub][jj] = full || ok[sub][jj] ? ex : 0.f;
                    l[nt] += pr[sub][jj];
                }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t hw[4], lw[4];
                pack2_split<BF16>(pr[2 * h][0], pr[2 * h][1], hw[0], lw[0]);
                pack2_split<BF16>(pr[2 * h][2], pr[2 * h][3], hw[1], lw[1]);
                pack2_split<BF16>(pr[2 * h + 1][0], pr[2 * h + 1][1], hw[2], lw[2]);
                pack2_split<BF16>(pr[2 * h + 1][2], pr[2 * h + 1][3], hw[3], lw[3]);
                Ahi[nt][h] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                Alo[nt][h] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
            }
        }
    };

    // O += P . V for the tile whose values are at vt, with P in Ahi / Alo.
    auto pv = [&](const char* vt) __attribute__((always_inline)) {
        // PV over the two 32-token halves h: B operand of dims [16dt, 16dt + 16) is two transposed
        // reads (sub-tiles 2h and 2h + 1).
        auto load_b = [&](int h, int dt) __attribute__((always_inline)) {
            const char* base = vt + trbase[dt & 3] + (dt >> 2) * 128 + 2 * h * 16 * kPRow;
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(base));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4_t*)(base + 16 * kPRow));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            return make_uint4(l2.x, l2.y, h2.x, h2.y);
        };
        // Loaded two products ahead; the lo products of a tile run one output tile behind its hi
        // products, so no two consecutive products share an accumulator.
        uint4 bq[4];  // ring: slot x % 4 holds product x's operand until its lo product is issued
        bq[0] = load_b(0, 0);
        bq[1] = load_b(0, 1);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            const int h = x >> 3, dt = x & 7;
            if (x + 2 < 16) bq[(x + 2) % 4] = load_b((x + 2) >> 3, (x + 2) & 7);
            const uint4 B = bq[x % 4];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) O[nt][dt] = mfma_k32<BF16>(Ahi[nt][h], B, O[nt][dt]);
            if constexpr (BF16) {
                if (x > 0) {
                    const int hp = (x - 1) >> 3, dp = (x - 1) & 7;
#pragma unroll
                    for (int nt = 0; nt < 2; ++nt) O[nt][dp] = mfma_k32<BF16>(Alo[nt][hp], bq[(x - 1) % 4], O[nt][dp]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (BF16) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) O[nt][7] = mfma_k32<BF16>(Alo[nt][1], bq[15 % 4], O[nt][7]);
        }
    };

    // Step jrel of both groups: group 0 on tile jrel, group 1 on tile mid + jrel (if still in its
    // range). Every barrier is reached by all 8 waves. Group 0 scores a tile and multiplies its values
    // in the same step; group 1 first multiplies the values of the tile it scored in the previous
    // step, then scores the current one. So the two waves of a SIMD (one per group) are in opposite
    // phases: while one runs its softmax on the VALU, the other's products keep the matrix core busy.
    // The loop of one group (G1: group 1), each group with its own copy of the code, so that the
    // probabilities group 1 carries from one step to the next never meet group 0's register peak.
    auto run = [&](auto g1) __attribute__((always_inline)) {
        constexpr bool G1 = decltype(g1)::value;
        bool have_prev = false;  // group 1: a scored tile still to be multiplied by its values
        const char* v_prev = s_pv2;
        auto step = [&](auto kst, int jrel) __attribute__((always_inline)) {
            constexpr int K = decltype(kst)::value;
            const int j = jbeg + jrel;
            const bool live = j < jend;
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // this wave's copies of tile j are in
            lds_barrier();                                      // everyone's are; the previous tile is done
            // A tile reaching past the context: zero its value rows past it (the copies brought
            // whatever the block holds there). The condition covers both groups' tiles, so the
            // barrier is uniform.
            const bool z0 = jrel < mid && (jrel + 1) * kPT > n;
            const bool z1 = mid + jrel < ntiles && (mid + jrel + 1) * kPT > n;
            if (z0 || z1) {
                if (live && (j + 1) * kPT > n) {
                    char* vs_ = pv_stage(grp, jrel);
                    for (int x = gtid; x < kPT * 16; x += 256) {
                        const int row = x >> 4;
                        if (j * kPT + row >= n) *reinterpret_cast<uint4*>(vs_ + row * kPRow + ((x & 15) << 4)) = make_uint4(0u, 0u, 0u, 0u);
                    }
                }
                __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
                lds_barrier();
            }
            if (j + 1 < jend) issue(std::integral_constant<int, K ^ 1>{}, j + 1);
            const bool runs = live && j < wave_tiles;
            if constexpr (!G1) {
                if (runs) {
                    scores(kst, j);
                    pv(pv_stage(0, jrel));
                }
            } else {
                if (have_prev) pv(v_prev);
                have_prev = runs;
                v_prev = pv_stage(1, jrel);
                if (runs) scores(kst, j);
            }
            // The block ids of tile j + 2, read after the products: scalar loads share their wait
            // counter with LDS reads, so issued before the score phase they would stall its first
            // LDS wait.
            prefetch(j + 2);
        };
        prefetch(jbeg);
        if (jbeg < jend) issue(std::integral_constant<int, 0>{}, jbeg);
        prefetch(jbeg + 1);
        for (int jrel = 0; jrel < mid; jrel += 2) {
            step(std::integral_constant<int, 0>{}, jrel);
            if (jrel + 1 < mid) step(std::integral_constant<int, 1>{}, jrel + 1);
        }
        if constexpr (G1) {
            if (have_prev) pv(v_prev);  // the last tile's values
        }
    };
    if (mid > 0) {
        if (grp == 0) run(std::false_type{});
        else run(std::true_type{});
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));

    // Row sums over the four lane groups: row 16 nt + c in lane c.
    float lt[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        lt[nt] = l[nt];
        lt[nt] += __shfl_xor(lt[nt], 16);
        lt[nt] += __shfl_xor(lt[nt], 32);
    }
    // Group 1 hands (m, l, O) of its rows to group 0 through the K and V stages, which are free once
    // every wave has passed its last product (the barrier below).
    lds_barrier();
    float* xo = reinterpret_cast<float*>(wv < 2 ? s_pk0 : s_pk1) + (wv & 1) * (32 * kD);  // 32 rows x 128
    float* xm = reinterpret_cast<float*>(s_pv0) + wv * 64;                                  // 32 rows x (m, l)
    if (grp == 1) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) xo[(16 * nt + 4 * g4 + jj) * kD + 16 * dt + c] = O[nt][dt][jj];
            if (g4 == 0) {
                xm[2 * (16 * nt + c)] = m[nt];
                xm[2 * (16 * nt + c) + 1] = lt[nt];
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    lds_barrier();

    // Group 0 merges its rows with group 1's and puts them, in the output type, into a row-major
    // staging tile [128 rows x 128 dims] (the second V stage, free by now); then all 8 waves write
    // the tile's rows out as 16-byte stores.
    char* stg = s_pv1;
    if (grp == 0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            // Weights of the two halves for row 16 nt + c: 2^(m_i - M) with M the larger reference (a
            // half without visible tokens has m = -inf and weight 0).
            const float m1 = xm[2 * (16 * nt + c)];
            const float l1 = xm[2 * (16 * nt + c) + 1];
            const float M = fmaxf(m[nt], m1);
            const float w0 = m[nt] == M ? 1.f : fast_exp2(m[nt] - M);
            const float w1 = m1 == M ? 1.f : fast_exp2(m1 - M);
            const float Lc = w0 * lt[nt] + w1 * l1;
            const float inv_c = Lc > 0.f ? 1.f / Lc : 0.f;  // no visible token (inconsistent lengths): output 0
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rl = 32 * wv + 16 * nt + 4 * g4 + jj;  // row within the work-group
                const float a0 = __shfl(w0 * inv_c, 4 * g4 + jj);
                const float a1 = __shfl(w1 * inv_c, 4 * g4 + jj);
                const float* x1 = xo + (16 * nt + 4 * g4 + jj) * kD + c;
                uint16_t* st = reinterpret_cast<uint16_t*>(stg + rl * kPRow) + c;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    st[16 * dt] = (uint16_t)(pack2<BF16>(fmaf(O[nt][dt][jj], a0, x1[16 * dt] * a1), 0.f) & 0xFFFFu);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    lds_barrier();
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int k = 0; k < kPRows * 16 / (64 * kPWaves); ++k) {
        const int t = threadIdx.x + 64 * kPWaves * k;
        const int rl = t >> 4, ch = t & 15;
        const int r = wg_r0 + rl;
        if (r < wg_rend) {
            const int pos = r / G;
            const int head = r - pos * G;
            *reinterpret_cast<uint4*>(out + ((size_t)(q0 + pos) * p.num_q_heads + hq0 + head) * kD + 8 * ch) =
                *reinterpret_cast<const uint4*>(stg + rl * kPRow + 16 * ch);
        }
    }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_kernel(PrefillParams p) {
    prefill_block<BF16>(p, blockIdx.x);
}

// A mixed call in one launch: the first work-groups take the decode rows on the grouped-query decode
// waves, the rest the chunk rows. Both kinds fit the same budget: 8 waves per work-group, two waves
// per SIMD; the chunk rows' LDS tiles (128 KB) limit a CU to one work-group, which is also the
// decode waves' register-limited occupancy, so the decode rows stream from HBM as they would alone
// and the chunk rows take over each CU as its decode work-groups retire. Of the orders measured
// (decode rows first, chunk rows first, alternating singly or in runs of 8) this one gives the
// shortest call: interleaving the two kinds leaves half the CUs streaming decode rows, and the
// register-limited decode waves of one CU cannot keep enough loads in flight to make up for it.
template <bool BF16>
__global__ __launch_bounds__(64 * kPWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void mixed_chunk_kernel(
    PrefillParams pp, DenseDecodeParams dp, int decode_wgs) {
    int b = blockIdx.x;
    const bool chunk = b >= decode_wgs;
    if (chunk) b -= decode_wgs;
    if (chunk) {
        prefill_block<BF16>(pp, b);
    } else {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        decode_mfma_wave<BF16>(dp, b * kPWaves + wave);
    }
}

namespace {

// Upper bound of the chunk-row work-groups: every sequence's rows rounded up to whole row blocks.
int64_t prefill_wgs(const PrefillParams& p) {
    const int64_t per_seq = ((int64_t)p.max_query_len * p.group + p.rows_per_item - 1) / p.rows_per_item;
    const int64_t bound = ((int64_t)p.total_q * p.group + p.rows_per_item - 1) / p.rows_per_item + p.num_seqs;
    return std::max<int64_t>(0, std::min(per_seq * p.num_seqs, bound) * p.num_kv_heads);
}

}  // namespace

hipError_t launch_prefill_chunk(const PrefillParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    const int64_t wgs = prefill_wgs(p);
    if (wgs <= 0) return hipSuccess;
    if (p.is_bf16)
        hipLaunchKernelGGL((prefill_mfma_kernel<true>), dim3((unsigned)wgs), dim3(64 * kPWaves), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_mfma_kernel<false>), dim3((unsigned)wgs), dim3(64 * kPWaves), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mixed_chunk(const PrefillParams& pp, const DenseDecodeParams& dp, hipStream_t stream) {
    const int64_t pw = pp.num_seqs > 0 ? prefill_wgs(pp) : 0;
    const int64_t dw = ((int64_t)dp.num_kv_heads * dp.num_seqs * dp.max_parts + kPWaves - 1) / kPWaves;
    if (pw + dw <= 0) return hipSuccess;
    if (pw + dw > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (pp.is_bf16)
        hipLaunchKernelGGL((mixed_chunk_kernel<true>), dim3((unsigned)(pw + dw)), dim3(64 * kPWaves), 0, stream, pp,
                           dp, (int)dw);
    else
        hipLaunchKernelGGL((mixed_chunk_kernel<false>), dim3((unsigned)(pw + dw)), dim3(64 * kPWaves), 0, stream, pp,
                           dp, (int)dw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || dp.max_parts <= 1) return e;
    return launch_decode_reduce(dp, stream);
}

}  // namespace pa

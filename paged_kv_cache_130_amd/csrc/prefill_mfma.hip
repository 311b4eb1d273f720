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
// Mapping: the rows of one K/V head are the (position, query head) pairs of the chunk, position-major.
// A wave owns NT 16-row tiles of them, which share every K/V tile it loads. Per 16-token K/V tile and
// row tile: S^T = K . Q^T on v_mfma_f32_16x16x32 (rows of Q are the B columns), causal and context
// masks, lazily rescaled online softmax, and O += P . V on v_mfma_f32_16x16x16. The operand orders
// are those of decode_mfma.hip (mfma_common.h). Sequences with a single query row are not handled
// here: they are the decode rows of the call and go through the split-context decode kernels.
//
// Block ids come through a broadcast load issued two tiles ahead, and K/V tiles through register
// prefetch one tile ahead. All loads are unconditional (past the end they read a cached query line),
// so the in-order wait counts stay exact and two tiles are in flight while one is computed.

#include "decode_common.h"
#include "mfma_common.h"

namespace pa {

namespace {

__device__ __forceinline__ int clamp_i(int v, int lo, int hi) { return max(lo, min(v, hi)); }

// Query length of sequence s (0 for single-row sequences, which are decode rows).
__device__ __forceinline__ int chunk_len(int s, const PrefillParams& p) {
    const int ql = clamp_i(p.query_start_loc[s + 1] - p.query_start_loc[s], 0, p.max_query_len);
    return ql >= 2 ? ql : 0;
}

__device__ __forceinline__ int row_blocks(int s, const PrefillParams& p) {
    return (chunk_len(s, p) * p.group + p.rows_per_item - 1) / p.rows_per_item;
}

// Work item w -> (sequence, row block), sequence-major, row blocks in descending order (the last row
// blocks see the longest causal range, so the longest items are dispatched first).
__device__ __forceinline__ bool find_chunk_work(int w, const PrefillParams& p, int& s_out, int& rb_out) {
    const int lane = threadIdx.x & 63;
    int done = 0;
    for (int base = 0; base < p.num_seqs; base += 64) {
        const int s = base + lane;
        const int n = s < p.num_seqs ? row_blocks(s, p) : 0;
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
            s_out = base + L;
            rb_out = cnt - 1 - (w - before);
            return true;
        }
        done += total;
    }
    return false;
}

}  // namespace

template <bool BF16, int NT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(PrefillParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g4 = lane >> 4;
    const int c = lane & 15;

    const int item = blockIdx.x * 4 + wave;
    const int kvh = item % p.num_kv_heads;
    int s, rb;
    if (!find_chunk_work(item / p.num_kv_heads, p, s, rb)) return;

    const int G = p.group;
    const int bs = p.block_size;
    const int q0 = __builtin_amdgcn_readfirstlane(p.query_start_loc[s]);
    const int qlen = __builtin_amdgcn_readfirstlane(chunk_len(s, p));
    const int64_t ncap = min((int64_t)p.max_seq_len, (int64_t)p.bt_stride * bs);
    const int n = (int)max((int64_t)0, min((int64_t)__builtin_amdgcn_readfirstlane(p.seq_lens[s]), ncap));
    const int R = qlen * G;              // rows of this K/V head in this chunk
    const int r0 = rb * 16 * NT;         // first row of this item
    const int rend = min(R, r0 + 16 * NT);
    const int a_max = n - qlen + (rend - 1) / G;  // causal limit of the item's last row
    const int hq0 = kvh * G;

    // Per row tile: Q of row r0 + 16*nt + c as the B operand, and that row's causal limit.
    const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q);
    uint4 qb[NT][4];
    int alim[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
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

    const int tpb_log2 = p.tiles_per_block_log2;
    const int tpb_mask = (1 << tpb_log2) - 1;
    const int ntiles = a_max >= 0 ? (a_max + 16) >> 4 : 0;
    const int last = ntiles - 1;
    const int32_t* bt = p.block_tables + (size_t)s * p.bt_stride;
    const int64_t krow = p.k_row_bytes, vrow = p.v_row_bytes;
    const uint32_t klane = (uint32_t)(kvh * (kD * 2) + 16 * g4) + (uint32_t)sigma(c) * (uint32_t)krow;
    const uint32_t vlane = (uint32_t)(kvh * (kD * 2) + 16 * c) + (uint32_t)g4 * (uint32_t)vrow;
    const uint32_t nb = (uint32_t)p.num_blocks;
    const char* dummy = reinterpret_cast<const char*>(qbase + (size_t)q0 * p.num_q_heads * kD);

    // Block id of tile j, loaded by every lane from the same address (one cached line).
    auto load_bid = [&](int j) { return bt[(j <= last ? j : 0) >> tpb_log2]; };
    auto load = [&](uint4 (&kk)[4], uint4 (&vv)[4], int j, int phys) {
        const bool real = j <= last;
        phys = ((uint32_t)phys < nb) ? phys : 0;  // an out-of-range id is masked when the tile is used
        const int64_t row0 = (int64_t)((j & tpb_mask) << 4);
        const char* kt = real ? p.k + (int64_t)phys * p.k_block_stride + row0 * krow : dummy;
        const char* vt = real ? p.v + (int64_t)phys * p.v_block_stride + row0 * vrow : dummy;
        const int64_t kstep = real ? 64 : 0, vstep = real ? 4 * vrow : 0;
        const uint32_t ko = real ? klane : 0u, vo = real ? vlane : 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kk[i] = *reinterpret_cast<const uint4*>(kt + i * kstep + ko);
            vv[i] = load_nt16(vt + i * vstep + vo);
        }
    };

    float m[NT], l[NT];
    f32x4_t O[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m[nt] = kNegInf;
        l[nt] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) O[nt][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = p.scale_log2;

    auto step = [&](const uint4 (&kk)[4], uint4 (&vv)[4], int j, bool bad) {
        const int t0 = j << 4;
        const int nvalid = bad ? 0 : min(16, n - t0);  // tokens of this tile inside the context
        bool inctx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            inctx[i] = g4 + 4 * i < nvalid;
            if (!inctx[i]) vv[i] = make_uint4(0u, 0u, 0u, 0u);  // rows past the context may hold NaN
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) S = mfma_k32<BF16>(kk[ks], qb[nt][ks], S);
            bool ok[4];
            float mx = kNegInf;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                ok[jj] = inctx[jj] && (t0 + g4 + 4 * jj <= alim[nt]);  // causal: token <= position
                mx = ok[jj] ? fmaxf(mx, S[jj]) : mx;
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float tmax = mx * sl2;
            const bool need = tmax > m[nt] + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                const float mnew = need ? tmax : m[nt];
                const float alpha = need ? fast_exp2(m[nt] - mnew) : 1.f;
                l[nt] *= alpha;
                m[nt] = mnew;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float a = __shfl(alpha, 4 * g4 + jj);
#pragma unroll
                    for (int e = 0; e < 8; ++e) O[nt][e][jj] *= a;
                }
            }
            float pr[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float ex = fast_exp2(fmaf(S[jj], sl2, -m[nt]));
                pr[jj] = ok[jj] ? ex : 0.f;
                l[nt] += pr[jj];
            }
            uint2 A, Alo;
            pack2_split<BF16>(pr[0], pr[1], A.x, Alo.x);
            pack2_split<BF16>(pr[2], pr[3], A.y, Alo.y);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint2 B = v_operand(vv, e);
                O[nt][e] = mfma_k16<BF16>(A, B, O[nt][e]);
                if constexpr (BF16) O[nt][e] = mfma_k16<BF16>(Alo, B, O[nt][e]);
            }
        }
    };

    if (ntiles > 0) {
        uint4 k0[4], v0[4], k1[4], v1[4];
        int bid_a = load_bid(0);
        int phys0 = __builtin_amdgcn_readfirstlane(bid_a);
        int bid_b = load_bid(1);
        load(k0, v0, 0, phys0);
        bool bad0 = (uint32_t)phys0 >= nb, bad1 = false;
        for (int j = 0; j < ntiles; j += 2) {
            bid_a = load_bid(j + 2);
            const int phys1 = __builtin_amdgcn_readfirstlane(bid_b);
            bad1 = (uint32_t)phys1 >= nb;
            load(k1, v1, j + 1, phys1);
            step(k0, v0, j, bad0);
            bid_b = load_bid(j + 3);
            const int phys2 = __builtin_amdgcn_readfirstlane(bid_a);
            bad0 = (uint32_t)phys2 >= nb;
            load(k0, v0, j + 2, phys2);
            if (j + 1 < ntiles) step(k1, v1, j + 1, bad1);
        }
    }

    uint16_t* out = reinterpret_cast<uint16_t*>(p.out);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float lt = l[nt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int r = r0 + 16 * nt + 4 * g4 + jj;
            const float L = __shfl(lt, 4 * g4 + jj);
            if (r >= rend) continue;
            const int pos = r / G;
            const int head = r - pos * G;
            const float inv = L > 0.f ? 1.f / L : 0.f;  // no visible token (inconsistent lengths): output 0
            uint4 o;
            o.x = pack2<BF16>(O[nt][0][jj] * inv, O[nt][1][jj] * inv);
            o.y = pack2<BF16>(O[nt][2][jj] * inv, O[nt][3][jj] * inv);
            o.z = pack2<BF16>(O[nt][4][jj] * inv, O[nt][5][jj] * inv);
            o.w = pack2<BF16>(O[nt][6][jj] * inv, O[nt][7][jj] * inv);
            *reinterpret_cast<uint4*>(out + ((size_t)(q0 + pos) * p.num_q_heads + hq0 + head) * kD + c * 8) = o;
        }
    }
}

hipError_t launch_prefill_chunk(const PrefillParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    // Upper bound of the work items: every sequence's rows rounded up to whole items.
    const int64_t items = ((int64_t)p.max_query_len * p.group + p.rows_per_item - 1) / p.rows_per_item;
    const int64_t waves = items * p.num_seqs * p.num_kv_heads;
    const int64_t bound = ((int64_t)p.total_q * p.group + p.rows_per_item - 1) / p.rows_per_item +
                          p.num_seqs;  // sum of per-sequence item counts is at most this
    const int64_t w = min(waves, bound * p.num_kv_heads);
    const int64_t wgs = (w + 3) / 4;
    if (wgs <= 0) return hipSuccess;
    if (p.is_bf16)
        hipLaunchKernelGGL((prefill_mfma_kernel<true, 2>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((prefill_mfma_kernel<false, 2>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

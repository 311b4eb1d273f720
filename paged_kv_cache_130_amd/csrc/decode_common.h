// Work mapping shared by the decode kernels: context clamping and the compact, partition-major
// list of (partition, sequence) items. Included only by .hip kernel files.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr float kNegInf = -__builtin_inff();

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Online softmax with a lazily moved reference: each row keeps a reference m (log2 domain) and
// accumulates p = 2^(s*scale*log2e - m). The reference moves only when a tile's maximum exceeds it
// by more than kRescaleSlack, so p <= 2^kRescaleSlack and the accumulators stay well inside fp32
// range. When no lane of the wave needs to move (the common case after the first tile), the rescale
// of l and the accumulators is skipped. The result is the same softmax: every p and the
// accumulators always share the same reference.
constexpr float kRescaleSlack = 8.f;

// s_waitcnt immediate: wait until at most vm vector-memory operations are outstanding and all LDS
// operations are done (expcnt not waited on).
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | ((vm >> 4) << 14); }

// Read of a wave-uniform address through the constant address space, so that it becomes a scalar
// load (counted by lgkmcnt). A vector load there would be counted by vmcnt, and waiting for it would
// also wait for every direct-to-LDS copy issued before it. Only for data no kernel of the call writes.
template <typename T>
__device__ __forceinline__ T load_scalar(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)ptr;
}

// Keeps the compiler from moving memory accesses across the hardware barrier next to it.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Work-group barrier for kernels that stage tiles with direct-to-LDS loads: the caller waits for its
// own copies with s_waitcnt first. (__syncthreads would also wait for every copy still in flight.)
__device__ __forceinline__ void lds_barrier() {
    compiler_fence();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Byte address in LDS of p, a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS copy of BYTES (4 or 16) per lane: lane i's BYTES at src land at LDS byte address
// lds + BYTES * i (lds is wave-uniform). It is the instruction __builtin_amdgcn_global_load_lds
// emits, issued through inline asm. The compiler counts the builtin as an outstanding flat access to
// LDS, and while one is in flight it waits for any LDS read by draining all LDS operations
// (lgkmcnt(0)), which in a pipeline that always has copies in flight defeats every operand prefetch.
// Hidden from the compiler, the copy is ordered only by the caller: an s_waitcnt vmcnt for its own
// copies, then a barrier, before anything reads the destination, and an s_waitcnt vmcnt(0) before
// the kernel ends. M0 (which the instruction takes the LDS address from) is set inside the asm, one
// wait state ahead of the copy (an SALU write of M0 followed by a global load into LDS needs one, as
// the compiler also inserts for the builtin); the kernels that use this helper use M0 for nothing else.
template <int BYTES>
__device__ __forceinline__ void lds_dma(const void* src, uint32_t lds) {
    static_assert(BYTES == 4 || BYTES == 16, "4 or 16 bytes per lane");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    if constexpr (BYTES == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "s"(m0) : "memory");
}

// The same copy from a wave-uniform base plus a per-lane 32-bit byte offset (the instruction's
// scalar-base form: no 64-bit address arithmetic per lane).
template <int BYTES>
__device__ __forceinline__ void lds_dma_sv(const void* base, uint32_t off, uint32_t lds) {
    static_assert(BYTES == 16, "16 bytes per lane");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
    const uint64_t b = (uint64_t)(uintptr_t)base;
    // readfirstlane returns int: both halves are zero-extended through uint32_t.
    const uint64_t sb = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(sb), "s"(m0)
                 : "memory");
}

// Two E4M3 codes (bytes 0, 1 of w, or bytes 2, 3 when HI) -> two bf16 in one dword, the first in the
// low half. Exact: every E4M3 value is a bf16 value, and the scale is 1.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_bf16(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// v_perm_b32 selectors: low 16-bit halves of (a, b) -> (a.lo, b.lo); high halves -> (a.hi, b.hi).
constexpr uint32_t kSelLo = 0x05040100u;
constexpr uint32_t kSelHi = 0x07060302u;

// 16 bytes through a nontemporal load: each K/V row is read once per call, so it should not displace
// lines that are reused.
__device__ __forceinline__ uint4 load_nt16(const char* ptr) {
    const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
    return make_uint4(a.x, a.y, a.z, a.w);
}

// Context length bounded to [0, min(max_context_len, bt_stride * block_size)], so that no read
// goes past the block table row.
__device__ __forceinline__ int clamp_context(int ctx, const DenseDecodeParams& p) {
    const int64_t cap = min((int64_t)p.max_context_len, (int64_t)p.bt_stride * p.block_size);
    return (int)max((int64_t)0, min((int64_t)ctx, cap));
}

// Work items of sequence s: one per partition; an empty context still owns one item, which writes
// the zero output. In a mixed prefill call only single-row sequences have items.
__device__ __forceinline__ int parts_of(int s, const DenseDecodeParams& p) {
    if (p.query_start_loc != nullptr && p.query_start_loc[s + 1] - p.query_start_loc[s] != 1) return 0;
    const int ctx = clamp_context(p.context_lens[s], p);
    return ctx == 0 ? 1 : (ctx + p.partition_tokens - 1) / p.partition_tokens;
}

// Row of q / out that holds sequence s's (single) query token.
__device__ __forceinline__ int query_row(int s, const DenseDecodeParams& p) {
    return p.query_start_loc != nullptr ? __builtin_amdgcn_readfirstlane(p.query_start_loc[s]) : s;
}

// Work item w of the list -> (sequence, partition, clamped context length). Returns false past
// the end.
//
// The list holds every full partition (partition_tokens tokens) first, in partition-major order,
// then one item per sequence for its last, partial partition (or for its empty context, which
// writes the zero output), ordered by decreasing length in 8 buckets of partition_tokens / 8
// tokens (empty contexts last) and by sequence within a bucket. Waves take items in list order, so
// items of equal length run together and the short ones run last: the waves of the call finish
// close together instead of waiting on a few full partitions dispatched at the end. (Partition
// boundaries depend only on logical positions, so the order changes no result.)
//
// Full part: C(q) = sum_s min(f_s, q), f_s = full partitions of s, counts the full items of
// partitions below q; item w lies in partition q with C(q) <= w < C(q+1) and is the (w - C(q))-th
// sequence (in order) with more than q full partitions. Partial part: bucket counts from the
// longest bucket down. Counts are summed as integers (the host bounds num_seqs * max_parts below
// 2^31).
//
// With up to 256 sequences the per-sequence values of all of them are read once into registers
// (sequence 64k + lane in register k), with every load issued before the first wait, so the search
// costs one memory round trip and then only register arithmetic. With more sequences they are
// re-read from memory for every count.
__device__ __forceinline__ bool find_work(int w, const DenseDecodeParams& p, int& s_out, int& part_out, int& ctx_out) {
    constexpr int NC = 4;
    constexpr int kBuckets = 8;
    const int lane = threadIdx.x & 63;
    const bool fast = p.num_seqs <= 64 * NC;
    const bool mixed = p.query_start_loc != nullptr;
    const int P = p.partition_tokens;
    // Full partitions of sequence s, and the key of its partial item: 1 + bucket for a partial
    // partition of r tokens (bucket (r - 1) * 8 / P), 0 for an empty context, -1 for none.
    auto seq_info = [&](int ctx_raw, bool takes_part, int& full, int& key, int& ctx) __attribute__((always_inline)) {
        ctx = clamp_context(ctx_raw, p);
        const int r = ctx % P;
        full = takes_part ? ctx / P : 0;
        key = !takes_part ? -1 : r > 0 ? 1 + ((r - 1) * kBuckets) / P : (ctx == 0 ? 0 : -1);
    };
    auto mem_info = [&](int s, int& full, int& key, int& ctx) __attribute__((always_inline)) {
        const bool takes = !mixed || p.query_start_loc[s + 1] - p.query_start_loc[s] == 1;
        seq_info(p.context_lens[s], takes, full, key, ctx);
    };
    int fv[NC], kv[NC], cv[NC];
    if (fast) {
        const int32_t* qsl = mixed ? p.query_start_loc : p.context_lens;  // any valid address if not mixed
        int cl[NC], q0[NC], q1[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int s = min(64 * k + lane, p.num_seqs - 1);
            cl[k] = p.context_lens[s];
            q0[k] = qsl[s];
            q1[k] = qsl[mixed ? s + 1 : s];
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const bool takes = 64 * k + lane < p.num_seqs && (!mixed || q1[k] - q0[k] == 1);
            seq_info(cl[k], takes, fv[k], kv[k], cv[k]);
        }
    }
    // Sum over sequences of f(full, key).
    auto count = [&](auto f) __attribute__((always_inline)) {
        int c = 0;
        if (fast) {
#pragma unroll
            for (int k = 0; k < NC; ++k) c += f(fv[k], kv[k]);
        } else {
            for (int s = lane; s < p.num_seqs; s += 64) {
                int full, key, ctx;
                mem_info(s, full, key, ctx);
                c += f(full, key);
            }
        }
        return __builtin_amdgcn_readfirstlane(wave_sum_int(c));
    };
    // The r-th sequence (in order) for which pred(full, key) holds; its full count and context in
    // full_out and ctx_out.
    auto nth = [&](int r, auto pred, int& s_found, int& full_out) __attribute__((always_inline)) -> bool {
        for (int base = 0; base < p.num_seqs; base += 64) {
            const int s = base + lane;
            int full = 0, key = -1, ctx = 0;
            if (fast) {
#pragma unroll
                for (int k = 0; k < NC; ++k)
                    if ((base >> 6) == k) {
                        full = fv[k];
                        key = kv[k];
                        ctx = cv[k];
                    }
            } else if (s < p.num_seqs) {
                mem_info(s, full, key, ctx);
            }
            const bool has = s < p.num_seqs && pred(full, key);
            const uint64_t mask = __builtin_amdgcn_ballot_w64(has);
            const int cnt = __builtin_popcountll(mask);
            if (r < cnt) {
                const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                const uint64_t hit = __builtin_amdgcn_ballot_w64(has && below == r);
                const int lh = __builtin_ctzll(hit);
                s_found = base + lh;
                full_out = __builtin_amdgcn_readlane(full, lh);
                ctx_out = __builtin_amdgcn_readlane(ctx, lh);
                return true;
            }
            r -= cnt;
        }
        return false;
    };
    int full_of_s = 0;
    const int F = count([&](int full, int) { return min(full, p.max_parts); });
    if (w < F) {
        int lo = 0, hi = p.max_parts;  // C(lo) <= w < C(hi)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (count([&](int full, int) { return min(full, mid); }) <= w) lo = mid;
            else hi = mid;
        }
        const int r = w - count([&](int full, int) { return min(full, lo); });
        part_out = lo;
        return nth(r, [&](int full, int) { return full > lo; }, s_out, full_of_s);
    }
    int r = w - F;
    for (int key = kBuckets; key >= 0; --key) {
        const int c = count([&](int, int k) { return k == key ? 1 : 0; });
        if (r < c) {
            if (!nth(r, [&](int, int k) { return k == key; }, s_out, full_of_s)) return false;
            part_out = full_of_s;
            return true;
        }
        r -= c;
    }
    return false;
}

// Merge n >= 1 partials (m_i, l_i, acc_i) of one (sequence, head) row, computed by one wave:
//     out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i,   M = max_i m_i
// (m in the log2 domain; acc_i unnormalised, sharing m_i's reference). Partial i's (m, l) pair is at
// ml + i * ml_stride and its D accumulators at acc + i * acc_stride. The weights 2^(m_i - M) / L are
// computed once, lane i % 64 holding partial i's, and broadcast with v_readlane; the accumulators of
// 16 partials are loaded per unrolled step so that many loads are in flight.
template <bool BF16, int D>
__device__ __forceinline__ void merge_partials(const float* ml, int64_t ml_stride, const float* acc,
                                               int64_t acc_stride, int n, uint16_t* out) {
    constexpr int DPL = D / 64;            // output values per lane
    constexpr int U = 16;                  // partials per unrolled step
    constexpr int P = D >= 512 ? 4 : 8;    // partials loaded before their weights are known
    const int lane = threadIdx.x & 63;
    const float* ap = acc + lane * DPL;
    // The first P partials' accumulators go out with the (m, l) loads, so that the common case (at
    // most P partials) waits for memory once. Indexes past n - 1 load the last partial again; their
    // weight is 0.
    float v0[P][DPL];
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const int jj = min(u, n - 1);
#pragma unroll
        for (int k = 0; k < DPL; ++k) v0[u][k] = ap[jj * acc_stride + k];
    }
    float mi = kNegInf, li = 0.f;
    if (lane < n) {
        mi = ml[lane * ml_stride];
        li = ml[lane * ml_stride + 1];
    }
    float M = mi;
    for (int i = lane + 64; i < n; i += 64) M = fmaxf(M, ml[i * ml_stride]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = lane < n ? fast_exp2(mi - M) * li : 0.f;
    for (int i = lane + 64; i < n; i += 64) L += fast_exp2(ml[i * ml_stride] - M) * ml[i * ml_stride + 1];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    const float invL = L > 0.f ? 1.f / L : 0.f;
    const float w0 = lane < n ? fast_exp2(mi - M) * invL : 0.f;  // partial `lane`'s weight
    float a[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) a[k] = 0.f;
#pragma unroll
    for (int u = 0; u < P; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w0), u));
#pragma unroll
        for (int k = 0; k < DPL; ++k) a[k] = fmaf(w, v0[u][k], a[k]);
    }
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        const float wl = base == 0 ? w0 : (i < n ? fast_exp2(ml[i * ml_stride] - M) * invL : 0.f);
        const int cnt = min(64, n - base);
        // Full steps of U partials, then steps of 4; indexes past cnt - 1 load a valid duplicate
        // whose weight is 0.
        auto step = [&](auto width, int j0) {
            constexpr int C = decltype(width)::value;
            float v[C][DPL];
#pragma unroll
            for (int u = 0; u < C; ++u) {
                const int jj = min(j0 + u, cnt - 1);
#pragma unroll
                for (int k = 0; k < DPL; ++k) v[u][k] = ap[(base + jj) * acc_stride + k];
            }
#pragma unroll
            for (int u = 0; u < C; ++u) {
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0 + u));
#pragma unroll
                for (int k = 0; k < DPL; ++k) a[k] = fmaf(w, v[u][k], a[k]);
            }
        };
        int j0 = base == 0 ? P : 0;  // the first P partials are already in
        for (; j0 + U <= cnt; j0 += U) step(std::integral_constant<int, U>{}, j0);
        for (; j0 < cnt; j0 += 4) step(std::integral_constant<int, 4>{}, j0);
    }
    uint16_t* o = out + lane * DPL;
    if constexpr (DPL == 1) {
        o[0] = (uint16_t)(pack2<BF16>(a[0], 0.f) & 0xFFFFu);
    } else if constexpr (DPL == 2) {
        *reinterpret_cast<uint32_t*>(o) = pack2<BF16>(a[0], a[1]);
    } else if constexpr (DPL == 4) {
        *reinterpret_cast<uint2*>(o) = make_uint2(pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]));
    } else {
        *reinterpret_cast<uint4*>(o) = make_uint4(pack2<BF16>(a[0], a[1]), pack2<BF16>(a[2], a[3]),
                                                  pack2<BF16>(a[4], a[5]), pack2<BF16>(a[6], a[7]));
    }
}

}  // namespace pa

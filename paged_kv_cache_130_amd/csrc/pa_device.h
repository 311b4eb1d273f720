// Device helpers for gfx950 (CDNA4, wave64): DPP row reductions, packed dot products,
// 16-bit <-> fp32 conversions. Included only by .hip kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within each 8-lane half row
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within each 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 4, 8, 16, 32, 64); every lane of a group gets the group
// sum. Within a 16-lane DPP row a butterfly of quad permutes and mirrors covers all lanes; wider
// groups add cross-row shuffles.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group width");
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    if constexpr (N >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp_mov<kDppRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
    return x;
}

// Integer sum over the 64 lanes of the wave (exact; every lane gets the sum).
__device__ __forceinline__ int wave_sum_int(int x) {
    x += __builtin_amdgcn_mov_dpp(x, kDppQuadXor1, 0xF, 0xF, true);
    x += __builtin_amdgcn_mov_dpp(x, kDppQuadXor2, 0xF, 0xF, true);
    x += __builtin_amdgcn_mov_dpp(x, kDppRowHalfMirror, 0xF, 0xF, true);
    x += __builtin_amdgcn_mov_dpp(x, kDppRowMirror, 0xF, 0xF, true);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one position in each 16-lane row), every lane
// of the four getting it. gfx950's row swaps do it on the VALU without an LDS round trip: with both
// operands x, v_permlane16_swap returns rows (0, 0, 2, 2) of x in one result and rows (1, 1, 3, 3)
// in the other, and v_permlane32_swap returns halves (0, 0) and (1, 1).
__device__ __forceinline__ float row_max4(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const uint32_t v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2-element dot product with fp32 accumulation (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <bool BF16>
__device__ __forceinline__ float dot2acc(uint32_t a, uint32_t b, float c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                               false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
    }
}

// Low / high 16-bit value of a packed pair to fp32.
template <bool BF16>
__device__ __forceinline__ float lo_f32(uint32_t w) {
    if constexpr (BF16) return __uint_as_float(w << 16);
    else return (float)__builtin_bit_cast(f16x2, w).x;
}
template <bool BF16>
__device__ __forceinline__ float hi_f32(uint32_t w) {
    if constexpr (BF16) return __uint_as_float(w & 0xFFFF0000u);
    else return (float)__builtin_bit_cast(f16x2, w).y;
}

// Two fp32 values to a packed 16-bit pair, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    if constexpr (BF16) {
        bf16x2 r;
        r.x = (__bf16)a;
        r.y = (__bf16)b;
        return __builtin_bit_cast(uint32_t, r);
    } else {
        f16x2 r;
        r.x = (_Float16)a;
        r.y = (_Float16)b;
        return __builtin_bit_cast(uint32_t, r);
    }
}

// Probability pairs as 16-bit operands of the PV product. For fp16 one packed pair carries 11
// significant bits, enough for the 2e-3 absolute tolerance. For bf16 one pair carries only 8, and a
// weight rounded by 2^-9 of itself can move a short row's output by more than that. So bf16 pairs
// come as hi + lo: hi = bf16(p), lo = bf16(p - hi), which holds p to about 2^-17. The caller
// accumulates both into the same fp32 sum.
template <bool BF16>
__device__ __forceinline__ void pack2_split(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack2<BF16>(a, b);
    if constexpr (BF16) lo = pack2<true>(a - lo_f32<true>(hi), b - hi_f32<true>(hi));
    else lo = 0u;
}

// Work-group index -> linear index such that consecutive linear indices run on the same XCD.
// Work-groups are dispatched round-robin over the 8 XCDs of an MI355X, so group b lands on
// XCD b % 8; giving each XCD a contiguous chunk keeps related work (same KV head) in one L2.
__device__ __forceinline__ int xcd_linear_block(int b, int grid) {
    const int per_xcd = grid >> 3;  // grid is a multiple of 8
    return (b & 7) * per_xcd + (b >> 3);
}

}  // namespace pa

// Matrix-core helpers shared by the MFMA decode and prefill kernels (gfx950).
//
// Operand conventions (16x16 MFMA tiles, wave64): the A operand's row is lane % 16, the B operand's
// column is lane % 16, and the output element D[4*(lane/16) + j][lane % 16] is register j of the lane.
// The k slots a lane holds (8 for the k=32 forms, 4 for the k=16 forms) are filled identically for A and
// B here, so the order the instruction reduces them in does not matter.
#pragma once

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                      0, 0, 0);
}

template <bool BF16>
__device__ __forceinline__ f32x4_t mfma_k16(uint2 a, uint2 b, f32x4_t c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                         c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c,
                                                     0, 0, 0);
}

constexpr int kD = 128;

// Token (row of a 16-token tile) whose K feeds A-row m of the score product S^T = K . Q^T. With
// sigma(m) = m/4 + 4*(m%4), output register j of lane group g (= lane/16) holds token g + 4j: exactly
// the V row that lane group loads for k-slot j of the PV product, so the probabilities are the PV
// A operand as they come out of the softmax.
__device__ __forceinline__ int sigma(int m) { return (m >> 2) + 4 * (m & 3); }

// B operand of the PV product for dim offset e (0..7): the 16-bit values of dim 8c + e of the four V
// rows a lane holds (rows g4, g4+4, g4+8, g4+12 of the tile), packed in k-slot order.
__device__ __forceinline__ uint2 v_operand(const uint4 (&vv)[4], int e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w0, w1, w2, w3;
    switch (e >> 1) {
        case 0: w0 = vv[0].x; w1 = vv[1].x; w2 = vv[2].x; w3 = vv[3].x; break;
        case 1: w0 = vv[0].y; w1 = vv[1].y; w2 = vv[2].y; w3 = vv[3].y; break;
        case 2: w0 = vv[0].z; w1 = vv[1].z; w2 = vv[2].z; w3 = vv[3].z; break;
        default: w0 = vv[0].w; w1 = vv[1].w; w2 = vv[2].w; w3 = vv[3].w; break;
    }
    return make_uint2(__builtin_amdgcn_perm(w1, w0, sel), __builtin_amdgcn_perm(w3, w2, sel));
}

}  // namespace pa

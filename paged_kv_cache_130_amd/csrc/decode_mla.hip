// MLA latent decode: the launches of decode_mla_kernel (decode_mla.h) and the merge of the partials.
// This file is compiled with -mllvm -amdgpu-mfma-vgpr-form (the MFMA accumulators in ordinary vector
// registers), which lets two waves of the decode kernel fit per SIMD.

#include "decode_mla.h"

namespace pa {

// Merge of the n >= 1 partials of one (sequence, head) row by one wave. Partial i holds its output
// a_i = O_i / l_i (bf16, 512 values at acc + i * acc_stride) and (m_i, l_i) at ml + i * ml_stride
// (m in the log2 domain). The row is
//     out = sum_i w_i a_i,   w_i = 2^(m_i - M) l_i / sum_k 2^(m_k - M) l_k,   M = max_i m_i,
// the same softmax as one pass over the whole context. Lane i % 64 computes partial i's weight; lane
// j holds output values 8j .. 8j + 7 and reads them from each partial as one 16-byte load, four
// partials per step.
__device__ __forceinline__ void mla_merge_row(const float* ml, int64_t ml_stride, const uint16_t* acc,
                                              int64_t acc_stride, int n, uint16_t* out) {
    const int lane = threadIdx.x & 63;
    float M = kNegInf;
    for (int i = lane; i < n; i += 64) M = fmaxf(M, ml[i * ml_stride]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    for (int i = lane; i < n; i += 64) L += fast_exp2(ml[i * ml_stride] - M) * ml[i * ml_stride + 1];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    const float invL = L > 0.f ? 1.f / L : 0.f;
    const uint16_t* ap = acc + 8 * lane;
    float a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = 0.f;
    for (int base = 0; base < n; base += 64) {
        const int i = base + lane;
        // Lanes past the last partial weigh 0, so the steps below may load a duplicate there.
        const float wl = i < n ? fast_exp2(ml[i * ml_stride] - M) * ml[i * ml_stride + 1] * invL : 0.f;
        const int cnt = min(64, n - base);
        for (int j0 = 0; j0 < cnt; j0 += 4) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = *reinterpret_cast<const uint4*>(ap + (int64_t)(base + min(j0 + u, cnt - 1)) * acc_stride);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), j0 + u));
                const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    a[2 * k] = fmaf(w, lo_f32<true>(d[k]), a[2 * k]);
                    a[2 * k + 1] = fmaf(w, hi_f32<true>(d[k]), a[2 * k + 1]);
                }
            }
        }
    }
    *reinterpret_cast<uint4*>(out + 8 * lane) = make_uint4(pack2<true>(a[0], a[1]), pack2<true>(a[2], a[3]),
                                                           pack2<true>(a[4], a[5]), pack2<true>(a[6], a[7]));
}

// One wave per (sequence, query head): merge the sequence's partials, or write the zero output of
// an empty context.
__global__ __launch_bounds__(256) void mla_merge_kernel(MlaDecodeParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;  // = s * Hq + head
    if (item >= p.num_seqs * p.num_q_heads) return;
    const int s = item / p.num_q_heads;
    const int head = item - s * p.num_q_heads;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + (size_t)item * 512;
    if (__builtin_amdgcn_readfirstlane(mla_ctx(s, p)) == 0) {
        *reinterpret_cast<uint4*>(out + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);
        return;
    }
    const int first = __builtin_amdgcn_readfirstlane(p.seq_meta[2 * s]);
    const int last = __builtin_amdgcn_readfirstlane(p.seq_meta[2 * s + 1]);
    if (last <= first) return;  // one segment: written by the decode kernel
    const size_t idx = (size_t)(s + first) * p.num_q_heads + head;
    mla_merge_row(p.part_ml + idx * 2, (int64_t)p.num_q_heads * 2, p.part_acc + idx * 512,
                  (int64_t)p.num_q_heads * 512, last - first + 1, out);
}

namespace {

template <int NW>
hipError_t launch_mla_typed(const MlaDecodeParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)p.num_wgs, (unsigned)(p.num_q_heads / p.heads_per_wg));
    if (p.slots != nullptr)
        hipLaunchKernelGGL((decode_mla_kernel<NW, true>), grid, dim3(64 * NW), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_mla_kernel<NW, false>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mla(const MlaDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    hipError_t e;
    switch (p.heads_per_wg) {
        case 64: e = launch_mla_typed<8>(p, stream); break;
        case 32: e = launch_mla_typed<4>(p, stream); break;
        case 16: e = launch_mla_typed<2>(p, stream); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    const int64_t items = (int64_t)p.num_seqs * p.num_q_heads;
    hipLaunchKernelGGL(mla_merge_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa

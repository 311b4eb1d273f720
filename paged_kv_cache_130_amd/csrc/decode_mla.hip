// MLA latent decode: the launches of decode_mla_kernel (decode_mla.h) and the merge of the partials.
// This file is compiled with -mllvm -amdgpu-mfma-vgpr-form (the MFMA accumulators in ordinary vector
// registers), which lets two waves of the decode kernel fit per SIMD.

#include "decode_mla.h"

namespace pa {

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
    merge_partials<true, 512>(p.part_ml + idx * 2, (int64_t)p.num_q_heads * 2, p.part_acc + idx * 512,
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

// Paged decode for grouped-query attention on the matrix cores: the kernel and its launch. The
// per-wave work (the mapping and the math) is in decode_mfma.h.

#include "decode_mfma.h"

namespace pa {

template <bool BF16, bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(FP8 ? 3 : 1))) void decode_mfma_kernel(DenseDecodeParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    decode_mfma_wave<BF16, FP8>(p, blockIdx.x * 4 + wave);
}

hipError_t launch_decode_mfma(const DenseDecodeParams& p, hipStream_t stream) {
    if (p.num_seqs <= 0) return hipSuccess;
    const int64_t items = (int64_t)p.num_kv_heads * p.num_seqs * p.max_parts;
    int64_t wgs = (items + 3) / 4;
    if (p.kv_fp8)
        hipLaunchKernelGGL((decode_mfma_kernel<true, true>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    else if (p.is_bf16)
        hipLaunchKernelGGL((decode_mfma_kernel<true, false>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<false, false>), dim3((unsigned)wgs), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.max_parts <= 1) return e;
    return launch_decode_reduce(p, stream);
}

}  // namespace pa

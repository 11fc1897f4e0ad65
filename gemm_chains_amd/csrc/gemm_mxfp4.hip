// Skinny split-K GEMM kernels with MXFP4 weights and e4m3 operands: partial-sum, store and fused-QKV
// epilogues (one translation unit per few instantiations so the build runs in parallel).
#include "gemm_kernel.hpp"

namespace frt {
template hipError_t launch_gemm_epi<FRT_MXFP4, kGemmPartial>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_MXFP4, kGemmStore>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_MXFP4, kGemmQkv>(const GemmParams&, const GemmShape&, hipStream_t);
}  // namespace frt

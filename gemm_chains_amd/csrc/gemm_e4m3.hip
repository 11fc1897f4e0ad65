// Skinny split-K GEMM kernels with e4m3 weights and operands: partial-sum, store and fused-QKV
// epilogues (one translation unit per few instantiations so the build runs in parallel).
#include "gemm_kernel.hpp"

namespace frt {
template hipError_t launch_gemm_epi<FRT_E4M3, kGemmPartial>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_E4M3, kGemmStore>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_E4M3, kGemmQkv>(const GemmParams&, const GemmShape&, hipStream_t);
}  // namespace frt

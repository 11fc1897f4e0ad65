// Skinny split-K GEMM kernels with bf16 weights and operands: partial-sum, store and fused-QKV
// epilogues (one translation unit per few instantiations so the build runs in parallel).
#include "gemm_kernel.hpp"

namespace frt {
template hipError_t launch_gemm_epi<FRT_BF16, kGemmPartial>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_BF16, kGemmStore>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_BF16, kGemmQkv>(const GemmParams&, const GemmShape&, hipStream_t);
}  // namespace frt

// Skinny split-K GEMM kernels with MXFP4 weights and e4m3 operands: SiLU-gate epilogues with a bf16
// or e4m3 output operand.
#include "gemm_kernel.hpp"

namespace frt {
template hipError_t launch_gemm_epi<FRT_MXFP4, kGemmSiluBf16>(const GemmParams&, const GemmShape&, hipStream_t);
template hipError_t launch_gemm_epi<FRT_MXFP4, kGemmSiluE4m3>(const GemmParams&, const GemmShape&, hipStream_t);
}  // namespace frt

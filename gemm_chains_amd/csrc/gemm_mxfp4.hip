// Skinny split-K GEMM kernels with MXFP4 weights and e4m3 operands (one translation unit
// per weight format so the instantiations compile in parallel).
#include "gemm_kernel.hpp"

namespace frt {
template hipError_t launch_gemm_typed<FRT_MXFP4>(const GemmParams& p, const GemmShape& sh, hipStream_t s);
}  // namespace frt

// Skinny split-K GEMM kernels with e4m3 operands (one translation unit per operand type
// so the instantiations compile in parallel).
#include "gemm_kernel.hpp"

namespace frt {
template hipError_t launch_gemm_typed<FRT_E4M3>(const GemmParams& p, const GemmShape& sh, hipStream_t s);
}  // namespace frt

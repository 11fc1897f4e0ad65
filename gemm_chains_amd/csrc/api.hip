// Diagnostics of the C ABI: status strings, the per-thread HIP error, the version.
#include "frt_internal.hpp"

namespace frt {
static thread_local int g_last_hip_error = 0;
void set_hip_error(int e) { g_last_hip_error = e; }
}  // namespace frt

extern "C" const char* frt_status_string(int status) {
  switch (status) {
    case FRT_OK: return "ok";
    case FRT_E_NULL: return "a required pointer is NULL";
    case FRT_E_SHAPE: return "a size is out of range or not a supported multiple";
    case FRT_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case FRT_E_DTYPE: return "unsupported dtype";
    case FRT_E_SPLITK: return "split count not supported or K not divisible";
    case FRT_E_WORKSPACE: return "workspace or arena too small";
    case FRT_E_ALIAS: return "an output overlaps an input";
    case FRT_E_STATE: return "invalid handle or buffer name";
    case FRT_E_HIP: return "a HIP runtime call failed";
    case FRT_E_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

extern "C" int frt_last_hip_error(void) { return frt::g_last_hip_error; }

extern "C" int frt_version(void) { return 100; }

// An empty kernel: what a dependent launch costs before any work.  Each workgroup writes
// nothing; one lane of workgroup 0 stores its id to `sink` only when `flag` is set (never
// by the diagnostic below), so the compiler keeps the kernel's body and dispatch.
__global__ void empty_kernel(unsigned* sink, int flag) {
  if (flag && blockIdx.x == 0 && threadIdx.x == 0) sink[0] = blockIdx.x;
}

extern "C" int frt_diag_empty_kernels(void* stream, int n, int workgroups) {
  FRT_CHECK(n >= 0 && n <= 100000, FRT_E_ARG);
  FRT_CHECK(workgroups >= 1 && workgroups <= 65536, FRT_E_ARG);
  for (int i = 0; i < n; ++i) {
    hipLaunchKernelGGL(empty_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, (unsigned*)nullptr, 0);
  }
  FRT_HIP(hipGetLastError());
  return FRT_OK;
}

// fa_kernel.h -- internal interface between the C-ABI shim and the kernel TU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa06 {
// Enqueue the forward kernel for BH = B*H independent heads (causal: key j
// hidden from query i when j > i + Nk - Nq).  Arguments are already validated
// by the caller.  Returns 0 or the hipError_t of the launch.
int launch_fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int64_t BH, int64_t Nq, int64_t Nk, float scale, bool causal, hipStream_t stream);
const char* kernel_config_string();
}  // namespace fa06

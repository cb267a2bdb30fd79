// stub_launch.cpp -- host-only stand-ins for the kernel launchers, so the
// C-ABI shim (fa_api.cpp) links without any GPU code for the sanitizer
// build.  Every launcher reports a failed launch; none runs anything.
#include <hip/hip_runtime.h>

#include "fa_kernel.h"

namespace fa06 {
int launch_fa_fwd(const LaunchArgs&, hipStream_t) { return 1; }
int noalloc_scratch(void**) { return 1; }
const char* kernel_config_string() { return "host stub"; }
int launch_fa_bwd(const BwdArgs&, hipStream_t) { return 1; }
const char* bwd_config_string() { return "host stub"; }
int launch_fa_fwd_mxfp8(const MxArgs&, hipStream_t) { return 1; }
int launch_mx_quantize_rows(const void*, void*, void*, int64_t, int64_t, int64_t, hipStream_t) { return 1; }
int launch_mx_quantize_vt(const void*, void*, void*, int64_t, int64_t, int64_t, hipStream_t) { return 1; }
const char* mxfp8_config_string() { return "host stub"; }
}  // namespace fa06

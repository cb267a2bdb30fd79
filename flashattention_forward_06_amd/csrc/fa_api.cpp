// fa_api.cpp -- C ABI of the fused attention forward pass: argument
// validation, device check and launch.  Declarations and the contract are in
// include/fa06.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa06.h"
#include "fa_kernel.h"

namespace {

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (na <= 0 || nb <= 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_DEVICE;
  int s = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? FA_OK : FA_ERR_DEVICE;
}

}  // namespace

namespace {

int validate_and_launch(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                        int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, const float* bias,
                        void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 1) return FA_ERR_INVALID_SHAPE;
  if (d != FA_HEAD_DIM) return FA_ERR_UNSUPPORTED;
  if (Nq > FA_MAX_SEQ || Nk > FA_MAX_SEQ) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (bias != nullptr) return FA_ERR_UNSUPPORTED;  // additive bias: not in this build
  // sizes: B*H*N*d*2 bytes must fit in int64 (N <= 2^23, d*2 = 2^8)
  if (B > 0 && H > INT64_MAX / B) return FA_ERR_INVALID_SHAPE;
  const int64_t BH = B * H;
  const int64_t row_bytes = FA_HEAD_DIM * 2;
  if (BH > (INT64_MAX / row_bytes) / FA_MAX_SEQ) return FA_ERR_INVALID_SHAPE;
  // a pointer may be NULL only when its buffer is empty
  if ((BH * Nq > 0 && (!Q || !O || !LSE)) || (BH > 0 && (!K || !V))) return FA_ERR_NULL_POINTER;
  // one workgroup per 128 query rows of a head; the grid has < 2^31 workgroups
  if (BH * ((Nq + 127) / 128) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_SCALE;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t q_bytes = BH * Nq * row_bytes, kv_bytes = BH * Nk * row_bytes, l_bytes = BH * Nq * 4;
  if (overlaps(O, q_bytes, Q, q_bytes) || overlaps(O, q_bytes, K, kv_bytes) || overlaps(O, q_bytes, V, kv_bytes) ||
      overlaps(LSE, l_bytes, Q, q_bytes) || overlaps(LSE, l_bytes, K, kv_bytes) ||
      overlaps(LSE, l_bytes, V, kv_bytes) || overlaps(LSE, l_bytes, O, q_bytes))
    return FA_ERR_ALIAS;
  if (BH * Nq == 0) return FA_OK;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  if (fa06::launch_fa_fwd(Q, K, V, O, LSE, BH, Nq, Nk, scale, causal == 1, static_cast<hipStream_t>(stream)) != 0)
    return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      float scale, void* stream) {
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, 0, nullptr, stream);
}

extern "C" int fa_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                             int causal, const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                             int64_t bias_stride_q, void* stream) {
  (void)bias_stride_b;
  (void)bias_stride_h;
  (void)bias_stride_q;
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, scale, causal, bias, stream);
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a pointer to a non-empty buffer is NULL";
    case FA_ERR_INVALID_SHAPE: return "FA_ERR_INVALID_SHAPE: B, H, Nq must be >= 0, Nk >= 1, and sizes must fit";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: d must be 128, N <= 2^23, pointers 16-byte aligned (LSE 4)";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: O or LSE overlaps Q, K, V or each other";
    case FA_ERR_INVALID_SCALE: return "FA_ERR_INVALID_SCALE: scale must be finite";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE: no HIP device, or the current device is not gfx950";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    default: return "unknown fa_status";
  }
}

extern "C" const char* fa_build_info(void) { return fa06::kernel_config_string(); }

// fa_kernel.h -- internal interface between the C-ABI shim and the kernel TU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa06 {

// One forward call over BH = B*H independent heads, already validated.
struct LaunchArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int64_t BH, H, Nq, Nk;
  int64_t d;            // head size of Q and K
  int64_t dv;           // head size of V and O; (d, dv) in (64, 64), (128, 128), (256, 256), (192, 128)
  float scale;
  bool causal;          // key j hidden from query i when j > i + Nk - Nq
  const float* bias;    // NULL, or fp32 bias[b*bias_sb + h*bias_sh + i*bias_sq + j]
  int64_t bias_sb, bias_sh, bias_sq;
  // key split (n_splits > 1): ranges of split_keys keys (a multiple of 64),
  // partial outputs Opart fp32 [n_splits, BH, Nq, dv] and Lpart fp32
  // [n_splits, BH, Nq], merged into O and LSE by a second kernel
  int n_splits;
  int split_keys;
  float* Opart;
  float* Lpart;
};

// Enqueues the kernel; returns 0 or the hipError_t of the launch.
int launch_fa_fwd(const LaunchArgs& args, hipStream_t stream);

// Size of the per-device scratch array that fa_fwd_splitkv_noalloc uses in
// place of a caller workspace (the key ranges' fp32 partial outputs and
// log-sum-exps).
constexpr int64_t kNoAllocScratchBytes = int64_t(48) << 20;
// Device address of that array on the current device (looked up once per
// device, then cached); returns 0, or non-zero if the lookup failed.
int noalloc_scratch(void** ptr);
const char* kernel_config_string();

// One backward call over BH = B*H heads, already validated.
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  void* dQ;
  void* dK;
  void* dV;
  float* Dws;           // [BH, Nq] fp32: receives D_i = dO_i . O_i
  int64_t BH, Nq, Nk;
  int64_t d, dv;        // head sizes: (64, 64), (128, 128) or (192, 128)
  float scale;
  bool causal;
  int64_t H;
  const float* bias;    // NULL, or the forward's fp32 bias (same strides)
  int64_t bias_sb, bias_sh, bias_sq;
};

// Enqueues the three backward kernels; returns 0 or non-zero if a launch failed.
int launch_fa_bwd(const BwdArgs& args, hipStream_t stream);
const char* bwd_config_string();

// One MXFP8 forward call (head size 128), already validated.
struct MxArgs {
  const void* Q8;   // [BH, Nq, 128] E4M3
  const void* Qs;   // [BH, Nq, 4] E8M0
  const void* K8;   // [BH, Nk, 128] E4M3
  const void* Ks;   // [BH, ldv, 4] E8M0 (rows >= Nk unused)
  const void* Vt8;  // [BH, 128, ldv] E4M3, keys >= Nk zero
  const void* Vs;   // [BH, ldv/32, 128] E8M0
  void* O;          // [BH, Nq, 128] bf16
  float* LSE;       // [BH, Nq]
  int64_t BH, Nq, Nk, ldv;
  float scale;
  bool causal;
};
int launch_fa_fwd_mxfp8(const MxArgs& args, hipStream_t stream);
int launch_mx_quantize_rows(const void* X, void* E, void* S, int64_t BH, int64_t N, int64_t ldS, hipStream_t stream);
int launch_mx_quantize_vt(const void* V, void* Vt, void* Vs, int64_t BH, int64_t Nk, int64_t ldv, hipStream_t stream);
const char* mxfp8_config_string();

}  // namespace fa06

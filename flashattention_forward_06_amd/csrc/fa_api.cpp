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

// Longest sequence for head size d: one (batch, head) slice of N rows of 2d
// bytes stays within 2^31 bytes (32-bit buffer offsets), and N <= 2^23.
int64_t max_seq(int64_t d) { return (int64_t(1) << 30) / d < FA_MAX_SEQ ? (int64_t(1) << 30) / d : FA_MAX_SEQ; }

}  // namespace

namespace {

// Largest per-wave bias extent, in elements: 31 row strides + one row + a
// tile of slack must stay below 2^29 so every byte offset fits 31 bits.
constexpr int64_t kBiasWaveSpan = int64_t(1) << 29;
// Largest bias extent over all (b, h, i, j), in elements.
constexpr int64_t kBiasMaxExtent = int64_t(1) << 60;

// (d, dv) pairs with a kernel: equal head sizes 64, 128, 256, and the split
// 192 / 128 of multi-head latent attention's prefill.
bool head_sizes_supported(int64_t d, int64_t dv) {
  return (d == dv && (d == 64 || d == 128 || d == 256)) || (d == 192 && dv == 128);
}

// Key split of a launch: n_splits ranges of split_keys keys (a multiple of 64,
// so a range starts on a tile of every kernel variant).  requested = 0 picks
// enough ranges for the grid to hold at least kSplitTargetWGs workgroups
// (two per CU), keeping every range at least kSplitMinKeys long; a request
// above the key count is cut to one range per 64 keys.
constexpr int64_t kSplitTargetWGs = 512;
constexpr int64_t kSplitMinKeys = 512;
constexpr int64_t kSplitMax = 1024;

struct SplitPlan {
  int64_t n_splits;
  int64_t split_keys;
};

SplitPlan plan_split(int64_t BH, int64_t Nq, int64_t Nk, int64_t requested) {
  int64_t s = requested;
  if (s == 0) {
    const int64_t nblk = BH * ((Nq + 127) / 128);
    s = nblk >= kSplitTargetWGs || nblk == 0 ? 1 : (kSplitTargetWGs + nblk - 1) / nblk;
    const int64_t cap = Nk / kSplitMinKeys;
    s = s < cap ? s : (cap > 1 ? cap : 1);
  }
  const int64_t tiles = (Nk + 63) / 64;
  s = s < tiles ? s : tiles;
  const int64_t keys = ((Nk + s - 1) / s + 63) / 64 * 64;
  return SplitPlan{(Nk + keys - 1) / keys, keys};
}

int64_t split_workspace_bytes(const SplitPlan& p, int64_t BH, int64_t Nq, int64_t dv) {
  return p.n_splits > 1 ? p.n_splits * BH * Nq * (dv * 4 + 4) : 0;
}

int validate_and_launch(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                        int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale, int causal,
                        const float* bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq, void* stream,
                        int64_t n_splits = 1, void* workspace = nullptr, int64_t workspace_bytes = 0,
                        bool use_scratch = false) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 1) return FA_ERR_INVALID_SHAPE;
  if (!head_sizes_supported(d, dv)) return FA_ERR_UNSUPPORTED;
  const int64_t dmax = d > dv ? d : dv;
  if (Nq > max_seq(dmax) || Nk > max_seq(dmax)) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  // sizes: B*H*N*d*2 bytes must fit in int64 (N*d*2 <= 2^31)
  if (B > 0 && H > INT64_MAX / B) return FA_ERR_INVALID_SHAPE;
  const int64_t BH = B * H;
  if (BH > (INT64_MAX / (dmax * 2)) / max_seq(dmax)) return FA_ERR_INVALID_SHAPE;
  // bias: non-negative element strides; the extent must be addressable
  int64_t bias_elems = 0;
  if (bias != nullptr) {
    if (bias_sb < 0 || bias_sh < 0 || bias_sq < 0) return FA_ERR_UNSUPPORTED;
    if (BH * Nq > 0) {
      const __int128 ext = (__int128)(B - 1) * bias_sb + (__int128)(H - 1) * bias_sh +
                           (__int128)(Nq - 1) * bias_sq + Nk;
      if (ext > kBiasMaxExtent) return FA_ERR_INVALID_SHAPE;
      bias_elems = (int64_t)ext;
      if ((__int128)31 * bias_sq + Nk + 128 > kBiasWaveSpan) return FA_ERR_UNSUPPORTED;
    }
  }
  // key split: the plan and its size limits
  if (n_splits < 0 || n_splits > kSplitMax) return FA_ERR_UNSUPPORTED;
  const SplitPlan plan = plan_split(BH, Nq, Nk, n_splits);
  if (plan.n_splits > 1) {
    // fp32 partial rows of one (range, head) slice use 32-bit byte offsets;
    // the merge grid (B*H*Nq / 4 blocks at d_v = 256) stays below 2^31
    if (Nq * dv * 4 > INT32_MAX) return FA_ERR_UNSUPPORTED;
    if (BH * Nq > (int64_t(1) << 33) - 4) return FA_ERR_UNSUPPORTED;
    if (BH * ((Nq + 127) / 128) * plan.n_splits > INT32_MAX) return FA_ERR_UNSUPPORTED;
  }
  // a pointer may be NULL only when its buffer is empty
  if ((BH * Nq > 0 && (!Q || !O || !LSE)) || (BH > 0 && (!K || !V))) return FA_ERR_NULL_POINTER;
  // one workgroup per 128 query rows of a head; the grid has < 2^31 workgroups
  if (BH * ((Nq + 127) / 128) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_SCALE;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_UNSUPPORTED;
  // the bias is read 16 bytes (4 keys) at a time: rows start 16-byte aligned
  if (bias != nullptr && (!aligned(bias, 16) || bias_sb % 4 != 0 || bias_sh % 4 != 0 || bias_sq % 4 != 0))
    return FA_ERR_UNSUPPORTED;
  const int64_t q_bytes = BH * Nq * d * 2, k_bytes = BH * Nk * d * 2, v_bytes = BH * Nk * dv * 2;
  const int64_t o_bytes = BH * Nq * dv * 2, l_bytes = BH * Nq * 4;
  const int64_t b_bytes = bias_elems * 4;
  if (overlaps(O, o_bytes, Q, q_bytes) || overlaps(O, o_bytes, K, k_bytes) || overlaps(O, o_bytes, V, v_bytes) ||
      overlaps(LSE, l_bytes, Q, q_bytes) || overlaps(LSE, l_bytes, K, k_bytes) ||
      overlaps(LSE, l_bytes, V, v_bytes) || overlaps(LSE, l_bytes, O, o_bytes) ||
      overlaps(O, o_bytes, bias, b_bytes) || overlaps(LSE, l_bytes, bias, b_bytes))
    return FA_ERR_ALIAS;
  // key split: the caller's workspace
  const int64_t ws_need = split_workspace_bytes(plan, BH, Nq, dv);
  if (use_scratch) {
    // the library's own scratch array stands in for the workspace
    if (ws_need > fa06::kNoAllocScratchBytes) return FA_ERR_SCRATCH;
  } else if (plan.n_splits > 1) {
    if (workspace == nullptr || workspace_bytes < ws_need || !aligned(workspace, 16)) return FA_ERR_WORKSPACE;
    if (overlaps(workspace, ws_need, Q, q_bytes) || overlaps(workspace, ws_need, K, k_bytes) ||
        overlaps(workspace, ws_need, V, v_bytes) || overlaps(workspace, ws_need, O, o_bytes) ||
        overlaps(workspace, ws_need, LSE, l_bytes) || overlaps(workspace, ws_need, bias, b_bytes))
      return FA_ERR_ALIAS;
  }
  if (BH * Nq == 0) return FA_OK;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  if (use_scratch && plan.n_splits > 1 && fa06::noalloc_scratch(&workspace) != 0) return FA_ERR_DEVICE;
  fa06::LaunchArgs a{};
  a.n_splits = (int)plan.n_splits;
  a.split_keys = (int)plan.split_keys;
  if (plan.n_splits > 1) {
    a.Opart = static_cast<float*>(workspace);
    a.Lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.n_splits * BH * Nq * dv * 4);
  }
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.LSE = LSE;
  a.BH = BH;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.dv = dv;
  a.scale = scale;
  a.causal = causal == 1;
  a.bias = bias;
  a.bias_sb = bias_sb;
  a.bias_sh = bias_sh;
  a.bias_sq = bias_sq;
  if (fa06::launch_fa_fwd(a, static_cast<hipStream_t>(stream)) != 0) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      float scale, void* stream) {
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, d, scale, 0, nullptr, 0, 0, 0, stream);
}

extern "C" int fa_fwd_masked(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                             int causal, const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                             int64_t bias_stride_q, void* stream) {
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, d, scale, causal, bias, bias_stride_b,
                             bias_stride_h, bias_stride_q, stream);
}

extern "C" int fa_fwd_dv(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale, int causal, const float* bias,
                         int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_stride_q, void* stream) {
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, dv, scale, causal, bias, bias_stride_b,
                             bias_stride_h, bias_stride_q, stream);
}

extern "C" int64_t fa_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t dv,
                                                  int64_t n_splits, int64_t* n_splits_used) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 1 || dv < 1 || dv > 256) return -FA_ERR_INVALID_SHAPE;
  if (n_splits < 0 || n_splits > kSplitMax) return -FA_ERR_UNSUPPORTED;
  if (Nq > FA_MAX_SEQ || Nk > FA_MAX_SEQ) return -FA_ERR_UNSUPPORTED;
  if (B > 0 && H > INT64_MAX / B) return -FA_ERR_INVALID_SHAPE;
  const int64_t BH = B * H;
  if (BH > (int64_t(1) << 40) / FA_MAX_SEQ) return -FA_ERR_INVALID_SHAPE;
  const SplitPlan p = plan_split(BH, Nq, Nk, n_splits);
  if (n_splits_used != nullptr) *n_splits_used = p.n_splits;
  return split_workspace_bytes(p, BH, Nq, dv);
}

extern "C" int fa_fwd_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
                              int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale, int causal,
                              const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                              int64_t bias_stride_q, int64_t n_splits, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, dv, scale, causal, bias, bias_stride_b,
                             bias_stride_h, bias_stride_q, stream, n_splits, workspace, workspace_bytes);
}

extern "C" int fa_fwd_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int64_t B,
                                      int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale,
                                      int causal, const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                                      int64_t bias_stride_q, int64_t n_splits, void* stream) {
  return validate_and_launch(Q, K, V, O, LSE, B, H, Nq, Nk, d, dv, scale, causal, bias, bias_stride_b,
                             bias_stride_h, bias_stride_q, stream, n_splits, nullptr, 0, true);
}

extern "C" int64_t fa_fwd_splitkv_noalloc_max_bytes(void) { return fa06::kNoAllocScratchBytes; }

namespace {

// (d, dv) pairs with backward kernels.  At head size 256 the dK/dV kernel
// runs once per gradient and the dQ kernel once per half of its columns, so
// that each fits one wave's registers.
bool bwd_head_sizes_supported(int64_t d, int64_t dv) {
  return (d == dv && (d == 64 || d == 128 || d == 256)) || (d == 192 && dv == 128);
}

int bwd_validate_and_launch(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                            const float* LSE, void* dQ, void* dK, void* dV, float* D, int64_t B, int64_t H,
                            int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale, int causal,
                            const float* bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq, void* stream) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 1) return FA_ERR_INVALID_SHAPE;
  if (!bwd_head_sizes_supported(d, dv)) return FA_ERR_UNSUPPORTED;
  const int64_t dmax = d > dv ? d : dv;
  if (Nq > max_seq(dmax) || Nk > max_seq(dmax)) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (B > 0 && H > INT64_MAX / B) return FA_ERR_INVALID_SHAPE;
  const int64_t BH = B * H;
  if (BH > (INT64_MAX / (dmax * 2)) / max_seq(dmax)) return FA_ERR_INVALID_SHAPE;
  // bias: the forward's rules, plus the span of one key column over all
  // query rows (the dK/dV kernel addresses it with 32-bit byte offsets)
  int64_t b_bytes = 0;
  if (bias != nullptr) {
    if (bias_sb < 0 || bias_sh < 0 || bias_sq < 0) return FA_ERR_UNSUPPORTED;
    if (BH * Nq > 0) {
      const __int128 ext = (__int128)(B - 1) * bias_sb + (__int128)(H - 1) * bias_sh +
                           (__int128)(Nq - 1) * bias_sq + Nk;
      if (ext > kBiasMaxExtent) return FA_ERR_INVALID_SHAPE;
      b_bytes = (int64_t)ext * 4;
      if ((__int128)(Nq - 1) * bias_sq + Nk + 128 > kBiasWaveSpan) return FA_ERR_UNSUPPORTED;
    }
  }
  const bool has_q = BH * Nq > 0, has_k = BH > 0;
  if ((has_q && (!Q || !O || !dO || !LSE || !dQ || !D)) || (has_k && (!K || !V || !dK || !dV)))
    return FA_ERR_NULL_POINTER;
  // one workgroup per 128 query rows (dQ) and per 128 keys (dK, dV) of a head
  if (BH * ((Nq + 127) / 128) > INT32_MAX || BH * ((Nk + 127) / 128) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_SCALE;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(dO, 16) ||
      !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) || !aligned(LSE, 4) || !aligned(D, 4))
    return FA_ERR_UNSUPPORTED;
  if (bias != nullptr && (!aligned(bias, 16) || bias_sb % 4 != 0 || bias_sh % 4 != 0 || bias_sq % 4 != 0))
    return FA_ERR_UNSUPPORTED;
  const int64_t q_bytes = BH * Nq * d * 2, k_bytes = BH * Nk * d * 2, v_bytes = BH * Nk * dv * 2;
  const int64_t o_bytes = BH * Nq * dv * 2, l_bytes = BH * Nq * 4;
  struct Buf {
    const void* p;
    int64_t n;
  };
  const Buf ins[] = {{Q, q_bytes}, {K, k_bytes}, {V, v_bytes}, {O, o_bytes}, {dO, o_bytes}, {LSE, l_bytes}};
  const Buf outs[] = {{dQ, q_bytes}, {dK, k_bytes}, {dV, v_bytes}, {D, l_bytes}};
  for (const Buf& o : outs) {
    if (overlaps(o.p, o.n, bias, b_bytes)) return FA_ERR_ALIAS;
    for (const Buf& i : ins)
      if (overlaps(o.p, o.n, i.p, i.n)) return FA_ERR_ALIAS;
    for (const Buf& o2 : outs)
      if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n)) return FA_ERR_ALIAS;
  }
  if (BH == 0) return FA_OK;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  fa06::BwdArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.LSE = LSE;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.Dws = D;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.dv = dv;
  a.scale = scale;
  a.causal = causal == 1;
  a.H = H;
  a.bias = bias;
  a.bias_sb = bias_sb;
  a.bias_sh = bias_sh;
  a.bias_sq = bias_sq;
  if (fa06::launch_fa_bwd(a, static_cast<hipStream_t>(stream)) != 0) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, float* D, int64_t B, int64_t H,
                      int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, void* stream) {
  return bwd_validate_and_launch(Q, K, V, O, dO, LSE, dQ, dK, dV, D, B, H, Nq, Nk, d, d, scale, causal, nullptr, 0,
                                 0, 0, stream);
}

extern "C" int fa_bwd_masked(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                             const float* LSE, void* dQ, void* dK, void* dV, float* D, int64_t B, int64_t H,
                             int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, const float* bias,
                             int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_stride_q, void* stream) {
  return bwd_validate_and_launch(Q, K, V, O, dO, LSE, dQ, dK, dV, D, B, H, Nq, Nk, d, d, scale, causal, bias,
                                 bias_stride_b, bias_stride_h, bias_stride_q, stream);
}

extern "C" int fa_bwd_dv(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                         const float* LSE, void* dQ, void* dK, void* dV, float* D, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale, int causal, const float* bias,
                         int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_stride_q, void* stream) {
  return bwd_validate_and_launch(Q, K, V, O, dO, LSE, dQ, dK, dV, D, B, H, Nq, Nk, d, dv, scale, causal, bias,
                                 bias_stride_b, bias_stride_h, bias_stride_q, stream);
}

// ---------------------------------------------------------------- MXFP8
namespace {
constexpr int64_t kMaxLdv = int64_t(1) << 24;  // 128 rows of V^T stay within 2^31 bytes

int check_mx_shapes(int64_t B, int64_t H, int64_t d) {
  if (B < 0 || H < 0) return FA_ERR_INVALID_SHAPE;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  if (B > 0 && H > INT64_MAX / B) return FA_ERR_INVALID_SHAPE;
  if (B * H > (INT64_MAX / 256) / FA_MAX_SEQ) return FA_ERR_INVALID_SHAPE;
  return FA_OK;
}
}  // namespace

extern "C" int fa_fwd_mxfp8(const void* Q8, const void* Qs, const void* K8, const void* Ks, const void* Vt8,
                            const void* Vs, void* O, float* LSE, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                            int64_t d, int64_t ldv, float scale, int causal, void* stream) {
  int st = check_mx_shapes(B, H, d);
  if (st != FA_OK) return st;
  if (Nq < 0 || Nk < 1) return FA_ERR_INVALID_SHAPE;
  if (Nq > FA_MAX_SEQ || Nk > FA_MAX_SEQ) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (ldv < Nk || ldv % 64 != 0 || ldv > kMaxLdv) return FA_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  if ((BH * Nq > 0 && (!Q8 || !Qs || !O || !LSE)) || (BH > 0 && (!K8 || !Ks || !Vt8 || !Vs)))
    return FA_ERR_NULL_POINTER;
  if (BH * ((Nq + 127) / 128) > INT32_MAX) return FA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_SCALE;
  if (!aligned(Q8, 16) || !aligned(K8, 16) || !aligned(Vt8, 16) || !aligned(Ks, 16) || !aligned(Vs, 16) ||
      !aligned(Qs, 4) || !aligned(O, 16) || !aligned(LSE, 4))
    return FA_ERR_UNSUPPORTED;
  const int64_t o_bytes = BH * Nq * 256, l_bytes = BH * Nq * 4;
  struct Buf {
    const void* p;
    int64_t n;
  };
  const Buf ins[] = {{Q8, BH * Nq * 128}, {Qs, BH * Nq * 4}, {K8, BH * Nk * 128}, {Ks, BH * ldv * 4},
                     {Vt8, BH * 128 * ldv}, {Vs, BH * (ldv / 32) * 128}};
  for (const Buf& i : ins)
    if (overlaps(O, o_bytes, i.p, i.n) || overlaps(LSE, l_bytes, i.p, i.n)) return FA_ERR_ALIAS;
  if (overlaps(O, o_bytes, LSE, l_bytes)) return FA_ERR_ALIAS;
  if (BH * Nq == 0) return FA_OK;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  fa06::MxArgs a{};
  a.Q8 = Q8;
  a.Qs = Qs;
  a.K8 = K8;
  a.Ks = Ks;
  a.Vt8 = Vt8;
  a.Vs = Vs;
  a.O = O;
  a.LSE = LSE;
  a.BH = BH;
  a.Nq = Nq;
  a.Nk = Nk;
  a.ldv = ldv;
  a.scale = scale;
  a.causal = causal == 1;
  if (fa06::launch_fa_fwd_mxfp8(a, static_cast<hipStream_t>(stream)) != 0) return FA_ERR_LAUNCH;
  return FA_OK;
}

extern "C" int fa_mxfp8_quantize_rows(const void* X, void* E, void* S, int64_t B, int64_t H, int64_t N, int64_t d,
                                      int64_t ldS, void* stream) {
  int st = check_mx_shapes(B, H, d);
  if (st != FA_OK) return st;
  if (N < 0 || ldS < N) return FA_ERR_INVALID_SHAPE;
  if (N > FA_MAX_SEQ || ldS > FA_MAX_SEQ) return FA_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  if (BH * N > 0 && (!X || !E || !S)) return FA_ERR_NULL_POINTER;
  if (!aligned(X, 16) || !aligned(E, 16)) return FA_ERR_UNSUPPORTED;
  const int64_t x_bytes = BH * N * 256, e_bytes = BH * N * 128, s_bytes = BH * ldS * 4;
  if (overlaps(E, e_bytes, X, x_bytes) || overlaps(S, s_bytes, X, x_bytes) || overlaps(S, s_bytes, E, e_bytes))
    return FA_ERR_ALIAS;
  if (BH * N == 0) return FA_OK;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  return fa06::launch_mx_quantize_rows(X, E, S, BH, N, ldS, static_cast<hipStream_t>(stream)) == 0 ? FA_OK
                                                                                                 : FA_ERR_LAUNCH;
}

extern "C" int fa_mxfp8_quantize_vt(const void* V, void* Vt, void* Vs, int64_t B, int64_t H, int64_t Nk, int64_t d,
                                    int64_t ldv, void* stream) {
  int st = check_mx_shapes(B, H, d);
  if (st != FA_OK) return st;
  if (Nk < 1) return FA_ERR_INVALID_SHAPE;
  if (Nk > FA_MAX_SEQ) return FA_ERR_UNSUPPORTED;
  if (ldv < Nk || ldv % 64 != 0 || ldv > kMaxLdv) return FA_ERR_UNSUPPORTED;
  const int64_t BH = B * H;
  if (BH > 0 && (!V || !Vt || !Vs)) return FA_ERR_NULL_POINTER;
  if (!aligned(V, 2) || !aligned(Vt, 16)) return FA_ERR_UNSUPPORTED;
  const int64_t v_bytes = BH * Nk * 256, t_bytes = BH * 128 * ldv, s_bytes = BH * (ldv / 32) * 128;
  if (overlaps(Vt, t_bytes, V, v_bytes) || overlaps(Vs, s_bytes, V, v_bytes) || overlaps(Vs, s_bytes, Vt, t_bytes))
    return FA_ERR_ALIAS;
  if (BH == 0) return FA_OK;
  const int dev = check_device();
  if (dev != FA_OK) return dev;
  return fa06::launch_mx_quantize_vt(V, Vt, Vs, BH, Nk, ldv, static_cast<hipStream_t>(stream)) == 0 ? FA_OK
                                                                                                  : FA_ERR_LAUNCH;
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a pointer to a non-empty buffer is NULL";
    case FA_ERR_INVALID_SHAPE: return "FA_ERR_INVALID_SHAPE: B, H, Nq must be >= 0, Nk >= 1, and sizes must fit";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: (d, d_v) must be (64, 64), (128, 128), (256, 256) or (192, 128) "
                                     "(d = 128 for MXFP8), N <= min(2^23, 2^30/d), "
                                     "pointers 16-byte aligned (LSE 4), "
                                     "bias strides non-negative multiples of 4 within the addressable span";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: O or LSE overlaps Q, K, V or each other";
    case FA_ERR_INVALID_SCALE: return "FA_ERR_INVALID_SCALE: scale must be finite";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE: no HIP device, or the current device is not gfx950";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace NULL, smaller than fa_fwd_splitkv_workspace_bytes "
                                  "reports, or not 16-byte aligned";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: fa_fwd_splitkv_noalloc: the key split needs more than the "
                                "library's scratch array holds (fa_fwd_splitkv_noalloc_max_bytes)";
    default: return "unknown fa_status";
  }
}

extern "C" const char* fa_build_info(void) { return fa06::kernel_config_string(); }

extern "C" const char* fa_bwd_build_info(void) { return fa06::bwd_config_string(); }

extern "C" const char* fa_mxfp8_build_info(void) { return fa06::mxfp8_config_string(); }

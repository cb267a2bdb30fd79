// sanitize_driver.cpp -- host-only run of the C-ABI validation path and of
// the fp64 oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (g++ only, no GPU code: the kernel launchers are stubs).
//
// Every entry point of include/fa06.h is called with each kind of argument it
// must reject (the status is checked), and once with valid arguments (then
// the status is FA_ERR_DEVICE without a GPU, or FA_ERR_LAUNCH from the stub
// launcher).  Host buffers stand in for device ones: validation compares
// pointers and never dereferences them.  The oracle's entry points run on
// small inputs, including the degenerate ones (one key, rows that see no key,
// -inf bias, a single head of one row), and their results are checked
// against closed forms: a constant value column gives that constant, and one
// key gives O = v, LSE = scale * q.k.
// Prints "SANITIZE_OK <n checks>" and exits 0 when every check passes; a
// sanitizer report aborts the process with a non-zero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

#include "fa06.h"

extern "C" {
int oracle_attn_fp64(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t, int64_t,
                     int64_t, float, double*, double*);
int oracle_attn_rows_fp64(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                          int64_t, int64_t, float, const int64_t*, int64_t, double*, double*);
int oracle_attn_masked_fp64(const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                            int64_t, int64_t, float, int, const float*, int64_t, int64_t, int64_t, const int64_t*,
                            int64_t, double*, double*);
int oracle_attn_bwd_fp64(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int64_t, int64_t,
                         int64_t, int64_t, int64_t, int64_t, float, int, const float*, int64_t, int64_t, int64_t,
                         double*, double*, double*, double*, double*);
int oracle_attn_bwd_dq_rows_fp64(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int64_t,
                                 int64_t, int64_t, int64_t, int64_t, int64_t, float, int, const float*, int64_t,
                                 int64_t, int64_t, const int64_t*, int64_t, double*);
int oracle_attn_bwd_dkdv_keys_fp64(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int64_t,
                                   int64_t, int64_t, int64_t, int64_t, int64_t, float, int, const float*, int64_t,
                                   int64_t, int64_t, const int64_t*, int64_t, double*, double*);
}

static int g_checks = 0;
static int g_fail = 0;

#define EXPECT(cond, ...)                                      \
  do {                                                         \
    ++g_checks;                                                \
    if (!(cond)) {                                             \
      ++g_fail;                                                \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                       \
      std::fprintf(stderr, "\n");                              \
    }                                                          \
  } while (0)

// A "no GPU here" call with valid arguments ends in the device check, or, on
// a machine with a gfx950 device, in the stub launcher.
static bool valid_end(int st) { return st == FA_ERR_DEVICE || st == FA_ERR_LAUNCH; }

// bf16 bits of a float that bf16 holds exactly
static uint16_t bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return (uint16_t)(u >> 16);
}
static double widen(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// deterministic small values: multiples of 1/64 in [-2, 2), exact in bf16
static void fill(std::vector<uint16_t>& v, uint32_t seed) {
  uint32_t s = seed * 2654435761u + 12345u;
  for (auto& x : v) {
    s = s * 1664525u + 1013904223u;
    x = bf16((float)((int)(s >> 24) - 128) / 64.0f);
  }
}

static void check_forward_validation() {
  const int64_t B = 2, H = 3, Nq = 100, Nk = 70, d = 128;
  std::vector<uint16_t> q(B * H * Nq * d + 8), k(B * H * Nk * d + 8), v(B * H * Nk * d + 8), o(B * H * Nq * d + 8);
  const int64_t ldb = 72;  // bias row stride: Nk rounded up to a multiple of 4
  std::vector<float> lse(B * H * Nq + 4), bias(B * H * Nq * ldb + 4);
  // 16-byte aligned views (vector storage is at least 16-byte aligned on x86-64 glibc)
  const void* Q = q.data();
  const void* K = k.data();
  const void* V = v.data();
  void* O = o.data();
  float* L = lse.data();
  const float sc = 0.0883883f;
  EXPECT(valid_end(fa_fwd(Q, K, V, O, L, B, H, Nq, Nk, d, sc, nullptr)), "valid fa_fwd");
  EXPECT(fa_fwd(Q, K, V, O, L, 0, H, Nq, Nk, d, sc, nullptr) == FA_OK, "empty batch is a no-op");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, 0, Nk, d, sc, nullptr) == FA_OK, "empty query set is a no-op");
  EXPECT(fa_fwd(Q, K, V, O, L, -1, H, Nq, Nk, d, sc, nullptr) == FA_ERR_INVALID_SHAPE, "B < 0");
  EXPECT(fa_fwd(Q, K, V, O, L, B, -1, Nq, Nk, d, sc, nullptr) == FA_ERR_INVALID_SHAPE, "H < 0");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, -1, Nk, d, sc, nullptr) == FA_ERR_INVALID_SHAPE, "Nq < 0");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, Nq, 0, d, sc, nullptr) == FA_ERR_INVALID_SHAPE, "Nk = 0");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, Nq, Nk, 96, sc, nullptr) == FA_ERR_UNSUPPORTED, "head size 96");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, Nq, FA_MAX_SEQ + 1, d, sc, nullptr) == FA_ERR_UNSUPPORTED, "Nk too long");
  EXPECT(fa_fwd(Q, K, V, O, L, INT64_MAX / 2, 3, Nq, Nk, d, sc, nullptr) == FA_ERR_INVALID_SHAPE, "B*H overflow");
  EXPECT(fa_fwd(nullptr, K, V, O, L, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_NULL_POINTER, "Q NULL");
  EXPECT(fa_fwd(Q, K, nullptr, O, L, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_NULL_POINTER, "V NULL");
  EXPECT(fa_fwd(Q, K, V, O, nullptr, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_NULL_POINTER, "LSE NULL");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, Nq, Nk, d, std::numeric_limits<float>::quiet_NaN(), nullptr) ==
             FA_ERR_INVALID_SCALE, "NaN scale");
  EXPECT(fa_fwd(Q, K, V, O, L, B, H, Nq, Nk, d, std::numeric_limits<float>::infinity(), nullptr) ==
             FA_ERR_INVALID_SCALE, "inf scale");
  EXPECT(fa_fwd((const char*)Q + 2, K, V, O, L, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_UNSUPPORTED, "Q misaligned");
  EXPECT(fa_fwd(Q, K, V, (char*)O + 8, L, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_UNSUPPORTED, "O misaligned");
  EXPECT(fa_fwd(Q, K, V, (void*)Q, L, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_ALIAS, "O aliases Q");
  EXPECT(fa_fwd(Q, K, V, O, (float*)O, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_ALIAS, "LSE aliases O");
  EXPECT(fa_fwd(Q, K, V, O, (float*)V, B, H, Nq, Nk, d, sc, nullptr) == FA_ERR_ALIAS, "LSE aliases V");
  // masked / bias / head sizes
  const float* bp = bias.data();
  EXPECT(valid_end(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 1, bp, H * Nq * ldb, Nq * ldb, ldb, nullptr)),
         "valid masked call");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 1, bp, H * Nq * Nk, Nq * Nk, Nk, nullptr) ==
             FA_ERR_UNSUPPORTED, "bias row stride 70 (not a multiple of 4)");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 2, nullptr, 0, 0, 0, nullptr) == FA_ERR_UNSUPPORTED,
         "causal flag 2");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 0, bp, -4, 0, 0, nullptr) == FA_ERR_UNSUPPORTED,
         "negative bias stride");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 0, bp, 0, 0, 6, nullptr) == FA_ERR_UNSUPPORTED,
         "bias stride not a multiple of 4");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 0, bp + 1, 0, 0, 0, nullptr) == FA_ERR_UNSUPPORTED,
         "bias misaligned");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 0, bp, 0, 0, int64_t(1) << 28, nullptr) ==
             FA_ERR_UNSUPPORTED, "bias wave span too large");
  EXPECT(fa_fwd_masked(Q, K, V, O, L, B, H, Nq, Nk, d, sc, 0, (const float*)O, 0, 0, 0, nullptr) == FA_ERR_ALIAS,
         "O aliases the bias");
  EXPECT(valid_end(fa_fwd_dv(Q, K, V, O, L, 1, 1, Nq, Nk, 192, 128, sc, 0, nullptr, 0, 0, 0, nullptr)),
         "valid (192, 128)");
  EXPECT(fa_fwd_dv(Q, K, V, O, L, 1, 1, Nq, Nk, 128, 64, sc, 0, nullptr, 0, 0, 0, nullptr) == FA_ERR_UNSUPPORTED,
         "(128, 64) not built");
  // key split and its workspace
  int64_t used = -1;
  const int64_t ws = fa_fwd_splitkv_workspace_bytes(1, 1, 128, 4096, 128, 4, &used);
  EXPECT(used == 4 && ws == 4 * 128 * (128 * 4 + 4), "split plan 4 ranges: used %lld bytes %lld", (long long)used,
         (long long)ws);
  EXPECT(fa_fwd_splitkv_workspace_bytes(1, 1, 128, 0, 128, 4, nullptr) == -FA_ERR_INVALID_SHAPE, "split Nk = 0");
  EXPECT(fa_fwd_splitkv_workspace_bytes(1, 1, 128, 100, 128, 5000, nullptr) == -FA_ERR_UNSUPPORTED,
         "split too many ranges");
  std::vector<float> wsbuf(ws / 4 + 8);
  EXPECT(fa_fwd_splitkv(Q, K, V, O, L, 1, 1, 128, 4096, d, d, sc, 0, nullptr, 0, 0, 0, 4, nullptr, 0, nullptr) ==
             FA_ERR_WORKSPACE, "split without workspace");
  EXPECT(fa_fwd_splitkv(Q, K, V, O, L, 1, 1, 128, 4096, d, d, sc, 0, nullptr, 0, 0, 0, 4, wsbuf.data(), ws - 4,
                        nullptr) == FA_ERR_WORKSPACE, "split workspace too small");
  EXPECT(fa_fwd_splitkv(Q, K, V, O, L, 1, 1, 128, 4096, d, d, sc, 0, nullptr, 0, 0, 0, 4, (void*)Q, ws, nullptr) ==
             FA_ERR_ALIAS, "split workspace aliases Q");
  std::vector<uint16_t> k2(4096 * 128), v2(4096 * 128);
  EXPECT(valid_end(fa_fwd_splitkv(Q, k2.data(), v2.data(), O, L, 1, 1, 128, 4096, d, d, sc, 0, nullptr, 0, 0, 0, 4,
                                  wsbuf.data(), ws, nullptr)),
         "valid split call");
}

static void check_backward_validation() {
  const int64_t B = 1, H = 2, Nq = 64, Nk = 96, d = 128;
  std::vector<uint16_t> q(B * H * Nq * d), k(B * H * Nk * d), v(B * H * Nk * d), o(B * H * Nq * d),
      dO(B * H * Nq * d), dq(B * H * Nq * d), dk(B * H * Nk * d), dv(B * H * Nk * d);
  std::vector<float> lse(B * H * Nq), D(B * H * Nq), bias(B * H * Nk);
  const float sc = 0.0883883f;
  EXPECT(valid_end(fa_bwd(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), dq.data(), dk.data(),
                          dv.data(), D.data(), B, H, Nq, Nk, d, sc, 0, nullptr)),
         "valid fa_bwd");
  EXPECT(fa_bwd(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), dq.data(), dk.data(), dv.data(),
                nullptr, B, H, Nq, Nk, d, sc, 0, nullptr) == FA_ERR_NULL_POINTER, "D NULL");
  EXPECT(fa_bwd(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), dq.data(), dk.data(), dv.data(),
                D.data(), B, H, Nq, Nk, 96, sc, 0, nullptr) == FA_ERR_UNSUPPORTED, "bwd head size 96");
  EXPECT(fa_bwd(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), (void*)q.data(), dk.data(),
                dv.data(), D.data(), B, H, Nq, Nk, d, sc, 0, nullptr) == FA_ERR_ALIAS, "dQ aliases Q");
  EXPECT(fa_bwd(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), dq.data(), dq.data(), dv.data(),
                D.data(), B, H, Nq, Nk, d, sc, 0, nullptr) == FA_ERR_ALIAS, "dK aliases dQ");
  EXPECT(fa_bwd_masked(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), dq.data(), dk.data(),
                       dv.data(), D.data(), B, H, Nq, Nk, 96, sc, 0, bias.data(), H * Nk, Nk, 0, nullptr) ==
             FA_ERR_UNSUPPORTED, "bias backward at head size 96");
  EXPECT(fa_bwd_dv(q.data(), k.data(), v.data(), o.data(), dO.data(), lse.data(), dq.data(), dk.data(), dv.data(),
                   D.data(), B, H, Nq, Nk, d, d, sc, 3, nullptr, 0, 0, 0, nullptr) == FA_ERR_UNSUPPORTED,
         "bwd causal flag 3");
}

static void check_mxfp8_validation() {
  const int64_t B = 1, H = 1, Nq = 64, Nk = 64, ldv = 64;
  std::vector<uint8_t> q8(Nq * 128), k8(Nk * 128), vt8(128 * ldv), vs((ldv / 32) * 128);
  std::vector<uint32_t> qs(Nq), ks(ldv);
  std::vector<uint16_t> o(Nq * 128), x(Nk * 128);
  std::vector<float> lse(Nq);
  EXPECT(valid_end(fa_fwd_mxfp8(q8.data(), qs.data(), k8.data(), ks.data(), vt8.data(), vs.data(), o.data(),
                                lse.data(), B, H, Nq, Nk, 128, ldv, 0.088f, 0, nullptr)),
         "valid mxfp8");
  EXPECT(fa_fwd_mxfp8(q8.data(), qs.data(), k8.data(), ks.data(), vt8.data(), vs.data(), o.data(), lse.data(), B, H,
                      Nq, Nk, 64, ldv, 0.088f, 0, nullptr) == FA_ERR_UNSUPPORTED, "mxfp8 head size 64");
  EXPECT(fa_fwd_mxfp8(q8.data(), qs.data(), k8.data(), ks.data(), vt8.data(), vs.data(), o.data(), lse.data(), B, H,
                      Nq, Nk, 128, 32, 0.088f, 0, nullptr) == FA_ERR_UNSUPPORTED, "ldv not a multiple of 64");
  EXPECT(fa_fwd_mxfp8(q8.data(), qs.data(), k8.data(), ks.data(), vt8.data(), vs.data(), (void*)q8.data(),
                      lse.data(), B, H, Nq, Nk, 128, ldv, 0.088f, 0, nullptr) == FA_ERR_ALIAS, "O aliases Q8");
  EXPECT(valid_end(fa_mxfp8_quantize_rows(x.data(), k8.data(), ks.data(), B, H, Nk, 128, Nk, nullptr)),
         "valid row encoder");
  EXPECT(fa_mxfp8_quantize_rows(x.data(), k8.data(), ks.data(), B, H, Nk, 128, Nk - 1, nullptr) ==
             FA_ERR_INVALID_SHAPE, "scale stride shorter than N");
  EXPECT(valid_end(fa_mxfp8_quantize_vt(x.data(), vt8.data(), vs.data(), B, H, Nk, 128, ldv, nullptr)),
         "valid V^T encoder");
  EXPECT(fa_mxfp8_quantize_vt(x.data(), vt8.data(), vs.data(), B, H, Nk, 128, ldv + 1, nullptr) ==
             FA_ERR_UNSUPPORTED, "V^T ldv not a multiple of 64");
  for (int s = 0; s <= 9; ++s) EXPECT(fa_status_string(s) != nullptr && fa_status_string(s)[0] != 0, "status %d", s);
  EXPECT(fa_build_info() != nullptr && fa_bwd_build_info() != nullptr && fa_mxfp8_build_info() != nullptr,
         "build strings");
}

static void check_oracle() {
  const int64_t B = 2, H = 2, Nq = 9, Nk = 13, d = 64, dv = 32;
  std::vector<uint16_t> Q(B * H * Nq * d), K(B * H * Nk * d), V(B * H * Nk * dv), dO(B * H * Nq * dv);
  fill(Q, 1);
  fill(K, 2);
  fill(V, 3);
  fill(dO, 4);
  // value column 5 is the constant 1.25: every O[., 5] equals it
  for (int64_t j = 0; j < B * H * Nk; ++j) V[j * dv + 5] = bf16(1.25f);
  const float sc = 0.125f;
  std::vector<double> O(B * H * Nq * dv), L(B * H * Nq);
  EXPECT(oracle_attn_fp64(Q.data(), K.data(), V.data(), B, H, Nq, Nk, d, dv, sc, O.data(), L.data()) == 0, "oracle");
  for (int64_t r = 0; r < B * H * Nq; ++r)
    EXPECT(std::fabs(O[r * dv + 5] - 1.25) < 1e-12 && std::isfinite(L[r]), "constant column, row %lld", (long long)r);
  // selected rows equal the full result bit for bit
  const int64_t rows[3] = {0, 17, B * H * Nq - 1};
  std::vector<double> Or(3 * dv), Lr(3);
  EXPECT(oracle_attn_rows_fp64(Q.data(), K.data(), V.data(), B, H, Nq, Nk, d, dv, sc, rows, 3, Or.data(),
                               Lr.data()) == 0, "oracle rows");
  for (int i = 0; i < 3; ++i)
    EXPECT(std::memcmp(&Or[i * dv], &O[rows[i] * dv], dv * 8) == 0 && Lr[i] == L[rows[i]], "row %d", i);
  // one key: O = v, LSE = scale * q.k
  std::vector<double> O1(Nq * dv), L1(Nq);
  EXPECT(oracle_attn_fp64(Q.data(), K.data(), V.data(), 1, 1, Nq, 1, d, dv, sc, O1.data(), L1.data()) == 0,
         "one key");
  for (int64_t i = 0; i < Nq; ++i) {
    double s = 0;
    for (int64_t c = 0; c < d; ++c) s += widen(Q[i * d + c]) * widen(K[c]);
    EXPECT(std::fabs(L1[i] - (double)sc * s) < 1e-12, "one-key LSE row %lld", (long long)i);
    for (int64_t c = 0; c < dv; ++c) EXPECT(O1[i * dv + c] == widen(V[c]), "one-key O");
  }
  // causal with Nq > Nk (leading rows see no key) and a bias with -inf entries
  const int64_t Nq2 = 20;
  std::vector<uint16_t> Q2(B * H * Nq2 * d);
  fill(Q2, 5);
  std::vector<float> bias(Nq2 * Nk);
  for (int64_t i = 0; i < Nq2 * Nk; ++i) bias[i] = (i % 7 == 0) ? -std::numeric_limits<float>::infinity() : 0.5f;
  std::vector<double> Om(B * H * Nq2 * dv), Lm(B * H * Nq2);
  EXPECT(oracle_attn_masked_fp64(Q2.data(), K.data(), V.data(), B, H, Nq2, Nk, d, dv, sc, 1, bias.data(), 0, 0, Nk,
                                 nullptr, B * H * Nq2, Om.data(), Lm.data()) == 0, "masked oracle");
  for (int64_t r = 0; r < B * H * Nq2; ++r) {
    const int64_t i = r % Nq2;
    if (i + Nk - Nq2 < 0) {
      EXPECT(std::isinf(Lm[r]) && Lm[r] < 0 && Om[r * dv] == 0.0, "row %lld sees no key", (long long)r);
    } else {
      EXPECT(std::isfinite(Om[r * dv]), "finite masked row %lld", (long long)r);
    }
  }
  // backward: full, rows and keys variants agree
  std::vector<double> dQ(B * H * Nq * d), dK(B * H * Nk * d), dV(B * H * Nk * dv), D(B * H * Nq), Lb(B * H * Nq);
  EXPECT(oracle_attn_bwd_fp64(Q.data(), K.data(), V.data(), dO.data(), B, H, Nq, Nk, d, dv, sc, 1, nullptr, 0, 0, 0,
                              dQ.data(), dK.data(), dV.data(), D.data(), Lb.data()) == 0, "bwd oracle");
  std::vector<double> dQr(2 * d);
  const int64_t r2[2] = {3, B * H * Nq - 2};
  EXPECT(oracle_attn_bwd_dq_rows_fp64(Q.data(), K.data(), V.data(), dO.data(), B, H, Nq, Nk, d, dv, sc, 1, nullptr, 0,
                                      0, 0, r2, 2, dQr.data()) == 0, "bwd rows");
  for (int i = 0; i < 2; ++i)
    for (int64_t c = 0; c < d; ++c) EXPECT(std::fabs(dQr[i * d + c] - dQ[r2[i] * d + c]) < 1e-12, "dQ row");
  std::vector<double> dKk(2 * d), dVk(2 * dv);
  const int64_t k2[2] = {0, B * H * Nk - 1};
  EXPECT(oracle_attn_bwd_dkdv_keys_fp64(Q.data(), K.data(), V.data(), dO.data(), B, H, Nq, Nk, d, dv, sc, 1, nullptr,
                                        0, 0, 0, k2, 2, dKk.data(), dVk.data()) == 0, "bwd keys");
  for (int i = 0; i < 2; ++i) {
    for (int64_t c = 0; c < d; ++c) EXPECT(std::fabs(dKk[i * d + c] - dK[k2[i] * d + c]) < 1e-12, "dK key");
    for (int64_t c = 0; c < dv; ++c) EXPECT(std::fabs(dVk[i * dv + c] - dV[k2[i] * dv + c]) < 1e-12, "dV key");
  }
  // rejected arguments
  EXPECT(oracle_attn_rows_fp64(Q.data(), K.data(), V.data(), B, H, Nq, Nk, d, dv, sc, nullptr, 2, Or.data(),
                               Lr.data()) != 0, "rows NULL");
  const int64_t bad[1] = {B * H * Nk};
  EXPECT(oracle_attn_bwd_dkdv_keys_fp64(Q.data(), K.data(), V.data(), dO.data(), B, H, Nq, Nk, d, dv, sc, 0, nullptr,
                                        0, 0, 0, bad, 1, dKk.data(), dVk.data()) != 0, "key index out of range");
}

int main() {
  check_forward_validation();
  check_backward_validation();
  check_mxfp8_validation();
  check_oracle();
  if (g_fail) {
    std::fprintf(stderr, "%d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("SANITIZE_OK %d\n", g_checks);
  return 0;
}

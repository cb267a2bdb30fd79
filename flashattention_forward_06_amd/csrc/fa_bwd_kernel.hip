// fa_bwd_kernel.hip -- gfx950 (CDNA4) attention backward kernels.
//
// Gradients of a loss through O = softmax_row(scale * Q K^T) V, given dO,
// by recomputing the attention matrix from the forward pass's per-row
// log-sum-exp (the recomputation named in "FlashAttention'ı Anlamak Bölüm 1",
// section 0; the gradient equations are the chain rule of the score and
// output equations of section 0.2):
//
//   P_ij  = exp(scale q_i.k_j - LSE_i)      dV_j = sum_i P_ij dO_i
//   dP_ij = dO_i . v_j                      D_i  = dO_i . O_i
//   dS_ij = P_ij (dP_ij - D_i)              dK_j = scale sum_i dS_ij q_i
//                                           dQ_i = scale sum_j dS_ij k_j
//
// Three kernels, no atomics (results do not depend on scheduling):
//   fa_bwd_delta  D_i from dO and O (one pass over 2 x [rows, 128] bf16).
//   fa_bwd_dkdv   one workgroup per 128 keys of a head; each wave owns 32
//                 keys (K and V as MFMA B operands in registers, dK^T and
//                 dV^T accumulators) and walks the query rows in blocks of
//                 64: S = Q K^T and dP = dO V^T, P and dS on the VALU,
//                 dV^T += dO^T P and dK^T += Q^T dS.  The accumulators give
//                 each lane one key and 16 query rows, so P and dS rounded
//                 to bf16 are directly the B operands of the next products
//                 and Q^T / dO^T come from the row-major LDS tiles through
//                 the transposing read (ds_read_b64_tr_b16).
//   fa_bwd_dq     one workgroup per 128 query rows (32 per wave), the
//                 forward's loop shape: S^T = K Q^T and dP^T = V dO^T, then
//                 dQ^T += K^T dS^T.
// S and dP are computed in both the dK/dV and the dQ kernel (seven matrix
// products instead of five) in exchange for no atomic accumulation of dQ.
// Tiles read both row-wise and transposed use the SWZ_BOTH swizzle.
// With an additive fp32 bias b (the mask term of the score equation) the
// logit is scale q_i.k_j + b_ij and P_ij = exp(logit - LSE_i); the gradients
// above are unchanged (no gradient is formed for b).  The bias is read from
// memory straight into registers; a row whose LSE is -inf (it saw no key)
// has its -LSE clamped to a large finite value, so -inf bias entries give
// P = 0 rather than NaN.
// At head sizes 128, (192, 128) and 256 both matrix kernels run one wave
// per SIMD (their accumulators and register-resident operands need ~350 or
// more registers; at 256 the dK/dV kernel is launched once per gradient to
// fit), so all overlap of VALU and MFMA work is inside the wave:
// each step computes two 32-row (or 32-key) sub-blocks, issues the products
// of the second before the softmax-gradient arithmetic of the first, and
// sched_group_barrier pins an interleave of one MFMA to a few VALU
// instructions (6 in dK/dV; 5 and 12 in dQ, chosen by timing; not in the dQ
// kernel at head size 256).  At head size 64 they fit two waves per SIMD.
// At head size 256 the dQ kernel is launched once per half of its output
// columns and the dK/dV kernel once per gradient (each launch recomputes S
// and dP as it needs them and spills nothing), with or without a bias.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernel.h"

namespace fa06 {
namespace {

// ---------------------------------------------------------------- delta
// DV/8 lanes per row (16 bytes each), 256/(DV/8) rows per 256-thread
// workgroup, grid-stride over all rows.
template <int DV>
__global__ void __launch_bounds__(256) fa_bwd_delta_kernel(const uint16_t* __restrict__ O,
                                                           const uint16_t* __restrict__ dO,
                                                           float* __restrict__ Dl, int64_t rows) {
  constexpr int LPR = DV / 8;   // lanes per row
  constexpr int RPB = 256 / LPR;
  const int part = threadIdx.x % LPR;
  const int sub = threadIdx.x / LPR;
  for (int64_t row = (int64_t)blockIdx.x * RPB + sub; row - sub < rows; row += (int64_t)gridDim.x * RPB) {
    float acc = 0.0f;
    if (row < rows) {
      const uintx4 o = *reinterpret_cast<const uintx4*>(O + row * DV + part * 8);
      const uintx4 g = *reinterpret_cast<const uintx4*>(dO + row * DV + part * 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc = __builtin_fmaf(__uint_as_float(o[k] << 16), __uint_as_float(g[k] << 16), acc);
        acc = __builtin_fmaf(__uint_as_float(o[k] & 0xFFFF0000u), __uint_as_float(g[k] & 0xFFFF0000u), acc);
      }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    if (row < rows && part == 0) Dl[row] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
constexpr int KV_KEYS = 128;  // keys per workgroup (32 per wave)
constexpr int KV_QB = 64;     // query rows per step
// LDS: Q[2] (rows of 2*DQK bytes), dO[2] (2*DV), LSE[2], D[2]: 66.5 KiB at
// head size 128, 82.5 KiB at (192, 128)
constexpr int kv_lds(int dqk, int dv) { return 2 * KV_QB * 2 * (dqk + dv) + 4 * KV_QB * 4; }

// Largest finite float: the clamp of -LSE * log2(e) for rows that saw no key.
constexpr float NL_MAX = 3.0e38f;

// Waves per SIMD of the dK/dV and dQ kernels.  At head size 64 both kernels
// fit two waves' registers (<= 256 each; without a bias no spills, with one
// 18-33 spilled registers) and their LDS (33 KiB / 32 KiB per workgroup)
// allows two workgroups per CU: the second wave hides the first's latency
// (backward at head size 64: +46 %, causal +38 %, with a bias +20 %, identical
// results).  Larger head sizes need more than 256 registers (accumulators,
// K/V or Q/dO operands and the S/dP tiles) and run one wave per SIMD, so the
// interleave of each wave's own MFMA and VALU work is all the overlap there is.
constexpr int bwd_waves_per_simd(int dqk) { return dqk == 64 ? 2 : 1; }
// At head size 128 the dK/dV kernel with the causal mask and the dQ kernel
// with a bias walk their tiles two per loop trip, so that each tile's LDS
// stage is a compile-time constant: the stage offset then sits in the
// fragment reads' immediate field, where a run-time stage costs a register
// per hoisted read address (and the register pressure moves the S and dP
// accumulators through AGPRs).  Measured on the backward at B=2, H=16,
// N=8192 with identical results: causal +4 %, causal with a per-key bias +5 %
// (dK/dV), with a bias +6 % (dQ).  Elsewhere it measured slower (dQ without a
// bias -7 %, dK/dV without the mask -1 %) or spills to scratch (other head
// sizes), and one tile per trip stays.
template <int DQK, int DV, bool CAUSAL, bool BIAS>
constexpr bool dkdv_unroll2() { return DQK == 128 && DV == 128 && CAUSAL; }
template <int DQK, int DV, bool CAUSAL, bool BIAS>
constexpr bool dq_unroll2() { return DQK == 128 && DV == 128 && BIAS; }
// What one launch of the dK/dV kernel writes: both gradients, or one of them
// (QHALF plays the same role for the dQ kernel's output columns).
// At head size 256 one wave cannot hold K and V rows and both accumulators
// (~200 registers spilled); a launch per gradient holds half the
// accumulators, and the products the other gradient needs are dead code
// (dV: S and P only; dK: S, dP and dS).  No spills either way: the backward
// there runs 1.4-1.6x faster although S is computed one more time.
enum DkdvPart { DKDV_BOTH = 0, DKDV_DV = 1, DKDV_DK = 2 };

template <int DQK, int DV, bool CAUSAL, bool BIAS, int PART>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd(DQK), bwd_waves_per_simd(DQK))))
fa_bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float* __restrict__ LSE, const float* __restrict__ Dl,
                   uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                   int Nq, int Nk, int n_ktiles, float c_log2, float scale,
                   const float* __restrict__ bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq, int H) {
  constexpr int RBQ = 2 * DQK;              // bytes per Q, K, dK row
  constexpr int RBV = 2 * DV;               // bytes per V, O, dO, dV row
  constexpr int KV_TILE_Q = KV_QB * RBQ;    // one Q tile
  constexpr int KV_TILE_O = KV_QB * RBV;    // one dO tile
  constexpr int NTQ = DQK / 16, NTV = DV / 16;   // 16-wide k steps
  constexpr int NCQ = DQK / 32, NCV = DV / 32;   // 32-column output blocks
  constexpr bool UNROLL2 = dkdv_unroll2<DQK, DV, CAUSAL, BIAS>();
  __shared__ __attribute__((aligned(1024))) char smem[kv_lds(DQK, DV)];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;

  // causal: key tile 0 is seen by the most query rows, so ascending tiles
  // are longest-first
  int bh, kt;
  if constexpr (BIAS) {
    // heads that share dense bias columns run side by side (one bias fetch)
    const HeadGroup hg = bias_head_group(gridDim.x / (n_ktiles * H), H, bias_sb, bias_sh, bias_sq);
    grouped_tile_map(blockIdx.x, gridDim.x, n_ktiles, CAUSAL, hg, bh, kt);
  } else {
    xcd_tile_map(blockIdx.x, gridDim.x, n_ktiles, CAUSAL, bh, kt);
  }
  const int k0 = kt * KV_KEYS;
  const int kw = k0 + wave * 32;  // this wave's first key
  const int key = kw + c;         // this lane's key

  const size_t head_q = (size_t)bh * (size_t)Nq;
  const size_t head_k = (size_t)bh * (size_t)Nk;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head_q * DQK, (uint32_t)Nq * RBQ);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dO + head_q * DV, (uint32_t)Nq * RBV);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(LSE + head_q, (uint32_t)Nq * 4u);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(Dl + head_q, (uint32_t)Nq * 4u);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head_k * DQK, (uint32_t)Nk * RBQ);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head_k * DV, (uint32_t)Nk * RBV);
  const __amdgpu_buffer_rsrc_t rdk = make_rsrc(dK + head_k * DQK, (uint32_t)Nk * RBQ);
  const __amdgpu_buffer_rsrc_t rdv = make_rsrc(dV + head_k * DV, (uint32_t)Nk * RBV);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // K and V rows of this wave's keys as B operands: kb[t] = K[key][16t + 8h .. +7]
  // (keys past Nk read as zero; their results are not stored)
  bf16x8 kb[NTQ], vb[NTV];
#pragma unroll
  for (int t = 0; t < NTQ; ++t)
    kb[t] = __builtin_bit_cast(bf16x8, buf_load16(rk, (uint32_t)key * RBQ + (uint32_t)(2 * t + h) * 16u));
#pragma unroll
  for (int t = 0; t < NTV; ++t)
    vb[t] = __builtin_bit_cast(bf16x8, buf_load16(rv, (uint32_t)key * RBV + (uint32_t)(2 * t + h) * 16u));

  // Bias column of this wave's 32 keys over all query rows: lane (c, h)
  // reads key kw + c of rows 8g + 4h + e of each 32-row sub-block, one dword
  // per load, the row offset in the scalar offset.  The resource ends at
  // the wave's last key of row Nq - 1.
  __amdgpu_buffer_rsrc_t rb = make_rsrc(nullptr, 0u);
  uint32_t bias_voff = 0;
  uint32_t bias_row_bytes = 0;
  if constexpr (BIAS) {
    const int b = bh / H;
    const int hd = bh - b * H;
    // kw_u, not kw: the resource must be provably wave-uniform, or the
    // compiler wraps every load in a loop over the distinct descriptors
    const int kw_u = k0 + wave_u * 32;
    const float* base = bias + (int64_t)b * bias_sb + (int64_t)hd * bias_sh + kw_u;
    const uint32_t bytes = kw_u < Nk ? (uint32_t)(((int64_t)(Nq - 1) * bias_sq + (Nk - kw_u)) * 4) : 0u;
    rb = make_rsrc(base, bytes);
    bias_row_bytes = (uint32_t)(bias_sq * 4);
    bias_voff = (uint32_t)c * 4u + (uint32_t)(4 * h) * bias_row_bytes;
  }
  // A bias that does not depend on the row (stride 0 over queries, e.g. a
  // key padding mask) is one value per lane for the whole kernel.
  const bool bias_per_key = BIAS && bias_sq == 0;
  float bias_key = 0.0f;
  if constexpr (BIAS) {
    if (bias_per_key) bias_key = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, bias_voff, 0, 0));
  }
  // bb[r]: bias of row qb*64 + ib*32 + 8(r/4) + 4h + r%4, key kw + c
  auto load_bias = [&](int qb, int ib, float (&bb)[16]) FA_INLINE {
    if (bias_per_key) {
#pragma unroll
      for (int r = 0; r < 16; ++r) bb[r] = bias_key;
      return;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const uint32_t row = (uint32_t)(qb * KV_QB + ib * 32 + 8 * (r >> 2) + (r & 3));
      bb[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rb, bias_voff, __builtin_amdgcn_readfirstlane(row * bias_row_bytes), 0));
    }
  };

  // query blocks that see at least one of the workgroup's keys, and the
  // first block in which every (row, key) pair is visible
  const int off = Nk - Nq;
  const int n_qb = (Nq + KV_QB - 1) / KV_QB;
  int qb_first = 0, qb_unmasked = 0;
  if constexpr (CAUSAL) {
    const int first_row = k0 - off;  // first row that sees key k0
    qb_first = first_row <= 0 ? 0 : first_row / KV_QB;
    const int last_hidden = k0 + KV_KEYS - 1 - off;  // rows below it miss some key
    qb_unmasked = last_hidden <= 0 ? 0 : (last_hidden + KV_QB - 1) / KV_QB;
    qb_first = qb_first < n_qb ? qb_first : n_qb;
    qb_unmasked = qb_unmasked < qb_first ? qb_first : (qb_unmasked > n_qb ? n_qb : qb_unmasked);
  }

  char* const qbuf0 = smem;
  char* const dobuf0 = smem + 2 * KV_TILE_Q;
  char* const lbuf0 = dobuf0 + 2 * KV_TILE_O;
  char* const dbuf0 = lbuf0 + 2 * KV_QB * 4;
  auto stage_in = [&](int qb, int st) FA_INLINE {
    tile_to_lds<KV_QB, SWZ_BOTH, DQK>(rq, (uint32_t)(qb * KV_QB), qbuf0 + st * KV_TILE_Q, wave_u, lane);
    tile_to_lds<KV_QB, SWZ_BOTH, DV>(rdo, (uint32_t)(qb * KV_QB), dobuf0 + st * KV_TILE_O, wave_u, lane);
    // 64 floats of LSE and of D: 16 lanes x 16 bytes each
    if (wave_u < 2 && lane < 16) {
      const __amdgpu_buffer_rsrc_t r = wave_u == 0 ? rl : rd;
      char* dst = (wave_u == 0 ? lbuf0 : dbuf0) + st * KV_QB * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_char*)dst, 16,
                                               (uint32_t)lane * 16u,
                                               __builtin_amdgcn_readfirstlane((uint32_t)(qb * KV_QB * 4)), 0, 0);
    }
  };

  floatx16 dvacc[NCV], dkacc[NCQ];
#pragma unroll
  for (int i = 0; i < NCV; ++i) dvacc[i] = floatx16{};
#pragma unroll
  for (int i = 0; i < NCQ; ++i) dkacc[i] = floatx16{};

  // At head size 128 without a bias the LDS fragments of the S/dP and dV/dK
  // products are read PFK MFMAs ahead of their use (a ring of PFK + 1), as in
  // the dQ kernel.  Backward at B=2, H=16, N=8192, identical results: 650 ->
  // 664 TFLOP/s with 2 ahead (3: 660), causal 624 -> 652 with 3 ahead (2:
  // 637); with a per-key bias (sequential step) it lost 5 % and is not used.
  constexpr int PFK = DQK == 128 && DV == 128 && !BIAS ? (CAUSAL ? 3 : 2) : 0;

  // dV^T += dO^T P and dK^T += Q^T dS, the two column-block loops interleaved
  constexpr int NCMAX = NCQ > NCV ? NCQ : NCV;
  auto dvdk = [&](const char* qs, const char* ds, int ib, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) FA_INLINE {
    if constexpr (PFK > 0) {
      // MFMA m: column block m >> 2, k half (m >> 1) & 1, dV (even m) or dK (odd m)
      constexpr int PF = PFK, NM = 4 * NCMAX;
      auto rd = [&](int m) FA_INLINE {
        return (m & 1) ? tr_read_a<SWZ_BOTH, DQK>(qs, ib * 32 + ((m >> 1) & 1) * 16, m >> 2, lane)
                       : tr_read_a<SWZ_BOTH, DV>(ds, ib * 32 + ((m >> 1) & 1) * 16, m >> 2, lane);
      };
      bf16x8 fr[PF + 1];
#pragma unroll
      for (int m = 0; m < PF; ++m) fr[m] = rd(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + PF < NM) fr[(m + PF) % (PF + 1)] = rd(m + PF);
        const int cb = m >> 2, ks = (m >> 1) & 1;
        if (m & 1)
          dkacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PF + 1)], dsb[ks], dkacc[cb], 0, 0, 0);
        else
          dvacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PF + 1)], pb[ks], dvacc[cb], 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int cb = 0; cb < NCMAX; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (cb < NCV)
          dvacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_read_a<SWZ_BOTH, DV>(ds, ib * 32 + ks * 16, cb, lane), pb[ks], dvacc[cb], 0, 0, 0);
        if (cb < NCQ)
          dkacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tr_read_a<SWZ_BOTH, DQK>(qs, ib * 32 + ks * 16, cb, lane), dsb[ks], dkacc[cb], 0, 0, 0);
      }
  };

  // Sequential step: one block of 64 query rows as two sub-blocks of 32, in
  // order, for the kernels where the pipelined form below would need more
  // registers than a wave has (a bias; the causal mask at (192, 128) and 64,
  // where it is also no faster).
  // MASK steps hide the pairs above the causal diagonal and, with a bias,
  // the rows past Nq of a ragged last block (whose zero Q and LSE would
  // otherwise give P = exp(bias), possibly infinite).
  // bb2: the step's bias, both sub-blocks (unused without BIAS)
  auto step_seq = [&](int qb, int st, auto mask_tag, const float (&bb2)[2][16]) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    const char* qs = qbuf0 + st * KV_TILE_Q;
    const char* ds = dobuf0 + st * KV_TILE_O;
    const char* ls = lbuf0 + st * KV_QB * 4;
    const char* dls = dbuf0 + st * KV_QB * 4;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
      const float (&bb)[16] = bb2[ib];
      floatx16 s = floatx16{}, dp = floatx16{};
#pragma unroll
      for (int t = 0; t < NTQ; ++t)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_a<SWZ_BOTH, DQK>(qs, ib * 32, t, c, h), kb[t], s, 0, 0,
                                                    0);
#pragma unroll
      for (int t = 0; t < NTV; ++t)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_a<SWZ_BOTH, DV>(ds, ib * 32, t, c, h), vb[t], dp, 0, 0,
                                                     0);
      // accumulator register r holds row ib*32 + 8(r/4) + 4h + r%4 of the block
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 l4 = *reinterpret_cast<const floatx4*>(ls + (ib * 32 + 8 * g + 4 * h) * 4);
        const floatx4 d4 = *reinterpret_cast<const floatx4*>(dls + (ib * 32 + 8 * g + 4 * h) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p;
          if constexpr (BIAS) {
            const float nl = fminf(-l4[e] * LOG2E, NL_MAX);
            p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, __builtin_fmaf(bb[r], LOG2E, nl)));
          } else {
            p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l4[e] * LOG2E));
          }
          if constexpr (MASK) {
            const int row = qb * KV_QB + ib * 32 + 8 * g + 4 * h + e;
            if ((CAUSAL && key > row + off) || (BIAS && row >= Nq)) p = 0.0f;
          }
          const float dsv = p * (dp[r] - d4[e]);
          pb[r >> 3][r & 7] = (__bf16)p;
          dsb[r >> 3][r & 7] = (__bf16)dsv;
        }
      }
      dvdk(qs, ds, ib, pb, dsb);
    }
  };

  // One block of 64 query rows as two sub-blocks of 32, software pipelined
  // inside the wave: S/dP of sub-block 1 are issued before the P/dS of
  // sub-block 0, and dV/dK of sub-block 0 before the P/dS of sub-block 1.
  auto sdp = [&](const char* qs, const char* ds, int ib, floatx16& s, floatx16& dp) FA_INLINE {
    s = floatx16{};
    dp = floatx16{};
    if constexpr (PFK > 0) {
      constexpr int NM = NTQ + NTV;
      auto rd = [&](int m) FA_INLINE {
        return m < NTQ ? row_read_a<SWZ_BOTH, DQK>(qs, ib * 32, m, c, h) : row_read_a<SWZ_BOTH, DV>(ds, ib * 32, m - NTQ, c, h);
      };
      bf16x8 fr[PFK + 1];
#pragma unroll
      for (int m = 0; m < PFK; ++m) fr[m] = rd(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + PFK < NM) fr[(m + PFK) % (PFK + 1)] = rd(m + PFK);
        if (m < NTQ)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PFK + 1)], kb[m], s, 0, 0, 0);
        else
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PFK + 1)], vb[m - NTQ], dp, 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < NTQ; ++t)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_a<SWZ_BOTH, DQK>(qs, ib * 32, t, c, h), kb[t], s, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NTV; ++t)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_a<SWZ_BOTH, DV>(ds, ib * 32, t, c, h), vb[t], dp, 0, 0, 0);
  };
  auto pds = [&](const char* ls, const char* dls, int qb, int ib, const floatx16& s, const floatx16& dp,
                 auto mask_tag, bf16x8 (&pb)[2], bf16x8 (&dsb)[2]) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
    // accumulator register r holds row ib*32 + 8(r/4) + 4h + r%4 of the
    // block; the key is hidden from that row when 8(r/4) + r%4 < kd
    const int kd = key - off - qb * KV_QB - ib * 32 - 4 * h;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const floatx4 l4 = *reinterpret_cast<const floatx4*>(ls + (ib * 32 + 8 * g + 4 * h) * 4);
      const floatx4 d4 = *reinterpret_cast<const floatx4*>(dls + (ib * 32 + 8 * g + 4 * h) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l4[e] * LOG2E));
        if constexpr (MASK) {
          if (8 * g + e < kd) p = 0.0f;
        }
        const float dsv = p * (dp[r] - d4[e]);
        pb[r >> 3][r & 7] = (__bf16)p;
        dsb[r >> 3][r & 7] = (__bf16)dsv;
      }
    }
  };
  auto step = [&](int qb, int st, auto mask_tag) FA_INLINE {
    const char* qs = qbuf0 + st * KV_TILE_Q;
    const char* ds = dobuf0 + st * KV_TILE_O;
    const char* ls = lbuf0 + st * KV_QB * 4;
    const char* dls = dbuf0 + st * KV_QB * 4;
    floatx16 s0, dp0, s1, dp1;
    bf16x8 p0[2], g0[2], p1[2], g1[2];
    sdp(qs, ds, 0, s0, dp0);
    sdp(qs, ds, 1, s1, dp1);
    pds(ls, dls, qb, 0, s0, dp0, mask_tag, p0, g0);
#pragma unroll
    for (int i = 0; i < NTQ + NTV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    dvdk(qs, ds, 0, p0, g0);
    pds(ls, dls, qb, 1, s1, dp1, mask_tag, p1, g1);
#pragma unroll
    for (int i = 0; i < 2 * (NCQ + NCV); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    dvdk(qs, ds, 1, p1, g1);
  };

  auto block = [&](int qb, int st) FA_INLINE {
    wait_vmem();
    __syncthreads();  // stage st landed for every wave; stage st^1 is free
    // the step's bias loads go out before the next stage's copies: loads
    // complete in order, so using the bias then waits for them alone
    float bb2[2][16];
    if constexpr (BIAS) {
      load_bias(qb, 0, bb2[0]);
      load_bias(qb, 1, bb2[1]);
    }
    if (qb + 1 < n_qb) stage_in(qb + 1, st ^ 1);
    if constexpr (CAUSAL && !BIAS && DQK == 128 && DV == 128) {
      // causal at head size 128: the pipelined step, masked on every block
      // (one variant in the loop fits the registers; two did not), +6 %
      // over the sequential step
      step(qb, st, std::true_type{});
    } else if constexpr (CAUSAL || BIAS) {
      // Where two step variants in one loop make the compiler spill (a bias
      // without the causal mask; the causal mask at (d, d_v) = (192, 128)),
      // every step is the masked one: its masks are exact on every block,
      // only a compare per element dearer.
      constexpr bool ALWAYS_MASK = (BIAS && !CAUSAL) || (CAUSAL && DQK + DV > 256);
      const bool mask = ALWAYS_MASK || (CAUSAL && qb < qb_unmasked) || (BIAS && qb == n_qb - 1 && Nq % KV_QB != 0);
      if (mask)
        step_seq(qb, st, std::true_type{}, bb2);
      else
        step_seq(qb, st, std::false_type{}, bb2);
    } else {
      step(qb, st, std::false_type{});
    }
  };
  if (qb_first < n_qb) stage_in(qb_first, 0);
  if constexpr (UNROLL2) {
    int qb = qb_first;
    for (; qb + 1 < n_qb; qb += 2) {
      block(qb, 0);
      block(qb + 1, 1);
    }
    if (qb < n_qb) block(qb, 0);
  } else {
    for (int qb = qb_first; qb < n_qb; ++qb) block(qb, (qb - qb_first) & 1);
  }

  if constexpr (PART != DKDV_DV) {
#pragma unroll
    for (int cb = 0; cb < NCQ; ++cb) store_bf16_row_block<DQK>(rdk, (uint32_t)key, cb, h, dkacc[cb], scale);
  }
  if constexpr (PART != DKDV_DK) {
#pragma unroll
    for (int cb = 0; cb < NCV; ++cb) store_bf16_row_block<DV>(rdv, (uint32_t)key, cb, h, dvacc[cb], 1.0f);
  }
}

// ---------------------------------------------------------------- dQ
constexpr int DQ_ROWS = 128;  // query rows per workgroup (32 per wave)
constexpr int DQ_BC = 64;     // keys per tile
// LDS: K[2] (rows of 2*DQK bytes), V[2] (2*DV)
constexpr int dq_lds(int dqk, int dv) { return 2 * DQ_BC * 2 * (dqk + dv); }

template <int DQK, int DV, bool CAUSAL, bool BIAS, int QHALF>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(bwd_waves_per_simd(DQK), bwd_waves_per_simd(DQK))))
fa_bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                 const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                 const float* __restrict__ LSE, const float* __restrict__ Dl, uint16_t* __restrict__ dQ,
                 int Nq, int Nk, int n_qtiles, float c_log2, float scale,
                 const float* __restrict__ bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq, int H) {
  constexpr int RBQ = 2 * DQK;
  constexpr int RBV = 2 * DV;
  constexpr int DQ_TILE_K = DQ_BC * RBQ;
  constexpr int DQ_TILE_V = DQ_BC * RBV;
  constexpr int NTQ = DQK / 16, NTV = DV / 16;
  constexpr int NCQ = DQK / 32;
  // output column blocks this launch accumulates and writes: all, or one half
  constexpr int CB0 = QHALF == 2 ? NCQ / 2 : 0;
  constexpr int CB1 = QHALF == 1 ? NCQ / 2 : NCQ;
  __shared__ __attribute__((aligned(1024))) char smem[dq_lds(DQK, DV)];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;

  int bh, qt;
  if constexpr (BIAS) {
    // heads that share dense bias rows run side by side (one bias fetch)
    const HeadGroup hg = bias_head_group(gridDim.x / (n_qtiles * H), H, bias_sb, bias_sh, bias_sq);
    grouped_tile_map(blockIdx.x, gridDim.x, n_qtiles, CAUSAL, hg, bh, qt);
  } else {
    xcd_tile_map(blockIdx.x, gridDim.x, n_qtiles, CAUSAL, bh, qt);
  }
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // the longest rows start first
  const int q0 = qt * DQ_ROWS;
  const int q = q0 + wave * 32 + c;  // this lane's query row

  const size_t head_q = (size_t)bh * (size_t)Nq;
  const size_t head_k = (size_t)bh * (size_t)Nk;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head_q * DQK, (uint32_t)Nq * RBQ);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(dO + head_q * DV, (uint32_t)Nq * RBV);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(LSE + head_q, (uint32_t)Nq * 4u);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(Dl + head_q, (uint32_t)Nq * 4u);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head_k * DQK, (uint32_t)Nk * RBQ);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head_k * DV, (uint32_t)Nk * RBV);
  const __amdgpu_buffer_rsrc_t rdq = make_rsrc(dQ + head_q * DQK, (uint32_t)Nq * RBQ);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  const int n_full = Nk / DQ_BC;
  int n_tiles = n_full + (Nk % DQ_BC != 0);
  int first_masked = n_full;
  int key_lim = Nk - 1;
  if constexpr (CAUSAL) {
    const int off = Nk - Nq;
    const int q_last = (q0 + DQ_ROWS < Nq ? q0 + DQ_ROWS : Nq) - 1;
    const int lim_last = q_last + off;
    const int lim_first = q0 + off;
    const int need = lim_last < 0 ? 0 : lim_last / DQ_BC + 1;
    n_tiles = need < n_tiles ? need : n_tiles;
    const int unmasked = lim_first + 1 <= 0 ? 0 : (lim_first + 1) / DQ_BC;
    first_masked = unmasked < first_masked ? unmasked : first_masked;
    key_lim = q + off < key_lim ? q + off : key_lim;
  }

  // Q and dO rows of this lane's query as B operands (rows past Nq read 0)
  bf16x8 qb[NTQ], dob[NTV];
#pragma unroll
  for (int t = 0; t < NTQ; ++t)
    qb[t] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)q * RBQ + (uint32_t)(2 * t + h) * 16u));
#pragma unroll
  for (int t = 0; t < NTV; ++t)
    dob[t] = __builtin_bit_cast(bf16x8, buf_load16(rdo, (uint32_t)q * RBV + (uint32_t)(2 * t + h) * 16u));
  float nl2 = -__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)q * 4u, 0, 0)) * LOG2E;
  if constexpr (BIAS) nl2 = fminf(nl2, NL_MAX);

  // Bias rows of this wave's 32 queries (the forward kernel's pattern): per
  // 32-key block, lane (c, h) loads keys 8g + 4h .. +3 (g = 0..3) of row
  // q0 + 32*wave + c as four 16-byte loads; the resource ends at the last key
  // of the wave's last valid row.
  __amdgpu_buffer_rsrc_t rb = make_rsrc(nullptr, 0u);
  uint32_t bias_voff = 0;
  if constexpr (BIAS) {
    const int b = bh / H;
    const int hd = bh - b * H;
    const int qw0 = q0 + wave_u * 32;  // wave-uniform resource (see the dK/dV kernel)
    const int nrows = Nq - qw0 < 32 ? Nq - qw0 : 32;
    const float* base = bias + (int64_t)b * bias_sb + (int64_t)hd * bias_sh + (int64_t)qw0 * bias_sq;
    const uint32_t bytes = nrows > 0 ? (uint32_t)(((int64_t)(nrows - 1) * bias_sq + Nk) * 4) : 0u;
    rb = make_rsrc(base, bytes);
    bias_voff = (uint32_t)((int64_t)c * bias_sq * 4) + 16u * (uint32_t)h;
  }
  auto load_bias = [&](int j, floatx4 (&bt)[2][4]) FA_INLINE {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)j * (uint32_t)(DQ_BC * 4));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bt[kb][g] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rb, bias_voff + (uint32_t)(kb * 128 + g * 32), soff, 0));
  };
  const float dq_d = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rd, (uint32_t)q * 4u, 0, 0));

  floatx16 dqacc[NCQ];
#pragma unroll
  for (int i = 0; i < NCQ; ++i) dqacc[i] = floatx16{};

  char* const kbuf0 = smem;
  char* const vbuf0 = smem + 2 * DQ_TILE_K;
  auto stage_in = [&](int j, int st) FA_INLINE {
    tile_to_lds<DQ_BC, SWZ_BOTH, DQK>(rk, (uint32_t)(j * DQ_BC), kbuf0 + st * DQ_TILE_K, wave_u, lane);
    tile_to_lds<DQ_BC, SWZ_ROW, DV>(rv, (uint32_t)(j * DQ_BC), vbuf0 + st * DQ_TILE_V, wave_u, lane);
  };

  // One K/V tile as two 32-key blocks, software pipelined inside the wave:
  // S/dP of block 1 are issued before the softmax of block 0, and dQ of
  // block 0 before the softmax of block 1, so the VALU work overlaps MFMAs.
  // At head size 128 the A fragments are read PFQ MFMAs ahead of their use (a
  // ring of PFQ + 1): one wave per SIMD has no other wave to cover the LDS
  // latency, and the compiler's own order read each one only one or two MFMAs
  // ahead.  Backward at B=2, H=16, N=8192, identical results: 647 -> 662
  // TFLOP/s, causal 603 -> 634, per-key bias 508 -> 518 (2 ahead: 660, 631,
  // 517).  At head size 64 with a bias the ring makes the kernel spill.
  constexpr int PFQ = DQK == 128 && DV == 128 ? 3 : 0;
  auto sdp = [&](const char* ks, const char* vs, int kb, floatx16& s, floatx16& dp) FA_INLINE {
    s = floatx16{};
    dp = floatx16{};
    if constexpr (PFQ > 0) {
      constexpr int NM = NTQ + NTV;
      auto rd = [&](int m) FA_INLINE {
        return m < NTQ ? row_read_a<SWZ_BOTH, DQK>(ks, kb * 32, m, c, h) : row_read_a<SWZ_ROW, DV>(vs, kb * 32, m - NTQ, c, h);
      };
      bf16x8 fr[PFQ + 1];
#pragma unroll
      for (int m = 0; m < PFQ; ++m) fr[m] = rd(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + PFQ < NM) fr[(m + PFQ) % (PFQ + 1)] = rd(m + PFQ);
        if (m < NTQ)
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PFQ + 1)], qb[m], s, 0, 0, 0);
        else
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PFQ + 1)], dob[m - NTQ], dp, 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < NTQ; ++t)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_a<SWZ_BOTH, DQK>(ks, kb * 32, t, c, h), qb[t], s, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < NTV; ++t)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_read_a<SWZ_ROW, DV>(vs, kb * 32, t, c, h), dob[t], dp, 0, 0, 0);
  };
  auto dsoft = [&](const floatx16& s, const floatx16& dp, int kb, int lim, auto mask_tag, const floatx4 (&bk)[4],
                   bf16x8 (&dsb)[2]) FA_INLINE {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p;
      if constexpr (BIAS)
        p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, __builtin_fmaf(bk[r >> 2][r & 3], LOG2E, nl2)));
      else
        p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, nl2));
      if constexpr (MASK) {
        const int kk = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (kk > lim) p = 0.0f;
      }
      dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dq_d));
    }
  };
  auto dq_acc = [&](const char* ks, int kb, const bf16x8 (&dsb)[2]) FA_INLINE {
    if constexpr (PFQ > 0) {
      constexpr int NM = 2 * (CB1 - CB0);
      auto rd = [&](int m) FA_INLINE { return tr_read_a<SWZ_BOTH, DQK>(ks, kb * 32 + (m & 1) * 16, CB0 + (m >> 1), lane); };
      bf16x8 fr[PFQ + 1];
#pragma unroll
      for (int m = 0; m < PFQ && m < NM; ++m) fr[m] = rd(m);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m + PFQ < NM) fr[(m + PFQ) % (PFQ + 1)] = rd(m + PFQ);
        const int cb = CB0 + (m >> 1);
        dqacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[m % (PFQ + 1)], dsb[m & 1], dqacc[cb], 0, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int cb = CB0; cb < CB1; ++cb)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        dqacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_read_a<SWZ_BOTH, DQK>(ks, kb * 32 + k2 * 16, cb, lane), dsb[k2], dqacc[cb], 0, 0, 0);
  };
  // bias of the tile being computed (bt) and of the next one (bn, loaded
  // one tile ahead so its latency hides behind a tile of work; at (192, 128)
  // the registers for that are not there, and each tile loads its own)
  constexpr bool BIAS_AHEAD = DQK + DV <= 256;
  // Explicit MFMA/VALU interleave of each step.  Not at head size 256: its
  // all-columns build spilled ~100 registers to scratch, and with the
  // interleave groups its dQ came out wrong on the masked tiles (causal
  // diagonal, ragged last tile) while the unmasked tiles and every other head
  // size were right; the default schedule of the same source matched the
  // oracle, and the half-column kernels used at that size keep it.  Not in
  // the head-size-64 kernels with a bias either, the other builds that spill
  // registers to scratch (19-21 dwords per lane): without the groups their
  // results are bit-identical and the backward with a per-key bias is 5 %
  // faster (2 % slower with the causal mask as well).
  constexpr bool DQ_INTERLEAVE = DQK != 256 && !(DQK == 64 && BIAS);
  floatx4 bt[2][4], bn[2][4];
  if constexpr (BIAS && BIAS_AHEAD) {
    if (n_tiles > 0) load_bias(0, bt);
  }
  auto step = [&](int j, int st, auto mask_tag) FA_INLINE {
    const char* ks = kbuf0 + st * DQ_TILE_K;
    const char* vs = vbuf0 + st * DQ_TILE_V;
    const int lim = key_lim - j * DQ_BC;
    floatx16 s0, dp0, s1, dp1;
    bf16x8 ds0[2], ds1[2];
    if constexpr (BIAS && BIAS_AHEAD) {
      if (j + 1 < n_tiles) load_bias(j + 1, bn);
    } else if constexpr (BIAS) {
      load_bias(j, bt);
    }
    sdp(ks, vs, 0, s0, dp0);
    sdp(ks, vs, 1, s1, dp1);
    dsoft(s0, dp0, 0, lim, mask_tag, bt[0], ds0);
    // the MFMAs of S/dP(1), each followed by 5 VALU of the softmax of block 0
    if constexpr (DQ_INTERLEAVE) {
#pragma unroll
      for (int i = 0; i < NTQ + NTV; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
      }
    }
    dq_acc(ks, 0, ds0);
    dsoft(s1, dp1, 1, lim, mask_tag, bt[1], ds1);
    if constexpr (DQ_INTERLEAVE) {
#pragma unroll
      for (int i = 0; i < 2 * NCQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
      }
    }
    dq_acc(ks, 1, ds1);
    if constexpr (BIAS && BIAS_AHEAD) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) bt[kb][g] = bn[kb][g];
    }
  };

  if (n_tiles > 0) stage_in(0, 0);
  if constexpr (dq_unroll2<DQK, DV, CAUSAL, BIAS>()) {
    auto tile = [&](int j, int st) FA_INLINE {
      wait_vmem();
      __syncthreads();
      if (j + 1 < n_tiles) stage_in(j + 1, st ^ 1);
      if (j >= first_masked)
        step(j, st, std::true_type{});
      else
        step(j, st, std::false_type{});
    };
    int j = 0;
    for (; j + 1 < n_tiles; j += 2) {
      tile(j, 0);
      tile(j + 1, 1);
    }
    if (j < n_tiles) tile(j, 0);
  } else {
    for (int j = 0; j < n_tiles; ++j) {
      const int st = j & 1;
      wait_vmem();
      __syncthreads();
      if (j + 1 < n_tiles) stage_in(j + 1, st ^ 1);
      if (j >= first_masked)
        step(j, st, std::true_type{});
      else
        step(j, st, std::false_type{});
    }
  }

#pragma unroll
  for (int cb = CB0; cb < CB1; ++cb) store_bf16_row_block<DQK>(rdq, (uint32_t)q, cb, h, dqacc[cb], scale);
}

// Kernels of one (d, d_v) pair.
struct BwdKernels {
  const void* delta;
  int delta_rows_per_block;
  const void* dkdv[2][2];        // [causal][bias]
  const void* dkdv_dv[2][2];     // [causal][bias]: dV only (head size 256)
  const void* dkdv_dk[2][2];     // [causal][bias]: dK only (head size 256)
  const void* dq_half[2][2][2];  // [causal][bias][half]: half of the dQ columns (head size 256)
  const void* dq[2][2];
  bool split;                    // head size 256: the split kernels above
};

template <int DQK, int DV>
BwdKernels bwd_kernels() {
  BwdKernels k{};
  k.delta = (const void*)&fa_bwd_delta_kernel<DV>;
  k.delta_rows_per_block = 256 / (DV / 8);
  k.split = DQK == 256;
  if constexpr (DQK == 256) {
    // one launch per gradient for dK/dV, one per half of the columns for dQ.
    // Each fits one wave's registers without spilling to scratch memory.
    // The all-in-one kernels at this size spilled 100-150 registers to
    // scratch, and two of those builds (the dQ kernel with explicit
    // interleave groups; the dQ kernel with a bias) returned wrong dQ while
    // the same source compiled without scratch spills matches the oracle.
    k.dkdv_dv[0][0] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, false, false, DKDV_DV>;
    k.dkdv_dv[1][0] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, true, false, DKDV_DV>;
    k.dkdv_dv[0][1] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, false, true, DKDV_DV>;
    k.dkdv_dv[1][1] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, true, true, DKDV_DV>;
    k.dkdv_dk[0][0] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, false, false, DKDV_DK>;
    k.dkdv_dk[1][0] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, true, false, DKDV_DK>;
    k.dkdv_dk[0][1] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, false, true, DKDV_DK>;
    k.dkdv_dk[1][1] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, true, true, DKDV_DK>;
    k.dq_half[0][0][0] = (const void*)&fa_bwd_dq_kernel<DQK, DV, false, false, 1>;
    k.dq_half[0][0][1] = (const void*)&fa_bwd_dq_kernel<DQK, DV, false, false, 2>;
    k.dq_half[1][0][0] = (const void*)&fa_bwd_dq_kernel<DQK, DV, true, false, 1>;
    k.dq_half[1][0][1] = (const void*)&fa_bwd_dq_kernel<DQK, DV, true, false, 2>;
    k.dq_half[0][1][0] = (const void*)&fa_bwd_dq_kernel<DQK, DV, false, true, 1>;
    k.dq_half[0][1][1] = (const void*)&fa_bwd_dq_kernel<DQK, DV, false, true, 2>;
    k.dq_half[1][1][0] = (const void*)&fa_bwd_dq_kernel<DQK, DV, true, true, 1>;
    k.dq_half[1][1][1] = (const void*)&fa_bwd_dq_kernel<DQK, DV, true, true, 2>;
  } else {
    k.dkdv[0][0] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, false, false, DKDV_BOTH>;
    k.dkdv[1][0] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, true, false, DKDV_BOTH>;
    k.dkdv[0][1] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, false, true, DKDV_BOTH>;
    k.dkdv[1][1] = (const void*)&fa_bwd_dkdv_kernel<DQK, DV, true, true, DKDV_BOTH>;
    k.dq[0][0] = (const void*)&fa_bwd_dq_kernel<DQK, DV, false, false, 0>;
    k.dq[1][0] = (const void*)&fa_bwd_dq_kernel<DQK, DV, true, false, 0>;
    k.dq[0][1] = (const void*)&fa_bwd_dq_kernel<DQK, DV, false, true, 0>;
    k.dq[1][1] = (const void*)&fa_bwd_dq_kernel<DQK, DV, true, true, 0>;
  }
  return k;
}

}  // namespace

int launch_fa_bwd(const BwdArgs& a, hipStream_t stream) {
  BwdKernels kn;
  if (a.d == 64 && a.dv == 64) kn = bwd_kernels<64, 64>();
  else if (a.d == 128 && a.dv == 128) kn = bwd_kernels<128, 128>();
  else if (a.d == 192 && a.dv == 128) kn = bwd_kernels<192, 128>();
  else if (a.d == 256 && a.dv == 256) kn = bwd_kernels<256, 256>();
  else return 1;
  // kernels for this call, checked before anything is enqueued
  const int ci = a.causal ? 1 : 0;
  const int bi = a.bias != nullptr ? 1 : 0;
  const bool split = kn.split;
  if (split ? (kn.dkdv_dv[ci][bi] == nullptr || kn.dkdv_dk[ci][bi] == nullptr || kn.dq_half[ci][bi][0] == nullptr ||
               kn.dq_half[ci][bi][1] == nullptr)
            : (kn.dkdv[ci][bi] == nullptr || kn.dq[ci][bi] == nullptr))
    return 1;
  const int64_t rows = a.BH * a.Nq;
  if (rows > 0) {
    const int64_t rpb = kn.delta_rows_per_block;
    const int64_t want = (rows + rpb - 1) / rpb;
    const unsigned grid = (unsigned)(want < (1 << 20) ? want : (1 << 20));
    const uint16_t* o = static_cast<const uint16_t*>(a.O);
    const uint16_t* g = static_cast<const uint16_t*>(a.dO);
    float* dl = a.Dws;
    int64_t n = rows;
    void* args[] = {&o, &g, &dl, &n};
    if (hipLaunchKernel(kn.delta, dim3(grid), dim3(256), args, 0, stream) != hipSuccess) return 1;
  }
  const float c_log2 = (float)((double)a.scale * 1.4426950408889634074);
  const uint16_t* q = static_cast<const uint16_t*>(a.Q);
  const uint16_t* k = static_cast<const uint16_t*>(a.K);
  const uint16_t* v = static_cast<const uint16_t*>(a.V);
  const uint16_t* g = static_cast<const uint16_t*>(a.dO);
  const float* lse = a.LSE;
  const float* dl = a.Dws;
  int nq = (int)a.Nq, nk = (int)a.Nk;
  float cl = c_log2, sc = a.scale;
  const float* bias = a.bias;
  int64_t sb = a.bias_sb, sh = a.bias_sh, sq = a.bias_sq;
  int heads = (int)a.H;
  {
    int n_kt = (int)((a.Nk + KV_KEYS - 1) / KV_KEYS);
    uint16_t* dk = static_cast<uint16_t*>(a.dK);
    uint16_t* dv = static_cast<uint16_t*>(a.dV);
    void* args[] = {&q, &k, &v, &g, &lse, &dl, &dk, &dv, &nq, &nk, &n_kt, &cl, &sc, &bias, &sb, &sh, &sq, &heads};
    if (split) {
      // one launch per gradient (head size 256)
      if (hipLaunchKernel(kn.dkdv_dv[ci][bi], dim3((unsigned)(a.BH * n_kt)), dim3(NTHREADS), args, 0, stream) !=
              hipSuccess ||
          hipLaunchKernel(kn.dkdv_dk[ci][bi], dim3((unsigned)(a.BH * n_kt)), dim3(NTHREADS), args, 0, stream) !=
              hipSuccess)
        return 1;
    } else if (hipLaunchKernel(kn.dkdv[ci][bi], dim3((unsigned)(a.BH * n_kt)), dim3(NTHREADS), args, 0, stream) !=
               hipSuccess) {
      return 1;
    }
  }
  if (rows > 0) {
    int n_qt = (int)((a.Nq + DQ_ROWS - 1) / DQ_ROWS);
    uint16_t* dq = static_cast<uint16_t*>(a.dQ);
    void* args[] = {&q, &k, &v, &g, &lse, &dl, &dq, &nq, &nk, &n_qt, &cl, &sc, &bias, &sb, &sh, &sq, &heads};
    if (split) {
      // one launch per half of the dQ columns (head size 256)
      for (int hf = 0; hf < 2; ++hf)
        if (hipLaunchKernel(kn.dq_half[ci][bi][hf], dim3((unsigned)(a.BH * n_qt)), dim3(NTHREADS), args, 0, stream) !=
            hipSuccess)
          return 1;
    } else if (hipLaunchKernel(kn.dq[ci][bi], dim3((unsigned)(a.BH * n_qt)), dim3(NTHREADS), args, 0, stream) !=
               hipSuccess) {
      return 1;
    }
  }
  return 0;
}

const char* bwd_config_string() {
  return "gfx950 fa_bwd v7: delta kernel; dK/dV kernel (128 keys per workgroup, 32 per wave, query blocks of 64, "
         "K and V in registers); dQ kernel (128 rows per workgroup, 64-key tiles); in-wave MFMA/VALU interleave "
         "(causal at d=128 too); two tiles per loop trip at d=128 for the causal dK/dV and the bias dQ kernels; "
         "LDS fragments read 2-3 MFMAs ahead at d=128; "
         "two waves per SIMD at head size 64; at head size 256 one dK/dV launch per gradient "
         "and one dQ launch per column half (bias too); "
         "head sizes 64, 128, 192/128, 256; "
         "fp32 bias; no atomics";
}

}  // namespace fa06

// fa_fwd_kernel.hip -- gfx950 (CDNA4) fused attention forward kernel.
//
// Computes O = softmax_row(scale * Q K^T) V and the per-row log-sum-exp for
// BF16 Q/K/V ("FlashAttention'ı Anlamak Bölüm 1", section 0.2, score and
// output equations): Q and K rows of head size d, V and O rows of d_v,
// (d, d_v) one of (64, 64), (128, 128), (256, 256) and (192, 128).  The
// headline shape is d = d_v = 128.
//
// Work partition (B200 article, section "Kernel işini nasıl
// bölümlendiriyor"): one workgroup per tile of BR query rows of one
// (batch, head); the Q tile is loaded once; the workgroup then walks the K/V
// sequence in tiles of BC keys, computing scores, updating the online
// softmax state (row max and row sum) and accumulating P V in registers; the
// accumulator is normalised once after the loop and written.
//
// MI355X mapping:
//   * 32 query rows per wave.  4 waves per workgroup, 2 workgroups per CU
//     (3 for the head-size-64 bias variant, 1 at head size 256); for the
//     plain head-size-128 kernel on grids that fill the chip, 8 waves per
//     workgroup and 1 workgroup per CU, so each K/V tile copied into LDS
//     serves 256 query rows (half the copies per FLOP), with the iteration
//     laid out as 32 fixed segments (below).
//   * Scores are produced transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (K is the A operand from LDS, Q^T the B operand
//     held in registers for the whole loop).  The accumulator then gives each
//     lane one query and 16 keys, so row max / row sum are in-lane reductions
//     plus one exchange between the two 32-lane halves, and the same
//     registers, rounded to bf16, are directly the B operand of
//     O^T += V^T P^T.  The key order inside an MFMA k-step is permuted
//     consistently on both operands (the contraction does not depend on it).
//     At head size 128 the K fragments are read from LDS two k-steps ahead
//     of the MFMAs that use them.
//   * V^T fragments come from the row-major V tile in LDS through
//     ds_read_b64_tr_b16 (a transposing LDS read), so V is never transposed
//     in memory.
//   * K/V tiles are double buffered in LDS and copied global -> LDS directly
//     (buffer loads with the LDS destination, no registers) while the
//     previous tiles are computed (the multi-stage pipeline of the 5090
//     article's "v3").  Inside a wave the work is software pipelined over
//     three tiles: iteration j computes the scores of tile j+2 and P V of
//     tile j on the MFMAs while the VALU runs the softmax of tile j+1, so
//     the exponentials overlap the matrix products of the same wave.
//   * LDS rows are 2*d (K) and 2*d_v (V) bytes; 16-byte chunks are
//     XOR-swizzled per row so the K fragment reads (ds_read_b128) and the V
//     transposing reads are free of bank conflicts (the swizzled shared
//     memory of the 5090 article's "v2", re-derived for the gfx950 LDS).
//   * The softmax scale is folded into exp2 as scale*log2(e).  The running
//     max is only raised when it has to be; otherwise the stale max is kept,
//     which is exact because the same max enters P, the row sum and the
//     output.  Tiles without a mask or bias do not even compute their max:
//     P = exp2(s*scale*log2(e) - m) uses the running max as it stands (bf16 P
//     has fp32's exponent range), and only when a lane's tile sum exceeds
//     2^16 (or is inf or NaN: the first tile, or a row that has only seen
//     -inf bias) is the tile recomputed with its max.  Tiles with a bias do
//     the same on their logits.  Masked tiles (causal diagonal, ragged end)
//     raise the max when the tile's exceeds it by more than RESCALE_SLACK.
//     This removes almost all O rescaling and most max reductions.
//   * Global accesses use buffer resources sized to each (batch, head)
//     slice: rows past Nq / Nk read as zero and stores past Nq are dropped,
//     so ragged sequence lengths need no special load or store paths.
//   * Workgroup ids are remapped so the q-tiles of one head run on the same
//     XCD (workgroups are dispatched round-robin over the 8 XCDs), sharing
//     that head's K/V in the XCD's L2.
//   * Mask term of the score equation, two forms: causal (a q-tile stops at
//     the last K/V tile its last row can see, only tiles that cross the
//     diagonal are masked per key, and the q-tiles with the most work are
//     dispatched first) and an fp32 additive bias with arbitrary broadcast
//     strides, read straight from memory into registers one tile ahead.
//   * Key split (SPLIT): workgroup (head, range, q-tile) attends to one range
//     of keys and writes fp32 partial results; fa_fwd_merge_kernel combines
//     the ranges (for launches with fewer than two workgroups per CU).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernel.h"

namespace fa06 {
namespace {

constexpr int BR = 128;         // query rows per 4-wave workgroup (8 waves: 256)
// LDS: the Q tile (BR rows, staged once) and K and V tiles of BC keys, two of
// each (K(j+2), K(j+3), V(j), V(j+1)): 64 KiB at head size 128 and BC = 64,
// 80 KiB at (d, d_v) = (192, 128), either way room for two workgroups per
// CU (160 KiB).
constexpr int lds_bytes(int bc, int dqk, int dv) {
  return 2 * bc * 2 * (dqk + dv) > BR * 2 * dqk ? 2 * bc * 2 * (dqk + dv) : BR * 2 * dqk;
}
// Waves per SIMD the register budget allows: head size 256 keeps a 32x256
// fp32 output accumulator (128 registers) per wave and runs one wave.  At
// head size 64 the bias variant (32-key tiles, 16 KiB of LDS) fits three
// waves' registers (<= 168, no spills): +12 % there.  The other head-size-64
// variants would spill at three waves and gain nothing, so they keep two.
constexpr int waves_per_simd(int dqk, int dv, bool bias) {
  return dqk == 256 || dv == 256 ? 1 : (dqk == 64 && bias ? 3 : 2);
}
constexpr float RESCALE_SLACK = 8.0f;        // log2 units: P stays <= 256

// One workgroup computes BR query rows of one (batch, head) against all keys.
//   BC        keys per K/V tile (64; 32 for the bias variant, whose bias
//             tiles live in registers)
//   NEG_SCALE the scale is negative: the largest logit is the smallest score
//   CAUSAL    key j is hidden from query i when j > i + (Nk - Nq); tiles past
//             a q-tile's diagonal are skipped, tiles crossing it are masked
//   BIAS      an fp32 bias is added to the scaled scores:
//             bias[b*sb + h*sh + i*sq + j] (element strides)
//   DQK, DV   head sizes of Q/K and of V/O
//   SPLIT     the keys are split into n_splits ranges of split_keys keys (a
//             multiple of BC); workgroup (head, split, q-tile) attends to its
//             range only and writes the range's normalised output in fp32
//             to Opart [n_splits, B*H, Nq, DV] and its log-sum-exp to Lpart
//             [n_splits, B*H, Nq]; a merge kernel combines the ranges
//   NW        waves per workgroup: 4, or 8 for the plain head-size-128 kernel
//             (SEG below), whose workgroups cover 256 query rows
//   KS2       (8 waves only) two groups of 4 waves attend to the two halves
//             of the key tiles for the same 128 query rows and combine their
//             results through LDS at the end: the key split inside one
//             workgroup, for launches with one 128-row workgroup per CU
template <int DQK, int DV, int BC, bool NEG_SCALE, bool CAUSAL, bool BIAS, bool SPLIT, int NW = 4, bool KS2 = false>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(waves_per_simd(DQK, DV, BIAS), waves_per_simd(DQK, DV, BIAS))))
fa_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
              const float* __restrict__ bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_sq, int H,
              int Nq, int Nk_all, int n_qtiles, float c_log2, float* __restrict__ Opart,
              float* __restrict__ Lpart, int split_keys, int n_splits) {
  // SEG: 8 waves share each K/V tile (SEG_ITER below: plain tiles run the
  // segmented iteration, iteration_seg: one MFMA per segment, the 16 of
  // S(j+2), then the 16 of P(j) V(j)... see there; with the causal mask the
  // tiles on the diagonal keep the masked iteration).
  constexpr bool SEG = NW == 8;
  // The segmented iteration also runs the plain tiles of the 4-wave head-size-
  // 128 kernels without a bias (including the key split): +6.5 % on a grid
  // of one workgroup per CU (B=1, H=8, Nq=4096, Nk=8192), identical results.
  // At head size 64 (16 MFMAs per tile, two scores per segment): +2 % at
  // B=2, H=32, N=8192 and +3 % at B=1, H=16, Nq=4096, Nk=8192.  With the
  // causal mask (the tiles below the diagonal; causal launches of 8192 rows
  // or more run 8 waves): +4 to +5.5 % at 2048 and 4096 rows, +3 % at head
  // size 64 and 8192 rows.  With a bias at head size 128 (32-key tiles: 16
  // MFMAs and 16 scores per tile, one score per segment): +9 % with a per-key
  // bias at B=2, H=16, N=8192 (causal +6 %), +20 % at B=1, H=8, Nq=4096,
  // Nk=8192.  At head size 64 with a bias (three waves per SIMD) it would
  // spill 21-29 registers.  Head sizes 192 and 256 have no whole number of
  // scores per segment (32 over 40 segments, 16 over 32): the scores are
  // spread as evenly as whole scores allow.  (192, 128): +7.6 % at B=2, H=16,
  // N=8192, +16 % with a per-key bias, +20 % causal with it; causal without
  // a bias (64-key tiles) it spills 37 registers (-12 %) and keeps the plain
  // iteration.  256: +30 % (causal +28 %), +14 % with a bias (causal +37 %).
  constexpr bool SEG_ITER = (((DQK == 64 && DV == 64) || (DQK == 128 && DV == 128)) && BC == 64 && !BIAS) ||
                            (DQK == 128 && DV == 128 && BC == 32 && BIAS) || (DQK == 192 && DV == 128 && (BIAS || !CAUSAL)) ||
                            (DQK == 256 && DV == 256) || SEG;
  static_assert(NW == 4 || (NW == 8 && DQK == 128 && DV == 128 && BC == 64 && !BIAS && !(SPLIT && CAUSAL)) ||
                    (NW == 8 && DQK == 64 && DV == 64 && BC == 64 && !BIAS && !CAUSAL && !SPLIT && !KS2),
                "8-wave workgroups: head size 128 without bias (key split: no mask), 64 without mask or bias");
  static_assert(!KS2 || (NW == 8 && !SPLIT && !BIAS), "the in-workgroup key split: 8 waves, no bias, no split");
  constexpr int NWR = KS2 ? NW / 2 : NW;      // waves per key group (all waves without KS2)
  constexpr int BR = 32 * NWR;                // query rows per workgroup
  constexpr int KB = BC / 32;                 // 32-key MFMA blocks per tile
  constexpr int RBQ = 2 * DQK;                // bytes per Q or K row
  constexpr int RBV = 2 * DV;                 // bytes per V or O row
  constexpr int NT = DQK / 16;                // 16-wide k steps over the Q/K head size
  constexpr int NCB = DV / 32;                // 32-column blocks of the output
  constexpr int K_TILE = BC * RBQ;            // one K tile
  constexpr int V_TILE = BC * RBV;            // one V tile
  __shared__ __attribute__((aligned(1024))) char smem[SEG ? 1024 : lds_bytes(BC, DQK, DV)];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;   // query column of the S^T / O^T accumulators
  const int h = lane >> 5;   // half of the wave
  const int wr = KS2 ? (wave & (NWR - 1)) : wave;  // which 32 rows of the workgroup
  const int kg_u = KS2 ? __builtin_amdgcn_readfirstlane(wave / NWR) : 0;  // key group (KS2)

  // XCD-aware remap: consecutive logical tiles (same head) go to one XCD.
  const int nblk = gridDim.x;
  int bh, qt, split = 0;
  if constexpr (SPLIT) {
    // logical order (head, split, q-tile): the q-tiles of one key range of
    // one head are consecutive, so they share that range in one XCD's L2
    int bid = blockIdx.x;
    const int nfull = nblk & ~7;
    if (bid < nfull) bid = (bid & 7) * (nfull >> 3) + (bid >> 3);
    const int per_bh = n_splits * n_qtiles;
    bh = bid / per_bh;
    const int rem = bid - bh * per_bh;
    split = rem / n_qtiles;
    qt = rem - split * n_qtiles;
  } else if constexpr (BIAS) {
    // heads that share dense bias rows run side by side (one bias fetch)
    const HeadGroup hg = bias_head_group(nblk / (n_qtiles * H), H, bias_sb, bias_sh, bias_sq);
    grouped_tile_map(blockIdx.x, nblk, n_qtiles, CAUSAL, hg, bh, qt);
  } else if constexpr (CAUSAL) {
    xcd_tile_map(blockIdx.x, nblk, n_qtiles, true, bh, qt);
  } else {
    // consecutive logical tiles (same head) go to one XCD
    int bid = blockIdx.x;
    const int nfull = nblk & ~7;
    if (bid < nfull) bid = (bid & 7) * (nfull >> 3) + (bid >> 3);
    bh = bid / n_qtiles;
    qt = bid - bh * n_qtiles;
  }
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // the longest rows of a head start first
  const int q0 = qt * BR;
  // this workgroup's keys: [k0, k0 + Nk) of the head's Nk_all
  // KS2: group g takes key tiles [g*G, (g+1)*G) of the tiles the q-tile
  // sees (all ceil(Nk/BC); with the causal mask those up to its last row's
  // diagonal), G = half of them rounded up; both groups run G iterations
  // (the second group's last one may lie past the visible keys: fully
  // masked, all weights 0), so every barrier is reached by all waves
  int ks_tiles = 0;
  if constexpr (KS2) {
    int total = (Nk_all + BC - 1) / BC;
    if constexpr (CAUSAL) {
      const int lim_last = (q0 + BR < Nq ? q0 + BR : Nq) - 1 + Nk_all - Nq;
      const int need = lim_last < 0 ? 0 : lim_last / BC + 1;
      total = need < total ? need : total;
    }
    ks_tiles = (total + 1) / 2;
  }
  const int k0 = SPLIT ? split * split_keys : (KS2 ? kg_u * ks_tiles * BC : 0);
  int Nk = SPLIT ? (Nk_all - k0 < split_keys ? Nk_all - k0 : split_keys) : Nk_all;
  if constexpr (KS2) Nk = Nk_all - k0 <= 0 ? 0 : (Nk_all - k0 < ks_tiles * BC ? Nk_all - k0 : ks_tiles * BC);
  // output rows: the head's O / LSE, or this range's slice of the partials
  const int BH = SPLIT ? nblk / (n_splits * n_qtiles) : 0;
  const size_t orow0 = SPLIT ? ((size_t)split * (size_t)BH + (size_t)bh) * (size_t)Nq : (size_t)bh * (size_t)Nq;

  const size_t bhs = (size_t)bh;
  const size_t kv_row0 = bhs * (size_t)Nk_all + (size_t)k0;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + bhs * (size_t)Nq * DQK, (uint32_t)Nq * RBQ);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + kv_row0 * DQK, (uint32_t)Nk * RBQ);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + kv_row0 * DV, (uint32_t)Nk * RBV);
  const __amdgpu_buffer_rsrc_t ro = SPLIT ? make_rsrc(Opart + orow0 * DV, (uint32_t)Nq * (uint32_t)(4 * DV))
                                          : make_rsrc(O + orow0 * DV, (uint32_t)Nq * RBV);
  float* const lse_out = SPLIT ? Lpart : LSE;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wr_u = __builtin_amdgcn_readfirstlane(wr);
  const int n_full = Nk / BC;  // tiles with BC valid keys
  int n_tiles = KS2 ? ks_tiles : n_full + (Nk % BC != 0);
  int first_masked = n_full;   // first tile that needs per-key masks
  // last key visible to this lane's query row (keys above it are masked)
  int key_lim = Nk - 1;
  if constexpr (CAUSAL) {
    const int off = Nk_all - k0 - Nq;  // key k0 + j is hidden from query i when j > i + off
    const int q_last = (q0 + BR < Nq ? q0 + BR : Nq) - 1;
    const int lim_last = q_last + off;  // the q-tile's last row sees keys <= lim_last
    const int lim_first = q0 + off;     // its first row sees keys <= lim_first
    const int need = lim_last < 0 ? 0 : lim_last / BC + 1;
    if constexpr (!KS2) n_tiles = need < n_tiles ? need : n_tiles;  // KS2: G for both groups
    const int unmasked = lim_first + 1 <= 0 ? 0 : (lim_first + 1) / BC;
    first_masked = unmasked < first_masked ? unmasked : first_masked;
    const int my_lim = q0 + wr * 32 + c + off;
    key_lim = my_lim < key_lim ? my_lim : key_lim;
    if (n_tiles == 0) {
      // no row of this q-tile sees any key: O = 0, LSE = -inf (KS2: both
      // groups come here together and write the same zeros)
      const int q = q0 + wr * 32 + c;
      constexpr uint32_t ORB = SPLIT ? 4 * DV : RBV;  // bytes per output row
#pragma unroll
      for (int i = 0; i < (int)ORB / 32; ++i)  // this lane's half row: bytes [ORB/2*h, ORB/2*(h+1))
        __builtin_amdgcn_raw_buffer_store_b128(uintx4{0u, 0u, 0u, 0u}, ro,
                                               (uint32_t)q * ORB + ORB / 2 * (uint32_t)h + 16u * (uint32_t)i, 0, 0);
      if (h == 0 && q < Nq) lse_out[orow0 + q] = -__builtin_inff();
      return;
    }
  }

  // Bias rows of this wave's 32 queries, read straight into registers: lane
  // (c, h) needs, per 32-key block, keys 8g + 4h .. 8g + 4h + 3 (g = 0..3) of
  // row q0 + 32*wave + c, i.e. four 16-byte loads.  The buffer ends at the
  // last key of the wave's last valid row, so keys past Nk (and rows past
  // Nq) read as zero; they are masked anyway.
  __amdgpu_buffer_rsrc_t rb = make_rsrc(nullptr, 0u);
  uint32_t bias_voff = 0;
  if constexpr (BIAS) {
    const int b = bh / H;
    const int hd = bh - b * H;
    // wave_u, not wave: the resource must be provably wave-uniform, or the
    // compiler wraps every load in a loop over the distinct descriptors
    const int qw0 = q0 + wr_u * 32;
    const int nrows = Nq - qw0 < 32 ? Nq - qw0 : 32;
    const float* base = bias + (int64_t)b * bias_sb + (int64_t)hd * bias_sh + (int64_t)qw0 * bias_sq + k0;
    const uint32_t bytes = nrows > 0 ? (uint32_t)(((int64_t)(nrows - 1) * bias_sq + Nk) * 4) : 0u;
    rb = make_rsrc(base, bytes);
    bias_voff = (uint32_t)((int64_t)c * bias_sq * 4) + 16u * (uint32_t)h;
  }
  auto load_bias = [&](int t, floatx4 (&bt)[KB][4]) FA_INLINE {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)t * (uint32_t)(BC * 4));
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        bt[kb][g] = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rb, bias_voff + (uint32_t)(kb * 128 + g * 32), soff, 0));
  };

  // LDS: two K buffers then two V buffers.  K runs two tiles ahead of V:
  // iteration j computes the scores of tile j+2 and accumulates P V of tile
  // j, so K(j+2) and V(j) are read while K(j+3) and V(j+1) are copied in.
  // With SEG each buffer is its own LDS array: every loop body reads one
  // buffer while the LDS-direct copies fill another, and as distinct objects
  // the compiler can tell that the reads need not wait for those copies.
  // (KS2: one K_TILE / V_TILE per key group in each array)
  constexpr int NKG = KS2 ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char seg_k0[SEG ? NKG * K_TILE : 16];
  __shared__ __attribute__((aligned(1024))) char seg_k1[SEG ? NKG * K_TILE : 16];
  __shared__ __attribute__((aligned(1024))) char seg_v0[SEG ? NKG * V_TILE : 16];
  __shared__ __attribute__((aligned(1024))) char seg_v1[SEG ? NKG * V_TILE : 16];
  auto kbuf = [&](int i) FA_INLINE -> char* {
    if constexpr (KS2) return (i ? seg_k1 : seg_k0) + kg_u * K_TILE;
    else if constexpr (SEG) return i ? seg_k1 : seg_k0;
    else return smem + i * K_TILE;
  };
  auto vbuf = [&](int i) FA_INLINE -> char* {
    if constexpr (KS2) return (i ? seg_v1 : seg_v0) + kg_u * V_TILE;
    else if constexpr (SEG) return i ? seg_v1 : seg_v0;
    else return smem + 2 * K_TILE + i * V_TILE;
  };

  // ---- prologue: the Q tile through LDS into registers.
  bf16x8 qb[NT];  // qb[t]: Q[q0 + wave*32 + c][16t + 8h .. +7]
  if constexpr (KS2) {
    // 128 rows in two 64-row pieces (the first K buffers), read by both groups
    tile_to_lds<64, SWZ_ROW, DQK, NW>(rq, q0, seg_k0, wave_u, lane);
    tile_to_lds<64, SWZ_ROW, DQK, NW>(rq, q0 + 64, seg_k1, wave_u, lane);
    wait_vmem();
    __syncthreads();
    const char* qs = (wr_u >> 1) == 0 ? seg_k0 : seg_k1;
    const uint32_t row = (wr_u & 1) * 32 + c;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      qb[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(qs + swz<SWZ_ROW, DQK>(row, 2 * t + h)));
  } else if constexpr (SEG) {
    // 256 rows in four 64-row pieces, one per K/V buffer
    tile_to_lds<64, SWZ_ROW, DQK, NW>(rq, q0, kbuf(0), wave_u, lane);
    tile_to_lds<64, SWZ_ROW, DQK, NW>(rq, q0 + 64, kbuf(1), wave_u, lane);
    tile_to_lds<64, SWZ_ROW, DQK, NW>(rq, q0 + 128, vbuf(0), wave_u, lane);
    tile_to_lds<64, SWZ_ROW, DQK, NW>(rq, q0 + 192, vbuf(1), wave_u, lane);
    wait_vmem();
    __syncthreads();
    const int piece = wave_u >> 1;
    const char* qs = piece == 0 ? kbuf(0) : piece == 1 ? kbuf(1) : piece == 2 ? vbuf(0) : vbuf(1);
    const uint32_t row = (wave_u & 1) * 32 + c;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      qb[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(qs + swz<SWZ_ROW, DQK>(row, 2 * t + h)));
  } else {
    tile_to_lds<BR, SWZ_ROW, DQK>(rq, q0, smem, wave_u, lane);
    wait_vmem();
    __syncthreads();
    const uint32_t row = wave * 32 + c;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      qb[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(smem + swz<SWZ_ROW, DQK>(row, 2 * t + h)));
  }
  __syncthreads();  // the Q staging area is reused from here on
  tile_to_lds<BC, SWZ_ROW, DQK, NWR>(rk, 0, kbuf(0), wr_u, lane);
  if (n_tiles > 1) tile_to_lds<BC, SWZ_ROW, DQK, NWR>(rk, BC, kbuf(1), wr_u, lane);
  tile_to_lds<BC, SWZ_TR, DV, NWR>(rv, 0, vbuf(0), wr_u, lane);
  floatx4 b0[KB][4], bcur[KB][4];  // bias of tile 0 / of the tile whose softmax is next
  if constexpr (BIAS) {
    load_bias(0, b0);
    if (n_tiles > 1) load_bias(1, bcur);
  }
  wait_vmem();
  __syncthreads();

  floatx16 oacc[NCB];
#pragma unroll
  for (int i = 0; i < NCB; ++i) oacc[i] = floatx16{};
  float m_run = -__builtin_inff();  // running max, log2 units, per query
  float l_run = 0.0f;               // partial row sum of this lane's keys (fp32 P, for LSE)
  float l_rnd = 0.0f;               // the same over the bf16-rounded P (normalises O)
  // With RSUM_MFMA the rounded-P sum is taken on the matrix core instead of
  // with bf16 dot products (each of which holds the SIMD about as long as
  // half an MFMA): next to each P V product, a 16x16x32 product of a 0/1 mask
  // with the same P fragment.  That product reads the fragment's lane
  // n + 16 g as column n % 16, k group g; the query of lane L is L % 32, so
  // mask row 0 (and 8) over the even groups sums query n and row 4 (and 12)
  // over the odd groups query n + 16.  Output register 0 of lane L is then
  // the rounded sum of query L % 32 over every key so far (registers 1-3
  // stay 0): it accumulates and is rescaled exactly as O is.  Off where its
  // 8 registers make the kernel spill much more: head size 256 with a bias,
  // and (192, 128) without mask or bias (-17 % there; +3-6 % elsewhere).
  constexpr bool RSUM_MFMA = !(DQK == 256 && BIAS) && !(DQK == 192 && !CAUSAL && !BIAS);
  floatx4 lt{0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 rmask;
  {
    const __bf16 one = ((lane & 3) == 0 && ((lane >> 2) & 1) == ((lane >> 4) & 1)) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) rmask[i] = one;
  }

  // S^T = K Q^T for the BC keys of one K buffer (32-key blocks).
  // The K fragments of k step t + KPF are read before the MFMAs of step t
  // (a ring of KPF + 1 fragment sets): written in this order, the
  // scheduler keeps the LDS reads further ahead of their use than it does
  // for a read-then-multiply loop (1.3-1.5 % at head size 128, 1.2 % at
  // (192, 128) without mask or bias; identical results).  Elsewhere KPF = 0
  // (read, then multiply): there the ring costs registers that are not
  // there (the causal (192, 128) kernel spills more and runs 22 % slower).
  constexpr int KPF = DQK == 128 && DV == 128 ? 2 : (DQK == 192 && !CAUSAL && !BIAS ? 1 : 0);
  auto scores = [&](const char* ks, floatx16 (&s)[KB]) FA_INLINE {
    auto kfrag = [&](int kb, int t) FA_INLINE {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(ks + swz<SWZ_ROW, DQK>(kb * 32 + c, 2 * t + h)));
    };
    if constexpr (KPF == 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = floatx16{};
#pragma unroll
        for (int t = 0; t < NT; ++t) s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(kb, t), qb[t], s[kb], 0, 0, 0);
      }
    } else {
      bf16x8 fr[KPF + 1][KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) s[kb] = floatx16{};
#pragma unroll
      for (int t = 0; t < KPF; ++t)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) fr[t][kb] = kfrag(kb, t);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (t + KPF < NT) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) fr[(t + KPF) % (KPF + 1)][kb] = kfrag(kb, t + KPF);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[t % (KPF + 1)][kb], qb[t], s[kb], 0, 0, 0);
      }
    }
  };

  // Row sum of one tile's P as rounded to bf16, i.e. of the weights the P V
  // product actually uses (where RSUM_MFMA is off).  O is divided by this sum, so the weights of every
  // output row sum to 1 whatever the rounding of P; the fp32 sum of the
  // unrounded P (l_run) gives the log-sum-exp.  With the running max kept
  // stale, the largest P of a row is no longer exactly 1 and carries a bf16
  // rounding error; dividing by the unrounded sum would leave that error
  // (up to 2^-8 of |v|) in the output.
  auto rounded_sum = [&](const bf16x8 (&pb)[2 * KB]) FA_INLINE -> float {
    if constexpr (RSUM_MFMA) return 0.0f;
    float acc = 0.0f;
    const bf16x2 one{(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int i = 0; i < 2 * KB; ++i) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 0, 1), one, acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 2, 3), one, acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 4, 5), one, acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i], pb[i], 6, 7), one, acc, false);
    }
    return acc;
  };

  // Online softmax of one tile's scores -> P (bf16, the B operand of the
  // P V product).  The decision to raise the running max is wave uniform
  // (ballot); returns the factor the output accumulator must be multiplied
  // by before the next P V is added (1 when unchanged).  MASK tiles hide the
  // keys above `lim` (this row's last visible key, relative to the tile's
  // first key).
  auto softmax = [&](floatx16 (&s)[KB], const floatx4 (&bt)[KB][4], bf16x8 (&pb)[2 * KB], int lim,
                     auto mask_tag, bool& rescale) FA_INLINE -> float {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr bool CAN_BE_EMPTY = CAUSAL || BIAS || KS2;  // a row may see no key (yet)
    // LOGIT: the tile's scores are first turned into log2-domain logits t
    // (bias added, hidden keys set to -inf), so the max and the exponent use
    // t directly and a hidden key gives exp2(-inf) = 0 whatever the scale
    // (-inf * scale would be NaN for a zero scale).  Unmasked tiles without
    // a bias keep the raw scores and fold the scale into one fma.
    constexpr bool LOGIT = BIAS || MASK;
    float m_tile;
    if constexpr (LOGIT) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t;
          if constexpr (BIAS)
            t = __builtin_fmaf(s[kb][r], c_log2, bt[kb][r >> 2][r & 3] * LOG2E);
          else
            t = s[kb][r] * c_log2;
          if constexpr (MASK) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key > lim) t = -__builtin_inff();
          }
          s[kb][r] = t;
        }
      float ext = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ext = fmaxf(ext, s[kb][r]);
      m_tile = wave_max_halves(ext);
    } else {
      float ext = s[0][0];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ext = NEG_SCALE ? fminf(ext, s[kb][r]) : fmaxf(ext, s[kb][r]);
      ext = NEG_SCALE ? wave_min_halves(ext) : wave_max_halves(ext);
      m_tile = ext * c_log2;
    }
    rescale = __ballot(m_tile > m_run + RESCALE_SLACK) != 0;
    const float m_new = rescale ? fmaxf(m_run, m_tile) : m_run;
    float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    // a row that has seen no key yet keeps m = -inf, l = 0 and O = 0; it
    // subtracts 0 instead, so its hidden keys give exp2(-inf) = 0, not NaN
    float m_use = m_new;
    if constexpr (CAN_BE_EMPTY) {
      const bool empty = m_new == -__builtin_inff();
      alpha = empty ? 1.0f : alpha;
      m_use = empty ? 0.0f : m_new;
    }
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = LOGIT ? s[kb][r] - m_use : __builtin_fmaf(s[kb][r], c_log2, -m_use);
        const float p = __builtin_amdgcn_exp2f(x);
        lsum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + lsum;
    l_rnd = l_rnd * alpha + rounded_sum(pb);
    return alpha;
  };

  // O^T += V^T P^T for the BC keys of one V buffer: 4 d-blocks x 2*KB key steps.
  auto accumulate = [&](const char* vs, const bf16x8 (&pb)[2 * KB]) FA_INLINE {
    const int g = lane >> 4;          // 16-lane group
    const int i16 = lane & 15;
    const int sub = i16 >> 2;         // which of the 4 keys this lane addresses
    const int q4 = i16 & 3;           // which 4-column piece of the 16 columns
    const int hh = g >> 1;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      const int d0 = cb * 32 + (g & 1) * 16 + q4 * 4;  // first of 4 d columns
      const uint32_t ch = (uint32_t)d0 >> 3;
      const uint32_t within = ((uint32_t)d0 & 7u) * 2u;
#pragma unroll
      for (int ks4 = 0; ks4 < 2 * KB; ++ks4) {
        const uint32_t r0 = ks4 * 16 + 4 * hh + sub;
        const uint32_t r1 = r0 + 8;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)((lds_char*)vs + swz<SWZ_TR, DV>(r0, ch) + within));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)((lds_char*)vs + swz<SWZ_TR, DV>(r1, ch) + within));
        // move the two 4-element results as whole dwords (no per-element
        // extraction): a = {lo[0..3], hi[0..3]}
        const uintx2 lo2 = __builtin_bit_cast(uintx2, lo);
        const uintx2 hi2 = __builtin_bit_cast(uintx2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, uintx4{lo2.x, lo2.y, hi2.x, hi2.y});
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks4], oacc[cb], 0, 0, 0);
        if (RSUM_MFMA && cb == NCB - 1) lt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rmask, pb[ks4], lt, 0, 0, 0);
      }
    }
  };

  // Plain tiles: P = exp2(s*c - m_run) with the running max as it stands, no
  // tile max.  bf16 P has fp32's exponent range, so this is exact as long as
  // the values stay moderate; a lane whose tile sum exceeds 2^16 (or is inf:
  // the first tile, m_run = -inf) sets `fix`, and the caller recomputes the
  // tile with a raised max (slow path, rare).
  auto softmax_fast = [&](const floatx16 (&s)[KB], bf16x8 (&pb)[2 * KB], float& lsum_out,
                          float& lrnd_out) FA_INLINE -> bool {
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_run));
        lsum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    lsum_out = lsum;
    lrnd_out = rounded_sum(pb);
    return __ballot(!(lsum <= 65536.0f)) != 0;
  };
  // slow path of a plain tile: raise the max to the tile's, recompute P
  auto softmax_fix = [&](const floatx16 (&s)[KB], bf16x8 (&pb)[2 * KB], float& lsum_out,
                         float& lrnd_out) FA_INLINE -> float {
    float ext = s[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ext = NEG_SCALE ? fminf(ext, s[kb][r]) : fmaxf(ext, s[kb][r]);
    ext = NEG_SCALE ? wave_min_halves(ext) : wave_max_halves(ext);
    const float m_new = fmaxf(m_run, ext * c_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_new));
        lsum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    lsum_out = lsum;
    lrnd_out = rounded_sum(pb);
    return alpha;
  };

  // The same for unmasked tiles with a bias.  At head size 64, P =
  // exp2(s*c + (b*log2(e) - m_run)) as two FMAs (+4 % with a per-key bias);
  // elsewhere the logits t = s*c + b*log2(e) and then exp2(t - m_run), the
  // form that measured faster there.  A row that has seen only -inf logits so
  // far (m_run = -inf) gives +inf or NaN, which sends the tile to the slow
  // path (softmax_fix_logits): it forms the logits and takes their max, and
  // rows that see only -inf keep P = 0 there.
  auto softmax_fast_bias = [&](const floatx16 (&s)[KB], const floatx4 (&bt)[KB][4], bf16x8 (&pb)[2 * KB],
                               float& lsum_out, float& lrnd_out) FA_INLINE -> bool {
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p;
        if constexpr (DQK == 64)
          p = __builtin_amdgcn_exp2f(
              __builtin_fmaf(s[kb][r], c_log2, __builtin_fmaf(bt[kb][r >> 2][r & 3], LOG2E, -m_run)));
        else
          p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, bt[kb][r >> 2][r & 3] * LOG2E) - m_run);
        lsum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    lsum_out = lsum;
    lrnd_out = rounded_sum(pb);
    return __ballot(!(lsum <= 65536.0f)) != 0;
  };
  auto softmax_fix_logits = [&](const floatx16 (&s)[KB], const floatx4 (&bt)[KB][4], bf16x8 (&pb)[2 * KB],
                                float& lsum_out, float& lrnd_out) FA_INLINE -> float {
    floatx16 t[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) t[kb][r] = __builtin_fmaf(s[kb][r], c_log2, bt[kb][r >> 2][r & 3] * LOG2E);
    float ext = t[0][0];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ext = fmaxf(ext, t[kb][r]);
    const float m_new = fmaxf(m_run, wave_max_halves(ext));
    const bool empty = m_new == -__builtin_inff();
    const float alpha = empty ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float m_use = empty ? 0.0f : m_new;
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(t[kb][r] - m_use);
        lsum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    lsum_out = lsum;
    lrnd_out = rounded_sum(pb);
    return alpha;
  };

  auto rescale_o = [&](float alpha) FA_INLINE {
#pragma unroll
    for (int i = 0; i < NCB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
    if constexpr (RSUM_MFMA) lt[0] *= alpha;
  };

  // ---- tiles 0 and 1: P(0) and S(1) before the loop.
  bf16x8 pb[2 * KB];  // P of the tile whose P V is next
  floatx16 s1[KB];    // scores of the tile whose softmax is next
  {
    floatx16 s0[KB];
    scores(kbuf(0), s0);
    bool rs;
    if (first_masked == 0)
      softmax(s0, b0, pb, key_lim, std::true_type{}, rs);
    else
      softmax(s0, b0, pb, key_lim, std::false_type{}, rs);
    // O is still zero: no rescale needed
    if (n_tiles > 1) scores(kbuf(1), s1);
  }
  __syncthreads();  // K(0) consumed: K(2) goes into its buffer
  if (n_tiles > 2) tile_to_lds<BC, SWZ_ROW, DQK, NWR>(rk, 2 * BC, kbuf(0), wr_u, lane);
  wait_vmem();
  __syncthreads();

  // Iteration j: three independent pieces of work, so the VALU softmax
  // overlaps the MFMAs of the same wave:
  //   S(j+2) = K(j+2) Q^T  (MFMA; K(j+2) in kbuf(j&1))      if HAS_S2
  //   softmax of tile j+1, scores computed one iteration earlier (VALU)
  //                                                         if HAS_S1
  //   O += P(j) V(j)       (MFMA; V(j) in vbuf(j&1))
  // while K(j+3) and V(j+1) are copied into the other buffers (and the bias
  // of tile j+2 into registers).  The output is rescaled after P(j) V(j),
  // before P(j+1) V(j+1) joins it.
  floatx4 bnext[KB][4];
  auto iteration = [&](int j, auto par_tag, auto has_s2_tag, auto has_s1_tag, auto mask1_tag) FA_INLINE {
    constexpr int P = decltype(par_tag)::value;  // == j & 1
    constexpr bool HAS_S2 = decltype(has_s2_tag)::value;
    constexpr bool HAS_S1 = decltype(has_s1_tag)::value;
    if (j + 3 < n_tiles) tile_to_lds<BC, SWZ_ROW, DQK, NWR>(rk, (j + 3) * BC, kbuf(P ^ 1), wr_u, lane);
    if constexpr (HAS_S1) tile_to_lds<BC, SWZ_TR, DV, NWR>(rv, (j + 1) * BC, vbuf(P ^ 1), wr_u, lane);
    if constexpr (BIAS && HAS_S2) load_bias(j + 2, bnext);
    floatx16 s2[KB];
    if constexpr (HAS_S2) scores(kbuf(P), s2);
    bf16x8 pn[2 * KB];
    bool rs = false;
    float alpha = 1.0f;
    // unmasked tiles take the fast path (no tile max), masked ones the max
    // path.  The causal (192, 128) kernel takes the max path everywhere: with
    // the fast path and its recompute branch next to the masked variant it
    // spills 11 registers instead of 7 and runs 21 % slower (at the other
    // head sizes the fast path wins by 3-5 %).
    constexpr bool FAST = !decltype(mask1_tag)::value && !(CAUSAL && DQK == 192 && !BIAS);
    float lsum_f = 0.0f, lrnd_f = 0.0f;
    bool fix = false;
    if constexpr (HAS_S1) {
      if constexpr (FAST && BIAS) fix = softmax_fast_bias(s1, bcur, pn, lsum_f, lrnd_f);
      else if constexpr (FAST) fix = softmax_fast(s1, pn, lsum_f, lrnd_f);
      else alpha = softmax(s1, bcur, pn, key_lim - (j + 1) * BC, mask1_tag, rs);
    }
    accumulate(vbuf(P), pb);
    if constexpr (HAS_S1) {
#pragma unroll
      for (int i = 0; i < 2 * KB; ++i) keep(pn[i]);
      if constexpr (FAST) {
        keep(lsum_f);
        keep(lrnd_f);
        if (fix) {
          if constexpr (BIAS) alpha = softmax_fix_logits(s1, bcur, pn, lsum_f, lrnd_f);
          else alpha = softmax_fix(s1, pn, lsum_f, lrnd_f);
          rs = true;
        }
        l_run = l_run * alpha + lsum_f;
        l_rnd = l_rnd * alpha + lrnd_f;
      }
      keep(l_run);
      keep(l_rnd);
      if (rs) rescale_o(alpha);
#pragma unroll
      for (int i = 0; i < 2 * KB; ++i) pb[i] = pn[i];
      if constexpr (HAS_S2) {
#pragma unroll
        for (int i = 0; i < KB; ++i) s1[i] = s2[i];
        if constexpr (BIAS) {
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) bcur[kb][g] = bnext[kb][g];
        }
      }
      wait_vmem();
      __syncthreads();
    }
  };

  // Iteration j on a plain tile with SEG_ITER: the same three pieces of work as
  // `iteration`, in a fixed order of scheduling segments, one MFMA each (32 at
  // head size 128 with 64-key tiles): the MFMAs of S(j+2), then those of
  // P(j) V(j) (those run on the V buffer the copies of this iteration do not
  // touch, and start late, after the copies have had half an iteration).
  // Segment i also reads the LDS operand of the MFMA PF segments later (a ring
  // of PF + 1 fragments per product) and advances the softmax of tile j+1:
  // the exponent of its scores of segment i + AHEAD + 1, the exponentials of
  // those of i + AHEAD and the row-sum adds of those of i + AHEAD - 1, each
  // step on results of the segment before, so that none waits for the
  // instruction just issued.  That is about four VALU instructions per MFMA:
  // about as much VALU work as an MFMA hides.  The compiler still places the
  // LDS waits, each for a read PF segments old.
  auto iteration_seg = [&](int j, auto par_tag) FA_INLINE {
    if constexpr (SEG_ITER) {
    constexpr int P = decltype(par_tag)::value;
    constexpr int PF = 3, AHEAD = 2;
    if (j + 3 < n_tiles) tile_to_lds<BC, SWZ_ROW, DQK, NWR>(rk, (j + 3) * BC, kbuf(P ^ 1), wr_u, lane);
    tile_to_lds<BC, SWZ_TR, DV, NWR>(rv, (j + 1) * BC, vbuf(P ^ 1), wr_u, lane);
    if constexpr (BIAS) load_bias(j + 2, bnext);
    const char* ks = kbuf(P);
    const char* vs = vbuf(P);
    // NS MFMAs of S (m < NS: key block m % KB, k step m / KB), then NP of
    // P V (NS + m: output block m % NCB, keys 16 (m / NCB) .. +15); SPS of
    // the lane's NSC scores per segment
    constexpr int NS = KB * NT, NP = NCB * (BC / 16), NM = NS + NP, NSC = 16 * KB, SPS = NSC / NM;
    // SPS_INT: SPS scores in every segment; else segment v's scores are
    // [sc0(v), sc0(v + 1)), spread as evenly as whole scores allow
    constexpr bool SPS_INT = SPS >= 1 && SPS * NM == NSC && (SPS == 1 || SPS % 2 == 0);
    constexpr int CSH = NCB == 8 ? 3 : (NCB == 4 ? 2 : 1);  // log2(NCB)
    static_assert(NCB == (1 << CSH), "output blocks");
    auto kfrag = [&](int m) FA_INLINE {
      return __builtin_bit_cast(bf16x8,
                                *reinterpret_cast<const uintx4*>(ks + swz<SWZ_ROW, DQK>((m % KB) * 32 + c, 2 * (m / KB) + h)));
    };
    auto vfrag = [&](int m) FA_INLINE {
      return tr_read_a<SWZ_TR, DV>(vs, (uint32_t)((m >> CSH) * 16), m & (NCB - 1), lane);
    };
    floatx16 s2[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s2[kb] = floatx16{};
    bf16x8 kf[PF + 1], vf[PF + 1], pn[2 * KB];
    float pe[NSC], xe[NSC];
    float lsum = 0.0f, lrnd = 0.0f;
    const bf16x2 one{(__bf16)1.0f, (__bf16)1.0f};
    // score r of this lane (key block r >> 4, row r & 15) in three steps, each
    // a segment after the one before, so that no VALU instruction waits for
    // the result of the one just issued: the exponent, the exponential, the
    // row sum
    auto st_fma = [&](int r) FA_INLINE {
      if (r >= NSC) return;
      if constexpr (BIAS)  // as in the plain iteration's fast path
        xe[r] = __builtin_fmaf(s1[r >> 4][r & 15], c_log2, bcur[r >> 4][(r & 15) >> 2][r & 3] * LOG2E) - m_run;
      else
        xe[r] = __builtin_fmaf(s1[r >> 4][r & 15], c_log2, -m_run);
    };
    auto st_exp = [&](int r) FA_INLINE {
      if (r < NSC) pe[r] = __builtin_amdgcn_exp2f(xe[r]);
    };
    auto st_add = [&](int r) FA_INLINE {
      if (r < NSC) lsum += pe[r];
    };
    auto pack = [&](int q) FA_INLINE {  // scores 2q, 2q + 1 -> bf16 (RNE), and their rounded sum
      const int r = 2 * q;
      const bf16x2 pr{(__bf16)pe[r], (__bf16)pe[r + 1]};
      pn[r >> 3][r & 7] = pr[0];
      pn[r >> 3][(r & 7) + 1] = pr[1];
      if constexpr (!RSUM_MFMA) lrnd = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lrnd, false);
    };
    auto sc0 = [](int v) FA_INLINE { return v <= 0 ? 0 : (v >= NM ? NSC : v * NSC / NM); };
#pragma unroll
    for (int i = 0; i < PF; ++i) kf[i] = kfrag(i);
#pragma unroll
    for (int r = 0; r < sc0(AHEAD + 1); ++r) st_fma(r);
#pragma unroll
    for (int r = 0; r < sc0(AHEAD); ++r) st_exp(r);
#pragma unroll
    for (int r = 0; r < sc0(AHEAD - 1); ++r) st_add(r);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      const int nxt = i + PF;  // the MFMA whose operand is read in this segment
      if (nxt < NS) kf[nxt % (PF + 1)] = kfrag(nxt);
      else if (nxt < NM) vf[(nxt - NS) % (PF + 1)] = vfrag(nxt - NS);
#pragma unroll
      for (int r = sc0(i + AHEAD + 1); r < sc0(i + AHEAD + 2); ++r) st_fma(r);
#pragma unroll
      for (int r = sc0(i + AHEAD); r < sc0(i + AHEAD + 1); ++r) st_exp(r);
#pragma unroll
      for (int r = sc0(i + AHEAD - 1); r < sc0(i + AHEAD); ++r) st_add(r);
      if constexpr (SPS_INT && SPS == 1) {
        if (i & 1) pack(i >> 1);
      } else if constexpr (SPS_INT) {
#pragma unroll
        for (int u = 0; u < SPS / 2; ++u) pack(i * (SPS / 2) + u);
      } else {
        // the pairs whose exponentials were all taken before this segment
#pragma unroll
        for (int q = sc0(i + AHEAD - 1) / 2; q < sc0(i + AHEAD) / 2; ++q) pack(q);
      }
      if (i < NS) {
        s2[i % KB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i % (PF + 1)], qb[i / KB], s2[i % KB], 0, 0, 0);
      } else {
        const int m = i - NS;
        oacc[m & (NCB - 1)] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[m % (PF + 1)], pb[m >> CSH], oacc[m & (NCB - 1)], 0, 0, 0);
        if (RSUM_MFMA && (m & (NCB - 1)) == NCB - 1)
          lt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rmask, pb[m >> CSH], lt, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // a lane's tile sum above 2^16 (or not finite): recompute with the max
    const bool fix = __ballot(!(lsum <= 65536.0f)) != 0;
#pragma unroll
    for (int i = 0; i < 2 * KB; ++i) keep(pn[i]);
    keep(lsum);
    keep(lrnd);
    float alpha = 1.0f;
    if (fix) {
      if constexpr (BIAS) alpha = softmax_fix_logits(s1, bcur, pn, lsum, lrnd);
      else alpha = softmax_fix(s1, pn, lsum, lrnd);
      rescale_o(alpha);
    }
    l_run = l_run * alpha + lsum;
    l_rnd = l_rnd * alpha + lrnd;
    keep(l_run);
    keep(l_rnd);
#pragma unroll
    for (int i = 0; i < 2 * KB; ++i) pb[i] = pn[i];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s1[kb] = s2[kb];
    if constexpr (BIAS) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) bcur[kb][g] = bnext[kb][g];
    }
    wait_vmem();
    __syncthreads();
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  // Iterations j in [j0, j1) with S(j+2) and the same masking of tile j+1;
  // the buffer parity (j & 1) is a compile-time constant of each
  // instantiation, so the loop is unrolled by two.
  auto run = [&](int j0, int j1, auto mask_tag) FA_INLINE {
    int j = j0;
    if (j < j1 && (j & 1)) {
      iteration(j, P1{}, T{}, T{}, mask_tag);
      ++j;
    }
    for (; j + 1 < j1; j += 2) {
      if constexpr (SEG_ITER && !decltype(mask_tag)::value) {
        iteration_seg(j, P0{});
        iteration_seg(j + 1, P1{});
      } else {
        iteration(j, P0{}, T{}, T{}, mask_tag);
        iteration(j + 1, P1{}, T{}, T{}, mask_tag);
      }
    }
    if (j < j1) iteration(j, P0{}, T{}, T{}, mask_tag);
  };
  // tile j+1 needs masks from first_masked on: at most the last tile
  // (ragged Nk) without CAUSAL, the tiles crossing the diagonal with it
  const int j_end = n_tiles - 2 > 0 ? n_tiles - 2 : 0;
  int j_split = first_masked - 1;
  j_split = j_split < 0 ? 0 : (j_split > j_end ? j_end : j_split);
  run(0, j_split, F{});
  // (KS2: the second group's range may end in a ragged and a fully masked tile)
  if constexpr (CAUSAL || KS2) run(j_split, j_end, T{});
  // iteration n_tiles-2: no S(j+2); the softmax of the last tile
  if (n_tiles >= 2) {
    const int j = n_tiles - 2;
    const bool mask = n_tiles - 1 >= first_masked;
    if (j & 1) {
      if (mask) iteration(j, P1{}, F{}, T{}, T{}); else iteration(j, P1{}, F{}, T{}, F{});
    } else {
      if (mask) iteration(j, P0{}, F{}, T{}, T{}); else iteration(j, P0{}, F{}, T{}, F{});
    }
  }
  // last iteration: P V of the last tile only
  if ((n_tiles - 1) & 1) iteration(n_tiles - 1, P1{}, F{}, F{}, F{}); else iteration(n_tiles - 1, P0{}, F{}, F{}, F{});

  // ---- epilogue: 1/l, bf16 (round to nearest even), LSE in natural log.
  float l_tot = wave_sum_halves(l_run);
  float l_rnd_tot = RSUM_MFMA ? lt[0] : wave_sum_halves(l_rnd);
  if constexpr (KS2) {
    // the second key group hands (O, m, l, l~) of its keys to the first
    // through LDS, which merges them as two blocks of the online softmax:
    // m = max(m0, m1), a_g = 2^(m_g - m), O = a0 O0 + a1 O1, l = a0 l0 + a1 l1
    __syncthreads();  // every wave is done with the K/V buffers
    float* const xo0 = reinterpret_cast<float*>(seg_k0);  // O blocks 0, 1: [32 values][256 lanes]
    float* const xo1 = reinterpret_cast<float*>(seg_k1);  // O blocks 2, 3
    float* const xs = reinterpret_cast<float*>(seg_v0);   // m, l, l~: [3][256 lanes]
    const int li = wr * 64 + lane;
    if (kg_u == 1) {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) (cb < 2 ? xo0 : xo1)[((cb & 1) * 16 + r) * 256 + li] = oacc[cb][r];
      xs[li] = m_run;
      xs[256 + li] = l_tot;
      xs[512 + li] = l_rnd_tot;
    }
    __syncthreads();
    if (kg_u == 1) return;
    const float m1 = xs[li];
    const float m = m_run > m1 ? m_run : m1;
    const float a0 = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        oacc[cb][r] = oacc[cb][r] * a0 + (cb < 2 ? xo0 : xo1)[((cb & 1) * 16 + r) * 256 + li] * a1;
    l_tot = l_tot * a0 + xs[256 + li] * a1;
    l_rnd_tot = l_rnd_tot * a0 + xs[512 + li] * a1;
    m_run = m;
  }
  // l = 0 only for a row that sees no key (causal or all-(-inf) bias):
  // O = 0, LSE = -inf
  constexpr bool CAN_BE_EMPTY = CAUSAL || BIAS || KS2;
  const float inv_l = (CAN_BE_EMPTY && l_tot == 0.0f) ? 0.0f : 1.0f / l_rnd_tot;
  const int q = q0 + wr * 32 + c;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = cb * 32 + g4 * 8 + 4 * h;
      if constexpr (SPLIT) {
        const floatx4 v{oacc[cb][4 * g4 + 0] * inv_l, oacc[cb][4 * g4 + 1] * inv_l, oacc[cb][4 * g4 + 2] * inv_l,
                        oacc[cb][4 * g4 + 3] * inv_l};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uintx4, v), ro, (uint32_t)q * (4 * DV) + d * 4, 0, 0);
        continue;
      }
      uint32_t w0, w1;
      {
        const __bf16 a0 = (__bf16)(oacc[cb][4 * g4 + 0] * inv_l);
        const __bf16 a1 = (__bf16)(oacc[cb][4 * g4 + 1] * inv_l);
        const __bf16 a2 = (__bf16)(oacc[cb][4 * g4 + 2] * inv_l);
        const __bf16 a3 = (__bf16)(oacc[cb][4 * g4 + 3] * inv_l);
        w0 = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
        w1 = (uint32_t)__builtin_bit_cast(uint16_t, a2) | ((uint32_t)__builtin_bit_cast(uint16_t, a3) << 16);
      }
      __builtin_amdgcn_raw_buffer_store_b64(uintx2{w0, w1}, ro, (uint32_t)q * RBV + d * 2, 0, 0);
    }
  if (h == 0 && q < Nq) {
    const float ln2 = 0.69314718055994530942f;
    lse_out[orow0 + q] = (CAN_BE_EMPTY && l_tot == 0.0f) ? -__builtin_inff() : (m_run + __log2f(l_tot)) * ln2;
  }
}

// Combines the key ranges of a split launch ("FlashAttention'ı Anlamak
// Bölüm 1", the online-softmax recurrence of section 0, applied once across
// ranges): per row, with L_s the ranges' log-sum-exps and O_s their
// normalised outputs, LSE = ln sum_s exp(L_s) and O = sum_s exp(L_s - LSE) O_s.
// A range that saw no key has L_s = -inf and weight 0; a row that saw none at
// all gets O = 0, LSE = -inf.  DV / 4 threads per row, 4 columns each.
template <int DV>
__global__ void __launch_bounds__(256)
fa_fwd_merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart, uint16_t* __restrict__ O,
                    float* __restrict__ LSE, int64_t rows, int n_splits) {
  constexpr int TPR = DV / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + (int64_t)(threadIdx.x / TPR);
  const int t = (int)(threadIdx.x % TPR);
  if (r >= rows) return;
  float m = -__builtin_inff();
  for (int s = 0; s < n_splits; ++s) m = fmaxf(m, Lpart[(int64_t)s * rows + r]);
  uint16_t* const o = O + r * DV + 4 * t;
  if (m == -__builtin_inff()) {
    *reinterpret_cast<uintx2*>(o) = uintx2{0u, 0u};
    if (t == 0) LSE[r] = -__builtin_inff();
    return;
  }
  floatx4 acc{0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t rs = (int64_t)s * rows + r;
    const float w = __builtin_amdgcn_exp2f((Lpart[rs] - m) * LOG2E);
    const floatx4 x = *reinterpret_cast<const floatx4*>(Opart + rs * DV + 4 * t);
    den += w;
    acc += w * x;
  }
  const float inv = 1.0f / den;
  const __bf16 a0 = (__bf16)(acc[0] * inv), a1 = (__bf16)(acc[1] * inv);
  const __bf16 a2 = (__bf16)(acc[2] * inv), a3 = (__bf16)(acc[3] * inv);
  *reinterpret_cast<uintx2*>(o) =
      uintx2{(uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16),
             (uint32_t)__builtin_bit_cast(uint16_t, a2) | ((uint32_t)__builtin_bit_cast(uint16_t, a3) << 16)};
  if (t == 0) LSE[r] = m + __log2f(den) * 0.69314718055994530942f;
}

template <int DQK, int DV, int BC, bool NEG_SCALE, bool CAUSAL, bool BIAS, bool SPLIT, int NW = 4, bool KS2 = false>
const void* kernel_ptr() {
  return (const void*)&fa_fwd_kernel<DQK, DV, BC, NEG_SCALE, CAUSAL, BIAS, SPLIT, NW, KS2>;
}

// Grids of the 8-wave kernel: at least one 256-row workgroup per CU (MI355X
// has 256); smaller launches keep 128-row workgroups, two per CU.  With the
// causal mask also at least 8192 query rows: each 256-row workgroup then
// masks 5 key tiles on its diagonal instead of 3, which the shorter
// sequences do not repay (causal, in one process: N = 8192 +1.4 %, 16384
// +2.0 %, 4096 -3.1 %).  A key split without the mask counts its
// ranges: B=1, H=8, Nq=4096, Nk=8192 in two ranges is 256 such workgroups.
constexpr int64_t kSegMinWorkgroups = 256;
constexpr int64_t kSegCausalMinRows = 8192;
bool use_seg(const LaunchArgs& a) {
  const int64_t ranges = a.n_splits > 1 ? a.n_splits : 1;
  if (a.bias != nullptr) return false;
  if (a.d == 64 && a.dv == 64) return !a.causal && ranges == 1 && a.BH * ((a.Nq + 255) / 256) >= kSegMinWorkgroups;
  if (a.d != 128 || a.dv != 128) return false;
  if (a.causal && (ranges > 1 || a.Nq < kSegCausalMinRows)) return false;
  return a.BH * ((a.Nq + 255) / 256) * ranges >= kSegMinWorkgroups;
}

// Kernel for one pair of head sizes: BC = 64 keys per tile (32 at head size
// 256, and with a bias, whose tiles live in registers).
template <int DQK, int DV, bool SPLIT>
const void* select_kernel(bool neg, bool causal, bool bias) {
  constexpr int BCP = DQK == 256 ? 32 : 64;
  // the sign of the scale needs no variant with a bias: the max is taken
  // over the biased logits themselves
  if (bias)
    return causal ? kernel_ptr<DQK, DV, 32, false, true, true, SPLIT>()
                  : kernel_ptr<DQK, DV, 32, false, false, true, SPLIT>();
  if (causal)
    return neg ? kernel_ptr<DQK, DV, BCP, true, true, false, SPLIT>()
               : kernel_ptr<DQK, DV, BCP, false, true, false, SPLIT>();
  return neg ? kernel_ptr<DQK, DV, BCP, true, false, false, SPLIT>()
             : kernel_ptr<DQK, DV, BCP, false, false, false, SPLIT>();
}

template <bool SPLIT>
const void* select_pair(int64_t d, int64_t dv, bool neg, bool causal, bool bias) {
  if (d == 64 && dv == 64) return select_kernel<64, 64, SPLIT>(neg, causal, bias);
  if (d == 128 && dv == 128) return select_kernel<128, 128, SPLIT>(neg, causal, bias);
  if (d == 256 && dv == 256) return select_kernel<256, 256, SPLIT>(neg, causal, bias);
  if (d == 192 && dv == 128) return select_kernel<192, 128, SPLIT>(neg, causal, bias);
  return nullptr;
}

// Scratch of the no-allocation key split: the ranges' fp32 partial outputs
// and log-sum-exps of one call, for callers that cannot allocate.  Every
// device that loads this code object holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels and copies take the address noalloc_scratch() returns.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return 1;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // once per device, with that device current: the array's address there
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return 1;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return 0;
}

// The in-workgroup key split (KS2): head size 128, no bias, no split, keys
// enough for each group to run a few tiles, and a grid of 256 to 512
// 128-row workgroups (one or two per CU) that does not take the 256-row
// 8-wave kernel.  Causal, in one process against the 4-wave kernel: 256
// workgroups +23-30 %, 384 +38 %, 512 +15 %, 640 -6 %, 768 -9 to -11 %,
// 1024 and more -6 to -19 %.
constexpr int64_t kKs2MinKeys = 1024;
bool use_ks2(const LaunchArgs& a) {
  const int64_t g128 = a.BH * ((a.Nq + 127) / 128);
  return a.d == 128 && a.dv == 128 && a.bias == nullptr && a.n_splits <= 1 && a.Nk >= kKs2MinKeys &&
         g128 >= kSegMinWorkgroups && g128 <= 2 * kSegMinWorkgroups;
}

int launch_fa_fwd(const LaunchArgs& a, hipStream_t stream) {
  const bool seg = use_seg(a);
  const bool ks2 = !seg && use_ks2(a);
  const int br = seg ? 2 * BR : BR;
  const int n_qtiles = (int)((a.Nq + br - 1) / br);
  const int64_t nblk = a.BH * n_qtiles;
  const float c_log2 = (float)((double)a.scale * 1.4426950408889634074);
  const uint16_t* q = static_cast<const uint16_t*>(a.Q);
  const uint16_t* k = static_cast<const uint16_t*>(a.K);
  const uint16_t* v = static_cast<const uint16_t*>(a.V);
  uint16_t* o = static_cast<uint16_t*>(a.O);
  float* lse = a.LSE;
  const float* bias = a.bias;
  int64_t sb = a.bias_sb, sh = a.bias_sh, sq = a.bias_sq;
  int heads = (int)a.H;
  int nq = (int)a.Nq, nk = (int)a.Nk;
  int nqt = n_qtiles;
  float cl = c_log2;
  const bool split = a.n_splits > 1;
  float* opart = a.Opart;
  float* lpart = a.Lpart;
  int split_keys = a.split_keys;
  int n_splits = split ? a.n_splits : 1;
  void* args[] = {&q, &k, &v, &o, &lse, &bias, &sb, &sh, &sq, &heads, &nq, &nk, &nqt, &cl,
                  &opart, &lpart, &split_keys, &n_splits};
  const bool neg = a.scale < 0.0f;
  const bool b = bias != nullptr;
  const void* fn = ks2 ? (a.causal ? (neg ? kernel_ptr<128, 128, 64, true, true, false, false, 8, true>()
                                          : kernel_ptr<128, 128, 64, false, true, false, false, 8, true>())
                                   : (neg ? kernel_ptr<128, 128, 64, true, false, false, false, 8, true>()
                                          : kernel_ptr<128, 128, 64, false, false, false, false, 8, true>()))
                   : seg && a.d == 64 ? (neg ? kernel_ptr<64, 64, 64, true, false, false, false, 8>()
                                             : kernel_ptr<64, 64, 64, false, false, false, false, 8>())
                   : seg && split ? (neg ? kernel_ptr<128, 128, 64, true, false, false, true, 8>()
                                       : kernel_ptr<128, 128, 64, false, false, false, true, 8>())
                   : seg   ? (a.causal ? (neg ? kernel_ptr<128, 128, 64, true, true, false, false, 8>()
                                              : kernel_ptr<128, 128, 64, false, true, false, false, 8>())
                                       : (neg ? kernel_ptr<128, 128, 64, true, false, false, false, 8>()
                                              : kernel_ptr<128, 128, 64, false, false, false, false, 8>()))
                   : split ? select_pair<true>(a.d, a.dv, neg, a.causal, b)
                           : select_pair<false>(a.d, a.dv, neg, a.causal, b);
  if (fn == nullptr) return (int)hipErrorInvalidValue;
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(nblk * n_splits)), dim3(seg || ks2 ? 2 * NTHREADS : NTHREADS),
                                 args, 0, stream);
  if (e != hipSuccess || !split) return e == hipSuccess ? 0 : (int)e;
  // merge the key ranges: DV / 4 threads per row
  const int64_t rows = a.BH * a.Nq;
  const int rpb = 256 / (int)(a.dv / 4);
  const void* mfn = a.dv == 64    ? (const void*)&fa_fwd_merge_kernel<64>
                    : a.dv == 256 ? (const void*)&fa_fwd_merge_kernel<256>
                                  : (const void*)&fa_fwd_merge_kernel<128>;
  const float* cop = opart;
  const float* clp = lpart;
  int64_t nrows = rows;
  void* margs[] = {&cop, &clp, &o, &lse, &nrows, &n_splits};
  e = hipLaunchKernel(mfn, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), margs, 0, stream);
  return e == hipSuccess ? 0 : (int)e;
}

const char* kernel_config_string() {
  return "gfx950 fa_fwd v19: BR=128 (4 waves x 32 rows; 256 = 8 waves for head size 128 without bias and 64 without mask or bias on grids of "
         ">= 256 workgroups incl. key-split ranges without mask, causal from 8192 rows; 8 waves as two key groups "
         "of 4 on 128 rows, merged in LDS, where 128-row workgroups give each CU one), plain tiles (below the diagonal with the causal mask; with a bias not at head size 64, "
         "(192, 128) causal only with a bias) in fixed MFMA segments (32 at head sizes 128 and 256, 40 at (192, 128), 16 "
         "at 64 and at 128 with a bias, 20 at (192, 128) with a bias), BC=64 (32 with bias), 3-stage K/V pipeline "
         "(S two tiles ahead of P V, softmax in between, its exponent, exponential and row sum a segment apart), "
         "direct-to-LDS, S^T=K.Q^T on mfma_f32_32x32x16_bf16 "
         "(K fragments read two k steps ahead at head size 128, one at (192, 128) without mask or bias; three waves "
         "per SIMD and a two-FMA exponent at head size 64 with a bias), "
         "V^T via ds_read_b64_tr_b16; O divided by the sum of the bf16 P taken on mfma_f32_16x16x32_bf16 with a 0/1 mask "
         "(bf16 dot products at head size 256 with a bias and (192, 128) without mask or bias); "
         "no tile max unless exp2 exceeds 2^16; causal tile skipping; "
         "fp32 additive bias; key split with LSE merge";
}

}  // namespace fa06

// fa_fwd_kernel.hip -- gfx950 (CDNA4) fused attention forward kernel.
//
// Computes O = softmax_row(scale * Q K^T) V and the per-row log-sum-exp for
// BF16 Q/K/V with head size 128 ("FlashAttention'ı Anlamak Bölüm 1",
// section 0.2, score and output equations without the mask term).
//
// Work partition (B200 article, section "Kernel işini nasıl
// bölümlendiriyor"): one workgroup per tile of BR query rows of one
// (batch, head); the Q tile is loaded once; the workgroup then walks the K/V
// sequence in tiles of BC keys, computing scores, updating the online
// softmax state (row max and row sum) and accumulating P V in registers; the
// accumulator is normalised once after the loop and written.
//
// MI355X mapping:
//   * 4 waves per workgroup, 32 query rows per wave, 2 workgroups per CU.
//   * Scores are produced transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (K is the A operand from LDS, Q^T the B operand
//     held in registers for the whole loop).  The accumulator then gives each
//     lane one query and 16 keys, so row max / row sum are in-lane reductions
//     plus one exchange between the two 32-lane halves, and the same
//     registers, rounded to bf16, are directly the B operand of
//     O^T += V^T P^T.  The key order inside an MFMA k-step is permuted
//     consistently on both operands (the contraction does not depend on it).
//   * V^T fragments come from the row-major V tile in LDS through
//     ds_read_b64_tr_b16 (a transposing LDS read), so V is never transposed
//     in memory.
//   * K/V tiles are double buffered in LDS: tile j+1 is copied global -> LDS
//     directly (buffer loads with the LDS destination, no registers) into
//     the other buffer while tile j is computed (the 2-stage pipeline of the
//     5090 article's "v3").
//   * LDS rows are 256 bytes; 16-byte chunks are XOR-swizzled per row so the
//     K fragment reads (ds_read_b128) and the V transposing reads are free
//     of bank conflicts (the swizzled shared memory of the 5090 article's
//     "v2", re-derived for the gfx950 LDS).
//   * The softmax scale is folded into exp2 as scale*log2(e).  The running
//     max is only raised when a row's new max exceeds it by more than
//     RESCALE_SLACK (in log2 units); otherwise the stale max is kept, which is
//     exact because the same max enters P, the row sum and the output.  This
//     removes almost all O rescaling from the loop.
//   * Global accesses use buffer resources sized to each (batch, head)
//     slice: rows past Nq / Nk read as zero and stores past Nq are dropped,
//     so ragged sequence lengths need no special load or store paths.
//   * Workgroup ids are remapped so the q-tiles of one head run on the same
//     XCD (workgroups are dispatched round-robin over the 8 XCDs), sharing
//     that head's K/V in the XCD's L2.
//   * Causal variant (the mask term of the score equation): a q-tile stops
//     at the last K/V tile its last row can see, only tiles that cross the
//     diagonal are masked per key, and the q-tiles with the most work are
//     dispatched first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_kernel.h"

namespace fa06 {
namespace {

constexpr int D = 128;          // head size (d = d_v)
constexpr int ROW_BYTES = D * 2; // one bf16 row
constexpr int BR = 128;         // query rows per workgroup
constexpr int BC = 64;          // keys per K/V tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr int TILE_BYTES = BC * ROW_BYTES;   // one K or V tile: 16 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K + V
constexpr int LDS_BYTES = 2 * STAGE_BYTES;   // double buffered: 64 KiB
constexpr float RESCALE_SLACK = 8.0f;        // log2 units: P stays <= 256

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef unsigned uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Buffer resource: base, no stride, num_records bytes; dword3 selects the
// 32-bit data format, which gfx9-family raw buffer accesses require.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uintx4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(uintx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}

// Swizzled byte offset of 16-byte chunk `ch` of row `row` in a K or Q tile:
// any 16 consecutive rows place a given chunk in 16 distinct bank groups.
__device__ inline uint32_t k_swz(uint32_t row, uint32_t ch) {
  return row * ROW_BYTES + ((ch ^ (row & 15u)) << 4);
}
// V tile: the transposing reads touch a 64-byte band (4 chunks) of 8 rows at
// once; XOR-ing the band index with row%4 spreads 4 rows over the 256 bytes.
__device__ inline uint32_t v_swz(uint32_t row, uint32_t ch) {
  return row * ROW_BYTES + ((ch ^ ((row & 3u) << 2)) << 4);
}

__device__ inline float wave_max_halves(float x) {
  // lanes l and l^32 hold the same query row
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float wave_min_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ inline float wave_sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Direct global -> LDS copy (buffer_load_dwordx4 ... lds): lane L of a wave
// writes its 16 bytes at lds_base + 16*L, so each instruction fills 1 KiB of
// LDS linearly.  The swizzle is applied on the source side: the lane that
// fills physical chunk P of row r loads logical chunk P ^ f(r).
// `rows` rows starting at global row `row0` (scalar) go to `lds`; every wave
// issues rows*16/64/NWAVES instructions.
template <int ROWS, bool IS_V>
__device__ inline void tile_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t row0, char* lds, int wave, int lane) {
  const uint32_t soff = __builtin_amdgcn_readfirstlane(row0 * ROW_BYTES);
  constexpr int N_INST = ROWS * 16 / 64 / NWAVES;
#pragma unroll
  for (int i = 0; i < N_INST; ++i) {
    const uint32_t blk = (uint32_t)(i * NWAVES + wave);      // which 1 KiB block (4 rows)
    const uint32_t row = blk * 4 + ((uint32_t)lane >> 4);
    const uint32_t pos = (uint32_t)lane & 15u;                // physical chunk in the row
    const uint32_t ch = IS_V ? (pos ^ ((row & 3u) << 2)) : (pos ^ (row & 15u));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)((lds_char*)lds + blk * 1024u), 16,
        row * ROW_BYTES + (ch << 4), soff, 0, 0);
  }
}

// Every helper lambda of the kernel is inlined: the loop body must stay one
// straight-line region with all state in registers.
#define FA_INLINE __attribute__((always_inline))

// Wait until this wave's outstanding global loads (incl. LDS-direct) landed.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// CAUSAL: key j is hidden from query i when j > i + (Nk - Nq); tiles past a
// q-tile's diagonal are skipped, tiles crossing it are masked per element.
template <bool NEG_SCALE, bool CAUSAL>
__global__ void __launch_bounds__(NTHREADS)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
              int Nq, int Nk, int n_qtiles, float c_log2) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;   // query column of the S^T / O^T accumulators
  const int h = lane >> 5;   // half of the wave

  // XCD-aware remap: consecutive logical tiles (same head) go to one XCD.
  int bid = blockIdx.x;
  const int nblk = gridDim.x;
  const int nfull = nblk & ~7;
  if (bid < nfull) bid = (bid & 7) * (nfull >> 3) + (bid >> 3);
  const int bh = bid / n_qtiles;
  int qt = bid - bh * n_qtiles;
  if (CAUSAL) qt = n_qtiles - 1 - qt;  // the longest rows of a head start first
  const int q0 = qt * BR;

  const size_t head_q = (size_t)bh * (size_t)Nq * D;
  const size_t head_k = (size_t)bh * (size_t)Nk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head_q, (uint32_t)Nq * ROW_BYTES);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head_k, (uint32_t)Nk * ROW_BYTES);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head_k, (uint32_t)Nk * ROW_BYTES);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + head_q, (uint32_t)Nq * ROW_BYTES);

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int n_full = Nk / BC;  // tiles with BC valid keys
  int n_tiles = n_full + (Nk % BC != 0);
  int first_masked = n_full;   // first tile that needs per-key masks
  // last key visible to this lane's query row (keys above it are masked)
  int key_lim = Nk - 1;
  if constexpr (CAUSAL) {
    const int off = Nk - Nq;
    const int q_last = (q0 + BR < Nq ? q0 + BR : Nq) - 1;
    const int lim_last = q_last + off;  // the q-tile's last row sees keys <= lim_last
    const int lim_first = q0 + off;     // its first row sees keys <= lim_first
    const int need = lim_last < 0 ? 0 : lim_last / BC + 1;
    n_tiles = need < n_tiles ? need : n_tiles;
    const int unmasked = lim_first + 1 <= 0 ? 0 : (lim_first + 1) / BC;
    first_masked = unmasked < first_masked ? unmasked : first_masked;
    const int my_lim = q0 + wave * 32 + c + off;
    key_lim = my_lim < key_lim ? my_lim : key_lim;
    if (n_tiles == 0) {
      // no row of this q-tile sees any key: O = 0, LSE = -inf
      const int q = q0 + wave * 32 + c;
#pragma unroll
      for (int i = 0; i < 8; ++i)  // this lane's half row: bytes [128h, 128h + 128)
        __builtin_amdgcn_raw_buffer_store_b128(uintx4{0u, 0u, 0u, 0u}, ro,
                                               (uint32_t)q * ROW_BYTES + 128u * (uint32_t)h + 16u * (uint32_t)i, 0, 0);
      if (h == 0 && q < Nq) LSE[(size_t)bh * Nq + q] = -__builtin_inff();
      return;
    }
  }

  // LDS: K buffers at [0, 32K), V buffers at [32K, 64K).  K runs one tile
  // ahead of V: while tile j's P V is accumulated, tile j+1's scores are
  // computed, so K(j+1) and V(j) are resident together.
  char* const kbuf0 = smem;
  char* const vbuf0 = smem + 2 * TILE_BYTES;
  auto kbuf = [&](int i) FA_INLINE { return kbuf0 + i * TILE_BYTES; };
  auto vbuf = [&](int i) FA_INLINE { return vbuf0 + i * TILE_BYTES; };

  // ---- prologue: Q (staged in the V buffers), K(0), K(1).
  tile_to_lds<BR, false>(rq, q0, vbuf0, wave_u, lane);
  tile_to_lds<BC, false>(rk, 0, kbuf(0), wave_u, lane);
  if (n_tiles > 1) tile_to_lds<BC, false>(rk, BC, kbuf(1), wave_u, lane);
  wait_vmem();
  __syncthreads();

  bf16x8 qb[8];  // qb[t]: Q[q0 + wave*32 + c][16t + 8h .. +7]
  {
    const uint32_t row = wave * 32 + c;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      qb[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(vbuf0 + k_swz(row, 2 * t + h)));
  }
  __syncthreads();  // the V buffers are reused from here on
  tile_to_lds<BC, true>(rv, 0, vbuf(0), wave_u, lane);

  floatx16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = floatx16{};
  float m_run = -__builtin_inff();  // running max, log2 units, per query
  float l_run = 0.0f;               // partial row sum of this lane's keys

  // S^T = K Q^T for the 64 keys of one K buffer (two 32-key blocks).
  auto scores = [&](const char* ks, floatx16 (&s)[2]) FA_INLINE {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
      const uint32_t row = kb * 32 + c;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(ks + k_swz(row, 2 * t + h)));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[t], s[kb], 0, 0, 0);
      }
    }
  };

  // Online softmax of one tile's scores -> P (bf16, B operand of the P V
  // product).  Branch free: the decision to raise the running max is wave
  // uniform (ballot); returns the factor the output accumulator must be
  // multiplied by before this tile's P V is added (1 when unchanged).
  // MASK tiles hide the keys above `lim` (this row's last visible key,
  // relative to the tile's first key).
  auto softmax = [&](floatx16 (&s)[2], bf16x8 (&pb)[4], int lim, auto mask_tag, bool& rescale) FA_INLINE -> float {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > lim) s[kb][r] = NEG_SCALE ? __builtin_inff() : -__builtin_inff();
        }
    }
    float ext = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ext = NEG_SCALE ? fminf(ext, s[kb][r]) : fmaxf(ext, s[kb][r]);
    ext = NEG_SCALE ? wave_min_halves(ext) : wave_max_halves(ext);
    const float m_tile = ext * c_log2;
    rescale = __ballot(m_tile > m_run + RESCALE_SLACK) != 0;
    const float m_new = rescale ? fmaxf(m_run, m_tile) : m_run;
    float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    // a causal row that has seen no key yet keeps m = -inf (and l = 0)
    if constexpr (CAUSAL) alpha = m_new == -__builtin_inff() ? 1.0f : alpha;
    m_run = m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_run));
        if constexpr (MASK) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key > lim) p = 0.0f;
        }
        lsum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + lsum;
    return alpha;
  };

  // O^T += V^T P^T for the 64 keys of one V buffer: 4 d-blocks x 4 key steps.
  auto accumulate = [&](const char* vs, const bf16x8 (&pb)[4]) FA_INLINE {
    const int g = lane >> 4;          // 16-lane group
    const int i16 = lane & 15;
    const int sub = i16 >> 2;         // which of the 4 keys this lane addresses
    const int q4 = i16 & 3;           // which 4-column piece of the 16 columns
    const int hh = g >> 1;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int d0 = cb * 32 + (g & 1) * 16 + q4 * 4;  // first of 4 d columns
      const uint32_t ch = (uint32_t)d0 >> 3;
      const uint32_t within = ((uint32_t)d0 & 7u) * 2u;
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
        const uint32_t r0 = ks4 * 16 + 4 * hh + sub;
        const uint32_t r1 = r0 + 8;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)((lds_char*)vs + v_swz(r0, ch) + within));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) shortx4*)((lds_char*)vs + v_swz(r1, ch) + within));
        // move the two 4-element results as whole dwords (no per-element
        // extraction): a = {lo[0..3], hi[0..3]}
        const uintx2 lo2 = __builtin_bit_cast(uintx2, lo);
        const uintx2 hi2 = __builtin_bit_cast(uintx2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, uintx4{lo2.x, lo2.y, hi2.x, hi2.y});
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks4], oacc[cb], 0, 0, 0);
      }
    }
  };

  auto rescale_o = [&](float alpha) FA_INLINE {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
  };

  // ---- tile 0: scores and softmax before the loop.
  bf16x8 pb[4];
  {
    floatx16 s[2];
    scores(kbuf(0), s);
    bool rs;
    if (first_masked == 0)
      softmax(s, pb, key_lim, std::true_type{}, rs);
    else
      softmax(s, pb, key_lim, std::false_type{}, rs);
    // O is still zero: no rescale needed
  }
  wait_vmem();
  __syncthreads();

  // Iteration j: P(j) V(j) accumulated while S(j+1) is computed and turned
  // into P(j+1).  On entry K(j+1) is in kbuf((j+1)&1), V(j) in vbuf(j&1);
  // the iteration prefetches K(j+2) into kbuf(j&1) and V(j+1) into
  // vbuf((j+1)&1), whose previous contents were consumed before the last
  // barrier.
  auto iteration = [&](int j, auto par_tag, auto has_next_tag, auto mask_next_tag) FA_INLINE {
    constexpr int P = decltype(par_tag)::value;  // == j & 1
    constexpr bool HAS_NEXT = decltype(has_next_tag)::value;
    if (j + 2 < n_tiles) tile_to_lds<BC, false>(rk, (j + 2) * BC, kbuf(P), wave_u, lane);
    if (HAS_NEXT) tile_to_lds<BC, true>(rv, (j + 1) * BC, vbuf(P ^ 1), wave_u, lane);
    if constexpr (HAS_NEXT) {
      floatx16 s[2];
      scores(kbuf(P ^ 1), s);
      bf16x8 pn[4];
      bool rs;
      const float alpha = softmax(s, pn, key_lim - (j + 1) * BC, mask_next_tag, rs);
      accumulate(vbuf(P), pb);
      if (rs) rescale_o(alpha);
#pragma unroll
      for (int i = 0; i < 4; ++i) pb[i] = pn[i];
      wait_vmem();
      __syncthreads();
    } else {
      accumulate(vbuf(P), pb);
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  if constexpr (!CAUSAL) {
    // iterations 0 .. n_tiles-3 compute S of a full tile
    int j = 0;
    for (; j + 1 < n_tiles - 2; j += 2) {
      iteration(j, P0{}, T{}, F{});
      iteration(j + 1, P1{}, T{}, F{});
    }
    if (j < n_tiles - 2) {
      iteration(j, P0{}, T{}, F{});
      ++j;
    }
    // iteration n_tiles-2 computes S of the last tile (masked if partial)
    if (j == n_tiles - 2) {
      const bool tail = first_masked < n_tiles;
      if (j & 1) {
        if (tail) iteration(j, P1{}, T{}, T{}); else iteration(j, P1{}, T{}, F{});
      } else {
        if (tail) iteration(j, P0{}, T{}, T{}); else iteration(j, P0{}, T{}, F{});
      }
    }
  } else {
    // Iterations j in [j0, j1) all compute S of a next tile with the same
    // masking; the K/V buffer parity (j & 1) is a compile-time constant of
    // each instantiation, so the loop is unrolled by two.
    auto run = [&](int j0, int j1, auto mask_tag) FA_INLINE {
      int j = j0;
      if (j < j1 && (j & 1)) {
        iteration(j, P1{}, T{}, mask_tag);
        ++j;
      }
      for (; j + 1 < j1; j += 2) {
        iteration(j, P0{}, T{}, mask_tag);
        iteration(j + 1, P1{}, T{}, mask_tag);
      }
      if (j < j1) iteration(j, P0{}, T{}, mask_tag);
    };
    // the next tile is unmasked for j + 1 < first_masked, masked from there on
    // (only the few tiles that cross the diagonal or hold the Nk tail)
    int j_split = first_masked - 1;
    j_split = j_split < 0 ? 0 : (j_split > n_tiles - 1 ? n_tiles - 1 : j_split);
    run(0, j_split, F{});
    run(j_split, n_tiles - 1, T{});
  }
  // last iteration: P V of the last tile only
  if ((n_tiles - 1) & 1) iteration(n_tiles - 1, P1{}, F{}, F{}); else iteration(n_tiles - 1, P0{}, F{}, F{});

  // ---- epilogue: 1/l, bf16 (round to nearest even), LSE in natural log.
  const float l_tot = wave_sum_halves(l_run);
  // l = 0 only for a causal row that sees no key: O = 0, LSE = -inf
  const float inv_l = (CAUSAL && l_tot == 0.0f) ? 0.0f : 1.0f / l_tot;
  const int q = q0 + wave * 32 + c;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d = cb * 32 + g4 * 8 + 4 * h;
      uint32_t w0, w1;
      {
        const __bf16 a0 = (__bf16)(oacc[cb][4 * g4 + 0] * inv_l);
        const __bf16 a1 = (__bf16)(oacc[cb][4 * g4 + 1] * inv_l);
        const __bf16 a2 = (__bf16)(oacc[cb][4 * g4 + 2] * inv_l);
        const __bf16 a3 = (__bf16)(oacc[cb][4 * g4 + 3] * inv_l);
        w0 = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
        w1 = (uint32_t)__builtin_bit_cast(uint16_t, a2) | ((uint32_t)__builtin_bit_cast(uint16_t, a3) << 16);
      }
      __builtin_amdgcn_raw_buffer_store_b64(uintx2{w0, w1}, ro, (uint32_t)q * ROW_BYTES + d * 2, 0, 0);
    }
  if (h == 0 && q < Nq) {
    const float ln2 = 0.69314718055994530942f;
    LSE[(size_t)bh * Nq + q] = (CAUSAL && l_tot == 0.0f) ? -__builtin_inff() : (m_run + __log2f(l_tot)) * ln2;
  }
}

}  // namespace

int launch_fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                  int64_t BH, int64_t Nq, int64_t Nk, float scale, bool causal, hipStream_t stream) {
  const int n_qtiles = (int)((Nq + BR - 1) / BR);
  const int64_t nblk = BH * n_qtiles;
  const float c_log2 = (float)((double)scale * 1.4426950408889634074);
  const uint16_t* q = static_cast<const uint16_t*>(Q);
  const uint16_t* k = static_cast<const uint16_t*>(K);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  uint16_t* o = static_cast<uint16_t*>(O);
  int nq = (int)Nq, nk = (int)Nk;
  void* args[] = {&q, &k, &v, &o, &LSE, &nq, &nk, (void*)&n_qtiles, (void*)&c_log2};
  const bool neg = scale < 0.0f;
  const void* fn = causal ? (neg ? (const void*)&fa_fwd_kernel<true, true> : (const void*)&fa_fwd_kernel<false, true>)
                          : (neg ? (const void*)&fa_fwd_kernel<true, false> : (const void*)&fa_fwd_kernel<false, false>);
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)nblk), dim3(NTHREADS), args, 0, stream);
  return e == hipSuccess ? 0 : (int)e;
}

const char* kernel_config_string() {
  return "gfx950 fa_fwd v3.1: BR=128 (4 waves x 32 rows), BC=64, K one tile ahead of V, direct-to-LDS, "
         "S^T=K.Q^T on mfma_f32_32x32x16_bf16, V^T via ds_read_b64_tr_b16; causal variant with tile skipping";
}

}  // namespace fa06

// fa_fwd_mxfp8.hip -- gfx950 attention forward on MXFP8 inputs.
//
// The computation is the forward pass of fa_fwd (the score and output
// equations of "FlashAttention'ı Anlamak Bölüm 1", section 0.2, with the
// optional causal mask) on inputs stored in the OCP microscaling format
// MXFP8: E4M3 elements, one E8M0 scale 2^(s-127) per block of 32 elements
// along each product's contraction axis -- Q and K along the head dimension,
// V along the keys (so V arrives transposed, V^T [d, keys]).  The pages name
// MXFP8 attention as the aim of their kernel work ("Flash Attention на 5090
// в CUDA C++", motivation and "Что дальше"); on gfx950 both products run on
// the block-scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4, which applies the
// E8M0 scales itself.  The probabilities P are converted to E4M3 (scale 1)
// for the P V product; the row sum l uses the unrounded fp32 P.
//
// MFMA lane layout (32x32x64, checked on the GPU): lane (row r = l%32,
// half g = l/32) holds 32 bytes of its row; bytes 0..15 are contraction
// indices 16g..16g+15 and bytes 16..31 are 32+16g..32+16g+15; the scale of
// (row r, contraction block b of 32) is lane r+32b's scale byte (op_sel picks
// the byte of the 32-bit scale register).  The output is the usual
// D[8(q/4) + 4g + q%4][r] for accumulator register q.
//
// Loop structure: as the bf16 kernel (waves of 32 query rows, 64-key tiles,
// three-stage pipeline: S of tile j+2 and P V of tile j on the MFMAs with the
// softmax of tile j+1 in between).  Workgroups have 8 waves (256 rows, one
// workgroup per CU, each K/V tile shared by twice the rows) on grids of at
// least 256 such workgroups and 4 waves (128 rows, two per CU) otherwise.
// Plain tiles run the iteration in a fixed order of 8 segments, one MFMA
// each, with the softmax scores and operand reads spread over them
// (iteration_seg); masked tiles keep the compiler-scheduled iteration.  S^T = K Q^T
// reads the K tile's rows in a permuted order so that each lane's 16
// accumulator rows are 16 consecutive keys: the two 32-key blocks of a tile
// then give each lane exactly the key bytes the P operand of the 64-key P V
// product needs, with no data movement.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_kernel.h"

namespace fa06 {
namespace {

typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int MX_BC = 64;              // keys per tile
constexpr int MX_KROW = 128;           // bytes per K row (d = 128 E4M3 elements)
constexpr int MX_KTILE = MX_BC * MX_KROW;        // 8 KiB
constexpr int MX_VROW = MX_BC;                   // bytes per V^T tile row (64 keys)
constexpr int MX_VTILE = D * MX_VROW;            // 8 KiB
constexpr int MX_SC = 256;                       // scale bytes per tile (K: 64x4, V: 2x128)
constexpr int MX_STAGE = MX_KTILE + MX_SC;       // K tile + its scales (V the same size)
constexpr int MX_LDS = 4 * MX_STAGE;             // K[2], V[2]

// Key held by accumulator row m of a 32-key block: rows 8a + 4g + e (the
// MFMA output order) map to key 16g + 4a + e, so lane half g's 16 rows are
// keys 16g..16g+15.
__device__ inline uint32_t key_of_row(uint32_t m) { return 16u * ((m >> 2) & 1u) + 4u * (m >> 3) + (m & 3u); }

// K tile (128-byte rows, 8 chunks): the 16 lanes of one read phase fetch one
// chunk of rows key_of_row(0..15) = {0-3, 16-19, 4-7, 20-23} (+8 in the other
// phase); rows of equal parity share a bank half, and the XOR below gives
// the 8 rows of each parity 8 distinct chunks.
__device__ inline uint32_t kx(uint32_t row) { return ((row >> 1) & 3u) | (((row >> 4) & 1u) << 2); }
// V^T tile (64-byte rows, 4 chunks): 16 lanes read one chunk of 16
// consecutive rows; rows d and d+4 share banks unless the chunk moves.
__device__ inline uint32_t vx(uint32_t row) { return (row >> 2) & 3u; }

__device__ inline intx8 lds_read32(const char* p0, const char* p1) {
  const uintx4 a = *reinterpret_cast<const uintx4*>(p0);
  const uintx4 b = *reinterpret_cast<const uintx4*>(p1);
  return intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// KS2 (8 waves only): two groups of 4 waves attend to the two halves of the
// key tiles that 128 query rows see and merge (O, m, l) through LDS at the
// end, for launches that give each CU one 128-row workgroup but too few
// 256-row ones.
template <bool NEG_SCALE, bool CAUSAL, int NW, bool KS2 = false>
__global__ void __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(2, 2)))
fa_fwd_mxfp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ Qs,
                    const uint8_t* __restrict__ K8, const uint8_t* __restrict__ Ks,
                    const uint8_t* __restrict__ Vt8, const uint8_t* __restrict__ Vs,
                    uint16_t* __restrict__ O, float* __restrict__ LSE,
                    int Nq, int Nk_all, int ldv, int n_qtiles, float c_log2) {
  static_assert(!KS2 || NW == 8, "key groups: 8 waves");
  constexpr int KB = 2;  // 32-key blocks per tile
  constexpr int NWR = KS2 ? NW / 2 : NW;  // waves per key group (all waves without KS2)
  constexpr int BR = 32 * NWR;  // query rows per workgroup
  constexpr int NKG = KS2 ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) char smem[NKG * MX_LDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 31;
  const int h = lane >> 5;
  const int wr = KS2 ? (wave & (NWR - 1)) : wave;  // which 32 rows of the workgroup
  const int kg_u = KS2 ? __builtin_amdgcn_readfirstlane(wave / NWR) : 0;  // key group

  int bh, qt;
  if constexpr (CAUSAL) {
    xcd_tile_map(blockIdx.x, gridDim.x, n_qtiles, true, bh, qt);  // longest-first over each XCD
    qt = n_qtiles - 1 - qt;
  } else {
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    const int nfull = nblk & ~7;
    if (bid < nfull) bid = (bid & 7) * (nfull >> 3) + (bid >> 3);
    bh = bid / n_qtiles;
    qt = bid - bh * n_qtiles;
  }
  const int q0 = qt * BR;

  // KS2: group g takes key tiles [g*G, (g+1)*G) of the tiles the q-tile sees,
  // G = half of them rounded up; both groups run G iterations (tiles past the
  // visible keys are fully masked), so every barrier is reached by all waves
  int ks_tiles = 0;
  if constexpr (KS2) {
    int total = (Nk_all + MX_BC - 1) / MX_BC;
    if constexpr (CAUSAL) {
      const int lim_last = (q0 + BR < Nq ? q0 + BR : Nq) - 1 + Nk_all - Nq;
      const int need = lim_last < 0 ? 0 : lim_last / MX_BC + 1;
      total = need < total ? need : total;
    }
    ks_tiles = (total + 1) / 2;
  }
  const int k0 = KS2 ? kg_u * ks_tiles * MX_BC : 0;  // this group's first key
  const int Nk = KS2 ? (Nk_all - k0 <= 0 ? 0 : (Nk_all - k0 < ks_tiles * MX_BC ? Nk_all - k0 : ks_tiles * MX_BC))
                     : Nk_all;
  const int vrest = ldv - k0 > 0 ? ldv - k0 : 0;  // V^T columns from k0 on

  const size_t bq = (size_t)bh * (size_t)Nq, bk = (size_t)bh * (size_t)Nk_all + (size_t)k0;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q8 + bq * D, (uint32_t)Nq * D);
  const __amdgpu_buffer_rsrc_t rqs = make_rsrc(Qs + bq * 4, (uint32_t)Nq * 4u);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K8 + bk * D, (uint32_t)Nk * D);
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(Ks + ((size_t)bh * (size_t)ldv + (size_t)k0) * 4, (uint32_t)Nk * 4u);
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(Vt8 + (size_t)bh * D * (size_t)ldv + (size_t)k0, (uint32_t)D * (uint32_t)ldv - (uint32_t)(ldv - vrest));
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(Vs + ((size_t)bh * (size_t)(ldv / 32) + (size_t)(k0 / 32)) * D,
                                               (uint32_t)(vrest / 32) * D);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + bq * D, (uint32_t)Nq * ROW_BYTES);
  const int wr_u = __builtin_amdgcn_readfirstlane(wr);

  const int n_full = Nk / MX_BC;
  int n_tiles = KS2 ? ks_tiles : n_full + (Nk % MX_BC != 0);
  int first_masked = n_full;
  int key_lim = Nk - 1;
  const int q = q0 + wr * 32 + c;
  if constexpr (CAUSAL) {
    const int off = Nk_all - k0 - Nq;  // key k0 + j is hidden from query i when j > i + off
    const int q_last = (q0 + BR < Nq ? q0 + BR : Nq) - 1;
    const int lim_last = q_last + off;
    const int lim_first = q0 + off;
    const int need = lim_last < 0 ? 0 : lim_last / MX_BC + 1;
    if constexpr (!KS2) n_tiles = need < n_tiles ? need : n_tiles;  // KS2: G for both groups
    const int unmasked = lim_first + 1 <= 0 ? 0 : (lim_first + 1) / MX_BC;
    first_masked = unmasked < first_masked ? unmasked : first_masked;
    key_lim = q + off < key_lim ? q + off : key_lim;
    if (n_tiles == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(uintx4{0u, 0u, 0u, 0u}, ro,
                                               (uint32_t)q * ROW_BYTES + 128u * (uint32_t)h + 16u * (uint32_t)i, 0, 0);
      if (h == 0 && q < Nq) LSE[bq + q] = -__builtin_inff();
      return;
    }
  }

  // LDS: K(j+2), K(j+3) tiles then V(j), V(j+1), each followed by its 256
  // scale bytes (K: 64 keys x 4 blocks; V: 2 key blocks x 128 rows).
  char* const kst0 = smem + kg_u * MX_LDS;
  char* const vst0 = kst0 + 2 * MX_STAGE;
  auto kbuf = [&](int i) FA_INLINE { return kst0 + i * MX_STAGE; };
  auto vbuf = [&](int i) FA_INLINE { return vst0 + i * MX_STAGE; };

  // tile j: K rows [64j, 64j+64) x 128 bytes and their scales
  auto k_to_lds = [&](int j, char* dst) FA_INLINE {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)j * (uint32_t)MX_KTILE);
#pragma unroll
    for (int i = 0; i < 8 / NWR; ++i) {
      const uint32_t blk = (uint32_t)(i * NWR + wr_u);  // 1 KiB = 8 rows
      const uint32_t row = blk * 8u + ((uint32_t)lane >> 3);
      const uint32_t ch = ((uint32_t)lane & 7u) ^ kx(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)((lds_char*)dst + blk * 1024u),
                                               16, row * MX_KROW + ch * 16u, soff, 0, 0);
    }
    if (wr_u == 2 && lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (__attribute__((address_space(3))) void*)((lds_char*)dst + MX_KTILE),
                                               16, (uint32_t)lane * 16u,
                                               __builtin_amdgcn_readfirstlane((uint32_t)j * (uint32_t)(MX_BC * 4)), 0, 0);
  };
  // tile j: V^T rows d = 0..127, keys [64j, 64j+64), and the scale rows of
  // key blocks 2j, 2j+1
  auto v_to_lds = [&](int j, char* dst) FA_INLINE {
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)j * (uint32_t)MX_BC);
#pragma unroll
    for (int i = 0; i < 8 / NWR; ++i) {
      const uint32_t blk = (uint32_t)(i * NWR + wr_u);  // 1 KiB = 16 rows
      const uint32_t row = blk * 16u + ((uint32_t)lane >> 2);
      const uint32_t ch = ((uint32_t)lane & 3u) ^ vx(row);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)((lds_char*)dst + blk * 1024u),
                                               16, row * (uint32_t)ldv + ch * 16u, soff, 0, 0);
    }
    if (wr_u == 3 && lane < 16)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, (__attribute__((address_space(3))) void*)((lds_char*)dst + MX_VTILE),
                                               16, (uint32_t)lane * 16u,
                                               __builtin_amdgcn_readfirstlane((uint32_t)j * 2u * (uint32_t)D), 0, 0);
  };

  // Q of this lane's row as the B operand of S^T = K Q^T, per 64-wide slab
  // t of the head dimension; its scale word shifted so that byte 2t is the
  // scale of block 2t + h
  intx8 qf[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uintx4 lo = buf_load16(rq, (uint32_t)q * D + (uint32_t)(64 * t + 16 * h));
    const uintx4 hi = buf_load16(rq, (uint32_t)q * D + (uint32_t)(64 * t + 32 + 16 * h));
    qf[t] = intx8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  }
  const int qsw = (int)(__builtin_amdgcn_raw_buffer_load_b32(rqs, (uint32_t)q * 4u, 0, 0) >> (8 * h));

  k_to_lds(0, kbuf(0));
  if (n_tiles > 1) k_to_lds(1, kbuf(1));
  v_to_lds(0, vbuf(0));
  wait_vmem();
  __syncthreads();

  floatx16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = floatx16{};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // S^T of one tile: block kb holds keys kb*32 + key_of_row(row) per
  // accumulator row, i.e. lane half h's register r is key kb*32 + 16h + r
  auto scores = [&](const char* ks, floatx16 (&s)[KB]) FA_INLINE {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = floatx16{};
      const uint32_t row = (uint32_t)kb * 32u + key_of_row((uint32_t)c);
      const char* rp = ks + row * MX_KROW;
      const int ksw = (int)(*reinterpret_cast<const uint32_t*>(ks + MX_KTILE + row * 4u) >> (8 * h));
      // head-dimension slabs t = 0, 1: op_sel 2t picks the scale of block 2t + h
      const intx8 a0 = lds_read32(rp + (((uint32_t)h ^ kx(row)) << 4), rp + (((uint32_t)(2 + h) ^ kx(row)) << 4));
      s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, qf[0], s[kb], 0, 0, 0, ksw, 0, qsw);
      const intx8 a1 = lds_read32(rp + (((uint32_t)(4 + h) ^ kx(row)) << 4), rp + (((uint32_t)(6 + h) ^ kx(row)) << 4));
      s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, qf[1], s[kb], 0, 0, 2, ksw, 2, qsw);
    }
  };

  // online softmax of one tile -> P in E4M3 (bytes 16kb + r of the B operand)
  auto softmax = [&](floatx16 (&s)[KB], intx8& pf, int lim, auto mask_tag, bool& rescale) FA_INLINE -> float {
    constexpr bool MASK = decltype(mask_tag)::value;
    float m_tile;
    if constexpr (MASK) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 16 * h + r;
          const float t = s[kb][r] * c_log2;
          s[kb][r] = key > lim ? -__builtin_inff() : t;
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
    rescale = __ballot(m_tile > m_run + 8.0f) != 0;
    const float m_new = rescale ? fmaxf(m_run, m_tile) : m_run;
    float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float m_use = m_new;
    if constexpr (CAUSAL) {
      const bool empty = m_new == -__builtin_inff();
      alpha = empty ? 1.0f : alpha;
      m_use = empty ? 0.0f : m_new;
    }
    m_run = m_new;
    float lsum = 0.0f;
    float p[KB][16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = MASK ? s[kb][r] - m_use : __builtin_fmaf(s[kb][r], c_log2, -m_use);
        p[kb][r] = __builtin_amdgcn_exp2f(x);
        lsum += p[kb][r];
      }
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r0], p[kb][r0 + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r0 + 2], p[kb][r0 + 3], v, true);
      pf[w] = v;
    }
    l_run = l_run * alpha + lsum;
    return alpha;
  };

  // Tiles without a mask skip the tile max: P = exp2(s*c - m_run) with the
  // running max as it stands, and only when a lane's tile sum exceeds 256
  // (so some P could pass E4M3's 448, or inf on the first tile) is the tile
  // recomputed with its max (softmax_fix).  The running max never exceeds the
  // true row max, so the largest P of a row stays >= 1, as with the max path.
  auto to_e4m3 = [&](const float (&p)[KB][16], intx8& pf) FA_INLINE {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kb = w >> 2, r0 = 4 * (w & 3);
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r0], p[kb][r0 + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(p[kb][r0 + 2], p[kb][r0 + 3], v, true);
      pf[w] = v;
    }
  };
  auto softmax_fast = [&](const floatx16 (&s)[KB], intx8& pf, float& lsum_out) FA_INLINE -> bool {
    float lsum = 0.0f;
    float p[KB][16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_run));
        lsum += p[kb][r];
      }
    to_e4m3(p, pf);
    lsum_out = lsum;
    return __ballot(!(lsum <= 256.0f)) != 0;
  };
  auto softmax_fix = [&](const floatx16 (&s)[KB], intx8& pf, float& lsum_out) FA_INLINE -> float {
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
    float p[KB][16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c_log2, -m_new));
        lsum += p[kb][r];
      }
    to_e4m3(p, pf);
    lsum_out = lsum;
    return alpha;
  };

  // O^T += V^T P^T over the tile's 64 keys, 4 blocks of 32 head columns
  auto accumulate = [&](const char* vs, const intx8& pf) FA_INLINE {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const uint32_t row = (uint32_t)(cb * 32 + c);
      const char* rp = vs + row * MX_VROW;
      const intx8 a = lds_read32(rp + (((uint32_t)h ^ vx(row)) << 4), rp + (((uint32_t)(2 + h) ^ vx(row)) << 4));
      const int vsw = (int)*reinterpret_cast<const uint8_t*>(vs + MX_VTILE + h * D + row);
      oacc[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pf, oacc[cb], 0, 0, 0, vsw, 0, 0x7F7F7F7F);
    }
  };
  auto rescale_o = [&](float alpha) FA_INLINE {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
  };

  intx8 pb;
  floatx16 s1[KB];
  {
    floatx16 s0[KB];
    scores(kbuf(0), s0);
    bool rs;
    if (first_masked == 0)
      softmax(s0, pb, key_lim, std::true_type{}, rs);
    else
      softmax(s0, pb, key_lim, std::false_type{}, rs);
    if (n_tiles > 1) scores(kbuf(1), s1);
  }
  __syncthreads();
  if (n_tiles > 2) k_to_lds(2, kbuf(0));
  wait_vmem();
  __syncthreads();

  auto iteration = [&](int j, auto par_tag, auto has_s2_tag, auto has_s1_tag, auto mask1_tag) FA_INLINE {
    constexpr int P = decltype(par_tag)::value;
    constexpr bool HAS_S2 = decltype(has_s2_tag)::value;
    constexpr bool HAS_S1 = decltype(has_s1_tag)::value;
    if (j + 3 < n_tiles) k_to_lds(j + 3, kbuf(P ^ 1));
    if constexpr (HAS_S1) v_to_lds(j + 1, vbuf(P ^ 1));
    floatx16 s2[KB];
    if constexpr (HAS_S2) scores(kbuf(P), s2);
    intx8 pn;
    bool rs = false;
    float alpha = 1.0f;
    constexpr bool FAST = !decltype(mask1_tag)::value;
    float lsum_f = 0.0f;
    bool fix = false;
    if constexpr (HAS_S1) {
      if constexpr (FAST) fix = softmax_fast(s1, pn, lsum_f);
      else alpha = softmax(s1, pn, key_lim - (j + 1) * MX_BC, mask1_tag, rs);
    }
    accumulate(vbuf(P), pb);
    if constexpr (HAS_S1) {
      asm volatile("" ::"v"(pn));
      if constexpr (FAST) {
        keep(lsum_f);
        if (fix) {
          alpha = softmax_fix(s1, pn, lsum_f);
          rs = true;
        }
        l_run = l_run * alpha + lsum_f;
      }
      keep(l_run);
      if (rs) rescale_o(alpha);
      pb = pn;
      if constexpr (HAS_S2) {
#pragma unroll
        for (int i = 0; i < KB; ++i) s1[i] = s2[i];
      }
      wait_vmem();
      __syncthreads();
    }
  };

  // Iteration j on a plain tile in a fixed order of 8 scheduling segments,
  // one MFMA each: the 4 of S(j+2) (key block m >> 1, head-dimension slab
  // m & 1), then the 4 of P(j) V(j) (output block m - 4).  Segment i also
  // reads the LDS operand (and scale) of the MFMA PF segments later and
  // computes 4 scores of the softmax of tile j+1 (AHEAD scores in advance),
  // packing the four it has finished into E4M3.
  auto iteration_seg = [&](int j, auto par_tag) FA_INLINE {
    constexpr int P = decltype(par_tag)::value;
    // measured best: PF 2 with 6 scores ahead at 8 waves, 4 ahead at 4 waves
    constexpr int PF = 2, AHEAD = NW == 8 ? 6 : 4;
    if (j + 3 < n_tiles) k_to_lds(j + 3, kbuf(P ^ 1));
    v_to_lds(j + 1, vbuf(P ^ 1));
    const char* ks = kbuf(P);
    const char* vs = vbuf(P);
    auto afrag = [&](int m, int& sc) FA_INLINE -> intx8 {
      if (m < 4) {
        const uint32_t row = (uint32_t)(m >> 1) * 32u + key_of_row((uint32_t)c);
        const char* rp = ks + row * MX_KROW;
        const uint32_t t4 = 4u * (uint32_t)(m & 1);
        sc = (int)(*reinterpret_cast<const uint32_t*>(ks + MX_KTILE + row * 4u) >> (8 * h));
        return lds_read32(rp + (((t4 + (uint32_t)h) ^ kx(row)) << 4), rp + (((t4 + 2u + (uint32_t)h) ^ kx(row)) << 4));
      }
      const uint32_t row = (uint32_t)((m - 4) * 32 + c);
      const char* rp = vs + row * MX_VROW;
      sc = (int)*reinterpret_cast<const uint8_t*>(vs + MX_VTILE + h * D + row);
      return lds_read32(rp + (((uint32_t)h ^ vx(row)) << 4), rp + (((2u + (uint32_t)h) ^ vx(row)) << 4));
    };
    floatx16 s2[KB];
    s2[0] = floatx16{};
    s2[1] = floatx16{};
    intx8 af[PF + 1];
    int asc[PF + 1];
    float pe[32];
    intx8 pn;
    float lsum = 0.0f;
    auto score = [&](int r) FA_INLINE {  // key block r >> 4, accumulator row r & 15
      pe[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r >> 4][r & 15], c_log2, -m_run));
      lsum += pe[r];
    };
    auto pack = [&](int w) FA_INLINE {  // scores 4w .. 4w+3 -> B operand word w
      int v = __builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w], pe[4 * w + 1], 0, false);
      v = __builtin_amdgcn_cvt_pk_fp8_f32(pe[4 * w + 2], pe[4 * w + 3], v, true);
      pn[w] = v;
    };
#pragma unroll
    for (int i = 0; i < PF; ++i) af[i] = afrag(i, asc[i]);
#pragma unroll
    for (int r = 0; r < AHEAD; ++r) score(r);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int nxt = i + PF;
      if (nxt < 8) af[nxt % (PF + 1)] = afrag(nxt, asc[nxt % (PF + 1)]);
#pragma unroll
      for (int r = 4 * i + AHEAD; r < 4 * i + 4 + AHEAD; ++r)
        if (r < 32) score(r);
      pack(i);
      const int slot = i % (PF + 1);
      if (i < 4) {
        const int kb = i >> 1;
        if (i & 1)
          s2[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[slot], qf[1], s2[kb], 0, 0, 2, asc[slot], 2, qsw);
        else
          s2[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[slot], qf[0], s2[kb], 0, 0, 0, asc[slot], 0, qsw);
      } else {
        oacc[i - 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[slot], pb, oacc[i - 4], 0, 0, 0, asc[slot], 0,
                                                                       0x7F7F7F7F);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const bool fix = __ballot(!(lsum <= 256.0f)) != 0;
    asm volatile("" ::"v"(pn));
    keep(lsum);
    float alpha = 1.0f;
    if (fix) {
      alpha = softmax_fix(s1, pn, lsum);
      rescale_o(alpha);
    }
    l_run = l_run * alpha + lsum;
    keep(l_run);
    pb = pn;
    s1[0] = s2[0];
    s1[1] = s2[1];
    wait_vmem();
    __syncthreads();
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using T = std::true_type;
  using F = std::false_type;
  auto run = [&](int j0, int j1, auto mask_tag) FA_INLINE {
    int j = j0;
    if (j < j1 && (j & 1)) {
      iteration(j, P1{}, T{}, T{}, mask_tag);
      ++j;
    }
    for (; j + 1 < j1; j += 2) {
      if constexpr (!decltype(mask_tag)::value) {
        iteration_seg(j, P0{});
        iteration_seg(j + 1, P1{});
      } else {
        iteration(j, P0{}, T{}, T{}, mask_tag);
        iteration(j + 1, P1{}, T{}, T{}, mask_tag);
      }
    }
    if (j < j1) iteration(j, P0{}, T{}, T{}, mask_tag);
  };
  const int j_end = n_tiles - 2 > 0 ? n_tiles - 2 : 0;
  int j_split = first_masked - 1;
  j_split = j_split < 0 ? 0 : (j_split > j_end ? j_end : j_split);
  run(0, j_split, F{});
  // (KS2: the second group's range may end in a ragged and a fully masked tile)
  if constexpr (CAUSAL || KS2) run(j_split, j_end, T{});
  if (n_tiles >= 2) {
    const int j = n_tiles - 2;
    const bool mask = n_tiles - 1 >= first_masked;
    if (j & 1) {
      if (mask) iteration(j, P1{}, F{}, T{}, T{}); else iteration(j, P1{}, F{}, T{}, F{});
    } else {
      if (mask) iteration(j, P0{}, F{}, T{}, T{}); else iteration(j, P0{}, F{}, T{}, F{});
    }
  }
  if ((n_tiles - 1) & 1) iteration(n_tiles - 1, P1{}, F{}, F{}, F{}); else iteration(n_tiles - 1, P0{}, F{}, F{}, F{});

  float l_tot = wave_sum_halves(l_run);
  if constexpr (KS2) {
    // the second key group hands (O, m, l) of its keys to the first through
    // LDS: m = max(m0, m1), a_g = 2^(m_g - m), O = a0 O0 + a1 O1, l = a0 l0 + a1 l1
    __syncthreads();  // every wave is done with the K/V stages
    float* const xo = reinterpret_cast<float*>(smem);  // [64 values][256 lanes]
    float* const xs = xo + 64 * 256;                  // m, l: [2][256 lanes]
    const int li = wr * 64 + lane;
    if (kg_u == 1) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(cb * 16 + r) * 256 + li] = oacc[cb][r];
      xs[li] = m_run;
      xs[256 + li] = l_tot;
    }
    __syncthreads();
    if (kg_u == 1) return;
    const float m1 = xs[li];
    const float m = m_run > m1 ? m_run : m1;
    const float a0 = m_run == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
    const float a1 = m1 == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[cb][r] = oacc[cb][r] * a0 + xo[(cb * 16 + r) * 256 + li] * a1;
    l_tot = l_tot * a0 + xs[256 + li] * a1;
    m_run = m;
  }
  constexpr bool CAN_BE_EMPTY = CAUSAL || KS2;  // a row may see no key (of a group)
  const float inv_l = (CAN_BE_EMPTY && l_tot == 0.0f) ? 0.0f : 1.0f / l_tot;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) store_bf16_row_block(ro, (uint32_t)q, cb, h, oacc[cb], inv_l);
  if (h == 0 && q < Nq)
    LSE[bq + q] = (CAN_BE_EMPTY && l_tot == 0.0f) ? -__builtin_inff() : (m_run + __log2f(l_tot)) * 0.69314718055994530942f;
}


// ---------------------------------------------------------------- MXFP8 encoding
// One thread per block of 32 elements: the block's largest magnitude sets
// the E8M0 scale 2^(floor(log2 amax) - 8) (an all-zero block gets 2^-127),
// every element is divided by it (exact: a power of two) and rounded to
// E4M3 by v_cvt_pk_fp8_f32 (nearest, ties to even) after saturation to
// +-448 (the conversion itself turns overflow into NaN).
__device__ inline uint32_t block_scale(float amax) {
  if (!(amax > 0.0f)) return 0u;  // zero block (NaN input: left to the elements)
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 127;  // floor(log2) of a normal value
  const int ef = e == -127 ? (31 - __builtin_clz(__float_as_uint(amax) & 0x7FFFFFu)) - 149 : e;  // subnormal amax
  int sh = ef - 8;
  sh = sh < -127 ? -127 : (sh > 127 ? 127 : sh);
  return (uint32_t)(sh + 127);
}
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// saturate to +-448; NaN stays NaN (and converts to the E4M3 NaN)
__device__ inline float sat448(float x) { return __builtin_isnan(x) ? x : fminf(fmaxf(x, -448.0f), 448.0f); }
// 4 floats -> 4 E4M3 bytes in one dword
__device__ inline uint32_t pack4(float a, float b, float c, float d) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), v, true);
  return (uint32_t)v;
}

// X [BH, N, d] bf16 -> E [BH, N, d] E4M3, S [BH, ldS, d/32] E8M0
__global__ void __launch_bounds__(256) mx_quantize_rows_kernel(const uint16_t* __restrict__ X, uint8_t* __restrict__ E,
                                                               uint8_t* __restrict__ S, int64_t N, int64_t ldS,
                                                               int64_t nblocks) {
  constexpr int BPR = D / 32;  // blocks per row
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks; b += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = b / BPR;  // global row bh*N + n
    const int blk = (int)(b - row * BPR);
    const int64_t bh = row / N, n = row - bh * N;
    const uint16_t* x = X + row * D + blk * 32;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uintx4 w = *reinterpret_cast<const uintx4*>(x + 8 * i);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[8 * i + 2 * k] = __uint_as_float(w[k] << 16);
        v[8 * i + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const uint32_t sbyte = block_scale(amax);
    const float inv = __uint_as_float((254u - sbyte) << 23);  // 2^(127 - sbyte), exact (sbyte in [0, 254])
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // sbyte = 0 gives inv = 2^127, finite; the block is all zero then
      out[i] = pack4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
    }
    uint8_t* e = E + row * D + blk * 32;
    *reinterpret_cast<uintx4*>(e) = uintx4{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<uintx4*>(e + 16) = uintx4{out[4], out[5], out[6], out[7]};
    S[(bh * ldS + n) * BPR + blk] = (uint8_t)sbyte;
  }
}

// V [BH, Nk, d] bf16 -> Vt [BH, d, ldv] E4M3 (keys >= Nk zero), Vs [BH, ldv/32, d]
// one thread per (bh, key block, column); consecutive threads take
// consecutive columns, so each key row is read coalesced
__global__ void __launch_bounds__(256) mx_quantize_vt_kernel(const uint16_t* __restrict__ V, uint8_t* __restrict__ Vt,
                                                             uint8_t* __restrict__ Vs, int64_t Nk, int64_t ldv,
                                                             int64_t nitems) {
  const int64_t kbs = ldv / 32;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < nitems; it += (int64_t)gridDim.x * blockDim.x) {
    const int col = (int)(it % D);
    const int64_t t = it / D;
    const int64_t kb = t % kbs, bh = t / kbs;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int64_t key = kb * 32 + e;
      v[e] = key < Nk ? bf16_to_f32(V[(bh * Nk + key) * D + col]) : 0.0f;
      amax = fmaxf(amax, fabsf(v[e]));
    }
    const uint32_t sbyte = block_scale(amax);
    const float inv = __uint_as_float((254u - sbyte) << 23);
    uint32_t out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = pack4(v[4 * i] * inv, v[4 * i + 1] * inv, v[4 * i + 2] * inv, v[4 * i + 3] * inv);
    uint8_t* dst = Vt + (bh * D + col) * ldv + kb * 32;
    *reinterpret_cast<uintx4*>(dst) = uintx4{out[0], out[1], out[2], out[3]};
    *reinterpret_cast<uintx4*>(dst + 16) = uintx4{out[4], out[5], out[6], out[7]};
    Vs[(bh * kbs + kb) * D + col] = (uint8_t)sbyte;
  }
}

}  // namespace

// Workgroups of 8 waves (256 query rows) share each K/V tile between twice
// the rows; they pay on grids that still give every CU a workgroup of them.
constexpr int64_t kMx8WaveMinWorkgroups = 256;

namespace {
template <int NW, bool KS2 = false>
int launch_mxfp8_nw(const MxArgs& a, hipStream_t stream) {
  constexpr int BR = KS2 ? 16 * NW : 32 * NW;  // query rows per workgroup
  int n_qtiles = (int)((a.Nq + BR - 1) / BR);
  const float c_log2 = (float)((double)a.scale * 1.4426950408889634074);
  const uint8_t *q = static_cast<const uint8_t*>(a.Q8), *qs = static_cast<const uint8_t*>(a.Qs);
  const uint8_t *k = static_cast<const uint8_t*>(a.K8), *ks = static_cast<const uint8_t*>(a.Ks);
  const uint8_t *v = static_cast<const uint8_t*>(a.Vt8), *vs = static_cast<const uint8_t*>(a.Vs);
  uint16_t* o = static_cast<uint16_t*>(a.O);
  float* lse = a.LSE;
  int nq = (int)a.Nq, nk = (int)a.Nk, ldv = (int)a.ldv;
  float cl = c_log2;
  void* args[] = {&q, &qs, &k, &ks, &v, &vs, &o, &lse, &nq, &nk, &ldv, &n_qtiles, &cl};
  const bool neg = a.scale < 0.0f;
  const void* fn = a.causal ? (neg ? (const void*)&fa_fwd_mxfp8_kernel<true, true, NW, KS2>
                                    : (const void*)&fa_fwd_mxfp8_kernel<false, true, NW, KS2>)
                            : (neg ? (const void*)&fa_fwd_mxfp8_kernel<true, false, NW, KS2>
                                    : (const void*)&fa_fwd_mxfp8_kernel<false, false, NW, KS2>);
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(a.BH * n_qtiles)), dim3(64 * NW), args, 0, stream);
  return e == hipSuccess ? 0 : (int)e;
}

}  // namespace

int launch_fa_fwd_mxfp8(const MxArgs& a, hipStream_t stream) {
  const int64_t wg8 = a.BH * ((a.Nq + 255) / 256);
  if (wg8 >= kMx8WaveMinWorkgroups) return launch_mxfp8_nw<8>(a, stream);
  // two key groups of 4 waves on 128 rows where 128-row workgroups give every
  // CU one and the keys are long enough for both groups to run a few tiles
  if (a.BH * ((a.Nq + 127) / 128) >= kMx8WaveMinWorkgroups && a.Nk >= 1024) return launch_mxfp8_nw<8, true>(a, stream);
  return launch_mxfp8_nw<4>(a, stream);
}

int launch_mx_quantize_rows(const void* X, void* E, void* S, int64_t BH, int64_t N, int64_t ldS, hipStream_t stream) {
  int64_t nblocks = BH * N * (D / 32);
  if (nblocks == 0) return 0;
  const int64_t want = (nblocks + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  const uint16_t* x = static_cast<const uint16_t*>(X);
  uint8_t* e = static_cast<uint8_t*>(E);
  uint8_t* sc = static_cast<uint8_t*>(S);
  int64_t n = N, ld = ldS;
  void* args[] = {&x, &e, &sc, &n, &ld, &nblocks};
  return hipLaunchKernel((const void*)&mx_quantize_rows_kernel, dim3(grid), dim3(256), args, 0, stream) == hipSuccess ? 0 : 1;
}

int launch_mx_quantize_vt(const void* V, void* Vt, void* Vs, int64_t BH, int64_t Nk, int64_t ldv, hipStream_t stream) {
  int64_t nitems = BH * (ldv / 32) * D;
  if (nitems == 0) return 0;
  const int64_t want = (nitems + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  const uint16_t* v = static_cast<const uint16_t*>(V);
  uint8_t* vt = static_cast<uint8_t*>(Vt);
  uint8_t* vs = static_cast<uint8_t*>(Vs);
  int64_t nk = Nk, ld = ldv;
  void* args[] = {&v, &vt, &vs, &nk, &ld, &nitems};
  return hipLaunchKernel((const void*)&mx_quantize_vt_kernel, dim3(grid), dim3(256), args, 0, stream) == hipSuccess ? 0 : 1;
}

const char* mxfp8_config_string() {
  return "gfx950 fa_fwd_mxfp8 v3: BR=256 (8 waves x 32 rows) on grids of >= 256 such workgroups, else 128 "
         "(4 waves), BC=64, 3-stage pipeline, plain tiles in 8 fixed MFMA segments, "
         "v_mfma_scale_f32_32x32x64_f8f6f4 for S^T=K.Q^T and O^T+=V^T.P^T, P in E4M3 (scale 1), "
         "no tile max unless a tile sum exceeds 256";
}

}  // namespace fa06

// fa_device.h -- device helpers shared by the attention kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa06 {
namespace {

constexpr int D = 128;           // head size (d = d_v)
constexpr int ROW_BYTES = D * 2; // one bf16 row
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr float LOG2E = 1.44269504088896340736f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef unsigned uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned uintx4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Buffer resource: base, no stride, num_records bytes; dword3 selects the
// 32-bit data format, which gfx9-family raw buffer accesses require.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ inline uintx4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(uintx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}

// LDS tiles hold rows of 2*DIM bytes (DIM/8 chunks of 16 bytes); the chunk
// index is XOR-swizzled per row.  Three swizzles, one per way a tile is read:
//   SWZ_ROW  16 lanes reading one chunk of 16 consecutive rows (ds_read_b128
//            MFMA operands) hit 16 distinct 16-byte bank groups.
//   SWZ_TR   the transposing reads (ds_read_b64_tr_b16) of 32 lanes cover
//            a 64-byte band of 4 rows; the 4 rows land in distinct groups.
//   SWZ_BOTH both at once, for tiles read both ways.
// With 256- or 512-byte rows every row starts at the same bank, so the XOR
// must separate rows: ROW uses chunk ^ (row % 16), TR chunk ^ 4*(row % 4),
// BOTH chunk ^ (4*(row % 4) + (row / 4) % 4) (the high two bits separate the
// 4 rows of a band, and the map is one-to-one over 16 rows).  With 128-byte
// rows (DIM = 64) odd rows start half way round the banks, so row pairs
// already differ; the XOR acts on row / 2: chunk ^ (4*((row/2) % 2) +
// (row/4) % 4), which serves both access patterns.  With 384-byte rows
// (DIM = 192, 24 chunks) odd rows also start half way round; ROW uses
// chunk ^ ((row/2) % 8), which stays inside the chunk's aligned group of 8
// (so inside the row) and makes 16 consecutive rows hit 16 distinct groups;
// BOTH uses the 128-byte-row formula, which also keeps a chunk inside its
// group of 8 and separates the two row pairs of a transposing read.
enum Swz { SWZ_ROW = 0, SWZ_TR = 1, SWZ_BOTH = 2 };

template <int S, int DIM = D>
__device__ inline uint32_t swz_chunk(uint32_t row, uint32_t ch) {
  static_assert(DIM == 64 || DIM == 128 || DIM == 256 || (DIM == 192 && S != SWZ_TR), "row width");
  if constexpr (DIM == 64 || (DIM == 192 && S == SWZ_BOTH)) return ch ^ ((((row >> 1) & 1u) << 2) | ((row >> 2) & 3u));
  else if constexpr (DIM == 192) return ch ^ ((row >> 1) & 7u);
  else if constexpr (S == SWZ_ROW) return ch ^ (row & 15u);
  else if constexpr (S == SWZ_TR) return ch ^ ((row & 3u) << 2);
  else return ch ^ (((row & 3u) << 2) | ((row >> 2) & 3u));
}
template <int S, int DIM = D>
__device__ inline uint32_t swz(uint32_t row, uint32_t ch) {
  return row * (uint32_t)(2 * DIM) + (swz_chunk<S, DIM>(row, ch) << 4);
}
__device__ inline uint32_t k_swz(uint32_t row, uint32_t ch) { return swz<SWZ_ROW>(row, ch); }
__device__ inline uint32_t v_swz(uint32_t row, uint32_t ch) { return swz<SWZ_TR>(row, ch); }

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
// LDS linearly.  The tile is contiguous in memory and in LDS, so byte x of
// the LDS tile is row x / (2*DIM), physical chunk (x % (2*DIM)) / 16 (a row
// may straddle two 1 KiB blocks when 2*DIM does not divide 1024).  The
// swizzle is applied on the source side: the lane that fills physical chunk
// P of row r loads logical chunk P ^ f(r) (every swizzle is an XOR, its own
// inverse).  `ROWS` rows starting at global row `row0` (scalar) go to `lds`;
// each of the workgroup's NW waves issues ROWS*2*DIM/1024/NW instructions.
template <int ROWS, int S, int DIM = D, int NW = NWAVES>
__device__ inline void tile_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t row0, char* lds, int wave, int lane) {
  constexpr uint32_t RB = 2 * DIM;          // bytes per row
  const uint32_t soff = __builtin_amdgcn_readfirstlane(row0 * RB);
  static_assert(ROWS * (int)RB % (1024 * NW) == 0, "tile must be whole 1 KiB blocks per wave");
  constexpr int N_INST = ROWS * (int)RB / 1024 / NW;
  if constexpr ((RB & (RB - 1)) == 0 && (NW * 1024 / (int)RB) % 16 == 0) {
    // Instruction i covers the rows of instruction 0 plus i*NW*1024/RB, a
    // multiple of 16 rows, so every swizzle maps them alike: one vector
    // offset, and the step in the scalar offset.
    const uint32_t row = (uint32_t)wave * (1024u / RB) + (uint32_t)lane / (RB / 16u);
    const uint32_t pos = (uint32_t)lane & (RB / 16u - 1u);
    const uint32_t voff = row * RB + (swz_chunk<S, DIM>(row, pos) << 4);
#pragma unroll
    for (int i = 0; i < N_INST; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)((lds_char*)lds + (uint32_t)(i * NW + wave) * 1024u), 16, voff,
          soff + (uint32_t)(i * NW) * 1024u, 0, 0);
    return;
  }
#pragma unroll
  for (int i = 0; i < N_INST; ++i) {
    const uint32_t blk = (uint32_t)(i * NW + wave);          // which 1 KiB block
    uint32_t row, pos;                                       // pos: physical chunk in the row
    if constexpr ((RB & (RB - 1)) == 0) {
      // whole rows per block: 1024 / RB rows, RB / 16 lanes per row
      row = blk * (1024u / RB) + (uint32_t)lane / (RB / 16u);
      pos = (uint32_t)lane & (RB / 16u - 1u);
    } else {
      const uint32_t x = blk * 1024u + 16u * (uint32_t)lane;  // byte of the tile
      row = x / RB;
      pos = (x % RB) >> 4;
    }
    const uint32_t ch = swz_chunk<S, DIM>(row, pos);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)((lds_char*)lds + blk * 1024u), 16,
        row * RB + (ch << 4), soff, 0, 0);
  }
}

// Workgroup id -> (head, tile) of a grid of n_tiles tiles per head.
// Workgroups are dispatched round-robin over the 8 XCDs, so the id is
// remapped to give each XCD a contiguous share of the tiles (the tiles of one
// head share that head's K/V in the XCD's L2).  With `lpt` (the tiles' work
// falls with the tile index, as in causal attention) and a share that holds
// whole heads, the share is ordered tile-major across its heads, so the
// longest tiles of all those heads start first.
__device__ inline void xcd_tile_map(int bid, int nblk, int n_tiles, bool lpt, int& bh, int& t) {
  const int nfull = nblk & ~7;
  const int per = nfull >> 3;
  if (lpt && bid < nfull && per % n_tiles == 0) {
    const int hpc = per / n_tiles;  // heads per XCD
    const int i = bid >> 3;
    bh = (bid & 7) * hpc + i % hpc;
    t = i / hpc;
    return;
  }
  if (bid < nfull) bid = (bid & 7) * per + (bid >> 3);
  bh = bid / n_tiles;
  t = bid - bh * n_tiles;
}

// Heads that read the same rows of a dense bias.  A bias broadcast over the
// batch (batch stride 0), over the heads (head stride 0) or over both is one
// block of rows for g heads at once; bh = outer * os + m * ms for member
// m < g of group `outer`.  g = 1 when nothing is shared or the bias has no
// rows (a per-key bias is a few KiB and stays in cache anyway).
struct HeadGroup {
  int g, os, ms;
};
__device__ inline HeadGroup bias_head_group(int B, int H, int64_t sb, int64_t sh, int64_t sq) {
  const bool over_b = sb == 0 && B > 1;
  const bool over_h = sh == 0 && H > 1;
  if (sq == 0 || (!over_b && !over_h)) return {1, 1, 0};
  if (over_b && over_h) return {B * H, 0, 1};
  if (over_b) return {B, 1, H};  // members are the batches of head `outer`
  return {H, H, 1};              // members are the heads of batch `outer`
}

// xcd_tile_map over "logical heads" in which the members of a bias group
// are adjacent, and without `lpt` also innermost: workgroups that read the
// same bias block get consecutive ids within one XCD's share, so they run
// at the same time and the block is fetched from HBM once instead of g times.
__device__ inline void grouped_tile_map(int bid, int nblk, int n_tiles, bool lpt, HeadGroup hg, int& bh, int& t) {
  if (lpt) {
    int lh;
    xcd_tile_map(bid, nblk, n_tiles, true, lh, t);
    const int outer = lh / hg.g;
    bh = outer * hg.os + (lh - outer * hg.g) * hg.ms;
    return;
  }
  const int nfull = nblk & ~7;
  if (bid < nfull) bid = (bid & 7) * (nfull >> 3) + (bid >> 3);
  const int rest = bid / hg.g;  // logical order (outer, tile, member)
  const int m = bid - rest * hg.g;
  const int outer = rest / n_tiles;
  t = rest - outer * n_tiles;
  bh = outer * hg.os + m * hg.ms;
}

// Every helper lambda of a kernel is inlined: loop bodies must stay one
// straight-line region with all state in registers.
#define FA_INLINE __attribute__((always_inline))

// Wait until this wave's outstanding global loads (incl. LDS-direct) landed.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Keeps a value live at this point, so the instructions that produce it stay
// ahead of it (in the same basic block) instead of being sunk into a later
// block by the compiler.
__device__ inline void keep(const bf16x8& x) { asm volatile("" ::"v"(__builtin_bit_cast(uintx4, x))); }
__device__ inline void keep(float x) { asm volatile("" ::"v"(x)); }

// Transposing LDS read of an MFMA A operand: lane (16-lane group g, i16)
// gets 8 bf16 of column block `cb` (32 columns) at rows r0 and r0 + 8 of
// `tile`, where r0 = row_base + 4*(g/2) + (i16/4).  Rows are the k index in
// the order the 32x32 accumulator holds them (rows 4h..4h+3 and 8+4h..8+4h+3
// of each 16), so an accumulator turned into bf16 is the matching B operand.
template <int S, int DIM = D>
__device__ inline bf16x8 tr_read_a(const char* tile, uint32_t row_base, int cb, int lane) {
  const int g = lane >> 4;
  const int i16 = lane & 15;
  const int sub = i16 >> 2;
  const int q4 = i16 & 3;
  const int hh = g >> 1;
  const int d0 = cb * 32 + (g & 1) * 16 + q4 * 4;
  const uint32_t ch = (uint32_t)d0 >> 3;
  const uint32_t within = ((uint32_t)d0 & 7u) * 2u;
  const uint32_t r0 = row_base + 4 * hh + sub;
  const uint32_t r1 = r0 + 8;
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)((lds_char*)tile + swz<S, DIM>(r0, ch) + within));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)((lds_char*)tile + swz<S, DIM>(r1, ch) + within));
  // move the two 4-element results as whole dwords: a = {lo[0..3], hi[0..3]}
  const uintx2 lo2 = __builtin_bit_cast(uintx2, lo);
  const uintx2 hi2 = __builtin_bit_cast(uintx2, hi);
  return __builtin_bit_cast(bf16x8, uintx4{lo2.x, lo2.y, hi2.x, hi2.y});
}

// Row read of an MFMA A operand: lane (c, h) gets chunk 2t+h of row
// row_base + c (8 bf16 along the contraction index).
template <int S, int DIM = D>
__device__ inline bf16x8 row_read_a(const char* tile, uint32_t row_base, int t, int c, int h) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uintx4*>(tile + swz<S, DIM>(row_base + c, 2 * t + h)));
}

// Stores a 32x32 fp32 accumulator block holding (column block cb, 32 rows
// of 4-row groups) as bf16: lane (c, h) writes row `row` (its column c of
// the transposed accumulator), columns cb*32 + 8*g4 + 4h .. +3.
template <int DIM = D>
__device__ inline void store_bf16_row_block(__amdgpu_buffer_rsrc_t r, uint32_t row, int cb, int h,
                                            const floatx16& acc, float mul) {
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    const int d = cb * 32 + g4 * 8 + 4 * h;
    const __bf16 a0 = (__bf16)(acc[4 * g4 + 0] * mul);
    const __bf16 a1 = (__bf16)(acc[4 * g4 + 1] * mul);
    const __bf16 a2 = (__bf16)(acc[4 * g4 + 2] * mul);
    const __bf16 a3 = (__bf16)(acc[4 * g4 + 3] * mul);
    const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, a0) | ((uint32_t)__builtin_bit_cast(uint16_t, a1) << 16);
    const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, a2) | ((uint32_t)__builtin_bit_cast(uint16_t, a3) << 16);
    __builtin_amdgcn_raw_buffer_store_b64(uintx2{w0, w1}, r, row * (uint32_t)(2 * DIM) + d * 2, 0, 0);
  }
}

}  // namespace
}  // namespace fa06

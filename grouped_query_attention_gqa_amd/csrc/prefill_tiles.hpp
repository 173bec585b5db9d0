// LDS tiles of 64 bf16 rows shared by the causal prefill kernels (forward
// and backward), and the per-lane offsets of the two ways the kernels read
// them as 32x32x16 MFMA operands.
//
// A tile holds 64 rows of D bf16 values (rows are keys, or query positions
// in the backward key/value kernel), in 16-byte chunks, with the chunk index
// XOR-ed by a permutation g of the row index (period 16 rows).  That single
// layout serves both reads without bank conflicts:
//   row reads   (ds_read_b128): an operand whose lane index l%32 is the row
//               and whose k-group l/32 picks 8 consecutive columns;
//   transposed  (two ds_read_b64_tr_b16): an operand whose lane index l%32
//               is the column and whose k-group l/32 picks 8 rows, namely
//               rows 16c + 4(l/32) + 0..3 and 16c + 8 + 4(l/32) + 0..3 of
//               16-row chunk c.  This is the row order in which a 32x32
//               MFMA result holds its rows (row 8(r/4) + 4(l/32) + r%4 in
//               register r), so a result can be fed, converted to bf16, as
//               the other operand of the next product.
// Tiles are filled by direct global-to-LDS buffer loads issued by a whole
// 256-thread workgroup, 16 bytes per lane per instruction.
#pragma once

#include "gqa_device.hpp"

namespace gqa {
namespace tiles {

constexpr int kRows = 64;       // rows per tile
constexpr int kThreads = 256;   // threads of the workgroups that fill a tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Physical 16-byte chunk of logical chunk c in row r: c ^ g(r).  The LDS
// serves 256 bytes per cycle (64 banks of 4 bytes): a row read (16 bytes
// per lane) takes 16 lanes per cycle, which are 16 consecutive rows at one
// logical chunk, and a transposed read (8 bytes per lane) takes 32 lanes,
// which are 4 consecutive rows (aligned to 4) at 4 consecutive chunks
// (aligned to 4).  Both are conflict-free when the 16 or 32 accesses land
// on distinct bank groups:
//   D = 128 (16 chunks, 256 B per row): g(r) swaps the two 2-bit fields of
//     r mod 16.  It is a permutation of 0..15 (row reads), and its upper
//     two bits, r mod 4, differ within every aligned quad of rows
//     (transposed reads: 4 rows x 4 chunks give 16 distinct chunks).
//   D = 64 (8 chunks, 128 B per row, two rows per 256 B): g(r) = 4 * (bit 1
//     of r) + (bits 2..3 of r).  Rows of one parity get distinct g (row
//     reads), and rows r, r + 2 of an aligned quad differ in g's upper bit
//     (transposed reads).
// (A one-bit rotation of r, used before, leaves the transposed reads with
// two-way conflicts; the replacement was measured conflict-free with the
// SQ_LDS_BANK_CONFLICT counter.)
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if (CPR == 16) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
  return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Global byte offsets (relative to the tile's first row) of the chunks that
// thread tid deposits: physical chunk p = tid + 256 i of the tile, at LDS
// byte 16 p, holds the logical chunk the swizzle places there.
template <int D>
struct TileFill {
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = kRows * CPR / kThreads;
  int src_off[LOADS];

  __device__ __forceinline__ explicit TileFill(int tid) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int p = tid + kThreads * i;
      const int row = p / CPR;
      src_off[i] = row * D * 2 + swz<CPR>(row, p % CPR) * 16;
    }
  }

  // Start loading rows row0 .. row0+63 of the buffer behind `src` into
  // `dst`; rows past the resource's range arrive as zeros.  Wave w fills
  // its 1 KiB blocks of each 4 KiB slice of the tile.
  __device__ __forceinline__ void issue(__bf16* dst, __amdgpu_buffer_rsrc_t src, int w, int row0) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int at = (w * 64 + kThreads * i) * 8;   // bf16 units
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)(dst + at), 16, row0 * D * 2 + src_off[i],
                                               0, 0, 0);
    }
  }

  // The same rows of two buffers into two tiles (K and V, or Q and dO),
  // the two loads of each chunk issued back to back.
  __device__ __forceinline__ void issue2(__bf16* dst_a, __amdgpu_buffer_rsrc_t src_a, __bf16* dst_b,
                                         __amdgpu_buffer_rsrc_t src_b, int w, int row0) const {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int at = (w * 64 + kThreads * i) * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src_a, (lds_ptr_t)(dst_a + at), 16,
                                               row0 * D * 2 + src_off[i], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src_b, (lds_ptr_t)(dst_b + at), 16,
                                               row0 * D * 2 + src_off[i], 0, 0, 0);
    }
  }
};

// One float per lane of a wavefront, dst[lane] = the float at byte offset
// voff of `src` (zero past its range), by a direct global-to-LDS load.
__device__ __forceinline__ void load_floats_lds(float* dst, __amdgpu_buffer_rsrc_t src, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)dst, 4, voff, 0, 0, 0);
}

// Element offset of logical chunk `chunk` of tile row `row`.
template <int D>
__device__ __forceinline__ int row_offset(int row, int chunk) {
  return row * D + swz<D / 8>(row, chunk) * 8;
}

// Transposed read of 16-row chunk c, column block db (32 columns), for lane
// `lane`: `rd` is the element offset of the first ds_read_b64_tr_b16 and
// rd + 8 D + dx that of the second (the same column 8 rows further down).
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int c, int db, int& rd, int& dx) {
  constexpr int CPR = D / 8;
  const int L = lane & 15;
  const int half = 16 * ((lane >> 4) & 1);   // which 16 of the 32 columns
  const int row = 16 * c + 4 * (lane >> 5) + (L >> 2);
  const int col = 32 * db + half + 4 * (L & 3);
  rd = row * D + swz<CPR>(row, col >> 3) * 8 + (col & 7);
  dx = (swz<CPR>(row + 8, col >> 3) - swz<CPR>(row, col >> 3)) * 8;
}

// The bf16x8 operand of a transposed read at (rd, dx).
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const __bf16* tile, int rd, int dx) {
  return concat(lds_read_tr16(tile + rd), lds_read_tr16(tile + rd + 8 * D + dx));
}

}  // namespace tiles
}  // namespace gqa

// ns_layout.h - index arithmetic of the Newton–Schulz kernels.
//
// Everything that turns (workgroup, thread, loop counter) into a global or
// LDS offset lives here as plain inline functions, usable from device code
// and from the host-side bounds checker (ns_boundscheck.cpp), so that the
// checker walks exactly the addresses the kernels touch.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define NS_HD __host__ __device__ __forceinline__
#else
#define NS_HD inline
#endif

namespace ns {

// Work modes of the tiled MFMA kernel.
enum GemmMode : int {
  MODE_GRAM = 0,    // lower-triangle tiles of P Pᵀ, mirrored, diagonal split
  MODE_POLY = 1,    // lower-triangle tiles of b A + c A A (+ a on diagonal)
  MODE_UPD_ROW = 2, // rectangle tiles of O_C X + d_C[row] * X
  MODE_UPD_COL = 3  // rectangle tiles of X O_C + d_C[col] * X
};

NS_HD constexpr bool mode_is_tri(int mode) { return mode == MODE_GRAM || mode == MODE_POLY; }

// How an operand tile is read from global memory.
enum OperandLayout : int {
  KCONT = 0,  // element (i, k) at base + i * ld + k   (k contiguous)
  MCONT = 1   // element (i, k) at base + k * ld + i   (i contiguous)
};

// The hardware hands workgroup w to XCD (w mod 8).  Remap so that each XCD
// works through one contiguous range of logical tile ids (neighbouring tiles
// share operand panels, which then stay in that XCD's L2).
NS_HD int xcd_remap(int w, int G) {
  const int per = G / 8, rem = G % 8;
  const int xcd = w % 8, local = w / 8;
  return (xcd < rem) ? xcd * (per + 1) + local
                     : rem * (per + 1) + (xcd - rem) * per + local;
}

// q-th tile of a lower triangle, row by row: (0,0) (1,0) (1,1) (2,0) ...
NS_HD void tri_decode(int q, int& ti, int& tj) {
  int i = (int)((__builtin_sqrtf(8.0f * (float)q + 1.0f) - 1.0f) * 0.5f);
  while (i > 0 && i * (i + 1) / 2 > q) --i;
  while ((i + 1) * (i + 2) / 2 <= q) ++i;
  ti = i;
  tj = q - i * (i + 1) / 2;
}

// q-th tile of a tiles_m x tiles_n rectangle, in groups of 8 tile rows
// walked column by column (a group shares its 8 row panels).
NS_HD void rect_decode(int q, int tiles_m, int tiles_n, int& ti, int& tj) {
  const int G = 8;
  const int per_group = G * tiles_n;
  const int g = q / per_group;
  const int first = g * G;
  const int gs = (tiles_m - first) < G ? (tiles_m - first) : G;
  const int r = q - g * per_group;
  ti = first + r % gs;
  tj = r / gs;
}

// LDS tile: rows of 8 chunks of 16 bytes.  The chunk position is XOR-swizzled
// with row bits 0-2 and 3-5 so that (a) 16 lanes reading the same logical
// chunk of 16 consecutive rows and (b) 8 lanes writing the same chunk of rows
// 8 apart both hit distinct bank groups.
NS_HD int lds_swz(int row, int ch) { return row * 8 + (ch ^ ((row ^ (row >> 3)) & 7)); }

// K-contiguous loader: chunk qd of an R x (8 chunks) stage.
struct KcontSrc {
  int row, ch;  // position in the tile
};
NS_HD KcontSrc kcont_src(int qd) { return KcontSrc{qd >> 3, qd & 7}; }

// M-contiguous loader: block qd of (R/EPC) x 8 blocks; each block is EPC
// k-rows by EPC consecutive i (one 16-byte load per k-row).
struct McontSrc {
  int ib, kb;  // block coordinates: rows ib*EPC.., k-chunk kb
};
NS_HD McontSrc mcont_src(int qd, int iblocks) { return McontSrc{qd % iblocks, qd / iblocks}; }

// Accumulator layout of v_mfma_f32_32x32x*: register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the 32x32 block.
NS_HD int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
NS_HD int acc_col(int lane) { return lane & 31; }

// Arguments of one tiled MFMA launch over `batch` slices.
// The kernel computes acc(i, j) = sum_k P(i, k) Q(j, k) over an M x N output,
// reduction length K, then applies the mode's epilogue (ns_layout.h).
struct GemmArgs {
  const void* P;      // operand P, slice 0
  const void* Q;      // operand Q, slice 0
  long long p_bs;     // slice strides, in elements
  long long q_bs;
  int ldp, ldq;       // leading dimensions, in elements
  int M, N, K;
  int tiles_m, tiles_n, tiles_per_slice, batch;
  void* out;          // output matrix (m x m for Gram/poly, X' for update)
  long long o_bs;
  int ldo;
  const void* E;      // epilogue matrix: O_A (poly) or X (update); unused for Gram
  long long e_bs;
  int lde;
  const float* d_in;  // diagonal vector read by the epilogue (poly: d_A, update: d_C)
  float* d_out;       // diagonal vector written (Gram: d_A, poly: d_C)
  long long d_bs;     // slice stride of both diagonal vectors
  float ca, cb, cc;   // quintic coefficients (poly only)
};

// Arguments of the two normalisation passes.
struct NormArgs {
  const void* x;       // input  [batch, elems]
  void* y;             // output [batch, elems] (scale pass), may equal x
  float* partials;     // [batch, chunks] sums of squares
  float* norms;        // optional [batch] Frobenius norms (scale pass)
  long long slice_vecs;  // 16-byte vectors per slice
  long long chunk_vecs;  // 16-byte vectors per block
  int chunks;          // blocks per slice
  float eps;
};

// Tile shape of the MFMA kernel per storage dtype: BM x BN output tile,
// WM x WN waves (64 lanes each); the K stage is 8 chunks of 16 bytes
// (64 bf16 or 32 fp32 values).
struct TileCfg {
  int bm, bn, wm, wn;
};
constexpr TileCfg kTileBf16 = {128, 128, 2, 2};
constexpr TileCfg kTileF32 = {128, 128, 2, 2};
NS_HD constexpr TileCfg tile_cfg(int dtype) { return dtype == 1 ? kTileBf16 : kTileF32; }
NS_HD constexpr int elems_per_chunk(int dtype) { return dtype == 1 ? 8 : 4; }

}  // namespace ns

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
  MODE_GRAM = 0,    // lower-triangle tiles of P Pᵀ, diagonal split; mirrored unless
                    // stored as the lower block triangle (out_t null)
  MODE_POLY = 1,    // lower-triangle tiles of b A + c A A (+ a on diagonal)
  MODE_UPD_ROW = 2, // rectangle tiles of O_C X + d_C[row] * X
  MODE_UPD_COL = 3  // rectangle tiles of X O_C + d_C[col] * X
};

NS_HD constexpr bool mode_is_tri(int mode) { return mode == MODE_GRAM || mode == MODE_POLY; }

// Tile shape of one kernel instance: BM x BN output tile, WM x WN waves of
// 64 lanes, CPR 16-byte chunks per LDS row (K stage = CPR * 16 bytes of each
// operand row), ST = K stages held in the LDS ring (loads run ST-1 stages
// ahead of the MFMAs), OCC = workgroups per CU the register budget is sized
// for.
struct TileCfg {
  int bm, bn, wm, wn, cpr, st, occ;
};

#ifndef NS_TILE_BF16_TRI
#define NS_TILE_BF16_TRI {128, 128, 2, 4, 8, 2, 2}
#endif
#ifndef NS_TILE_BF16_TRI_WIDE
#define NS_TILE_BF16_TRI_WIDE {192, 192, 6, 2, 8, 2, 1}
#endif
#ifndef NS_TILE_BF16_TRI_BIG
#define NS_TILE_BF16_TRI_BIG {256, 256, 2, 4, 8, 2, 1}
#endif
#ifndef NS_TILE_BF16_RECT
#define NS_TILE_BF16_RECT {256, 256, 2, 4, 8, 2, 1}
#endif
#ifndef NS_TILE_F32_TRI
#define NS_TILE_F32_TRI {128, 128, 2, 2, 8, 3, 1}
#endif
#ifndef NS_TILE_F32_RECT
#define NS_TILE_F32_RECT {128, 128, 2, 2, 8, 3, 1}
#endif
constexpr TileCfg kTileBf16Tri = NS_TILE_BF16_TRI;
constexpr TileCfg kTileBf16TriWide = NS_TILE_BF16_TRI_WIDE;
constexpr TileCfg kTileBf16TriBig = NS_TILE_BF16_TRI_BIG;
constexpr TileCfg kTileBf16Rect = NS_TILE_BF16_RECT;
constexpr TileCfg kTileF32Tri = NS_TILE_F32_TRI;
constexpr TileCfg kTileF32Rect = NS_TILE_F32_RECT;

// Triangle kernels (Gram, poly) have two bf16 tile shapes: 128 x 128 with
// two workgroups per CU, and 192 x 192 with one.  A launch with few lower
// triangle tiles (fewer than two rounds of 512 workgroup slots at 128) would
// leave a nearly empty last round, so it takes the larger tile instead
// (m = 4096: 528 tiles at 128, 253 tiles at 192 on 256 CUs).
// The 192 tile runs 12 MFMA waves of 32 x 96 (6 x 2), three per SIMD, so
// that while one wave waits for its fragment reads the other two keep the
// matrix core busy, and 12 waves share each stage's LDS-direct loads (four
// instructions each).  Its 36 blocks of 32 x 32 do not split over 8 waves.
// Lower-triangle tiles of `tile` rows over a stack of m x m results.
NS_HD constexpr long long tri_tiles(long long batch, long long m, int tile) {
  return batch * ((m + tile - 1) / tile) * ((m + tile - 1) / tile + 1) / 2;
}
// Triangle tile class of a launch: narrow (128), wide (192, see above) or,
// for the bf16 Gram of a launch with at least four rounds of 256 x 256
// triangle tiles, big (256): the Gram has a long K (the long side) and a
// plain epilogue, so the larger tile's halved operand traffic outweighs its
// diagonal-tile waste.  The poly keeps 128: its epilogue holds the O_A
// quads of the whole wave tile in registers.  t128 / t256: the launch's
// triangle tiles at 128 and at 256 (summed over every stack it covers).
enum TriClass { TRI_NARROW = 0, TRI_WIDE = 1, TRI_BIG = 2 };
// Rounds of a launch of `tiles` workgroups over `slots` resident ones.
NS_HD constexpr long long launch_rounds(long long tiles, long long slots) { return (tiles + slots - 1) / slots; }
// A launch whose stacks all have m >= 4096 (so K >= 4096 for both products)
// also takes the 192 tile when its last round would otherwise be nearly
// empty: when the CU work of its rounds, rounds x 192², is below that of the
// 128 tile's, rounds x 2 x 128² (m = 8192: 4 rounds of 192 against 5 of 128,
// the fifth holding 32 of 2080 tiles).  At shorter K the 192 tile runs below
// the 128 tile's rate.  min_m: the smallest m of the launch's stacks.
NS_HD constexpr int tri_class_of_tiles(int dtype, long long t128, long long t192, long long t256, bool gram,
                                       long long min_m) {
  return (dtype == 1 && (t128 < 1024 || (min_m >= 4096 && launch_rounds(t192, 256) * 192 * 192 <
                                                               launch_rounds(t128, 512) * 2 * 128 * 128)))
             ? TRI_WIDE
         : (gram && dtype == 1 && t256 >= 1024) ? TRI_BIG
                                                : TRI_NARROW;
}
NS_HD constexpr int tri_class(int dtype, long long batch, long long m, bool gram) {
  return tri_class_of_tiles(dtype, tri_tiles(batch, m, 128), tri_tiles(batch, m, 192), tri_tiles(batch, m, 256), gram,
                            m);
}
NS_HD constexpr TileCfg tile_cfg(int dtype, bool tri, int tri_cls = TRI_NARROW) {
  return dtype == 1 ? (tri ? (tri_cls == TRI_WIDE ? kTileBf16TriWide
                              : tri_cls == TRI_BIG ? kTileBf16TriBig
                                                   : kTileBf16Tri)
                           : kTileBf16Rect)
                    : (tri ? kTileF32Tri : kTileF32Rect);
}
NS_HD constexpr int elems_per_chunk(int dtype) { return dtype == 1 ? 8 : 4; }

// LDS of one kernel instance, in 16-byte chunks: the ring of ST K stages of
// both operands, or the epilogue's staged output tile (rows padded by one
// chunk), whichever is larger.
NS_HD constexpr int epi_row_chunks(int bn, int esize) { return bn * esize / 16 + 1; }
NS_HD constexpr int lds_chunks(int bm, int bn, int cpr, int st, int esize) {
  return st * (bm + bn) * cpr > bm * epi_row_chunks(bn, esize) ? st * (bm + bn) * cpr
                                                               : bm * epi_row_chunks(bn, esize);
}

// The hardware hands workgroup w to XCD (w mod 8).  Remap so that each XCD
// works through one contiguous range of logical tile ids (neighbouring tiles
// share operand panels, which then stay in that XCD's L2).
NS_HD int xcd_remap(int w, int G) {
  const int per = G / 8, rem = G % 8;
  const int xcd = w % 8, local = w / 8;
  return (xcd < rem) ? xcd * (per + 1) + local
                     : rem * (per + 1) + (xcd - rem) * per + local;
}

// q-th tile of a lower triangle of T tile rows, in bands of kTriBand tile
// rows walked column by column, so that a run of consecutive tiles (what one
// XCD runs together, as xcd_remap hands each XCD a contiguous range) covers
// a few tile rows and several columns: few operand panels per XCD's L2.
// Band b0 (rows b0 .. b0 + h - 1, h = min(kTriBand, T - b0)) holds the b0 h
// tiles left of its diagonal block, column by column, then the h (h + 1) / 2
// tiles of that block, column by column.
constexpr int kTriBand = 8;
NS_HD void tri_decode(int q, int T, int& ti, int& tj) {
  int b0 = 0;
  for (;;) {
    const int h = T - b0 < kTriBand ? T - b0 : kTriBand;
    const int n = b0 * h + h * (h + 1) / 2;
    if (q < n || b0 + h >= T) {
      if (q < b0 * h) {
        tj = q / h;
        ti = b0 + q % h;
      } else {
        int r = q - b0 * h, c = 0;
        while (r >= h - c) {
          r -= h - c;
          ++c;
        }
        tj = b0 + c;
        ti = b0 + c + r;
      }
      return;
    }
    q -= n;
    b0 += h;
  }
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

// K-stage operand tile in LDS: rows of CPR (4, 8 or 16) chunks of 16 bytes.
// Chunk ch of a row is stored at position ch ^ f(row) with
// f(row) = (row ^ (row >> log2 CPR)) & (CPR - 1), so that the 8 or 16 lanes
// that the LDS serves together, reading one logical chunk of consecutive
// rows, hit distinct bank groups.  XOR is its own inverse: the loader puts
// the global chunk phys ^ f(row) at position phys.
NS_HD int swz_f(int row, int cpr) {
  const int sh = cpr == 4 ? 2 : cpr == 8 ? 3 : 4;
  return (row ^ (row >> sh)) & (cpr - 1);
}
NS_HD int lds_swz(int row, int ch, int cpr) { return row * cpr + (ch ^ swz_f(row, cpr)); }

// An operand is read either as K-contiguous rows (KCONT: element (i, k) at
// base + i ld + k) or in its natural layout (NAT: element (i, k) at
// base + k ld + i, i.e. rows of the stored matrix are the k index).  A NAT
// stage sits in LDS as BK rows (k) of R / EPC chunks (i); chunk c of k-row kr
// is stored at position c ^ nat_swz(kr), which keeps the transposed fragment
// reads below free of bank conflicts (checked for R = 128, 192, 256 bf16 and
// R = 128 fp32).
NS_HD int nat_swz(int kr, int row_chunks, int esize) {
  if (esize == 4) return (kr & 7) << 1;
  return row_chunks % 16 == 0 ? (kr & 3) << 2 : (kr >> 1) & 7;
}

// Loader: each wave instruction fills 64 consecutive chunks of a stage (one
// 16-byte chunk per lane).  Instruction idx of a stage covers chunk positions
// [64 idx, 64 idx + 64): the P tile first, then the Q tile.  For a KCONT tile
// `row` is the tile row and `kpos` the k offset (in elements) of the lane's
// chunk; for a NAT tile `row` is the tile column (first of EPC) and `kpos`
// the k row.
struct DmaSrc {
  bool is_p;     // operand P (else Q)
  int row;       // tile row (KCONT) or first tile column of the chunk (NAT)
  int kpos;      // k offset within the stage
  int lds_pos;   // chunk position in the stage slot written by this lane
};
NS_HD DmaSrc dma_src(int idx, int lane, int bm, int bn, int cpr, int epc, bool p_nat, bool q_nat, int esize) {
  const int p = idx * 64 + lane;
  const bool is_p = p < bm * cpr;
  const int pp = is_p ? p : p - bm * cpr;
  const bool nat = is_p ? p_nat : q_nat;
  if (!nat) {
    const int row = pp / cpr, phys = pp % cpr;
    return DmaSrc{is_p, row, (phys ^ swz_f(row, cpr)) * epc, p};
  }
  const int rc = (is_p ? bm : bn) / epc;  // chunks per k row
  const int kr = pp / rc, phys = pp % rc;
  return DmaSrc{is_p, (phys ^ nat_swz(kr, rc, esize)) * epc, kr, p};
}

// Transposed fragment read of a NAT bf16 tile with ds_read_b64_tr_b16.  In a
// group of 16 lanes, lane t receives element t % 4 of the 4-element vectors
// addressed by lanes 4e + t / 4 (e = 0..3).  With lane l addressing k row
// 16 s + 8 (l / 32) + 4 h + (l % 16) / 4 and columns rb + 16 ((l / 16) % 2) +
// 4 (l % 4) .. +3, lane l receives column rb + l % 32 at k rows
// 16 s + 8 (l / 32) + 4 h + 0..3: two reads (h = 0, 1) give the same 8 k
// values per lane as a K-contiguous chunk read.
NS_HD int nat_tr_kr(int s, int h, int lane) { return 16 * s + 8 * (lane >> 5) + 4 * h + ((lane & 15) >> 2); }
NS_HD int nat_tr_col(int rb, int lane) { return rb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3); }

// Fragment reads as a per-lane base plus a compile-time offset (LDS bytes
// within one operand region of a stage), so that the K loop spends no VALU
// work on addresses.
//  K-contiguous: step s of block a (rows w0 + 32 a + lane % 32, chunk
//  2 s + lane / 32; w0 a multiple of 32) reads
//    kc_lane_byte(w0, s ^ kc_sigma(a, cpr), lane, cpr) + 32 a cpr 16.
//  Rows 32 apart differ in their swizzle only in bit 2 of the chunk (cpr 8)
//  or not at all (cpr 4), and flipping bit 2 of chunk 2 s + h is s ^ 2.
NS_HD int kc_lane_byte(int w0, int s, int lane, int cpr) {
  return lds_swz(w0 + (lane & 31), 2 * s + (lane >> 5), cpr) * 16;
}
NS_HD constexpr int kc_sigma(int a, int cpr) { return cpr == 8 ? 2 * (a & 1) : 0; }
//  NAT bf16: read h of step s of the block at column rb reads
//    nat_lane_byte_bf16(rb, h, lane, rc) + 16 s rc 16
//  (a step moves the k row by 16, and nat_swz does not see that move).
NS_HD int nat_lane_byte_bf16(int rb, int h, int lane, int rc) {
  const int kr = nat_tr_kr(0, h, lane), col = nat_tr_col(rb, lane);
  return (kr * rc + ((col >> 3) ^ nat_swz(kr, rc, 2))) * 16 + (col & 7) * 2;
}
//  NAT fp32: element e (k row 8 s + 4 (lane / 32) + e, column rb + lane % 32)
//  reads nat_lane_byte_f32(rb, e, lane, rc) + 8 s rc 16.
NS_HD int nat_lane_byte_f32(int rb, int e, int lane, int rc) {
  const int kr = 4 * (lane >> 5) + e, col = rb + (lane & 31);
  return (kr * rc + ((col >> 2) ^ nat_swz(kr, rc, 4))) * 16 + (col & 3) * 4;
}
NS_HD constexpr int nat_step_bytes(int rc, int esize) { return (esize == 2 ? 16 : 8) * rc * 16; }

// Mirror store of a staged bf16 tile (the transposes of its rows): one wave
// instruction per unit u of 16 tile columns x 32 tile rows.  Lane l writes
// 16 bytes of transposed row `col` (tile column 16 (u % (bn / 16)) + l % 16)
// holding tile rows row0 .. row0 + 7, row0 = 8 (4 (u / (bn / 16)) + l / 16),
// so one instruction covers 16 output rows with 64 contiguous bytes each.
// It gathers them with two transposing LDS reads (ds_read_b64_tr_b16), for
// which it addresses tile row src_row[h] at columns src_col .. + 3: in each
// 16-lane group lane t then receives column cb + t of rows row0 + 4 h .. + 3.
struct MirrorLane {
  int col, row0, src_row[2], src_col;
};
NS_HD MirrorLane mirror_lane(int u, int lane, int bn) {
  const int cgroups = bn / 16, cb = 16 * (u % cgroups), rq = u / cgroups, l16 = lane & 15;
  MirrorLane m;
  m.col = cb + l16;
  m.row0 = 8 * (4 * rq + (lane >> 4));
  m.src_row[0] = m.row0 + (l16 >> 2);
  m.src_row[1] = m.row0 + 4 + (l16 >> 2);
  m.src_col = cb + 4 * (l16 & 3);
  return m;
}

// Operand layouts: K-contiguous rows (KCONT), the stored matrix read down its
// columns (NAT), or a symmetric matrix of which only the lower block triangle
// is stored (SYM: tiles of sym_tile rows, diagonal tiles whole).  A SYM
// operand reads rows r0 .. r0 + R of k block [k0, k0 + BK) as K-contiguous
// rows while that k block lies at or left of r0's diagonal block, and from
// the transposed, stored tile (a NAT read) once it lies to the right: with
// sym_tile a multiple of BK and R <= sym_tile, every stage then reads stored
// elements only (the row block spans at most two stored blocks, and the
// right-hand k blocks are at or below the diagonal of both).  The kernel
// runs the K loop in phases of fixed layouts that start at multiples of the
// ring depth st, so sym_tile / BK must also be a multiple of st.
enum OperandLayout { LAY_KCONT = 0, LAY_NAT = 1, LAY_SYM = 2 };
NS_HD constexpr int sym_nat_from(int r0, int sym_tile, int bk) { return (r0 / sym_tile + 1) * sym_tile / bk; }
NS_HD constexpr bool sym_layout_ok(int rows, int sym_tile, int bk, int st) {
  return sym_tile > 0 && sym_tile % bk == 0 && (sym_tile / bk) % st == 0 && rows <= sym_tile;
}

// Diagonal tiles of the triangle kernels with 2 x 4 MFMA waves: only their
// 32 x 32 blocks on or below the diagonal are computed (the others are
// replaced by the mirror of the lower half when stored), and the waves of
// tile row half 1 take the columns in the order 3, 2, 0, 1, so that the two
// waves of each SIMD (w and w + 4) hold about the same number of those
// blocks: 10, 10, 8, 8 of 16 block products per k step on a 256 tile
// instead of 15, 11, 7, 3; 3, 3, 2, 2 of 4 on a 128 tile instead of
// 4, 3, 2, 1.
NS_HD int tri_wave_col(int wm, int wn, int wn_count, bool diag) {
  return (diag && wm == 1 && wn_count == 4) ? (0x1023 >> (4 * wn)) & 0xF : wn;
}
// Block (a, b) of the wave at (wm, wn) (sm x sn blocks per wave) lies wholly
// above the diagonal of a diagonal tile.
NS_HD bool tri_block_above(int wm, int wn, int a, int b, int sm, int sn) { return wn * sn + b > wm * sm + a; }

// MFMA operand roles: the A operand is the Q tile (output column j), the B
// operand the P tile (output row i).  Register r of lane l of a 32x32 block
// then holds row i = l % 32 and column j = 8 (r / 4) + 4 (l / 32) + r % 4,
// so each group of 4 registers is 4 consecutive columns of one row.
NS_HD int acc_i(int lane) { return lane & 31; }
NS_HD int acc_j(int rgroup, int lane) { return 8 * rgroup + 4 * (lane >> 5); }

// Arguments of one tiled MFMA launch over `batch` slices.  The kernel forms
// acc(i, j) = sum_k P(i, k) Q(j, k) over an M x N output with reduction
// length K (each operand KCONT or NAT, a template choice), applies the mode's
// epilogue, stores the tile to `out` and, if out_t is set, its transpose to
// out_t.
struct GemmArgs {
  const void* P;      // operand P rows, slice 0
  const void* Q;      // operand Q rows, slice 0
  long long p_bs;     // slice strides, in elements
  long long q_bs;
  int ldp, ldq;       // leading dimensions, in elements
  int M, N, K;
  int tiles_m, tiles_n, tiles_per_slice, batch;
  void* out;          // output (m x m for Gram/poly, X' for update)
  long long o_bs;
  int ldo;
  void* out_t;        // transposed output (mirror for Gram/poly, X'ᵀ), or null
  long long ot_bs;
  int ldt;
  const float* d_in;  // diagonal vector read by the epilogue (poly: d_A, update: d_C)
  float* d_out;       // diagonal vector written (Gram: d_A, poly: d_C)
  long long d_bs;     // slice stride of both diagonal vectors
  float ca, cb, cc;   // quintic coefficients (poly only)
  // First step on an unnormalised input: d_norm holds the slice's partial
  // sums of squares of the raw input (norm_n per slice), whose total is
  // ||x||_F^2.  With inv = 1 / (||x||_F + eps) the Gram scales its result by
  // inv^2 (A of X0 = inv x) and the update scales its result by inv, so X0 is
  // never formed.  Null: the operands already are X_s.
  const float* d_norm;
  int norm_n;
  float eps;
  int sym_tile;       // stored tile of LAY_SYM operands (rows of the producer's tiles)
};

// One launch of the MFMA kernel over NG groups of slices: group i has
// start[i + 1] - start[i] tiles (the last one up to the grid's end), each
// group its own shapes, strides and buffers; the tile class and operand
// layouts are the launch's.  NG = 1 is a plain launch.  The groups travel in
// the kernel arguments (at most 4 KiB), read with scalar loads; workgroups
// map to (group, tile) through xcd_group_tile.
constexpr int kMaxLaunchGroups = 16;
template <int NG> struct GemmLaunch {
  GemmArgs g[NG];
  int start[NG];  // first logical tile id of each group; start[0] = 0
  int n;          // groups in use, 1..NG
};

// Workgroup w of a launch over n groups (group i: ids [start[i], start[i+1]),
// the last one up to G) -> group *grp and tile id within it.  Tiles of
// different groups cost different amounts (their K differs), so rather than
// one contiguous range of the launch per XCD (xcd_remap), each XCD (w mod 8)
// takes a contiguous run of about an eighth of EVERY group, in group order.
// Group i's T tiles split into eight runs of T / 8, the T % 8 XCDs that take
// one more being dealt out cyclically from where the previous group's
// remainder ended; so XCD x's runs add up to exactly its workgroup count,
// G / 8 (+1 for the first G % 8 XCDs).  With one group this is xcd_remap.
NS_HD int xcd_group_tile(int w, int G, const int* start, int n, int* grp) {
  const int x = w % 8;
  int l = w / 8, o = 0;
  for (int g = 0; g < n; ++g) {
    const int T = (g + 1 < n ? start[g + 1] : G) - start[g];
    const int q = T / 8, r = T % 8;
    const int p = q + (((x - o + 8) % 8) < r ? 1 : 0);  // this XCD's run of group g
    if (l < p || g == n - 1) {
      int before = 0;  // XCDs below x that take one more tile of group g
      for (int y = 0; y < x; ++y) before += ((y - o + 8) % 8) < r ? 1 : 0;
      *grp = g;
      return x * q + before + l;
    }
    l -= p;
    o = (o + r) % 8;
  }
  *grp = 0;
  return 0;
}

// Group of logical block `lin`: the last group whose first block is <= lin
// (a wave-uniform scan, at most kMaxLaunchGroups steps).
NS_HD int launch_group(int lin, const int* start, int n) {
  int grp = 0;
  for (int i = 1; i < n; ++i)
    if (lin >= start[i]) grp = i;
  return grp;
}

// Zero-padded copies of odd shapes, by 16-byte vectors: vector v of a padded
// slice (vpr vectors per row) holds row v / vpr, columns (v % vpr) epv ..
// + epv - 1 (epv elements per vector).  32-bit: a slice has fewer than 2^29
// elements.
NS_HD void pad_vec(int v, int vpr, int epv, int* row, int* col0) {
  *row = v / vpr;
  *col0 = (v - *row * vpr) * epv;
}

// Normalisation: per-slice sum of squares over 32 KiB blocks, then a scale
// pass over the same blocks.
struct NormArgs {
  const void* x;         // input  [batch, rows, cols]
  void* y;               // X0 [batch, rows, cols] (scale pass), may equal x
  float* partials;       // [batch, chunks] sums of squares
  float* norms;          // optional [batch] Frobenius norms (scale pass)
  long long slice_vecs;  // 16-byte vectors per slice
  long long chunk_vecs;  // 16-byte vectors per block
  int chunks;            // blocks per slice
  float eps;
};

// Sums of squares over NG groups of slices in one launch: block b of the
// 1-D grid belongs to the last group with start[i] <= b and covers block
// (b - start[i]) of that group's batch x chunks blocks, slice-major.
template <int NG> struct NormLaunch {
  NormArgs a[NG];
  int start[NG];
  int n;
};

}  // namespace ns

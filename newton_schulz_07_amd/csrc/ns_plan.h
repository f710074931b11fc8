// ns_plan.h - workspace layout of one call and the launch arguments of each
// stage.  Plain C++ (no HIP types) so that the host-side bounds checker
// builds exactly the arguments the driver passes to the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ns_layout.h"

namespace ns {

constexpr float kNormEps = 1e-7f;             // added to the Frobenius norm
constexpr long long kNormChunkVecs = 2048;    // 16-byte vectors per norm block (32 KiB)
constexpr size_t kWsAlign = 256;

inline size_t elem_size(int dtype) { return dtype == 1 ? 2 : 4; }
inline size_t ws_align(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
inline int tiles_of(int64_t extent, int tile) { return (int)((extent + tile - 1) / tile); }

// One call on [batch, rows, cols].  The Gram side is m = min(rows, cols).
// A shape whose rows or cols is not a multiple of 8 runs on a zero-padded
// copy (rows and cols rounded up to 8): zero rows and columns only add zero
// singular values, which every step maps to zero, so NS of [X 0; 0 0] is
// [NS(X) 0; 0 0] and the Frobenius norm is unchanged.  rows / cols are then
// the padded sizes, urows / ucols the caller's, and the workspace holds the
// padded input and output.
struct Plan {
  int64_t batch, rows, cols, m, n;
  bool tall;
  int dtype;
  int norm_chunks;
  bool padded;
  int64_t urows, ucols;
  // workspace offsets (bytes)
  size_t off_xtmp, off_oa, off_oc, off_da, off_dc, off_part, off_pin, off_pout, total;
};

inline int64_t round_up8(int64_t v) { return (v + 7) / 8 * 8; }

inline Plan make_plan(int64_t batch, int64_t urows, int64_t ucols, int dtype) {
  const int64_t rows = round_up8(urows), cols = round_up8(ucols);
  Plan p{};
  p.padded = rows != urows || cols != ucols;
  p.urows = urows;
  p.ucols = ucols;
  p.batch = batch;
  p.rows = rows;
  p.cols = cols;
  p.tall = rows > cols;
  p.m = p.tall ? cols : rows;
  p.n = p.tall ? rows : cols;
  p.dtype = dtype;
  const size_t es = elem_size(dtype);
  const long long vecs = rows * cols * (long long)es / 16;
  p.norm_chunks = (int)((vecs + kNormChunkVecs - 1) / kNormChunkVecs);
  size_t off = 0;
  p.off_xtmp = off;
  off += ws_align((size_t)batch * rows * cols * es);
  p.off_oa = off;
  off += ws_align((size_t)batch * p.m * p.m * es);
  p.off_oc = off;
  off += ws_align((size_t)batch * p.m * p.m * es);
  p.off_da = off;
  off += ws_align((size_t)batch * p.m * 4);
  p.off_dc = off;
  off += ws_align((size_t)batch * p.m * 4);
  p.off_part = off;
  off += ws_align((size_t)batch * p.norm_chunks * 4);
  p.off_pin = p.off_pout = off;
  if (p.padded) {
    off += ws_align((size_t)batch * rows * cols * es);
    p.off_pout = off;
    off += ws_align((size_t)batch * rows * cols * es);
  }
  p.total = off;
  return p;
}

// Zero-padded copy in (pad, fused with the sum-of-squares pass) or the
// caller's block out (unpad) of a padded plan, by 16-byte vectors of the
// padded slice (pad_vec).
struct PadArgs {
  const void* src;
  void* dst;
  long long batch, urows, ucols, rows, cols;  // caller's and padded slice sizes
  bool to_padded;                            // pad (true) or unpad (false)
};
inline PadArgs pad_args(const Plan& p, const void* src, void* dst, bool to_padded) {
  return PadArgs{src, dst, p.batch, p.urows, p.ucols, p.rows, p.cols, to_padded};
}

// The iterate X_s (s = 0 after normalisation) is held in `out` when
// (steps - s) is even and in the workspace temporary otherwise, so the last
// step writes `out` and no update reads the buffer it writes.  When the
// normalisation is folded into the first step (fold_normalisation), X_0 is
// the raw input itself.
inline bool iterate_in_out(int steps, int s) { return ((steps - s) % 2) == 0; }

inline NormArgs norm_args(const Plan& p, const void* x, void* y, float* norms, float* partials) {
  NormArgs g{};
  g.x = x;
  g.y = y;
  g.partials = partials;
  g.norms = norms;
  g.slice_vecs = p.rows * p.cols * (long long)elem_size(p.dtype) / 16;
  g.chunk_vecs = kNormChunkVecs;
  g.chunks = p.norm_chunks;
  g.eps = kNormEps;
  return g;
}

// Splits groups [0, n) of a grouped launch: the first k of them (at most
// kMaxLaunchGroups, fewer if the launch's ids would pass 2^30) go into one
// launch.  units(i) is group i's workgroups; start[i] receives its first id
// and *total the launch's grid size.  Returns k.
template <typename Units>
inline int launch_chunk(int n, Units units, int* start, long long* total) {
  long long t = 0;
  int k = 0;
  for (; k < n && k < kMaxLaunchGroups; ++k) {
    const long long u = units(k);
    if (k > 0 && t + u >= (1LL << 30)) break;
    start[k] = (int)t;
    t += u;
  }
  *total = t;
  return k;
}

// Which kernel instance a stage launches.
struct StageKind {
  int mode;
  bool p_nat, q_nat;  // operand read in its natural layout (see ns_layout.h)
  int tri_cls;        // triangle tile class (TriClass)
  bool p_sym = false, q_sym = false;  // LAY_SYM operand (lower block triangle stored)
};

// Tile classes of the triangle launches of one call.  A call over several
// stacks (ns_orthogonalize_grouped) runs one Gram launch per orientation
// (wide stacks read rows of X, tall ones columns) and one poly launch over
// all of them, so each class follows the tile count of its launch.
struct TileChoice {
  int gram_wide, gram_tall;  // Gram class of the wide / tall stacks' launch
  int poly;                  // poly class (one launch over every stack)
  // The poly reads A as its lower block triangle (LAY_SYM) and the Gram
  // stores no mirror: bf16, poly at 128, and every Gram tile a multiple of
  // the poly's K stage and at least as tall as the poly's tile.
  // (The kernels instantiate that read for the bf16 poly's 128 tile.)
  bool lower_only;
  int gram(bool tall) const { return tall ? gram_tall : gram_wide; }
};

inline TileChoice choose_tiles(const Plan* ps, int n) {
  long long t128[2] = {0, 0}, t192[2] = {0, 0}, t256[2] = {0, 0};
  long long min_m[2] = {1LL << 40, 1LL << 40};
  int dtype = n > 0 ? ps[0].dtype : 1;
  for (int i = 0; i < n; ++i) {
    const Plan& p = ps[i];
    t128[p.tall] += tri_tiles(p.batch, p.m, 128);
    t192[p.tall] += tri_tiles(p.batch, p.m, 192);
    t256[p.tall] += tri_tiles(p.batch, p.m, 256);
    if (p.m < min_m[p.tall]) min_m[p.tall] = p.m;
  }
  TileChoice c;
  c.gram_wide = tri_class_of_tiles(dtype, t128[0], t192[0], t256[0], true, min_m[0]);
  c.gram_tall = tri_class_of_tiles(dtype, t128[1], t192[1], t256[1], true, min_m[1]);
  c.poly = tri_class_of_tiles(dtype, t128[0] + t128[1], t192[0] + t192[1], t256[0] + t256[1], false,
                              min_m[0] < min_m[1] ? min_m[0] : min_m[1]);
  const TileCfg tp = tile_cfg(dtype, true, c.poly);
  bool ok = dtype == 1 && c.poly == TRI_NARROW;
  for (int o = 0; o < 2; ++o)
    if (t128[o] > 0)
      ok = ok && sym_layout_ok(tp.bm, tile_cfg(dtype, true, c.gram(o != 0)).bm,
                               tp.cpr * (16 / (int)elem_size(dtype)), tp.st);
  c.lower_only = ok;
  return c;
}
inline TileChoice choose_tiles(const Plan& p) { return choose_tiles(&p, 1); }

inline int plan_tri_class(const Plan& p, bool gram) {
  const TileChoice c = choose_tiles(p);
  return gram ? c.gram(p.tall) : c.poly;
}
inline bool gram_lower_only(const Plan& p) { return choose_tiles(p).lower_only; }

// A = X Xᵀ (rows <= cols: rows of X are K-contiguous) or Xᵀ X (rows > cols:
// columns of X, read in X's natural layout), mirrored into one m x m matrix.
// mirror: also store the transposes of the off-diagonal tiles (a whole
// symmetric A); otherwise only the lower block triangle is stored.
inline GemmArgs gram_args(const Plan& p, const TileChoice& tc, const void* x, void* oa, float* da,
                          StageKind* kind, const float* d_norm = nullptr, bool mirror = true) {
  const int cls = tc.gram(p.tall);
  const TileCfg t = tile_cfg(p.dtype, true, cls);
  GemmArgs g{};
  g.P = g.Q = x;
  g.p_bs = g.q_bs = p.rows * p.cols;
  g.ldp = g.ldq = (int)p.cols;
  g.M = g.N = (int)p.m;
  g.K = (int)p.n;
  g.tiles_m = g.tiles_n = tiles_of(p.m, t.bm);
  g.tiles_per_slice = g.tiles_m * (g.tiles_m + 1) / 2;
  g.batch = (int)p.batch;
  g.out = oa;
  g.out_t = mirror ? oa : nullptr;
  g.o_bs = g.ot_bs = p.m * p.m;
  g.ldo = g.ldt = (int)p.m;
  g.d_out = da;
  g.d_bs = p.m;
  g.d_norm = d_norm;
  g.norm_n = p.norm_chunks;
  g.eps = kNormEps;
  *kind = StageKind{MODE_GRAM, p.tall, p.tall, cls};
  return g;
}
inline GemmArgs gram_args(const Plan& p, const void* x, void* oa, float* da, StageKind* kind,
                          const float* d_norm = nullptr, bool mirror = true) {
  return gram_args(p, choose_tiles(p), x, oa, da, kind, d_norm, mirror);
}

// C = a I + b A + c A A from the split A, written split the same way.
inline GemmArgs poly_args(const Plan& p, const TileChoice& tc, const void* oa, const float* da, void* oc,
                          float* dc, float a, float b, float c, StageKind* kind) {
  const TileCfg t = tile_cfg(p.dtype, true, tc.poly);
  GemmArgs g{};
  g.P = g.Q = oa;
  g.p_bs = g.q_bs = p.m * p.m;
  g.ldp = g.ldq = (int)p.m;
  g.M = g.N = g.K = (int)p.m;
  g.tiles_m = g.tiles_n = tiles_of(p.m, t.bm);
  g.tiles_per_slice = g.tiles_m * (g.tiles_m + 1) / 2;
  g.batch = (int)p.batch;
  g.out = g.out_t = oc;
  g.o_bs = g.ot_bs = p.m * p.m;
  g.ldo = g.ldt = (int)p.m;
  g.d_in = da;
  g.d_out = dc;
  g.d_bs = p.m;
  g.ca = a;
  g.cb = b;
  g.cc = c;
  *kind = StageKind{MODE_POLY, false, false, tc.poly};
  if (tc.lower_only) {  // read A as its lower block triangle
    kind->p_sym = kind->q_sym = true;
    g.sym_tile = tile_cfg(p.dtype, true, tc.gram(p.tall)).bm;
  }
  return g;
}
inline GemmArgs poly_args(const Plan& p, const void* oa, const float* da, void* oc, float* dc, float a,
                          float b, float c, StageKind* kind) {
  return poly_args(p, choose_tiles(p), oa, da, oc, dc, a, b, c, kind);
}

// Update launches of at most this many tiles (four rounds on 256 CUs) issue
// each stage's operand loads after the stage's first k step rather than
// before it: their MFMA work, not their loads, sets their pace, and the
// loads then leave the MFMAs' start alone.
constexpr long long kLateIssueMaxTiles = 1024;
// Larger bf16 update launches with at least this many K stages stagger the
// load issue of the two tile-row halves by one k step (see the kernel).
// Larger launches too short for that (no group with this many stages) take
// the late issue: on 128 slices of 2048 x 768 (K = 768, 12 stages) it beats
// issuing at the barrier, while on the long-K stacks the stagger beats it.
constexpr int kStaggerMinStages = 16;
// K stages of a bf16 update launch over K (its k step: cpr chunks of 8).
inline int update_k_stages(int K) {
  const int bk = kTileBf16Rect.cpr * 8;
  return (K + bk - 1) / bk;
}
// tiles: over all groups of the launch; max_k: the largest K among them
inline bool late_issue(int dtype, long long tiles, int max_k) {
  return dtype == 1 && (tiles <= kLateIssueMaxTiles || update_k_stages(max_k) < kStaggerMinStages);
}

// X' = C X (rows <= cols) or X C (rows > cols), C = O_C + diag(d_C).
inline GemmArgs update_args(const Plan& p, const void* x, const void* oc, const float* dc, void* xo,
                            StageKind* kind, const float* d_norm = nullptr) {
  const TileCfg t = tile_cfg(p.dtype, false);
  GemmArgs g{};
  if (!p.tall) {  // P = rows of O_C, Q(j, k) = X[k][j] (natural layout)
    g.P = oc;
    g.p_bs = p.m * p.m;
    g.ldp = (int)p.m;
    g.Q = x;
    g.q_bs = p.rows * p.cols;
    g.ldq = (int)p.cols;
    *kind = StageKind{MODE_UPD_ROW, false, true, TRI_NARROW};
  } else {  // P = rows of X, Q = rows of O_C (C is symmetric)
    g.P = x;
    g.p_bs = p.rows * p.cols;
    g.ldp = (int)p.cols;
    g.Q = oc;
    g.q_bs = p.m * p.m;
    g.ldq = (int)p.m;
    *kind = StageKind{MODE_UPD_COL, false, false, TRI_NARROW};
  }
  g.M = (int)p.rows;
  g.N = (int)p.cols;
  g.K = (int)p.m;
  g.tiles_m = tiles_of(p.rows, t.bm);
  g.tiles_n = tiles_of(p.cols, t.bn);
  g.tiles_per_slice = g.tiles_m * g.tiles_n;
  g.batch = (int)p.batch;
  g.out = xo;
  g.o_bs = p.rows * p.cols;
  g.ldo = (int)p.cols;
  g.out_t = nullptr;
  g.d_in = dc;
  g.d_out = nullptr;
  g.d_bs = p.m;
  g.d_norm = d_norm;
  g.norm_n = p.norm_chunks;
  g.eps = kNormEps;
  return g;
}

// Whenever there is a step, the first step runs on the raw input: one
// sum-of-squares pass gives ||x||_F, the first Gram scales A by 1/||x||^2 and
// the first update scales X_1 by 1/||x|| (X0 = x/||x|| is never written).
// Every product that sees raw values is then X Xᵀ, whose range is that of the
// sum of squares itself.  When out == in and the step count is odd, the first
// update would write `out`, the input it still reads: the input is then first
// copied to the temporary, which serves as X_0 (the result stays bitwise the
// same).
inline bool fold_normalisation(int steps) { return steps >= 1; }
inline bool input_copy_needed(int steps, bool out_is_in) { return steps >= 1 && out_is_in && (steps & 1); }

}  // namespace ns

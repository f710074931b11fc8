// ns_boundscheck.cpp - host-side walk of every address the kernels of one
// ns_orthogonalize call touch, for given shapes, without a GPU.
//
// It builds the launch arguments with the driver's own functions (ns_plan.h),
// replays the kernels' index arithmetic (ns_layout.h) for every workgroup and
// thread, and checks that
//   * every workgroup id maps to a distinct tile of a valid slice,
//   * every global load and store stays inside the buffer its pointer names,
//   * every LDS index stays inside the operand's LDS region,
//   * every output element (and diagonal entry) is written exactly once.
// K stages other than the first and the last only move the k offset between
// those two, so only those two are replayed.
//
// Build: g++ -O2 -std=c++17 -I<csrc> ns_boundscheck.cpp -o ns_boundscheck
// Run:   ns_boundscheck dtype batch rows cols steps [dtype batch rows cols steps ...]
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "ns_layout.h"
#include "ns_plan.h"

using namespace ns;

namespace {

struct Buf {
  std::string name;
  size_t bytes;
};
std::map<uintptr_t, Buf> g_bufs;
long long g_checks = 0;
int g_fail = 0;

void* reg(uintptr_t base, const std::string& name, size_t bytes) {
  g_bufs[base] = Buf{name, bytes};
  return reinterpret_cast<void*>(base);
}

void fail(const std::string& msg) {
  if (g_fail < 20) std::fprintf(stderr, "VIOLATION: %s\n", msg.c_str());
  ++g_fail;
}

void access(const void* ptr, long long byte_off, int len, const char* what) {
  ++g_checks;
  auto it = g_bufs.find(reinterpret_cast<uintptr_t>(ptr));
  if (it == g_bufs.end()) {
    fail(std::string(what) + ": pointer is not a registered buffer");
    return;
  }
  if (byte_off < 0 || (size_t)(byte_off + len) > it->second.bytes)
    fail(std::string(what) + ": offset " + std::to_string(byte_off) + "+" + std::to_string(len) +
         " outside " + it->second.name + " (" + std::to_string(it->second.bytes) + " bytes)");
}

void lds_index(int idx, int limit, const char* what) {
  ++g_checks;
  if (idx < 0 || idx >= limit)
    fail(std::string(what) + ": LDS chunk " + std::to_string(idx) + " outside [0," + std::to_string(limit) + ")");
}

// One operand's loads of stage k0 for one thread (mirrors OperandLoader).
void replay_loader(int layout, int es, int R, int NT, const void* base, long long slice_off, int ld, int r0,
                   int rmax, int k0, int kmax, int tid, const char* what) {
  const int EPC = 16 / es;
  if (layout == KCONT) {
    const int NCH = R * 8, ITER = (NCH + NT - 1) / NT;
    for (int it = 0; it < ITER; ++it) {
      const int qd = tid + it * NT;
      if (qd >= NCH) continue;
      const KcontSrc s = kcont_src(qd);
      lds_index(lds_swz(s.row, s.ch), R * 8, what);
      const int gi = r0 + s.row, gk = k0 + s.ch * EPC;
      if (gi < rmax && gk < kmax) access(base, (slice_off + (long long)gi * ld + gk) * es, 16, what);
    }
  } else {
    const int IB = R / EPC, NBLK = IB * 8, ITER = (NBLK + NT - 1) / NT;
    for (int it = 0; it < ITER; ++it) {
      const int qd = tid + it * NT;
      if (qd >= NBLK) continue;
      const McontSrc s = mcont_src(qd, IB);
      for (int ii = 0; ii < EPC; ++ii) lds_index(lds_swz(s.ib * EPC + ii, s.kb), R * 8, what);
      const int gi = r0 + s.ib * EPC;
      if (gi >= rmax) continue;
      for (int kk = 0; kk < EPC; ++kk) {
        const int gk = k0 + s.kb * EPC + kk;
        if (gk < kmax) access(base, (slice_off + (long long)gk * ld + gi) * es, 16, what);
      }
    }
  }
}

// Replays one launch of gemm_kernel (grid = tiles_per_slice * batch).
void replay_gemm(const GemmArgs& g, const StageKind& k, int dtype, bool coverage, const char* what) {
  const TileCfg t = tile_cfg(dtype);
  const int es = (int)elem_size(dtype);
  const int EPC = 16 / es, BK = 8 * EPC;
  const int NT = t.wm * t.wn * 64, WTM = t.bm / t.wm, WTN = t.bn / t.wn;
  const int SM = WTM / 32, SN = WTN / 32;
  const int G = g.tiles_per_slice * g.batch;
  const bool tri = mode_is_tri(k.mode);
  const int nk = (g.K + BK - 1) / BK;

  std::vector<uint8_t> seen(G, 0);
  const long long out_elems = (long long)g.o_bs * g.batch;
  std::vector<uint8_t> cover, dcover;
  if (coverage) {
    cover.assign(out_elems, 0);
    if (g.d_out) dcover.assign((size_t)g.d_bs * g.batch, 0);
  }
  // fragment reads stay inside each region (independent of the block)
  for (int wave = 0; wave < t.wm * t.wn; ++wave)
    for (int lane = 0; lane < 64; ++lane)
      for (int s = 0; s < 4; ++s) {
        const int ch = 2 * s + (lane >> 5), wm = wave / t.wn, wn = wave % t.wn;
        for (int a = 0; a < SM; ++a) lds_index(lds_swz(wm * WTM + a * 32 + (lane & 31), ch), t.bm * 8, what);
        for (int b = 0; b < SN; ++b) lds_index(lds_swz(wn * WTN + b * 32 + (lane & 31), ch), t.bn * 8, what);
      }

  for (int w = 0; w < G; ++w) {
    const int lin = xcd_remap(w, G);
    if (lin < 0 || lin >= G || seen[lin]) {
      fail(std::string(what) + ": xcd_remap is not a bijection");
      continue;
    }
    seen[lin] = 1;
    const int slice = lin / g.tiles_per_slice, q = lin - slice * g.tiles_per_slice;
    int ti, tj;
    if (tri) tri_decode(q, ti, tj);
    else rect_decode(q, g.tiles_m, g.tiles_n, ti, tj);
    if (slice >= g.batch || ti < 0 || tj < 0 || ti >= g.tiles_m || tj >= g.tiles_n || (tri && tj > ti)) {
      fail(std::string(what) + ": tile decode out of range");
      continue;
    }
    const int i0 = ti * t.bm, j0 = tj * t.bn;
    const int kstages[2] = {0, nk - 1};
    for (int si = 0; si < (nk > 1 ? 2 : 1); ++si) {
      const int k0 = kstages[si] * BK;
      for (int tid = 0; tid < NT; ++tid) {
        replay_loader(k.p_layout, es, t.bm, NT, g.P, (long long)slice * g.p_bs, g.ldp, i0, g.M, k0, g.K, tid, what);
        replay_loader(k.q_layout, es, t.bn, NT, g.Q, (long long)slice * g.q_bs, g.ldq, j0, g.N, k0, g.K, tid, what);
      }
    }
    // epilogue (mirrors gemm_kernel)
    const bool diag_tile = tri && ti == tj;
    const long long ob = (long long)slice * g.o_bs, eb = (long long)slice * g.e_bs, db = (long long)slice * g.d_bs;
    for (int tid = 0; tid < NT; ++tid) {
      const int lane = tid & 63, wave = tid >> 6, wm = wave / t.wn, wn = wave % t.wn;
      for (int a = 0; a < SM; ++a)
        for (int b = 0; b < SN; ++b)
          for (int r = 0; r < 16; ++r) {
            const int row = i0 + wm * WTM + a * 32 + acc_row(r, lane);
            const int col = j0 + wn * WTN + b * 32 + acc_col(lane);
            if (row >= g.M || col >= g.N) continue;
            auto wr = [&](long long e) {
              access(g.out, (ob + e) * es, es, what);
              if (coverage && ob + e >= 0 && ob + e < out_elems) cover[ob + e]++;
            };
            if (tri) {
              if (diag_tile && row < col) continue;
              if (row == col) {
                if (k.mode == MODE_POLY) access(g.d_in, (db + row) * 4, 4, what);
                access(g.d_out, (db + row) * 4, 4, what);
                if (coverage) dcover[db + row]++;
                wr((long long)row * g.ldo + col);
              } else {
                if (k.mode == MODE_POLY) {
                  access(g.E, (eb + (long long)row * g.lde + col) * es, es, what);
                  access(g.d_in, (db + row) * 4, 4, what);
                  access(g.d_in, (db + col) * 4, 4, what);
                }
                wr((long long)row * g.ldo + col);
                wr((long long)col * g.ldo + row);
              }
            } else {
              access(g.d_in, (db + (k.mode == MODE_UPD_ROW ? row : col)) * 4, 4, what);
              access(g.E, (eb + (long long)row * g.lde + col) * es, es, what);
              wr((long long)row * g.ldo + col);
            }
          }
    }
  }
  if (coverage) {
    long long bad = 0;
    for (int s = 0; s < g.batch; ++s)
      for (int i = 0; i < g.M; ++i)
        for (int j = 0; j < g.N; ++j)
          if (cover[(long long)s * g.o_bs + (long long)i * g.ldo + j] != 1) ++bad;
    for (size_t i = 0; i < dcover.size(); ++i)
      if (dcover[i] != 1) ++bad;
    if (bad) fail(std::string(what) + ": " + std::to_string(bad) + " output elements not written exactly once");
  }
}

void replay_norm(const NormArgs& g, int batch, bool scale, const char* what) {
  const int NT = 256;
  for (int slice = 0; slice < batch; ++slice)
    for (int chunk = 0; chunk < g.chunks; ++chunk) {
      const long long v0 = (long long)chunk * g.chunk_vecs;
      const long long v1 = (v0 + g.chunk_vecs < g.slice_vecs) ? v0 + g.chunk_vecs : g.slice_vecs;
      if (v0 >= g.slice_vecs) fail(std::string(what) + ": empty norm block");
      // first and last vector of each thread's strided walk
      for (int tid = 0; tid < NT; ++tid) {
        const long long first = v0 + tid;
        if (first >= v1) continue;
        const long long last = first + ((v1 - 1 - first) / NT) * NT;
        for (long long v : {first, last}) {
          access(g.x, ((long long)slice * g.slice_vecs + v) * 16, 16, what);
          if (scale) access(g.y, ((long long)slice * g.slice_vecs + v) * 16, 16, what);
        }
      }
      if (scale) {
        for (int i = 0; i < g.chunks; ++i) access(g.partials, ((long long)slice * g.chunks + i) * 4, 4, what);
        if (g.norms) access(g.norms, (long long)slice * 4, 4, what);
      } else {
        access(g.partials, ((long long)slice * g.chunks + chunk) * 4, 4, what);
      }
    }
}

// Replays one ns_orthogonalize call as the driver sequences it.
void replay_call(int dtype, long long batch, long long rows, long long cols, int steps, bool alias) {
  g_bufs.clear();
  const Plan p = make_plan(batch, rows, cols, dtype);
  const size_t xbytes = (size_t)batch * rows * cols * elem_size(dtype);
  const size_t mm = (size_t)batch * p.m * p.m * elem_size(dtype);
  void* in = reg(uintptr_t(1) << 44, "in", xbytes);
  void* out = alias ? in : reg(uintptr_t(2) << 44, "out", xbytes);
  void* xtmp = reg(uintptr_t(3) << 44, "xtmp", xbytes);
  void* oa = reg(uintptr_t(4) << 44, "oa", mm);
  void* oc = reg(uintptr_t(5) << 44, "oc", mm);
  float* da = (float*)reg(uintptr_t(6) << 44, "da", (size_t)batch * p.m * 4);
  float* dc = (float*)reg(uintptr_t(7) << 44, "dc", (size_t)batch * p.m * 4);
  float* part = (float*)reg(uintptr_t(8) << 44, "partials", (size_t)batch * p.norm_chunks * 4);
  if (p.off_part + (size_t)batch * p.norm_chunks * 4 > p.total) fail("workspace plan too small");

  auto buf = [&](int s) -> void* { return iterate_in_out(steps, s) ? out : xtmp; };
  const NormArgs ng = norm_args(p, in, buf(0), nullptr, part);
  replay_norm(ng, (int)batch, false, "sumsq");
  replay_norm(ng, (int)batch, true, "scale");
  const bool cov = (long long)batch * std::max<long long>(p.m * p.m, rows * cols) <= 80LL * 1000 * 1000;
  for (int s = 1; s <= steps; ++s) {
    if (s != 1 && s != steps) continue;  // middle steps differ only in which buffer is which
    StageKind k;
    GemmArgs g = gram_args(p, buf(s - 1), oa, da, &k);
    replay_gemm(g, k, dtype, cov, "gram");
    g = poly_args(p, oa, da, oc, dc, 3.4445f, -4.775f, 2.0315f, &k);
    replay_gemm(g, k, dtype, cov, "poly");
    if (buf(s - 1) == buf(s)) fail("update reads the buffer it writes");
    g = update_args(p, buf(s - 1), oc, dc, buf(s), &k);
    replay_gemm(g, k, dtype, cov, "update");
  }
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 6 || (argc - 1) % 5 != 0) {
    std::fprintf(stderr, "usage: %s dtype batch rows cols steps [...]\n", argv[0]);
    return 2;
  }
  for (int a = 1; a + 4 < argc; a += 5) {
    const int dtype = std::atoi(argv[a]);
    const long long batch = std::atoll(argv[a + 1]), rows = std::atoll(argv[a + 2]), cols = std::atoll(argv[a + 3]);
    const int steps = std::atoi(argv[a + 4]);
    for (int alias = 0; alias < 2; ++alias) {
      const int before = g_fail;
      replay_call(dtype, batch, rows, cols, steps, alias != 0);
      std::printf("%s dtype=%d batch=%lld rows=%lld cols=%lld steps=%d alias=%d\n",
                  g_fail == before ? "OK  " : "FAIL", dtype, batch, rows, cols, steps, alias);
    }
  }
  std::printf("checks=%lld violations=%d\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}

// ns_boundscheck.cpp - host-side walk of every address the kernels of one
// ns_orthogonalize call touch, for given shapes, without a GPU.
//
// It builds the launch arguments with the driver's own functions (ns_plan.h),
// replays the kernels' index arithmetic (ns_layout.h) for every workgroup and
// thread, and checks that
//   * every workgroup id maps to a distinct tile of a valid slice,
//   * every global load and store stays inside the buffer its pointer names,
//   * every LDS index stays inside the operand's LDS region,
//   * every output element (and diagonal entry) is written exactly once
//     (a Gram without its mirror: exactly its lower block triangle),
//   * in shapes small enough for coverage maps, every load of a matrix some
//     earlier kernel of the call produced reads only elements it wrote.
// K stages of one layout other than the first and the last only move the k
// offset between those two, so only those (and the stages where an operand
// changes layout) are replayed, except for operands read as their lower
// block triangle in coverage runs, where every stage is.
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
// elements each buffer's producer wrote (coverage runs): consumers may read
// only these (or zero-fill past the buffer's range)
std::map<uintptr_t, std::vector<uint8_t>> g_written;
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

// A whole aligned 16-byte block read from a 16-byte aligned buffer: it must
// hold at least one byte of the buffer (it then lies in that byte's page; it
// may run past the buffer's end by up to 15 bytes, never before its start).
void access_block(const void* ptr, long long byte_off, const char* what) {
  ++g_checks;
  auto it = g_bufs.find(reinterpret_cast<uintptr_t>(ptr));
  if (it == g_bufs.end()) {
    fail(std::string(what) + ": pointer is not a registered buffer");
    return;
  }
  if (reinterpret_cast<uintptr_t>(ptr) % 16 || byte_off % 16 || byte_off < 0 ||
      (size_t)byte_off >= it->second.bytes)
    fail(std::string(what) + ": block at " + std::to_string(byte_off) + " holds no byte of " + it->second.name +
         " (" + std::to_string(it->second.bytes) + " bytes) or is misaligned");
}

void lds_index(int idx, int limit, const char* what) {
  ++g_checks;
  if (idx < 0 || idx >= limit)
    fail(std::string(what) + ": LDS chunk " + std::to_string(idx) + " outside [0," + std::to_string(limit) + ")");
}

// One wave's load instructions of stage kt (mirrors issue() in gemm_kernel):
// every lane either reads 16 in-range bytes of its operand slice or uses an
// offset at or past the slice end (which the buffer range check turns into
// zeros); every LDS write lands inside the stage slot.
void replay_dma(int wave, int niw, const TileCfg& t, int es, bool pnat, bool qnat, int k0, const GemmArgs& g,
                int slice, int i0, int j0, int stage_chunks, int slot, int lds_limit, const char* what) {
  const int EPC = 16 / es;
  const unsigned kOut = 0x80000000u;
  const long long pbytes = g.p_bs * es, qbytes = g.q_bs * es;
  if (pbytes >= (long long)kOut || qbytes >= (long long)kOut) fail(std::string(what) + ": slice too large for the range trick");
  for (int ti = 0; ti < niw; ++ti) {
    const int idx = wave * niw + ti;
    for (int lane = 0; lane < 64; ++lane) {
      const DmaSrc d = dma_src(idx, lane, t.bm, t.bn, t.cpr, EPC, pnat, qnat, es);
      if ((idx * 64 < t.bm * t.cpr) != d.is_p) fail(std::string(what) + ": load instruction spans both operands");
      lds_index(slot * stage_chunks + idx * 64 + lane, lds_limit, what);
      if (idx * 64 + lane >= stage_chunks) fail(std::string(what) + ": load outside its stage slot");
      const bool nat = d.is_p ? pnat : qnat;
      const int ld = d.is_p ? g.ldp : g.ldq;
      const int g_row = (d.is_p ? i0 : j0) + d.row;
      const bool row_ok = g_row < (d.is_p ? g.M : g.N);
      const bool ok = row_ok && k0 + d.kpos < g.K;
      if (d.row < 0 || d.row >= (d.is_p ? t.bm : t.bn) || d.kpos < 0 || d.kpos >= t.cpr * EPC)
        fail(std::string(what) + ": loader index outside the tile");
      // the offset exactly as issue() forms it (32-bit unsigned arithmetic)
      const int BK = t.cpr * EPC, kt = k0 / BK;
      const unsigned src_off = row_ok ? (unsigned)(nat ? ((long long)d.kpos * ld + g_row) * es
                                                       : ((long long)g_row * ld + d.kpos) * es)
                                      : kOut;
      const unsigned step = nat ? (unsigned)(BK * ld * es) : (unsigned)(BK * es);
      const unsigned long long run = (unsigned long long)src_off + (unsigned long long)kt * step;
      if (run >= (1ull << 32)) fail(std::string(what) + ": DMA offset wraps 32 bits");
      const bool full = k0 + BK <= g.K;
      const unsigned off = (full || k0 + d.kpos < g.K) ? (unsigned)run : kOut;
      const long long range = d.is_p ? pbytes : qbytes;
      if (!ok) {
        if ((long long)off < range) fail(std::string(what) + ": zero-fill lane reads inside the slice");
        continue;  // past the range check: reads zeros
      }
      const long long want = nat ? ((long long)(k0 + d.kpos) * ld + g_row) * es : ((long long)g_row * ld + k0 + d.kpos) * es;
      if ((long long)off != want) fail(std::string(what) + ": DMA offset differs from the element's");
      if (want + 16 > range || want >= (long long)kOut)
        fail(std::string(what) + ": in-range load past the slice");
      const void* src = d.is_p ? g.P : g.Q;
      const long long ebase = (long long)slice * (d.is_p ? g.p_bs : g.q_bs) + want / es;
      access(src, ebase * es, 16, what);
      auto wr = g_written.find(reinterpret_cast<uintptr_t>(src));
      if (wr != g_written.end())
        for (int e = 0; e < EPC; ++e)
          if (wr->second[ebase + e] != 1) {
            fail(std::string(what) + ": load of an element its producer did not write");
            break;
          }
    }
  }
}

// Fragment reads of one operand region (mirrors load_step()/nat_frag): the
// kernel reads per-lane bases plus compile-time offsets (kc_lane_byte,
// nat_lane_byte_*).  Every such byte address must equal the address of the
// element the DMA layout (lds_swz / nat_swz) puts there, and lie inside the
// region.
void replay_frag_reads(const TileCfg& t, int es, bool nat, int rows_region, int wave_rows, int nblk, int wofs,
                       const char* what) {
  const int EPC = 16 / es, rc = rows_region / EPC, region = rows_region * t.cpr;
  const int nh = es == 2 ? 2 : 4;
  if (t.cpr != 4 && t.cpr != 8) fail(std::string(what) + ": fragment addressing needs 4 or 8 chunks per row");
  for (int lane = 0; lane < 64; ++lane)
    for (int s = 0; s < t.cpr / 2; ++s)
      for (int a = 0; a < nblk; ++a) {
        const int rb = wofs + a * 32;
        if (!nat) {
          const int got = kc_lane_byte(wofs, s ^ kc_sigma(a, t.cpr), lane, t.cpr) + a * 32 * t.cpr * 16;
          const int want = lds_swz(rb + (lane & 31), 2 * s + (lane >> 5), t.cpr) * 16;
          if (got != want) fail(std::string(what) + ": K-contiguous fragment base + offset != swizzled chunk");
          lds_index(got / 16, region, what);
          continue;
        }
        for (int h = 0; h < nh; ++h) {
          const int got = (es == 2 ? nat_lane_byte_bf16(rb, h, lane, rc) : nat_lane_byte_f32(rb, h, lane, rc)) +
                          s * nat_step_bytes(rc, es);
          int kr, col, c, want;
          if (es == 2) {
            kr = nat_tr_kr(s, h, lane);
            col = nat_tr_col(rb, lane);
            if (col + 3 >= rows_region) fail(std::string(what) + ": transposed read outside tile");
            c = (col >> 3) ^ nat_swz(kr, rc, es);
            want = (kr * rc + c) * 16 + (col & 7) * 2;
          } else {
            kr = 8 * s + 4 * (lane >> 5) + h;
            col = rb + (lane & 31);
            c = (col >> 2) ^ nat_swz(kr, rc, es);
            want = (kr * rc + c) * 16 + (col & 3) * 4;
          }
          if (kr >= t.cpr * EPC) fail(std::string(what) + ": natural read past the stage's k rows");
          if (c >= rc) fail(std::string(what) + ": swizzled chunk past the row");
          if (got != want) fail(std::string(what) + ": natural fragment base + offset != swizzled element");
          lds_index(got / 16, region, what);
        }
      }
  (void)wave_rows;
}

// Replays one launch of gemm_kernel (grid = tiles_per_slice * batch), or,
// with `lins`, the workgroups of a grouped launch that fall on this group
// (their logical tile ids within the group).
void replay_gemm(const GemmArgs& g, const StageKind& kind, int dtype, bool coverage, const char* what,
                 const std::vector<int>* lins = nullptr) {
  const int mode = kind.mode;
  const bool tri = mode_is_tri(mode);
  const TileCfg t = tile_cfg(dtype, tri, kind.tri_cls);
  const int es = (int)elem_size(dtype);
  const int EPC = 16 / es, BK = t.cpr * EPC;
  const int NT = t.wm * t.wn * 64, WTM = t.bm / t.wm, WTN = t.bn / t.wn;  // threads of the MFMA waves
  const int SM = WTM / 32, SN = WTN / 32;
  const int G = g.tiles_per_slice * g.batch;
  const int nk = (g.K + BK - 1) / BK;
  const int LP = t.bm * t.cpr, LQ = t.bn * t.cpr, STAGE = LP + LQ;
  const int LDS = lds_chunks(t.bm, t.bn, t.cpr, t.st, es);
  const int ERC = epi_row_chunks(t.bn, es), SROW = ERC * EPC;
  const int NW = t.wm * t.wn, NIW = STAGE / 64 / NW;  // every wave issues loads and stores

  if (t.st * STAGE > LDS) fail(std::string(what) + ": the K-stage ring does not fit the LDS array");
  if (STAGE % (64 * NW) != 0 || LP % 64 != 0) fail(std::string(what) + ": stage does not split into wave loads");
  if (t.bm * SROW * es > LDS * 16) fail(std::string(what) + ": staged tile does not fit the LDS array");

  std::vector<uint8_t> seen(G, 0);
  const long long out_elems = (long long)g.o_bs * g.batch;
  std::vector<uint8_t> cover, tcover, dcover;
  if (coverage) {
    cover.assign(out_elems, 0);
    if (g.out_t && g.out_t != g.out) tcover.assign((size_t)g.ot_bs * g.batch, 0);
    if (g.d_out) dcover.assign((size_t)g.d_bs * g.batch, 0);
  }
  // fragment reads stay inside each operand region of a slot
  for (int wave = 0; wave < t.wm * t.wn; ++wave) {
    const int wm = wave / t.wn, wn = wave % t.wn;
    replay_frag_reads(t, es, kind.p_nat, t.bm, WTM, SM, wm * WTM, what);
    replay_frag_reads(t, es, kind.q_nat, t.bn, WTN, SN, wn * WTN, what);
    if (kind.p_sym) replay_frag_reads(t, es, true, t.bm, WTM, SM, wm * WTM, what);
    if (kind.q_sym) replay_frag_reads(t, es, true, t.bn, WTN, SN, wn * WTN, what);
  }

  std::vector<int> order;
  if (lins) {
    order = *lins;
    if ((long long)order.size() != G) fail(std::string(what) + ": grouped launch gives a group the wrong tile count");
  } else {
    for (int w = 0; w < G; ++w) order.push_back(xcd_remap(w, G));
  }
  for (int lin : order) {
    if (lin < 0 || lin >= G || seen[lin]) {
      fail(std::string(what) + ": tile ids are not a bijection");
      continue;
    }
    seen[lin] = 1;
    const int slice = lin / g.tiles_per_slice, q = lin - slice * g.tiles_per_slice;
    int ti, tj;
    if (tri) tri_decode(q, g.tiles_m, ti, tj);
    else rect_decode(q, g.tiles_m, g.tiles_n, ti, tj);
    // the kernel's wave column (diagonal triangle tiles remap row half 1)
    auto wave_col = [&](int wm_, int wn_) {
      const bool remap = tri && t.wm == 2 && t.wn == 4 && !(t.bm == 256 && kind.p_nat);
      return remap ? tri_wave_col(wm_, wn_, t.wn, ti == tj) : wn_;
    };
    if (slice >= g.batch || ti < 0 || tj < 0 || ti >= g.tiles_m || tj >= g.tiles_n || (tri && tj > ti)) {
      fail(std::string(what) + ": tile decode out of range");
      continue;
    }
    const int i0 = ti * t.bm, j0 = tj * t.bn;
    // first stage of natural-layout reads of each operand (mirrors gemm_kernel)
    const int nat_p = kind.p_sym ? sym_nat_from(i0, g.sym_tile, BK) : (kind.p_nat ? 0 : 0x7fffffff);
    const int nat_q = kind.q_sym ? sym_nat_from(j0, g.sym_tile, BK) : (kind.q_nat ? 0 : 0x7fffffff);
    if (kind.p_sym || kind.q_sym) {
      if (!sym_layout_ok(std::max(kind.p_sym ? t.bm : 0, kind.q_sym ? t.bn : 0), g.sym_tile, BK, t.st))
        fail(std::string(what) + ": symmetric operand layout not valid for this tile");
      if ((kind.p_sym && nat_p < nk && nat_p % t.st) || (kind.q_sym && nat_q < nk && nat_q % t.st))
        fail(std::string(what) + ": layout phase does not start at a multiple of the ring depth");
      if (kind.p_sym && kind.q_sym && nat_q > nat_p) fail(std::string(what) + ": Q must switch layouts first");
    }
    std::vector<int> kst;
    if (coverage && (kind.p_sym || kind.q_sym)) {
      for (int kt = 0; kt < nk; ++kt) kst.push_back(kt);
    } else {
      kst.push_back(0);
      if (nk > 1) kst.push_back(nk - 1);
      for (int b : {nat_p - 1, nat_p, nat_q - 1, nat_q})
        if (b > 0 && b < nk - 1) kst.push_back(b);
    }
    // a diagonal Gram or poly tile (2-slot ring) loads the P rows only, spread over
    // every wave, and reads its Q fragments from the P region: the operands
    // must be the same rows of the same matrix
    const bool dshare = (mode == MODE_GRAM || mode == MODE_POLY) && t.st == 2 && ti == tj &&
                        kind.p_nat == kind.q_nat && kind.p_sym == kind.q_sym;
    if (dshare && (g.P != g.Q || g.ldp != g.ldq || g.p_bs != g.q_bs || i0 != j0 || t.bm != t.bn || NIW % 2 ||
                   nat_p != nat_q || NW * (NIW / 2) * 64 != t.bm * t.cpr))  // ... and cover every P chunk
      fail(std::string(what) + ": diagonal tile shares operands that differ");
    for (int kt : kst)
      for (int wave = 0; wave < NW; ++wave)
        replay_dma(wave, dshare ? NIW / 2 : NIW, t, es, kt >= nat_p, kt >= nat_q, kt * BK, g, slice, i0, j0, STAGE,
                   kt % t.st, LDS, what);
    // norm folded into the first step: the slice's partial sums of squares
    if (mode != MODE_POLY && g.d_norm != nullptr)
      for (int i = 0; i < g.norm_n; ++i) access(g.d_norm, ((long long)slice * g.norm_n + i) * 4, 4, what);
    if (mode == MODE_POLY && g.d_norm != nullptr) fail(std::string(what) + ": poly takes no norm");
    // epilogue operands captured from the K stages (mirrors capture())
    const long long db0 = (long long)slice * g.d_bs;
    const int RCQ = t.bn / EPC;
    for (int kt = 0; kt < nk && mode != MODE_GRAM; ++kt) {
      const int k0 = kt * BK, slot = kt % t.st;
      if (mode == MODE_POLY && kt >= nat_p) {
        bool any = false;
        for (int wn = 0; wn < t.wn; ++wn)
          for (int b = 0; b < SN; ++b) {
            const int jb = j0 + wn * WTN + b * 32;
            any = any || (jb >= k0 && jb < k0 + BK);
          }
        if (any) fail(std::string(what) + ": poly capture at a stage where P is not K-contiguous");
        continue;  // the kernel compiles no capture in its natural-layout phase
      }
      for (int tid = 0; tid < NT; ++tid) {
        const int lane = tid & 63, wave = tid >> 6, wm = wave / t.wn, wn = wave_col(wm, wave % t.wn);
        if (mode == MODE_UPD_ROW) {
          for (int a = 0; a < SM; ++a) {
            const int ib = i0 + wm * WTM + a * 32;
            if (kt == 0 && ib + (lane & 31) < g.M) access(g.d_in, (db0 + ib + (lane & 31)) * 4, 4, what);
            if (ib < k0 || ib >= k0 + BK) continue;
            const int kr = ib - k0 + (lane & 31);
            for (int b = 0; b < SN; ++b)
              for (int rg = 0; rg < 4; ++rg) {
                const int jl = wn * WTN + b * 32 + acc_j(rg, lane);
                const int c = (jl / EPC) ^ nat_swz(kr, RCQ, es);
                if (kr >= BK || c >= RCQ) fail(std::string(what) + ": capture read outside the NAT tile");
                lds_index(slot * STAGE + LP + kr * RCQ + c, LDS, what);
              }
          }
        } else {
          for (int b = 0; b < SN; ++b) {
            const int jb = j0 + wn * WTN + b * 32;
            if (jb < k0 || jb >= k0 + BK) continue;
            for (int rg = 0; rg < 4; ++rg) {
              const int j = jb + acc_j(rg, lane), kk = j - k0;
              if (mode == MODE_UPD_COL) {
                // buffer load over the slice's d_bs floats: in range exactly
                // when j < N (then all 16 bytes are), else it reads zeros
                const long long off = (long long)(jb * 4) + acc_j(rg, lane) * 4, range = g.d_bs * 4;
                if ((off < range) != (j < g.N)) fail(std::string(what) + ": d_C buffer range != column range");
                if (off < range) {
                  if (off + 16 > range) fail(std::string(what) + ": d_C read straddles the range end");
                  access(g.d_in, (db0 + j) * 4, 16, what);
                }
              }
              for (int a = 0; a < SM; ++a) {
                const int il = wm * WTM + a * 32 + (lane & 31);
                if (kk / EPC >= t.cpr) fail(std::string(what) + ": capture chunk outside the stage");
                lds_index(slot * STAGE + lds_swz(il, kk / EPC, t.cpr), slot * STAGE + LP, what);
              }
            }
          }
        }
      }
    }
    // epilogue step 1 (mirrors gemm_kernel): registers -> staged tile
    const bool diag_tile = tri && ti == tj;
    const long long ob = (long long)slice * g.o_bs, db = (long long)slice * g.d_bs;
    const int qsz = 4 * es;  // bytes of 4 consecutive elements
    for (int tid = 0; tid < NT; ++tid) {
      const int lane = tid & 63, wave = tid >> 6, wm = wave / t.wn, wn = wave_col(wm, wave % t.wn);
      for (int a = 0; a < SM; ++a) {
        const int il = wm * WTM + a * 32 + acc_i(lane), i = i0 + il;
        for (int b = 0; b < SN; ++b)
          for (int rg = 0; rg < 4; ++rg) {
            const int jl = wn * WTN + b * 32 + acc_j(rg, lane), j = j0 + jl;
            if (i >= g.M || j >= g.N) continue;
            if (j + 3 >= g.N) fail(std::string(what) + ": quad crosses N");
            const long long sbyte = ((long long)il * SROW + jl) * es;
            if (sbyte < 0 || sbyte + qsz > (long long)LDS * 16 || sbyte % qsz != 0)
              fail(std::string(what) + ": staged write outside LDS or misaligned");
            if (mode == MODE_GRAM || mode == MODE_POLY) {
              if (mode == MODE_POLY) {
                access(g.d_in, (db + j) * 4, 16, what);
                access(g.d_in, (db + i) * 4, 4, what);
              }
              for (int e = 0; e < 4; ++e)
                if (i == j + e) {
                  access(g.d_out, (db + i) * 4, 4, what);
                  if (coverage) dcover[db + i]++;
                }
            }
          }
      }
    }
    // step 2: direct store of tile rows
    const int CPT = t.bn / EPC;
    for (int qd = 0; qd < t.bm * CPT; ++qd) {
      const int il = qd / CPT, c = qd % CPT, i = i0 + il, j = j0 + c * EPC;
      if (i >= g.M || j >= g.N) continue;
      if (diag_tile && c * EPC + EPC - 1 > il) {
        for (int e = 0; e < EPC; ++e) {
          const int jl = c * EPC + e;
          const long long src = (jl <= il) ? (long long)il * SROW + jl : (long long)jl * SROW + il;
          if (src * es + es > (long long)LDS * 16) fail(std::string(what) + ": mirror read outside LDS");
        }
      }
      access(g.out, (ob + (long long)i * g.ldo + j) * es, 16, what);
      if (coverage)
        for (int e = 0; e < EPC; ++e) cover[ob + (long long)i * g.ldo + j + e]++;
    }
    // step 3: transposed store (bf16: transposing LDS reads, mirror_lane)
    if (g.out_t != nullptr && !diag_tile) {
      const long long tb = (long long)slice * g.ot_bs;
      auto store_t = [&](int j, int i) {
        access(g.out_t, (tb + (long long)j * g.ldt + i) * es, 16, what);
        if (coverage) {
          std::vector<uint8_t>& cv = (g.out_t == g.out) ? cover : tcover;
          for (int e = 0; e < EPC; ++e) cv[tb + (long long)j * g.ldt + i + e]++;
        }
      };
      if (es == 2) {
        const int U = (t.bn / 16) * (t.bm / 32);
        if (t.bn % 16 || t.bm % 32 || U % NW) fail(std::string(what) + ": mirror units do not split into waves");
        for (int u = 0; u < U; ++u)
          for (int lane = 0; lane < 64; ++lane) {
            const MirrorLane ml = mirror_lane(u, lane, t.bn);
            // every lane reads (the transposing read exchanges data in 16-lane groups)
            for (int h = 0; h < 2; ++h) {
              const long long e0 = (long long)ml.src_row[h] * SROW + ml.src_col;
              if (ml.src_row[h] >= t.bm || ml.src_col + 3 >= t.bn || (e0 * es) % 8)
                fail(std::string(what) + ": transposing read outside the staged tile or misaligned");
              if ((e0 + 4) * es > (long long)LDS * 16) fail(std::string(what) + ": transposed read outside LDS");
            }
            if (ml.col >= t.bn || ml.row0 + 7 >= t.bm) fail(std::string(what) + ": mirror lane outside the tile");
            const int j = j0 + ml.col, i = i0 + ml.row0;
            if (j < g.N && i < g.M) store_t(j, i);
          }
        // the exchange model: lane t of a 16-lane group gets element t % 4 of
        // the vectors read by lanes 4 e + t / 4; with the source addresses
        // above that is column cb + t, rows row0 + 4 h + e
        for (int u = 0; u < U; ++u)
          for (int lane = 0; lane < 64; ++lane) {
            const MirrorLane ml = mirror_lane(u, lane, t.bn);
            const int t16 = lane & 15, g16 = lane & ~15;
            for (int h = 0; h < 2; ++h)
              for (int e = 0; e < 4; ++e) {
                const MirrorLane src = mirror_lane(u, g16 + 4 * e + t16 / 4, t.bn);
                const int row = src.src_row[h], col = src.src_col + t16 % 4;
                if (row != ml.row0 + 4 * h + e || col != ml.col)
                  fail(std::string(what) + ": transposing read does not deliver the mirror element");
              }
          }
      } else {
        const int RCH = t.bm / EPC;
        for (int qd = 0; qd < t.bn * RCH; ++qd) {
          const int jl = qd % t.bn, rc = qd / t.bn, j = j0 + jl, i = i0 + rc * EPC;
          if (j >= g.N || i >= g.M) continue;
          if (((long long)(rc * EPC + EPC - 1) * SROW + jl) * es + es > (long long)LDS * 16)
            fail(std::string(what) + ": transposed read outside LDS");
          store_t(j, i);
        }
      }
    }
  }
  if (coverage) {
    long long bad = 0;
    // a triangle kernel without a transposed store writes its lower block
    // triangle only (tiles of t.bm rows; diagonal tiles whole)
    const bool lower_only = tri && g.out_t == nullptr;
    for (int s = 0; s < g.batch; ++s)
      for (int i = 0; i < g.M; ++i)
        for (int j = 0; j < g.N; ++j) {
          const uint8_t c = cover[(long long)s * g.o_bs + (long long)i * g.ldo + j];
          const uint8_t want = (lower_only && j / t.bm > i / t.bm) ? 0 : 1;
          if (c != want) ++bad;
          if (!tcover.empty() && tcover[(long long)s * g.ot_bs + (long long)j * g.ldt + i] != 1) ++bad;
        }
    for (size_t i = 0; i < dcover.size(); ++i)
      if (dcover[i] != 1) ++bad;
    if (bad) fail(std::string(what) + ": " + std::to_string(bad) + " output elements not written exactly once");
    g_written[reinterpret_cast<uintptr_t>(g.out)] = cover;
  }
}

// A launch over several groups (mirrors launch_mode / gemm_kernel with NG >
// 1): split as the launcher splits, map every workgroup of each launch to
// its group and tile id, then replay each group on exactly those ids.
void replay_gemm_grouped(const std::vector<GemmArgs>& gs, const StageKind& kind, int dtype, bool coverage,
                         const char* what) {
  if (gs.size() == 1) {
    replay_gemm(gs[0], kind, dtype, coverage, what);
    return;
  }
  for (int g0 = 0; g0 < (int)gs.size();) {
    int start[kMaxLaunchGroups];
    long long total = 0;
    const int k = launch_chunk(
        (int)gs.size() - g0, [&](int i) { return (long long)gs[g0 + i].tiles_per_slice * gs[g0 + i].batch; },
        start, &total);
    if (k < 1) {
      fail(std::string(what) + ": empty launch");
      return;
    }
    std::vector<std::vector<int>> lins(k);
    std::vector<int> xcd_tiles(8, 0), xcd_first_group(8, 0);
    for (long long w = 0; w < total; ++w) {
      int grp = -1;
      const int lin = xcd_group_tile((int)w, (int)total, start, k, &grp);
      if (grp < 0 || grp >= k) {
        fail(std::string(what) + ": workgroup mapped to no group");
        continue;
      }
      // each XCD walks the groups in order
      if (grp < xcd_first_group[w % 8]) fail(std::string(what) + ": an XCD goes back to an earlier group");
      xcd_first_group[w % 8] = grp;
      lins[grp].push_back(lin);
    }
    for (int i = 0; i < k; ++i) replay_gemm(gs[g0 + i], kind, dtype, coverage, what, &lins[i]);
    g0 += k;
  }
}

void replay_norm(const NormArgs& g, int batch, bool scale, const char* what) {
  const int NT = 256;
  for (int slice = 0; slice < batch; ++slice)
    for (int chunk = 0; chunk < g.chunks; ++chunk) {
      const long long v0 = (long long)chunk * g.chunk_vecs;
      const long long v1 = (v0 + g.chunk_vecs < g.slice_vecs) ? v0 + g.chunk_vecs : g.slice_vecs;
      if (v0 >= g.slice_vecs) fail(std::string(what) + ": empty norm block");
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

// The grouped sum-of-squares launch (mirrors sumsq_grouped_kernel): every
// block maps to a distinct (group, slice, chunk), and each group's blocks
// are then the plain launch's.
void replay_norm_grouped(const std::vector<NormArgs>& gs, const std::vector<int>& batch, const char* what) {
  for (int g0 = 0; g0 < (int)gs.size();) {
    int start[kMaxLaunchGroups];
    long long total = 0;
    const int k = launch_chunk(
        (int)gs.size() - g0, [&](int i) { return (long long)gs[g0 + i].chunks * batch[g0 + i]; }, start, &total);
    std::vector<std::vector<uint8_t>> seen(k);
    for (int i = 0; i < k; ++i) seen[i].assign((size_t)gs[g0 + i].chunks * batch[g0 + i], 0);
    for (long long b = 0; b < total; ++b) {
      const int grp = launch_group((int)b, start, k);
      const long long local = b - start[grp];
      const NormArgs& a = gs[g0 + grp];
      const long long slice = local / a.chunks, chunk = local % a.chunks;
      if (slice >= batch[g0 + grp] || local >= (long long)seen[grp].size() || seen[grp][local]++)
        fail(std::string(what) + ": grouped norm block maps outside its group or twice");
      (void)chunk;
    }
    for (int i = 0; i < k; ++i) {
      for (uint8_t v : seen[i])
        if (v != 1) fail(std::string(what) + ": grouped norm block not covered once");
      replay_norm(gs[g0 + i], batch[g0 + i], false, what);
    }
    g0 += k;
  }
}

// Pad (mirrors pad_sumsq_kernel's gathers; its vector ranges and partials
// are those of the sum-of-squares replay over the padded copy) or unpad
// (mirrors unpad_kernel): the first and last 16-byte vector of every row
// visited, through the kernels' own pad_vec, with every element read or
// written in bounds.
void replay_pad(const PadArgs& g, int es, const char* what) {
  if (g.urows > g.rows || g.ucols > g.cols || g.rows % 8 || g.cols % 8) fail(std::string(what) + ": bad padded shape");
  if (g.rows * g.cols >= (1LL << 29)) fail(std::string(what) + ": slice too large for 32-bit vector indexes");
  const int epv = 16 / es, vpr = (int)(g.cols / epv);
  const long long rows_v = g.to_padded ? g.rows : g.urows;
  for (long long b = 0; b < g.batch; ++b)
    for (long long i = 0; i < rows_v; ++i)
      for (int c : {0, vpr - 1}) {
        const int v = (int)(i * vpr + c);
        int r, j0;
        pad_vec(v, vpr, epv, &r, &j0);
        if (r != i || j0 != c * epv) fail(std::string(what) + ": pad_vec maps a vector to the wrong place");
        const long long padded_vec = (b * g.rows * vpr + v) * 16;
        if (g.to_padded) {
          access(g.dst, padded_vec, 16, what);
          if (r < g.urows && j0 < g.ucols) {  // mirrors pad_sumsq_kernel
            const long long n = std::min<long long>(epv, g.ucols - j0);
            const long long a = ((b * g.urows + r) * g.ucols + j0) * es, sh = a % 16;
            access(g.src, a, (int)(n * es), what);  // the elements the vector takes
            access_block(g.src, a - sh, what);
            // the second block, clamped to the block holding the array's last byte
            const long long last = (g.batch * g.urows * g.ucols * es - 1) / 16 * 16;
            access_block(g.src, std::min(a - sh + 16, last), what);
            if (sh + n * es > 16 && a - sh + 16 > last) fail(std::string(what) + ": needed block past the last one");
          }
        }
      }
  if (g.to_padded) return;
  // unpad: every 16-byte block of the caller's array (mirrors unpad_kernel)
  const long long per_slice = g.urows * g.ucols, total = g.batch * per_slice;
  for (long long e0 = 0; e0 < total; e0 += epv) {
    long long sl = e0 / per_slice;
    long long rr = e0 - sl * per_slice, i = rr / g.ucols, j = rr - i * g.ucols;
    if (j + epv <= g.ucols && e0 + epv <= total) {  // one padded row: aligned blocks of it
      const long long row = (sl * g.rows + i) * g.cols * es, sh = (j * es) % 16;
      if (row % 16) fail(std::string(what) + ": padded row not 16-byte aligned");
      access(g.src, row + j * es - sh, 16, what);
      if (sh) access(g.src, row + j * es - sh + 16, 16, what);
      if (row + j * es - sh + (sh ? 32 : 16) > row + g.cols * es) fail(std::string(what) + ": block outside its row");
      access(g.dst, e0 * es, 16, what);
      continue;
    }
    for (int k = 0; k < epv; ++k) {
      if (e0 + k < total) {
        if (i >= g.urows || j >= g.ucols || sl >= g.batch) fail(std::string(what) + ": element outside the block");
        access(g.src, ((sl * g.rows + i) * g.cols + j) * es, es, what);
        if (e0 + epv > total) access(g.dst, (e0 + k) * es, es, what);
      }
      if (++j == g.ucols) {
        j = 0;
        if (++i == g.urows) {
          i = 0;
          ++sl;
        }
      }
    }
    if (e0 + epv <= total) access(g.dst, e0 * es, 16, what);
  }
}

// Replays one ns_orthogonalize call as the driver sequences it.
void replay_call(int dtype, long long batch, long long urows, long long ucols, int steps, bool alias) {
  g_bufs.clear();
  g_written.clear();
  const Plan p = make_plan(batch, urows, ucols, dtype);
  const long long rows = p.rows, cols = p.cols;  // padded to multiples of 8
  const int es = (int)elem_size(dtype);
  const size_t ubytes = (size_t)batch * urows * ucols * es;
  const size_t xbytes = (size_t)batch * rows * cols * es;
  const size_t mm = (size_t)batch * p.m * p.m * es;
  void* uin = reg(uintptr_t(1) << 44, "in", ubytes);
  void* uout = alias ? uin : reg(uintptr_t(2) << 44, "out", ubytes);
  void* in = uin;
  void* out = uout;
  if (p.padded) {  // the method runs on zero-padded workspace copies
    if (p.off_pout - p.off_pin < xbytes || p.total - p.off_pout < xbytes) fail("workspace plan: padded buffers");
    in = reg(uintptr_t(9) << 44, "padded in", xbytes);
    out = reg(uintptr_t(10) << 44, "padded out", xbytes);
    replay_pad(pad_args(p, uin, in, true), es, "pad");
  } else if (ubytes != xbytes) {
    fail("unpadded plan with a padded size");
  }
  alias = in == out;
  void* xtmp = reg(uintptr_t(3) << 44, "xtmp", xbytes);
  void* oa = reg(uintptr_t(4) << 44, "oa", mm);
  void* oc = reg(uintptr_t(5) << 44, "oc", mm);
  float* da = (float*)reg(uintptr_t(6) << 44, "da", (size_t)batch * p.m * 4);
  float* dc = (float*)reg(uintptr_t(7) << 44, "dc", (size_t)batch * p.m * 4);
  float* part = (float*)reg(uintptr_t(8) << 44, "partials", (size_t)batch * p.norm_chunks * 4);
  if (p.off_part + (size_t)batch * p.norm_chunks * 4 > p.total) fail("workspace plan too small");
  if (p.off_oa - p.off_xtmp < xbytes) fail("workspace plan overlaps the iterate buffer");

  const bool fold = fold_normalisation(steps);
  const bool copy_in = input_copy_needed(steps, alias);
  auto wbuf = [&](int s) -> void* { return iterate_in_out(steps, s) ? out : xtmp; };
  auto buf = [&](int s) -> void* { return (s == 0 && fold) ? (copy_in ? xtmp : in) : wbuf(s); };
  {
    const NormArgs ng = norm_args(p, in, fold ? nullptr : wbuf(0), nullptr, part);
    replay_norm(ng, (int)batch, false, "sumsq");
    if (!fold) replay_norm(ng, (int)batch, true, "scale");
  }
  const bool cov = (long long)batch * std::max<long long>(p.m * p.m, rows * cols) <= 80LL * 1000 * 1000;
  for (int s = 1; s <= steps; ++s) {
    if (s != 1 && s != steps && s != 2) continue;  // later steps differ only in which buffer is which
    const float* dn = (fold && s == 1) ? part : nullptr;
    StageKind kind;
    GemmArgs g = gram_args(p, buf(s - 1), oa, da, &kind, dn, !gram_lower_only(p));
    replay_gemm(g, kind, dtype, cov, "gram");
    g = poly_args(p, oa, da, oc, dc, 3.4445f, -4.775f, 2.0315f, &kind);
    replay_gemm(g, kind, dtype, cov, "poly");
    if (buf(s - 1) == wbuf(s)) fail("update reads the buffer it writes");
    g = update_args(p, buf(s - 1), oc, dc, wbuf(s), &kind, dn);
    replay_gemm(g, kind, dtype, cov, "update");
  }
  if (steps >= 1 && wbuf(steps) != out) fail("the last step does not write the result buffer");
  if (p.padded) replay_pad(pad_args(p, out, uout, false), es, "unpad");
}

// Replays one ns_orthogonalize_grouped call as the driver sequences it.
struct Shape {
  long long batch, rows, cols;
};
void replay_grouped_call(int dtype, int steps, const std::vector<Shape>& shapes, bool alias) {
  if (steps == 0) {  // the driver normalises the stacks one by one
    for (const Shape& sh : shapes)
      if (sh.batch > 0) replay_call(dtype, sh.batch, sh.rows, sh.cols, 0, alias);
    return;
  }
  g_bufs.clear();
  g_written.clear();
  struct G {
    Plan p;
    void *uin, *uout, *in, *out, *xtmp, *oa, *oc;
    float *da, *dc, *part;
    bool copy_in;
  };
  std::vector<G> gs;
  const int es = (int)elem_size(dtype);
  for (size_t i = 0; i < shapes.size(); ++i) {
    const Shape& sh = shapes[i];
    if (sh.batch == 0) continue;
    G g{};
    g.p = make_plan(sh.batch, sh.rows, sh.cols, dtype);
    const Plan& p = g.p;
    auto at = [&](int k) { return (uintptr_t(16 * (i + 1) + k)) << 40; };
    const std::string id = "[" + std::to_string(i) + "]";
    const size_t ubytes = (size_t)sh.batch * sh.rows * sh.cols * es, xbytes = (size_t)p.batch * p.rows * p.cols * es;
    const size_t mm = (size_t)p.batch * p.m * p.m * es;
    g.uin = reg(at(1), "in" + id, ubytes);
    g.uout = alias ? g.uin : reg(at(2), "out" + id, ubytes);
    g.in = g.uin;
    g.out = g.uout;
    if (p.padded) {
      g.in = reg(at(9), "padded in" + id, xbytes);
      g.out = reg(at(10), "padded out" + id, xbytes);
      replay_pad(pad_args(p, g.uin, g.in, true), es, "pad");
    }
    g.xtmp = reg(at(3), "xtmp" + id, xbytes);
    g.oa = reg(at(4), "oa" + id, mm);
    g.oc = reg(at(5), "oc" + id, mm);
    g.da = (float*)reg(at(6), "da" + id, (size_t)p.batch * p.m * 4);
    g.dc = (float*)reg(at(7), "dc" + id, (size_t)p.batch * p.m * 4);
    g.part = (float*)reg(at(8), "partials" + id, (size_t)p.batch * p.norm_chunks * 4);
    g.copy_in = input_copy_needed(steps, g.in == g.out);
    gs.push_back(g);
  }
  if (gs.empty()) return;
  std::vector<Plan> plans;
  for (const G& g : gs) plans.push_back(g.p);
  const TileChoice tc = choose_tiles(plans.data(), (int)plans.size());
  {
    // padded stacks: the pad pass computes their sums of squares (the same
    // blocks over the padded copy); the grouped launch covers the others
    std::vector<NormArgs> na;
    std::vector<int> nb;
    for (const G& g : gs) {
      if (g.p.padded) {
        replay_norm(norm_args(g.p, g.in, nullptr, nullptr, g.part), (int)g.p.batch, false, "pad sumsq");
        continue;
      }
      na.push_back(norm_args(g.p, g.in, nullptr, nullptr, g.part));
      nb.push_back((int)g.p.batch);
    }
    if (!na.empty()) replay_norm_grouped(na, nb, "grouped sumsq");
  }
  auto wbuf = [&](const G& g, int s) -> void* { return iterate_in_out(steps, s) ? g.out : g.xtmp; };
  auto buf = [&](const G& g, int s) -> void* { return s == 0 ? (g.copy_in ? g.xtmp : g.in) : wbuf(g, s); };
  long long elems = 0;
  for (const G& g : gs) elems += g.p.batch * std::max<long long>(g.p.m * g.p.m, g.p.rows * g.p.cols);
  const bool cov = elems <= 80LL * 1000 * 1000;
  for (int s = 1; s <= steps; ++s) {
    if (s != 1 && s != steps && s != 2) continue;
    StageKind kind;
    for (int o = 0; o < 2; ++o) {
      std::vector<GemmArgs> ga;
      for (const G& g : gs)
        if (g.p.tall == (o == 1))
          ga.push_back(gram_args(g.p, tc, buf(g, s - 1), g.oa, g.da, &kind, s == 1 ? g.part : nullptr,
                                 !tc.lower_only));
      if (!ga.empty()) replay_gemm_grouped(ga, kind, dtype, cov, "grouped gram");
    }
    {
      std::vector<GemmArgs> ga;
      for (const G& g : gs) ga.push_back(poly_args(g.p, tc, g.oa, g.da, g.oc, g.dc, 3.4445f, -4.775f, 2.0315f, &kind));
      replay_gemm_grouped(ga, kind, dtype, cov, "grouped poly");
    }
    for (int o = 0; o < 2; ++o) {
      std::vector<GemmArgs> ga;
      for (const G& g : gs)
        if (g.p.tall == (o == 1)) {
          if (buf(g, s - 1) == wbuf(g, s)) fail("update reads the buffer it writes");
          ga.push_back(update_args(g.p, buf(g, s - 1), g.oc, g.dc, wbuf(g, s), &kind, s == 1 ? g.part : nullptr));
        }
      if (!ga.empty()) replay_gemm_grouped(ga, kind, dtype, cov, "grouped update");
    }
  }
  for (const G& g : gs) {
    if (steps >= 1 && wbuf(g, steps) != g.out) fail("the last step does not write the result buffer");
    if (g.p.padded) replay_pad(pad_args(g.p, g.out, g.uout, false), es, "unpad");
  }
}

}  // namespace

// The grouped tile map: one group is xcd_remap; for several groups every
// XCD holds a near-equal share (at most one tile more or less) of each.
void check_group_map() {
  for (int G = 1; G <= 2000; ++G) {
    const int st0[1] = {0};
    for (int w = 0; w < G; ++w) {
      int grp = -1;
      if (xcd_group_tile(w, G, st0, 1, &grp) != xcd_remap(w, G) || grp != 0)
        fail("xcd_group_tile with one group differs from xcd_remap");
    }
  }
  for (int trial = 0; trial < 200; ++trial) {
    const int n = 2 + trial % 15;
    int start[kMaxLaunchGroups];
    int G = 0;
    for (int i = 0; i < n; ++i) {
      start[i] = G;
      G += 1 + (trial * 7919 + i * 104729) % 997;
    }
    std::vector<std::vector<int>> per(n, std::vector<int>(8, 0));
    std::vector<std::vector<uint8_t>> seen(n);
    for (int i = 0; i < n; ++i) seen[i].assign((i + 1 < n ? start[i + 1] : G) - start[i], 0);
    for (int w = 0; w < G; ++w) {
      int grp = -1;
      const int lin = xcd_group_tile(w, G, start, n, &grp);
      if (grp < 0 || grp >= n || lin < 0 || lin >= (int)seen[grp].size() || seen[grp][lin]++) {
        fail("xcd_group_tile is not a bijection onto the groups' tiles");
        return;
      }
      per[grp][w % 8]++;
    }
    for (int i = 0; i < n; ++i) {
      const int T = (int)seen[i].size();
      for (int x = 0; x < 8; ++x)
        if (per[i][x] < T / 8 || per[i][x] > T / 8 + 1) fail("an XCD's share of a group is not T/8 (+1)");
    }
  }
}

// The diagonal tiles' wave columns are a permutation within each row half,
// and the blocks they skip lie wholly above the diagonal.
// tri_decode maps the tiles of every triangle size onto the lower triangle
// one to one
void check_tri_decode() {
  for (int T = 1; T <= 300; ++T) {
    std::vector<char> seen((size_t)T * T, 0);
    const int n = T * (T + 1) / 2;
    for (int q = 0; q < n; ++q) {
      int ti = -1, tj = -1;
      tri_decode(q, T, ti, tj);
      if (ti < 0 || ti >= T || tj < 0 || tj > ti || seen[(size_t)ti * T + tj]++)
        fail("tri_decode: tile " + std::to_string(q) + " of " + std::to_string(T) + " rows maps wrongly");
    }
  }
}

void check_diag_waves() {
  for (int wm = 0; wm < 2; ++wm) {
    int seen = 0;
    for (int wn = 0; wn < 4; ++wn) seen |= 1 << tri_wave_col(wm, wn, 4, true);
    if (seen != 0xF) fail("tri_wave_col is not a permutation of the wave columns");
  }
  for (int bm : {128, 256}) {
    const int SM = bm / 2 / 32, SN = bm / 4 / 32, nb = bm / 32;
    std::vector<int> per_simd(4, 0), needed(nb * nb, 0);
    for (int wave = 0; wave < 8; ++wave) {
      const int wm = wave / 4, wn = tri_wave_col(wm, wave % 4, 4, true);
      for (int a = 0; a < SM; ++a)
        for (int b = 0; b < SN; ++b) {
          const int rb = wm * SM + a, cb = wn * SN + b;
          const bool above = tri_block_above(wm, wn, a, b, SM, SN);
          if (above != (cb > rb)) fail("tri_block_above disagrees with the block's position");
          if (!above) {
            per_simd[wave % 4]++;
            needed[rb * nb + cb]++;
          }
        }
    }
    for (int rb = 0; rb < nb; ++rb)
      for (int cb = 0; cb < nb; ++cb)
        if (needed[rb * nb + cb] != (cb <= rb ? 1 : 0)) fail("a block on or below the diagonal is not computed once");
    const int mx = *std::max_element(per_simd.begin(), per_simd.end());
    if (mx > (bm == 256 ? 10 : 3)) fail("diagonal-tile blocks are not balanced over the SIMDs");
  }
}

int main(int argc, char** argv) {
  check_group_map();
  check_tri_decode();
  check_diag_waves();
  // grouped call: --group dtype steps b r c [b r c ...]
  if (argc >= 7 && std::string(argv[1]) == "--group" && (argc - 4) % 3 == 0) {
    const int dtype = std::atoi(argv[2]), steps = std::atoi(argv[3]);
    std::vector<Shape> shapes;
    for (int a = 4; a + 2 < argc; a += 3)
      shapes.push_back(Shape{std::atoll(argv[a]), std::atoll(argv[a + 1]), std::atoll(argv[a + 2])});
    for (int alias = 0; alias < 2; ++alias) {
      const int before = g_fail;
      replay_grouped_call(dtype, steps, shapes, alias != 0);
      std::printf("%s grouped dtype=%d steps=%d stacks=%d alias=%d\n", g_fail == before ? "OK  " : "FAIL", dtype,
                  steps, (int)shapes.size(), alias);
    }
    std::printf("checks=%lld violations=%d\n", g_checks, g_fail);
    return g_fail == 0 ? 0 : 1;
  }
  if (argc < 6 || (argc - 1) % 5 != 0) {
    std::fprintf(stderr, "usage: %s dtype batch rows cols steps [...]\n       %s --group dtype steps b r c [...]\n",
                 argv[0], argv[0]);
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

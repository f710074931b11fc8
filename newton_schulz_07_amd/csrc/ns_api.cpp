// ns_api.cpp - host driver of libns_hip.so: argument checks, workspace,
// and the sequence of launches of one Newton–Schulz call.
//
// One call on a [batch, rows, cols] stack enqueues 2 + 3 * ns_steps kernels
// on the caller's stream, each covering the whole stack (the batch is part of
// the grid, so a stack of experts is one launch per stage; prime-rl PR #3873,
// "Summary" item 2, and param-decomp PR #978, "What").
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/ns_hip.h"
#include "ns_kernels.h"
#include "ns_layout.h"
#include "ns_plan.h"

namespace {

using ns::GemmArgs;
using ns::NormArgs;
using ns::Plan;
using ns::make_plan;

thread_local std::string t_err;
thread_local std::string t_cfg;

int fail(int status, const std::string& msg) {
  t_err = msg;
  return status;
}

size_t esize(int dtype) { return ns::elem_size(dtype); }

int check_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return NS_OK;
  return fail(NS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// ---------------------------------------------------------------- checks

int check_dtype(int dtype) {
  if (dtype != NS_DTYPE_F32 && dtype != NS_DTYPE_BF16)
    return fail(NS_ERR_DTYPE, "dtype must be 0 (fp32) or 1 (bf16), got " + std::to_string(dtype));
  return NS_OK;
}

// any_dims: rows and cols need not be multiples of 8 (ns_orthogonalize pads
// such shapes; the stage exports do not)
int check_shape(int64_t batch, int64_t rows, int64_t cols, bool any_dims = false) {
  if (batch < 0) return fail(NS_ERR_INVALID_ARG, "batch must be >= 0");
  if (rows <= 0 || cols <= 0) return fail(NS_ERR_INVALID_ARG, "rows and cols must be > 0");
  if (!any_dims && (rows % 8 != 0 || cols % 8 != 0))
    return fail(NS_ERR_ALIGNMENT, "rows and cols must be multiples of 8 (16-byte rows), got " +
                                      std::to_string(rows) + "x" + std::to_string(cols));
  if (rows >= (int64_t(1) << 29) || cols >= (int64_t(1) << 29) ||
      ns::round_up8(rows) * ns::round_up8(cols) >= (int64_t(1) << 29))
    return fail(NS_ERR_INVALID_ARG, "a slice must hold fewer than 2^29 elements (2 GiB of fp32)");
  if (batch > 65535) return fail(NS_ERR_INVALID_ARG, "batch must be <= 65535");
  return NS_OK;
}

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(NS_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(NS_ERR_ALIGNMENT, std::string(name) + " is not 16-byte aligned");
  return NS_OK;
}

std::mutex g_arch_mu;
std::map<int, int> g_arch;  // device -> NS_OK or NS_ERR_ARCH

int check_arch() {
  int dev = 0;
  if (int s = check_hip(hipGetDevice(&dev), "hipGetDevice")) return s;
  std::lock_guard<std::mutex> lk(g_arch_mu);
  auto it = g_arch.find(dev);
  if (it == g_arch.end()) {
    hipDeviceProp_t prop;
    if (int s = check_hip(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties")) return s;
    const int ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? NS_OK : NS_ERR_ARCH;
    it = g_arch.emplace(dev, ok).first;
    if (ok != NS_OK) t_err = std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950";
  }
  if (it->second != NS_OK) return fail(NS_ERR_ARCH, "current device is not gfx950");
  return NS_OK;
}

// ------------------------------------------------------------- workspace

struct Ws {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mu;
std::map<std::pair<int, void*>, Ws> g_ws;
// Buffers replaced by a larger one.  Work queued earlier may still read
// them, and another thread may hold the pointer between taking it and
// enqueueing its launches, so they are freed only by ns_release_workspace.
std::vector<std::pair<int, void*>> g_ws_retired;
std::atomic<int64_t> g_ws_allocs{0};

// The workspace of (current device, st), grown to at least `bytes`.  A warm
// workspace is returned without any HIP call, so calls on a stream that has
// seen a call of the same or a larger size enqueue only kernels and copies
// (graph capture needs exactly that).
int get_workspace(hipStream_t st, size_t bytes, char** out) {
  int dev = 0;
  if (int s = check_hip(hipGetDevice(&dev), "hipGetDevice")) return s;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Ws& w = g_ws[{dev, (void*)st}];
  if (w.bytes < bytes) {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return fail(NS_ERR_OOM, "workspace allocation of " + std::to_string(bytes) + " bytes failed");
    }
    ++g_ws_allocs;
    if (w.ptr != nullptr) g_ws_retired.emplace_back(dev, w.ptr);
    w.ptr = p;
    w.bytes = bytes;
  }
  *out = static_cast<char*>(w.ptr);
  return NS_OK;
}

// ---------------------------------------------------------------- timing

struct TimingRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_t_mu;
int g_t_mask = 0;
int g_t_every = 1, g_t_offset = 0;     // launch i of a kind is timed when i % every == offset
int64_t g_t_count[NS_KIND_COUNT] = {};  // launches of each kind since the last reset
std::vector<TimingRec> g_t_recs;
std::vector<hipEvent_t> g_t_pool;

hipEvent_t take_event() {
  if (!g_t_pool.empty()) {
    hipEvent_t e = g_t_pool.back();
    g_t_pool.pop_back();
    return e;
  }
  // Timing-only events: no system-scope fence when recorded.  With the
  // default flags every record writes back and invalidates the caches, which
  // costs the timed kernels time of their own and slows the kernel after
  // them.  Their timestamps are only read after the stream has been
  // synchronised (ns_timing_query).
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

// Set while the allocation-free entry point enqueues: its launches are
// neither timed nor counted (timing may create events).
thread_local bool t_untimed = false;

// The events travel in the kernel's dispatch packet (ns::set_launch_events),
// so timing adds no packets between the kernels of a call.
template <typename F>
hipError_t timed_launch(int kind, hipStream_t st, F&& f) {
  if (t_untimed) return f();
  std::unique_lock<std::mutex> lk(g_t_mu);
  const bool on = ((g_t_mask >> kind) & 1) && g_t_count[kind]++ % g_t_every == g_t_offset;
  hipEvent_t a = nullptr, b = nullptr;
  if (on) {
    a = take_event();
    b = take_event();
  }
  lk.unlock();
  const bool timed = on && a && b;
  if (timed) ns::set_launch_events(a, b);
  hipError_t e = f();
  if (on) {
    ns::set_launch_events(nullptr, nullptr);
    lk.lock();
    if (timed && e == hipSuccess) {
      g_t_recs.push_back(TimingRec{kind, a, b});
    } else {  // nothing recorded them: back to the pool
      if (a) g_t_pool.push_back(a);
      if (b) g_t_pool.push_back(b);
    }
  }
  return e;
}

// ---------------------------------------------------------------- stages

// sums_done: the partials are already there (a padded call's pad pass
// computes them).
int run_normalize(const void* x, void* y, float* norms, const Plan& p, float* partials, hipStream_t st,
                  bool sums_done = false) {
  const NormArgs g = ns::norm_args(p, x, y, norms, partials);
  const int batch = (int)p.batch;
  if (!sums_done)
    if (int s = check_hip(timed_launch(NS_KIND_SUMSQ, st, [&] { return ns::launch_sumsq(p.dtype, g, batch, st); }),
                          "sum-of-squares launch"))
      return s;
  if (y == nullptr) return NS_OK;  // sums of squares only (folded normalisation)
  return check_hip(timed_launch(NS_KIND_SCALE, st, [&] { return ns::launch_scale(p.dtype, g, batch, st); }),
                   "scale launch");
}

int launch_stage(int kind_id, const char* what, const Plan& p, const GemmArgs& g, const ns::StageKind& k,
                 hipStream_t st) {
  return check_hip(timed_launch(kind_id, st, [&] { return ns::launch_gemm(p.dtype, k, g, st); }), what);
}

int run_gram(const void* x, void* oa, float* da, const Plan& p, hipStream_t st, const float* d_norm = nullptr,
             bool mirror = true) {
  ns::StageKind k;
  const GemmArgs g = ns::gram_args(p, x, oa, da, &k, d_norm, mirror);
  return launch_stage(NS_KIND_GRAM, "gram launch", p, g, k, st);
}

int run_poly(const void* oa, const float* da, void* oc, float* dc, const Plan& p, float a, float b,
             float c, hipStream_t st) {
  ns::StageKind k;
  const GemmArgs g = ns::poly_args(p, oa, da, oc, dc, a, b, c, &k);
  return launch_stage(NS_KIND_POLY, "poly launch", p, g, k, st);
}

int run_update(const void* x, const void* oc, const float* dc, void* xo, const Plan& p, hipStream_t st,
               const float* d_norm = nullptr) {
  ns::StageKind k;
  const GemmArgs g = ns::update_args(p, x, oc, dc, xo, &k, d_norm);
  return launch_stage(NS_KIND_UPDATE, "update launch", p, g, k, st);
}

void record_config(const Plan& p, int steps) {
  const ns::TileCfg tg = ns::tile_cfg(p.dtype, true, ns::plan_tri_class(p, true));
  const ns::TileCfg tp = ns::tile_cfg(p.dtype, true, ns::plan_tri_class(p, false));
  const ns::TileCfg tr = ns::tile_cfg(p.dtype, false);
  char buf[768];
  std::snprintf(buf, sizeof(buf),
                "dtype=%s batch=%lld rows=%lld cols=%lld m=%lld %s steps=%d | norm: %s (%lldx16B blocks) | "
                "mfma=%s | gram: lower-tri tile=%dx%d waves=%dx%d k=%dB ring=%d operands=%s | poly: lower-tri "
                "tile=%dx%d waves=%dx%d k=%dB ring=%d | update: %s tile=%dx%d waves=%dx%d k=%dB ring=%d X-operand=%s loads=%s",
                p.dtype == NS_DTYPE_BF16 ? "bf16" : "fp32", (long long)p.batch, (long long)p.rows,
                (long long)p.cols, (long long)p.m, p.tall ? "tall" : "wide", steps,
                ns::fold_normalisation(steps) ? "sumsq, 1/||x|| folded into step 1" : "sumsq+scale",
                ns::kNormChunkVecs, p.dtype == NS_DTYPE_BF16 ? "32x32x16_bf16" : "32x32x2_f32", tg.bm, tg.bn, tg.wm,
                tg.wn, tg.cpr * 16, tg.st, p.tall ? "columns(transposed-read)" : "rows", tp.bm, tp.bn, tp.wm, tp.wn,
                tp.cpr * 16, tp.st, p.tall ? "X*C" : "C*X", tr.bm, tr.bn, tr.wm, tr.wn, tr.cpr * 16, tr.st,
                p.tall ? "rows" : "columns(transposed-read)",
                ns::late_issue(p.dtype, (long long)ns::tiles_of(p.rows, tr.bm) * ns::tiles_of(p.cols, tr.bn) * p.batch,
                               (int)p.m)
                    ? "after-k-steps-0-1"
                    : (p.dtype == NS_DTYPE_BF16 && ns::update_k_stages((int)p.m) >= ns::kStaggerMinStages
                           ? "staggered"
                           : "stage-start"));
  t_cfg = buf;
  if (p.padded)
    t_cfg += " | zero-padded from " + std::to_string(p.urows) + "x" + std::to_string(p.ucols) + " to " +
             std::to_string(p.rows) + "x" + std::to_string(p.cols);
}

int common_checks(int64_t batch, int64_t rows, int64_t cols, int dtype, bool any_dims = false) {
  if (int s = check_dtype(dtype)) return s;
  return check_shape(batch, rows, cols, any_dims);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

// ------------------------------------------------------- grouped calls

// One stack of a grouped call: its plan, its part of the shared workspace
// and its buffers (in / out are the zero-padded workspace copies when the
// plan is padded).
struct Group {
  Plan p;
  size_t ws_off;
  const void* uin;
  void* uout;
  const void* in;
  void* out;
  bool copy_in;
  void *xtmp, *oa, *oc;
  float *da, *dc, *part;
};

// Plans of the non-empty stacks and the workspace they need together.
size_t plan_groups(int n, const int64_t* batch, const int64_t* rows, const int64_t* cols, int dtype,
                   std::vector<Group>* gs) {
  size_t off = 0;
  for (int i = 0; i < n; ++i) {
    if (batch[i] == 0) continue;
    Group g{};
    g.p = make_plan(batch[i], rows[i], cols[i], dtype);
    g.ws_off = off;
    off += ns::ws_align(g.p.total);
    if (gs) gs->push_back(g);
  }
  return off;
}

int check_grouped(int n, const void* const* in, void* const* out, const int64_t* batch, const int64_t* rows,
                  const int64_t* cols, int dtype) {
  if (n < 0 || n > NS_MAX_GROUPS)
    return fail(NS_ERR_INVALID_ARG, "n_groups must be in [0, " + std::to_string(NS_MAX_GROUPS) + "]");
  if (n == 0) return NS_OK;
  if (!batch || !rows || !cols) return fail(NS_ERR_INVALID_ARG, "batch, rows and cols arrays must not be NULL");
  if (int s = check_dtype(dtype)) return s;
  for (int i = 0; i < n; ++i)
    if (int s = check_shape(batch[i], rows[i], cols[i], true))
      return fail(s, "stack " + std::to_string(i) + ": " + t_err);
  if (in == nullptr && out == nullptr) return NS_OK;  // sizes only (workspace query)
  if (!in || !out) return fail(NS_ERR_INVALID_ARG, "in and out arrays must not be NULL");
  std::vector<size_t> bytes(n, 0);
  for (int i = 0; i < n; ++i) {
    if (batch[i] == 0) continue;  // skipped stack: its pointers are never used
    const std::string who = "stack " + std::to_string(i) + ": ";
    if (int s = check_ptr(in[i], "in")) return fail(s, who + t_err);
    if (int s = check_ptr(out[i], "out")) return fail(s, who + t_err);
    bytes[i] = (size_t)batch[i] * rows[i] * cols[i] * esize(dtype);
    if (in[i] != out[i] && overlaps(in[i], bytes[i], out[i], bytes[i]))
      return fail(NS_ERR_INVALID_ARG, who + "out overlaps in without being the same pointer");
  }
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      if (i == j || bytes[i] == 0 || bytes[j] == 0) continue;
      if (overlaps(out[i], bytes[i], in[j], bytes[j]) || (i < j && overlaps(out[i], bytes[i], out[j], bytes[j])))
        return fail(NS_ERR_INVALID_ARG,
                    "out of stack " + std::to_string(i) + " overlaps the buffers of stack " + std::to_string(j));
    }
  return NS_OK;
}

// The method on the non-empty stacks gs (plans, workspace offsets and the
// caller's pointers set), sharing each stage's launches among them: per step
// one Gram launch per orientation (wide stacks read rows of X, tall ones
// columns), one poly launch over all and one update per orientation.  Odd
// shapes run on zero-padded copies (see ns_plan.h); an in-place call with an
// odd step count starts from a copy of the input.  With no step each stack
// is normalised on its own (sum of squares, then scale).  *tc and launches
// (Gram, poly, update launches of one step) describe what ran.
std::atomic<int> g_poison{0};  // ns_set_workspace_poison

//
// The workspace is the library's cache for (device, st), or `given` (at
// least ws_bytes) when that is not null.
int run_stacks(std::vector<Group>& gs, size_t ws_bytes, int ns_steps, float a, float b, float c, hipStream_t st,
               ns::TileChoice* tc, int launches[3], char* given = nullptr) {
  const int dtype = gs[0].p.dtype;
  char* ws = given;
  if (ws == nullptr)
    if (int s = get_workspace(st, ws_bytes, &ws)) return s;
  if (g_poison.load() && ws_bytes > 0)
    if (int s = check_hip(hipMemsetAsync(ws, 0xFF, ws_bytes, st), "workspace poison fill")) return s;
  std::vector<Plan> plans;
  for (Group& g : gs) {
    char* w = ws + g.ws_off;
    g.in = g.uin;
    g.out = g.uout;
    g.xtmp = w + g.p.off_xtmp;
    g.oa = w + g.p.off_oa;
    g.oc = w + g.p.off_oc;
    g.da = reinterpret_cast<float*>(w + g.p.off_da);
    g.dc = reinterpret_cast<float*>(w + g.p.off_dc);
    g.part = reinterpret_cast<float*>(w + g.p.off_part);
    plans.push_back(g.p);
  }
  const int n = (int)gs.size();
  *tc = ns::choose_tiles(plans.data(), n);
  launches[0] = launches[1] = launches[2] = 0;

  for (Group& g : gs) {
    if (g.p.padded) {  // the padded copy and its sums of squares in one pass
      g.in = ws + g.ws_off + g.p.off_pin;
      g.out = ws + g.ws_off + g.p.off_pout;
      const ns::PadArgs pa = ns::pad_args(g.p, g.uin, const_cast<void*>(g.in), true);
      const NormArgs na = ns::norm_args(g.p, g.in, nullptr, nullptr, g.part);
      if (int s = check_hip(timed_launch(NS_KIND_SUMSQ, st,
                                         [&] { return ns::launch_pad_sumsq(dtype, pa, na, (int)g.p.batch, st); }),
                            "pad launch"))
        return s;
    }
    g.copy_in = ns::input_copy_needed(ns_steps, g.in == g.out);
  }
  if (ns_steps == 0) {  // X0 = x / (||x||_F + eps), in place if out == in
    for (const Group& g : gs)
      if (int s = run_normalize(g.in, g.out, nullptr, g.p, g.part, st, g.p.padded)) return s;
  } else {
    // one sum-of-squares launch over every stack not padded (the pad pass
    // did those); 1/||x|| rides in step 1
    std::vector<NormArgs> na;
    std::vector<int> nb;
    for (const Group& g : gs) {
      if (g.p.padded) continue;
      na.push_back(ns::norm_args(g.p, g.in, nullptr, nullptr, g.part));
      nb.push_back((int)g.p.batch);
    }
    if (!na.empty())
      if (int s = check_hip(timed_launch(NS_KIND_SUMSQ, st,
                                         [&] {
                                           return ns::launch_sumsq_grouped(dtype, na.data(), nb.data(),
                                                                           (int)na.size(), st);
                                         }),
                            "sum-of-squares launch"))
        return s;
    for (const Group& g : gs)
      if (g.copy_in) {
        const size_t pb = (size_t)g.p.batch * g.p.rows * g.p.cols * esize(dtype);
        if (int s = check_hip(hipMemcpyAsync(g.xtmp, g.in, pb, hipMemcpyDeviceToDevice, st), "input copy")) return s;
      }
  }
  auto buf = [&](const Group& g, int s) -> const void* {
    if (s == 0) return g.copy_in ? g.xtmp : g.in;
    return ns::iterate_in_out(ns_steps, s) ? g.out : g.xtmp;
  };
  auto wbuf = [&](const Group& g, int s) -> void* { return ns::iterate_in_out(ns_steps, s) ? g.out : g.xtmp; };
  auto launch = [&](int kind, const char* what, const ns::StageKind& k, const std::vector<GemmArgs>& ga) {
    return check_hip(
        timed_launch(kind, st, [&] { return ns::launch_gemm_grouped(dtype, k, ga.data(), (int)ga.size(), st); }),
        what);
  };
  for (int s = 1; s <= ns_steps; ++s) {
    const bool first = s == 1;  // the Gram and the update of step 1 see the raw input
    for (int o = 0; o < 2; ++o) {  // Gram: wide stacks, then tall ones
      std::vector<GemmArgs> ga;
      ns::StageKind k{};
      for (const Group& g : gs)
        if (g.p.tall == (o == 1))
          ga.push_back(ns::gram_args(g.p, *tc, buf(g, s - 1), g.oa, g.da, &k, first ? g.part : nullptr,
                                     !tc->lower_only));
      if (ga.empty()) continue;
      launches[0] += first;
      if (int e = launch(NS_KIND_GRAM, "gram launch", k, ga)) return e;
    }
    {
      std::vector<GemmArgs> ga;
      ns::StageKind k{};
      for (const Group& g : gs) ga.push_back(ns::poly_args(g.p, *tc, g.oa, g.da, g.oc, g.dc, a, b, c, &k));
      launches[1] += first;
      if (int e = launch(NS_KIND_POLY, "poly launch", k, ga)) return e;
    }
    for (int o = 0; o < 2; ++o) {  // update: wide stacks, then tall ones
      std::vector<GemmArgs> ga;
      ns::StageKind k{};
      for (const Group& g : gs)
        if (g.p.tall == (o == 1))
          ga.push_back(ns::update_args(g.p, buf(g, s - 1), g.oc, g.dc, wbuf(g, s), &k, first ? g.part : nullptr));
      if (ga.empty()) continue;
      launches[2] += first;
      if (int e = launch(NS_KIND_UPDATE, "update launch", k, ga)) return e;
    }
  }
  for (const Group& g : gs)
    if (g.p.padded) {
      const ns::PadArgs pa = ns::pad_args(g.p, g.out, g.uout, false);
      if (int s = check_hip(ns::launch_unpad(dtype, pa, st), "unpad launch")) return s;
    }
  return NS_OK;
}

void record_config_grouped(const std::vector<Group>& gs, const ns::TileChoice& tc, int steps, int launches[3]) {
  const int dtype = gs[0].p.dtype;
  int nt = 0;
  for (const Group& g : gs) nt += g.p.tall;
  const ns::TileCfg tw = ns::tile_cfg(dtype, true, tc.gram_wide), tt = ns::tile_cfg(dtype, true, tc.gram_tall);
  const ns::TileCfg tp = ns::tile_cfg(dtype, true, tc.poly), tr = ns::tile_cfg(dtype, false);
  char buf[512];
  std::snprintf(buf, sizeof(buf),
                "grouped: %d stacks (%d wide, %d tall) dtype=%s steps=%d | norm: sumsq, one launch, 1/||x|| folded "
                "into step 1 | launches per step: gram %d, poly %d, update %d | gram wide: lower-tri tile=%dx%d | "
                "gram tall: lower-tri tile=%dx%d | poly: lower-tri tile=%dx%d%s | update: tile=%dx%d",
                (int)gs.size(), (int)gs.size() - nt, nt, dtype == NS_DTYPE_BF16 ? "bf16" : "fp32", steps,
                launches[0], launches[1], launches[2], tw.bm, tw.bn, tt.bm, tt.bn, tp.bm, tp.bn,
                tc.lower_only ? " (A read as its lower block triangle)" : "", tr.bm, tr.bn);
  t_cfg = buf;
  t_cfg += " | stacks:";
  for (size_t i = 0; i < gs.size() && i < 64; ++i) {
    const Plan& p = gs[i].p;
    t_cfg += " " + std::to_string(p.batch) + "x" + std::to_string(p.urows) + "x" + std::to_string(p.ucols);
  }
  if (gs.size() > 64) t_cfg += " ...";
}

}  // namespace

// =================================================================== C ABI

extern "C" {

int ns_orthogonalize(const void* in, void* out, int64_t batch, int64_t rows, int64_t cols, int dtype,
                     int ns_steps, float a, float b, float c, void* stream) {
  t_err.clear();
  if (int s = common_checks(batch, rows, cols, dtype, true)) return s;
  if (ns_steps < 0) return fail(NS_ERR_INVALID_ARG, "ns_steps must be >= 0");
  if (int s = check_ptr(in, "in")) return s;
  if (int s = check_ptr(out, "out")) return s;
  const size_t bytes = (size_t)batch * rows * cols * esize(dtype);
  if (in != out && overlaps(in, bytes, out, bytes))
    return fail(NS_ERR_INVALID_ARG, "out overlaps in without being the same pointer");
  if (batch == 0) return NS_OK;
  if (int s = check_arch()) return s;

  std::vector<Group> gs(1);
  gs[0].p = make_plan(batch, rows, cols, dtype);
  gs[0].ws_off = 0;
  gs[0].uin = in;
  gs[0].uout = out;
  ns::TileChoice tc;
  int launches[3];
  if (int s = run_stacks(gs, gs[0].p.total, ns_steps, a, b, c, static_cast<hipStream_t>(stream), &tc, launches))
    return s;
  const Plan& p = gs[0].p;
  record_config(p, ns_steps);
  return NS_OK;
}

int ns_orthogonalize_noalloc(const void* in, void* out, int64_t batch, int64_t rows, int64_t cols, int dtype,
                             int ns_steps, float a, float b, float c, void* stream) {
  t_err.clear();
  if (int s = common_checks(batch, rows, cols, dtype, true)) return s;
  if (ns_steps < 0) return fail(NS_ERR_INVALID_ARG, "ns_steps must be >= 0");
  if (int s = check_ptr(in, "in")) return s;
  if (int s = check_ptr(out, "out")) return s;
  const size_t bytes = (size_t)batch * rows * cols * esize(dtype);
  if (in != out && overlaps(in, bytes, out, bytes))
    return fail(NS_ERR_INVALID_ARG, "out overlaps in without being the same pointer");
  if (batch == 0) return NS_OK;
  std::vector<Group> gs(1);
  gs[0].p = make_plan(batch, rows, cols, dtype);
  if (gs[0].p.total > NS_NOALLOC_SCRATCH_BYTES)
    return fail(NS_ERR_SCRATCH, "this call needs " + std::to_string(gs[0].p.total) +
                                    " bytes of workspace, more than the fixed scratch of " +
                                    std::to_string(NS_NOALLOC_SCRATCH_BYTES) + " bytes");
  if (int s = check_arch()) return s;
  int dev = 0;
  if (int s = check_hip(hipGetDevice(&dev), "hipGetDevice")) return s;
  char* ws = nullptr;
  if (int s = check_hip(ns::noalloc_scratch(dev, &ws), "scratch address (hipGetSymbolAddress)")) return s;
  gs[0].ws_off = 0;
  gs[0].uin = in;
  gs[0].uout = out;
  ns::TileChoice tc;
  int launches[3];
  t_untimed = true;
  const int s = run_stacks(gs, gs[0].p.total, ns_steps, a, b, c, static_cast<hipStream_t>(stream), &tc, launches, ws);
  t_untimed = false;
  if (s) return s;
  record_config(gs[0].p, ns_steps);
  t_cfg += " | workspace: fixed scratch";
  return NS_OK;
}

int ns_orthogonalize_grouped(int n_groups, const void* const* in, void* const* out, const int64_t* batch,
                             const int64_t* rows, const int64_t* cols, int dtype, int ns_steps, float a, float b,
                             float c, void* stream) {
  t_err.clear();
  if (in == nullptr || out == nullptr) {
    if (n_groups > 0) return fail(NS_ERR_INVALID_ARG, "in and out arrays must not be NULL");
  }
  if (int s = check_grouped(n_groups, in, out, batch, rows, cols, dtype)) return s;
  if (ns_steps < 0) return fail(NS_ERR_INVALID_ARG, "ns_steps must be >= 0");
  std::vector<Group> gs;
  const size_t total = plan_groups(n_groups, batch, rows, cols, dtype, &gs);
  if (gs.empty()) return NS_OK;
  if (int s = check_arch()) return s;
  for (int i = 0, k = 0; i < n_groups; ++i) {
    if (batch[i] == 0) continue;
    gs[k].uin = in[i];
    gs[k].uout = out[i];
    ++k;
  }
  ns::TileChoice tc;
  int launches[3];
  if (int s = run_stacks(gs, total, ns_steps, a, b, c, static_cast<hipStream_t>(stream), &tc, launches)) return s;
  record_config_grouped(gs, tc, ns_steps, launches);
  return NS_OK;
}

size_t ns_workspace_bytes_grouped(int n_groups, const int64_t* batch, const int64_t* rows, const int64_t* cols,
                                  int dtype) {
  if (check_grouped(n_groups, nullptr, nullptr, batch, rows, cols, dtype) != NS_OK) return 0;
  if (n_groups == 0) return 0;
  return plan_groups(n_groups, batch, rows, cols, dtype, nullptr);
}

size_t ns_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int dtype) {
  if (check_dtype(dtype) != NS_OK || check_shape(batch, rows, cols, true) != NS_OK) return 0;
  return make_plan(batch, rows, cols, dtype).total;
}

int ns_release_workspace(void) {
  t_err.clear();
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int status = NS_OK;
  int cur = 0;
  (void)hipGetDevice(&cur);
  std::vector<std::pair<int, void*>> bufs = g_ws_retired;
  for (auto& kv : g_ws)
    if (kv.second.ptr != nullptr) bufs.emplace_back(kv.first.first, kv.second.ptr);
  std::map<int, bool> synced;
  for (auto& db : bufs) {
    if (hipSetDevice(db.first) != hipSuccess) {
      status = fail(NS_ERR_HIP, "hipSetDevice failed");
      continue;
    }
    if (!synced[db.first]) {
      (void)hipDeviceSynchronize();
      synced[db.first] = true;
    }
    if (hipFree(db.second) != hipSuccess) status = fail(NS_ERR_HIP, "hipFree failed");
  }
  g_ws.clear();
  g_ws_retired.clear();
  (void)hipSetDevice(cur);
  return status;
}

int64_t ns_workspace_allocations(void) { return g_ws_allocs.load(); }

const char* ns_status_string(int status) {
  switch (status) {
    case NS_OK: return "NS_OK";
    case NS_ERR_INVALID_ARG: return "NS_ERR_INVALID_ARG: invalid argument";
    case NS_ERR_DTYPE: return "NS_ERR_DTYPE: unsupported dtype";
    case NS_ERR_ALIGNMENT: return "NS_ERR_ALIGNMENT: pointers must be 16-byte aligned (stage exports: dims multiples of 8)";
    case NS_ERR_ARCH: return "NS_ERR_ARCH: device is not gfx950";
    case NS_ERR_OOM: return "NS_ERR_OOM: workspace allocation failed";
    case NS_ERR_HIP: return "NS_ERR_HIP: HIP runtime error";
    case NS_ERR_SCRATCH: return "NS_ERR_SCRATCH: the call needs more than the fixed no-alloc scratch";
    default: return "unknown status";
  }
}

const char* ns_last_error(void) { return t_err.c_str(); }

int ns_query_last_config(char* buf, size_t n) {
  if (buf != nullptr && n > 0) {
    std::strncpy(buf, t_cfg.c_str(), n - 1);
    buf[n - 1] = '\0';
  }
  return (int)t_cfg.size();
}

int ns_timing_enable(int mask) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  g_t_mask = mask;
  return NS_OK;
}

int ns_timing_sample(int every, int offset) {
  t_err.clear();
  if (every < 1 || offset < 0 || offset >= every)
    return fail(NS_ERR_INVALID_ARG, "timing sample needs every >= 1 and 0 <= offset < every");
  std::lock_guard<std::mutex> lk(g_t_mu);
  g_t_every = every;
  g_t_offset = offset;
  return NS_OK;
}

int ns_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_t_mu);
  for (auto& c : g_t_count) c = 0;
  for (auto& r : g_t_recs) {
    g_t_pool.push_back(r.a);
    g_t_pool.push_back(r.b);
  }
  g_t_recs.clear();
  return NS_OK;
}

int ns_timing_query(int kind, double* total_ms, int64_t* launches) {
  t_err.clear();
  if (kind < 0 || kind >= NS_KIND_COUNT || total_ms == nullptr || launches == nullptr)
    return fail(NS_ERR_INVALID_ARG, "bad timing query");
  std::lock_guard<std::mutex> lk(g_t_mu);
  double sum = 0.0;
  int64_t count = 0;
  for (auto& r : g_t_recs) {
    if (r.kind != kind) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(NS_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(NS_ERR_HIP, "hipEventElapsedTime failed");
    sum += ms;
    ++count;
  }
  *total_ms = sum;
  *launches = count;
  return NS_OK;
}

int ns_stage_normalize(const void* x, void* x0, float* norms, int64_t batch, int64_t rows, int64_t cols,
                       int dtype, void* stream) {
  t_err.clear();
  if (int s = common_checks(batch, rows, cols, dtype)) return s;
  if (int s = check_ptr(x, "x")) return s;
  if (int s = check_ptr(x0, "x0")) return s;
  const size_t bytes = (size_t)batch * rows * cols * esize(dtype);
  if (x != x0 && overlaps(x, bytes, x0, bytes)) return fail(NS_ERR_INVALID_ARG, "x0 overlaps x");
  if (batch == 0) return NS_OK;
  if (int s = check_arch()) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Plan p = make_plan(batch, rows, cols, dtype);
  char* ws = nullptr;
  if (int s = get_workspace(st, p.total, &ws)) return s;
  return run_normalize(x, x0, norms, p, reinterpret_cast<float*>(ws + p.off_part), st);
}

int ns_stage_gram(const void* x, void* a_off, float* a_diag, int64_t batch, int64_t rows, int64_t cols,
                  int dtype, void* stream) {
  t_err.clear();
  if (int s = common_checks(batch, rows, cols, dtype)) return s;
  if (int s = check_ptr(x, "x")) return s;
  if (int s = check_ptr(a_off, "a_off")) return s;
  if (int s = check_ptr(a_diag, "a_diag")) return s;
  if (batch == 0) return NS_OK;
  if (int s = check_arch()) return s;
  const Plan p = make_plan(batch, rows, cols, dtype);
  return run_gram(x, a_off, a_diag, p, static_cast<hipStream_t>(stream));
}

int ns_stage_poly(const void* a_off, const float* a_diag, void* c_off, float* c_diag, int64_t batch, int64_t m,
                  int dtype, float a, float b, float c, void* stream) {
  t_err.clear();
  if (int s = common_checks(batch, m, m, dtype)) return s;
  if (int s = check_ptr(a_off, "a_off")) return s;
  if (int s = check_ptr(a_diag, "a_diag")) return s;
  if (int s = check_ptr(c_off, "c_off")) return s;
  if (int s = check_ptr(c_diag, "c_diag")) return s;
  const size_t bytes = (size_t)batch * m * m * esize(dtype);
  if (overlaps(a_off, bytes, c_off, bytes)) return fail(NS_ERR_INVALID_ARG, "c_off overlaps a_off");
  if (batch == 0) return NS_OK;
  if (int s = check_arch()) return s;
  const Plan p = make_plan(batch, m, m, dtype);
  return run_poly(a_off, a_diag, c_off, c_diag, p, a, b, c, static_cast<hipStream_t>(stream));
}

int ns_stage_update(const void* x, const void* c_off, const float* c_diag, void* x_out, int64_t batch,
                    int64_t rows, int64_t cols, int dtype, void* stream) {
  t_err.clear();
  if (int s = common_checks(batch, rows, cols, dtype)) return s;
  if (int s = check_ptr(x, "x")) return s;
  if (int s = check_ptr(c_off, "c_off")) return s;
  if (int s = check_ptr(c_diag, "c_diag")) return s;
  if (int s = check_ptr(x_out, "x_out")) return s;
  const size_t bytes = (size_t)batch * rows * cols * esize(dtype);
  if (overlaps(x, bytes, x_out, bytes)) return fail(NS_ERR_INVALID_ARG, "x_out overlaps x");
  if (batch == 0) return NS_OK;
  if (int s = check_arch()) return s;
  const Plan p = make_plan(batch, rows, cols, dtype);
  return run_update(x, c_off, c_diag, x_out, p, static_cast<hipStream_t>(stream));
}

int ns_set_workspace_poison(int on) {
  g_poison.store(on != 0);
  return NS_OK;
}

int ns_peak_mfma(int dtype, int64_t iters, double* tflops, double* clock_mhz, void* stream) {
  t_err.clear();
  if (int s = check_dtype(dtype)) return s;
  if (tflops == nullptr || clock_mhz == nullptr) return fail(NS_ERR_INVALID_ARG, "tflops and clock_mhz must be non-NULL");
  if (iters < 4 || iters > (int64_t(1) << 30) || iters % 4 != 0)
    return fail(NS_ERR_INVALID_ARG, "iters must be a multiple of 4 in [4, 2^30]");
  if (int s = check_arch()) return s;
  int dev = 0, cus = 0, wall_khz = 0;
  if (int s = check_hip(hipGetDevice(&dev), "hipGetDevice")) return s;
  if (int s = check_hip(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count")) return s;
  if (int s = check_hip(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev), "wall clock rate"))
    return s;
  // two workgroups of four waves per CU: two waves on each SIMD
  const int blocks = 2 * cus;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* sink = nullptr;
  unsigned long long* clocks = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int status = NS_OK;
  auto cleanup = [&]() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (sink) (void)hipFree(sink);
    if (clocks) (void)hipFree(clocks);
  };
  if ((status = check_hip(hipMalloc(&sink, sizeof(float) * blocks * ns::kPeakThreads), "hipMalloc")) ||
      (status = check_hip(hipMalloc(&clocks, sizeof(unsigned long long) * 4 * blocks), "hipMalloc")) ||
      (status = check_hip(hipEventCreate(&e0), "hipEventCreate")) ||
      (status = check_hip(hipEventCreate(&e1), "hipEventCreate")) ||
      (status = check_hip(hipEventRecord(e0, st), "hipEventRecord")) ||
      (status = check_hip(ns::launch_mfma_peak(dtype, blocks, (int)iters, sink, clocks, st), "peak launch")) ||
      (status = check_hip(hipEventRecord(e1, st), "hipEventRecord")) ||
      (status = check_hip(hipEventSynchronize(e1), "hipEventSynchronize"))) {
    cleanup();
    return status;
  }
  float ms = 0.0f;
  std::vector<unsigned long long> c(4 * (size_t)blocks);
  if ((status = check_hip(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime")) ||
      (status = check_hip(hipMemcpy(c.data(), clocks, c.size() * sizeof(c[0]), hipMemcpyDeviceToHost), "hipMemcpy"))) {
    cleanup();
    return status;
  }
  cleanup();
  const double waves = (double)blocks * ns::kPeakThreads / 64.0;
  const double flops = waves * (double)iters * ns::mfma_peak_acc() * (double)ns::mfma_peak_flops_per_inst(dtype);
  *tflops = ms > 0.0f ? flops / (ms * 1e-3) / 1e12 : 0.0;
  // average over workgroups of (shader cycles / wall ticks) x wall rate
  double ratio = 0.0;
  int n = 0;
  for (int b = 0; b < blocks; ++b) {
    const unsigned long long dt = c[4 * b + 1] - c[4 * b], dr = c[4 * b + 3] - c[4 * b + 2];
    if (dr > 0) {
      ratio += (double)dt / (double)dr;
      ++n;
    }
  }
  *clock_mhz = n ? ratio / n * wall_khz / 1000.0 : 0.0;
  return NS_OK;
}

}  // extern "C"

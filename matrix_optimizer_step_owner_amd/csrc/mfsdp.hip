// Host side of the owner-local optimizer step: argument validation, the
// grouped launch plan, and the C ABI declared in include/mfsdp.h.
//
// Source of the operations: "MatrixFSDP: communication-free matrix optimizers
// under ZeRO-3 parameter sharding" (arxivlens page, Abstract): the owner of a
// whole 2D weight runs Muon's Newton-Schulz on it locally, and the tensors
// that are not 2D matrices, gathered in packed form on tail owners, take
// AdamW.  One call covers the owner's whole list: every kernel is one grouped
// launch over all owned matrices.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/mfsdp.h"
#include "common.hpp"
#include "ew_kernels.hpp"
#include "ns_gemm.hpp"
#include "ns_small.hpp"
#include "planner.hpp"
#include "probe_kernels.hpp"
#include "stats_kernels.hpp"
#include "tail_kernels.hpp"

namespace {

using namespace mfsdp;

thread_local std::string g_last_error;

mfsdp_status_t fail(mfsdp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr size_t kWsAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

bool finite(float x) { return std::isfinite(x); }

size_t elem_size(mfsdp_dtype_t dt) { return dt == MFSDP_DTYPE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// Kernel timing (measurement only).
// ---------------------------------------------------------------------------
struct TimingRec {
  int kind;
  hipEvent_t start, stop;
};

struct TimingState {
  bool enabled = false;
  std::vector<hipEvent_t> free_events;
  std::vector<TimingRec> pending;
  double total_ms[MFSDP_KERNEL_KINDS] = {};
  int64_t count[MFSDP_KERNEL_KINDS] = {};
};

thread_local TimingState g_timing;

hipError_t take_event(hipEvent_t* ev) {
  if (!g_timing.free_events.empty()) {
    *ev = g_timing.free_events.back();
    g_timing.free_events.pop_back();
    return hipSuccess;
  }
  return hipEventCreate(ev);
}

hipError_t drain_timing() {
  for (const TimingRec& r : g_timing.pending) {
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return e;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return e;
    g_timing.total_ms[r.kind] += ms;
    g_timing.count[r.kind] += 1;
    g_timing.free_events.push_back(r.start);
    g_timing.free_events.push_back(r.stop);
  }
  g_timing.pending.clear();
  return hipSuccess;
}

// Launch helper: records the optional timing events and checks the launch.
template <class F>
hipError_t launch(int kind, hipStream_t stream, F&& f) {
  hipEvent_t a = nullptr, b = nullptr;
  // events taken but not recorded as a pair go back to the free list
  auto give_back = [&] {
    if (a) g_timing.free_events.push_back(a);
    if (b) g_timing.free_events.push_back(b);
  };
  if (g_timing.enabled) {
    hipError_t e = take_event(&a);
    if (e == hipSuccess) e = take_event(&b);
    if (e == hipSuccess) e = hipEventRecord(a, stream);
    if (e != hipSuccess) {
      give_back();
      return e;
    }
  }
  f();
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && g_timing.enabled) e = hipEventRecord(b, stream);
  if (e != hipSuccess) {
    give_back();
    return e;
  }
  if (g_timing.enabled) g_timing.pending.push_back({kind, a, b});
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Plan of one mfsdp_muon_step call.
// ---------------------------------------------------------------------------
struct MatGeom {
  int64_t rows, cols, m, n, m_pad, n_pad;
  bool tall;
  bool small;   // whole Newton-Schulz chain in one workgroup (ns_small.hpp)
  int64_t ew_tiles_j, ew_ntiles, ew_th, ew_tw;
};

struct Plan {
  std::vector<MatGeom> geom;
  size_t off_descs = 0, off_lists = 0, off_tiles = 0, off_scales = 0, off_partials = 0;
  size_t off_small = 0;             // int32 indices of the small matrices
  std::vector<int64_t> small;
  size_t blob_bytes = 0;            // descriptors + work lists (host upload)
  std::vector<size_t> off_x0, off_x1, off_a, off_b;
  size_t total = 0;
  int64_t ew_total = 0, gram_total = 0, upd_total = 0;
  int64_t ew_wg_total = 0;          // momentum workgroups (kEwSub blocks each)
  // Newton-Schulz groups: matrices split into flop-balanced groups whose
  // iterations run on separate streams (see enqueue_muon).  Per group: its
  // matrices and the offsets/counts of its tile tables (in int2 entries from
  // off_tiles): symmetric (Gram and polynomial), update, final-wide,
  // final-tall.
  struct Group {
    std::vector<int64_t> mats;
    int64_t sym = 0, upd = 0, fin_wide = 0, fin_tall = 0;
    int64_t t_sym = 0, t_upd = 0, t_fin_wide = 0, t_fin_tall = 0;
  };
  std::vector<Group> groups;
};

// Tile table of one launch over matrices `mats`: by decreasing k_of (stable),
// tiles_of(i) tiles per matrix, balanced over the XCDs.
template <class KOf, class TilesOf>
void launch_order(std::vector<int64_t> mats, KOf k_of, TilesOf tiles_of, int2* out) {
  std::stable_sort(mats.begin(), mats.end(),
                   [&](int64_t x, int64_t y) { return k_of(x) > k_of(y); });
  std::vector<int2> seq;
  std::vector<int64_t> cost;
  for (int64_t i : mats) {
    const int64_t nt = tiles_of(i);
    for (int64_t q = 0; q < nt; ++q) {
      seq.push_back(make_int2(static_cast<int>(i), static_cast<int>(q)));
      cost.push_back(k_of(i));
    }
  }
  xcd_balance(seq, cost, kXcds, out);
}

// Work-group count that one launch needs to fill the MI355X (256 CUs).
constexpr int64_t kCus = 256;
constexpr int kMaxGroups = 4;

// Number of Newton-Schulz groups for a call: one when a single grouped launch
// already has many rounds of tiles, more when few rounds would leave CUs idle
// at the end of each launch.  MFSDP_NS_GROUPS overrides it (debugging).
int choose_groups(int64_t n, int64_t upd_total, int max_groups) {
  int g;
  const int64_t rounds = upd_total / kCus;
  if (upd_total < kCus / 4) g = 1;          // latency-bound; not worth streams
  else if (rounds >= 6) g = 1;
  else g = 2;
  if (const char* env = getenv("MFSDP_NS_GROUPS")) {
    const int v = atoi(env);
    if (v >= 1 && v <= kMaxGroups) g = v;
  }
  return static_cast<int>(std::min<int64_t>(std::min(g, max_groups), n));
}

mfsdp_status_t make_geom(const mfsdp_matrix_t& mt, int64_t idx, MatGeom* g, size_t es) {
  if (mt.rows < 1 || mt.cols < 1)
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: rows=%lld cols=%lld must be >= 1",
                (long long)idx, (long long)mt.rows, (long long)mt.cols);
  g->rows = mt.rows;
  g->cols = mt.cols;
  g->tall = mt.rows > mt.cols;
  g->m = std::min(mt.rows, mt.cols);
  g->n = std::max(mt.rows, mt.cols);
  g->m_pad = round_up(g->m, kTile);
  g->n_pad = round_up(g->n, kTile);
  g->small = small_path(g->m, g->n);
  // Kernels address an iterate with 32-bit byte offsets from its base.
  if (g->n_pad > (int64_t(1) << 24) || g->m_pad * g->n_pad >= (int64_t(1) << 31) ||
      g->m_pad * g->n_pad * static_cast<int64_t>(es) >= (int64_t(1) << 32))
    return fail(MFSDP_ERR_UNSUPPORTED,
                "matrix %lld: %lld x %lld exceeds the iterate size limit (2^31 elements, "
                "2^32 bytes)",
                (long long)idx, (long long)mt.rows, (long long)mt.cols);
  // momentum blocks: kEwRows x kEwCols in the stored layout
  g->ew_th = g->tall ? kEwCols : kEwRows;
  g->ew_tw = g->tall ? kEwRows : kEwCols;
  g->ew_tiles_j = g->n_pad / g->ew_tw;
  g->ew_ntiles = (g->m_pad / g->ew_th) * g->ew_tiles_j;
  return MFSDP_OK;
}

mfsdp_status_t build_plan(const mfsdp_matrix_t* mats, int64_t n, mfsdp_dtype_t dt, Plan* p,
                          int max_groups = kMaxGroups) {
  const size_t es = elem_size(dt);
  p->geom.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    mfsdp_status_t st = make_geom(mats[i], i, &p->geom[i], es);
    if (st != MFSDP_OK) return st;
    p->ew_total += p->geom[i].ew_ntiles;
    p->ew_wg_total += (p->geom[i].ew_ntiles + kEwSub - 1) / kEwSub;
    if (p->geom[i].small) {
      p->small.push_back(i);
      continue;
    }
    const int64_t tm = p->geom[i].m_pad / kTile, tn = p->geom[i].n_pad / kTile;
    p->gram_total += tm * (tm + 1) / 2;
    p->upd_total += tm * tn;
  }
  // flop-balanced groups of the tiled matrices (largest first onto the least
  // loaded group); small matrices are outside the groups
  {
    std::vector<int64_t> order, work(n, 0);
    for (int64_t i = 0; i < n; ++i) {
      const MatGeom& g = p->geom[i];
      if (g.small) continue;
      const int64_t tm = g.m_pad / kTile, tn = g.n_pad / kTile;
      work[i] = tm * (tm + 1) / 2 * (g.n_pad + g.m_pad) + tm * tn * g.m_pad;
      order.push_back(i);
    }
    const int ng = order.empty()
                       ? 0
                       : choose_groups(static_cast<int64_t>(order.size()), p->upd_total,
                                       max_groups);
    p->groups.assign(ng, Plan::Group{});
    std::vector<int64_t> load(ng, 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int64_t a, int64_t b) { return work[a] > work[b]; });
    for (int64_t i : order) {
      const int gi = static_cast<int>(std::min_element(load.begin(), load.end()) - load.begin());
      load[gi] += work[i];
      p->groups[gi].mats.push_back(i);
    }
    int64_t off_t = 0;
    for (Plan::Group& gr : p->groups) {
      std::sort(gr.mats.begin(), gr.mats.end());
      for (int64_t i : gr.mats) {
        const MatGeom& g = p->geom[i];
        const int64_t tm = g.m_pad / kTile, tn = g.n_pad / kTile;
        gr.sym += tm * (tm + 1) / 2;
        gr.upd += tm * tn;
        if (g.tall) gr.fin_tall += tm * tn; else gr.fin_wide += tm * tn;
      }
      gr.t_sym = off_t;
      gr.t_upd = gr.t_sym + gr.sym;
      gr.t_fin_wide = gr.t_upd + gr.upd;
      gr.t_fin_tall = gr.t_fin_wide + gr.fin_wide;
      off_t = gr.t_fin_tall + gr.fin_tall;
    }
  }
  if (p->ew_total >= (int64_t(1) << 31) || p->upd_total >= (int64_t(1) << 31))
    return fail(MFSDP_ERR_UNSUPPORTED, "too many tiles in one call");
  size_t off = 0;
  p->off_descs = off;
  off = align_up(off + n * sizeof(MatDesc), kWsAlign);
  p->off_lists = off;
  // block work list (mat[n], begin[n+1]) and momentum workgroup list (same form)
  off = align_up(off + (4 * n + 2) * sizeof(int32_t), kWsAlign);
  // per-tile (matrix, tile) tables, per group: symmetric launches, updates,
  // final update over wide matrices, final update over tall matrices
  p->off_tiles = off;
  off = align_up(off + (p->gram_total + 2 * p->upd_total) * sizeof(int2), kWsAlign);
  p->off_small = off;
  off = align_up(off + p->small.size() * sizeof(int32_t), kWsAlign);
  p->blob_bytes = off;
  p->off_scales = off;
  off = align_up(off + n * sizeof(float), kWsAlign);
  p->off_partials = off;
  off = align_up(off + p->ew_total * sizeof(double), kWsAlign);
  p->off_x0.resize(n);
  p->off_x1.resize(n);
  p->off_a.resize(n);
  p->off_b.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    const MatGeom& g = p->geom[i];
    const size_t xb = size_t(g.m_pad) * size_t(g.n_pad) * es;
    const size_t ab = size_t(g.m_pad) * size_t(g.m_pad) * es;
    p->off_x0[i] = off; off = align_up(off + xb, kWsAlign);
    p->off_x1[i] = off; off = align_up(off + xb, kWsAlign);
    p->off_a[i] = off;  off = align_up(off + ab, kWsAlign);
    p->off_b[i] = off;  off = align_up(off + ab, kWsAlign);
  }
  p->total = off;
  return MFSDP_OK;
}

struct Range {
  uintptr_t lo, hi;
  const char* what;
  int64_t idx;
};

mfsdp_status_t check_aliasing(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  size_t far = 0;  // range with the highest end so far
  for (size_t i = 1; i < rs.size(); ++i) {
    if (rs[i].lo < rs[far].hi)
      return fail(MFSDP_ERR_ALIAS, "%s of matrix %lld overlaps %s of matrix %lld",
                  rs[i].what, (long long)rs[i].idx, rs[far].what, (long long)rs[far].idx);
    if (rs[i].hi > rs[far].hi) far = i;
  }
  return MFSDP_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Auxiliary streams and fork/join events for the Newton-Schulz groups, one
// set per (device, caller stream): calls on different caller streams never
// share an auxiliary stream, so they do not wait for each other's groups.
// Created on first use and kept until the process ends (host objects, no
// device memory).  Every stream has the default priority.  A destroyed
// caller stream whose handle is reused by a new stream reuses its set, which
// is harmless: the set only orders work behind its current caller stream.
struct StreamPool {
  hipStream_t aux[kMaxGroups - 1] = {};
  hipEvent_t fork = nullptr;
  hipEvent_t join[kMaxGroups - 1] = {};
};

std::mutex g_pool_mu;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<StreamPool>> g_pools;

hipError_t get_pool(hipStream_t caller, StreamPool** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  auto key = std::make_pair(dev, caller);
  auto it = g_pools.find(key);
  if (it == g_pools.end()) {
    std::unique_ptr<StreamPool> sp(new StreamPool);
    for (int i = 0; i < kMaxGroups - 1; ++i) {
      e = hipStreamCreateWithFlags(&sp->aux[i], hipStreamNonBlocking);
      if (e != hipSuccess) return e;
      e = hipEventCreateWithFlags(&sp->join[i], hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
    e = hipEventCreateWithFlags(&sp->fork, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    it = g_pools.emplace(key, std::move(sp)).first;
  }
  *out = it->second.get();
  return hipSuccess;
}

// The step and statistics calls upload their launch tables with a copy from
// host memory that is freed when the call returns; a graph captured around
// such a copy would replay a dangling host pointer.  Capture is refused
// (before anything is enqueued, so the capture itself stays valid).
mfsdp_status_t refuse_capture(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess)
    return fail(MFSDP_ERR_HIP, "hipStreamIsCapturing: %s", hipGetErrorString(e));
  if (cs != hipStreamCaptureStatusNone)
    return fail(MFSDP_ERR_UNSUPPORTED,
                "the stream is being captured into a graph; the call uploads its launch "
                "tables from host memory and cannot be captured");
  return MFSDP_OK;
}

// MFSDP_LOG=1: print the launch plan of a step to stderr (debugging aid).
bool log_enabled() {
  const char* v = getenv("MFSDP_LOG");
  return v && v[0] == '1';
}

void log_plan(const Plan& p, int64_t n, mfsdp_dtype_t dt, int ns_steps, hipStream_t stream) {
  fprintf(stderr,
          "mfsdp_muon_step: %lld matrices, %s, ns_steps %d, stream %p, workspace %zu bytes, "
          "momentum blocks %lld, %zu Newton-Schulz group(s)\n",
          (long long)n, dt == MFSDP_DTYPE_BF16 ? "bf16" : "fp32", ns_steps,
          static_cast<void*>(stream), p.total, (long long)p.ew_total, p.groups.size());
  for (size_t g = 0; g < p.groups.size(); ++g) {
    const Plan::Group& gr = p.groups[g];
    std::map<std::pair<int64_t, int64_t>, int> shapes;   // (m_pad, n_pad) -> count
    for (int64_t i : gr.mats) shapes[{p.geom[i].m_pad, p.geom[i].n_pad}] += 1;
    fprintf(stderr,
            "  group %zu on %s: %zu matrices; tiles per launch: gram/poly %lld, update %lld, "
            "final wide %lld, final tall %lld; padded shapes (m x n):",
            g, g == 0 ? "the caller's stream" : "an auxiliary stream", gr.mats.size(),
            (long long)gr.sym, (long long)gr.upd, (long long)gr.fin_wide,
            (long long)gr.fin_tall);
    for (const auto& kv : shapes)
      fprintf(stderr, " %lldx%lld*%d", (long long)kv.first.first, (long long)kv.first.second,
              kv.second);
    fprintf(stderr, "\n");
  }
}

// Newton-Schulz iterations of one group on one stream.
template <class E>
hipError_t enqueue_ns_group(const Plan& p, const Plan::Group& gr, const MatDesc* descs,
                            const int2* tiles, const float* scales, float decay, int ns_steps,
                            float a, float b, float c, hipStream_t stream) {
  const bool skip_poly = (c == 0.f);
  hipError_t e = hipSuccess;
  for (int it = 0; it < ns_steps; ++it) {
    NsEpi ep;
    ep.cur = it & 1;
    ep.first = it == 0;
    ep.b_is_A = skip_poly ? 1 : 0;
    ep.fold = skip_poly ? 0 : 1;
    ep.a = a;
    ep.b = b;
    ep.c = c;
    ep.kb = skip_poly ? b : 1.f;
    ep.decay = decay;
    e = launch(MFSDP_KERNEL_GRAM, stream, [&] {
      ns_gemm_kernel<E, kModeGram><<<dim3(static_cast<unsigned>(gr.sym)), dim3(kNsThreads), 0,
                                     stream>>>(descs, tiles + gr.t_sym, scales, ep);
    });
    if (e != hipSuccess) return e;
    if (!skip_poly) {
      e = launch(MFSDP_KERNEL_POLY, stream, [&] {
        ns_gemm_kernel<E, kModePoly><<<dim3(static_cast<unsigned>(gr.sym)), dim3(kNsThreads), 0,
                                       stream>>>(descs, tiles + gr.t_sym, scales, ep);
      });
      if (e != hipSuccess) return e;
    }
    if (it + 1 < ns_steps) {
      e = launch(MFSDP_KERNEL_UPDATE, stream, [&] {
        ns_gemm_kernel<E, kModeUpdate><<<dim3(static_cast<unsigned>(gr.upd)), dim3(kNsThreads), 0,
                                         stream>>>(descs, tiles + gr.t_upd, scales, ep);
      });
      if (e != hipSuccess) return e;
    } else {
      if (gr.fin_wide > 0) {
        e = launch(MFSDP_KERNEL_FINAL, stream, [&] {
          ns_gemm_kernel<E, kModeApplyWide><<<dim3(static_cast<unsigned>(gr.fin_wide)),
                                              dim3(kNsThreads), 0, stream>>>(
              descs, tiles + gr.t_fin_wide, scales, ep);
        });
        if (e != hipSuccess) return e;
      }
      if (gr.fin_tall > 0) {
        e = launch(MFSDP_KERNEL_FINAL, stream, [&] {
          ns_gemm_kernel<E, kModeApplyTall><<<dim3(static_cast<unsigned>(gr.fin_tall)),
                                              dim3(kNsThreads), 0, stream>>>(
              descs, tiles + gr.t_fin_tall, scales, ep);
        });
        if (e != hipSuccess) return e;
      }
    }
  }
  return e;
}

// Whole step.  Momentum and norm run on the caller's stream; then the
// Newton-Schulz groups fork onto the caller's stream plus auxiliary streams
// (their launches overlap, so one group's partial last round of tiles is
// filled by another group's tiles) and join back before returning.  Results
// do not depend on the grouping: every matrix is computed the same way.
template <class E>
hipError_t enqueue_muon(const Plan& p, int64_t n, char* ws, float beta, int nesterov,
                        float decay, int ns_steps, float a, float b, float c,
                        hipStream_t stream) {
  const MatDesc* descs = reinterpret_cast<const MatDesc*>(ws + p.off_descs);
  const int32_t* lists = reinterpret_cast<const int32_t*>(ws + p.off_lists);
  WorkList wl_ew;
  wl_ew.mat = lists;
  wl_ew.begin = lists + n;
  wl_ew.n_items = static_cast<int32_t>(n);
  WorkList wl_mom;
  wl_mom.mat = lists + 2 * n + 1;
  wl_mom.begin = lists + 3 * n + 1;
  wl_mom.n_items = static_cast<int32_t>(n);
  const int2* tiles = reinterpret_cast<const int2*>(ws + p.off_tiles);
  float* scales = reinterpret_cast<float*>(ws + p.off_scales);
  double* partials = reinterpret_cast<double*>(ws + p.off_partials);

  hipError_t e = launch(MFSDP_KERNEL_MOMENTUM, stream, [&] {
    momentum_kernel<E><<<dim3(static_cast<unsigned>(p.ew_wg_total)), dim3(kThreads), 0,
                         stream>>>(descs, wl_mom, partials, beta, nesterov);
  });
  if (e != hipSuccess) return e;
  e = launch(MFSDP_KERNEL_NORM, stream, [&] {
    norm_finalize_kernel<<<dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream>>>(
        descs, partials, scales, MFSDP_NS_EPS);
  });
  if (e != hipSuccess) return e;

  if (ns_steps == 0) {
    return launch(MFSDP_KERNEL_APPLY, stream, [&] {
      apply_x0_kernel<E><<<dim3(static_cast<unsigned>(p.ew_total)), dim3(kThreads), 0, stream>>>(
          descs, wl_ew, scales, decay);
    });
  }

  if (!p.small.empty()) {
    SmallNsArgs sa;
    sa.mats = reinterpret_cast<const int32_t*>(ws + p.off_small);
    sa.a = a;
    sa.b = b;
    sa.c = c;
    sa.ns_steps = ns_steps;
    sa.decay = decay;
    e = launch(MFSDP_KERNEL_SMALL, stream, [&] {
      small_ns_kernel<E><<<dim3(static_cast<unsigned>(p.small.size())), dim3(kSmallThreads), 0,
                           stream>>>(descs, scales, sa);
    });
    if (e != hipSuccess) return e;
  }

  const int ng = static_cast<int>(p.groups.size());
  if (ng == 0) return hipSuccess;
  if (ng == 1)
    return enqueue_ns_group<E>(p, p.groups[0], descs, tiles, scales, decay, ns_steps, a, b, c,
                               stream);

  StreamPool* pool = nullptr;
  e = get_pool(stream, &pool);
  if (e != hipSuccess) return e;
  e = hipEventRecord(pool->fork, stream);
  if (e != hipSuccess) return e;
  for (int g = 1; g < ng; ++g) {
    e = hipStreamWaitEvent(pool->aux[g - 1], pool->fork, 0);
    if (e != hipSuccess) return e;
  }
  for (int g = 0; g < ng; ++g) {
    hipStream_t s = g == 0 ? stream : pool->aux[g - 1];
    e = enqueue_ns_group<E>(p, p.groups[g], descs, tiles, scales, decay, ns_steps, a, b, c, s);
    if (e != hipSuccess) return e;
  }
  for (int g = 1; g < ng; ++g) {
    e = hipEventRecord(pool->join[g - 1], pool->aux[g - 1]);
    if (e != hipSuccess) return e;
    e = hipStreamWaitEvent(stream, pool->join[g - 1], 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Preconditioner statistics (Shampoo-type): L <- beta*L + alpha*G G^T,
// R <- beta*R + alpha*G^T G for each gradient of the list.
// ---------------------------------------------------------------------------
struct StatsPlan {
  std::vector<int64_t> r_pad, c_pad;
  std::vector<size_t> off_xg, off_xt;
  int64_t prep_tiles = 0, syrk_tiles = 0, n_syrk = 0;
  size_t off_prep = 0, off_syrk = 0, off_lists = 0, off_tiles = 0, off_scales = 0;
  size_t blob_bytes = 0, total = 0;
};

mfsdp_status_t build_stats_plan(const mfsdp_stats_matrix_t* mats, int64_t n, size_t es,
                                StatsPlan* p) {
  p->r_pad.resize(n);
  p->c_pad.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t r = mats[i].rows, c = mats[i].cols;
    if (r < 1 || c < 1)
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: rows=%lld cols=%lld must be >= 1",
                  (long long)i, (long long)r, (long long)c);
    const int64_t rp = round_up(r, kTile), cp = round_up(c, kTile);
    if (rp > (int64_t(1) << 24) || cp > (int64_t(1) << 24) || rp * cp >= (int64_t(1) << 31) ||
        rp * cp * static_cast<int64_t>(es) >= (int64_t(1) << 32) ||
        std::max(r, c) * std::max(r, c) >= (int64_t(1) << 31))
      return fail(MFSDP_ERR_UNSUPPORTED, "matrix %lld: %lld x %lld exceeds the size limit",
                  (long long)i, (long long)r, (long long)c);
    p->r_pad[i] = rp;
    p->c_pad[i] = cp;
    p->prep_tiles += (rp / kEwTile) * (cp / kEwTile);
    const int64_t tr = rp / kTile, tc = cp / kTile;
    p->syrk_tiles += tr * (tr + 1) / 2;
    p->n_syrk += 1;
    if (mats[i].right) {
      p->syrk_tiles += tc * (tc + 1) / 2;
      p->n_syrk += 1;
    }
  }
  if (p->prep_tiles >= (int64_t(1) << 31) || p->syrk_tiles >= (int64_t(1) << 31))
    return fail(MFSDP_ERR_UNSUPPORTED, "too many tiles in one call");
  size_t off = 0;
  p->off_prep = off;
  off = align_up(off + n * sizeof(MatDesc), kWsAlign);
  p->off_syrk = off;
  off = align_up(off + p->n_syrk * sizeof(MatDesc), kWsAlign);
  p->off_lists = off;
  off = align_up(off + (2 * n + 1) * sizeof(int32_t), kWsAlign);
  p->off_tiles = off;
  off = align_up(off + p->syrk_tiles * sizeof(int2), kWsAlign);
  p->off_scales = off;
  off = align_up(off + p->n_syrk * sizeof(float), kWsAlign);
  p->blob_bytes = off;
  p->off_xg.resize(n);
  p->off_xt.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    const size_t xb = size_t(p->r_pad[i]) * size_t(p->c_pad[i]) * es;
    p->off_xg[i] = off; off = align_up(off + xb, kWsAlign);
    p->off_xt[i] = off; off = align_up(off + xb, kWsAlign);
  }
  p->total = off;
  return MFSDP_OK;
}

mfsdp_status_t stats_validate(const mfsdp_stats_matrix_t* mats, int64_t n, mfsdp_dtype_t dtype) {
  if (n < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "n_mats < 0");
  if (n > 0 && !mats) return fail(MFSDP_ERR_INVALID_ARGUMENT, "mats is NULL");
  if (dtype != MFSDP_DTYPE_F32 && dtype != MFSDP_DTYPE_BF16)
    return fail(MFSDP_ERR_UNSUPPORTED, "dtype %d", static_cast<int>(dtype));
  if (n > (int64_t(1) << 24)) return fail(MFSDP_ERR_UNSUPPORTED, "too many matrices");
  return MFSDP_OK;
}

template <class E>
hipError_t enqueue_stats(const StatsPlan& p, int64_t n, char* ws, float alpha, float beta,
                         hipStream_t stream) {
  const MatDesc* prep = reinterpret_cast<const MatDesc*>(ws + p.off_prep);
  const MatDesc* syrk = reinterpret_cast<const MatDesc*>(ws + p.off_syrk);
  const int32_t* lists = reinterpret_cast<const int32_t*>(ws + p.off_lists);
  WorkList wl;
  wl.mat = lists;
  wl.begin = lists + n;
  wl.n_items = static_cast<int32_t>(n);
  hipError_t e = launch(MFSDP_KERNEL_STATS_PREP, stream, [&] {
    stats_prep_kernel<E><<<dim3(static_cast<unsigned>(p.prep_tiles)), dim3(kThreads), 0,
                           stream>>>(prep, wl);
  });
  if (e != hipSuccess) return e;
  NsEpi ep{};
  ep.cur = 0;
  ep.a = alpha;
  ep.b = beta;
  return launch(MFSDP_KERNEL_SYRK, stream, [&] {
    ns_gemm_kernel<E, kModeSyrk><<<dim3(static_cast<unsigned>(p.syrk_tiles)), dim3(kNsThreads), 0,
                                   stream>>>(syrk, reinterpret_cast<const int2*>(ws + p.off_tiles),
                                             reinterpret_cast<const float*>(ws + p.off_scales),
                                             ep);
  });
}

mfsdp_status_t stats_impl(const mfsdp_stats_matrix_t* mats, int64_t n, mfsdp_dtype_t dtype,
                          float beta, float alpha, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  g_last_error.clear();
  mfsdp_status_t st = stats_validate(mats, n, dtype);
  if (st != MFSDP_OK) return st;
  if (!std::isfinite(beta) || !std::isfinite(alpha))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "beta and alpha must be finite");
  if (n == 0) return MFSDP_OK;
  const size_t es = elem_size(dtype);
  StatsPlan p;
  st = build_stats_plan(mats, n, es, &p);
  if (st != MFSDP_OK) return st;
  if (!workspace || workspace_bytes < p.total)
    return fail(MFSDP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                p.total);
  if (!aligned(workspace, kWsAlign))
    return fail(MFSDP_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kWsAlign);
  std::vector<Range> rs;
  rs.push_back({reinterpret_cast<uintptr_t>(workspace),
                reinterpret_cast<uintptr_t>(workspace) + p.total, "workspace", -1});
  for (int64_t i = 0; i < n; ++i) {
    const mfsdp_stats_matrix_t& m = mats[i];
    if (!m.grad || !m.left)
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: grad and left are required",
                  (long long)i);
    if (!aligned(m.grad, es) || !aligned(m.left, 4) || (m.right && !aligned(m.right, 4)))
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: misaligned buffer", (long long)i);
    const uintptr_t g = reinterpret_cast<uintptr_t>(m.grad);
    const uintptr_t l = reinterpret_cast<uintptr_t>(m.left);
    rs.push_back({g, g + size_t(m.rows) * size_t(m.cols) * es, "grad", i});
    rs.push_back({l, l + size_t(m.rows) * size_t(m.rows) * 4, "left", i});
    if (m.right) {
      const uintptr_t r = reinterpret_cast<uintptr_t>(m.right);
      rs.push_back({r, r + size_t(m.cols) * size_t(m.cols) * 4, "right", i});
    }
  }
  st = check_aliasing(rs);
  if (st != MFSDP_OK) return st;

  char* ws = static_cast<char*>(workspace);
  std::vector<char> blob(p.blob_bytes, 0);
  MatDesc* prep = reinterpret_cast<MatDesc*>(blob.data() + p.off_prep);
  MatDesc* syrk = reinterpret_cast<MatDesc*>(blob.data() + p.off_syrk);
  int32_t* lists = reinterpret_cast<int32_t*>(blob.data() + p.off_lists);
  int2* tab = reinterpret_cast<int2*>(blob.data() + p.off_tiles);
  int64_t acc = 0, k = 0;
  for (int64_t i = 0; i < n; ++i) {
    const mfsdp_stats_matrix_t& m = mats[i];
    MatDesc& d = prep[i];
    d.G = m.grad;
    d.X0 = ws + p.off_xg[i];
    d.X1 = ws + p.off_xt[i];
    d.rows = static_cast<int32_t>(m.rows);
    d.cols = static_cast<int32_t>(m.cols);
    d.m_pad = static_cast<int32_t>(p.r_pad[i]);
    d.n_pad = static_cast<int32_t>(p.c_pad[i]);
    d.ew_tiles_j = static_cast<int32_t>(p.c_pad[i] / kEwTile);
    lists[i] = static_cast<int32_t>(i);
    lists[n + i] = static_cast<int32_t>(acc);
    acc += (p.r_pad[i] / kEwTile) * (p.c_pad[i] / kEwTile);
    // L = Xg Xg^T (valid rows x rows); R = Xt Xt^T (valid cols x cols)
    for (int side = 0; side < 2; ++side) {
      if (side == 1 && !m.right) continue;
      MatDesc& s = syrk[k];
      s.X0 = side == 0 ? d.X0 : d.X1;
      s.A = side == 0 ? static_cast<void*>(m.left) : static_cast<void*>(m.right);
      s.m = static_cast<int32_t>(side == 0 ? m.rows : m.cols);
      s.m_pad = static_cast<int32_t>(side == 0 ? p.r_pad[i] : p.c_pad[i]);
      s.n_pad = static_cast<int32_t>(side == 0 ? p.c_pad[i] : p.r_pad[i]);
      ++k;
    }
  }
  lists[2 * n] = static_cast<int32_t>(acc);
  {
    std::vector<int64_t> all(static_cast<size_t>(k));
    for (int64_t j = 0; j < k; ++j) all[j] = j;
    launch_order(
        all, [&](int64_t j) { return static_cast<int64_t>(syrk[j].n_pad); },
        [&](int64_t j) {
          const int64_t tm = syrk[j].m_pad / kTile;
          return tm * (tm + 1) / 2;
        },
        tab);
  }
  st = refuse_capture(stream);
  if (st != MFSDP_OK) return st;
  hipError_t e = hipMemcpyAsync(ws, blob.data(), p.blob_bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "descriptor upload: %s", hipGetErrorString(e));
  e = dtype == MFSDP_DTYPE_BF16 ? enqueue_stats<ElemBF16>(p, n, ws, alpha, beta, stream)
                                : enqueue_stats<ElemF32>(p, n, ws, alpha, beta, stream);
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return MFSDP_OK;
}

}  // namespace

extern "C" {

mfsdp_status_t mfsdp_stats_workspace_size(const mfsdp_stats_matrix_t* mats, int64_t n_mats,
                                          mfsdp_dtype_t dtype, size_t* out_bytes) {
  try {
    g_last_error.clear();
    if (!out_bytes) return fail(MFSDP_ERR_INVALID_ARGUMENT, "out_bytes is NULL");
    mfsdp_status_t st = stats_validate(mats, n_mats, dtype);
    if (st != MFSDP_OK) return st;
    if (n_mats == 0) {
      *out_bytes = 0;
      return MFSDP_OK;
    }
    StatsPlan p;
    st = build_stats_plan(mats, n_mats, elem_size(dtype), &p);
    if (st != MFSDP_OK) return st;
    *out_bytes = p.total;
    return MFSDP_OK;
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_shampoo_stats(const mfsdp_stats_matrix_t* mats, int64_t n_mats,
                                   mfsdp_dtype_t dtype, float beta, float alpha,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    return stats_impl(mats, n_mats, dtype, beta, alpha, workspace, workspace_bytes, stream);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

const char* mfsdp_status_string(mfsdp_status_t s) {
  switch (s) {
    case MFSDP_OK: return "MFSDP_OK";
    case MFSDP_ERR_INVALID_ARGUMENT: return "MFSDP_ERR_INVALID_ARGUMENT";
    case MFSDP_ERR_UNSUPPORTED: return "MFSDP_ERR_UNSUPPORTED";
    case MFSDP_ERR_WORKSPACE: return "MFSDP_ERR_WORKSPACE";
    case MFSDP_ERR_ALIAS: return "MFSDP_ERR_ALIAS";
    case MFSDP_ERR_HIP: return "MFSDP_ERR_HIP";
  }
  return "MFSDP_UNKNOWN_STATUS";
}

const char* mfsdp_last_error(void) { return g_last_error.c_str(); }

static mfsdp_status_t workspace_size_impl(const mfsdp_matrix_t* mats, int64_t n_mats,
                                          mfsdp_dtype_t dtype, size_t* out_bytes) {
  g_last_error.clear();
  if (!out_bytes) return fail(MFSDP_ERR_INVALID_ARGUMENT, "out_bytes is null");
  *out_bytes = 0;
  if (dtype != MFSDP_DTYPE_F32 && dtype != MFSDP_DTYPE_BF16)
    return fail(MFSDP_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dtype);
  if (n_mats < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "n_mats < 0");
  if (n_mats == 0) return MFSDP_OK;
  if (!mats) return fail(MFSDP_ERR_INVALID_ARGUMENT, "mats is null");
  if (n_mats > (int64_t(1) << 20)) return fail(MFSDP_ERR_UNSUPPORTED, "too many matrices");
  Plan p;
  mfsdp_status_t st = build_plan(mats, n_mats, dtype, &p);
  if (st != MFSDP_OK) return st;
  *out_bytes = p.total;
  return MFSDP_OK;
}

static mfsdp_status_t muon_step_impl(const mfsdp_matrix_t* mats, int64_t n_mats,
                                     mfsdp_dtype_t dtype, float lr, float beta, int nesterov,
                                     float weight_decay, int ns_steps, float a, float b,
                                     float c, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream, int max_groups = kMaxGroups) {
  g_last_error.clear();
  if (dtype != MFSDP_DTYPE_F32 && dtype != MFSDP_DTYPE_BF16)
    return fail(MFSDP_ERR_UNSUPPORTED, "unsupported dtype %d", (int)dtype);
  if (n_mats < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "n_mats < 0");
  if (!finite(lr) || !finite(beta) || !finite(weight_decay) || !finite(a) || !finite(b) ||
      !finite(c))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "non-finite hyperparameter");
  if (ns_steps < 0 || ns_steps > 100)
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "ns_steps=%d outside [0, 100]", ns_steps);
  if (n_mats == 0) return MFSDP_OK;
  if (!mats) return fail(MFSDP_ERR_INVALID_ARGUMENT, "mats is null");
  if (n_mats > (int64_t(1) << 20)) return fail(MFSDP_ERR_UNSUPPORTED, "too many matrices");

  Plan p;
  mfsdp_status_t st = build_plan(mats, n_mats, dtype, &p, max_groups);
  if (st != MFSDP_OK) return st;

  const size_t es = elem_size(dtype);
  std::vector<Range> ranges;
  ranges.reserve(4 * n_mats + 1);
  for (int64_t i = 0; i < n_mats; ++i) {
    const mfsdp_matrix_t& mt = mats[i];
    if (!mt.weight || !mt.grad || !mt.momentum)
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: null weight/grad/momentum",
                  (long long)i);
    if (!aligned(mt.weight, MFSDP_ALIGNMENT) || !aligned(mt.grad, MFSDP_ALIGNMENT) ||
        !aligned(mt.momentum, MFSDP_ALIGNMENT) ||
        (mt.update_out && !aligned(mt.update_out, MFSDP_ALIGNMENT)))
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: buffers must be %d-byte aligned",
                  (long long)i, MFSDP_ALIGNMENT);
    if (!finite(mt.scale) || !(mt.scale > 0.f))
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "matrix %lld: scale must be finite and > 0",
                  (long long)i);
    const size_t bytes = size_t(mt.rows) * size_t(mt.cols) * es;
    auto add = [&](const void* ptr, size_t nb, const char* what) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(ptr);
      ranges.push_back({lo, lo + nb, what, i});
    };
    add(mt.weight, bytes, "weight");
    add(mt.grad, bytes, "grad");
    add(mt.momentum, bytes, "momentum");
    if (mt.update_out) add(mt.update_out, size_t(mt.rows) * size_t(mt.cols) * 4, "update_out");
  }
  if (!workspace) return fail(MFSDP_ERR_WORKSPACE, "workspace is null");
  if (!aligned(workspace, kWsAlign))
    return fail(MFSDP_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kWsAlign);
  if (workspace_bytes < p.total)
    return fail(MFSDP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                p.total);
  {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace);
    ranges.push_back({lo, lo + p.total, "workspace", -1});
  }
  st = check_aliasing(ranges);
  if (st != MFSDP_OK) return st;

  // Host image of descriptors and work lists.
  char* ws = static_cast<char*>(workspace);
  std::vector<char> blob(p.blob_bytes, 0);
  MatDesc* descs = reinterpret_cast<MatDesc*>(blob.data() + p.off_descs);
  int32_t* lists = reinterpret_cast<int32_t*>(blob.data() + p.off_lists);
  int64_t ew_acc = 0;
  for (int64_t i = 0; i < n_mats; ++i) {
    const MatGeom& g = p.geom[i];
    const mfsdp_matrix_t& mt = mats[i];
    MatDesc& d = descs[i];
    d.W = mt.weight;
    d.G = mt.grad;
    d.M = mt.momentum;
    d.upd = mt.update_out;
    d.X0 = ws + p.off_x0[i];
    d.X1 = ws + p.off_x1[i];
    d.A = ws + p.off_a[i];
    d.B = ws + p.off_b[i];
    d.rows = static_cast<int32_t>(g.rows);
    d.cols = static_cast<int32_t>(g.cols);
    d.m = static_cast<int32_t>(g.m);
    d.n = static_cast<int32_t>(g.n);
    d.m_pad = static_cast<int32_t>(g.m_pad);
    d.n_pad = static_cast<int32_t>(g.n_pad);
    d.tall = g.tall ? 1 : 0;
    d.ew_tile0 = static_cast<int32_t>(ew_acc);
    d.ew_tiles_j = static_cast<int32_t>(g.ew_tiles_j);
    d.ew_ntiles = static_cast<int32_t>(g.ew_ntiles);
    d.ew_th = static_cast<int32_t>(g.ew_th);
    d.ew_tw = static_cast<int32_t>(g.ew_tw);
    d.lr_scale = lr * mt.scale;
    d.vec_ok = (g.cols % static_cast<int64_t>(16 / es)) == 0 ? 1 : 0;
    ew_acc += g.ew_ntiles;
  }
  // blocks (and momentum workgroups) in list order: partial sums of a matrix
  // stay contiguous in the order the finalization reads them.
  {
    int32_t* mat = lists;
    int32_t* begin = mat + n_mats;
    int32_t* wmat = lists + 2 * n_mats + 1;
    int32_t* wbegin = wmat + n_mats;
    int64_t acc = 0, wacc = 0;
    for (int64_t i = 0; i < n_mats; ++i) {
      mat[i] = wmat[i] = static_cast<int32_t>(i);
      begin[i] = static_cast<int32_t>(acc);
      wbegin[i] = static_cast<int32_t>(wacc);
      acc += p.geom[i].ew_ntiles;
      wacc += (p.geom[i].ew_ntiles + kEwSub - 1) / kEwSub;
    }
    begin[n_mats] = static_cast<int32_t>(acc);
    wbegin[n_mats] = static_cast<int32_t>(wacc);
  }
  // per-group tile tables: each launch's tiles by decreasing K (a matrix's
  // tiles together), balanced over the XCDs
  {
    int2* tab = reinterpret_cast<int2*>(blob.data() + p.off_tiles);
    auto sym_tiles = [&](int64_t i) {
      const int64_t tm = p.geom[i].m_pad / kTile;
      return tm * (tm + 1) / 2;
    };
    auto all_tiles = [&](int64_t i) {
      return (p.geom[i].m_pad / kTile) * (p.geom[i].n_pad / kTile);
    };
    // The Gram (K = n) and polynomial (K = m) launches share one table: by
    // decreasing n, then m, in runs of equal (n, m), so that both K are
    // balanced over the XCDs.
    auto k_sym = [&](int64_t i) { return (p.geom[i].n_pad << 24) | p.geom[i].m_pad; };
    auto k_mm = [&](int64_t i) { return p.geom[i].m_pad; };   // update, apply
    for (const Plan::Group& gr : p.groups) {
      std::vector<int64_t> wide, tall;
      for (int64_t i : gr.mats) (p.geom[i].tall ? tall : wide).push_back(i);
      launch_order(gr.mats, k_sym, sym_tiles, tab + gr.t_sym);
      launch_order(gr.mats, k_mm, all_tiles, tab + gr.t_upd);
      launch_order(wide, k_mm, all_tiles, tab + gr.t_fin_wide);
      launch_order(tall, k_mm, all_tiles, tab + gr.t_fin_tall);
    }
  }

  st = refuse_capture(stream);
  if (st != MFSDP_OK) return st;
  if (log_enabled()) log_plan(p, n_mats, dtype, ns_steps, stream);

  {
    int32_t* sm = reinterpret_cast<int32_t*>(blob.data() + p.off_small);
    for (size_t j = 0; j < p.small.size(); ++j) sm[j] = static_cast<int32_t>(p.small[j]);
  }

  hipError_t e = hipMemcpyAsync(ws, blob.data(), p.blob_bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "descriptor upload: %s", hipGetErrorString(e));

  const float decay = 1.f - lr * weight_decay;
  if (dtype == MFSDP_DTYPE_BF16)
    e = enqueue_muon<ElemBF16>(p, n_mats, ws, beta, nesterov ? 1 : 0, decay, ns_steps, a, b, c,
                               stream);
  else
    e = enqueue_muon<ElemF32>(p, n_mats, ws, beta, nesterov ? 1 : 0, decay, ns_steps, a, b, c,
                              stream);
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "launch: %s", hipGetErrorString(e));
  return MFSDP_OK;
}

static mfsdp_status_t adamw_tail_impl(float* param, const float* grad, float* exp_avg,
                                      float* exp_avg_sq, int64_t n, float lr, float beta1,
                                      float beta2, float eps, float weight_decay, int64_t step,
                                      hipStream_t stream) {
  g_last_error.clear();
  if (n < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "n < 0");
  if (!finite(lr) || !finite(beta1) || !finite(beta2) || !finite(eps) || !finite(weight_decay))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "non-finite hyperparameter");
  if (!(beta1 >= 0.f && beta1 < 1.f) || !(beta2 >= 0.f && beta2 < 1.f))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "beta1, beta2 must be in [0, 1)");
  if (eps < 0.f) return fail(MFSDP_ERR_INVALID_ARGUMENT, "eps < 0");
  if (step < 1) return fail(MFSDP_ERR_INVALID_ARGUMENT, "step=%lld must be >= 1", (long long)step);
  if (n == 0) return MFSDP_OK;
  if (!param || !grad || !exp_avg || !exp_avg_sq)
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "null tail buffer");
  if (!aligned(param, MFSDP_ALIGNMENT) || !aligned(grad, MFSDP_ALIGNMENT) ||
      !aligned(exp_avg, MFSDP_ALIGNMENT) || !aligned(exp_avg_sq, MFSDP_ALIGNMENT))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "tail buffers must be %d-byte aligned",
                MFSDP_ALIGNMENT);
  if (n > (int64_t(1) << 40)) return fail(MFSDP_ERR_UNSUPPORTED, "n too large");
  std::vector<Range> rs;
  const size_t nb = size_t(n) * 4;
  rs.push_back({reinterpret_cast<uintptr_t>(param), reinterpret_cast<uintptr_t>(param) + nb, "param", 0});
  rs.push_back({reinterpret_cast<uintptr_t>(grad), reinterpret_cast<uintptr_t>(grad) + nb, "grad", 0});
  rs.push_back({reinterpret_cast<uintptr_t>(exp_avg), reinterpret_cast<uintptr_t>(exp_avg) + nb, "exp_avg", 0});
  rs.push_back({reinterpret_cast<uintptr_t>(exp_avg_sq), reinterpret_cast<uintptr_t>(exp_avg_sq) + nb, "exp_avg_sq", 0});
  mfsdp_status_t st = check_aliasing(rs);
  if (st != MFSDP_OK) return st;

  AdamWArgs args;
  args.decay = 1.f - lr * weight_decay;
  args.beta1 = beta1;
  args.beta2 = beta2;
  args.one_m_beta1 = 1.f - beta1;
  args.one_m_beta2 = 1.f - beta2;
  const double bc1 = 1.0 - std::pow(static_cast<double>(beta1), static_cast<double>(step));
  const double bc2 = 1.0 - std::pow(static_cast<double>(beta2), static_cast<double>(step));
  args.step_size = static_cast<float>(static_cast<double>(lr) / bc1);
  args.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(bc2));
  args.eps = eps;
  // one workgroup per kThreads * U 16-byte groups; at least one for the
  // n % 4 remainder
  const bool large = (n >> 2) >= kAdamLargeGroups;
  const int64_t per_block = int64_t(kThreads) * (large ? 4 : 1);
  const int64_t blocks = std::max<int64_t>(((n >> 2) + per_block - 1) / per_block, 1);
  hipError_t e = launch(MFSDP_KERNEL_ADAMW, stream, [&] {
    if (large)
      adamw_kernel<4, true><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(
          param, grad, exp_avg, exp_avg_sq, n, args);
    else
      adamw_kernel<1, false><<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(
          param, grad, exp_avg, exp_avg_sq, n, args);
  });
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "adamw launch: %s", hipGetErrorString(e));
  return MFSDP_OK;
}

// ---------------------------------------------------------------------------
// Step without a caller workspace, for callers that cannot allocate device
// memory: the workspace is a file-scope device array of fixed size, one copy
// per GPU, which the loader places when the library's code object is loaded
// on that GPU and which stays until the process ends.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[MFSDP_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each device, taken once per device with that
// device current.  The host-side name `scratch` is only a stand-in: kernels
// receive these addresses, never the name.
static std::mutex g_scratch_mu;
static std::map<int, void*> g_scratch_ptr;

static mfsdp_status_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(MFSDP_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return MFSDP_OK;
}

// Same step as mfsdp_muon_step with the static scratch as its workspace.  The
// size check comes first, before the device is touched.  Every Newton-Schulz
// group stays on the caller's stream, so the call creates no auxiliary
// stream or event.  Nothing in the workspace has to start at zero: the
// momentum kernel writes every iterate's padding and each launch overwrites
// the tables and partial sums it reads.
static mfsdp_status_t muon_noalloc_impl(const mfsdp_matrix_t* mats, int64_t n_mats,
                                        mfsdp_dtype_t dtype, float lr, float beta,
                                        int nesterov, float weight_decay, int ns_steps,
                                        float a, float b, float c, hipStream_t stream) {
  size_t need = 0;
  mfsdp_status_t st = workspace_size_impl(mats, n_mats, dtype, &need);
  if (st != MFSDP_OK) return st;
  if (need > MFSDP_NOALLOC_SCRATCH_BYTES)
    return fail(MFSDP_ERR_WORKSPACE,
                "the list needs %zu bytes of workspace; the static scratch of "
                "mfsdp_muon_step_noalloc holds %zu (MFSDP_NOALLOC_SCRATCH_BYTES): split the list "
                "or call mfsdp_muon_step with a workspace",
                need, static_cast<size_t>(MFSDP_NOALLOC_SCRATCH_BYTES));
  if (n_mats == 0)   // validation of the hyperparameters, no device access
    return muon_step_impl(mats, 0, dtype, lr, beta, nesterov, weight_decay, ns_steps, a, b, c,
                          nullptr, 0, stream, 1);
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != MFSDP_OK) return st;
  return muon_step_impl(mats, n_mats, dtype, lr, beta, nesterov, weight_decay, ns_steps, a, b,
                        c, ws, MFSDP_NOALLOC_SCRATCH_BYTES, stream, 1);
}

// No C++ exception crosses the ABI: allocation failures of the host-side plan
// become MFSDP_ERR_UNSUPPORTED.
mfsdp_status_t mfsdp_muon_workspace_size(const mfsdp_matrix_t* mats, int64_t n_mats,
                                         mfsdp_dtype_t dtype, size_t* out_bytes) {
  try {
    return workspace_size_impl(mats, n_mats, dtype, out_bytes);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_muon_step(const mfsdp_matrix_t* mats, int64_t n_mats, mfsdp_dtype_t dtype,
                               float lr, float beta, int nesterov, float weight_decay,
                               int ns_steps, float a, float b, float c, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  try {
    return muon_step_impl(mats, n_mats, dtype, lr, beta, nesterov, weight_decay, ns_steps, a, b,
                          c, workspace, workspace_bytes, stream);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_muon_step_noalloc(const mfsdp_matrix_t* mats, int64_t n_mats,
                                       mfsdp_dtype_t dtype, float lr, float beta, int nesterov,
                                       float weight_decay, int ns_steps, float a, float b,
                                       float c, hipStream_t stream) {
  try {
    return muon_noalloc_impl(mats, n_mats, dtype, lr, beta, nesterov, weight_decay, ns_steps,
                             a, b, c, stream);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_adamw_tail(float* param, const float* grad, float* exp_avg,
                                float* exp_avg_sq, int64_t n, float lr, float beta1, float beta2,
                                float eps, float weight_decay, int64_t step,
                                hipStream_t stream) {
  try {
    return adamw_tail_impl(param, grad, exp_avg, exp_avg_sq, n, lr, beta1, beta2, eps,
                           weight_decay, step, stream);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_plan_owners(const double* cost_ms, const int64_t* bytes, int64_t n_items,
                                 int32_t n_ranks, double byte_slack, int32_t* owner,
                                 double* rank_ms, int64_t* rank_bytes) {
  try {
    g_last_error.clear();
    if (n_items < 0 || n_ranks < 1)
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "n_items=%lld n_ranks=%d", (long long)n_items,
                  n_ranks);
    if (!rank_ms || !rank_bytes || (n_items > 0 && (!cost_ms || !bytes || !owner)))
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "null pointer");
    if (!(byte_slack >= 0.0) || !std::isfinite(byte_slack))
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "byte_slack must be finite and >= 0");
    for (int64_t i = 0; i < n_items; ++i) {
      if (!(cost_ms[i] >= 0.0) || !std::isfinite(cost_ms[i]))
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "item %lld: cost must be finite and >= 0",
                    (long long)i);
      if (bytes[i] < 0)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "item %lld: bytes < 0", (long long)i);
    }
    plan_lpt(cost_ms, bytes, n_items, n_ranks, byte_slack, owner, rank_ms, rank_bytes);
    return MFSDP_OK;
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_tail_layout(const int64_t* numel, int64_t n, int64_t* offsets,
                                 int64_t* total) {
  g_last_error.clear();
  if (n < 0 || !total || (n > 0 && (!numel || !offsets)))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "bad tail layout arguments");
  for (int64_t i = 0; i < n; ++i)
    if (numel[i] < 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "tensor %lld: numel < 0",
                                  (long long)i);
  *total = tail_layout(numel, n, offsets);
  return MFSDP_OK;
}

}  // extern "C"

namespace {

// Shared by pack (to_packed) and unpack: validate, then copy in launches of
// up to kTailSegs segments.
mfsdp_status_t tail_copy(float* packed_rw, int64_t packed_numel, float* const* tensors,
                         const int64_t* numel, const int64_t* offsets, int64_t n, bool to_packed,
                         hipStream_t stream) {
  g_last_error.clear();
  if (n < 0 || packed_numel < 0)
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "n=%lld packed_numel=%lld", (long long)n,
                (long long)packed_numel);
  if (n == 0) return MFSDP_OK;
  if (!numel || !offsets || !tensors || !packed_rw)
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "null pointer");
  if (!aligned(packed_rw, 16))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "packed buffer must be 16-byte aligned");
  std::vector<int64_t> order(n);
  for (int64_t i = 0; i < n; ++i) {
    if (numel[i] < 0 || offsets[i] < 0 || offsets[i] % kTailAlign != 0)
      return fail(MFSDP_ERR_INVALID_ARGUMENT,
                  "tensor %lld: numel >= 0 and a non-negative offset multiple of %lld needed",
                  (long long)i, (long long)kTailAlign);
    const int64_t span = (numel[i] + kTailAlign - 1) / kTailAlign * kTailAlign;
    if (offsets[i] + span > packed_numel)
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "tensor %lld: segment ends past the buffer",
                  (long long)i);
    if (numel[i] > 0 && !tensors[i])
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "tensor %lld: null pointer", (long long)i);
    if (numel[i] > 0 && (reinterpret_cast<uintptr_t>(tensors[i]) & 3) != 0)
      return fail(MFSDP_ERR_INVALID_ARGUMENT, "tensor %lld: not 4-byte aligned", (long long)i);
    order[i] = i;
  }
  // empty segments occupy nothing and are left out of the overlap check
  order.erase(std::remove_if(order.begin(), order.end(),
                             [&](int64_t i) { return numel[i] == 0; }),
              order.end());
  std::sort(order.begin(), order.end(),
            [&](int64_t a, int64_t b) { return offsets[a] < offsets[b]; });
  for (size_t j = 1; j < order.size(); ++j) {
    const int64_t a = order[j - 1], b = order[j];
    const int64_t span_a = (numel[a] + kTailAlign - 1) / kTailAlign * kTailAlign;
    if (offsets[a] + span_a > offsets[b])
      return fail(MFSDP_ERR_ALIAS, "segments of tensors %lld and %lld overlap", (long long)a,
                  (long long)b);
  }
  // tensors must not overlap the packed buffer
  {
    std::vector<Range> rs;
    rs.push_back({reinterpret_cast<uintptr_t>(packed_rw),
                  reinterpret_cast<uintptr_t>(packed_rw + packed_numel), "packed buffer", -1});
    for (int64_t i = 0; i < n; ++i)
      if (numel[i] > 0)
        rs.push_back({reinterpret_cast<uintptr_t>(tensors[i]),
                      reinterpret_cast<uintptr_t>(tensors[i] + numel[i]), "tensor", i});
    if (!to_packed) {   // unpack writes every tensor: they must not overlap each other either
      mfsdp_status_t st = check_aliasing(rs);
      if (st != MFSDP_OK) return st;
    } else {
      const uintptr_t lo = rs[0].lo, hi = rs[0].hi;
      for (size_t k = 1; k < rs.size(); ++k)
        if (rs[k].lo < hi && lo < rs[k].hi)
          return fail(MFSDP_ERR_ALIAS, "tensor %lld overlaps the packed buffer",
                      (long long)rs[k].idx);
    }
  }
  TailBatch b{};
  auto flush = [&]() -> hipError_t {
    if (b.count == 0) return hipSuccess;
    const int64_t blocks = b.block0[b.count];
    hipError_t e = hipSuccess;
    if (blocks > 0) {
      tail_copy_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(b);
      e = hipGetLastError();
    }
    b = TailBatch{};
    return e;
  };
  for (int64_t i = 0; i < n; ++i) {
    const int64_t span = to_packed ? (numel[i] + kTailAlign - 1) / kTailAlign * kTailAlign
                                   : numel[i];
    if (span == 0) continue;
    TailSeg& g = b.seg[b.count];
    if (to_packed) {
      g.src = tensors[i];
      g.dst = packed_rw + offsets[i];
    } else {
      g.src = packed_rw + offsets[i];
      g.dst = tensors[i];
    }
    g.n = numel[i];
    g.span = span;
    b.block0[b.count + 1] = b.block0[b.count] + (span + kTailBlockElems - 1) / kTailBlockElems;
    ++b.count;
    if (b.count == kTailSegs || b.block0[b.count] > (int64_t(1) << 30)) {
      hipError_t e = flush();
      if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "tail copy: %s", hipGetErrorString(e));
    }
  }
  hipError_t e = flush();
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "tail copy: %s", hipGetErrorString(e));
  return MFSDP_OK;
}

}  // namespace

extern "C" {

mfsdp_status_t mfsdp_tail_pack(const float* const* src, const int64_t* numel,
                               const int64_t* offsets, int64_t n, float* packed,
                               int64_t packed_numel, hipStream_t stream) {
  try {
    return tail_copy(packed, packed_numel, const_cast<float* const*>(src), numel, offsets, n,
                     true, stream);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_tail_unpack(const float* packed, int64_t packed_numel, float* const* dst,
                                 const int64_t* numel, const int64_t* offsets, int64_t n,
                                 hipStream_t stream) {
  try {
    return tail_copy(const_cast<float*>(packed), packed_numel, dst, numel, offsets, n, false,
                     stream);
  } catch (const std::exception& ex) {
    return fail(MFSDP_ERR_UNSUPPORTED, "host exception: %s", ex.what());
  }
}

mfsdp_status_t mfsdp_mfma_probe(float* out, int64_t blocks, int iters, hipStream_t stream) {
  g_last_error.clear();
  if (!out) return fail(MFSDP_ERR_INVALID_ARGUMENT, "out is NULL");
  if (blocks < 1 || blocks > (int64_t(1) << 16) || iters < 1 || iters > (1 << 20))
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "blocks=%lld iters=%d outside [1, 65536] x [1, 2^20]",
                (long long)blocks, iters);
  if (blocks * static_cast<int64_t>(iters) > (int64_t(1) << 28))
    return fail(MFSDP_ERR_INVALID_ARGUMENT,
                "blocks * iters = %lld exceeds 2^28 (about half a second of MFMA work)",
                (long long)(blocks * static_cast<int64_t>(iters)));
  if (!aligned(out, 4)) return fail(MFSDP_ERR_INVALID_ARGUMENT, "out must be 4-byte aligned");
  mfma_probe_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kProbeThreads), 0, stream>>>(
      out, iters);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "probe launch: %s", hipGetErrorString(e));
  return MFSDP_OK;
}

mfsdp_status_t mfsdp_timing_enable(int enable) {
  g_last_error.clear();
  g_timing.enabled = enable != 0;
  return MFSDP_OK;
}

mfsdp_status_t mfsdp_timing_reset(void) {
  g_last_error.clear();
  hipError_t e = drain_timing();
  for (int k = 0; k < MFSDP_KERNEL_KINDS; ++k) {
    g_timing.total_ms[k] = 0.0;
    g_timing.count[k] = 0;
  }
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "timing: %s", hipGetErrorString(e));
  return MFSDP_OK;
}

mfsdp_status_t mfsdp_timing_read(mfsdp_kernel_kind_t kind, double* total_ms, int64_t* launches) {
  g_last_error.clear();
  if (kind < 0 || kind >= MFSDP_KERNEL_KINDS || !total_ms || !launches)
    return fail(MFSDP_ERR_INVALID_ARGUMENT, "bad timing query");
  hipError_t e = drain_timing();
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "timing: %s", hipGetErrorString(e));
  *total_ms = g_timing.total_ms[kind];
  *launches = g_timing.count[kind];
  return MFSDP_OK;
}

}  // extern "C"

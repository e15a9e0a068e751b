// Host side of the owner-local optimizer step: argument validation, the
// grouped launch plan, and the C ABI declared in include/mfsdp.h.
//
// Source of the operations: "MatrixFSDP: communication-free matrix optimizers
// under ZeRO-3 parameter sharding" (arxivlens page, Abstract): the owner of a
// whole 2D weight runs Muon's Newton-Schulz on it locally, and non-matrix
// tensors packed into tail owners take AdamW.  One call covers the owner's
// whole list: every kernel is one grouped launch over all owned matrices.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <exception>
#include <string>
#include <vector>

#include "../../include/mfsdp.h"
#include "common.hpp"
#include "ew_kernels.hpp"
#include "ns_gemm.hpp"

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
  if (g_timing.enabled) {
    hipError_t e = take_event(&a);
    if (e == hipSuccess) e = take_event(&b);
    if (e == hipSuccess) e = hipEventRecord(a, stream);
    if (e != hipSuccess) return e;
  }
  f();
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g_timing.enabled) {
    e = hipEventRecord(b, stream);
    if (e != hipSuccess) return e;
    g_timing.pending.push_back({kind, a, b});
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Plan of one mfsdp_muon_step call.
// ---------------------------------------------------------------------------
struct MatGeom {
  int64_t rows, cols, m, n, m_pad, n_pad;
  bool tall;
  int64_t ew_tiles_j, ew_ntiles;
};

struct Plan {
  std::vector<MatGeom> geom;
  size_t off_descs = 0, off_lists = 0, off_tiles = 0, off_scales = 0, off_partials = 0;
  size_t blob_bytes = 0;            // descriptors + work lists (host upload)
  std::vector<size_t> off_x0, off_x1, off_a, off_b;
  size_t total = 0;
  int64_t ew_total = 0, gram_total = 0, upd_total = 0;
  int64_t upd_wide_total = 0;       // tiles of matrices stored wide (rows <= cols)
};

mfsdp_status_t make_geom(const mfsdp_matrix_t& mt, int64_t idx, MatGeom* g) {
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
  if (g->n_pad > (int64_t(1) << 24) || g->m_pad * g->n_pad >= (int64_t(1) << 31))
    return fail(MFSDP_ERR_UNSUPPORTED,
                "matrix %lld: %lld x %lld exceeds the 2^31-element iterate limit",
                (long long)idx, (long long)mt.rows, (long long)mt.cols);
  g->ew_tiles_j = g->n_pad / kEwTile;
  g->ew_ntiles = (g->m_pad / kEwTile) * g->ew_tiles_j;
  return MFSDP_OK;
}

mfsdp_status_t build_plan(const mfsdp_matrix_t* mats, int64_t n, mfsdp_dtype_t dt, Plan* p) {
  const size_t es = elem_size(dt);
  p->geom.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    mfsdp_status_t st = make_geom(mats[i], i, &p->geom[i]);
    if (st != MFSDP_OK) return st;
    p->ew_total += p->geom[i].ew_ntiles;
    const int64_t tm = p->geom[i].m_pad / kTile, tn = p->geom[i].n_pad / kTile;
    p->gram_total += tm * (tm + 1) / 2;
    p->upd_total += tm * tn;
    if (!p->geom[i].tall) p->upd_wide_total += tm * tn;
  }
  if (p->ew_total >= (int64_t(1) << 31) || p->upd_total >= (int64_t(1) << 31))
    return fail(MFSDP_ERR_UNSUPPORTED, "too many tiles in one call");
  size_t off = 0;
  p->off_descs = off;
  off = align_up(off + n * sizeof(MatDesc), kWsAlign);
  p->off_lists = off;
  // three work lists (momentum, symmetric products, update): mat[n], begin[n+1]
  off = align_up(off + 3 * (2 * n + 1) * sizeof(int32_t), kWsAlign);
  // per-tile (matrix, tile) tables of the symmetric and update launches
  p->off_tiles = off;
  // tables: symmetric launches, updates, then the final update split into
  // wide-matrix tiles followed by tall-matrix tiles
  off = align_up(off + (p->gram_total + 2 * p->upd_total) * sizeof(int2), kWsAlign);
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

// Work list: items sorted by `key` descending (largest K first).
void fill_list(int32_t* mat, int32_t* begin, const std::vector<int64_t>& tiles,
               const std::vector<int64_t>& key) {
  const int64_t n = static_cast<int64_t>(tiles.size());
  std::vector<int64_t> order(n);
  for (int64_t i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int64_t a, int64_t b) { return key[a] > key[b]; });
  int64_t acc = 0;
  for (int64_t i = 0; i < n; ++i) {
    mat[i] = static_cast<int32_t>(order[i]);
    begin[i] = static_cast<int32_t>(acc);
    acc += tiles[order[i]];
  }
  begin[n] = static_cast<int32_t>(acc);
}

template <class E>
hipError_t enqueue_muon(const Plan& p, int64_t n, char* ws, float beta, int nesterov,
                        float decay, int ns_steps, float a, float b, float c,
                        hipStream_t stream) {
  const MatDesc* descs = reinterpret_cast<const MatDesc*>(ws + p.off_descs);
  const int32_t* lists = reinterpret_cast<const int32_t*>(ws + p.off_lists);
  auto list = [&](int which) {
    WorkList wl;
    wl.mat = lists + which * (2 * n + 1);
    wl.begin = wl.mat + n;
    wl.n_items = static_cast<int32_t>(n);
    return wl;
  };
  const WorkList wl_ew = list(0);
  const int2* tiles_sym = reinterpret_cast<const int2*>(ws + p.off_tiles);
  const int2* tiles_upd = tiles_sym + p.gram_total;
  const int2* tiles_fin_wide = tiles_upd + p.upd_total;
  const int2* tiles_fin_tall = tiles_fin_wide + p.upd_wide_total;
  const int64_t fin_tall_total = p.upd_total - p.upd_wide_total;
  float* scales = reinterpret_cast<float*>(ws + p.off_scales);
  double* partials = reinterpret_cast<double*>(ws + p.off_partials);

  hipError_t e = launch(MFSDP_KERNEL_MOMENTUM, stream, [&] {
    momentum_kernel<E><<<dim3(static_cast<unsigned>(p.ew_total)), dim3(kThreads), 0, stream>>>(
        descs, wl_ew, partials, beta, nesterov);
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

  const bool skip_poly = (c == 0.f);
  for (int it = 0; it < ns_steps; ++it) {
    NsEpi ep;
    ep.cur = it & 1;
    ep.first = it == 0;
    ep.b_is_A = skip_poly ? 1 : 0;
    ep.a = a;
    ep.b = b;
    ep.c = c;
    ep.kb = skip_poly ? b : 1.f;
    ep.decay = decay;
    e = launch(MFSDP_KERNEL_GRAM, stream, [&] {
      ns_gemm_kernel<E, kModeGram><<<dim3(static_cast<unsigned>(p.gram_total)), dim3(kThreads), 0,
                                     stream>>>(descs, tiles_sym, scales, ep);
    });
    if (e != hipSuccess) return e;
    if (!skip_poly) {
      e = launch(MFSDP_KERNEL_POLY, stream, [&] {
        ns_gemm_kernel<E, kModePoly><<<dim3(static_cast<unsigned>(p.gram_total)), dim3(kThreads), 0,
                                       stream>>>(descs, tiles_sym, scales, ep);
      });
      if (e != hipSuccess) return e;
    }
    if (it + 1 < ns_steps) {
      e = launch(MFSDP_KERNEL_UPDATE, stream, [&] {
        ns_gemm_kernel<E, kModeUpdate><<<dim3(static_cast<unsigned>(p.upd_total)), dim3(kThreads),
                                         0, stream>>>(descs, tiles_upd, scales, ep);
      });
    } else {
      if (p.upd_wide_total > 0) {
        e = launch(MFSDP_KERNEL_FINAL, stream, [&] {
          ns_gemm_kernel<E, kModeApplyWide><<<dim3(static_cast<unsigned>(p.upd_wide_total)),
                                              dim3(kThreads), 0, stream>>>(
              descs, tiles_fin_wide, scales, ep);
        });
        if (e != hipSuccess) return e;
      }
      if (fin_tall_total > 0) {
        e = launch(MFSDP_KERNEL_FINAL, stream, [&] {
          ns_gemm_kernel<E, kModeApplyTall><<<dim3(static_cast<unsigned>(fin_tall_total)),
                                              dim3(kThreads), 0, stream>>>(
              descs, tiles_fin_tall, scales, ep);
        });
      }
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

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
                                     hipStream_t stream) {
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
  mfsdp_status_t st = build_plan(mats, n_mats, dtype, &p);
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
  std::vector<int64_t> t_ew(n_mats), t_sym(n_mats), t_upd(n_mats), k_gram(n_mats), k_upd(n_mats),
      zero(n_mats, 0);
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
    d.lr_scale = lr * mt.scale;
    d.vec_ok = (g.cols % static_cast<int64_t>(16 / es)) == 0 ? 1 : 0;
    ew_acc += g.ew_ntiles;
    const int64_t tm = g.m_pad / kTile, tn = g.n_pad / kTile;
    t_ew[i] = g.ew_ntiles;
    t_sym[i] = tm * (tm + 1) / 2;
    t_upd[i] = tm * tn;
    k_gram[i] = g.n_pad;
    k_upd[i] = g.m_pad;
  }
  // momentum tiles in list order: partial sums of a matrix stay contiguous
  // in the order the finalization reads them.
  {
    int32_t* mat = lists;
    int32_t* begin = mat + n_mats;
    int64_t acc = 0;
    for (int64_t i = 0; i < n_mats; ++i) {
      mat[i] = static_cast<int32_t>(i);
      begin[i] = static_cast<int32_t>(acc);
      acc += t_ew[i];
    }
    begin[n_mats] = static_cast<int32_t>(acc);
  }
  fill_list(lists + (2 * n_mats + 1), lists + (2 * n_mats + 1) + n_mats, t_sym, k_gram);
  fill_list(lists + 2 * (2 * n_mats + 1), lists + 2 * (2 * n_mats + 1) + n_mats, t_upd, k_upd);
  {
    // expand the two GEMM work lists into per-tile tables
    int2* tab = reinterpret_cast<int2*>(blob.data() + p.off_tiles);
    for (int which = 1; which <= 2; ++which) {
      const int32_t* mat = lists + which * (2 * n_mats + 1);
      const int32_t* begin = mat + n_mats;
      for (int64_t it = 0; it < n_mats; ++it)
        for (int32_t t = 0; t < begin[it + 1] - begin[it]; ++t) *tab++ = make_int2(mat[it], t);
    }
    // final update: the update list's wide matrices, then its tall ones
    const int32_t* mat = lists + 2 * (2 * n_mats + 1);
    const int32_t* begin = mat + n_mats;
    for (int tall = 0; tall <= 1; ++tall)
      for (int64_t it = 0; it < n_mats; ++it)
        if (p.geom[mat[it]].tall == (tall == 1))
          for (int32_t t = 0; t < begin[it + 1] - begin[it]; ++t) *tab++ = make_int2(mat[it], t);
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
  const int64_t groups = std::max<int64_t>((n >> 2), 1);
  const int64_t blocks = std::min<int64_t>((groups + kThreads - 1) / kThreads, 16384);
  hipError_t e = launch(MFSDP_KERNEL_ADAMW, stream, [&] {
    adamw_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream>>>(
        param, grad, exp_avg, exp_avg_sq, n, args);
  });
  if (e != hipSuccess) return fail(MFSDP_ERR_HIP, "adamw launch: %s", hipGetErrorString(e));
  return MFSDP_OK;
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

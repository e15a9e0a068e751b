// Preparation of a gradient for its preconditioner statistics (Shampoo-type
// L = G G^T and R = G^T G): G (rows x cols, storage dtype, row-major) is
// copied into the workspace twice, as Xg (r_pad x c_pad) and as its transpose
// Xt (c_pad x r_pad), both in iter_off layout, zero outside G, so that both
// statistics are Gram products of a 256-padded operand (kModeSyrk of
// ns_gemm_kernel).
#pragma once

#include "common.hpp"

namespace mfsdp {

// One 256-thread workgroup per 64 x 64 tile of the padded G.  Descriptor
// fields: G, rows, cols; X0 = Xg, X1 = Xt; m_pad = r_pad, n_pad = c_pad;
// ew_tiles_j = c_pad / 64.
template <class E>
__global__ __launch_bounds__(kThreads) void stats_prep_kernel(const MatDesc* __restrict__ descs,
                                                              WorkList wl) {
  using S = typename E::storage_t;
  constexpr int T = kEwTile;
  __shared__ S sT[T][T + 1];
  const int bid = blockIdx.x;
  const int item = find_item(wl, bid);
  const MatDesc d = descs[wl.mat[item]];
  const int local = bid - wl.begin[item];
  const int r0 = (local / d.ew_tiles_j) * T, c0 = (local % d.ew_tiles_j) * T;
  const S* G = static_cast<const S*>(d.G);
  S* Xg = static_cast<S*>(d.X0);
  S* Xt = static_cast<S*>(d.X1);
  const S zero = E::from_f32(0.f);
  for (int e = threadIdx.x; e < T * T; e += kThreads) {
    const int r = e / T, c = e % T;
    const int gr = r0 + r, gc = c0 + c;
    const S v = (gr < d.rows && gc < d.cols) ? G[static_cast<size_t>(gr) * d.cols + gc] : zero;
    Xg[iter_off<E>(gr, gc, d.n_pad)] = v;
    sT[r][c] = v;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < T * T; e += kThreads) {
    const int c = e / T, r = e % T;
    Xt[iter_off<E>(c0 + c, r0 + r, d.m_pad)] = sT[r][c];
  }
}

}  // namespace mfsdp

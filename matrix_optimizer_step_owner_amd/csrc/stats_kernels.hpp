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
// ew_tiles_j = c_pad / 64.  When every row of G starts on 16 bytes (an aligned
// base and a multiple of 16 bytes per row), G is read and both copies written
// in 16-byte vectors: eight bf16 (four fp32) columns from a multiple of eight
// (four) are contiguous in the iter_off layout too.  The tile goes through
// LDS for the transposed copy.
template <class E>
__global__ __launch_bounds__(kThreads) void stats_prep_kernel(const MatDesc* __restrict__ descs,
                                                              WorkList wl) {
  using S = typename E::storage_t;
  constexpr int T = kEwTile;
  constexpr int V = E::kVec;
  __shared__ S sT[T][T + 1];
  const int bid = blockIdx.x;
  const int item = find_item(wl, bid);
  const MatDesc d = descs[wl.mat[item]];
  const int local = bid - wl.begin[item];
  const int r0 = (local / d.ew_tiles_j) * T, c0 = (local % d.ew_tiles_j) * T;
  const S* G = static_cast<const S*>(d.G);
  S* Xg = static_cast<S*>(d.X0);
  S* Xt = static_cast<S*>(d.X1);
  const bool vec = (d.cols % V) == 0 && (reinterpret_cast<uintptr_t>(G) & 15) == 0;
  if (vec) {
    constexpr int VPR = T / V;   // vectors per tile row
    for (int e = threadIdx.x; e < T * VPR; e += kThreads) {
      const int r = e / VPR, c = (e % VPR) * V;
      const int gr = r0 + r, gc = c0 + c;
      // cols is a multiple of V: a vector is wholly inside G or wholly outside
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      if (gr < d.rows && gc < d.cols) raw = gld<uint4>(G + static_cast<size_t>(gr) * d.cols + gc);
      gst<uint4>(Xg + iter_off<E>(gr, gc, d.n_pad), raw);
      S w[V];
      __builtin_memcpy(w, &raw, sizeof(w));
#pragma unroll
      for (int k = 0; k < V; ++k) sT[r][c + k] = w[k];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < T * VPR; e += kThreads) {
      const int c = e / VPR, r = (e % VPR) * V;
      S w[V];
#pragma unroll
      for (int k = 0; k < V; ++k) w[k] = sT[r + k][c];
      uint4 raw;
      __builtin_memcpy(&raw, w, sizeof(raw));
      gst<uint4>(Xt + iter_off<E>(c0 + c, r0 + r, d.m_pad), raw);
    }
    return;
  }
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

// Newton-Schulz for small matrices, whole in one workgroup's LDS.
//
// A matrix whose wide iterate X (m x n, m = min(rows, cols) <= kSmallMaxM) and
// the two m x m products A and B fit in LDS at once runs every iteration of
// its Newton-Schulz chain, and the final apply, in one workgroup: the
// products are fp32 dot products on the vector ALUs, read from LDS, instead
// of 256 x 256 MFMA tiles (which pad a 64 x 128 matrix sixteen-fold) spread
// over three launches per iteration.  The iteration is the one of the tiled
// path:
//   A  = alpha_A X X^T             (alpha_A = s^2 on the first iteration)
//   B' = a I + b A + c A A         (c == 0: B' = a I + b A)
//   X' = alpha_X B' X              (alpha_X = s on the first iteration)
// with X, A and B' rounded to the storage dtype between products (bf16:
// round to nearest even) and fp32 accumulation; the last X' is not rounded
// before the apply, W <- decay W - lr*scale*O.  Which path a matrix takes
// depends on its shape alone, so results do not depend on the list.
#pragma once

#include "common.hpp"

namespace mfsdp {

// Largest m of the small path, and its LDS budget.  Rows are stored with K
// padded to a multiple of four (zeros) and an odd number of 16-byte chunks
// per row, so that 16-byte reads of consecutive rows hit different banks:
// X is m4 x px, A and B' are m4 x pa (m4 = m rounded up to 4).
constexpr int kSmallMaxM = 128;
constexpr int kSmallLdsFloats = 38400;   // 150 KB

__host__ __device__ constexpr int64_t small_pitch(int64_t cols) {
  return 4 * ((((cols + 3) / 4)) | 1);
}

__host__ __device__ constexpr int64_t small_lds_floats(int64_t m, int64_t n) {
  return ((m + 3) / 4 * 4) * (small_pitch(n) + 2 * small_pitch(m));
}

// Threads of the small-matrix workgroup (8 waves, two per SIMD, each with
// room for 256 registers) and the four-by-four output blocks of X' each one
// holds at most.
constexpr int kSmallThreads = 512;
constexpr int kSmallBlocksPerThread = 2;

__host__ __device__ constexpr bool small_path(int64_t m, int64_t n) {
  return m <= kSmallMaxM && small_lds_floats(m, n) <= kSmallLdsFloats &&
         ((m + 3) / 4) * ((n + 3) / 4) <= kSmallBlocksPerThread * kSmallThreads;
}

struct SmallNsArgs {
  const int32_t* mats;   // indices of the small matrices, one per workgroup
  float a, b, c;
  int ns_steps;
  float decay;           // 1 - lr*wd
};

// LDS float (32-bit addresses, ds_* instructions) and four of them.
typedef MFSDP_LDS float lds_float;
typedef MFSDP_LDS f32x4_t lds_f32x4;

template <class E>
__device__ __forceinline__ float small_round(float v) {
  if constexpr (E::kVec == 8) return bf16_to_f32(f32_to_bf16_rne(v));
  return v;
}

__device__ __forceinline__ f32x4_t ld4(const lds_float* p) {
  return *reinterpret_cast<const lds_f32x4*>(p);
}

// out[i][j] = alpha * sum_k P[i][k] * Q[j][k] (+ beta * R[i][j] + diag on i == j)
// for i < M, j < N, k < K4 (a multiple of four; padded columns are zero).
// A thread holds rows i0..i0+3 and the interleaved columns j = bj + t*nbj
// (t = 0..3), so the 16-byte Q reads of neighbouring threads are neighbouring
// rows.  Results are rounded to the storage dtype (bf16: to nearest even).
template <class E>
__device__ __forceinline__ void small_nt(lds_float* out, int po, const lds_float* P, int pp,
                                         const lds_float* Q, int pq, int M, int N, int K4,
                                         float alpha, const lds_float* R, int pr, float beta,
                                         float diag) {
  const int nbi = (M + 3) >> 2, nbj = (N + 3) >> 2;
  for (int blk = threadIdx.x; blk < nbi * nbj; blk += kSmallThreads) {
  const int i0 = (blk / nbj) << 2, bj = blk % nbj;
  float acc[4][4] = {};
  const lds_float* p[4];
  const lds_float* q[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    p[r] = P + min(i0 + r, M - 1) * pp;
    q[r] = Q + min(bj + r * nbj, N - 1) * pq;
  }
#pragma unroll 1
  for (int k = 0; k < K4; k += 4) {
    f32x4_t pv[4], qv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = ld4(p[r] + k);
      qv[r] = ld4(q[r] + k);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[r][t] = fmaf(pv[r][kk], qv[t][kk], acc[r][t]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + r;
    if (i >= M) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int j = bj + t * nbj;
      if (j >= N) continue;
      float v = alpha * acc[r][t];
      if (R) v = fmaf(beta, R[i * pr + j], v);
      if (i == j) v += diag;
      out[i * po + j] = small_round<E>(v);
    }
  }
  }
}

// X' = alpha * B' X (m x n, K = m4), into registers first, so that X can be
// overwritten after a barrier; a thread holds up to kSmallBlocksPerThread
// blocks of rows i0..i0+3 and columns j0..j0+3.  X' is rounded to the storage dtype unless `round` is false (the
// last iteration, whose O is applied unrounded).
template <class E>
__device__ __forceinline__ void small_update(lds_float* X, int px, const lds_float* Bp, int pb,
                                             int m, int n, float alpha, bool round) {
  const int m4 = (m + 3) & ~3;
  const int nbi = (m + 3) >> 2, nbj = (n + 3) >> 2;
  float acc[kSmallBlocksPerThread][4][4] = {};
#pragma unroll
  for (int u = 0; u < kSmallBlocksPerThread; ++u) {
    const int blk = threadIdx.x + u * kSmallThreads;
    if (blk >= nbi * nbj) break;
    const int i0 = (blk / nbj) << 2, j0 = (blk % nbj) << 2;
#pragma unroll 1
    for (int k = 0; k < m4; k += 4) {
      f32x4_t bv[4], xv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bv[r] = ld4(Bp + min(i0 + r, m - 1) * pb + k);
        xv[r] = ld4(X + (k + r) * px + j0);
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[u][r][t] = fmaf(bv[r][kk], xv[kk][t], acc[u][r][t]);
    }
  }
  __syncthreads();   // every read of X is done
#pragma unroll
  for (int u = 0; u < kSmallBlocksPerThread; ++u) {
    const int blk = threadIdx.x + u * kSmallThreads;
    if (blk >= nbi * nbj) break;
    const int i0 = (blk / nbj) << 2, j0 = (blk % nbj) << 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + r;
      if (i >= m) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int j = j0 + t;
        if (j >= n) continue;
        const float o = alpha * acc[u][r][t];
        X[i * px + j] = round ? small_round<E>(o) : o;
      }
    }
  }
  __syncthreads();
}

// One workgroup per small matrix: the whole Newton-Schulz chain and the apply.
// The iterate X0 holds U (wide layout, iter_off addressing) from the momentum
// kernel; scales[k] = 1 / (||U||_F + eps).
template <class E>
__global__ __launch_bounds__(kSmallThreads) void small_ns_kernel(
    const MatDesc* __restrict__ descs, const float* __restrict__ scales, SmallNsArgs args) {
  using S = typename E::storage_t;
  __shared__ __align__(16) float lds[kSmallLdsFloats];
  const int k = args.mats[blockIdx.x];
  const MatDesc d = descs[k];
  const int m = d.m, n = d.n;
  const int m4 = (m + 3) & ~3, n4 = (n + 3) & ~3;
  const int px = static_cast<int>(small_pitch(n)), pa = static_cast<int>(small_pitch(m));
  lds_float* X = (lds_float*)lds;
  lds_float* A = X + m4 * px;
  lds_float* B = A + m4 * pa;
  const int used = m4 * (px + 2 * pa);
  // zeros in every padding row and column: products read K up to m4 or n4
  for (int e = threadIdx.x; e < used; e += kSmallThreads) X[e] = 0.f;
  __syncthreads();
  const float s = scales[k];
  const S* X0 = static_cast<const S*>(d.X0);
  for (int e = threadIdx.x; e < m * n; e += kSmallThreads) {
    const int i = e / n, j = e % n;
    X[i * px + j] = E::to_f32(gld<S>(X0 + iter_off<E>(i, j, d.n_pad)));
  }
  __syncthreads();
  for (int it = 0; it < args.ns_steps; ++it) {
    const bool first = it == 0;
    const bool last = it + 1 == args.ns_steps;
    small_nt<E>(A, pa, X, px, X, px, m, m, n4, first ? s * s : 1.f, nullptr, 0, 0.f, 0.f);
    __syncthreads();
    if (args.c != 0.f)
      small_nt<E>(B, pa, A, pa, A, pa, m, m, m4, args.c, A, pa, args.b, args.a);
    else
      small_nt<E>(B, pa, A, pa, A, pa, m, m, 0, 0.f, A, pa, args.b, args.a);
    __syncthreads();
    small_update<E>(X, px, B, pa, m, n, first ? s : 1.f, !last);
  }
  // Apply O = X (wide (i, j) is stored (i, j), or (j, i) for a tall matrix):
  // W <- decay*W - lr*scale*O, and update_out <- O.
  S* W = static_cast<S*>(d.W);
  for (int e = threadIdx.x; e < m * n; e += kSmallThreads) {
    const int i = e / n, j = e % n;
    const float o = X[i * px + j];
    const size_t off = d.tall ? static_cast<size_t>(j) * d.cols + i
                              : static_cast<size_t>(i) * d.cols + j;
    const float w = E::to_f32(gld<S>(W + off));
    gst<S>(W + off, E::from_f32(fmaf(-d.lr_scale, o, args.decay * w)));
    if (d.upd) gst<float>(d.upd + off, o);
  }
}

}  // namespace mfsdp

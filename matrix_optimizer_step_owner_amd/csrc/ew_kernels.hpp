// Elementwise kernels of the owner-local step: momentum + Nesterov + norm
// partials (written in the wide Newton-Schulz layout), per-matrix norm
// finalization, the apply used when no Newton-Schulz iteration runs, and the
// AdamW tail.  All are HBM-bound; loads and stores are 16-byte vectors where
// the row alignment allows it.
#pragma once

#include "common.hpp"

namespace mfsdp {

// Momentum M' = beta*M + G, Nesterov U = G + beta*M' (or U = M'), sum of U^2
// per block, and U stored into X0 in wide layout (transposed when rows > cols;
// iter_off addressing),
// zero in the tile padding.  A block is 64 stored rows x 128 stored columns
// (kEwRows x kEwCols) and owns one partial sum of U^2; one 256-thread
// workgroup covers kEwSub consecutive blocks of one matrix, with every load of
// all of them issued before the first store.  `wl` lists, per matrix, its
// workgroups (ceil(blocks / kEwSub) of them).
template <class E>
__global__ __launch_bounds__(kThreads) void momentum_kernel(
    const MatDesc* __restrict__ descs, WorkList wl, double* __restrict__ partials,
    float beta, int nesterov) {
  using S = typename E::storage_t;
  constexpr int V = E::kVec;
  constexpr int SR = kEwRows, SC = kEwCols;
  constexpr int SUB = kEwSub;
  // U staged in the storage type (values rounded as X0 stores them): 16.6 KB
  // per block in bf16.  Rows padded to 65 (bf16) or 129 (fp32) 4-byte words:
  // both the row-wise writes and the column-wise reads are free of bank
  // conflicts.
  constexpr int kPad = 4 / static_cast<int>(sizeof(S));
  __shared__ S sU[SUB][SR][SC + kPad];
  __shared__ float sRed[SUB][kThreads / 64];
  // 16 bytes of staged storage elements -> one vector
  auto pack_raw = [](const S (&w)[V]) -> uint4 {
    if constexpr (V == 8) {
      return make_uint4(w[0] | (static_cast<uint32_t>(w[1]) << 16),
                        w[2] | (static_cast<uint32_t>(w[3]) << 16),
                        w[4] | (static_cast<uint32_t>(w[5]) << 16),
                        w[6] | (static_cast<uint32_t>(w[7]) << 16));
    } else {
      return make_uint4(__float_as_uint(w[0]), __float_as_uint(w[1]), __float_as_uint(w[2]),
                        __float_as_uint(w[3]));
    }
  };

  const int bid = blockIdx.x;
  const int item = find_item(wl, bid);
  const MatDesc d = descs[wl.mat[item]];
  const int first = (bid - wl.begin[item]) * SUB;   // first block of this workgroup
  const int nsub = min(SUB, d.ew_ntiles - first);   // blocks it covers (>= 1)
  const int tid = threadIdx.x;

  const S* G = static_cast<const S*>(d.G);
  S* M = static_cast<S*>(d.M);
  S* X0 = static_cast<S*>(d.X0);
  float ssq[SUB];
  int i0s[SUB], j0s[SUB];
#pragma unroll
  for (int q = 0; q < SUB; ++q) {
    ssq[q] = 0.f;
    const int local = first + min(q, nsub - 1);
    const int ti = local / d.ew_tiles_j, tj = local % d.ew_tiles_j;
    i0s[q] = ti * d.ew_th;   // wide block origin
    j0s[q] = tj * d.ew_tw;
  }

  if (d.vec_ok) {
    constexpr int VPR = SC / V;                 // vectors per stored row
    constexpr int NV = SR * VPR / kThreads;     // vectors per thread per block
    // All of this thread's loads first (the stores to M may alias G and M as
    // far as the compiler knows, so interleaving would serialize latency).
    // G, M' and U are streamed (non-temporal); M is loaded through the caches
    // because its line is written back in place.
    uint4 graw[SUB][NV], mraw[SUB][NV];
#pragma unroll
    for (int q = 0; q < SUB; ++q) {
      const int sr0 = d.tall ? j0s[q] : i0s[q], sc0 = d.tall ? i0s[q] : j0s[q];
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e = tid + it * kThreads;
        const int sr = sr0 + e / VPR, sc = sc0 + (e % VPR) * V;
        if (q < nsub && sr < d.rows && sc < d.cols) {
          const size_t off = static_cast<size_t>(sr) * d.cols + sc;
          graw[q][it] = gld_stream(G + off);
          mraw[q][it] = gld<uint4>(M + off);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < SUB; ++q) {
      if (q >= nsub) break;
      const int sr0 = d.tall ? j0s[q] : i0s[q], sc0 = d.tall ? i0s[q] : j0s[q];
#pragma unroll
      for (int it = 0; it < NV; ++it) {
        const int e = tid + it * kThreads;
        const int r = e / VPR, cv = e % VPR;
        const int sr = sr0 + r, sc = sc0 + cv * V;
        float u[V];
        if (sr < d.rows && sc < d.cols) {
          const size_t off = static_cast<size_t>(sr) * d.cols + sc;
          float g[V], mo[V], mn[V];
          Vec16<E>::unpack(graw[q][it], g);
          Vec16<E>::unpack(mraw[q][it], mo);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            mn[k] = fmaf(beta, mo[k], g[k]);
            u[k] = nesterov ? fmaf(beta, mn[k], g[k]) : mn[k];
            ssq[q] = fmaf(u[k], u[k], ssq[q]);
          }
          gst_stream(M + off, Vec16<E>::pack(mn));
        } else {
#pragma unroll
          for (int k = 0; k < V; ++k) u[k] = 0.f;
        }
        if (d.tall) {   // four 4-byte words at word cv*4 of staged row r
          const uint4 pk = Vec16<E>::pack(u);
          uint32_t* row = reinterpret_cast<uint32_t*>(&sU[q][r][0]) + cv * 4;
          row[0] = pk.x;
          row[1] = pk.y;
          row[2] = pk.z;
          row[3] = pk.w;
        } else {  // same layout: straight to X0
          gst_stream(X0 + iter_off<E>(i0s[q] + r, j0s[q] + cv * V, d.n_pad), Vec16<E>::pack(u));
        }
      }
    }
  } else {
    for (int q = 0; q < nsub; ++q) {
      const int sr0 = d.tall ? j0s[q] : i0s[q], sc0 = d.tall ? i0s[q] : j0s[q];
      for (int e = tid; e < SR * SC; e += kThreads) {
        const int r = e / SC, cc = e % SC;
        const int sr = sr0 + r, sc = sc0 + cc;
        float u = 0.f;
        if (sr < d.rows && sc < d.cols) {
          const size_t off = static_cast<size_t>(sr) * d.cols + sc;
          const float g = E::load(G + off);
          const float mn = fmaf(beta, E::load(M + off), g);
          u = nesterov ? fmaf(beta, mn, g) : mn;
          ssq[q] = fmaf(u, u, ssq[q]);
          M[off] = E::from_f32(mn);
        }
        sU[q][r][cc] = E::from_f32(u);
      }
    }
  }
  __syncthreads();

  // Store U into X0 (wide layout, iter_off addressing, padding included):
  // wide row ii of a block is stored row ii (wide) or stored column ii (tall).
  // The vector path of a wide matrix has already stored it.
  for (int q = 0; q < nsub; ++q) {
    if (!d.tall && !d.vec_ok) {
      constexpr int VPR = SC / V;
      for (int e = tid; e < SR * VPR; e += kThreads) {
        const int ii = e / VPR, jv = e % VPR;
        S w[V];
#pragma unroll
        for (int k = 0; k < V; ++k) w[k] = sU[q][ii][jv * V + k];
        gst_stream(X0 + iter_off<E>(i0s[q] + ii, j0s[q] + jv * V, d.n_pad), pack_raw(w));
      }
    } else if (d.tall) {
      constexpr int VPR = SR / V;
      for (int e = tid; e < SC * VPR; e += kThreads) {
        const int ii = e / VPR, jv = e % VPR;
        S w[V];
#pragma unroll
        for (int k = 0; k < V; ++k) w[k] = sU[q][jv * V + k][ii];
        gst_stream(X0 + iter_off<E>(i0s[q] + ii, j0s[q] + jv * V, d.n_pad), pack_raw(w));
      }
    }
  }

  // Deterministic block reductions of the sums of squares, one per block.
#pragma unroll
  for (int q = 0; q < SUB; ++q) {
    const float v = warp_sum(ssq[q]);
    if ((tid & 63) == 0) sRed[q][tid >> 6] = v;
  }
  __syncthreads();
  if (tid < nsub) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) sum += static_cast<double>(sRed[tid][w]);
    partials[d.ew_tile0 + first + tid] = sum;
  }
}

// scale[k] = 1 / (sqrt(sum of matrix k's partials) + eps), summed in a fixed
// order.  One workgroup per matrix.
__global__ __launch_bounds__(kThreads) void norm_finalize_kernel(
    const MatDesc* __restrict__ descs, const double* __restrict__ partials,
    float* __restrict__ scales, float eps) {
  __shared__ double sRed[kThreads / 64];
  const MatDesc d = descs[blockIdx.x];
  double s = 0.0;
  for (int t = threadIdx.x; t < d.ew_ntiles; t += kThreads) s += partials[d.ew_tile0 + t];
  s = warp_sum(s);
  if ((threadIdx.x & 63) == 0) sRed[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) tot += sRed[w];
    scales[blockIdx.x] = static_cast<float>(1.0 / (sqrt(tot) + static_cast<double>(eps)));
  }
}

// Apply with no Newton-Schulz iteration: O = s * U, W <- decay*W - lr*scale*O.
template <class E>
__global__ __launch_bounds__(kThreads) void apply_x0_kernel(
    const MatDesc* __restrict__ descs, WorkList wl, const float* __restrict__ scales,
    float decay) {
  using S = typename E::storage_t;
  const int bid = blockIdx.x;
  const int item = find_item(wl, bid);
  const int k = wl.mat[item];
  const MatDesc d = descs[k];
  const int local = bid - wl.begin[item];
  const int i0 = (local / d.ew_tiles_j) * d.ew_th, j0 = (local % d.ew_tiles_j) * d.ew_tw;
  const float s = scales[k];
  const S* X0 = static_cast<const S*>(d.X0);
  S* W = static_cast<S*>(d.W);
  for (int e = threadIdx.x; e < d.ew_th * d.ew_tw; e += kThreads) {
    const int i = i0 + e / d.ew_tw, j = j0 + e % d.ew_tw;
    if (i >= d.m || j >= d.n) continue;
    const float o = s * E::to_f32(X0[iter_off<E>(i, j, d.n_pad)]);
    const size_t off = d.tall ? static_cast<size_t>(j) * d.cols + i
                              : static_cast<size_t>(i) * d.cols + j;
    W[off] = E::from_f32(fmaf(-d.lr_scale, o, decay * E::to_f32(W[off])));
    if (d.upd) d.upd[off] = o;
  }
}

// Decoupled AdamW on a packed fp32 buffer; 16-byte vectors over n/4 groups,
// the n%4 remainder by the first threads.
struct AdamWArgs {
  float decay;       // 1 - lr*wd
  float beta1, beta2;
  float one_m_beta1, one_m_beta2;
  float step_size;   // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
};

__device__ __forceinline__ void adamw_elem(float& p, float g, float& m, float& v,
                                           const AdamWArgs& a) {
  m = fmaf(a.beta1, m, a.one_m_beta1 * g);
  v = fmaf(a.beta2, v, a.one_m_beta2 * g * g);
  const float denom = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
  p = fmaf(-a.step_size, m / denom, p * a.decay);
}

// Each thread owns U 16-byte groups of every array, kThreads groups apart
// (coalesced per unrolled step); all its loads are issued before any
// arithmetic or store.  g and the new p, m, v are always streamed
// (non-temporal).  Large tails (U = 4) stream the loads of p, m and v too:
// 6.0 against 5.6 TB/s at 2^28 elements.  Small tails (U = 1, more
// workgroups per CU) read p, m and v through the caches, which keeps a tail
// that is still resident in the MALL from the previous step there.
template <int U, bool kStreamState>
__global__ __launch_bounds__(kThreads) void adamw_kernel(
    float* __restrict__ p, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, int64_t n, AdamWArgs a) {
  const int64_t n4 = n >> 2;
  const int64_t q0 = static_cast<int64_t>(blockIdx.x) * (kThreads * U) + threadIdx.x;
  auto ld = [](const float* x) { return kStreamState ? gld_stream(x) : gld<uint4>(x); };
  uint4 pr[U], gr[U], mr[U], vr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t q = q0 + u * kThreads;
    if (q < n4) {
      pr[u] = ld(p + 4 * q);
      gr[u] = gld_stream(g + 4 * q);
      mr[u] = ld(m + 4 * q);
      vr[u] = ld(v + 4 * q);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t q = q0 + u * kThreads;
    if (q < n4) {
      float pp[4], gg[4], mm[4], vv[4];
      Vec16<ElemF32>::unpack(pr[u], pp);
      Vec16<ElemF32>::unpack(gr[u], gg);
      Vec16<ElemF32>::unpack(mr[u], mm);
      Vec16<ElemF32>::unpack(vr[u], vv);
#pragma unroll
      for (int k = 0; k < 4; ++k) adamw_elem(pp[k], gg[k], mm[k], vv[k], a);
      gst_stream(p + 4 * q, Vec16<ElemF32>::pack(pp));
      gst_stream(m + 4 * q, Vec16<ElemF32>::pack(mm));
      gst_stream(v + 4 * q, Vec16<ElemF32>::pack(vv));
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t i = (n4 << 2) + threadIdx.x;
    float pp = p[i], mm = m[i], vv = v[i];
    adamw_elem(pp, g[i], mm, vv, a);
    p[i] = pp;
    m[i] = mm;
    v[i] = vv;
  }
}

// Tails of at least this many 16-byte groups take the unrolled, fully
// streamed kernel (8M elements: 8 workgroups per CU of 4 groups per thread).
constexpr int64_t kAdamLargeGroups = int64_t(1) << 21;

}  // namespace mfsdp

// Newton-Schulz products on MFMA for gfx950.
//
// One Newton-Schulz iteration on a wide m x n iterate X is three grouped
// launches over every owned matrix:
//   gram    A = alpha X X^T          (upper 256x256 tiles, mirrored store)
//   poly    B = b A + c A A          (A symmetric, so A A = A A^T: same core)
//   update  X' = alpha (a X + B X)   (last iteration applies W instead)
// alpha folds the Frobenius normalization into the first iteration: the
// first gram uses the un-normalized U with alpha = s^2 and the first update
// alpha = s, where s = 1 / (||U||_F + eps).
//
// Kernel shape: 256 threads (4 waves) per 256x256 output tile, each wave a
// 128x128 quadrant of 4x4 MFMA 32x32 blocks.  The K loop stages 256 x 128-byte
// panels of both operands in LDS (double buffered, 128 KB), rows XOR-swizzled
// in 16-byte chunks so the fragment reads are bank-conflict free.  The
// K-strided operand of the update (X, read by columns) is transposed in
// registers on its way into LDS, so both LDS panels are K-contiguous.
#pragma once

#include "common.hpp"

namespace mfsdp {

enum NsMode { kModeGram = 0, kModePoly = 1, kModeUpdate = 2 };

struct NsEpi {
  int cur;        // 0: the current iterate is X0, 1: X1
  int first;      // first iteration (apply the normalization factor)
  int last;       // last iteration (apply W and update_out)
  int b_is_A;     // c == 0: the update multiplies A (scaled by kb = b)
  float a, b, c;
  float kb;       // factor of the B X product in the update epilogue
  float decay;    // 1 - lr*wd
};

template <class E>
struct Mma;

template <>
struct Mma<ElemBF16> {
  __device__ __forceinline__ static void run(f32x16_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

template <>
struct Mma<ElemF32> {
  // Lane half h supplies K slot h of each 32x32x2 instruction; element e of
  // the 16-byte vectors feeds instruction e, identically for both operands.
  __device__ __forceinline__ static void run(f32x16_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// 16-byte element `cc` extraction helpers for the register transpose.
template <class E>
struct Transpose;

template <>
struct Transpose<ElemBF16> {
  // in[r] holds row r (8 bf16 along j); out[c] gets column c (8 bf16 along k).
  __device__ __forceinline__ static void run(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t w[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint4& r0 = in[2 * d];
        const uint4& r1 = in[2 * d + 1];
        const uint32_t s0 = (c >> 1) == 0 ? r0.x : (c >> 1) == 1 ? r0.y : (c >> 1) == 2 ? r0.z : r0.w;
        const uint32_t s1 = (c >> 1) == 0 ? r1.x : (c >> 1) == 1 ? r1.y : (c >> 1) == 2 ? r1.z : r1.w;
        w[d] = (c & 1) ? ((s0 >> 16) | (s1 & 0xffff0000u)) : ((s0 & 0xffffu) | (s1 << 16));
      }
      out[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
};

template <>
struct Transpose<ElemF32> {
  __device__ __forceinline__ static void run(const uint4 (&in)[4], uint4 (&out)[4]) {
    out[0] = make_uint4(in[0].x, in[1].x, in[2].x, in[3].x);
    out[1] = make_uint4(in[0].y, in[1].y, in[2].y, in[3].y);
    out[2] = make_uint4(in[0].z, in[1].z, in[2].z, in[3].z);
    out[3] = make_uint4(in[0].w, in[1].w, in[2].w, in[3].w);
  }
};

__device__ __forceinline__ void upper_tile(int local, int T, int& ti, int& tj) {
  int r = 0;
  while (local >= T - r) {
    local -= T - r;
    ++r;
  }
  ti = r;
  tj = r + local;
}

// Eight consecutive storage elements <-> fp32 (one bf16 16-byte vector, or
// two fp32 ones).  `p` must be 16-byte aligned.
template <class E>
__device__ __forceinline__ void load8(const typename E::storage_t* p, float (&v)[8]) {
  if constexpr (E::kVec == 8) {
    Vec16<E>::unpack(gld<uint4>(p), v);
  } else {
    float a[4], b[4];
    Vec16<E>::unpack(gld<uint4>(p), a);
    Vec16<E>::unpack(gld<uint4>(p + 4), b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[k + 4] = b[k];
    }
  }
}

template <class E>
__device__ __forceinline__ void store8(typename E::storage_t* p, const float (&v)[8]) {
  if constexpr (E::kVec == 8) {
    gst<uint4>(p, Vec16<E>::pack(v));
  } else {
    const float a[4] = {v[0], v[1], v[2], v[3]};
    const float b[4] = {v[4], v[5], v[6], v[7]};
    gst<uint4>(p, Vec16<E>::pack(a));
    gst<uint4>(p + 4, Vec16<E>::pack(b));
  }
}

// W <- decay*W - lr*scale*O and update_out <- O for eight consecutive stored
// elements at `off` (row-major in the user layout), `cnt` of them valid.
template <class E>
__device__ __forceinline__ void apply8(const MatDesc& d, size_t off, int cnt, bool vec,
                                       const float (&o)[8], float decay) {
  using S = typename E::storage_t;
  S* W = static_cast<S*>(d.W);
  if (vec && cnt == 8) {
    float w[8];
    load8<E>(W + off, w);
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = fmaf(-d.lr_scale, o[k], decay * w[k]);
    store8<E>(W + off, w);
    if (d.upd) {
      gst<float4>(d.upd + off, make_float4(o[0], o[1], o[2], o[3]));
      gst<float4>(d.upd + off + 4, make_float4(o[4], o[5], o[6], o[7]));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < cnt) {
        const float w = E::to_f32(gld<S>(W + off + k));
        gst<S>(W + off + k, E::from_f32(fmaf(-d.lr_scale, o[k], decay * w)));
        if (d.upd) gst<float>(d.upd + off + k, o[k]);
      }
    }
  }
}

template <class E, int MODE>
__global__ __launch_bounds__(kThreads) void ns_gemm_kernel(
    const MatDesc* __restrict__ descs, WorkList wl, const float* __restrict__ scales,
    NsEpi ep) {
  using S = typename E::storage_t;
  constexpr int V = E::kVec;            // elements per 16-byte chunk
  constexpr int BK = 8 * V;             // K elements per 128-byte panel row
  constexpr int PANEL = kTile * 8;      // uint4 per operand panel

  __shared__ uint4 smem[2][2][PANEL];   // [buffer][operand P/Q][row*8+chunk]

  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  const int item = find_item(wl, bid);
  const int k = wl.mat[item];
  const MatDesc d = descs[k];
  const int local = bid - wl.begin[item];

  int ti, tj;
  if (MODE == kModeUpdate) {
    const int tn = d.n_pad / kTile;
    ti = local / tn;
    tj = local % tn;
  } else {
    upper_tile(local, d.m_pad / kTile, ti, tj);
  }
  const int row0 = ti * kTile, col0 = tj * kTile;

  const S* Xcur = static_cast<const S*>(ep.cur ? d.X1 : d.X0);
  const S* P;
  const S* Q;
  int ldp, ldq, K;
  if (MODE == kModeGram) {
    P = Xcur; Q = Xcur; ldp = ldq = d.n_pad; K = d.n_pad;
  } else if (MODE == kModePoly) {
    P = static_cast<const S*>(d.A); Q = P; ldp = ldq = d.m_pad; K = d.m_pad;
  } else {
    P = static_cast<const S*>(ep.b_is_A ? d.A : d.B); ldp = d.m_pad;
    Q = Xcur; ldq = d.n_pad; K = d.m_pad;
  }

  // ---- global -> register staging -------------------------------------
  // Operand P (and Q for gram/poly): rows of the output tile, K-contiguous.
  const int prow = tid >> 3, pchunk = tid & 7;
  const int pswz = pchunk ^ (prow & 7);
  const S* pbase = P + static_cast<size_t>(row0 + prow) * ldp + pchunk * V;
  const S* qbase_nt = Q + static_cast<size_t>(col0 + prow) * ldq + pchunk * V;
  uint4 rp[8], rq[8];

  auto load_p = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 8; ++q)
      rp[q] = gld<uint4>(pbase + static_cast<size_t>(q * 32) * ldp + k0);
  };
  auto load_q = [&](int k0) {
    if constexpr (MODE != kModeUpdate) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        rq[q] = gld<uint4>(qbase_nt + static_cast<size_t>(q * 32) * ldq + k0);
    } else {
      // V x V element blocks: rows k0 + kb*V + r, columns col0 + jb*V.
#pragma unroll
      for (int h = 0; h < 8 / V; ++h) {
        const int bi = tid + h * kThreads;
        const int kb = bi & 7, jb = bi >> 3;
#pragma unroll
        for (int r = 0; r < V; ++r)
          rq[h * V + r] = gld<uint4>(Q + static_cast<size_t>(k0 + kb * V + r) * ldq + col0 + jb * V);
      }
    }
  };
  auto store_lds = [&](int buf) {
    uint4* sP = smem[buf][0];
    uint4* sQ = smem[buf][1];
#pragma unroll
    for (int q = 0; q < 8; ++q) sP[(q * 32 + prow) * 8 + pswz] = rp[q];
    if constexpr (MODE != kModeUpdate) {
#pragma unroll
      for (int q = 0; q < 8; ++q) sQ[(q * 32 + prow) * 8 + pswz] = rq[q];
    } else {
#pragma unroll
      for (int h = 0; h < 8 / V; ++h) {
        const int bi = tid + h * kThreads;
        const int kb = bi & 7, jb = bi >> 3;
        uint4 in[V], out[V];
#pragma unroll
        for (int r = 0; r < V; ++r) in[r] = rq[h * V + r];
        Transpose<E>::run(in, out);
#pragma unroll
        for (int c = 0; c < V; ++c) {
          const int j = jb * V + c;
          sQ[j * 8 + (kb ^ (j & 7))] = out[c];
        }
      }
    }
  };

  // ---- MFMA main loop -----------------------------------------------------
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int lrow = lane & 31, lhalf = lane >> 5;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int nk = K / BK;
  load_p(0);
  load_q(0);
  store_lds(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_p((kt + 1) * BK);
      load_q((kt + 1) * BK);
    }
    const uint4* sP = smem[cur][0];
    const uint4* sQ = smem[cur][1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int ch = (2 * s + lhalf) ^ (lrow & 7);
      uint4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = sP[(wr * 128 + i * 32 + lrow) * 8 + ch];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = sQ[(wc * 128 + j * 32 + lrow) * 8 + ch];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mma<E>::run(acc[i][j], fa[i], fb[j]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue through LDS -------------------------------------------------
  // acc[i][j][r] sits at tile row wr*128 + i*32 + (r/4)*8 + lhalf*4 + r%4,
  // tile column wc*128 + j*32 + lrow.  For each i, the four waves stage their
  // 32 x 128 slices in LDS (fp32, padded pitch), then all threads process the
  // 64 x 256 block with 16-byte row-contiguous global accesses; a second,
  // column-wise pass writes the mirrored tile of a symmetric product or the
  // transposed apply of a tall matrix.
  constexpr int SP = 132;               // staged row pitch in floats
  constexpr int WREG = 32 * SP;         // floats per wave slice
  float* stage = reinterpret_cast<float*>(&smem[0][0][0]);
  const float s_norm = scales[k];
  const bool sym = MODE != kModeUpdate;
  const bool mirror = sym && ti != tj;
  const bool tall_apply = MODE == kModeUpdate && ep.last && d.tall;
  const float alpha = MODE == kModeGram ? (ep.first ? s_norm * s_norm : 1.f)
                    : MODE == kModeUpdate ? (ep.first ? s_norm : 1.f) : 1.f;
  S* out = static_cast<S*>(MODE == kModeGram ? d.A : MODE == kModePoly ? d.B
                                             : (ep.cur ? d.X0 : d.X1));
  const int ldo = sym ? d.m_pad : d.n_pad;
  const bool vec = d.vec_ok != 0;

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    {
      float* reg = stage + wave * WREG;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          reg[((r >> 2) * 8 + lhalf * 4 + (r & 3)) * SP + j * 32 + lrow] = acc[i][j][r];
    }
    __syncthreads();

    // Pass A: row-major, eight consecutive columns per thread.
    for (int p = 0; p < 8; ++p) {
      const int it = p * kThreads + tid;
      const int rr = it >> 5, cv = it & 31;
      const int wrr = rr >> 5, r_in = rr & 31, wcc = cv >> 4, c_in = (cv & 15) * 8;
      float* src = stage + (wrr * 2 + wcc) * WREG + r_in * SP + c_in;
      const float4 lo = *reinterpret_cast<const float4*>(src);
      const float4 hi = *reinterpret_cast<const float4*>(src + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int grow = row0 + wrr * 128 + i * 32 + r_in;
      const int gcol = col0 + wcc * 128 + c_in;
      const size_t goff = static_cast<size_t>(grow) * ldo + gcol;
      if (MODE == kModeGram) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= alpha;
      } else if (MODE == kModePoly) {
        float a8[8];
        load8<E>(static_cast<const S*>(d.A) + goff, a8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = fmaf(ep.c, v[e], ep.b * a8[e]);
      } else {
        float x8[8];
        load8<E>(Xcur + goff, x8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = alpha * fmaf(ep.kb, v[e], ep.a * x8[e]);
      }
      if (MODE != kModeUpdate || !ep.last) {
        store8<E>(out + goff, v);
      } else if (!d.tall) {
        if (grow < d.m && gcol < d.n)
          apply8<E>(d, static_cast<size_t>(grow) * d.cols + gcol, min(8, d.n - gcol), vec, v,
                    ep.decay);
      }
      if (mirror || tall_apply) {
        *reinterpret_cast<float4*>(src) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(src + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }

    // Pass B: column-wise, eight consecutive tile rows of one tile column.
    if (mirror || tall_apply) {
      __syncthreads();
      for (int p = 0; p < 8; ++p) {
        const int it = p * kThreads + tid;
        const int tc = it >> 3, q = it & 7;
        const int wrr = q >> 2, sub = q & 3, wcc = tc >> 7, c_in = tc & 127;
        const float* src = stage + (wrr * 2 + wcc) * WREG + (sub * 8) * SP + c_in;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = src[e * SP];
        const int grow0 = row0 + wrr * 128 + i * 32 + sub * 8;
        const int gcol = col0 + tc;
        if (mirror) {
          store8<E>(out + static_cast<size_t>(gcol) * ldo + grow0, v);
        } else if (gcol < d.n && grow0 < d.m) {
          apply8<E>(d, static_cast<size_t>(gcol) * d.cols + grow0, min(8, d.m - grow0), vec, v,
                    ep.decay);
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace mfsdp

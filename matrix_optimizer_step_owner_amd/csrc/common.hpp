// Shared device-side helpers of the owner-local optimizer step (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mfsdp {

// Newton-Schulz output tile (rows and columns) of the MFMA kernels; every
// iterate buffer is padded to a multiple of it.
constexpr int kTile = 256;
// Tile edge of the elementwise momentum kernel (divides kTile).
constexpr int kEwTile = 64;
// Momentum-kernel block in the caller's (stored) layout: 64 rows x 128
// columns, so each row segment is 256 contiguous bytes (bf16).  In the wide
// layout that is 64 x 128 for a wide matrix and 128 x 64 for a tall one.
constexpr int kEwRows = 64;
constexpr int kEwCols = 128;
// Momentum-kernel blocks covered by one workgroup (each keeps its own norm
// partial, so the summation structure does not depend on it).  Two blocks
// keep sixteen 16-byte loads in flight per thread: +2-4% on the Llama-3-8B
// and 32B-class shares over one block, while four lost 5-20% on the small
// shares.
constexpr int kEwSub = 2;
constexpr int kThreads = 256;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32, which also
// keeps NaN a NaN).  Two values per instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Global-address-space accessors.  Pointers that come from descriptors are
// generic; casting them to address space 1 makes the compiler emit global_*
// instructions instead of flat_* ones (flat loads also count against the LDS
// wait counter, which would serialize global prefetch with LDS traffic).
#define MFSDP_GLOBAL __attribute__((address_space(1)))
#define MFSDP_LDS __attribute__((address_space(3)))

typedef short v4i16_t __attribute__((ext_vector_type(4)));


template <class T>
__device__ __forceinline__ T gld(const void* p) {
  return *(const MFSDP_GLOBAL T*)(p);
}

template <class T>
__device__ __forceinline__ void gst(void* p, const T& v) {
  *(MFSDP_GLOBAL T*)(p) = v;
}

// HIP's uint4/float4 are class types; go through clang vector types.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <>
__device__ __forceinline__ uint4 gld<uint4>(const void* p) {
  const u32x4_t v = *(const MFSDP_GLOBAL u32x4_t*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <>
__device__ __forceinline__ void gst<uint4>(void* p, const uint4& v) {
  *(MFSDP_GLOBAL u32x4_t*)(p) = u32x4_t{v.x, v.y, v.z, v.w};
}

template <>
__device__ __forceinline__ float4 gld<float4>(const void* p) {
  const f32x4_t v = *(const MFSDP_GLOBAL f32x4_t*)(p);
  return make_float4(v.x, v.y, v.z, v.w);
}

template <>
__device__ __forceinline__ void gst<float4>(void* p, const float4& v) {
  *(MFSDP_GLOBAL f32x4_t*)(p) = f32x4_t{v.x, v.y, v.z, v.w};
}

// Streaming (non-temporal) 16-byte accesses, for data touched once per step:
// they keep the caches for the data that is re-read.
__device__ __forceinline__ uint4 gld_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const MFSDP_GLOBAL u32x4_t*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void gst_stream(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, (MFSDP_GLOBAL u32x4_t*)(p));
}

// Element traits: storage type, elements per 16-byte vector, conversions.
struct ElemBF16 {
  using storage_t = uint16_t;
  static constexpr int kVec = 8;
  __device__ __forceinline__ static float load(const storage_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static float to_f32(storage_t s) { return bf16_to_f32(s); }
  __device__ __forceinline__ static storage_t from_f32(float f) { return f32_to_bf16_rne(f); }
};

struct ElemF32 {
  using storage_t = float;
  static constexpr int kVec = 4;
  __device__ __forceinline__ static float load(const storage_t* p) { return *p; }
  __device__ __forceinline__ static float to_f32(storage_t s) { return s; }
  __device__ __forceinline__ static storage_t from_f32(float f) { return f; }
};

// Unpack / pack a 16-byte vector of storage elements.
template <class E>
struct Vec16 {
  static constexpr int N = E::kVec;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&out)[N]);
  __device__ __forceinline__ static uint4 pack(const float (&in)[N]);
};

template <>
struct Vec16<ElemBF16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&out)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float (&in)[8]) {
    return make_uint4(pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                      pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7]));
  }
};

template <>
struct Vec16<ElemF32> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&out)[4]) {
    out[0] = __uint_as_float(v.x);
    out[1] = __uint_as_float(v.y);
    out[2] = __uint_as_float(v.z);
    out[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float (&in)[4]) {
    return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]),
                      __float_as_uint(in[2]), __float_as_uint(in[3]));
  }
};

// Element offset of (r, c) in a Newton-Schulz iterate of row length n_pad
// (a multiple of 256; m_pad too).  bf16 iterates are stored in blocks of 256
// rows x 32 columns (16 KB, row-major inside), block (r / 256, c / 32) at
// ((r / 256) * (n_pad / 32) + c / 32) * 8192: one K step of a 256-row Gram
// panel is then one contiguous block, and 32 rows of one column block are 2 KB
// contiguous, so every DMA request of the Gram and update operands covers
// whole 128-byte lines.  Eight consecutive columns from a multiple of eight
// stay contiguous (16-byte vectors).  fp32 iterates are row-major.
template <class E>
__host__ __device__ __forceinline__ size_t iter_off(int64_t r, int64_t c, int64_t n_pad) {
  if constexpr (E::kVec == 8)
    return static_cast<size_t>((((r >> 8) * (n_pad >> 5) + (c >> 5)) << 13) + ((r & 255) << 5) +
                               (c & 31));
  else
    return static_cast<size_t>(r * n_pad + c);
}

// Per-matrix device descriptor, written by the host into the workspace.
// "Wide" coordinates (i < m, j < n) index the Newton-Schulz iterate; a tall
// matrix (rows > cols) maps wide (i, j) to stored (j, i).
struct MatDesc {
  void* W;            // rows x cols, storage dtype
  const void* G;      // rows x cols
  void* M;            // rows x cols
  float* upd;         // rows x cols fp32 or null
  void* X0;           // m_pad x n_pad (iter_off layout): U, then even iterates
  void* X1;           // m_pad x n_pad (iter_off layout): odd iterates
  void* A;            // m_pad x m_pad: X X^T
  void* B;            // m_pad x m_pad: b A + c A A
  int32_t rows, cols;
  int32_t m, n, m_pad, n_pad;
  int32_t tall;
  int32_t ew_tile0;   // first momentum-kernel tile of this matrix
  int32_t ew_tiles_j; // momentum-kernel tiles along the wide n axis
  int32_t ew_ntiles;  // momentum-kernel tiles of this matrix
  int32_t ew_th, ew_tw;  // momentum-kernel tile height / width in the wide layout
  float lr_scale;     // lr * scale
  int32_t vec_ok;     // rows of W/G/M/upd start 16-byte aligned
};

// Grouped launch: work item p covers tiles [begin[p], begin[p+1]) of matrix
// mat[p].  Each workgroup finds its item by binary search.
struct WorkList {
  const int32_t* mat;
  const int32_t* begin;  // n_items + 1 entries
  int32_t n_items;
};

__device__ __forceinline__ int find_item(const WorkList& wl, int32_t bid) {
  int lo = 0, hi = wl.n_items - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (wl.begin[mid] <= bid) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), and each XCD has its own L2.  Remap so that XCD x processes a
// contiguous range of logical tiles, in order: neighbouring tiles (which share
// operand panels) then run on the same XCD and hit in its L2.  A bijection on
// [0, nblocks).
constexpr int kXcds = 8;

__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int x = b % kXcds, i = b / kXcds;
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  return x * q + (x < r ? x : r) + i;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double warp_sum(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace mfsdp

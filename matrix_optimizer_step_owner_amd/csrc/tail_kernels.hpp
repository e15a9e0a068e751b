// Packing of non-matrix tensors into an owner's packed fp32 tail buffer and
// back (gist.science summaries, "Méthodologie", part 1: 1D and other non-2D
// tensors are grouped into a tail assigned to one owner, which keeps AdamW on
// them).  Each segment starts on a 16-byte boundary of the packed buffer;
// packing zero-fills the gap up to the next segment, so AdamW over the whole
// buffer leaves the gaps at zero.
#pragma once

#include "common.hpp"

namespace mfsdp {

constexpr int kTailSegs = 64;          // segments per launch (kernel-argument table)
constexpr int kTailBlockElems = 4096;  // elements per workgroup (16 per thread)

struct TailSeg {
  const float* src;
  float* dst;
  int64_t n;      // elements copied from src
  int64_t span;   // elements written at dst (n, or n rounded up to 4 when packing)
};

struct TailBatch {
  TailSeg seg[kTailSegs];
  int64_t block0[kTailSegs + 1];   // first workgroup of each segment; block0[count] = total
  int32_t count;
};

// One workgroup copies kTailBlockElems elements of one segment: 16-byte
// accesses when both sides are 16-byte aligned, else 4-byte ones.
__global__ __launch_bounds__(kThreads) void tail_copy_kernel(TailBatch b) {
  const int64_t blk = blockIdx.x;
  int s = 0;
  while (s + 1 < b.count && b.block0[s + 1] <= blk) ++s;
  const TailSeg g = b.seg[s];
  const int64_t base = (blk - b.block0[s]) * kTailBlockElems;
  const int64_t end = min(base + static_cast<int64_t>(kTailBlockElems), g.span);
  const bool vec = ((reinterpret_cast<uintptr_t>(g.src) | reinterpret_cast<uintptr_t>(g.dst)) & 15) == 0;
  if (vec) {
    for (int64_t e = base + 4 * threadIdx.x; e < end; e += 4 * kThreads) {
      float4 v;
      if (e + 4 <= g.n) {
        v = gld<float4>(g.src + e);
      } else {
        v.x = e + 0 < g.n ? g.src[e + 0] : 0.f;
        v.y = e + 1 < g.n ? g.src[e + 1] : 0.f;
        v.z = e + 2 < g.n ? g.src[e + 2] : 0.f;
        v.w = e + 3 < g.n ? g.src[e + 3] : 0.f;
      }
      if (e + 4 <= end) {
        gst<float4>(g.dst + e, v);
      } else {
        const float t[4] = {v.x, v.y, v.z, v.w};
        for (int q = 0; q < 4 && e + q < end; ++q) g.dst[e + q] = t[q];
      }
    }
  } else {
    for (int64_t e = base + threadIdx.x; e < end; e += kThreads)
      g.dst[e] = e < g.n ? g.src[e] : 0.f;
  }
}

}  // namespace mfsdp

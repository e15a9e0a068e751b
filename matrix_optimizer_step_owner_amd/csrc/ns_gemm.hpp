// Newton-Schulz products on MFMA for gfx950.
//
// One Newton-Schulz iteration on a wide m x n iterate X is three grouped
// launches over every owned matrix:
//   gram    A = alpha X X^T              (upper 256x256 tiles, mirrored store)
//   poly    B' = a I + b A + c A A       (A symmetric, so A A = A A^T: same core)
//   update  X' = alpha B' X              (last iteration applies W instead)
// (with c = 0 the poly launch is skipped and the update computes
// X' = alpha (a X + b A X)).  alpha folds the Frobenius normalization into
// the first iteration: the first gram uses the un-normalized U with
// alpha = s^2 and the first update alpha = s, where s = 1 / (||U||_F + eps).
//
// Kernel shape: one workgroup per 256x256 output tile, 8 waves, each a
// 128x64 block of 4x2 MFMA 32x32 tiles.  Operand panels (one K step: 64
// bf16 or 32 fp32 per row) go from global memory straight into LDS
// (global_load_lds_dwordx4, no register staging) in four 32 KB stages; in
// bf16 every panel comes from a blocked matrix (iter_off) by whole 128-byte
// lines.  K-contiguous panel rows are XOR-swizzled in 16-byte chunks so
// fragment reads are free of bank conflicts.  The update's X, read along K,
// is read with the gfx950 transposing LDS load (ds_read_b64_tr_b16), which
// hands each lane four consecutive K values of its own column.  The
// epilogue stages the accumulators through the freed stages in 64-row
// blocks for 16-byte, whole-line stores: in bf16, column-major and already
// rounded, where the output is a plain scaling (Gram, folded update); in
// fp32 otherwise.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mfsdp {

// kModeUpdate writes the next iterate.  The update of the last iteration
// applies W (and update_out) instead: kModeApplyWide for matrices stored
// wide (rows <= cols, row-major apply), kModeApplyTall for tall ones (the
// transposed apply).  Separate kernels keep each one's code small: the
// epilogue runs once per tile and is fetched into the instruction cache anew.
// kModeSyrk is the Gram product of a padded gradient accumulated into a
// caller's fp32 statistics matrix (Shampoo-type preconditioner statistics):
// out <- b*out + a*X X^T over the valid m x m block (NsEpi a, b), the upper
// tiles computed and mirrored.
enum NsMode {
  kModeGram = 0,
  kModePoly = 1,
  kModeUpdate = 2,
  kModeApplyWide = 3,
  kModeApplyTall = 4,
  kModeSyrk = 5
};

// out <- beta*out + alpha*v for the elements of a row segment that lie inside
// the valid m x m block (fp32, row pitch m).  beta == 0 ignores the old value.
__device__ __forceinline__ void syrk_acc8(float* out, int m, int row, int col0,
                                          const float (&v)[8], float alpha, float beta) {
  if (row >= m) return;
  float* q0 = out + static_cast<size_t>(row) * m + col0;
  if (col0 + 8 <= m && ((reinterpret_cast<uintptr_t>(q0) & 15) == 0)) {
    float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
    if (beta != 0.f) {
      lo = gld<float4>(q0);
      hi = gld<float4>(q0 + 4);
    }
    gst<float4>(q0, make_float4(fmaf(beta, lo.x, alpha * v[0]), fmaf(beta, lo.y, alpha * v[1]),
                                fmaf(beta, lo.z, alpha * v[2]), fmaf(beta, lo.w, alpha * v[3])));
    gst<float4>(q0 + 4, make_float4(fmaf(beta, hi.x, alpha * v[4]), fmaf(beta, hi.y, alpha * v[5]),
                                    fmaf(beta, hi.z, alpha * v[6]), fmaf(beta, hi.w, alpha * v[7])));
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (col0 + e < m) {
      float* q = out + static_cast<size_t>(row) * m + col0 + e;
      *q = beta == 0.f ? alpha * v[e] : fmaf(beta, *q, alpha * v[e]);
    }
  }
}

struct NsEpi {
  int cur;        // 0: the current iterate is X0, 1: X1
  int first;      // first iteration (apply the normalization factor)
  int b_is_A;     // c == 0: the update multiplies A (scaled by kb = b)
  int fold;       // the poly stores B' = aI + bA + cA^2, so the update is
                  // X' = B'X with no read of X in its epilogue
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

// Eight consecutive storage elements as raw 16-byte words (bf16: a only).
struct Raw8 {
  uint4 a, b;
};

template <class E>
__device__ __forceinline__ Raw8 load_raw8(const typename E::storage_t* p) {
  Raw8 r;
  r.a = gld<uint4>(p);
  if constexpr (E::kVec == 4)
    r.b = gld<uint4>(p + 4);
  else
    r.b = make_uint4(0, 0, 0, 0);
  return r;
}

template <class E>
__device__ __forceinline__ void unpack_raw8(const Raw8& r, float (&v)[8]) {
  if constexpr (E::kVec == 8) {
    Vec16<E>::unpack(r.a, v);
  } else {
    float a[4], b[4];
    Vec16<E>::unpack(r.a, a);
    Vec16<E>::unpack(r.b, b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[k + 4] = b[k];
    }
  }
}

// W <- decay*W - lr*scale*O and update_out <- O for eight consecutive stored
// elements at `off` (row-major in the user layout); `w` holds their current
// values (loaded beforehand).
template <class E>
__device__ __forceinline__ void apply8_vec(const MatDesc& d, size_t off, const Raw8& w,
                                           const float (&o)[8], float decay) {
  using S = typename E::storage_t;
  float wv[8];
  unpack_raw8<E>(w, wv);
#pragma unroll
  for (int k = 0; k < 8; ++k) wv[k] = fmaf(-d.lr_scale, o[k], decay * wv[k]);
  store8<E>(static_cast<S*>(d.W) + off, wv);
  if (d.upd) {
    gst<float4>(d.upd + off, make_float4(o[0], o[1], o[2], o[3]));
    gst<float4>(d.upd + off + 4, make_float4(o[4], o[5], o[6], o[7]));
  }
}

// Same for `cnt` (< 8 or unaligned) elements, one at a time.
template <class E>
__device__ __forceinline__ void apply8_scalar(const MatDesc& d, size_t off, int cnt,
                                              const float (&o)[8], float decay) {
  using S = typename E::storage_t;
  S* W = static_cast<S*>(d.W);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < cnt) {
      const float w = E::to_f32(gld<S>(W + off + k));
      gst<S>(W + off + k, E::from_f32(fmaf(-d.lr_scale, o[k], decay * w)));
      if (d.upd) gst<float>(d.upd + off + k, o[k]);
    }
  }
}

// One wave-wide global -> LDS copy of 64 x 16 bytes (global_load_lds_dwordx4):
// lane l reads 16 bytes at sbase + voff and writes them to LDS at
// lds + 16*l.  Issued as inline assembly so that the compiler does not track
// it: its wait-count pass cannot tell the pipeline stages apart and would
// wait for every DMA in flight before each LDS read.  The kernel waits for
// these copies itself (vmcnt) before the block barriers that publish them.
// M0 holds the LDS base; nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_dma16(uint32_t lds, uint32_t voff, const void* sbase) {
  // The base is wave-uniform; make that explicit so it lives in SGPRs.
  // readfirstlane returns a signed int: widen through uint32_t, never
  // directly (a sign extension would corrupt the high word of any address
  // whose bit 31 is set).
  const uint64_t b = reinterpret_cast<uintptr_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint64_t ub = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  // One wait state between the SALU write of M0 and the LDS DMA that reads it
  // (a GFX9 hazard that the hardware does not interlock).
  const uint32_t ulds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(ulds), "v"(voff), "s"(ub) : "memory", "m0");
}

// LDS byte address of a __shared__ object (a link-time constant).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((MFSDP_LDS const void*)p));
}

// XOR swizzle of the 16-byte chunks of a K-contiguous LDS panel row (64 bytes).
// The LDS serves 16 lanes x 16 bytes per cycle from 64 banks, i.e. four panel
// rows per bank row; a fragment read touches 16 consecutive rows at one
// chunk, which (row >> 2) & 3 spreads over all 16 bank groups.
__device__ __forceinline__ int kswz(int row) { return (row >> 2) & 3; }

// Eight waves per 256x256 tile, two per SIMD, each wave a 128 x 64 block of
// 4x2 MFMA 32x32 tiles (128 accumulator registers, ~250 VGPRs in all).  With
// two waves per SIMD, one wave's stalls (an LDS instruction it cannot issue
// yet, its epilogue loads, staging and stores) leave the MFMA pipe to the
// other.
constexpr int kNsWaves = 8;
constexpr int kNsThreads = 64 * kNsWaves;
constexpr int kWaveCols = 2 * kTile / kNsWaves;   // 64 output columns per wave
constexpr int kWaveColsLog2 = 6;
constexpr int kWaveRowLog2 = 2;                   // wave index -> 128-row half
static_assert(kWaveCols == 1 << kWaveColsLog2 && kNsWaves / 2 == 1 << kWaveRowLog2, "powers of two");
constexpr int kBJ = kWaveCols / 32;               // 32-column MFMA blocks per wave
constexpr int kSlots = 4 * kBJ;                   // MFMAs per wave per K sub-step
constexpr int kPieces = 32 / kNsWaves;            // 1 KB DMA pieces per wave per K step
constexpr int kPPW = kPieces / 2;                 // of them per operand panel
constexpr int kEpIt = 64 * kTile / 8 / kNsThreads;   // epilogue 8-element groups per thread

// Which DMA piece (0..2*bj-1, or -1 for none) a K step issues in MFMA slot
// idx of sub-step sub, for waves with bj 32-column blocks: the pieces of a
// stage are spread over the step, one every fourth MFMA slot of both
// sub-steps, so that the vector-memory queue never holds up the MFMA issue
// for long.  The waves of a CU share one texture addresser: issuing a step's
// pieces in a burst (the first eight slots of sub-step 0) kept it busy long
// enough to stall MFMA issue and was 3% slower on the d=2048 block.
__host__ __device__ constexpr int dma_slot_piece(int bj, int sub, int idx) {
  return (idx & 3) == 0 ? bj * sub + idx / 4 : -1;
}

// Tile rows per band of the update's tile order (see ns_gemm_kernel).
constexpr int kUpdBandRows = 4;

template <class E, int MODE>
__global__ __launch_bounds__(kNsThreads) void ns_gemm_kernel(
    const MatDesc* __restrict__ descs, const int2* __restrict__ tiles,
    const float* __restrict__ scales, NsEpi ep) {
  using S = typename E::storage_t;
  constexpr int V = E::kVec;            // elements per 16-byte chunk
  constexpr int BK = 4 * V;             // K elements per 64-byte panel row
  constexpr int PANEL = kTile * 4;      // uint4 per operand panel (16 KB)
  constexpr int kStages = 4;            // LDS pipeline depth (4 x 32 KB)

  // Pipeline stages, each holding the P panel then the Q panel.  Separate
  // objects so that the compiler can tell a DMA into one stage from reads of
  // another and does not serialize them.
  __shared__ uint4 st0[2 * PANEL];
  __shared__ uint4 st1[2 * PANEL];
  __shared__ uint4 st2[2 * PANEL];
  __shared__ uint4 st3[2 * PANEL];

  const int tid = threadIdx.x;
  // tiles[b] = (matrix, tile index within it) of logical tile b
  const int2 tile = tiles[xcd_remap(blockIdx.x, gridDim.x)];
  const int k = tile.x;
  const int local = tile.y;
  const MatDesc d = descs[k];

  constexpr bool kApply = MODE == kModeApplyWide || MODE == kModeApplyTall;
  constexpr bool kUpd = MODE == kModeUpdate || kApply;
  int ti, tj;
  if (kUpd) {
    // Bands of kUpdBandRows tile rows, walked column by column: the tiles an
    // XCD runs together then share few operand panels (4 B' row panels and 8
    // X column panels for 32 tiles, against 2 and 22 in row-major order),
    // which cut the update time by 14% on the Llama-3-8B share.
    const int tn = d.n_pad / kTile, tm = d.m_pad / kTile;
    const int band = local / (kUpdBandRows * tn), r = local - band * (kUpdBandRows * tn);
    const int rows = min(kUpdBandRows, tm - band * kUpdBandRows);
    ti = band * kUpdBandRows + r % rows;
    tj = r / rows;
  } else {
    upper_tile(local, d.m_pad / kTile, ti, tj);
  }
  const int row0 = ti * kTile, col0 = tj * kTile;

  const S* Xcur = static_cast<const S*>(ep.cur ? d.X1 : d.X0);
  const S* P;
  const S* Q;
  int ldp, ldq, K;
  if (MODE == kModeGram || MODE == kModeSyrk) {
    P = Xcur; Q = Xcur; ldp = ldq = d.n_pad; K = d.n_pad;
  } else if (MODE == kModePoly) {
    P = static_cast<const S*>(d.A); Q = P; ldp = ldq = d.m_pad; K = d.m_pad;
  } else {
    P = static_cast<const S*>(ep.b_is_A ? d.A : d.B); ldp = d.m_pad;
    Q = Xcur; ldq = d.n_pad; K = d.m_pad;
  }

  // ---- operand panels: global -> LDS by DMA ---------------------------------
  // Each wave issues global_load_lds_dwordx4: lane l's 16 bytes land at
  // LDS base + 16*l, so the lane picks the global chunk that belongs at that
  // swizzled position.  K-contiguous panels: 256 rows x 4 chunks of 16 bytes,
  // chunk c of row r stored at r*4 + (c ^ kswz(r)).
  // In bf16 every Newton-Schulz matrix (X, A and B') is stored in 256 x 32
  // blocks (iter_off), so a K step of a 256-row panel is one contiguous 16 KB
  // block: every P panel, and the Q panel of the Gram and polynomial, arrives
  // by whole 128-byte lines (the texture path that feeds these DMAs is the
  // busiest unit of the K loop on long-K products, and a 64-byte half line
  // costs it as much as a whole one).  The update's Q panel (X read along K,
  // 32 rows of 256 columns) is eight 2 KB runs, one per 32-column block, kept
  // in that order in LDS (column block cb, k-row kk, 16-byte unit u at
  // cb*2048 + kk*64 + u*16) and read with the transposing LDS load.  fp32
  // matrices are row-major: K-contiguous panels read 64-byte row pieces, and
  // the update's X panel is 16 k-rows x 64 chunks, unswizzled.
  constexpr bool kPB = V == 8;                   // P: row panel of a blocked matrix
  constexpr bool kQB = V == 8 && !kUpd;          // Q: row panel of a blocked matrix
  constexpr bool kQT = kUpd;                     // Q read along K (the update's X)
  constexpr bool kUB = kUpd && V == 8;           // ... from the blocked iterate
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> kWaveRowLog2, wc = wave & (kNsWaves / 2 - 1);
  const int lrow = lane & 31, lhalf = lane >> 5;

  // DMA piece q (0..kPieces-1) of one K step, per wave: the first kPPW fill
  // this wave's share of the P panel, the others its share of the Q panel;
  // each piece is one 1 KB wave instruction.  The per-lane byte offset of a
  // piece is fixed for the whole K loop; only the uniform base moves with k0
  // (SGPR base + constant VGPR offset, no address VALU).
  uint32_t doff[kPieces];
#pragma unroll
  for (int q = 0; q < kPieces; ++q) {
    const int u = wave * (kPPW * 64) + (q % kPPW) * 64 + lane;
    const int ld = q < kPPW ? ldp : ldq;
    const int r0 = q < kPPW ? row0 : col0;
    if (q < kPPW ? kPB : kQB) {
      const int row = u >> 2, c = (u & 3) ^ kswz(row);
      doff[q] = static_cast<uint32_t>(((row << 5) + c * V) * sizeof(S));
    } else if (q >= kPPW && kUB) {
      const int cb = u >> 7, kk = (u >> 2) & 31, c = u & 3;
      doff[q] = static_cast<uint32_t>(((cb << 13) + (kk << 5) + c * V) * sizeof(S));
    } else if (!(q < kPPW ? false : kQT)) {
      const int row = u >> 2, c = (u & 3) ^ kswz(row);
      doff[q] = static_cast<uint32_t>((static_cast<size_t>(r0 + row) * ld + c * V) * sizeof(S));
    } else {
      constexpr int UPR = kTile / V;    // 16-byte chunks per k-row
      const int kk = u / UPR, pc = u % UPR;
      const int c = (V == 8) ? (pc ^ (4 * (kk & 3))) : pc;
      doff[q] = static_cast<uint32_t>((static_cast<size_t>(kk) * ld + r0 + c * V) * sizeof(S));
    }
  }
  // Every DMA destination is a link-time constant (the stage object and the
  // piece) plus this wave's uniform offset: no per-lane address work.
  const uint32_t wave_off = static_cast<uint32_t>(wave) * (kPPW * 1024u);
  auto dma_piece = [&](auto stage_c, int k0, int q) {
    constexpr int stage = decltype(stage_c)::value;
    const uint4* sbuf = stage == 0 ? st0 : stage == 1 ? st1 : stage == 2 ? st2 : st3;
    // block (r / 256, c / 32) of a blocked matrix with row length ld
    auto blk = [](int r, int c, int ld) {
      return static_cast<size_t>((r >> 8) * (ld >> 5) + (c >> 5)) << 13;
    };
    const char* base;
    if (q < kPPW)
      base = reinterpret_cast<const char*>(kPB ? P + blk(row0, k0, ldp) : P + k0);
    else if (kQB)
      base = reinterpret_cast<const char*>(Q + blk(col0, k0, ldq));
    else if (!kQT)
      base = reinterpret_cast<const char*>(Q + k0);
    else if (kUB)
      base = reinterpret_cast<const char*>(Q + blk(k0, col0, ldq) + ((k0 & 255) << 5));
    else
      base = reinterpret_cast<const char*>(Q + static_cast<size_t>(k0) * ldq);
    const uint32_t dst = lds_addr(sbuf) + wave_off + (q < kPPW ? 0u : PANEL * 16u) +
                         static_cast<uint32_t>(q % kPPW) * 1024u;
    lds_dma16(dst, doff[q], base);
  };

  // ---- fragments --------------------------------------------------------------
  // Lane l holds, for K sub-step s (0, 1), the 16-byte K-slice 2s + l/32
  // (bf16: K = 8*(2s + l/32) .. +8) of output row l%32 of each 32-row block.
  // Read piece p: 0..3 the P fragments fa[i]; then the Q fragments (NT: one
  // piece per fb[j]; bf16 update: two transposing reads per fb[j]).
  constexpr int kPReads = 4;
  constexpr int kReadPieces = kPReads + ((kQT && V == 8) ? 2 * kBJ : kBJ);
  // Transposing read of half r of the fragment of the update's X panel
  // (chunk-major: consecutive k-rows of a column block are 64 bytes apart and
  // need no swizzle) whose 32 columns start at n_base: within each 16-lane
  // group, lane i points at k-row kb + i/4, columns n0 + 4*(i%4) .. +4; lane j
  // receives column n0 + j at k-rows kb .. kb+3.
  auto tr_read = [&](const uint4* panel, int s, int n_base, int r, uint4& f) {
    const int il = lane & 15;
    const int n = n_base + 16 * ((lane >> 4) & 1) + 4 * (il & 3);
    const int kk = 16 * s + 8 * lhalf + 4 * r + (il >> 2);
    const int byte = (n >> 5) * 2048 + kk * 64 + (((n >> 3) & 3) << 4) + ((n & 7) << 1);
    const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (MFSDP_LDS v4i16_t*)(reinterpret_cast<const char*>(panel) + byte));
    const uint32_t w0 = static_cast<uint16_t>(t[0]) |
                        (static_cast<uint32_t>(static_cast<uint16_t>(t[1])) << 16);
    const uint32_t w1 = static_cast<uint16_t>(t[2]) |
                        (static_cast<uint32_t>(static_cast<uint16_t>(t[3])) << 16);
    if (r == 0) {
      f.x = w0;
      f.y = w1;
    } else {
      f.z = w0;
      f.w = w1;
    }
  };
  auto read_piece = [&](const uint4* buf, int s, int p, uint4 (&fa)[4], uint4 (&fb)[kBJ]) {
    const int c = 2 * s + lhalf;
    if (p < kPReads) {
      const int row = wr * 128 + p * 32 + lrow;
      fa[p] = buf[row * 4 + (c ^ kswz(row))];
      return;
    }
    const uint4* qp = buf + PANEL;
    const int q = p - kPReads;
    if constexpr (!kQT) {
      const int j = q;
      const int row = wc * kWaveCols + j * 32 + lrow;
      fb[j] = qp[row * 4 + (c ^ kswz(row))];
    } else if constexpr (V == 8) {
      tr_read(qp, s, wc * kWaveCols + (q >> 1) * 32, q & 1, fb[q >> 1]);
    } else {
      const int j = q;
      const float* qf = reinterpret_cast<const float*>(qp);
      const int n = wc * kWaveCols + j * 32 + lrow;
      const int kk = 4 * c;
      fb[j] = make_uint4(__float_as_uint(qf[(kk + 0) * kTile + n]),
                         __float_as_uint(qf[(kk + 1) * kTile + n]),
                         __float_as_uint(qf[(kk + 2) * kTile + n]),
                         __float_as_uint(qf[(kk + 3) * kTile + n]));
    }
  };

  f32x16_t acc[4][kBJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kBJ; ++j) acc[i][j] = f32x16_t{};

  uint4 fa[2][4], fb[2][kBJ];

  // One K step t on stage buffer X.  Sub-step 0 issues its kSlots MFMAs one per
  // slot; slot idx also issues fragment reads idx, idx + kSlots, ... of
  // sub-step 1 and (every fourth slot, when DMA) one DMA piece of step
  // t + kStages - 1 into stage Y, the buffer of
  // step t - 1.  Then: wait until the DMA of step t + 1 has landed (the two
  // most recent steps' DMAs may stay in flight), block barrier.  Sub-step 1's
  // MFMAs overlap the fragment reads of step t + 1 from stage N.
  // The barrier also orders every wave's last reads of stage Y (issued before
  // the previous barrier) before the DMA into Y.
  auto kstep = [&](const uint4* X, auto Y, const uint4* N, int k_dma, auto dma_c,
                   auto next_c, auto wait_all_c) {
    constexpr bool do_dma = decltype(dma_c)::value;
    constexpr bool has_next = decltype(next_c)::value;
    constexpr bool wait_all = decltype(wait_all_c)::value;
#pragma unroll
    for (int idx = 0; idx < kSlots; ++idx) {
      Mma<E>::run(acc[idx / kBJ][idx % kBJ], fa[0][idx / kBJ], fb[0][idx % kBJ]);
#pragma unroll
      for (int rp = idx; rp < kReadPieces; rp += kSlots) read_piece(X, 1, rp, fa[1], fb[1]);
      if constexpr (do_dma) {
        if (dma_slot_piece(kBJ, 0, idx) >= 0) dma_piece(Y, k_dma, dma_slot_piece(kBJ, 0, idx));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Block barrier without the release fence of __syncthreads(), which would
    // also wait for the DMAs still in flight; the memory clobber keeps the
    // compiler from moving LDS accesses across it.
    // DMAs that may stay in flight at the barrier of step t: the kPieces of
    // step t - 1 and the half that step t issued before its barrier (step
    // t + 1's must be done).
    static_assert(kPieces == 4, "wait count below: 4 + 2 pieces in flight");
    if constexpr (wait_all)
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int idx = 0; idx < kSlots; ++idx) {
      Mma<E>::run(acc[idx / kBJ][idx % kBJ], fa[1][idx / kBJ], fb[1][idx % kBJ]);
      if constexpr (has_next) {
#pragma unroll
        for (int rp = idx; rp < kReadPieces; rp += kSlots) read_piece(N, 0, rp, fa[0], fb[0]);
      }
      if constexpr (do_dma) {
        if (dma_slot_piece(kBJ, 1, idx) >= 0) dma_piece(Y, k_dma, dma_slot_piece(kBJ, 1, idx));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- main loop: four stages, unrolled by four ----------------------------
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  const int nk = K / BK;                // multiple of 8: K is a multiple of 256
  // prologue: steps 0..2 in flight, wait for step 0
#pragma unroll
  for (int q = 0; q < kPieces; ++q) dma_piece(S0{}, 0, q);
#pragma unroll
  for (int q = 0; q < kPieces; ++q) dma_piece(S1{}, BK, q);
#pragma unroll
  for (int q = 0; q < kPieces; ++q) dma_piece(S2{}, 2 * BK, q);
  // the two later stages (2 x kPieces) may stay in flight
  asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int p = 0; p < kReadPieces; ++p) read_piece(st0, 0, p, fa[0], fb[0]);
  int t = 0;
  for (; t + 8 <= nk; t += 4) {
    kstep(st0, S3{}, st1, (t + 3) * BK, yes{}, yes{}, no{});
    kstep(st1, S0{}, st2, (t + 4) * BK, yes{}, yes{}, no{});
    kstep(st2, S1{}, st3, (t + 5) * BK, yes{}, yes{}, no{});
    kstep(st3, S2{}, st0, (t + 6) * BK, yes{}, yes{}, no{});
  }
  // last four steps: only the first still has a step (nk - 1) to prefetch
  kstep(st0, S3{}, st1, (t + 3) * BK, yes{}, yes{}, yes{});
  kstep(st1, S0{}, st2, 0, no{}, yes{}, yes{});
  kstep(st2, S1{}, st3, 0, no{}, yes{}, yes{});
  kstep(st3, S2{}, st0, 0, no{}, no{}, yes{});
  __syncthreads();

  // ---- epilogue through LDS -------------------------------------------------
  // acc[i][j][r] sits at tile row wr*128 + i*32 + (r/4)*8 + lhalf*4 + r%4,
  // tile column wc*kWaveCols + j*32 + lrow.  For each i, the waves stage their
  // 32 x kWaveCols slices in LDS (fp32), then all threads process the 64 x 256
  // block with 16-byte row-contiguous global accesses (pass A); a second,
  // column-wise pass writes the mirrored tile of a symmetric product or the
  // transposed apply of a tall matrix (pass B).  Every global input of a pass
  // is loaded before its first store: the stores may alias the inputs as far
  // as the compiler knows, so interleaving them would serialize on latency.
  constexpr int SP = kWaveCols;         // staged row pitch in floats
  // column c of staged row r lives at r*SP + (c ^ 4*((r >> 2) & 7))
  auto sidx = [](int r, int c) { return r * SP + (c ^ (((r >> 2) & 7) << 2)); };
  // Two staging halves h = 0, 1, so that block i + 1 is staged while block i
  // is stored: wave slice w (32 x kWaveCols floats, 8 KB) of half h lives in
  // stage array w / 2, at byte offset (w % 2) * 8 KB + h * 16 KB of its 32 KB.
  static_assert(kNsWaves == 8 && 32 * kWaveCols * 4 == 8192, "two 8 KB slices per half stage");
  auto slice_of = [&](int w, int h) -> float* {
    const int sa = w >> 1;
    float* b = reinterpret_cast<float*>(sa == 0 ? st0 : sa == 1 ? st1 : sa == 2 ? st2 : st3);
    return b + (w & 1) * (32 * kWaveCols) + h * (64 * kWaveCols);
  };
  const float s_norm = scales[k];
  constexpr bool sym = !kUpd;
  const bool mirror = sym && ti != tj;
  constexpr bool wide_apply = MODE == kModeApplyWide;
  constexpr bool tall_apply = MODE == kModeApplyTall;
  const float alpha = MODE == kModeGram ? (ep.first ? s_norm * s_norm : 1.f)
                    : kUpd ? (ep.first ? s_norm : 1.f) : 1.f;
  S* out = static_cast<S*>(MODE == kModeGram ? d.A : MODE == kModePoly ? d.B
                                             : (ep.cur ? d.X0 : d.X1));
  const S* ein = MODE == kModePoly ? static_cast<const S*>(d.A) : Xcur;  // epilogue input
  S* W = static_cast<S*>(d.W);
  const int ldo = sym ? d.m_pad : d.n_pad;
  const bool vec = d.vec_ok != 0;

  // bf16 outputs that are a plain scaling of the accumulators -- the Gram,
  // and the update when the polynomial is folded -- are scaled and rounded in
  // registers (bitwise the values the fp32 staging below would store) and
  // staged in bf16, column-major: half the LDS bytes, four consecutive rows
  // of a column per 8-byte write.  A staging half is two quarters of 128 tile
  // columns x 64 staged rows (pitch kQP elements; staged row wr*32 + rr is
  // tile row wr*128 + 32*i + rr of block i), quarter q of half h in stage
  // array 2h + q.  Row segments are read back with the transposing LDS load
  // (16 lanes: 16 consecutive rows, 4 columns each) and the mirror's with
  // plain 8-byte loads; every wave store writes 16 rows x 64 bytes of one
  // 256 x 32 block, i.e. eight whole lines.
  constexpr bool kB16Stage = V == 8 && (MODE == kModeGram || MODE == kModeUpdate);
  if constexpr (kB16Stage) {
    if (MODE == kModeGram || ep.fold) {
      constexpr int kQP = 68;   // staged column pitch (bf16): 8-byte aligned, 34 banks
      auto quarter = [&](int h, int q) -> uint16_t* {
        const int sa = 2 * h + q;
        return reinterpret_cast<uint16_t*>(sa == 0 ? st0 : sa == 1 ? st1 : sa == 2 ? st2 : st3);
      };
      auto stage16 = [&](auto i_c, int h) {
        constexpr int i = decltype(i_c)::value;
        uint16_t* qb = quarter(h, wc >> 1);
#pragma unroll
        for (int j = 0; j < kBJ; ++j) {
          const int cl = (wc & 1) * kWaveCols + j * 32 + lrow;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const uint2 pk = make_uint2(
                pack_bf16x2(alpha * acc[i][j][4 * q4], alpha * acc[i][j][4 * q4 + 1]),
                pack_bf16x2(alpha * acc[i][j][4 * q4 + 2], alpha * acc[i][j][4 * q4 + 3]));
            *reinterpret_cast<uint2*>(qb + cl * kQP + wr * 32 + q4 * 8 + lhalf * 4) = pk;
          }
        }
      };
      const int g = lane >> 4, jl = lane & 15;
      // row segments: unit u = (16 staged rows rg, one 32-column block cb)
      auto pass_rows = [&](auto i_c, int h) {
        constexpr int i = decltype(i_c)::value;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int u = p * kNsWaves + wave;
          const int rg = u >> 3, cb = u & 7;
          const char* qb = reinterpret_cast<const char*>(quarter(h, cb >> 2));
          const int cq = (cb & 3) * 32 + 8 * g;
          uint32_t w[4];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int byte = ((cq + 4 * hh + (jl >> 2)) * kQP + rg * 16 + 4 * (jl & 3)) * 2;
            const v4i16_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (MFSDP_LDS v4i16_t*)(qb + byte));
            w[2 * hh] = static_cast<uint16_t>(t[0]) |
                        (static_cast<uint32_t>(static_cast<uint16_t>(t[1])) << 16);
            w[2 * hh + 1] = static_cast<uint16_t>(t[2]) |
                            (static_cast<uint32_t>(static_cast<uint16_t>(t[3])) << 16);
          }
          const int sr = rg * 16 + jl;
          const int grow = row0 + (sr >> 5) * 128 + i * 32 + (sr & 31);
          const int gcol = col0 + cb * 32 + 8 * g;
          gst<uint4>(out + iter_off<E>(grow, gcol, ldo), make_uint4(w[0], w[1], w[2], w[3]));
        }
      };
      // mirror segments: unit u = (16 tile columns cg, one 32-row half wrr)
      auto pass_mirror = [&](auto i_c, int h) {
        constexpr int i = decltype(i_c)::value;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int u = p * kNsWaves + wave;
          const int cg = u >> 1, wrr = u & 1;
          const int c = cg * 16 + jl;
          const uint16_t* src = quarter(h, c >> 7) + (c & 127) * kQP + wrr * 32 + 8 * g;
          const uint2 lo = *reinterpret_cast<const uint2*>(src);
          const uint2 hi = *reinterpret_cast<const uint2*>(src + 4);
          const int grow_m = row0 + wrr * 128 + i * 32 + 8 * g;
          gst<uint4>(out + iter_off<E>(col0 + c, grow_m, ldo), make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
      };
      using J0 = std::integral_constant<int, 0>;
      using J1 = std::integral_constant<int, 1>;
      using J2 = std::integral_constant<int, 2>;
      using J3 = std::integral_constant<int, 3>;
      // block i + 1 is staged while block i is stored, as below
      stage16(J0{}, 0);
      __syncthreads();
      stage16(J1{}, 1);
      pass_rows(J0{}, 0);
      if (mirror) pass_mirror(J0{}, 0);
      __syncthreads();
      stage16(J2{}, 0);
      pass_rows(J1{}, 1);
      if (mirror) pass_mirror(J1{}, 1);
      __syncthreads();
      stage16(J3{}, 1);
      pass_rows(J2{}, 0);
      if (mirror) pass_mirror(J2{}, 0);
      __syncthreads();
      pass_rows(J3{}, 1);
      if (mirror) pass_mirror(J3{}, 1);
      return;
    }
  }

  // pass A coordinates of iteration p: tile row, tile column, staged slice
  auto coordA = [&](int i, int p, int& grow, int& gcol, int& sl, int& r_in, int& c_in) {
    const int it = p * kNsThreads + tid;
    const int rr = it >> 5, col = (it & 31) * 8;
    const int wrr = rr >> 5, wcc = col >> kWaveColsLog2;
    r_in = rr & 31;
    c_in = col & (kWaveCols - 1);
    sl = (wrr << kWaveRowLog2) + wcc;
    grow = row0 + wrr * 128 + i * 32 + r_in;
    gcol = col0 + col;
  };

  // pass B coordinates of iteration p: eight consecutive tile rows of one
  // tile column
  auto coordB = [&](int i, int p, int& gcol, int& grow0, int& sl, int& sub, int& c_in) {
    const int it = p * kNsThreads + tid;
    const int tc = it >> 3, q = it & 7;
    const int wrr = q >> 2, wcc = tc >> kWaveColsLog2;
    sub = q & 3;
    c_in = tc & (kWaveCols - 1);
    sl = (wrr << kWaveRowLog2) + wcc;
    grow0 = row0 + wrr * 128 + i * 32 + sub * 8;
    gcol = col0 + tc;
  };

  // Global inputs of block i (the iterate or A, and the weights: pass A
  // coordinates for a wide apply, pass B for a tall one), issued one block
  // ahead so that their latency overlaps the previous block's stores.
  auto load_in = [&](auto i_c, Raw8 (&xin)[kEpIt], Raw8 (&win)[kEpIt]) {
    constexpr int i = decltype(i_c)::value;
#pragma unroll
    for (int p = 0; p < kEpIt; ++p) {
      int grow, gcol, sl, r_in, c_in;
      coordA(i, p, grow, gcol, sl, r_in, c_in);
      if (MODE != kModeGram && MODE != kModeSyrk && !(kUpd && ep.fold))
        xin[p] = load_raw8<E>(ein + iter_off<E>(grow, gcol, ldo));
      if (wide_apply && vec && grow < d.m && gcol + 8 <= d.n)
        win[p] = load_raw8<E>(W + static_cast<size_t>(grow) * d.cols + gcol);
      if constexpr (tall_apply && V == 8) {   // fp32: loaded in pass B (registers)
        int bcol, brow0, bsl, bsub, bc_in;
        coordB(i, p, bcol, brow0, bsl, bsub, bc_in);
        if (vec && bcol < d.n && brow0 + 8 <= d.m)
          win[p] = load_raw8<E>(W + static_cast<size_t>(bcol) * d.cols + brow0);
      }
    }
  };

  // This wave's accumulators of row block i (64 x 256 over the workgroup)
  // into staging half h.  i is a compile-time constant in these helpers so
  // that acc stays in registers.
  auto stage_acc = [&](auto i_c, int h) {
    constexpr int i = decltype(i_c)::value;
    float* reg = slice_of(wave, h);
#pragma unroll
    for (int j = 0; j < kBJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        reg[sidx((r >> 2) * 8 + lhalf * 4 + (r & 3), j * 32 + lrow)] = acc[i][j][r];
  };

  // Passes A and B of block i, staged in half h (after a barrier that
  // follows its staging).
  auto passes = [&](auto i_c, int h, const Raw8 (&xin)[kEpIt], const Raw8 (&win)[kEpIt]) {
    constexpr int i = decltype(i_c)::value;
    // Pass A: row-major, eight consecutive columns per thread.
#pragma unroll
    for (int p = 0; p < kEpIt; ++p) {
      int grow, gcol, sl, r_in, c_in;
      coordA(i, p, grow, gcol, sl, r_in, c_in);
      float* slice = slice_of(sl, h);
      float* src_lo = slice + sidx(r_in, c_in);
      float* src_hi = slice + sidx(r_in, c_in + 4);
      const float4 lo = *reinterpret_cast<const float4*>(src_lo);
      const float4 hi = *reinterpret_cast<const float4*>(src_hi);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const size_t goff = iter_off<E>(grow, gcol, ldo);
      if (MODE == kModeGram) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] *= alpha;
      } else if (MODE != kModeSyrk) {
        float x8[8];
        unpack_raw8<E>(xin[p], x8);
        if (MODE == kModePoly) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = fmaf(ep.c, v[e], ep.b * x8[e]);
          if (ep.fold && ti == tj) {   // + aI on the diagonal
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (grow == gcol + e) v[e] += ep.a;
          }
        } else if (ep.fold) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] *= alpha;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = alpha * fmaf(ep.kb, v[e], ep.a * x8[e]);
        }
      }
      if constexpr (MODE == kModeSyrk) {
        syrk_acc8(static_cast<float*>(d.A), d.m, grow, gcol, v, ep.a, ep.b);
      } else if constexpr (!kApply) {
        store8<E>(out + goff, v);
      } else if (wide_apply && grow < d.m && gcol < d.n) {
        const size_t uo = static_cast<size_t>(grow) * d.cols + gcol;
        if (vec && gcol + 8 <= d.n)
          apply8_vec<E>(d, uo, win[p], v, ep.decay);
        else
          apply8_scalar<E>(d, uo, min(8, d.n - gcol), v, ep.decay);
      }
      if (mirror || tall_apply) {
        *reinterpret_cast<float4*>(src_lo) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(src_hi) = make_float4(v[4], v[5], v[6], v[7]);
      }
    }

    // Pass B: column-wise, eight consecutive tile rows of one tile column.
    if (mirror || tall_apply) {
      __syncthreads();
#pragma unroll
      for (int p = 0; p < kEpIt; ++p) {
        int gcol, grow0, sl, sub, c_in;
        coordB(i, p, gcol, grow0, sl, sub, c_in);
        const float* slice = slice_of(sl, h);
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = slice[sidx(sub * 8 + e, c_in)];
        if constexpr (MODE == kModeSyrk) {
          syrk_acc8(static_cast<float*>(d.A), d.m, gcol, grow0, v, ep.a, ep.b);
        } else if constexpr (sym) {
          store8<E>(out + iter_off<E>(gcol, grow0, ldo), v);
        } else if (tall_apply && gcol < d.n && grow0 < d.m) {
          const size_t uo = static_cast<size_t>(gcol) * d.cols + grow0;
          if (vec && grow0 + 8 <= d.m) {
            if constexpr (V == 8)
              apply8_vec<E>(d, uo, win[p], v, ep.decay);
            else
              apply8_vec<E>(d, uo, load_raw8<E>(W + uo), v, ep.decay);
          } else {
            apply8_scalar<E>(d, uo, min(8, d.m - grow0), v, ep.decay);
          }
        }
      }
    }
  };

  // Block i + 1 is loaded and staged (half (i + 1) % 2) before block i's
  // passes read half i % 2; one barrier per block then both frees half i % 2
  // for block i + 2 and publishes half (i + 1) % 2.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  Raw8 xa[kEpIt], wa[kEpIt], xb[kEpIt], wb[kEpIt];
  load_in(I0{}, xa, wa);
  stage_acc(I0{}, 0);
  __syncthreads();
  load_in(I1{}, xb, wb);
  stage_acc(I1{}, 1);
  passes(I0{}, 0, xa, wa);
  __syncthreads();
  load_in(I2{}, xa, wa);
  stage_acc(I2{}, 0);
  passes(I1{}, 1, xb, wb);
  __syncthreads();
  load_in(I3{}, xb, wb);
  stage_acc(I3{}, 1);
  passes(I2{}, 0, xa, wa);
  __syncthreads();
  passes(I3{}, 1, xb, wb);
}

}  // namespace mfsdp

// Host-side owner planner, packed-tail layout and launch tile order.
//
// Source: "MatrixFSDP: communication-free matrix optimizers under ZeRO-3
// parameter sharding" -- arxivlens page, Methodology (a balance-aware owner
// planner assigns ownership by bytes and by work); gist.science summaries,
// "Méthodologie", part 2, first mechanism (a global planner picks owners so
// that resident bytes and optimizer work are balanced across the ranks), and
// part 1 (1D and other non-2D tensors are grouped on a separate tail owner).
//
// The pages give no algorithm.  This planner is greedy longest-processing-
// time-first scheduling (Graham, 1969) with a per-owner byte cap: whole items
// in decreasing predicted cost, each onto the owner that would finish first
// among those that keep their resident bytes under the cap.  Without a
// binding cap its makespan is within (4/3 - 1/(3R)) of the optimum on R
// owners (Graham's bound).
#pragma once

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <numeric>
#include <vector>

namespace mfsdp {

// Byte cap per owner: (1 + slack) * max(total / R, largest item).
inline int64_t owner_byte_cap(const int64_t* bytes, int64_t n, int r, double slack) {
  int64_t total = 0, largest = 0;
  for (int64_t i = 0; i < n; ++i) {
    total += bytes[i];
    largest = std::max(largest, bytes[i]);
  }
  const double base = std::max(static_cast<double>(total) / r, static_cast<double>(largest));
  return static_cast<int64_t>(std::ceil(base * (1.0 + slack)));
}

// Greedy LPT with a byte cap.  Deterministic: ties in cost go to the larger
// item, then the lower index; ties between owners to the lower rank.
inline void plan_lpt(const double* cost, const int64_t* bytes, int64_t n, int r, double slack,
                     int32_t* owner, double* rank_cost, int64_t* rank_bytes) {
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), int64_t(0));
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (cost[a] != cost[b]) return cost[a] > cost[b];
    if (bytes[a] != bytes[b]) return bytes[a] > bytes[b];
    return a < b;
  });
  const int64_t cap = owner_byte_cap(bytes, n, r, slack);
  std::fill(rank_cost, rank_cost + r, 0.0);
  std::fill(rank_bytes, rank_bytes + r, int64_t(0));
  for (int64_t i : order) {
    int best = -1;
    for (int k = 0; k < r; ++k) {
      if (rank_bytes[k] + bytes[i] > cap) continue;
      if (best < 0 || rank_cost[k] < rank_cost[best]) best = k;
    }
    if (best < 0) {  // no owner keeps the cap: the one with the fewest bytes
      best = 0;
      for (int k = 1; k < r; ++k)
        if (rank_bytes[k] < rank_bytes[best]) best = k;
    }
    owner[i] = best;
    rank_cost[best] += cost[i];
    rank_bytes[best] += bytes[i];
  }
}

// Element offsets of tensors packed in order into one fp32 buffer, each
// segment starting on a 16-byte (4-element) boundary.
constexpr int64_t kTailAlign = 4;

inline int64_t tail_layout(const int64_t* numel, int64_t n, int64_t* offsets) {
  int64_t off = 0;
  for (int64_t i = 0; i < n; ++i) {
    offsets[i] = off;
    off += (numel[i] + kTailAlign - 1) / kTailAlign * kTailAlign;
  }
  return off;
}

// Order of the tiles of one grouped launch.  The device remaps workgroups so
// that XCD x runs the contiguous logical range [x*q + min(x, r), +q + (x < r))
// of the T tiles (q = T / n_xcd, r = T % n_xcd), in order.  The tiles come
// sorted by decreasing cost (K length; the longest are dispatched first).
// Each run of equal cost is cut into n_xcd contiguous parts, one per XCD,
// whose sizes differ by at most one, the larger parts rotating over the XCDs
// from run to run.  Every XCD thus gets the same mix of long and short tiles,
// longest first, in runs of neighbouring tiles (shared operand panels stay in
// its L2).  A plain sorted list would put all the long tiles on the first XCDs
// and leave the others idle once their short tiles are done.
template <class Entry>
void xcd_balance(const std::vector<Entry>& tiles, const std::vector<int64_t>& cost, int n_xcd,
                 Entry* out) {
  const int64_t T = static_cast<int64_t>(tiles.size());
  std::vector<std::vector<Entry>> per(n_xcd);
  int rot = 0;
  for (int64_t b = 0; b < T;) {
    int64_t e = b;
    while (e < T && cost[e] == cost[b]) ++e;
    const int64_t nc = e - b, each = nc / n_xcd;
    const int extra = static_cast<int>(nc % n_xcd);
    int64_t idx = b;
    for (int x = 0; x < n_xcd; ++x) {
      const int64_t take = each + (((x - rot + n_xcd) % n_xcd) < extra ? 1 : 0);
      per[x].insert(per[x].end(), tiles.begin() + idx, tiles.begin() + idx + take);
      idx += take;
    }
    rot = (rot + extra) % n_xcd;
    b = e;
  }
  for (const std::vector<Entry>& v : per) out = std::copy(v.begin(), v.end(), out);
}

}  // namespace mfsdp

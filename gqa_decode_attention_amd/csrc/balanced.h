// Balanced work split of the matrix-core attention kernels (ragged batches).
//
// The batch's work is a sequence of units: sequence b holds Hkv / hp items of
// u_b = C + c_b units each, where an item is hp adjacent kv-heads (hp = 1, or
// the workgroup's wave count when its waves take one kv-head each over the
// same slots) -- C units standing for the fixed cost of a piece (its start-up
// and merge), then its c_b tiles (its attended slots -- in the sliding
// window's virtual order when one is set -- in tiles of 2^shift slots, at
// least one tile so an empty sequence still writes its zero rows).  Item
// (b, i) is units [P_b + i u_b, P_b + (i + 1) u_b), P_b = (Hkv / hp) * sum of
// u_b' over b' < b; its tile j is unit P_b + i u_b + C + j.  The units are cut
// into gridDim.x equal contiguous ranges, one per workgroup, so a workgroup
// holding many short items gets fewer tiles.  A workgroup attends every
// item's tiles inside its range: a whole item writes its output rows; an item
// cut between ranges leaves partial rows (m, l, o of its G * hp heads) at
// workspace row 2 * blockIdx + 1 if the piece holds the item's first tile (the
// range's last piece), else 2 * blockIdx (the range's first piece), and the
// balanced combine pass merges them.  The offsets P_b (and the total) are
// written to the workspace by workgroup 0 for that pass.
#pragma once

#include "device_common.h"
#include "internal.h"
#include "variants.h"

namespace gqa {

__device__ __forceinline__ int seq_tiles(const AttnArgs& a, int b, int shift) {
  int n = a.lengths[b] + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  if (a.window > 0) n = seq_view(a, b, n).nv;
  return max(1, (n + (1 << shift) - 1) >> shift);
}

// Block-wide exclusive scan of the unit counts into pre[0..B] (LDS, B + 1
// entries); `wsum` holds one int per wave.  Called by every thread of the
// workgroup (it holds barriers); at most 16 sequences per thread.
__device__ __forceinline__ void balanced_scan(const AttnArgs& a, int shift, int32_t* pre, int32_t* wsum) {
  const int B = a.B;
  const int nt = blockDim.x;
  const int per_t = (B + nt - 1) / nt;  // consecutive sequences per thread
  const int b0 = threadIdx.x * per_t;
  int cnt[16];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    cnt[i] = (i < per_t && b0 + i < B) ? (a.Hkv / a.hp) * (a.bal_cost + seq_tiles(a, b0 + i, shift)) : 0;
    sum += cnt[i];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = sum;  // inclusive scan within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int run = base + inc - sum;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < per_t && b0 + i < B) pre[b0 + i] = run;
    run += cnt[i];
  }
  if (threadIdx.x == nt - 1) pre[B] = base + inc;
  __syncthreads();
  if (blockIdx.x == 0) {  // the offsets for the combine pass
    for (int i = threadIdx.x; i <= B; i += nt) a.bal_pre[i] = pre[i];
  }
}

// The workgroup's tile range [lo, hi) (empty when lo >= hi).
__device__ __forceinline__ void balanced_range(const int32_t* pre, int B, int* lo, int* hi) {
  const int T = pre[B];
  const int per = (T + (int)gridDim.x - 1) / (int)gridDim.x;
  *lo = (int)blockIdx.x * per;
  *hi = min(*lo + per, T);
}

// The piece of the range [lo, hi) at unit t (the range's start or an item's
// first unit): item (b, h), its tiles [j0, j1) inside the range (none when
// j0 >= j1: the range holds only cost units of the item), whether that is the
// whole item, its partial row base, and the unit where the next piece starts.
struct BalancedPiece {
  int b, h, j0, j1;
  bool whole;
  int64_t pbase;
  int next;
};
__device__ __forceinline__ BalancedPiece balanced_piece(const AttnArgs& a, const int32_t* pre, int t, int hi) {
  int l0 = 0, l1 = a.B;  // pre[l0] <= t < pre[l1]
  while (l1 - l0 > 1) {
    const int mid = (l0 + l1) >> 1;
    if (pre[mid] <= t) l0 = mid;
    else l1 = mid;
  }
  BalancedPiece p;
  p.b = l0;
  const int ub = (pre[l0 + 1] - pre[l0]) / (a.Hkv / a.hp);  // units per item
  const int cb = ub - a.bal_cost;                  // tiles per item
  p.h = (t - pre[l0]) / ub;
  const int s = pre[l0] + p.h * ub + a.bal_cost;   // unit of the item's tile 0
  p.j0 = max(0, t - s);
  p.j1 = min(cb, hi - s);
  const bool first = p.j0 == 0, last = p.j1 == cb;
  p.whole = first && last;
  p.pbase = (2 * (int64_t)blockIdx.x + (first && !last ? 1 : 0)) * a.G * a.hp;
  p.next = min(s + cb, hi);
  return p;
}

}  // namespace gqa

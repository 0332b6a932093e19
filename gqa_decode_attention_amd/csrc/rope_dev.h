// Rotary encoding inside the matrix-core kernels (head width 128; CLIKA
// runtime "groupQueryAttention" API page: q and the new key rotated with the
// rope planes, optional post-rotation RMS norm with gains).
//
// A lane holds four chunks of 8 consecutive elements of one vector; chunk k
// starts at position pos[k], and in every layout used here chunk k ^ 2 starts
// 64 positions away, so the partner of an element in the "half" pairing
// (i, i + 64) sits in the same lane, and in the "interleaved" pairing (2i,
// 2i + 1) it is the neighbour within the chunk.  The arithmetic is that of the
// rotary append kernel: each product and sum rounded separately (no fused
// multiply-add), then, with a gain, x / sqrt(mean(x^2) + eps) * gain.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace gqa {

__device__ __forceinline__ float rope_rot(bool first, float x, float xp, float c, float s) {
#pragma clang fp contract(off)
  const float a = x * c;
  const float b = xp * s;
  return first ? a - b : a + b;
}

// Table row of sequence b's new token (slot L unless positions are given),
// clamped into the table.
__device__ __forceinline__ int rope_row(const AttnArgs& a, int b, int L) {
  const int p = a.rope_pos != nullptr ? a.rope_pos[b] : L;
  return min(max(p, 0), a.rope_max_pos - 1);
}

// Rotate x (and normalize it when `gain` is set) in place.  The vector's other
// 96 elements are held by the lanes 16 apart (rows of the same column): the
// mean square is reduced over them.  All 64 lanes must take part.
__device__ __forceinline__ void rope_chunks(const AttnArgs& a, int p, const int (&pos)[4], float (&x)[4][8],
                                            const float* gain) {
  // The table rows are 16-byte aligned (the host checks it): a chunk's angles
  // are 8 consecutive entries (half: j = d mod 64) or 4 (interleaved: j = d / 2).
  const f32x4* cs = reinterpret_cast<const f32x4*>(a.rope_cos + (int64_t)p * 64);
  const f32x4* sn = reinterpret_cast<const f32x4*>(a.rope_sin + (int64_t)p * 64);
  const bool half = a.rope_mode == GQA_ROPE_HALF;
  float y[4][8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j0 = half ? (pos[k] & 63) : (pos[k] >> 1);  // multiple of 4
    const f32x4 c0 = cs[j0 >> 2], s0 = sn[j0 >> 2];
    const f32x4 c1 = half ? cs[(j0 >> 2) + 1] : c0, s1 = half ? sn[(j0 >> 2) + 1] : s0;
    const float cv[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = pos[k] + e;
      const bool first = half ? d < 64 : (e & 1) == 0;
      const float xp = half ? x[k ^ 2][e] : x[k][e ^ 1];
      const int je = half ? e : (e >> 1);  // index of the angle within the loaded run
      y[k][e] = rope_rot(first, x[k][e], xp, cv[je], sv[je]);
    }
  }
  if (gain != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += y[k][e] * y[k][e];
    ss = rows_sum(ss);
    const float rn = 1.0f / sqrtf(ss / 128.f + a.norm_eps);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) y[k][e] = (y[k][e] * rn) * gain[pos[k] + e];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[k][e] = y[k][e];
}

}  // namespace gqa

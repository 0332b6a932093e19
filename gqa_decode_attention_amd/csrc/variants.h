// Softmax variants shared by the attention kernels (CLIKA runtime,
// "groupQueryAttention" API page: head sink, smooth softmax, softcap, sliding
// window with a kept prefix).
//
// Sliding window.  Of a sequence's n valid slots the query (the newest token,
// slot n - 1) attends the last W and the first P ("kept prefix"): slots j with
// j < P or j >= n - W.  The kernels walk a virtual slot range [0, nv) that
// skips most of the unattended middle: virtual slot v is physical slot v for
// v < pv and v + gap beyond, with pv and gap multiples of 16 (so a 16-slot
// tile that starts on a multiple of 16 stays contiguous, and in one block of
// a paged pool).  The few unattended rows left inside [0, nv) -- physical
// [mlo, mhi) -- are masked to weight 0.  Without a window the view is the
// identity over n slots.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace gqa {

struct SeqView {
  int nv;        // virtual slots to walk
  int pv, gap;   // virtual v -> physical v (v < pv) or v + gap
  int mlo, mhi;  // physical rows in [mlo, mhi) are not attended
};

__device__ __forceinline__ SeqView seq_view(const AttnArgs& a, int b, int n) {
  if (a.window <= 0) return SeqView{n, n, 0, 0, 0};
  const int W = min(a.window, n);
  int P = a.prefix_seq != nullptr ? a.prefix_seq[b] : a.prefix;
  P = max(0, min(P, n - W));
  const int pv = min((P + 15) & ~15, n - W);
  const int gap = (n - W - pv) & ~15;
  return SeqView{n - gap, pv, gap, P, n - W};
}

__device__ __forceinline__ int phys_slot(const SeqView& v, int t) { return t < v.pv ? t : t + v.gap; }
__device__ __forceinline__ bool unattended(const SeqView& v, int tp) { return tp >= v.mlo && tp < v.mhi; }

// Soft-capping of a raw score s = q.k: with T = cap * sqrt(D) (so that the
// scaled score s / sqrt(D) becomes cap * tanh(s / (sqrt(D) cap))), returns
// T tanh(s / T); tanh(x) = 1 - 2 / (e^(2x) + 1) with the hardware exponential
// and reciprocal (about 1 ulp each), exact limits +-1.
__device__ __forceinline__ float cap_score(float s, float T, float invT) {
  const float e = fast_exp2(s * invT * 2.8853900817779268f);  // e^(2x), 2 log2(e)
  return T * (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f));
}

// The sink logit of query head hq in log2 units, or -inf when there is none.
__device__ __forceinline__ float sink_log2(const AttnArgs& a, int hq) {
  if (a.smooth) return 0.f;
  if (a.sink == nullptr) return -__builtin_inff();
  return a.sink[hq] * 1.4426950408889634f;
}

// Final normalization o / l of a row whose partial sums O, Lsum are relative
// to the reference M (log2 units), with the sink's term exp(sink) added to the
// denominator.  Lsum = 0 (no attended slot) gives 0.
__device__ __forceinline__ float finish_row(const AttnArgs& a, int hq, float M, float O, float Lsum) {
  const float sk = sink_log2(a, hq);
  if (sk != -__builtin_inff()) {
    const float Mn = fmaxf(M, sk);
    const float f = M == -__builtin_inff() ? 0.f : fast_exp2(M - Mn);
    O *= f;
    Lsum = Lsum * f + fast_exp2(sk - Mn);
  }
  return Lsum > 0.f ? O / Lsum : 0.f;
}

// The factor that turns the unnormalised sums O (relative to the reference M,
// log2 units) of query head hq into its output, sink term included; 0 when
// nothing is attended.
__device__ __forceinline__ float finish_scale(const AttnArgs& a, int hq, float M, float Lsum) {
  const float sk = sink_log2(a, hq);
  float f = 1.f;
  if (sk != -__builtin_inff()) {
    const float Mn = fmaxf(M, sk);
    f = M == -__builtin_inff() ? 0.f : fast_exp2(M - Mn);
    Lsum = Lsum * f + fast_exp2(sk - Mn);
  }
  return Lsum > 0.f ? f / Lsum : 0.f;
}

}  // namespace gqa

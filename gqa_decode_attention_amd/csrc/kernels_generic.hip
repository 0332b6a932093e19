// Generic kernels of the GQA decode step for gfx950: the in-place append, a
// vector-ALU split attention that takes any head width D <= 256 in f32 or bf16
// storage, and the log-sum-exp combine of split partials.
//
// Semantics: TensorTonic "Grouped-Query Decode Step" (JAX) page, problem
// statement -- query head h reads cache head floor(h/G); only slots
// j < lengths[b] count; s_j = q.K_j/sqrt(D); o = sum_j softmax(s)_j V_j; all in
// float32.  Append: TensorTonic "KV cache decode step" page -- the new key/value
// take the position after the cached tokens.
//
// The split attention evaluates the same softmax with the online (running
// maximum) formulation: for a stream of scores it keeps m = max so far,
// l = sum exp(s - m) and o = sum exp(s - m) V, rescaling l and o by exp(m_old -
// m_new) whenever the maximum grows.  Partial (m, l, o) triples over disjoint
// token ranges merge exactly: M = max m_i, l = sum l_i exp(m_i - M), o = sum
// o_i exp(m_i - M); the output is o / l.  Exponentials are base 2 with log2(e)
// folded into the score scale.
#include <mutex>
#include <type_traits>

#include "cache_map.h"
#include "variants.h"
#include "device_common.h"
#include "internal.h"

namespace gqa {

constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// Append: one thread per element of the new K/V; raw copy of the stored bits.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(AttnArgs a, T* __restrict__ kc, T* __restrict__ vc) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.Hkv * a.D;
  if (i >= total) return;
  const int32_t d = (int32_t)(i % a.D);
  const int64_t bh = i / a.D;
  const int32_t h = (int32_t)(bh % a.Hkv);
  const int32_t b = (int32_t)(bh / a.Hkv);
  const int32_t pos = a.lengths[b];
  if (pos < 0 || pos >= a.S) return;  // out of contract: nothing written
  const int64_t off = slot_offset_checked(a, b, h, pos);
  if (off < 0) return;                // the map names no valid row/block
  kc[off + d] = reinterpret_cast<const T*>(a.k_new)[i];
  vc[off + d] = reinterpret_cast<const T*>(a.v_new)[i];
}

hipError_t launch_append(const AttnArgs& a, void* k_cache, void* v_cache, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.Hkv * a.D;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  AttnArgs arg = a;
  void* params[] = {&arg, &k_cache, &v_cache};
  const void* fn = a.kv_dtype == GQA_F32 ? reinterpret_cast<const void*>(&append_kernel<uint32_t>)
                                         : reinterpret_cast<const void*>(&append_kernel<uint16_t>);
  return hipLaunchKernel(fn, dim3(blocks), dim3(256), params, 0, s);
}

// ---------------------------------------------------------------------------
// Quantizing append into int8 caches (CANN "aclnnMlaPrologV3WeightNz" page,
// dynamic-quantization formula): one wave per (b, kv-head); each new K and V
// row (D <= 256 elements, in the query/output storage type) gets
// scale = max|x| / 127 and codes round-half-even(x / scale), with correctly
// rounded float32 divisions; a zero row stores scale 0 and codes 0.  Fp8
// caches: scale = max|x| / 448 and codes the E4M3 value nearest to x / scale
// clamped to [-448, 448] (e4m3_encode).
// ---------------------------------------------------------------------------

// One row held as elements d = lane + 64 i (i < 4, d < D) of a wave, quantized
// into one-byte codes (int8, or E4M3 when FP8) at dst[off + d] and its scale at
// sdst[off / D].
template <bool FP8>
__device__ __forceinline__ void store_q8_row(const float (&x)[4], int lane, int D, uint8_t* dst, float* sdst,
                                             int64_t off) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(x[i]));  // lanes past D hold 0
  amax = wave_max(amax);
  constexpr float QMAX = FP8 ? 448.f : 127.f;
  const float scale = amax / QMAX;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    if (d < D) {
      if constexpr (FP8) {
        dst[off + d] = (uint8_t)(amax > 0.f ? e4m3_encode(fminf(fmaxf(x[i] / scale, -QMAX), QMAX)) : 0u);
      } else {
        const float c = amax > 0.f ? fminf(fmaxf(rintf(x[i] / scale), -127.f), 127.f) : 0.f;
        dst[off + d] = (uint8_t)(int32_t)c;
      }
    }
  }
  if (lane == 0) sdst[off / D] = scale;
}

// One wave per (b, kv-head, K or V) row, four per workgroup.
template <int NEW, bool FP8>
__global__ __launch_bounds__(256) void append_q8_kernel(AttnArgs a, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // 2 (b * Hkv + h) + which
  const int lane = threadIdx.x & 63;
  if (item >= 2 * (int64_t)a.B * a.Hkv) return;  // whole waves; no barrier follows
  const int64_t row = item >> 1;
  const int which = (int)(item & 1);
  const int b = (int)(row / a.Hkv);
  const int h = (int)(row % a.Hkv);
  const int pos = a.lengths[b];
  if (pos < 0 || pos >= a.S) return;        // out of contract: nothing written
  const int64_t off = slot_offset_checked(a, b, h, pos);
  if (off < 0) return;
  const int D = a.D;
  const void* src = which ? a.v_new : a.k_new;
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lane + 64 * i;
    x[i] = d < D ? Store<NEW>::load1_cached(src, row * D + d) : 0.f;
  }
  store_q8_row<FP8>(x, lane, D, which ? vc : kc, which ? a.v_scale_w : a.k_scale_w, off);
}

hipError_t launch_append_q8(const AttnArgs& a, void* k_cache, void* v_cache, hipStream_t s) {
  const unsigned blocks = (unsigned)((2 * (int64_t)a.B * a.Hkv + 3) / 4);
  AttnArgs arg = a;
  void* params[] = {&arg, &k_cache, &v_cache};
  const bool fp8 = a.kv_dtype == GQA_FP8;
  const void* fn = a.qo_dtype == GQA_F32
                       ? (fp8 ? reinterpret_cast<const void*>(&append_q8_kernel<GQA_F32, true>)
                              : reinterpret_cast<const void*>(&append_q8_kernel<GQA_F32, false>))
                       : (fp8 ? reinterpret_cast<const void*>(&append_q8_kernel<GQA_BF16, true>)
                              : reinterpret_cast<const void*>(&append_q8_kernel<GQA_BF16, false>));
  return hipLaunchKernel(fn, dim3(blocks), dim3(256), params, 0, s);
}

// ---------------------------------------------------------------------------
// Rotary append (CLIKA "groupQueryAttention" page: q and the new k rotated with
// the rope planes, optional post-rotation RMS norm with gains, the rotated key
// appended in place).  The rows of (b, kv-head) are k, v, then its G query
// heads (rotated q is written only when a.q_rot is set).  A row is held as elements d = lane + 64 i; the partner of a rotation
// pair comes from another lane by a cross-lane read.  Products and sums are
// rounded separately (no contraction), so the rotation is reproducible.  The
// value row is a raw copy (int8 caches: quantized like the key).  One wave per
// row, four per workgroup, so every row's load-reduce-store chain runs in
// parallel.
// ---------------------------------------------------------------------------
// One element of a rotated pair: x1 c - x2 s for the first, x2 c + x1 s for the
// second (x = this element, xp = its partner), each product and the sum
// rounded separately: contraction into a fused multiply-add is off here.
__device__ __forceinline__ float rope_pair(bool first, float x, float xp, float c, float s) {
#pragma clang fp contract(off)
  const float a = x * c;
  const float b = xp * s;
  return first ? a - b : a + b;
}

template <int KV, int QO>
__global__ __launch_bounds__(256) void rope_append_kernel(AttnArgs a, void* __restrict__ kc, void* __restrict__ vc) {
  constexpr bool QUANT = KV == GQA_I8 || KV == GQA_FP8;  // one-byte codes with row scales
  constexpr int NEW = QUANT ? QO : KV;                    // storage of k_new / v_new
  const int nrows = 2 + (a.q_rot != nullptr ? a.G : 0);  // k, v, then the query heads
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= (int64_t)a.B * a.Hkv * nrows) return;     // whole waves; no barrier follows
  const int bh = (int)(item / nrows);                    // b * Hkv + h
  const int row = (int)(item - (int64_t)bh * nrows);
  const int b = bh / a.Hkv;
  const int h = bh - b * a.Hkv;
  const int lane = threadIdx.x & 63;
  const int D = a.D;
  const int half = D >> 1;
  const int L = a.lengths[b];
  int p = a.rope_pos != nullptr ? a.rope_pos[b] : L;
  p = min(max(p, 0), a.rope_max_pos - 1);      // memory-safe for out-of-contract positions
  const float* cs = a.rope_cos + (int64_t)p * half;
  const float* sn = a.rope_sin + (int64_t)p * half;
  const int64_t off = (L >= 0 && L < a.S) ? slot_offset_checked(a, b, h, L) : -1;
  {
    const bool isv = row == 1;
    const bool isq = row >= 2;
    if (!isq && off < 0) return;               // the map names no valid slot: nothing appended
    const int64_t base = isq ? ((int64_t)b * a.Hq + (int64_t)h * a.G + (row - 2)) * D : (int64_t)bh * D;
    if (isv && !QUANT) {
      for (int d = lane; d < D; d += 64) {
        if constexpr (KV == GQA_BF16)
          reinterpret_cast<uint16_t*>(vc)[off + d] = reinterpret_cast<const uint16_t*>(a.v_new)[base + d];
        else
          reinterpret_cast<uint32_t*>(vc)[off + d] = reinterpret_cast<const uint32_t*>(a.v_new)[base + d];
      }
      return;
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = lane + 64 * i;
      x[i] = d >= D ? 0.f
             : isq  ? Store<QO>::load1_cached(a.q, base + d)
                    : Store<NEW>::load1_cached(isv ? a.v_new : a.k_new, base + d);
    }
    if (!isv) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        bool first;
        int dp, j;
        if (a.rope_mode == GQA_ROPE_HALF) {
          first = d < half;
          dp = first ? d + half : d - half;
          j = first ? d : d - half;
        } else {
          first = (d & 1) == 0;
          dp = d ^ 1;
          j = d >> 1;
        }
        float xp = 0.f;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float t = __shfl(x[ii], dp & 63);
          if ((dp >> 6) == ii) xp = t;
        }
        const bool in = d < D;
        const float c = in ? cs[j] : 0.f;
        const float sv = in ? sn[j] : 0.f;
        y[i] = rope_pair(first, x[i], xp, c, sv);
      }
      const float* gain = isq ? a.q_gain : a.k_gain;
      if (gain != nullptr) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) ss += y[i] * y[i];  // lanes past D hold 0
        ss = wave_sum(ss);
        const float r = 1.0f / sqrtf(ss / (float)D + a.norm_eps);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = lane + 64 * i;
          y[i] = d < D ? (y[i] * r) * gain[d] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = y[i];
    }
    if (isq) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) Store<QO>::store1(a.q_rot, base + d, x[i]);
      }
    } else if constexpr (QUANT) {
      store_q8_row<KV == GQA_FP8>(x, lane, D, reinterpret_cast<uint8_t*>(isv ? vc : kc),
                                  isv ? a.v_scale_w : a.k_scale_w, off);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = lane + 64 * i;
        if (d < D) Store<KV>::store1(kc, off + d, x[i]);
      }
    }
  }
}

hipError_t launch_rope_append(const AttnArgs& a, void* k_cache, void* v_cache, hipStream_t s) {
  AttnArgs arg = a;
  void* params[] = {&arg, &k_cache, &v_cache};
  const void* fn;
  const bool f32 = a.qo_dtype == GQA_F32;
  if (a.kv_dtype == GQA_I8)
    fn = f32 ? reinterpret_cast<const void*>(&rope_append_kernel<GQA_I8, GQA_F32>)
             : reinterpret_cast<const void*>(&rope_append_kernel<GQA_I8, GQA_BF16>);
  else if (a.kv_dtype == GQA_FP8)
    fn = f32 ? reinterpret_cast<const void*>(&rope_append_kernel<GQA_FP8, GQA_F32>)
             : reinterpret_cast<const void*>(&rope_append_kernel<GQA_FP8, GQA_BF16>);
  else if (a.kv_dtype == GQA_BF16)
    fn = f32 ? reinterpret_cast<const void*>(&rope_append_kernel<GQA_BF16, GQA_F32>)
             : reinterpret_cast<const void*>(&rope_append_kernel<GQA_BF16, GQA_BF16>);
  else
    fn = f32 ? reinterpret_cast<const void*>(&rope_append_kernel<GQA_F32, GQA_F32>)
             : reinterpret_cast<const void*>(&rope_append_kernel<GQA_F32, GQA_BF16>);
  const int64_t items = (int64_t)a.B * a.Hkv * (2 + (a.q_rot != nullptr ? a.G : 0));
  return hipLaunchKernel(fn, dim3((unsigned)((items + 3) / 4)), dim3(256), params, 0, s);
}

// ---------------------------------------------------------------------------
// Generic split attention.
//
// Grid: blockIdx.x = ((b * Hkv + h) * head_chunks + c) * nsplit + split; the
// split index varies fastest so neighbouring workgroups (which the dispatcher
// deals round-robin to the 8 XCDs) take different token ranges of the same
// (b, h).  Block: 4 waves.  The lanes of a wave form row groups of LPR lanes;
// a row group handles one slot at a time and each lane holds NCH chunks of VEC
// consecutive elements of the row (element d = (c * LPR + lane_in_group) * VEC
// + e).  A workgroup serves up to kGenericHeadChunk query heads of one kv-head,
// so each K/V row it loads is used by all of them.
// ---------------------------------------------------------------------------
template <int KV, int QO, int VEC, int NCH, int LPR>
__global__ __launch_bounds__(256) void attend_generic_kernel(AttnArgs a) {
  constexpr int EPL = VEC * NCH;
  constexpr int RPW = 64 / LPR;
  constexpr int NRG = 4 * RPW;
  constexpr int GC = kGenericHeadChunk;
  constexpr int KB = Store<KV>::kBytes;

  __shared__ float sm_o[4][GC][256];
  __shared__ float sm_m[4][GC];
  __shared__ float sm_l[4][GC];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rl = lane % LPR;
  const int rg = wave * RPW + lane / LPR;

  int x = blockIdx.x;
  const int split = x % a.nsplit;
  x /= a.nsplit;
  const int hc = x % a.head_chunks;
  x /= a.head_chunks;
  const int h = x % a.Hkv;
  const int b = x / a.Hkv;
  const int g0 = hc * GC;
  const int gc = min(GC, a.G - g0);
  const int D = a.D;

  int n = a.lengths[b] + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  // Slots are walked in the sliding window's virtual order (the identity
  // without a window).
  const SeqView view = seq_view(a, b, n);
  const int t_begin = split * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, view.nv);
  // Splits holding valid slots.  A lone active split (or split 0 when n = 0)
  // writes the output itself and the combine pass leaves that sequence alone.
  const int nact = view.nv == 0 ? 0 : min(a.nsplit, (view.nv + a.split_tokens - 1) / a.split_tokens);
  if (split >= max(nact, 1)) return;

  const int64_t qrow0 = ((int64_t)b * a.Hq + (int64_t)h * a.G + g0) * D;
  float qv[GC][EPL];
#pragma unroll
  for (int g = 0; g < GC; ++g)
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int d = (c * LPR + rl) * VEC + e;
        qv[g][c * VEC + e] = (g < gc && d < D) ? Store<QO>::load1_cached(a.q, qrow0 + (int64_t)g * D + d) : 0.f;
      }

  float m[GC], l[GC], acc[GC][EPL];
#pragma unroll
  for (int g = 0; g < GC; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const char* kb = reinterpret_cast<const char*>(a.k_cache);
  const char* vb = reinterpret_cast<const char*>(a.v_cache);
  // Fused step (float32 / bf16 caches): the new token, virtual slot Lv, is
  // read from k_new / v_new instead of the cache, and head chunk 0 of the
  // split that holds it stores it at slot lengths[b] after the loop.  No other
  // workgroup reads that slot (the other head chunks take it from k_new too).
  const int L0 = a.lengths[b];
  const int Lv = L0 - view.gap;
  const bool fused_new = KV != GQA_I8 && a.k_new != nullptr;
  const int64_t nrow = ((int64_t)b * a.Hkv + h) * D;

  for (int t = t_begin + rg; t < t_end; t += NRG) {
    const int tp = phys_slot(view, t);
    if (unattended(view, tp)) continue;  // uniform within the row group
    const bool is_new = fused_new && t == Lv;
    const int64_t row = is_new ? nrow : slot_offset(a, b, h, tp);
    const char* kbr = is_new ? reinterpret_cast<const char*>(a.k_new) : kb;
    const char* vbr = is_new ? reinterpret_cast<const char*>(a.v_new) : vb;
    float kv[EPL], vv[EPL];
    float ks = 1.f, vs = 1.f;  // int8 caches: the row scales
    if constexpr (KV == GQA_I8) {
      ks = a.k_scale[row / D];
      vs = a.v_scale[row / D];
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int d0 = (c * LPR + rl) * VEC;
      if constexpr (VEC > 1) {
        if (d0 < D) {
          widen16<KV>(load_nt16(kbr + (row + d0) * KB), &kv[c * VEC]);
          widen16<KV>(load_nt16(vbr + (row + d0) * KB), &vv[c * VEC]);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) kv[c * VEC + e] = vv[c * VEC + e] = 0.f;
        }
      } else {
        kv[c] = d0 < D ? Store<KV>::load1(kbr, row + d0) : 0.f;
        vv[c] = d0 < D ? Store<KV>::load1(vbr, row + d0) : 0.f;
      }
    }
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part = fmaf(qv[g][e], kv[e], part);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) part += __shfl_xor(part, off);
      float s;
      if (a.cap_T > 0.f)
        s = cap_score(KV == GQA_I8 ? part * ks : part, a.cap_T, a.cap_invT) * a.scale_log2;
      else
        s = part * (KV == GQA_I8 ? ks * a.scale_log2 : a.scale_log2);
      const float mn = fmaxf(m[g], s);
      const float alpha = fast_exp2(m[g] - mn);  // 0 on the first slot (m = -inf)
      const float p = fast_exp2(s - mn);
      l[g] = l[g] * alpha + p;
      const float pv = KV == GQA_I8 ? p * vs : p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pv, vv[e], acc[g][e] * alpha);
      m[g] = mn;
    }
  }

  // Merge the row groups of each wave (partials over disjoint slot sets).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a1 = m[g] == kNegInf ? 0.f : fast_exp2(m[g] - mn);
      const float a2 = mo == kNegInf ? 0.f : fast_exp2(mo - mn);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }
  // Merge the 4 waves through LDS; row group 0 of each wave holds its wave's totals.
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GC; ++g) {
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int d = (c * LPR + rl) * VEC + e;
          if (d < D) sm_o[wave][g][d] = acc[g][c * VEC + e];
        }
      if (rl == 0) {
        sm_m[wave][g] = m[g];
        sm_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < gc * D; idx += 256) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_m[w][g]);
    float O = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = sm_m[w][g];
      const float sc = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      O += sm_o[w][g][d] * sc;
      L += sm_l[w][g] * sc;
    }
    const int hq = h * a.G + g0 + g;
    if (nact <= 1) {
      Store<QO>::store1(a.out, ((int64_t)b * a.Hq + hq) * D + d,
                        a.sink != nullptr || a.smooth ? O * finish_scale(a, hq, M, L) : (L > 0.f ? O / L : 0.f));
    } else {
      const int64_t pi = ((int64_t)b * a.Hq + hq) * a.nsplit + split;
      a.part_o[pi * D + d] = O;
      if (d == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = L;
      }
    }
  }
  if constexpr (KV != GQA_I8) {
    if (fused_new && hc == 0 && Lv >= t_begin && Lv < t_end) {  // the appended slot (raw bits)
      const int64_t off = slot_offset_checked(a, b, h, L0);
      if (off >= 0) {
        for (int d = threadIdx.x; d < D; d += 256) {
          Store<KV>::copy1(a.k_cache_w, off + d, a.k_new, nrow + d);
          Store<KV>::copy1(a.v_cache_w, off + d, a.v_new, nrow + d);
        }
      }
    }
  }
}

template <int KV, int QO, int VEC, int NCH, int LPR>
static hipError_t launch_generic_t(const AttnArgs& a, const Plan& p, hipStream_t s) {
  AttnArgs arg = a;
  void* params[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&attend_generic_kernel<KV, QO, VEC, NCH, LPR>),
                         dim3(p.grid), dim3(256), params, 0, s);
}

// vec_path: every cache row starts 16-byte aligned and D is a multiple of the
// 16-byte vector (8 bf16 or 4 f32), so rows are read with 16-byte loads.
template <int KV, int QO>
static hipError_t dispatch_generic(const AttnArgs& a, const Plan& p, int vec_path, hipStream_t s) {
  const int D = a.D;
  if (vec_path) {
    if constexpr (KV == GQA_I8) {
      if (D <= 64) return launch_generic_t<KV, QO, 16, 1, 4>(a, p, s);
      if (D <= 128) return launch_generic_t<KV, QO, 16, 1, 8>(a, p, s);
      return launch_generic_t<KV, QO, 16, 1, 16>(a, p, s);
    } else if constexpr (KV == GQA_BF16) {
      if (D <= 32) return launch_generic_t<KV, QO, 8, 1, 4>(a, p, s);
      if (D <= 128) return launch_generic_t<KV, QO, 8, 1, 16>(a, p, s);
      return launch_generic_t<KV, QO, 8, 1, 32>(a, p, s);
    } else {
      if (D <= 16) return launch_generic_t<KV, QO, 4, 1, 4>(a, p, s);
      if (D <= 64) return launch_generic_t<KV, QO, 4, 1, 16>(a, p, s);
      return launch_generic_t<KV, QO, 4, 1, 64>(a, p, s);
    }
  }
  if (D <= 4) return launch_generic_t<KV, QO, 1, 1, 4>(a, p, s);
  if (D <= 16) return launch_generic_t<KV, QO, 1, 1, 16>(a, p, s);
  if (D <= 64) return launch_generic_t<KV, QO, 1, 1, 64>(a, p, s);
  return launch_generic_t<KV, QO, 1, 4, 64>(a, p, s);
}

hipError_t launch_attend_generic(const AttnArgs& a, const Plan& p, int vec_path, hipStream_t s) {
  if (a.kv_dtype == GQA_FP8) return hipErrorInvalidValue;  // fp8 caches: the matrix-core kernel only
  if (a.kv_dtype == GQA_I8)
    return a.qo_dtype == GQA_F32 ? dispatch_generic<GQA_I8, GQA_F32>(a, p, vec_path, s)
                                 : dispatch_generic<GQA_I8, GQA_BF16>(a, p, vec_path, s);
  if (a.kv_dtype == GQA_F32 && a.qo_dtype == GQA_F32) return dispatch_generic<GQA_F32, GQA_F32>(a, p, vec_path, s);
  if (a.kv_dtype == GQA_F32) return dispatch_generic<GQA_F32, GQA_BF16>(a, p, vec_path, s);
  if (a.qo_dtype == GQA_F32) return dispatch_generic<GQA_BF16, GQA_F32>(a, p, vec_path, s);
  return dispatch_generic<GQA_BF16, GQA_BF16>(a, p, vec_path, s);
}

// ---------------------------------------------------------------------------
// Small head widths (D <= 16, capacity <= 512, plain softmax): one wave per
// (sequence, query head), four per workgroup; lane j takes slot j of each
// 64-slot chunk with its whole key and value row (D elements), so a chunk is
// one dot product per lane, a wave maximum and sum, and the weighted rows
// summed across lanes at the end -- a short dependent chain for steps whose
// time is all latency.  The new token of a step (slot lengths[b]) is read
// from k_new / v_new, and the wave of the kv-head's first query head stores
// it; no other wave reads that slot.
// ---------------------------------------------------------------------------
template <int KV, int QO, int DMAX, bool MAPPED>
__global__ __launch_bounds__(256) void attend_small_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  // b * Hq + hq (fits 32 bits), uniform over the wave, so lengths and q come by scalar loads.
  const int bq = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (bq >= a.B * a.Hq) return;  // whole waves only; no workgroup barrier follows
  const int b = bq / a.Hq;
  const int hq = bq - b * a.Hq;
  const int h = hq / a.G;
  const int D = a.D;
  const int L0 = a.lengths[b];
  int n = L0 + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  // Elements d >= D of a row read element D - 1 (in bounds, same row) and meet a
  // zero query element, so every load is unconditional.
  float q[DMAX];
#pragma unroll
  for (int d = 0; d < DMAX; ++d)
    q[d] = d < D ? Store<QO>::load1_cached(a.q, (int64_t)bq * D + d) : 0.f;
  const bool fused = a.k_new != nullptr;
  const int64_t nrow = ((int64_t)b * a.Hkv + h) * D;
  const int64_t base = MAPPED ? 0 : row_head_offset(a, b, h);
  float m = kNegInf, l = 0.f, o[DMAX];
#pragma unroll
  for (int d = 0; d < DMAX; ++d) o[d] = 0.f;
  for (int j0 = 0; j0 < n; j0 += 64) {  // uniform over the wave
    const int j = j0 + lane;
    float s = kNegInf, v[DMAX];
#pragma unroll
    for (int d = 0; d < DMAX; ++d) v[d] = 0.f;
    if (j < n) {
      const bool is_new = fused && j == L0;
      const int64_t off = is_new ? nrow : (MAPPED ? slot_offset(a, b, h, j) : base + (int64_t)j * a.st);
      const void* kb = is_new ? a.k_new : a.k_cache;
      const void* vb = is_new ? a.v_new : a.v_cache;
      float kx[DMAX];
#pragma unroll
      for (int d = 0; d < DMAX; ++d) {
        const int dd = d < D ? d : D - 1;
        kx[d] = Store<KV>::load1_cached(kb, off + dd);
        v[d] = Store<KV>::load1_cached(vb, off + dd);
      }
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DMAX; ++d) dot = fmaf(q[d], kx[d], dot);
      s = dot * a.scale_log2;
    }
    const float mn = fmaxf(m, wave_max_dpp(s));
    const float alpha = m == kNegInf ? 0.f : fast_exp2(m - mn);
    const float p = j < n ? fast_exp2(s - mn) : 0.f;
    l = l * alpha + wave_sum_dpp(p);
#pragma unroll
    for (int d = 0; d < DMAX; ++d) o[d] = fmaf(p, v[d], o[d] * alpha);
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int d = 0; d < DMAX; ++d) {
    if (d < D) {  // uniform
      const float od = wave_sum_dpp(o[d]);
      if (lane == d) Store<QO>::store1(a.out, (int64_t)bq * D + d, od * inv);
    }
  }
  if (fused && hq == h * a.G && lane < D) {  // the appended slot (raw bits)
    const int64_t off = (L0 >= 0 && L0 < a.S) ? slot_offset_checked(a, b, h, L0) : -1;
    if (off >= 0) {
      Store<KV>::copy1(a.k_cache_w, off + lane, a.k_new, nrow + lane);
      Store<KV>::copy1(a.v_cache_w, off + lane, a.v_new, nrow + lane);
    }
  }
}

template <int KV, int QO, bool MAPPED>
static const void* small_kernel(int D) {
  if (D <= 4) return reinterpret_cast<const void*>(&attend_small_kernel<KV, QO, 4, MAPPED>);
  if (D <= 8) return reinterpret_cast<const void*>(&attend_small_kernel<KV, QO, 8, MAPPED>);
  return reinterpret_cast<const void*>(&attend_small_kernel<KV, QO, 16, MAPPED>);
}

template <int KV, int QO>
static const void* small_kernel(int D, bool mapped) {
  return mapped ? small_kernel<KV, QO, true>(D) : small_kernel<KV, QO, false>(D);
}

hipError_t launch_attend_small(const AttnArgs& a, const Plan& p, hipStream_t s) {
  if (a.D > 16 || a.kv_dtype == GQA_I8 || a.kv_dtype == GQA_FP8 || p.grid < 1) return hipErrorInvalidValue;
  AttnArgs arg = a;
  void* params[] = {&arg};
  const bool mapped = a.map_kind != 0;
  const void* fn;
  if (a.kv_dtype == GQA_F32)
    fn = a.qo_dtype == GQA_F32 ? small_kernel<GQA_F32, GQA_F32>(a.D, mapped) : small_kernel<GQA_F32, GQA_BF16>(a.D, mapped);
  else
    fn = a.qo_dtype == GQA_F32 ? small_kernel<GQA_BF16, GQA_F32>(a.D, mapped)
                               : small_kernel<GQA_BF16, GQA_BF16>(a.D, mapped);
  return hipLaunchKernel(fn, dim3(p.grid), dim3(256), params, 0, s);
}

// ---------------------------------------------------------------------------
// Combine: one wave per (b, query head), four per workgroup.  Lane i holds
// split i's maximum and denominator (at most 64 splits), so the merged maximum
// M, the weights 2^(m_i - M) and the merged denominator are wave reductions;
// each lane then sums up to four output columns over the active splits with
// independent loads.
// ---------------------------------------------------------------------------

template <int QO>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + hq
  if (bh >= (int64_t)a.B * a.Hq) return;  // whole waves only; no workgroup barrier follows
  const int b = (int)(bh / a.Hq);
  int n = a.lengths[b] + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  if (a.window > 0) n = seq_view(a, b, n).nv;  // the splits cover the window's virtual slots
  const int nact = n == 0 ? 0 : min(a.nsplit, (n + a.split_tokens - 1) / a.split_tokens);
  if (nact <= 1) return;  // the attention pass wrote this sequence's output itself
  const int64_t pbase = bh * a.nsplit;
  const float mi = lane < nact ? a.part_m[pbase + lane] : kNegInf;
  const float li = lane < nact ? a.part_l[pbase + lane] : 0.f;
  const float M = wave_max(mi);
  const float wi = lane < nact ? fast_exp2(mi - M) : 0.f;
  const float L = wave_sum(wi * li);
  const int D = a.D;
  float O[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < nact; ++i) {
    const float w = __shfl(wi, i);
    const float* po = a.part_o + (pbase + i) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = lane + 64 * k;
      if (d < D) O[k] = fmaf(w, po[d], O[k]);
    }
  }
  const bool sink = a.sink != nullptr || a.smooth;
  const float fs = sink ? finish_scale(a, (int)(bh - (int64_t)b * a.Hq), M, L) : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int d = lane + 64 * k;
    if (d < D) Store<QO>::store1(a.out, bh * D + d, sink ? O[k] * fs : (L > 0.f ? O[k] / L : 0.f));
  }
}

// Combine for head width 128 with an aligned output.  One wave per
// (b, query head); lane j merges output columns 2j and 2j + 1.  Every lane
// reads the splits' maxima and denominators itself (the same values across the
// wave), so the merge takes no cross-lane step.  NS > 0: the split count is at
// most NS and the splits are unrolled, every load issued before any result is
// needed (the sequence length, the (m, l) pairs, the lane's columns of each
// partial row; indices past the split count repeat the last split), so the pass
// costs about one memory round trip.  NS = 0: any split count, in loops.
// Partial rows of inactive splits are never used (their m and l may be stale
// NaN or Inf: they are selected away, not multiplied by zero).
template <int QO, int NS>
__global__ __launch_bounds__(256) void combine128_kernel(AttnArgs a) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + hq
  if (bh >= (int64_t)a.B * a.Hq) return;  // whole waves only; no workgroup barrier follows
  const int b = (int)(bh / a.Hq);
  const int ns = a.nsplit;
  const int64_t pbase = bh * ns;
  const f32x2* po = reinterpret_cast<const f32x2*>(a.part_o) + lane;  // split i: po[(pbase + i) * 64]
  float mr[NS > 0 ? NS : 1], lr[NS > 0 ? NS : 1];
  f32x2 o[NS > 0 ? NS : 1];
  if constexpr (NS > 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int64_t pi = pbase + min(i, ns - 1);
      mr[i] = a.part_m[pi];
      lr[i] = a.part_l[pi];
      o[i] = po[pi * 64];
    }
  }
  int n = a.lengths[b] + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  if (a.window > 0) n = seq_view(a, b, n).nv;  // the splits cover the window's virtual slots
  const int nact = n == 0 ? 0 : min(ns, (n + a.split_tokens - 1) / a.split_tokens);
  if (nact <= 1) return;  // the attention pass wrote this sequence's output itself
  float M = kNegInf, L = 0.f;
  f32x2 acc = {0.f, 0.f};
  if constexpr (NS > 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i) M = i < nact ? fmaxf(M, mr[i]) : M;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const float w = i < nact ? fast_exp2(mr[i] - M) : 0.f;
      L += i < nact ? w * lr[i] : 0.f;
      acc += i < nact ? w * o[i] : f32x2{0.f, 0.f};
    }
  } else {
    for (int i = 0; i < nact; ++i) M = fmaxf(M, a.part_m[pbase + i]);
    for (int i = 0; i < nact; ++i) {
      const float w = fast_exp2(a.part_m[pbase + i] - M);
      L += w * a.part_l[pbase + i];
      acc += w * po[(pbase + i) * 64];
    }
  }
  const float inv = a.sink != nullptr || a.smooth ? finish_scale(a, (int)(bh - (int64_t)b * a.Hq), M, L)
                                                  : (L > 0.f ? 1.f / L : 0.f);
  if (QO == GQA_F32) {
    reinterpret_cast<f32x2*>(a.out)[bh * 64 + lane] = acc * inv;
  } else {
    reinterpret_cast<uint32_t*>(a.out)[bh * 64 + lane] =
        (uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16);
  }
}

// Balanced-mode combine (head width 128): one wave per (b, hq) row, lane j
// merging output columns 2j and 2j + 1.  Item (b, i) -- kv-heads
// [i hp, (i + 1) hp) of sequence b, so query heads [i G hp, (i + 1) G hp) --
// covers tiles [s, e) of the batch's tile sequence (offsets written by the
// attention pass); workgroup k of `a.bal_units` held tiles [k per, (k + 1) per).
// An item inside one workgroup's range was written by the attention pass; a cut
// one left a partial in every workgroup it touched: row 2k + 1 of the first
// workgroup when the item starts inside its range, row 2k + 0 otherwise.  The
// partials merge by the same log-sum-exp rule as the split combine, any number
// of them: every lane reads the pieces' (m, l) itself (no cross-lane step), the
// first eight pieces' loads issued together, the rest in loops.
template <int QO>
__global__ __launch_bounds__(256) void combine_balanced_kernel(AttnArgs a) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int lane = threadIdx.x & 63;
  const int64_t bh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + hq
  if (bh >= (int64_t)a.B * a.Hq) return;  // whole waves only; no workgroup barrier follows
  const int b = (int)(bh / a.Hq);
  const int hq = (int)(bh - (int64_t)b * a.Hq);
  const int GI = a.G * a.hp;   // query heads per item
  const int h = hq / GI;       // item within the sequence
  const int g = hq - h * GI;
  const int* pre = a.bal_pre;
  const int T = pre[a.B];
  const int W = a.bal_units;  // workgroups of the attention pass
  const int per = (T + W - 1) / W;
  const int ub = (pre[b + 1] - pre[b]) / (a.Hkv / a.hp);  // units per item
  const int cb = ub - a.bal_cost;                // tiles per item
  const int s0 = pre[b] + h * ub + a.bal_cost;   // unit of the item's tile 0
  const int k0 = s0 / per, k1 = (s0 + cb - 1) / per;
  if (k0 == k1) return;  // whole in one workgroup: written by the attention pass
  const int np = k1 - k0 + 1;
  auto row = [&](int i) -> int64_t {  // partial row of the i-th piece (the first holds the item's first tile)
    return (2 * (int64_t)(k0 + i) + (i == 0 ? 1 : 0)) * GI + g;
  };
  const f32x2* po = reinterpret_cast<const f32x2*>(a.part_o) + lane;  // row r: po[r * 64]
  constexpr int U = 8;
  float mr[U], lr[U];
  f32x2 o[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const int64_t r = row(min(i, np - 1));
    mr[i] = a.part_m[r];
    lr[i] = a.part_l[r];
    o[i] = po[r * 64];
  }
  float M = kNegInf, L = 0.f;
  f32x2 acc = {0.f, 0.f};
#pragma unroll
  for (int i = 0; i < U; ++i) M = i < np ? fmaxf(M, mr[i]) : M;
  for (int i = U; i < np; ++i) M = fmaxf(M, a.part_m[row(i)]);
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const float w = i < np ? fast_exp2(mr[i] - M) : 0.f;
    L += i < np ? w * lr[i] : 0.f;
    acc += i < np ? w * o[i] : f32x2{0.f, 0.f};
  }
  for (int i = U; i < np; ++i) {
    const int64_t r = row(i);
    const float w = fast_exp2(a.part_m[r] - M);
    L += w * a.part_l[r];
    acc += w * po[r * 64];
  }
  const float inv = a.sink != nullptr || a.smooth ? finish_scale(a, hq, M, L) : (L > 0.f ? 1.f / L : 0.f);
  if (QO == GQA_F32) {
    reinterpret_cast<f32x2*>(a.out)[bh * 64 + lane] = acc * inv;
  } else {
    reinterpret_cast<uint32_t*>(a.out)[bh * 64 + lane] =
        (uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16);
  }
}

hipError_t launch_combine(const AttnArgs& a, const Plan& p, hipStream_t s) {
  (void)p;
  const unsigned blocks = (unsigned)(((int64_t)a.B * a.Hq + 3) / 4);
  AttnArgs arg = a;
  void* params[] = {&arg};
  const bool fast = a.D == 128 && (reinterpret_cast<uintptr_t>(a.out) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(a.part_o) & 15) == 0;
  const void* fn;
  if (a.bal_pre != nullptr) {
    if (a.D != 128 || !fast) return hipErrorInvalidValue;
    fn = a.qo_dtype == GQA_F32 ? reinterpret_cast<const void*>(&combine_balanced_kernel<GQA_F32>)
                               : reinterpret_cast<const void*>(&combine_balanced_kernel<GQA_BF16>);
  } else if (fast) {
    const bool f32 = a.qo_dtype == GQA_F32;
    auto pick = [&](auto ns) -> const void* {
      constexpr int NS = decltype(ns)::value;
      return f32 ? reinterpret_cast<const void*>(&combine128_kernel<GQA_F32, NS>)
                 : reinterpret_cast<const void*>(&combine128_kernel<GQA_BF16, NS>);
    };
    fn = a.nsplit <= 2   ? pick(std::integral_constant<int, 2>{})
         : a.nsplit <= 4 ? pick(std::integral_constant<int, 4>{})
         : a.nsplit <= 8 ? pick(std::integral_constant<int, 8>{})
                         : pick(std::integral_constant<int, 0>{});
  } else {
    fn = a.qo_dtype == GQA_F32 ? reinterpret_cast<const void*>(&combine_kernel<GQA_F32>)
                               : reinterpret_cast<const void*>(&combine_kernel<GQA_BF16>);
  }
  return hipLaunchKernel(fn, dim3(blocks), dim3(256), params, 0, s);
}

// ---------------------------------------------------------------------------
// Length check (debugging aid): one workgroup counts the entries outside
// [lo, hi] and stores the count in a device variable the host copies back.
// ---------------------------------------------------------------------------
__device__ int32_t g_bad_lengths;

__global__ __launch_bounds__(1024) void check_lengths_kernel(const int32_t* lengths, int32_t B, int32_t lo,
                                                             int32_t hi) {
  __shared__ int32_t part[16];
  int32_t cnt = 0;
  for (int32_t i = threadIdx.x; i < B; i += blockDim.x) {
    const int32_t v = lengths[i];
    cnt += (v < lo || v > hi) ? 1 : 0;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x < 64) {
    int32_t t = threadIdx.x < (blockDim.x >> 6) ? part[threadIdx.x] : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
    if (threadIdx.x == 0) g_bad_lengths = t;
  }
}

hipError_t run_check_lengths(const int32_t* lengths, int32_t B, int32_t lo, int32_t hi, hipStream_t s,
                             int32_t* bad) {
  static std::mutex mu;  // one device variable per GPU: serialise the calls
  std::lock_guard<std::mutex> lock(mu);
  const int32_t* lp = lengths;
  void* params[] = {&lp, &B, &lo, &hi};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&check_lengths_kernel), dim3(1), dim3(1024), params,
                                 0, s);
  if (e != hipSuccess) return e;
  int32_t host = 0;
  e = hipMemcpyFromSymbolAsync(&host, HIP_SYMBOL(g_bad_lengths), sizeof(host), 0, hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  *bad = host;
  return hipSuccess;
}

}  // namespace gqa

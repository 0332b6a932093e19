// Matrix-core attention kernel of the GQA decode step, head width 128, bf16
// q/out: scores and the V sum on MFMA with K/V rows loaded straight into the
// MFMA operands (no LDS staging).  Serves bf16 caches with up to 16 query
// heads per kv-head, and int8 or fp8 (E4M3) caches with per-row float32 scales
// (Huawei CANN "aclnnMlaPrologV3WeightNz" page, dynamic-quantization formula: a
// cached value reads as code * row scale) with up to 64.  What is computed is
// the JAX "Grouped-Query Decode Step" page's definition over the dequantized
// rows, with an online softmax over 16-slot tiles.
//
// One workgroup = NW waves = one (sequence, kv-head, head chunk, split); each
// wave walks its own run of 16-slot tiles for HB blocks of 16 query heads:
// HB = 1 (4 waves) up to 16 heads; HB = 2 (8 waves, 32 heads per chunk) for
// int8 and fp8 caches with more, where the widened codes of a tile then serve
// twice as many heads.  Lane l = 16 r + c.  Per tile and head block:
//   scores  S(16 slots x 16 heads) = K(16 x 128) . Q^T as four
//           v_mfma_f32_16x16x32_bf16: lane (r, c) supplies A-operand pieces of
//           cache row t0 + c.  bf16 caches: bytes 16r + 64kk of the row for
//           MFMA kk.  int8 / fp8: two 16-byte loads (bytes 16r + 64j, j = 0,
//           1) give 32 codes, widened exactly to bf16 (|code| <= 127; every
//           E4M3 value is a bf16 value); MFMA 2j + h
//           takes codes 64j + 16r + 8h .. +7, and the query operand holds the
//           same head-width positions (the dot product does not care how the
//           positions are dealt, only that both operands agree).  Lane (r, c)
//           then holds the scores of slots 4r .. 4r + 3 for head c; 8-bit
//           rows multiply them by their key scales.
//   softmax per head c, as in the other kernels (lazy rescale, exp2 with the
//           scale folded in).
//   V sum   O^T(128 x 16 heads) += V^T(128 x 16 slots) . P'(16 slots x 16
//           heads) as eight v_mfma_f32_16x16x32_bf16, e = 0..7.  Lane (r, c)
//           loads slots 4r + i (i = 0..3) at elements 8c .. 8c + 7; the A
//           operand of MFMA e is element 8c + e of its four slots, twice (so
//           MFMA e covers head-width positions e, 8 + e, ..., 120 + e), and
//           the B operand is the lane's own four weights of head c (times the
//           value scales of 8-bit rows) split into bf16 hi and lo parts, the
//           K axis holding each slot once with each part.  Lane (r, c)
//           receives head c at positions 8(4r + i) + e: complete sums, no
//           cross-lane reduction.
// Scores are exact products (bf16 values) summed in float32; each
// weight reaches the V sum as hi + lo (about 16 significant bits) and the
// products accumulate in float32, as does the denominator l.
//
// Fused step: the new token (slot lengths[b]) is not read from the cache; the
// last wave of the workgroup whose split holds it runs one extra tile whose
// only valid row comes from k_new / v_new (int8 caches: quantized in the
// kernel by the per-row rule), and writes that row (and its scales) into the
// cache slot after its loop.  No other workgroup reads that slot, so the write
// cannot race a read.
//
// Paged bf16 caches (CLIKA runtime "groupQueryAttention" API page, block
// table): with a block size that is a multiple of 16, every 16-slot tile lies
// in one block, whose table entry each wave loads a tile pair ahead.
#include <algorithm>
#include <type_traits>

#include "balanced.h"
#include "cache_map.h"
#include "device_common.h"
#include "internal.h"
#include "variants.h"

namespace gqa {

namespace qkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInfQ = -__builtin_inff();
constexpr int kDq = 128;
constexpr float kSlackQ = 8.f;  // lazy rescale threshold, log2 units
// Merge-buffer row pitch in floats: a head's 128 sums plus 16 bytes, so the
// 16-byte stores of eight lanes holding eight different heads fall on
// different LDS banks (with a 512-byte pitch they would all share one).
constexpr int kMergePitch = kDq + 4;

template <int I, int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll<I + 1, N>(f);
  }
}

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Two floats to a bf16 pair (low half = lo), round to nearest even.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Signed byte B of w as a float (one SDWA conversion).
template <int B>
__device__ __forceinline__ float sbyte(uint32_t w) {
  return (float)(int32_t)((int32_t)(w << (24 - 8 * B)) >> 24);
}

// Value of lane I of this lane's group of four (DPP quad permutation).
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), I * 0x55, 0xf, 0xf, false));
}

__device__ __forceinline__ u32x2_t load_nt8(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

// One tile's loads.  bf16: k[kk] = A pieces of MFMA kk, v[i] = 16 bytes of slot
// 4r + i.  int8 or fp8 codes: k[0..1] = 32 codes, v[i] = 8 codes of slot
// 4r + i, ks / vs = the scales of slot 4r + (c & 3).
template <int KV>
struct Tile;
template <>
struct Tile<GQA_BF16> {
  u32x4 k[4];
  u32x4 v[4];
};
template <>
struct Tile<GQA_I8> {
  u32x4 k[2];
  u32x2_t v[4];
  float ks, vs;
};
template <>
struct Tile<GQA_FP8> : Tile<GQA_I8> {};  // fp8 codes: the same bytes, another code

// Caches of one-byte codes with per-row scales (int8 or fp8).
template <int KV>
constexpr bool kQuant = KV != GQA_BF16;

// Two fp8 (E4M3) codes, bytes 2 HI .. 2 HI + 1 of w, as a bf16 pair (exact:
// every E4M3 value is a bf16 value; the conversion's scale is 1).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Online-softmax state of one wave: HB blocks of 16 query heads, each with its
// running reference maximum m (log2 units), denominator l and the transposed
// output sums (lane (r, c): head 16 hb + c at positions 8(4r + i) + e).
template <int HB>
struct State {
  float m[HB], l[HB];
  f32x4 acc[HB][8];
};

// Softmax variants inside a tile (VAR): soft-capped scores, and the rows of
// the tile (from virtual slot t0) that the sliding window leaves unattended.
struct TileVar {
  const AttnArgs* a;
  const SeqView* sv;
  int t0;
};

// One 16-slot tile for HB head blocks: the K and V operands are loaded and
// widened once and serve every block.
template <int KV, bool VAR, int HB>
__device__ __forceinline__ void tile_math(State<HB>& st, const u32x4 (&qf)[HB][4], const Tile<KV>& t, int lo,
                                          int valid, int r, float scale_log2,
                                          TileVar tvar = TileVar{nullptr, nullptr, 0}) {
  // Scores.
  u32x4 kf[4];
  if constexpr (KV == GQA_BF16) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[kk] = t.k[kk];
  } else if constexpr (KV == GQA_FP8) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = t.k[j][2 * h], w1 = t.k[j][2 * h + 1];
        kf[2 * j + h] = u32x4{fp8x2_bf16<false>(w0), fp8x2_bf16<true>(w0), fp8x2_bf16<false>(w1), fp8x2_bf16<true>(w1)};
      }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = t.k[j][2 * h], w1 = t.k[j][2 * h + 1];
        kf[2 * j + h] = u32x4{pk_bf16(sbyte<0>(w0), sbyte<1>(w0)), pk_bf16(sbyte<2>(w0), sbyte<3>(w0)),
                              pk_bf16(sbyte<0>(w1), sbyte<1>(w1)), pk_bf16(sbyte<2>(w1), sbyte<3>(w1))};
      }
  }
  float sv[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s = mfma_k32(kf[kk], qf[hb][kk], s);
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[hb][i] = s[i];
  }
  // Rows of this lane's four slots that take no weight.
  bool dead[4] = {false, false, false, false};
  if constexpr (VAR) {
    const AttnArgs& a = *tvar.a;
    if (a.window > 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dead[i] = unattended(*tvar.sv, phys_slot(*tvar.sv, tvar.t0 + 4 * r + i));
    }
  }
  if (lo > 0 || valid < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dead[i] = dead[i] || 4 * r + i < lo || 4 * r + i >= valid;
  }
  float ksc[4], vsc[4];
  if constexpr (kQuant<KV>) {
    ksc[0] = quad_bcast<0>(t.ks);
    ksc[1] = quad_bcast<1>(t.ks);
    ksc[2] = quad_bcast<2>(t.ks);
    ksc[3] = quad_bcast<3>(t.ks);
    vsc[0] = quad_bcast<0>(t.vs);
    vsc[1] = quad_bcast<1>(t.vs);
    vsc[2] = quad_bcast<2>(t.vs);
    vsc[3] = quad_bcast<3>(t.vs);
  }
  u32x4 pb[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    float* sc = sv[hb];
    if constexpr (kQuant<KV>) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[i] *= ksc[i];
    }
    if constexpr (VAR) {
      const AttnArgs& a = *tvar.a;
      if (a.cap_T > 0.f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = cap_score(sc[i], a.cap_T, a.cap_invT);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (dead[i]) sc[i] = kNegInfQ;
    // Softmax (per head 16 hb + c = this lane's column).  The reference m of
    // head c is the same in its four rows, so a lane tests its own scores
    // against it; the head's maximum over the tile (a cross-row reduction) is
    // needed only when some score jumped past it.
    const float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__any(mx * scale_log2 > st.m[hb] + kSlackQ)) {
      const float mc = rows_max(mx) * scale_log2;
      const float m_new = fmaxf(st.m[hb], mc);
      const float alpha = fast_exp2(st.m[hb] - m_new);  // 0 on the first tile
      st.l[hb] *= alpha;
      st.m[hb] = m_new;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[hb][e] *= alpha;
    }
    // With the sliding window a wave can meet tiles with no attended row before
    // its first attended one (m still -inf): their weights are 0, not NaN.
    const float nm = VAR && st.m[hb] == kNegInfQ ? 0.f : -st.m[hb];
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sc[i], scale_log2, nm));
    st.l[hb] += (p[0] + p[1]) + (p[2] + p[3]);
    if constexpr (kQuant<KV>) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] *= vsc[i];
    }
    // Each weight enters the V sum as a pair of bf16 values hi = bf16(p) and
    // lo = bf16(p - hi), so it is carried to about 2^-17 of its value (float32
    // arithmetic within the tolerance of a float32 sum).  The pair is stacked
    // along the K axis of one 16x16x32 MFMA: k = 8r + i is slot 4r + i times
    // its hi part, k = 8r + 4 + i the same slot times its lo part.
    const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
    pb[hb] = u32x4{h01, h23, pk_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01)),
                   pk_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23))};
  }
  // V sum: A operand of MFMA e = element 8c + e of slots 4r .. 4r + 3 (twice),
  // shared by the head blocks.  fp8: one byte permutation gathers element
  // pairs e, e + 1 of two slots, one conversion each turns them into bf16
  // pairs (vb[e][0]: slots 0 and 1, vb[e][1]: slots 2 and 3).
  uint32_t vb[8][2];
  if constexpr (KV == GQA_FP8) {
#pragma unroll
    for (int wd = 0; wd < 2; ++wd)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        constexpr uint32_t sel0 = 0x05010400u, sel1 = 0x07030602u;  // bytes {2k, 4+2k, 2k+1, 4+2k+1}
        const uint32_t sel = k == 0 ? sel0 : sel1;
        const uint32_t p01 = __builtin_amdgcn_perm(t.v[1][wd], t.v[0][wd], sel);
        const uint32_t p23 = __builtin_amdgcn_perm(t.v[3][wd], t.v[2][wd], sel);
        const int e0 = 4 * wd + 2 * k;
        vb[e0][0] = fp8x2_bf16<false>(p01);
        vb[e0 + 1][0] = fp8x2_bf16<true>(p01);
        vb[e0][1] = fp8x2_bf16<false>(p23);
        vb[e0 + 1][1] = fp8x2_bf16<true>(p23);
      }
  }
  unroll<0, 8>([&](auto ei) {
    constexpr int e = decltype(ei)::value;
    u32x2_t va;
    if constexpr (KV == GQA_FP8) {
      va = u32x2_t{vb[e][0], vb[e][1]};
    } else if constexpr (KV == GQA_BF16) {
      constexpr uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      va = u32x2_t{__builtin_amdgcn_perm(t.v[1][e >> 1], t.v[0][e >> 1], sel),
                   __builtin_amdgcn_perm(t.v[3][e >> 1], t.v[2][e >> 1], sel)};
    } else {
      constexpr int wd = e >> 2, by = e & 3;
      va = u32x2_t{pk_bf16(sbyte<by>(t.v[0][wd]), sbyte<by>(t.v[1][wd])),
                   pk_bf16(sbyte<by>(t.v[2][wd]), sbyte<by>(t.v[3][wd]))};
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) st.acc[hb][e] = mfma_k32(u32x4{va[0], va[1], va[0], va[1]}, pb[hb], st.acc[hb][e]);
  });
}

// One piece of work of a workgroup: virtual slots [t_begin, t_end) of
// (sequence b, kv-head h, query-head chunk hc).  `whole`: the piece is all of
// the sequence's slots, so its rows are final and go to `out`; otherwise they
// are partials (m, l, o) at rows pbase + pstride * g of the split workspace
// (g = head within the chunk).  Every wave of the workgroup calls it with the
// same arguments (it holds workgroup barriers).
struct Piece {
  int b, h, hc;
  int t_begin, t_end;  // virtual slots
  int L;               // lengths[b]
  SeqView view;
  bool whole;
  int64_t pbase, pstride;
};

// HP = 1: the workgroup's waves share one kv-head and split the piece's tiles
// into runs.  HP = NW (head-parallel, caches (B, S, Hkv, D)): the piece is a
// group of NW adjacent kv-heads and wave w takes kv-head w of the group over
// all of the piece's tiles, so the workgroup reads NW x 256 contiguous bytes
// of every slot row at once; each wave's heads are its own (no merge).
template <int KV, int NW, int HB, int HP, bool PAGED, bool VAR>
__device__ __forceinline__ void attend_piece(const AttnArgs& a, const Piece& pc, float (*sm_o)[16 * HB][kMergePitch],
                                             float (*sm_m)[16 * HB], float (*sm_l)[16 * HB]) {
  static_assert(HP == 1 || (HP == NW && HB == 1), "head-parallel waves carry one head block");
  constexpr int GW = 16 * HB;               // query heads per wave (and per workgroup)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 4;
  const int c = lane & 15;
  const int b = pc.b, h = HP > 1 ? pc.h * HP + wave : pc.h, hc = pc.hc;
  const int hq0 = h * a.G + GW * hc;       // first query head of this workgroup
  const int G = min(GW, a.G - GW * hc);   // query heads in this workgroup
  const int L = pc.L;
  const SeqView& view = pc.view;
  const int Lv = L - view.gap;
  const int t_begin = pc.t_begin;
  const int t_end = pc.t_end;

  // Fused step: slot L is taken from k_new / v_new (int8 caches: quantized here).
  const bool own_new = a.k_new != nullptr && Lv >= t_begin && Lv < t_end;
  const int t_cache_end = own_new ? Lv : t_end;

  constexpr int EB = KV == GQA_BF16 ? 2 : 1;  // bytes per cached element
  const int64_t base = PAGED ? 0 : row_head_offset(a, b, h);  // dense or slot-indexed row
  const int64_t rs = a.st;  // elements between consecutive slots (paged: within a block)

  // Tile grid.  When a kv-head's rows are contiguous, tiles start at 16-row
  // aligned cache addresses (4 KB for bf16, measured faster than tiles that
  // straddle 4 KB boundaries); a paged cache (block size a multiple of 16)
  // starts them at multiples of 16 slots, so a tile never crosses a block.
  // The leading rows before t_begin are masked.
  int tv = t_begin;
  if (PAGED) {
    tv = t_begin & ~15;
  } else if (rs == kDq && !VAR) {
    const uint64_t row = (reinterpret_cast<uintptr_t>(a.k_cache) / (kDq * EB)) + (uint64_t)(base / kDq + t_begin);
    tv = t_begin - (int)(row & 15);
  }
  // This wave's run: the split's tiles dealt out evenly (wave w takes tiles
  // [ceil(w T / NW), ceil((w + 1) T / NW))), so short sequences use every wave
  // too; only wave 0's first tile can hold leading rows, and it always holds a
  // valid one.  The new token goes to the last wave.
  const int ntile = t_cache_end > t_begin ? (t_cache_end - tv + 15) >> 4 : 0;
  constexpr int RUNS = HP > 1 ? 1 : NW;   // waves sharing the piece's tiles
  const int run = HP > 1 ? 0 : wave;
  const int w0 = tv + 16 * ((run * ntile + RUNS - 1) / RUNS);
  const int w1 = min(tv + 16 * (((run + 1) * ntile + RUNS - 1) / RUNS), t_cache_end);
  const bool new_here = own_new && run == RUNS - 1;

  // Query operand: positions matching the K operand's.
  const int64_t qrow = ((int64_t)b * a.Hq + hq0 + c) * kDq;
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + qrow;
  u32x4 qf[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int d0 = KV == GQA_BF16 ? 32 * kk + 8 * r : 64 * (kk >> 1) + 16 * r + 8 * (kk & 1);
      qf[hb][kk] = (16 * hb + c < G) ? *reinterpret_cast<const u32x4*>(qp + 16 * hb * kDq + d0) : u32x4{0, 0, 0, 0};
    }

  State<HB> st;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    st.m[hb] = kNegInfQ;
    st.l[hb] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[hb][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Rows are clamped into [t_begin, w1 - 1]: every load is in bounds and reads
  // a valid slot; clamped rows are masked to weight 0.
  const uint32_t rsb = (uint32_t)rs * EB;
  const char* kl = reinterpret_cast<const char*>(a.k_cache) + base * EB + 16 * r;
  const char* vl = reinterpret_cast<const char*>(a.v_cache) + base * EB + (KV == GQA_BF16 ? 16 : 8) * c;
  const int64_t sbase = base / kDq;     // scale index of slot 0 (dense rows are multiples of D)
  const int64_t sst = rs / kDq;         // scale entries between slots
  // Paged: a tile's rows lie in the block of its 16-slot origin (clamped into
  // the wave's run, so prefetches past the end stay in a mapped block); `blk`
  // is that block's table entry, loaded a tile pair ahead.
  const int last16 = max((w1 - 1) & ~15, tv);
  auto tile_origin = [&](int t0) { return max(min(t0, last16), tv); };
  auto entry = [&](int t0) -> int32_t {
    if (!PAGED) return 0;
    return a.map[(int64_t)b * a.max_blocks + (VAR ? phys_slot(view, tile_origin(t0)) : tile_origin(t0)) / a.bs];
  };
  // Virtual slot -> physical slot.  Paged tiles start on multiples of 16 and
  // the window's split point and gap are multiples of 16, so a whole paged
  // tile moves by the same amount (its block is that of its physical origin).
  auto phys = [&](int t) { return VAR ? phys_slot(view, t) : t; };
  auto load_tile = [&](int t0, Tile<KV>& t, int32_t blk) {
    const char* kt = kl;
    const char* vt = vl;
    int tc = 0;       // virtual origin of the tile's block (paged)
    int shift = 0;    // physical - virtual for the whole tile (paged)
    int64_t sb = sbase;  // int8: scale index of the row the tile's rows count from
    if (PAGED) {
      tc = tile_origin(t0);
      shift = phys(tc) - tc;
      const int64_t eoff = block_head_offset(a, blk, h) + (int64_t)((tc + shift) % a.bs) * rs;
      kt = reinterpret_cast<const char*>(a.k_cache) + eoff * EB + 16 * r;
      vt = reinterpret_cast<const char*>(a.v_cache) + eoff * EB + (KV == GQA_BF16 ? 16 : 8) * c;
      sb = eoff / kDq;  // rows are whole multiples of D elements
    }
    auto row = [&](int tvirt) -> uint32_t {  // row offset from the tile's block (paged) or slot 0
      const int cl = max(min(tvirt, w1 - 1), t_begin);
      return (uint32_t)(PAGED ? cl - tc : phys(cl));
    };
    const uint32_t rk = row(t0 + c);
    const char* p = kt + (uint64_t)rk * rsb;
    if constexpr (KV == GQA_BF16) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) t.k[kk] = load_nt16(p + 64 * kk);
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) t.k[j] = load_nt16(p + 64 * j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t rv = row(t0 + 4 * r + i);
      if constexpr (KV == GQA_BF16)
        t.v[i] = load_nt16(vt + (uint64_t)rv * rsb);
      else
        t.v[i] = load_nt8(vt + (uint64_t)rv * rsb);
    }
    if constexpr (kQuant<KV>) {
      const int64_t rsc = sb + (int64_t)row(t0 + 4 * r + (c & 3)) * sst;
      t.ks = __uint_as_float(load_nt4(a.k_scale + rsc));
      t.vs = __uint_as_float(load_nt4(a.v_scale + rsc));
    }
  };

  // Fused step, bf16: the new token is a tile whose only valid row is
  // k_new / v_new (row 0: lanes c = 0 for K, slot 0 = lanes of row r = 0, i = 0
  // for V); its bits are copied to slot L after the loop (read again there, so
  // the tile holds no registers across the loop).
  Tile<KV> tn;
  float new_ks = 0.f, new_vs = 0.f;  // int8: the new rows' scales
  if constexpr (KV == GQA_BF16) {
    if (new_here) {
      const int64_t nrow = ((int64_t)b * a.Hkv + h) * kDq;
      const uint16_t* knp = reinterpret_cast<const uint16_t*>(a.k_new) + nrow;
      const uint16_t* vnp = reinterpret_cast<const uint16_t*>(a.v_new) + nrow;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        tn.k[kk] = (c == 0) ? *reinterpret_cast<const u32x4*>(knp + 32 * kk + 8 * r) : u32x4{0, 0, 0, 0};
      tn.v[0] = (r == 0) ? *reinterpret_cast<const u32x4*>(vnp + 8 * c) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 1; i < 4; ++i) tn.v[i] = u32x4{0, 0, 0, 0};
    }
  } else {
    // Int8 (and fp8) caches: the new rows (bf16 activations) are quantized here by the
    // per-row rule (float32 row maximum, scale = max / 127 and codes =
    // round-half-even(x / scale) with correctly rounded divisions, clamped to
    // +-127; a zero row has scale 0 and codes 0).  Lane l quantizes elements
    // 2l and 2l + 1 of each row; the codes are regrouped into the tile's layout
    // (lanes (r, 0) hold key codes 64j + 16r .. +15, lanes (0, c) value codes
    // 8c .. 8c + 7) through this wave's merge buffer, which is idle until the
    // merge at the end of the piece.
    if (new_here) {
      const int64_t nrow = ((int64_t)b * a.Hkv + h) * kDq;
      const uint32_t kp = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(a.k_new) + nrow)[lane];
      const uint32_t vp = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(a.v_new) + nrow)[lane];
      const float k0 = bf16_lo(kp), k1 = bf16_hi(kp), v0 = bf16_lo(vp), v1 = bf16_hi(vp);
      const float kmax = wave_max(fmaxf(fabsf(k0), fabsf(k1)));
      const float vmax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
      // fp8 caches: the same rule with the code's largest value, 448, and the
      // E4M3 code of the clamped quotient (ties to even).
      constexpr float QMAX = KV == GQA_FP8 ? 448.f : 127.f;
      const float ksc = kmax / QMAX, vsc = vmax / QMAX;
      auto code = [](float x, float amax, float sc) -> uint32_t {
        if constexpr (KV == GQA_FP8) {
          return amax > 0.f ? e4m3_encode(fminf(fmaxf(x / sc, -QMAX), QMAX)) : 0u;
        } else {
          const float q = amax > 0.f ? fminf(fmaxf(rintf(x / sc), -127.f), 127.f) : 0.f;
          return (uint32_t)(int32_t)q & 0xffu;
        }
      };
      uint16_t* xb = reinterpret_cast<uint16_t*>(&sm_o[wave][0][0]);  // key codes at bytes 0..127, values 128..255
      xb[lane] = (uint16_t)(code(k0, kmax, ksc) | (code(k1, kmax, ksc) << 8));
      xb[64 + lane] = (uint16_t)(code(v0, vmax, vsc) | (code(v1, vmax, vsc) << 8));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint8_t* xr = reinterpret_cast<const uint8_t*>(xb);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(xr + 64 * j + 16 * r);
        tn.k[j] = c == 0 ? w : u32x4{0, 0, 0, 0};
      }
      const u32x2_t wv = *reinterpret_cast<const u32x2_t*>(xr + 128 + 8 * c);
      tn.v[0] = r == 0 ? wv : u32x2_t{0u, 0u};
#pragma unroll
      for (int i = 1; i < 4; ++i) tn.v[i] = u32x2_t{0u, 0u};
      tn.ks = new_ks = ksc;
      tn.vs = new_vs = vsc;
    }
  }

  // DEPTH tile register sets rotate, so the next DEPTH - 1 tiles' loads are
  // in flight during a tile's math (two sets: one tile ahead, with the
  // workgroup's waves sharing each CU's SIMDs).  The tile loaded at step d of
  // an iteration from t0 is t0 + 16 (d + DEPTH - 1), into set
  // (d + DEPTH - 1) mod DEPTH; en[s] is the table entry of the tile set s loads
  // next, fetched an iteration ahead.
  constexpr int DEPTH = 2;
  auto next_of = [](int s) { return s == DEPTH - 1 ? DEPTH - 1 : DEPTH + s; };  // tile offset set s loads, in tiles
  Tile<KV> ts[DEPTH];
  int32_t en[DEPTH];
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s) load_tile(w0 + 16 * s, ts[s], entry(w0 + 16 * s));
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) en[s] = entry(w0 + 16 * next_of(s));
  if (new_here) tile_math<KV, VAR, HB>(st, qf, tn, 0, 1, r, a.scale_log2, TileVar{&a, &view, Lv});
  if (w0 < w1) {
    const int nt = (w1 - w0 + 15) >> 4;
    int t0 = w0;
    for (int it = 0; it < nt / DEPTH; ++it) {
      int32_t nx[DEPTH];
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) nx[s] = entry(t0 + 16 * (DEPTH + next_of(s)));
      unroll<0, DEPTH>([&](auto di) {
        constexpr int d = decltype(di)::value;
        constexpr int s = (d + DEPTH - 1) % DEPTH;
        load_tile(t0 + 16 * (d + DEPTH - 1), ts[s], en[s]);  // past w1 it re-reads row w1 - 1
        tile_math<KV, VAR, HB>(st, qf, ts[d], t_begin - t0 - 16 * d, w1 - t0 - 16 * d, r, a.scale_log2,
                               TileVar{&a, &view, t0 + 16 * d});
      });
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) en[s] = nx[s];
      t0 += 16 * DEPTH;
    }
    // The remaining nt mod DEPTH (< DEPTH) tiles are already in sets 0 .. DEPTH - 2.
    unroll<0, DEPTH - 1>([&](auto di) {
      constexpr int d = decltype(di)::value;
      if (d < nt % DEPTH)
        tile_math<KV, VAR, HB>(st, qf, ts[d], t_begin - t0 - 16 * d, w1 - t0 - 16 * d, r, a.scale_log2,
                               TileVar{&a, &view, t0 + 16 * d});
    });
  }
  if constexpr (KV == GQA_BF16) {
    if (new_here && hc == 0) {  // one head chunk writes the appended row: a copy of k_new / v_new
      const int64_t off = slot_offset_checked(a, b, h, L);
      const int64_t nrow = ((int64_t)b * a.Hkv + h) * kDq;
      uint16_t* kw = reinterpret_cast<uint16_t*>(a.k_cache_w) + off;
      uint16_t* vw = reinterpret_cast<uint16_t*>(a.v_cache_w) + off;
      if (off >= 0 && c == 0) {
        const uint16_t* knp = reinterpret_cast<const uint16_t*>(a.k_new) + nrow;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          *reinterpret_cast<u32x4*>(kw + 32 * kk + 8 * r) = *reinterpret_cast<const u32x4*>(knp + 32 * kk + 8 * r);
      }
      if (off >= 0 && r == 0)
        *reinterpret_cast<u32x4*>(vw + 8 * c) =
            *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.v_new) + nrow + 8 * c);
    }
  } else {
    if (new_here && hc == 0) {  // the codes still sit in this wave's merge buffer
      const int64_t off = slot_offset_checked(a, b, h, L);
      int8_t* kw = reinterpret_cast<int8_t*>(a.k_cache_w) + off;
      int8_t* vw = reinterpret_cast<int8_t*>(a.v_cache_w) + off;
      const uint8_t* xr = reinterpret_cast<const uint8_t*>(&sm_o[wave][0][0]);
      if (off >= 0 && c == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          *reinterpret_cast<u32x4*>(kw + 64 * j + 16 * r) = *reinterpret_cast<const u32x4*>(xr + 64 * j + 16 * r);
      }
      if (off >= 0 && r == 0) *reinterpret_cast<u32x2_t*>(vw + 8 * c) = *reinterpret_cast<const u32x2_t*>(xr + 128 + 8 * c);
      if (off >= 0 && lane == 0) {
        a.k_scale_w[off / kDq] = new_ks;
        a.v_scale_w[off / kDq] = new_vs;
      }
    }
  }
  if constexpr (HP > 1) {
    // Head-parallel: lane (r, c) holds complete sums of head c at positions
    // 8(4r + i) + e; the wave stores its rows itself.
    const float lsum = rows_sum(st.l[0]);
    const int hq = hq0 + c;
    if (c < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 8 * (4 * r + i);
        if (pc.whole) {
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float x0 = st.acc[0][2 * e2][i], x1 = st.acc[0][2 * e2 + 1][i];
            if (VAR || a.sink != nullptr || a.smooth) {
              x0 = finish_row(a, hq, st.m[0], x0, lsum);
              x1 = finish_row(a, hq, st.m[0], x1, lsum);
            } else {
              const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
              x0 *= inv;
              x1 *= inv;
            }
            w[e2] = (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
          }
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + hq) * kDq + d0) =
              u32x4{w[0], w[1], w[2], w[3]};
        } else {
          const int64_t pi = pc.pbase + pc.pstride * (wave * a.G + c);
          float* po = a.part_o + pi * kDq + d0;
          *reinterpret_cast<f32x4*>(po) = f32x4{st.acc[0][0][i], st.acc[0][1][i], st.acc[0][2][i], st.acc[0][3][i]};
          *reinterpret_cast<f32x4*>(po + 4) =
              f32x4{st.acc[0][4][i], st.acc[0][5][i], st.acc[0][6][i], st.acc[0][7][i]};
          if (r == 0 && i == 0) {
            a.part_m[pi] = st.m[0];
            a.part_l[pi] = lsum;
          }
        }
      }
    }
    return;
  }
  // The merge below overwrites the merge buffers (the int8 new row's codes).
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Each lane holds complete sums of head 16 hb + c at positions 8(4r + i) + e.
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const float lsum = rows_sum(st.l[hb]);
    const int g = 16 * hb + c;
    if (g < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // positions 8(4r + i) .. +7: two 16-byte stores
        float* row = &sm_o[wave][g][8 * (4 * r + i)];
        *reinterpret_cast<f32x4*>(row) = f32x4{st.acc[hb][0][i], st.acc[hb][1][i], st.acc[hb][2][i], st.acc[hb][3][i]};
        *reinterpret_cast<f32x4*>(row + 4) =
            f32x4{st.acc[hb][4][i], st.acc[hb][5][i], st.acc[hb][6][i], st.acc[hb][7][i]};
      }
      if (r == 0) {
        sm_m[wave][g] = st.m[hb];
        sm_l[wave][g] = lsum;
      }
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * kDq; idx += 64 * NW) {
    const int g = idx / kDq;
    const int d = idx - g * kDq;
    float M = kNegInfQ;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
    float O = 0.f, Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][g];
      const float sc = mw == kNegInfQ ? 0.f : fast_exp2(mw - M);
      O += sm_o[w][g][d] * sc;
      Lsum += sm_l[w][g] * sc;
    }
    const int hq = hq0 + g;
    if (pc.whole) {
      reinterpret_cast<uint16_t*>(a.out)[((int64_t)b * a.Hq + hq) * kDq + d] =
          f32_to_bf16_rne(VAR || a.sink != nullptr || a.smooth ? finish_row(a, hq, M, O, Lsum)
                                                              : (Lsum > 0.f ? O / Lsum : 0.f));
    } else {
      const int64_t pi = pc.pbase + pc.pstride * g;
      a.part_o[pi * kDq + d] = O;
      if (d == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = Lsum;
      }
    }
  }
}


template <int KV, int NW, int HB, int HP, bool PAGED, bool VAR>
__global__ __launch_bounds__(64 * NW) void attend_mfma_qkv_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float sm_o[NW][16 * HB][kMergePitch];
  __shared__ float sm_m[NW][16 * HB];
  __shared__ float sm_l[NW][16 * HB];
  extern __shared__ int32_t sm_pre[];  // balanced mode: tile offsets of the sequences (B + 1 entries)

  auto piece_of = [&](int b, int h, int hc, int t_begin, int t_end, bool whole, int64_t pbase, int64_t pstride) {
    Piece pc;
    pc.b = b;
    pc.h = h;
    pc.hc = hc;
    pc.L = a.lengths[b];
    int n = pc.L + a.len_offset;
    n = n < 0 ? 0 : (n > a.S ? a.S : n);
    // Slots are walked in the sliding window's virtual order (the identity
    // without a window); the new token is the last virtual slot.
    pc.view = SeqView{n, n, 0, 0, 0};
    if constexpr (VAR) pc.view = seq_view(a, b, n);
    pc.t_begin = t_begin;
    pc.t_end = min(t_end, pc.view.nv);
    pc.whole = whole;
    pc.pbase = pbase;
    pc.pstride = pstride;
    return pc;
  };

  int lo = 0, hi = 0;  // balanced mode: this workgroup's tile range
  Piece split_piece;   // split mode: the workgroup's piece
  if (a.bal_pre != nullptr) {
    // Balanced mode (ragged batches), 16-slot tiles: see balanced.h.
    __shared__ int32_t wsum[NW];
    balanced_scan(a, 4, sm_pre, wsum);
    balanced_range(sm_pre, a.B, &lo, &hi);
    if (lo >= hi) return;
  } else {
    // Split mode: workgroup -> (split, query-head chunk, b, kv-head).  Groups
    // of more than 16 query heads are served 16 at a time by head chunks that
    // all read the same K/V rows; the chunks of one (b, kv-head) are numbered 8
    // apart, so the round-robin dispatch puts them on the same XCD at about the
    // same time and only the first of them reads the rows from HBM (the others
    // from L2).
    int x = blockIdx.x;
    const int split = x % a.nsplit;
    x /= a.nsplit;
    const int items = a.Hkv / HP;  // work items per sequence
    int hc = 0, bh = x;
    if (a.head_chunks > 1) {
      const int HC = a.head_chunks;
      const int units = a.B * items;
      const int grp = x / (8 * HC);
      const int gsz = min(8, units - grp * 8);  // the last group may hold fewer (b, kv-head) units
      const int rem = x - grp * 8 * HC;
      hc = rem / gsz;
      bh = grp * 8 + rem % gsz;
    }
    const int h = bh % items;
    const int b = bh / items;
    const int t_begin = split * a.split_tokens;
    Piece pc = piece_of(b, h, hc, t_begin, t_begin + a.split_tokens, false, 0, 0);
    const int nv = pc.view.nv;
    const int nact = nv == 0 ? 0 : min(a.nsplit, (nv + a.split_tokens - 1) / a.split_tokens);
    if (split >= max(nact, 1)) return;
    pc.whole = nact <= 1;
    pc.pbase = ((int64_t)b * a.Hq + h * HP * a.G + 16 * HB * hc) * a.nsplit + split;
    pc.pstride = a.nsplit;
    split_piece = pc;
  }

  // Split mode: the one piece; balanced mode: the pieces of [lo, hi), in order
  // (a range that holds only cost units of an item has no piece of it).
  if (a.bal_pre == nullptr) {
    attend_piece<KV, NW, HB, HP, PAGED, VAR>(a, split_piece, sm_o, sm_m, sm_l);
    return;
  }
  bool sync = false;
  for (int t = lo; t < hi;) {
    const BalancedPiece bp = balanced_piece(a, sm_pre, t, hi);
    t = bp.next;
    if (bp.j0 >= bp.j1) continue;
    if (sync) __syncthreads();  // the next piece reuses the merge buffers
    sync = true;
    attend_piece<KV, NW, HB, HP, PAGED, VAR>(a, piece_of(bp.b, bp.h, 0, 16 * bp.j0, 16 * bp.j1, bp.whole, bp.pbase, 1), sm_o,
                                     sm_m, sm_l);
  }
}


}  // namespace qkv

using qkv::attend_mfma_qkv_kernel;

// Dynamic LDS that, with the one-block kernel's 34 KB static arrays, exceeds
// half of a CU's 160 KB (one workgroup per CU).  The 135 KB of merge buffers
// of the two-block kernel already allow only one.
constexpr unsigned kOneWorkgroupLds = 48u * 1024u;

const bool kHaveMfmaQk = true;
const bool kHaveMfmaQkI8 = true;

template <int NW, int HB, int HP>
static const void* qk_kernel(const AttnArgs& a, bool var) {
  if (a.kv_dtype == GQA_I8 && a.map_kind == GQA_MAP_PAGED)
    return var ? reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_I8, NW, HB, HP, true, true>)
               : reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_I8, NW, HB, HP, true, false>);
  if (a.kv_dtype == GQA_I8)
    return var ? reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_I8, NW, HB, HP, false, true>)
               : reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_I8, NW, HB, HP, false, false>);
  if (a.kv_dtype == GQA_FP8 && a.map_kind == GQA_MAP_PAGED)
    return var ? reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_FP8, NW, HB, HP, true, true>)
               : reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_FP8, NW, HB, HP, true, false>);
  if (a.kv_dtype == GQA_FP8)
    return var ? reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_FP8, NW, HB, HP, false, true>)
               : reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_FP8, NW, HB, HP, false, false>);
  if (HB == 1 && a.map_kind == GQA_MAP_PAGED)
    return var ? reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_BF16, NW, HB, HP, true, true>)
               : reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_BF16, NW, HB, HP, true, false>);
  if (HB == 1)
    return var ? reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_BF16, NW, HB, HP, false, true>)
               : reinterpret_cast<const void*>(&attend_mfma_qkv_kernel<GQA_BF16, NW, HB, HP, false, false>);
  // bf16 caches with more than 16 heads run on the large-group kernel (two or
  // four head blocks per wave, K/V in registers, measured slower there).
  return nullptr;
}

// bf16 caches with up to 16 query heads per kv-head: 4 waves of one 16-head
// block each.  Int8 caches: the same for up to 16 heads; for 17..64 heads, 8
// waves of two 16-head blocks each (32 query heads per workgroup and head
// chunk).  Dense, slot-indexed or paged (block size a multiple of 16) caches.
hipError_t launch_attend_mfma_qk(const AttnArgs& a, const Plan& p, hipStream_t s) {
  if (a.head_chunks < 1) return hipErrorInvalidValue;
  const int per = (a.G + a.head_chunks - 1) / a.head_chunks;  // query heads per workgroup
  if (per > 32) return hipErrorInvalidValue;
  const int HB = per > 16 ? 2 : 1;
  const int NW = HB == 2 ? 8 : 4;
  if (a.D != qkv::kDq || a.G > 16 * HB * a.head_chunks || p.block != 64 * NW) return hipErrorInvalidValue;
  if (a.hp != 1 && (a.hp != NW || HB != 1 || a.Hkv % a.hp != 0)) return hipErrorInvalidValue;
  const bool var = a.window > 0 || a.cap_T > 0.f;  // in-loop variants (the sink is applied at the end)
  if ((a.kv_dtype == GQA_I8 || a.kv_dtype == GQA_FP8) &&
      (a.k_scale == nullptr || a.v_scale == nullptr || a.qo_dtype != GQA_BF16 ||
       (a.k_new != nullptr && (a.k_cache_w == nullptr || a.k_scale_w == nullptr || a.v_scale_w == nullptr))))
    return hipErrorInvalidValue;
  const void* fn = HB == 2     ? qk_kernel<8, 2, 1>(a, var)
                   : a.hp == 4 ? qk_kernel<4, 1, 4>(a, var)
                               : qk_kernel<4, 1, 1>(a, var);
  if (fn == nullptr) return hipErrorInvalidValue;
  AttnArgs arg = a;
  void* params[] = {&arg};
  // Balanced mode: one workgroup per CU (the tile ranges are equal only if all
  // of them run at once).  The dynamic LDS holds the sequences' tile offsets.
  unsigned lds = 0;
  if (a.bal_pre != nullptr) {
    if (a.B > kMaxBalancedBatch || a.head_chunks != 1 || p.grid < 1 || p.grid != a.bal_units)
      return hipErrorInvalidValue;
    lds = (unsigned)(a.B + 1) * 4u;
    if (HB == 1) lds = std::max<unsigned>(kOneWorkgroupLds, lds);
  }
  return hipLaunchKernel(fn, dim3(p.grid), dim3(p.block), params, lds, s);
}

}  // namespace gqa

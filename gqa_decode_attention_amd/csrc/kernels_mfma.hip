// Matrix-core (MFMA) attention kernels of the GQA decode step for gfx950,
// bf16 storage, head width 128.
//
// What is computed is the JAX "Grouped-Query Decode Step" page's definition
// (query head h reads cache head floor(h/G); s_j = q.K_j/sqrt(D) over the
// valid slots; softmax; o = sum_j w_j V_j) with the step of the "KV cache
// decode step" page (the new token's key/value are attended and appended at
// slot lengths[b]).  The softmax is evaluated online over 16-slot tiles
// (running maximum m, denominator l, unnormalised output o, rescaled by
// 2^(m_old - m_new) when the maximum grows); splits of the token axis leave
// (m, l, o) partials that the combine kernel merges.
//
// Kernel MFMA_QK (G <= 16).  One workgroup = NW waves (4) = one (sequence,
// kv-head, split); the split's valid 16-slot tiles are dealt out evenly and
// each wave walks its own run of them.  Per tile:
//   scores  S(16 slots x 16 heads) = K_tile(16 x 128) . Q^T(128 x 16) as four
//           v_mfma_f32_16x16x32_bf16.  Lane l = 16*r + c loads 16-byte pieces of
//           cache row t0 + c straight into the A operand (bytes 16r + 64kk of
//           the row for MFMA kk, so one instruction covers 16 rows x 64
//           contiguous bytes); the B operand holds query head c at the same
//           head-width positions (zero for c >= G).  Lane l then holds the
//           scores of slots t0 + 4r .. t0 + 4r + 3 for head c.
//   softmax the tile maximum per head is a max over the lane's 4 slots and
//           the 4 rows of lanes (two cross-row exchanges); exp2 with log2(e)
//           folded into the scale.
//   V sum   on the vector ALU in float32: lane l loads slots t0 + 4r + i,
//           elements 8c .. 8c + 7 (each load instruction covers 4 full rows),
//           and takes the weight of (slot, head g) from lane 16r + g with a DPP
//           row broadcast.
// Scores are exact products of bf16 values summed in float32; weights and sums
// stay float32 (bf16 only for the stored output).
//
// Fused step: the new token (slot lengths[b]) is not read from the cache; the
// workgroup whose split holds it runs one extra tile whose only valid row comes
// from k_new/v_new, and writes those bits into the cache slot.  No other
// workgroup reads that slot, so the write cannot race a read.
#include <type_traits>

#include "cache_map.h"
#include "device_common.h"
#include "internal.h"

namespace gqa {

const bool kHaveMfmaQk = true;
const bool kHaveMfmaAll = true;
const bool kHaveMfmaQkI8 = false;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInfM = -__builtin_inff();
constexpr int kD = 128;

// Lazy rescaling: a tile whose maximum exceeds the running reference m by at
// most this much (log2 units) keeps m, so its weights reach at most 2^8; only a
// larger jump moves m and rescales o and l.  o / l is the same softmax either
// way, and partials carry their own reference m into the combine.
constexpr float kRescaleSlack = 8.f;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Value of lane (16 * row + G) of `x`, in every lane of the same 16-lane row.
template <int G>
__device__ __forceinline__ float row_bcast(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + G, 0xf, 0xf, false));
}

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Online-softmax state of one wave: lane (r, c) keeps m (running max, log2
// units) and l (its own slots' share of the denominator) for head c, and the
// unnormalised output of head g at elements 8c .. 8c + 7 summed over its
// row's slots.
template <int GP>
struct WaveState {
  float m, l;
  float acc[GP][8];
};

// One 16-slot tile.  kf: this lane's A-operand pieces; vf[i]: slot t0 + 4r + i,
// elements 8c..8c+7; rows lo .. valid - 1 of the tile (from t0) are valid, the
// others are masked.
template <int GP>
__device__ __forceinline__ void tile_update(WaveState<GP>& st, const u32x4 (&qf)[4], const u32x4 (&kf)[4],
                                            const u32x4 (&vf)[4], int lo, int valid, int r, float scale_log2) {
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) s = mfma_16x16x32(kf[kk], qf[kk], s);
  // Raw scores; the scale log2(e)/sqrt(D) > 0 is folded into the exponent.
  float sv[4] = {s[0], s[1], s[2], s[3]};
  if (lo > 0 || valid < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * r + i < lo || 4 * r + i >= valid) sv[i] = kNegInfM;
  }
  float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mx = rows_max(mx);
  const float mc = mx * scale_log2;
  if (__any(mc > st.m + kRescaleSlack)) {  // some head's maximum jumped: move the reference
    const float m_new = fmaxf(st.m, mc);
    const float alpha = fast_exp2(st.m - m_new);  // 0 on the first tile
    st.l *= alpha;
    st.m = m_new;
    static_for<0, GP>([&](auto gi) {
      constexpr int g = decltype(gi)::value;
      const float ag = row_bcast<g>(alpha);
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[g][e] *= ag;
    });
  }
  const float nm = -st.m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sv[i], scale_log2, nm));
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[8];
    widen16<1>(vf[i], v);
    static_for<0, GP>([&](auto gi) {
      constexpr int g = decltype(gi)::value;
      const float pg = row_bcast<g>(p[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(pg, v[e], st.acc[g][e]);
    });
  }
}

template <int GP, int NW, bool PAGED>
__global__ __launch_bounds__(64 * NW) void attend_mfma_qk_kernel(AttnArgs a) {
  __shared__ float sm_o[NW][GP][kD];
  __shared__ float sm_m[NW][GP];
  __shared__ float sm_l[NW][GP];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 4;
  const int c = lane & 15;

  int x = blockIdx.x;
  const int split = x % a.nsplit;
  x /= a.nsplit;
  const int h = x % a.Hkv;
  const int b = x / a.Hkv;
  const int G = a.G;

  const int L = a.lengths[b];
  int n = L + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int t_begin = split * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, n);
  // Splits holding valid slots; split 0 always runs (it writes the output,
  // zeros when n = 0, if it is the only active split).
  const int nact = n == 0 ? 0 : min(a.nsplit, (n + a.split_tokens - 1) / a.split_tokens);
  if (split >= max(nact, 1)) return;

  // Fused step: slot L holds the new token; it is taken from k_new/v_new.
  const bool own_new = a.k_new != nullptr && L >= t_begin && L < t_end;
  const int t_cache_end = own_new ? L : t_end;

  const int64_t base = PAGED ? 0 : row_head_offset(a, b, h);  // dense or slot-indexed row
  const int64_t rs = a.st;  // elements between consecutive slots (paged: within a block)

  // Tile grid.  When a kv-head's slots are contiguous 256-byte rows, the
  // 16-slot tiles start at 4 KB-aligned cache addresses (measured faster than
  // tiles that straddle 4 KB boundaries); the grid then begins up to 15 slots
  // before t_begin and those leading rows are masked.  A paged cache (block
  // size a multiple of 16) starts tiles at multiples of 16 slots, so a tile
  // never crosses a block.
  int tv = t_begin;
  if (PAGED) {
    tv = t_begin & ~15;
  } else if (rs == kD) {
    const uint64_t row = (reinterpret_cast<uintptr_t>(a.k_cache) >> 8) + (uint64_t)((base >> 7) + t_begin);
    tv = t_begin - (int)(row & 15);
  }
  // This wave's run of cache slots: the split's 16-slot tiles dealt out
  // evenly (counts differ by at most one tile), so short sequences use every
  // wave too.  The run boundaries depend on lengths, the grid does not.
  // Wave w takes tiles [ceil(w T / NW), ceil((w + 1) T / NW)): the first waves
  // take the extra tiles and the last wave never has more than any other.
  // Only wave 0's first tile can hold leading rows; it always holds a valid one.
  const int ntile = t_cache_end > t_begin ? (t_cache_end - tv + 15) >> 4 : 0;
  const int w0 = tv + 16 * ((wave * ntile + NW - 1) / NW);
  const int w1 = min(tv + 16 * (((wave + 1) * ntile + NW - 1) / NW), t_cache_end);
  // The new token goes to the last wave.
  const bool new_here = own_new && wave == NW - 1;

  const int64_t qrow = ((int64_t)b * a.Hq + (int64_t)h * G + c) * kD;
  u32x4 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qf[kk] = (c < G) ? load16(reinterpret_cast<const uint16_t*>(a.q) + qrow + 32 * kk + 8 * r) : u32x4{0, 0, 0, 0};
  }

  WaveState<GP> st;
  st.m = kNegInfM;
  st.l = 0.f;
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[g][e] = 0.f;

  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k_cache) + base;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v_cache) + base;

  // Rows past the wave's last valid slot are clamped to that slot, rows before
  // t_begin to t_begin: every load is unconditional and in bounds, nothing at
  // or beyond the valid length is ever read, and the clamped rows get score
  // -inf, i.e. weight exactly 0, on finite values.  A row address is one
  // 32 x 32 -> 64-bit multiply-add (the byte stride between slots fits 32 bits
  // and clamped rows are never negative).
  const uint32_t rsb = (uint32_t)rs * 2u;
  const char* kl = reinterpret_cast<const char*>(kb) + 16 * r;
  const char* vl = reinterpret_cast<const char*>(vb) + 16 * c;
  // Paged: a tile's rows lie in the block of its 16-slot origin tc (clamped
  // into the wave's run, so prefetches past the end stay in a mapped block);
  // `blk` is that block's table entry, loaded a tile pair ahead and kept in a
  // vector register until its tile is loaded (its wait is then far behind it).
  const int last16 = max((w1 - 1) & ~15, tv);
  auto tile_origin = [&](int t0) { return max(min(t0, last16), tv); };
  auto entry = [&](int t0) -> int32_t {
    if (!PAGED) return 0;
    return a.map[(int64_t)b * a.max_blocks + tile_origin(t0) / a.bs];
  };
  auto load_tile = [&](int t0, u32x4 (&k)[4], u32x4 (&v)[4], int32_t blk) {
    const char* kt = kl;
    const char* vt = vl;
    int tc = 0;
    if (PAGED) {
      tc = tile_origin(t0);
      const int64_t off = (block_head_offset(a, blk, h) + (int64_t)(tc % a.bs) * rs) * 2;
      kt = reinterpret_cast<const char*>(a.k_cache) + off + 16 * r;
      vt = reinterpret_cast<const char*>(a.v_cache) + off + 16 * c;
    }
    const uint32_t rk = (uint32_t)(max(min(t0 + c, w1 - 1), t_begin) - tc);
    const char* p = kt + (uint64_t)rk * rsb;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) k[kk] = load_nt16(p + 64 * kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t rv = (uint32_t)(max(min(t0 + 4 * r + i, w1 - 1), t_begin) - tc);
      v[i] = load_nt16(vt + (uint64_t)rv * rsb);
    }
  };

  // The new token is a tile whose only valid row is k_new/v_new; its loads are
  // issued before the first cache tile's, and its bits are copied to slot L
  // after the loop (no store is in flight while the tiles stream).
  u32x4 knw[4], vnw;
  if (new_here) {
    const int64_t nrow = ((int64_t)b * a.Hkv + h) * kD;
    const uint16_t* knp = reinterpret_cast<const uint16_t*>(a.k_new) + nrow;
    const uint16_t* vnp = reinterpret_cast<const uint16_t*>(a.v_new) + nrow;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) knw[kk] = (c == 0) ? load16(knp + 32 * kk + 8 * r) : u32x4{0, 0, 0, 0};
    vnw = (r == 0) ? load16(vnp + 8 * c) : u32x4{0, 0, 0, 0};
  }
  // Two register sets alternate, so the next tile's loads are in flight during
  // this tile's math and no register copy waits for them.
  u32x4 ka[4], va[4], kc[4], vc[4];
  int32_t eC = entry(w0 + 16), eA = entry(w0 + 32);  // table entries of the first tile pair's successors
  load_tile(w0, ka, va, entry(w0));
  if (new_here) {
    const u32x4 vf[4] = {vnw, u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}, u32x4{0, 0, 0, 0}};
    tile_update<GP>(st, qf, knw, vf, 0, 1, r, a.scale_log2);
  }
  if (w0 < w1) {
    const int nt = (w1 - w0 + 15) >> 4;
    int t0 = w0;
    for (int it = 0; it < nt / 2; ++it) {
      const int32_t nC = entry(t0 + 48), nA = entry(t0 + 64);
      load_tile(t0 + 16, kc, vc, eC);
      tile_update<GP>(st, qf, ka, va, t_begin - t0, w1 - t0, r, a.scale_log2);
      load_tile(t0 + 32, ka, va, eA);  // past w1 it re-reads row w1 - 1
      tile_update<GP>(st, qf, kc, vc, t_begin - t0 - 16, w1 - t0 - 16, r, a.scale_log2);
      eC = nC;
      eA = nA;
      t0 += 32;
    }
    if (nt & 1) tile_update<GP>(st, qf, ka, va, t_begin - t0, w1 - t0, r, a.scale_log2);
  }
  if (new_here) {
    const int64_t off = slot_offset_checked(a, b, h, L);  // -1: the map names no valid row/block
    uint16_t* kw = reinterpret_cast<uint16_t*>(a.k_cache_w) + off;
    uint16_t* vw = reinterpret_cast<uint16_t*>(a.v_cache_w) + off;
    if (off >= 0 && c == 0) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) store16(kw + 32 * kk + 8 * r, knw[kk]);
    }
    if (off >= 0 && r == 0) store16(vw + 8 * c, vnw);
  }

  // Merge the 4 rows of lanes of each wave (disjoint slots, same running max).
  st.l = rows_sum(st.l);
#pragma unroll
  for (int g = 0; g < GP; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st.acc[g][e] = rows_sum(st.acc[g][e]);
    }
  if (r == 0) {
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[wave][g][8 * c + e] = st.acc[g][e];
    if (c < GP) {
      sm_m[wave][c] = st.m;
      sm_l[wave][c] = st.l;
    }
  }
  __syncthreads();

  // Merge the NW waves; write the output, or this split's partial.
  for (int idx = threadIdx.x; idx < G * kD; idx += 64 * NW) {
    const int g = idx / kD;
    const int d = idx - g * kD;
    float M = kNegInfM;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
    float O = 0.f, Lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][g];
      const float sc = mw == kNegInfM ? 0.f : fast_exp2(mw - M);
      O += sm_o[w][g][d] * sc;
      Lsum += sm_l[w][g] * sc;
    }
    const int hq = h * G + g;
    if (nact <= 1) {
      reinterpret_cast<uint16_t*>(a.out)[((int64_t)b * a.Hq + hq) * kD + d] =
          f32_to_bf16_rne(Lsum > 0.f ? O / Lsum : 0.f);
    } else {
      const int64_t pi = ((int64_t)b * a.Hq + hq) * a.nsplit + split;
      a.part_o[pi * kD + d] = O;
      if (d == 0) {
        a.part_m[pi] = M;
        a.part_l[pi] = Lsum;
      }
    }
  }
}

template <int GP>
static hipError_t launch_qk_t(const AttnArgs& a, const Plan& p, hipStream_t s) {
  constexpr int NW = 4;
  if (p.block != 64 * NW) return hipErrorInvalidValue;
  AttnArgs arg = a;
  void* params[] = {&arg};
  const void* fn = a.map_kind == GQA_MAP_PAGED ? reinterpret_cast<const void*>(&attend_mfma_qk_kernel<GP, NW, true>)
                                               : reinterpret_cast<const void*>(&attend_mfma_qk_kernel<GP, NW, false>);
  return hipLaunchKernel(fn, dim3(p.grid), dim3(p.block), params, 0, s);
}

hipError_t launch_attend_mfma_qk(const AttnArgs& a, const Plan& p, hipStream_t s) {
  if (a.D != kD || a.G > 16) return hipErrorInvalidValue;
  if (a.G <= 1) return launch_qk_t<1>(a, p, s);
  if (a.G <= 2) return launch_qk_t<2>(a, p, s);
  if (a.G <= 4) return launch_qk_t<4>(a, p, s);
  if (a.G <= 8) return launch_qk_t<8>(a, p, s);
  return launch_qk_t<16>(a, p, s);
}

// ---------------------------------------------------------------------------
// Kernel MFMA_ALL (16 < G <= 64): scores and the V sum both on MFMA.
//
// One workgroup = 4 waves = one (sequence, kv-head, split).  The workgroup
// stages 32-slot K and V tiles in LDS (double-buffered, rows padded to 288
// bytes to spread LDS banks); wave w owns query heads 16w .. 16w + 15 and
// reads every tile from LDS.  Per tile and wave:
//   scores  two 16-slot halves, S^T(16 slots x 16 heads) = K(16 x 128) . Q^T,
//           four v_mfma_f32_16x16x32_bf16 each (A operand: 16-byte LDS reads of
//           K rows; B operand: the wave's query heads).  Lane (r, c) holds slots
//           4r .. 4r+3 of each half for head c.
//   softmax as in MFMA_QK, over the 32 slots.
//   V sum   O(16 heads x 128) += P(16 x 32 slots) . V(32 x 128) as eight MFMAs
//           (one per 16-column block).  The A operand is the weights lane (r, c)
//           already holds (head c; slots 4r..4r+3 of the first half then of the
//           second half, rounded to bf16); the B operand -- V transposed, 8 slots
//           of one column per lane -- comes from two ds_read_b64_tr_b16 per
//           block: within each 16-lane group, lane rho names the 4 elements at
//           slot 4r + rho/4, columns 16nb + 4(rho mod 4) .. +3, and lane c
//           receives column 16nb + c of the 4 slots.
// The weights enter the V-sum MFMA rounded to bf16 (their sum l stays float32);
// the accumulation is float32.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kTileT = 32;    // slots per LDS tile
constexpr int kPitch = 144;   // LDS row pitch in bf16 elements (288 bytes)

__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(const_cast<uint16_t*>(p))));
}

// Two floats to a bf16 pair (low half = lo) with gfx950's v_cvt_pk_bf16_f32,
// round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}


template <bool PAGED>
__global__ __launch_bounds__(256) void attend_mfma_all_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sk[2][kTileT * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sv[2][kTileT * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane >> 4;
  const int c = lane & 15;

  int x = blockIdx.x;
  const int split = x % a.nsplit;
  x /= a.nsplit;
  const int h = x % a.Hkv;
  const int b = x / a.Hkv;
  const int G = a.G;

  const int L = a.lengths[b];
  int n = L + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int t_begin = split * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, n);
  const int nact = n == 0 ? 0 : min(a.nsplit, (n + a.split_tokens - 1) / a.split_tokens);
  if (split >= max(nact, 1)) return;
  const bool own_new = a.k_new != nullptr && L >= t_begin && L < t_end;

  const int hw = wave * 16;  // first head of this wave
  const int64_t qrow = ((int64_t)b * a.Hq + (int64_t)h * G + hw + c) * kD;
  u32x4 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = (hw + c < G) ? load16(reinterpret_cast<const uint16_t*>(a.q) + qrow + 32 * kk + 8 * r)
                          : u32x4{0, 0, 0, 0};

  float m = kNegInfM, l = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) O[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t base = PAGED ? 0 : row_head_offset(a, b, h);  // dense or slot-indexed row
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k_cache) + base;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v_cache) + base;
  const int64_t rs = a.st;
  const int64_t nrow = ((int64_t)b * a.Hkv + h) * kD;
  // Tile grid origin: the split start, or for a paged cache (block size a
  // multiple of 16) the multiple of 16 at or below it, so each 16-row half of a
  // tile lies in one block; rows before t_begin are clamped and masked.
  const int tv = PAGED ? (t_begin & ~15) : t_begin;
  const int last16 = max((t_end - 1) & ~15, tv);

  // Cooperative tile load: thread t moves 16 bytes (piece t & 15) of rows
  // t >> 4 and 16 + (t >> 4) of a 32-slot tile.  Rows past the split's last
  // valid slot are clamped to it, so every load reads a valid slot and no load
  // carries a condition (the count of loads in flight is then the same on every
  // path, and each LDS write waits only for its own tile).
  // Fused step: the appended slot L is the owning split's last valid slot.  The
  // cache still holds stale bits there, so when the tile holding L is written
  // to LDS its rows >= L take the new key/value from registers (rows past L are
  // masked and only need finite values); the new bits are copied to the cache
  // slot after the loop (no store is in flight while the tiles stream).
  const int prow = tid >> 4;
  const int piece = tid & 15;
  struct Regs {
    u32x4 k[2], v[2];
  };
  u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
  if (own_new) {
    kn = load16(reinterpret_cast<const uint16_t*>(a.k_new) + nrow + 8 * piece);
    vn = load16(reinterpret_cast<const uint16_t*>(a.v_new) + nrow + 8 * piece);
  }
  // Paged: the table entries of a tile's two 16-row halves, loaded a tile pair
  // before the tile itself (clamped into the split, like the rows).
  struct Ent {
    int32_t e[2];
  };
  auto entries = [&](int t0) -> Ent {
    Ent en = {{0, 0}};
    if (PAGED) {
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int hc = max(min(t0 + 16 * q2, last16), tv);
        en.e[q2] = a.map[(int64_t)b * a.max_blocks + hc / a.bs];
      }
    }
    return en;
  };
  auto gload = [&](int t0, Regs& R, const Ent& en) {
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int rc = max(min(t0 + prow + 16 * q2, t_end - 1), t_begin);
      int64_t off;
      if (PAGED) {
        const int hc = max(min(t0 + 16 * q2, last16), tv);
        off = block_head_offset(a, en.e[q2], h) + (int64_t)(hc % a.bs + (rc - hc)) * rs + 8 * piece;
      } else {
        off = (int64_t)rc * rs + 8 * piece;
      }
      R.k[q2] = load_nt16(kb + off);
      R.v[q2] = load_nt16(vb + off);
    }
  };
  auto swrite = [&](int t0, int buf, const Regs& R) {
    const bool holds_new = own_new && t0 + kTileT > L;  // uniform
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int row = prow + 16 * q2;
      const bool nw = holds_new && t0 + row >= L;
      *reinterpret_cast<u32x4*>(&sk[buf][row * kPitch + 8 * piece]) = nw ? kn : R.k[q2];
      *reinterpret_cast<u32x4*>(&sv[buf][row * kPitch + 8 * piece]) = nw ? vn : R.v[q2];
    }
  };

  // One tile: compute on LDS buffer `buf`, then move the next tile (register
  // set Rn) into the other buffer; Rl receives the tile after that.
  auto compute_tile = [&](int t0, int buf) {
    const uint16_t* K = sk[buf];
    const uint16_t* V = sv[buf];
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(&K[c * kPitch + 32 * kk + 8 * r]);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(&K[(16 + c) * kPitch + 32 * kk + 8 * r]);
      s0 = mfma_16x16x32(a0, qf[kk], s0);
      s1 = mfma_16x16x32(a1, qf[kk], s1);
    }
    // Raw scores; the scale log2(e)/sqrt(D) is positive, so the maximum is
    // taken on raw scores and the scale is folded into the exponent's fma.
    float sc[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    if (t0 + kTileT > t_end || t0 < t_begin) {  // the split's first (paged) or last, partial tile
      const int valid = t_end - t0;
      const int lo = t_begin - t0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * r + i >= valid || 4 * r + i < lo) sc[i] = kNegInfM;
        if (16 + 4 * r + i >= valid || 16 + 4 * r + i < lo) sc[4 + i] = kNegInfM;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = rows_max(mx);
    const float mc = mx * a.scale_log2;
    if (__any(mc > m + kRescaleSlack)) {  // some head's maximum jumped: move the reference
      const float m_new = fmaxf(m, mc);
      const float alpha = fast_exp2(m - m_new);  // 0 on the first tile
      l *= alpha;
      m = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * r + i);  // alpha of head 4r + i
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) O[nb][i] *= ai;
      }
    }
    const float nm = -m;
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = fast_exp2(fmaf(sc[i], a.scale_log2, nm));
      ps += p[i];
    }
    l += ps;
    const u32x4 pa = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])};
    const int trow = 4 * r + (c >> 2);
    const int tcol = 4 * (c & 3);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const s16x4 lo = lds_read_tr16(&V[trow * kPitch + 16 * nb + tcol]);
      const s16x4 hi = lds_read_tr16(&V[(16 + trow) * kPitch + 16 * nb + tcol]);
      const u32x4 vt = {(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                        (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                        (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                        (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
      O[nb] = mfma_16x16x32(pa, vt, O[nb]);
    }
  };
  // Two register sets keep two tiles in flight: at the top of each iteration
  // tile t0 sits in LDS buffer `buf` and R1 is loading tile t0 + T.  Loads of
  // tiles past the end clamp to the last valid row (cache hits, never used), so
  // every path issues the same loads, the loop has one exit, and each LDS write
  // waits only for its own tile's loads.
  if (t_begin < t_end) {
    const int ntile = (t_end - tv + kTileT - 1) / kTileT;
    Regs R0, R1;
    gload(tv, R0, entries(tv));
    gload(tv + kTileT, R1, entries(tv + kTileT));
    Ent e2 = entries(tv + 2 * kTileT), e3 = entries(tv + 3 * kTileT);
    swrite(tv, 0, R0);
    __syncthreads();
    int buf = 0;
    int t0 = tv;
    for (int it = 0; it < ntile / 2; ++it) {
      const Ent n2 = entries(t0 + 4 * kTileT), n3 = entries(t0 + 5 * kTileT);
      gload(t0 + 2 * kTileT, R0, e2);
      compute_tile(t0, buf);
      swrite(t0 + kTileT, buf ^ 1, R1);
      __syncthreads();
      buf ^= 1;
      gload(t0 + 3 * kTileT, R1, e3);
      compute_tile(t0 + kTileT, buf);
      swrite(t0 + 2 * kTileT, buf ^ 1, R0);
      __syncthreads();
      buf ^= 1;
      e2 = n2;
      e3 = n3;
      t0 += 2 * kTileT;
    }
    if (ntile & 1) compute_tile(t0, buf);
  }

  if (own_new && prow == 0) {  // the appended slot (skipped if the map names no valid row/block)
    const int64_t off = slot_offset_checked(a, b, h, L);
    if (off >= 0) {
      store16(reinterpret_cast<uint16_t*>(a.k_cache_w) + off + 8 * piece, kn);
      store16(reinterpret_cast<uint16_t*>(a.v_cache_w) + off + 8 * piece, vn);
    }
  }

  // Denominator and max per head: lane (r, c) holds head c; the output rows of
  // lane (r, c) are heads 4r + i.
  l = rows_sum(l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * r + i;  // head within the wave
    const float li = __shfl(l, hl);
    const float mi = __shfl(m, hl);
    if (hw + hl >= G) continue;
    const int hq = h * G + hw + hl;
    if (nact <= 1) {
      const float inv = li > 0.f ? 1.f / li : 0.f;
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + hq) * kD;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb + c] = f32_to_bf16_rne(O[nb][i] * inv);
    } else {
      const int64_t pi = ((int64_t)b * a.Hq + hq) * a.nsplit + split;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) a.part_o[pi * kD + 16 * nb + c] = O[nb][i];
      if (c == 0) {
        a.part_m[pi] = mi;
        a.part_l[pi] = li;
      }
    }
  }
}

hipError_t launch_attend_mfma_all(const AttnArgs& a, const Plan& p, hipStream_t s) {
  if (a.D != kD || a.G > 64) return hipErrorInvalidValue;
  AttnArgs arg = a;
  void* params[] = {&arg};
  const void* fn = a.map_kind == GQA_MAP_PAGED ? reinterpret_cast<const void*>(&attend_mfma_all_kernel<true>)
                                               : reinterpret_cast<const void*>(&attend_mfma_all_kernel<false>);
  return hipLaunchKernel(fn, dim3(p.grid), dim3(256), params, 0, s);
}

}  // namespace gqa

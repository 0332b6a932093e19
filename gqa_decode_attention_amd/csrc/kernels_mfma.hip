// Matrix-core (MFMA) attention kernel of the GQA decode step for gfx950 for
// large groups (16 < G <= 64), bf16 storage, head width 128.  (Groups of up to
// 16 query heads, and int8 and fp8 caches, run the kernel in kernels_mfma_qkv.hip.)
//
// What is computed is the JAX "Grouped-Query Decode Step" page's definition
// (query head h reads cache head floor(h/G); s_j = q.K_j/sqrt(D) over the
// valid slots; softmax; o = sum_j w_j V_j) with the step of the "KV cache
// decode step" page (the new token's key/value are attended and appended at
// slot lengths[b]).  The softmax is evaluated online over 32-slot tiles
// (running maximum m, denominator l, unnormalised output o, rescaled by
// 2^(m_old - m_new) when the maximum grows past a slack); splits of the token
// axis leave (m, l, o) partials that the combine kernel merges.
//
// Fused step: the new token (slot lengths[b]) is not read from the cache; the
// workgroup whose split holds it substitutes k_new/v_new for that row, and
// writes those bits into the cache slot.  No other workgroup reads that slot,
// so the write cannot race a read.
#include <type_traits>

#include "cache_map.h"
#include "device_common.h"
#include "internal.h"
#include "rope_dev.h"
#include "variants.h"

namespace gqa {

const bool kHaveMfmaAll = true;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInfM = -__builtin_inff();
constexpr int kD = 128;

// Lazy rescaling: a tile whose maximum exceeds the running reference m by at
// most 8 (log2 units) keeps m, so its weights reach at most 2^8; only a larger
// jump -- a weight above 2^8 -- moves m and rescales o and l.  o / l is the
// same softmax either way, and partials carry their own reference m into the
// combine.
constexpr float kRescaleJump = 256.f;

__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------------------
// Kernel MFMA_ALL (16 < G <= 64): scores and the V sum both on MFMA.
//
// Split form: one workgroup = 4 waves = one (sequence, kv-head, split).  The
// workgroup stages 32-slot K and V tiles in LDS (three buffers, rows padded to
// 288 bytes to spread LDS banks); wave w owns query heads 16w .. 16w + 15 and
// reads every tile from LDS.  (The whole-item form further below runs the same
// tile math in 8-wave workgroups over whole items.)  Per tile and wave:
//   scores  two 16-slot halves, S^T(16 slots x 16 heads) = K(16 x 128) . Q^T,
//           four v_mfma_f32_16x16x32_bf16 each (A operand: 16-byte LDS reads of
//           K rows; B operand: the wave's query heads).  Lane (r, c) holds slots
//           4r .. 4r+3 of each half for head c.
//   softmax as in MFMA_QK, over the 32 slots.
//   V sum   O(16 heads x 128) += P(16 x 32 slots) . V(32 x 128) as eight MFMAs
//           (one per 16-column block).  The A operand is the weights lane (r, c)
//           already holds (head c; slots 4r..4r+3 of the first half then of the
//           second half); the B operand -- V transposed, 8 slots
//           of one column per lane -- comes from two ds_read_b64_tr_b16 per
//           block: within each 16-lane group, lane rho names the 4 elements at
//           slot 4r + rho/4, columns 16nb + 4(rho mod 4) .. +3, and lane c
//           receives column 16nb + c of the 4 slots.  Each weight is split
//           into bf16 hi and lo parts with one MFMA each (sixteen per tile).
// Scores are exact products summed in float32; the weights reach the V sum
// with about 16 significant bits (hi + lo) and everything accumulates in
// float32.
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

// One step of the tile loop for the wave's 16 query heads (see the kernel
// comment below).  SCORES: the scores of the K tile in LDS (virtual slots t0
// ..), masking of the slots outside [t_begin, t_end) (and the window's
// unattended rows), and their weights, packed as bf16 hi / lo pairs into
// (pa, pl) for the next step; the running reference m and the denominator l
// follow.  VSUM: the V sum of the previous tile (V tile in LDS, its weights in
// (pa, pl) from the step before) into O.  One step does both, so the matrix
// cores run one tile's V sum while the vector ALU computes the next tile's
// weights: those are computed against the current reference, and recomputed
// only when some score jumped past it (O -- the V sum just issued included --
// and l are then rescaled first).
template <bool VAR, bool SCORES, bool VSUM>
__device__ __forceinline__ void all_step(const AttnArgs& a, const uint16_t* K, const uint16_t* V,
                                         const u32x4 (&qf)[4], int t0, int t_begin, int t_end,
                                         const SeqView& view, float& m, float& l, f32x4 (&O)[8], u32x4& pa,
                                         u32x4& pl) {
  const int lane = threadIdx.x & 63;
  const int r = lane >> 4;
  const int c = lane & 15;
  float sc[8];
  if constexpr (SCORES) {
    auto phys = [&](int t) { return VAR ? phys_slot(view, t) : t; };
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = s0[i];
      sc[4 + i] = s1[i];
    }
    if constexpr (VAR) {
      if (a.cap_T > 0.f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = cap_score(sc[i], a.cap_T, a.cap_invT);
      }
      if (a.window > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (unattended(view, phys(t0 + 4 * r + i))) sc[i] = kNegInfM;
          if (unattended(view, phys(t0 + 16 + 4 * r + i))) sc[4 + i] = kNegInfM;
        }
      }
    }
    // A piece's first (paged) or last, partial tile: a real (uniform) branch,
    // so whole tiles run no per-row compares.
    if (__builtin_expect(__builtin_amdgcn_readfirstlane(t0 + kTileT > t_end || t0 < t_begin), 0)) {
      const int valid = t_end - t0;
      const int lo = t_begin - t0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * r + i >= valid || 4 * r + i < lo) sc[i] = kNegInfM;
        if (16 + 4 * r + i >= valid || 16 + 4 * r + i < lo) sc[4 + i] = kNegInfM;
      }
    }
  }
  if constexpr (VSUM) {
    // O(16 heads x 128) += P(16 x 32 slots) . V(32 x 128), each weight as its
    // bf16 hi part then its lo part (about 16 significant bits, so the
    // weighted sum keeps float32 accuracy), accumulating in float32.
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
      O[nb] = mfma_16x16x32(pl, vt, mfma_16x16x32(pa, vt, O[nb]));
    }
  }
  if constexpr (SCORES) {
    // The weights against the current reference, and their largest value: a
    // weight above 2^slack means some score jumped past the reference.  (With
    // no reference yet, m = -inf, any attended score gives an infinite weight
    // and so the rescale; masked scores give 0.)  Testing the weights rather
    // than the scores keeps their computation ahead of the branch, next to
    // the V sum's MFMAs.
    auto weights = [&](float nm, u32x4& wa, u32x4& wl, float& pmax) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(sc[i], a.scale_log2, nm));
      pmax = fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])), fmaxf(fmaxf(p[4], p[5]), fmaxf(p[6], p[7])));
      wa = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                 pack_bf16x2(p[6], p[7])};
      wl = u32x4{pack_bf16x2(p[0] - bf16_lo(wa[0]), p[1] - bf16_hi(wa[0])),
                 pack_bf16x2(p[2] - bf16_lo(wa[1]), p[3] - bf16_hi(wa[1])),
                 pack_bf16x2(p[4] - bf16_lo(wa[2]), p[5] - bf16_hi(wa[2])),
                 pack_bf16x2(p[6] - bf16_lo(wa[3]), p[7] - bf16_hi(wa[3]))};
      return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    };
    u32x4 wa, wl;
    float pmax;
    float ps = weights(m == kNegInfM ? __FLT_MAX__ : -m, wa, wl, pmax);
    if (__any(pmax > kRescaleJump)) {  // some head's maximum jumped: move the reference
      // The reference m of head c is the same in its four rows; the head's
      // new maximum over the tile is a cross-row reduction.
      const float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      const float mc = rows_max(mx) * a.scale_log2;
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
      // With the sliding window a head can still have no attended row (m
      // stays -inf): its weights are 0, not NaN.
      ps = weights(m == kNegInfM ? 0.f : -m, wa, wl, pmax);
    }
    l += ps;
    pa = wa;
    pl = wl;
  }
}

// The wave's query operands: head hw + c (zero past G) at head-width
// positions 32kk + 8r .. 32kk + 8r + 7, rotated (and normalized) at rotary
// row rp when `rope`.
__device__ __forceinline__ void load_q_frags(const AttnArgs& a, int b, int h, int hw, bool rope, int rp,
                                             u32x4 (&qf)[4]) {
  const int lane = threadIdx.x & 63;
  const int r = lane >> 4;
  const int c = lane & 15;
  const int G = a.G;
  const int64_t qrow = ((int64_t)b * a.Hq + (int64_t)h * G + hw + c) * kD;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = (hw + c < G) ? load16(reinterpret_cast<const uint16_t*>(a.q) + qrow + 32 * kk + 8 * r)
                          : u32x4{0, 0, 0, 0};
  if (rope) {
    float x[4][8];
    const int pos[4] = {8 * r, 32 + 8 * r, 64 + 8 * r, 96 + 8 * r};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) widen16<GQA_BF16>(qf[kk], x[kk]);
    rope_chunks(a, rp, pos, x, a.q_gain);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = hw + c < G ? u32x4{pack_bf16x2(x[kk][0], x[kk][1]), pack_bf16x2(x[kk][2], x[kk][3]),
                                  pack_bf16x2(x[kk][4], x[kk][5]), pack_bf16x2(x[kk][6], x[kk][7])}
                          : u32x4{0, 0, 0, 0};
  }
}

// The new key and value of kv-head row nrow (element offset), 16-byte piece
// `piece` (elements 8 piece .. 8 piece + 7); with `rope` the key is rotated
// (and normalized) at rotary row rp.  Each 16-lane group holds the whole key:
// the half pairing's partner piece is loaded as well, and the norm reduces
// over the group.
__device__ __forceinline__ void load_new_kv(const AttnArgs& a, int64_t nrow, int piece, bool rope, int rp, u32x4& kn,
                                            u32x4& vn) {
  kn = load16(reinterpret_cast<const uint16_t*>(a.k_new) + nrow + 8 * piece);
  vn = load16(reinterpret_cast<const uint16_t*>(a.v_new) + nrow + 8 * piece);
  if (!rope) return;
  const u32x4 kp = load16(reinterpret_cast<const uint16_t*>(a.k_new) + nrow + 8 * (piece ^ 8));
  float x[8], xp[8], y[8];
  widen16<GQA_BF16>(kn, x);
  widen16<GQA_BF16>(kp, xp);
  const float* cs = a.rope_cos + (int64_t)rp * 64;
  const float* sn = a.rope_sin + (int64_t)rp * 64;
  const bool half = a.rope_mode == GQA_ROPE_HALF;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * piece + e;
    const bool first = half ? d < 64 : (e & 1) == 0;
    const int j = half ? (d & 63) : (d >> 1);
    y[e] = rope_rot(first, x[e], half ? xp[e] : x[e ^ 1], cs[j], sn[j]);
  }
  if (a.k_gain != nullptr) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off);
    const float rn = 1.0f / sqrtf(ss / 128.f + a.norm_eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (y[e] * rn) * a.k_gain[8 * piece + e];
  }
  kn = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}

// The end of a piece for the wave's 16 heads hw .. hw + 15 of item (b, h):
// lane (r, c) holds m and l of head c and the sums of heads 4r .. 4r + 3
// (O[nb][i] at column 16 nb + c).  A whole piece writes the output rows; a
// cut one the partial rows pbase + g * pstride of its heads g (m, l, o).
// `scaled`: the softmax has a sink or the smooth variant, or the window may
// leave a head with no attended slot (finish_scale covers each).
__device__ __forceinline__ void all_finish(const AttnArgs& a, int b, int h, int hw, bool whole, int64_t pbase,
                                           int64_t pstride, float m, float l, const f32x4 (&O)[8], bool scaled) {
  const int lane = threadIdx.x & 63;
  const int r = lane >> 4;
  const int c = lane & 15;
  const int G = a.G;
  l = rows_sum(l);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * r + i;  // head within the wave
    const float li = __shfl(l, hl);
    const float mi = __shfl(m, hl);
    if (hw + hl >= G) continue;
    const int hq = h * G + hw + hl;
    if (whole) {
      const float inv = scaled ? finish_scale(a, hq, mi, li) : (li > 0.f ? 1.f / li : 0.f);
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + hq) * kD;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) o[16 * nb + c] = f32_to_bf16_rne(O[nb][i] * inv);
    } else {
      const int64_t pi = pbase + (int64_t)(hw + hl) * pstride;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) a.part_o[pi * kD + 16 * nb + c] = O[nb][i];
      if (c == 0) {
        a.part_m[pi] = mi;
        a.part_l[pi] = li;
      }
    }
  }
}


template <bool PAGED, bool VAR, bool BUF>
__global__ __launch_bounds__(256) void attend_mfma_all_kernel(AttnArgs a) {
  static_assert(!BUF || (!PAGED && !VAR), "buffer loads serve dense rows without a window");
  __shared__ __attribute__((aligned(16))) uint16_t sk[3][kTileT * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t sv[3][kTileT * kPitch];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;

  int x = blockIdx.x;
  const int split = x % a.nsplit;
  x /= a.nsplit;
  const int h = x % a.Hkv;
  const int b = x / a.Hkv;
  const int G = a.G;

  const int L0 = a.lengths[b];
  int n = L0 + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  // Slots are walked in the sliding window's virtual order (the identity
  // without a window); the new token is the last virtual slot, L.
  SeqView view{n, n, 0, 0, 0};
  if constexpr (VAR) view = seq_view(a, b, n);
  auto phys = [&](int t) { return VAR ? phys_slot(view, t) : t; };
  const int nv = view.nv;
  const int L = L0 - view.gap;
  const int t_begin = split * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, nv);
  const int nact = nv == 0 ? 0 : min(a.nsplit, (nv + a.split_tokens - 1) / a.split_tokens);
  if (split >= max(nact, 1)) return;
  const bool own_new = a.k_new != nullptr && L >= t_begin && L < t_end;

  const int hw = wave * 16;  // first head of this wave
  // Rotary step: q and the new key are rotated (and normalized) here, at the
  // new token's position.
  const bool rope = a.rope_cos != nullptr;
  const int rp = rope ? rope_row(a, b, L0) : 0;
  u32x4 qf[4];
  load_q_frags(a, b, h, hw, rope, rp, qf);

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
  u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};  // the new key / value, piece `piece`
  if (own_new) load_new_kv(a, nrow, piece, rope, rp, kn, vn);
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
        en.e[q2] = a.map[(int64_t)b * a.max_blocks + phys(hc) / a.bs];
      }
    }
    return en;
  };
  // Buffer-load path (dense or slot-indexed rows, no window): a tile's
  // resource starts at its first row and holds its rows up to the split's
  // end, so a lane's byte offset is the same for every tile and rows past the
  // end read as zeros without being loaded (their scores are masked).  The
  // launcher takes this path only when a kv-head's capacity fits the
  // resource's 31-bit byte count.
  const uint32_t rsb = (uint32_t)rs * 2u;  // bytes between consecutive slots
  const uint32_t lane_off0 = (uint32_t)prow * rsb + 16u * (uint32_t)piece;
  const uint32_t lane_off1 = lane_off0 + 16u * rsb;
  auto tile_rsrc = [&](const uint16_t* base, int t0) {
    const int rows = max(0, t_end - t0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + (int64_t)t0 * rs), (short)0,
                                             (int)((uint32_t)rows * rsb), 0x00020000);
  };
  auto gload = [&](int t0, Regs& R, const Ent& en) {
    if constexpr (BUF) {
      const auto rk = tile_rsrc(kb, t0), rv = tile_rsrc(vb, t0);
      const u32x4 k0 = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)lane_off0, 0, 2);  // 2: non-temporal
      const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lane_off0, 0, 2);
      const u32x4 k1 = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)lane_off1, 0, 2);
      const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lane_off1, 0, 2);
      R.k[0] = k0;
      R.v[0] = v0;
      R.k[1] = k1;
      R.v[1] = v1;
      return;
    }
    if constexpr (!PAGED) {
      // Dense or slot-indexed rows (tiles start at t_begin, so only the end
      // clamps): one 32x32->64-bit multiply-add per row address (slot strides
      // fit 32 bits: the descriptor check refuses larger ones).
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int rc = min(t0 + prow + 16 * q2, t_end - 1);
        const uint64_t off = (uint64_t)(uint32_t)phys(rc) * (uint32_t)rs + (uint32_t)(8 * piece);
        R.k[q2] = load_nt16(kb + off);
        R.v[q2] = load_nt16(vb + off);
      }
      return;
    }
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int rc = max(min(t0 + prow + 16 * q2, t_end - 1), t_begin);
      int64_t off;
      if (PAGED) {  // a 16-row half lies in one block and moves with its (16-aligned) origin
        const int hc = max(min(t0 + 16 * q2, last16), tv);
        off = block_head_offset(a, en.e[q2], h) + (int64_t)(phys(hc) % a.bs + (rc - hc)) * rs + 8 * piece;
      } else {
        off = (int64_t)phys(rc) * rs + 8 * piece;
      }
      R.k[q2] = load_nt16(kb + off);
      R.v[q2] = load_nt16(vb + off);
    }
  };
  auto swrite = [&](int t0, int buf, const Regs& R) {
#pragma unroll
    for (int q2 = 0; q2 < 2; ++q2) {
      const int row = prow + 16 * q2;
      *reinterpret_cast<u32x4*>(&sk[buf][row * kPitch + 8 * piece]) = R.k[q2];
      *reinterpret_cast<u32x4*>(&sv[buf][row * kPitch + 8 * piece]) = R.v[q2];
    }
    if (own_new && t0 + kTileT > L) {  // uniform: the tile holding the new token; rows >= L take it
#pragma unroll
      for (int q2 = 0; q2 < 2; ++q2) {
        const int row = prow + 16 * q2;
        if (t0 + row >= L) {
          *reinterpret_cast<u32x4*>(&sk[buf][row * kPitch + 8 * piece]) = kn;
          *reinterpret_cast<u32x4*>(&sv[buf][row * kPitch + 8 * piece]) = vn;
        }
      }
    }
  };

  // The loop runs one tile behind on the V sum: iteration t issues the V sum
  // of the walk's tile t (LDS buffer t mod 3) with the scores and weights of
  // its tile t + 1 (buffer t + 1 mod 3), writes tile t + 2 to buffer t + 2
  // mod 3 and starts the loads of tile t + 3.  Two register sets keep two
  // tiles in flight (tile k in set k mod 2).  Loads of tiles past the end clamp to the last
  // valid row (cache hits, never used), so every path issues the same loads,
  // the loop has one exit, and each LDS write waits only for its own tile's
  // loads.
  u32x4 pa = {0u, 0u, 0u, 0u}, pl = {0u, 0u, 0u, 0u};  // the weights of the tile whose V sum is next
  if (t_begin < t_end) {
    const int ntile = (t_end - tv + kTileT - 1) / kTileT;
    // The split's tiles are walked from a start tile that moves with the item
    // (tile k of the walk is tile (k + rot) mod ntile), so the workgroups of
    // one XCD, which hold consecutive items whose regions are equally aligned,
    // do not all read the same offset of their regions at the same time
    // (measured on MI355X: 2-3 % on the large-group shapes).  Positions past
    // the last tile are the clamped prefetches of the loop's end.
    const int rot = __builtin_amdgcn_readfirstlane(((b * a.Hkv + h) >> 1) % ntile);
    auto tp = [&](int k) {
      if (k >= ntile) return tv + k * kTileT;
      int x = k + rot;
      x -= x >= ntile ? ntile : 0;
      return tv + x * kTileT;
    };
    auto next3 = [](int x) { return x == 2 ? 0 : x + 1; };
    Regs R0, R1;
    gload(tp(0), R0, entries(tp(0)));
    gload(tp(1), R1, entries(tp(1)));
    const Ent e2 = entries(tp(2));
    Ent e3 = entries(tp(3));
    swrite(tp(0), 0, R0);
    __syncthreads();
    gload(tp(2), R0, e2);
    all_step<VAR, true, false>(a, sk[0], sv[0], qf, tp(0), t_begin, t_end, view, m, l, O, pa, pl);
    swrite(tp(1), 1, R1);
    __syncthreads();
    int k = 0;   // the walk position of the tile whose V sum runs next
    int bt = 0;  // its buffer
    const int nit = ntile - 1;
    for (int it = 0; it < nit / 2; ++it) {
      {
        const Ent en = entries(tp(k + 4));
        gload(tp(k + 3), R1, e3);
        e3 = en;
        const int b1 = next3(bt), b2 = next3(b1);
        all_step<VAR, true, true>(a, sk[b1], sv[bt], qf, tp(k + 1), t_begin, t_end, view, m, l, O, pa, pl);
        swrite(tp(k + 2), b2, R0);
        __syncthreads();
        bt = b1;
        ++k;
      }
      {
        const Ent en = entries(tp(k + 4));
        gload(tp(k + 3), R0, e3);
        e3 = en;
        const int b1 = next3(bt), b2 = next3(b1);
        all_step<VAR, true, true>(a, sk[b1], sv[bt], qf, tp(k + 1), t_begin, t_end, view, m, l, O, pa, pl);
        swrite(tp(k + 2), b2, R1);
        __syncthreads();
        bt = b1;
        ++k;
      }
    }
    if (nit & 1) {  // the last tile's scores (it is in LDS already)
      const int b1 = next3(bt);
      all_step<VAR, true, true>(a, sk[b1], sv[bt], qf, tp(k + 1), t_begin, t_end, view, m, l, O, pa, pl);
      bt = b1;
      ++k;
    }
    all_step<VAR, false, true>(a, sk[bt], sv[bt], qf, tp(k), t_begin, t_end, view, m, l, O, pa, pl);
  }

  if (own_new && prow == 0) {  // the appended slot (skipped if the map names no valid row/block)
    const int64_t off = slot_offset_checked(a, b, h, L0);
    if (off >= 0) {
      store16(reinterpret_cast<uint16_t*>(a.k_cache_w) + off + 8 * piece, kn);
      store16(reinterpret_cast<uint16_t*>(a.v_cache_w) + off + 8 * piece, vn);
    }
  }

  all_finish(a, b, h, hw, nact <= 1, ((int64_t)b * a.Hq + (int64_t)h * G) * a.nsplit + split, a.nsplit, m, l, O,
             VAR || a.sink != nullptr || a.smooth);
}

// ---------------------------------------------------------------------------
// Kernel MFMA_ALL, whole-item form: no split of the token axis, so no partials
// and no combine pass; for batches whose (sequence, kv-head) items fill the
// device, or when one split is asked for.
//
// One workgroup = 8 waves = one item and its G query heads in HB 16-head
// blocks (HB = 2 for G <= 32, 4 above).  Wave w owns head block w mod HB and
// sub-tile w / HB of each step: a step stages 8 / HB 32-slot sub-tiles of K
// and V in LDS (two buffers, loaded by all 512 threads) and each wave runs the
// tile math above on its sub-tile for its 16 heads (scores, weights as bf16
// hi / lo pairs, V sum, online softmax with lazy rescale).  The sub-tile waves
// of a head block end with one (m, l, o) each for their heads, merged through
// LDS to the block's common maximum before the output rows are written.
// ---------------------------------------------------------------------------
constexpr int kMergePitch = 132;  // floats per merge row (16-byte aligned rows, spread over the banks)

template <int HB, bool VAR, bool BUF>
__global__ __launch_bounds__(512) void attend_mfma_all8_kernel(AttnArgs a) {
  static_assert(HB == 2 || HB == 4, "two or four 16-head blocks per workgroup");
  static_assert(!BUF || !VAR, "buffer loads serve dense rows without a window");
  constexpr int SUB = 8 / HB;            // sub-tiles per step
  constexpr int STEP = SUB * kTileT;     // slots per step
  constexpr int HALF = STEP * kPitch;    // bf16 elements of one K (or V) buffer
  // LDS: K buffers 0, 1 then V buffers 0, 1; after the loop the merge rows.
  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * HALF];
  static_assert(HB * SUB * 16 * kMergePitch * 4 + HB * SUB * 32 * 4 <= 4 * HALF * 2, "merge rows fit the tiles");
  auto skb = [&](int buf) { return lds + buf * HALF; };
  auto svb = [&](int buf) { return lds + (2 + buf) * HALF; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane >> 4;
  const int c = lane & 15;
  const int hb = wave % HB;   // head block within the workgroup
  const int sub = wave / HB;  // sub-tile of each step
  const int G = a.G;

  const int h = blockIdx.x % a.Hkv;
  const int b = blockIdx.x / a.Hkv;

  const int L0 = a.lengths[b];
  int n = L0 + a.len_offset;
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  SeqView view{n, n, 0, 0, 0};
  if constexpr (VAR) view = seq_view(a, b, n);
  auto phys = [&](int t) { return VAR ? phys_slot(view, t) : t; };
  const int nv = view.nv;
  const int L = L0 - view.gap;
  const int t_begin = 0, t_end = nv;  // the whole sequence
  const bool own_new = a.k_new != nullptr && L >= 0 && L < nv;

  const int hw = hb * 16;     // first head of this wave
  const bool active = hw < G;  // (a head block past G holds no head)
  const bool rope = a.rope_cos != nullptr;
  const int rp = rope ? rope_row(a, b, L0) : 0;
  u32x4 qf[4];
  load_q_frags(a, b, h, hw, rope, rp, qf);

  float m = kNegInfM, l = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) O[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t base = row_head_offset(a, b, h);  // dense or slot-indexed row
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k_cache) + base;
  const uint16_t* vb = reinterpret_cast<const uint16_t*>(a.v_cache) + base;
  const int64_t rs = a.st;
  const int64_t nrow = ((int64_t)b * a.Hkv + h) * kD;

  // Cooperative step load: thread t moves 16 bytes (piece t & 15) of row
  // t >> 4 of each sub-tile.  Rows past the last valid slot are clamped to it
  // (buffer loads: read as zeros), so every load is unconditional.  The step
  // holding the new token L takes it for its rows >= L when written to LDS
  // (rows past L are masked and only need finite values); the new bits go to
  // the cache slot after the loop.
  const int prow = tid >> 4;
  const int piece = tid & 15;
  struct Regs {
    u32x4 k[SUB], v[SUB];
  };
  u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
  if (own_new) load_new_kv(a, nrow, piece, rope, rp, kn, vn);
  const uint32_t rsb = (uint32_t)rs * 2u;  // bytes between consecutive slots
  const uint32_t lane_off = (uint32_t)prow * rsb + 16u * (uint32_t)piece;
  auto step_rsrc = [&](const uint16_t* p, int t0) {
    // (readfirstlane: a resource the compiler cannot prove uniform turns each
    // load into a loop over the lanes' resources)
    const int rows = __builtin_amdgcn_readfirstlane(max(0, t_end - t0));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p + (int64_t)t0 * rs), (short)0,
                                             (int)((uint32_t)rows * rsb), 0x00020000);
  };
  auto gload = [&](int t0, Regs& R) {
    if constexpr (BUF) {
      const auto rk = step_rsrc(kb, t0), rv = step_rsrc(vb, t0);
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
        const int so = (int)((uint32_t)(q * kTileT) * rsb);
        R.k[q] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)lane_off, so, 2);  // 2: non-temporal
        R.v[q] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lane_off, so, 2);
      }
    } else {
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
        const int rc = min(t0 + prow + q * kTileT, t_end - 1);
        const uint64_t off = (uint64_t)(uint32_t)phys(rc) * (uint32_t)rs + (uint32_t)(8 * piece);
        R.k[q] = load_nt16(kb + off);
        R.v[q] = load_nt16(vb + off);
      }
    }
  };
  auto swrite = [&](int t0, int buf, const Regs& R) {
#pragma unroll
    for (int q = 0; q < SUB; ++q) {
      const int row = prow + q * kTileT;
      *reinterpret_cast<u32x4*>(skb(buf) + row * kPitch + 8 * piece) = R.k[q];
      *reinterpret_cast<u32x4*>(svb(buf) + row * kPitch + 8 * piece) = R.v[q];
    }
    if (own_new && t0 + STEP > L) {  // uniform: the step holding the new token
#pragma unroll
      for (int q = 0; q < SUB; ++q) {
        const int row = prow + q * kTileT;
        if (t0 + row >= L) {
          *reinterpret_cast<u32x4*>(skb(buf) + row * kPitch + 8 * piece) = kn;
          *reinterpret_cast<u32x4*>(svb(buf) + row * kPitch + 8 * piece) = vn;
        }
      }
    }
  };
  // The wave's sub-tile of the step in buffer `buf`: scores and weights, then
  // the V sum with those weights (a sub-tile past the end is skipped).
  u32x4 pa = {0u, 0u, 0u, 0u}, pl = {0u, 0u, 0u, 0u};
  auto tile = [&](int buf, int t0) {
    const int ts = t0 + sub * kTileT;
    if (active && ts < t_end) {
      const uint16_t* K = skb(buf) + sub * kTileT * kPitch;
      const uint16_t* V = svb(buf) + sub * kTileT * kPitch;
      all_step<VAR, true, false>(a, K, V, qf, ts, t_begin, t_end, view, m, l, O, pa, pl);
      all_step<VAR, false, true>(a, K, V, qf, ts, t_begin, t_end, view, m, l, O, pa, pl);
    }
  };

  // Two register sets keep two steps in flight (step k in set k mod 2); steps
  // run in pairs with one exit, so each LDS write waits only for its own loads.
  if (t_begin < t_end) {
    const int nstep = (t_end - t_begin + STEP - 1) / STEP;
    Regs R0, R1;
    gload(t_begin, R0);
    gload(t_begin + STEP, R1);
    swrite(t_begin, 0, R0);
    __syncthreads();
    gload(t_begin + 2 * STEP, R0);
    int t0 = t_begin;
    for (int it = 0; it < nstep / 2; ++it) {
      tile(0, t0);
      swrite(t0 + STEP, 1, R1);
      __syncthreads();
      gload(t0 + 3 * STEP, R1);
      tile(1, t0 + STEP);
      swrite(t0 + 2 * STEP, 0, R0);
      __syncthreads();
      gload(t0 + 4 * STEP, R0);
      t0 += 2 * STEP;
    }
    if (nstep & 1) tile(0, t0);
  }

  if (own_new && prow == 0) {  // the appended slot (skipped if the map names no valid row)
    const int64_t off = slot_offset_checked(a, b, h, L0);
    if (off >= 0) {
      store16(reinterpret_cast<uint16_t*>(a.k_cache_w) + off + 8 * piece, kn);
      store16(reinterpret_cast<uint16_t*>(a.v_cache_w) + off + 8 * piece, vn);
    }
  }

  // Merge of the SUB sub-tile waves of each head block.  Lane (r, c) holds m
  // of head c, a part of its l, and the sums of heads 4r .. 4r + 3 (O[nb][i]
  // at column 16 nb + c).  Each wave stores (m, l) of its heads, then its sums
  // scaled to the block's common maximum; wave (hb, sub) then adds the SUB
  // waves' sums for its share of the columns and writes those outputs.
  __syncthreads();  // every wave is done with the tile buffers
  float* mo = reinterpret_cast<float*>(lds);                          // [hb][sub][16 heads][kMergePitch]
  float* ml = mo + HB * SUB * 16 * kMergePitch;                       // [hb][sub][m, l][16 heads]
  auto mrow = [&](int s2, int what) { return ml + ((hb * SUB + s2) * 2 + what) * 16; };
  const float lw = rows_sum(l);
  if (r == 0) {
    mrow(sub, 0)[c] = m;
    mrow(sub, 1)[c] = lw;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * r + i;
    float M = kNegInfM;
#pragma unroll
    for (int s2 = 0; s2 < SUB; ++s2) M = fmaxf(M, mrow(s2, 0)[hl]);
    const float alpha = M == kNegInfM ? 0.f : fast_exp2(mrow(sub, 0)[hl] - M);
    float* row = mo + ((hb * SUB + sub) * 16 + hl) * kMergePitch;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) row[16 * nb + c] = O[nb][i] * alpha;
  }
  __syncthreads();
  {
    constexpr int CW = 128 / SUB;  // columns per wave
    constexpr int CL = CW / 4;     // columns per lane (8 or 16)
    const int hl = lane >> 2;
    const int col = CW * sub + CL * (lane & 3);
    float M = kNegInfM;
#pragma unroll
    for (int s2 = 0; s2 < SUB; ++s2) M = fmaxf(M, mrow(s2, 0)[hl]);
    float lsum = 0.f;
    float acc[CL];
#pragma unroll
    for (int e = 0; e < CL; ++e) acc[e] = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < SUB; ++s2) {
      lsum += (M == kNegInfM ? 0.f : fast_exp2(mrow(s2, 0)[hl] - M)) * mrow(s2, 1)[hl];
      const float* row = mo + ((hb * SUB + s2) * 16 + hl) * kMergePitch + col;
#pragma unroll
      for (int e4 = 0; e4 < CL; e4 += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(row + e4);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e4 + e] += x[e];
      }
    }
    if (hw + hl < G) {
      const int hq = h * G + hw + hl;
      const bool scaled = VAR || a.sink != nullptr || a.smooth;
      const float inv = scaled ? finish_scale(a, hq, M, lsum) : (lsum > 0.f ? 1.f / lsum : 0.f);
      uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.Hq + hq) * kD + col;
#pragma unroll
      for (int e8 = 0; e8 < CL; e8 += 8)
        store16(o + e8, u32x4{pack_bf16x2(acc[e8] * inv, acc[e8 + 1] * inv),
                              pack_bf16x2(acc[e8 + 2] * inv, acc[e8 + 3] * inv),
                              pack_bf16x2(acc[e8 + 4] * inv, acc[e8 + 5] * inv),
                              pack_bf16x2(acc[e8 + 6] * inv, acc[e8 + 7] * inv)});
    }
  }
}

hipError_t launch_attend_mfma_all(const AttnArgs& a, const Plan& p, hipStream_t s) {
  if (a.D != kD || a.G > 64) return hipErrorInvalidValue;
  AttnArgs arg = a;
  void* params[] = {&arg};
  const bool var = a.window > 0 || a.cap_T > 0.f;  // in-loop variants (the sink is applied at the end)
  const bool paged = a.map_kind == GQA_MAP_PAGED;
  if (a.kv_dtype != GQA_BF16 || a.qo_dtype != GQA_BF16) return hipErrorInvalidValue;
  // Buffer loads need every byte offset of a kv-head's rows in 31 bits.
  const bool buf = !paged && !var && (int64_t)a.S * a.st * 2 <= INT32_MAX;
  if (p.all8) {
    if (paged || p.all8 != (a.G > 32 ? 4 : 2) || p.nsplit != 1 || (int64_t)p.grid != (int64_t)a.B * a.Hkv)
      return hipErrorInvalidValue;
    // Buffer loads: every byte offset of a step's rows, up to two steps past
    // the capacity, in 31 bits.
    const bool wbuf = !var && (int64_t)(a.S + 256) * a.st * 2 <= INT32_MAX;
    const void* wf;
    if (p.all8 == 4)
      wf = var ? reinterpret_cast<const void*>(&attend_mfma_all8_kernel<4, true, false>)
           : wbuf ? reinterpret_cast<const void*>(&attend_mfma_all8_kernel<4, false, true>)
                  : reinterpret_cast<const void*>(&attend_mfma_all8_kernel<4, false, false>);
    else
      wf = var ? reinterpret_cast<const void*>(&attend_mfma_all8_kernel<2, true, false>)
           : wbuf ? reinterpret_cast<const void*>(&attend_mfma_all8_kernel<2, false, true>)
                  : reinterpret_cast<const void*>(&attend_mfma_all8_kernel<2, false, false>);
    return hipLaunchKernel(wf, dim3(p.grid), dim3(512), params, 0, s);
  }
  const void* fn = paged ? (var ? reinterpret_cast<const void*>(&attend_mfma_all_kernel<true, true, false>)
                                : reinterpret_cast<const void*>(&attend_mfma_all_kernel<true, false, false>))
                   : var ? reinterpret_cast<const void*>(&attend_mfma_all_kernel<false, true, false>)
                   : buf ? reinterpret_cast<const void*>(&attend_mfma_all_kernel<false, false, true>)
                         : reinterpret_cast<const void*>(&attend_mfma_all_kernel<false, false, false>);
  return hipLaunchKernel(fn, dim3(p.grid), dim3(256), params, 0, s);
}

}  // namespace gqa

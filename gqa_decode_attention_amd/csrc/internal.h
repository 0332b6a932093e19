// Host-side interface between the C ABI (gqa_decode.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gqa_decode.h"

namespace gqa {

// Everything a kernel needs, resolved on the host from the descriptor.
struct AttnArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* k_cache_w;       // fused step: cache written with the new K/V (else null)
  void* v_cache_w;
  const void* k_new;     // fused step: new K/V (else null)
  const void* v_new;
  const int32_t* lengths;
  void* out;
  float* part_o;         // split partials: [B][Hq][nsplit][D] unnormalised sums
  float* part_m;         // [B][Hq][nsplit] running max (log2 units)
  float* part_l;         // [B][Hq][nsplit] softmax denominators
                         // (balanced mode: rows [grid][2][G] instead of [B][Hq][nsplit])
  int32_t B, Hq, Hkv, D, S, G;
  int64_t sb, sh, st;    // cache element strides of cache row, kv-head, slot (paged: within a block)
  // Cache map (mapped entry points): map_kind 0 = dense (row b), GQA_MAP_SLOTS
  // (row map[b]), GQA_MAP_PAGED (slot t in block map[b * max_blocks + t / bs]).
  const int32_t* map;
  int32_t map_kind, map_rows, bs, max_blocks;
  int64_t sblk;          // paged: elements between pool blocks
  // Int8 caches: float32 row scales, indexed by a row's element offset / D
  // (read by attention; the quantizing append writes the appended rows).
  const float* k_scale;
  const float* v_scale;
  float* k_scale_w;
  float* v_scale_w;
  // Rotary encoding (the rope append kernel): float32 (max_pos, D/2) tables,
  // the new token's position per sequence (null: lengths[b]), optional norm
  // gains, and the rotated q it writes (qo_dtype, (B, Hq, D)).
  const float* rope_cos;
  const float* rope_sin;
  const int32_t* rope_pos;
  const float* q_gain;
  const float* k_gain;
  void* q_rot;
  int32_t rope_max_pos, rope_mode;
  float norm_eps;
  // Softmax variants (attention passes and the combine): per-query-head sink
  // logits (natural units) or smooth softmax (a zero logit), softcap as
  // T = cap * sqrt(D) on raw scores (0: none), sliding window (0: none) with a
  // kept prefix (one value, or one per sequence when prefix_seq is set).
  const float* sink;
  int32_t smooth;
  float cap_T, cap_invT;
  int32_t window, prefix;
  const int32_t* prefix_seq;
  // Balanced mode (MFMA_QK): tile offsets of the sequences (B + 1 entries,
  // written by the attention pass for the combine pass), or null in split mode.
  int32_t* bal_pre;
  int32_t bal_units;     // balanced mode: workgroups of the attention pass
  int32_t bal_cost;      // balanced mode: units charged per item besides its tiles
  int32_t hp;            // MFMA_QK: kv-heads per work item (4: head-parallel waves, BSHD caches; else 1)
  int32_t nsplit, split_tokens;
  int32_t head_chunks;   // generic kernel: query-head chunks per kv-head
  int32_t len_offset;    // slots attended = lengths[b] + len_offset (1 for a step, 0 for attend)
  int32_t kv_dtype, qo_dtype;
  float scale_log2;      // log2(e) / sqrt(D)
};

struct Plan {
  int32_t kernel;
  int32_t nsplit;
  int32_t split_tokens;
  int32_t head_chunks;   // generic kernel: query-head chunks per kv-head
  int32_t grid;
  int32_t block;
  int32_t combine;
  size_t workspace_bytes;
  size_t off_m, off_l;   // byte offsets of part_m / part_l inside the workspace
  int32_t balanced;      // 1: equal unit ranges per workgroup (see AttnArgs::bal_pre)
  int32_t bal_cost;      // balanced mode: units charged per item besides its tiles
  int32_t hp;            // MFMA_QK: kv-heads per work item (see AttnArgs::hp)
  size_t off_pre;        // byte offset of the tile offsets inside the workspace
  int32_t all8;          // MFMA_ALL whole-item form (8-wave workgroups, no split): 16-head blocks
                         // per workgroup (2 or 4); 0 = the split form
};

// Which matrix-core kernels this build provides (the planner falls back to the
// generic kernel for the others).
extern const bool kHaveMfmaQk;
extern const bool kHaveMfmaAll;
extern const bool kHaveMfmaQkI8;  // int8 caches on the G <= 16 matrix-core kernel

constexpr int kDefaultCUs = 256;      // MI355X: 8 XCDs x 32 CUs (the plan's CU count when no device is visible)
constexpr int kMaxSplits = 64;        // one lane per split in the combine pass
constexpr int kGenericHeadChunk = 8;  // query heads per workgroup in the generic kernel
constexpr int kMaxBalancedBatch = 4096;  // most sequences in the balanced mode (16 per thread of its scan)
// Balanced mode: tiles charged per item besides its own (bf16 / int8 caches;
// contiguous or strided slots of a kv-head), from sweeps on ragged batches.
// Strided (BSHD) items are four kv-heads whose tiles carry four times the
// bytes of a one-head tile, so the same fixed cost is fewer of their tiles.
constexpr int kBalancedCostBf16 = 12;
constexpr int kBalancedCostI8 = 28;
constexpr int kBalancedCostBf16Strided = 0;
constexpr int kBalancedCostI8Strided = 5;

// Launchers (return hipSuccess or the launch error).
hipError_t launch_append(const AttnArgs& a, void* k_cache, void* v_cache, hipStream_t s);
// Rotary append: rotates (and normalizes) the new key, writes it and the value
// at slot lengths[b] (int8 caches: quantized), and, when a.q_rot is set, the
// rotated (and normalized) q into a.q_rot.
hipError_t launch_rope_append(const AttnArgs& a, void* k_cache, void* v_cache, hipStream_t s);
// Quantizing append into int8 caches (new K/V in a.qo_dtype).
hipError_t launch_append_q8(const AttnArgs& a, void* k_cache, void* v_cache, hipStream_t s);
hipError_t launch_attend_generic(const AttnArgs& a, const Plan& p, int vec_path, hipStream_t s);
hipError_t launch_attend_small(const AttnArgs& a, const Plan& p, hipStream_t s);
hipError_t launch_attend_mfma_qk(const AttnArgs& a, const Plan& p, hipStream_t s);
hipError_t launch_attend_mfma_all(const AttnArgs& a, const Plan& p, hipStream_t s);
hipError_t launch_combine(const AttnArgs& a, const Plan& p, hipStream_t s);
// Count lengths[b] outside [lo, hi] (synchronous; *bad receives the count).
hipError_t run_check_lengths(const int32_t* lengths, int32_t B, int32_t lo, int32_t hi, hipStream_t s,
                             int32_t* bad);

}  // namespace gqa

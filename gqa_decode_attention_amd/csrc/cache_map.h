// Device-side addressing of the caches: dense (row b), slot-indexed (row
// map[b]) or paged (slot t of batch row b in block map[b * max_blocks + t / bs]),
// CLIKA runtime "groupQueryAttention" API page, slot_ids and block-table notes.
// Entries the host validated are in range; a device table that differs from
// the validated host copy is clamped for reads (never out of bounds) and makes
// appends skip their write.
#pragma once

#include "internal.h"

namespace gqa {

// Element offset of cache row (b's row) and kv-head h: dense and slots.
__device__ __forceinline__ int64_t row_head_offset(const AttnArgs& a, int b, int h) {
  int row = b;
  if (a.map_kind == GQA_MAP_SLOTS) {
    row = a.map[b];
    row = row < 0 ? 0 : (row >= a.map_rows ? a.map_rows - 1 : row);
  }
  return (int64_t)row * a.sb + (int64_t)h * a.sh;
}

// Paged: element offset of block `blk`, kv-head h, in-block slot 0 (an entry
// outside [0, map_rows) reads block 0).
__device__ __forceinline__ int64_t block_head_offset(const AttnArgs& a, int32_t blk, int h) {
  blk = (blk < 0 || blk >= a.map_rows) ? 0 : blk;
  return (int64_t)blk * a.sblk + (int64_t)h * a.sh;
}

// Element offset of slot t of (b, h) for any map kind (per-row lookup).
__device__ __forceinline__ int64_t slot_offset(const AttnArgs& a, int b, int h, int t) {
  if (a.map_kind != GQA_MAP_PAGED) return row_head_offset(a, b, h) + (int64_t)t * a.st;
  const int32_t blk = a.map[(int64_t)b * a.max_blocks + t / a.bs];
  return block_head_offset(a, blk, h) + (int64_t)(t % a.bs) * a.st;
}

// As slot_offset, but -1 when the table names no valid block (append skips).
__device__ __forceinline__ int64_t slot_offset_checked(const AttnArgs& a, int b, int h, int t) {
  if (a.map_kind == GQA_MAP_SLOTS) {
    const int row = a.map[b];
    if (row < 0 || row >= a.map_rows) return -1;
    return (int64_t)row * a.sb + (int64_t)h * a.sh + (int64_t)t * a.st;
  }
  if (a.map_kind == GQA_MAP_PAGED) {
    const int32_t blk = a.map[(int64_t)b * a.max_blocks + t / a.bs];
    if (blk < 0 || blk >= a.map_rows) return -1;
    return (int64_t)blk * a.sblk + (int64_t)h * a.sh + (int64_t)(t % a.bs) * a.st;
  }
  return (int64_t)b * a.sb + (int64_t)h * a.sh + (int64_t)t * a.st;
}

}  // namespace gqa

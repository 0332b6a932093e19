// C ABI of the GQA decode step: argument validation, planning and launch.
//
// Every condition the host can check is checked before the first HIP call,
// so an error return means nothing was enqueued (CLIKA groupQueryAttention
// page: every argument is checked before any data is read, and a malformed
// one is refused with INVALID_ARGUMENT; CANN aclnnMlaPrologV3WeightNz page: the first phase
// verifies parameters and reports the workspace size).  The plan -- kernel,
// split of the token axis, grid, workspace -- is a pure function of the
// descriptor: `lengths` stays on the device and is never read here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <vector>

#include "gqa_decode.h"
#include "internal.h"

using namespace gqa;

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(int32_t dt) { return dt == GQA_F32 ? 4 : dt == GQA_BF16 ? 2 : 1; }

// Checked product of non-negative factors; false on overflow past 2^62.
bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > ((int64_t)1 << 62) / a) return false;
  *r = a * b;
  return true;
}

gqa_status_t check_desc(const gqa_decode_desc_t* d) {
  if (d == nullptr) return GQA_ERR_INVALID_ARGUMENT;
  if (d->batch < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 || d->capacity < 1)
    return GQA_ERR_INVALID_ARGUMENT;
  if (d->num_q_heads % d->num_kv_heads != 0) return GQA_ERR_INVALID_ARGUMENT;
  if (d->layout != GQA_LAYOUT_BHSD && d->layout != GQA_LAYOUT_BSHD) return GQA_ERR_INVALID_ARGUMENT;
  if ((d->kv_dtype != GQA_F32 && d->kv_dtype != GQA_BF16 && d->kv_dtype != GQA_I8 && d->kv_dtype != GQA_FP8) ||
      (d->qo_dtype != GQA_F32 && d->qo_dtype != GQA_BF16))
    return GQA_ERR_INVALID_ARGUMENT;
  if (d->num_splits < 0) return GQA_ERR_INVALID_ARGUMENT;
  if (d->head_dim > 256) return GQA_ERR_UNSUPPORTED;
  // Sizes must be addressable with 64-bit element offsets and the grids with 32-bit counts.
  int64_t t;
  if (!mul_ok(d->batch, d->num_kv_heads, &t) || !mul_ok(t, d->capacity, &t) || !mul_ok(t, d->head_dim, &t) ||
      !mul_ok(t, 4, &t))
    return GQA_ERR_UNSUPPORTED;
  if (!mul_ok(d->batch, d->num_q_heads, &t) || t > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  // The byte stride between consecutive slots must fit 32 bits.
  if (!mul_ok(d->num_kv_heads, d->head_dim, &t) || t * 4 > (int64_t)UINT32_MAX) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Caches of one-byte codes with per-row float32 scales.
bool quantized(int32_t dt) { return dt == GQA_I8 || dt == GQA_FP8; }

bool is_matrix_core(int32_t kernel) { return kernel == GQA_KERNEL_MFMA_QK || kernel == GQA_KERNEL_MFMA_ALL; }

// Which attention kernel serves the descriptor (pointer alignment is checked
// separately: a misaligned call of a fast-path descriptor is refused).
int32_t choose_kernel(const gqa_decode_desc_t* d) {
  const int32_t G = d->num_q_heads / d->num_kv_heads;
  const bool bf16 = d->kv_dtype == GQA_BF16 && d->qo_dtype == GQA_BF16;
  if (quantized(d->kv_dtype)) {
    // Fp8 codes are served by the G <= 16 kernel only (the planner refuses
    // other shapes).
    // G <= 16 on the G <= 16 kernel (which quantizes a step's new rows itself),
    // 16 < G <= 64 on the large-group kernel (codes widened into its LDS tiles).
    // Int8 caches, G <= 64: the G <= 16 kernel (17..64 heads as 32-head chunks
    // of 8 waves, K/V codes read once per chunk and widened in registers;
    // measured faster than the large-group kernel's widened LDS tiles).
    if (d->qo_dtype != GQA_BF16 || d->head_dim != 128) return GQA_KERNEL_GENERIC;
    if (G <= 64 && kHaveMfmaQkI8) return GQA_KERNEL_MFMA_QK;
    return GQA_KERNEL_GENERIC;
  }
  if (bf16 && d->head_dim == 128 && G <= 16 && kHaveMfmaQk) return GQA_KERNEL_MFMA_QK;
  if (bf16 && d->head_dim == 128 && G > 16 && G <= 64 && kHaveMfmaAll) return GQA_KERNEL_MFMA_ALL;
  return GQA_KERNEL_GENERIC;
}

// Compute units of the current device, read once per device; without a
// visible device (host-only planning) the MI355X count.
int32_t device_cus() {
  constexpr int kMaxDev = 256;
  static std::atomic<int32_t> cached[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return kDefaultCUs;
  int32_t v = cached[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = kDefaultCUs;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Plan: a pure function of the descriptor and the device's CU count.
// `span` > 0 bounds the slots any sequence walks (a sliding window with a
// host-known prefix); the splits then cover [0, span) instead of the capacity.
// `generic` forces the vector kernel (paged caches whose blocks the
// matrix-core kernels cannot tile); `small` allows the small-head-width kernel
// (plain calls: it applies no softmax variant).
gqa_status_t make_plan(const gqa_decode_desc_t* d, Plan* p, int64_t span = 0, bool generic = false,
                       bool small = true, bool paged = false) {
  gqa_status_t st = check_desc(d);
  if (st != GQA_OK) return st;
  std::memset(p, 0, sizeof(*p));
  p->hp = 1;
  const int64_t cus = device_cus();
  const int64_t B = d->batch, Hq = d->num_q_heads, Hkv = d->num_kv_heads, D = d->head_dim;
  const int64_t S = span > 0 ? std::min<int64_t>(span, d->capacity) : d->capacity;
  const int64_t G = Hq / Hkv;
  p->kernel = generic ? GQA_KERNEL_GENERIC : choose_kernel(d);
  // Small head widths on short caches, no forced split: one wave per
  // (sequence, query head) with one slot per lane (latency-bound steps).
  if (d->kv_dtype == GQA_FP8 && p->kernel != GQA_KERNEL_MFMA_QK) return GQA_ERR_UNSUPPORTED;
  if (small && p->kernel == GQA_KERNEL_GENERIC && D <= 16 && d->capacity <= 512 && !quantized(d->kv_dtype) &&
      d->num_splits <= 1) {
    p->kernel = GQA_KERNEL_SMALL;
    p->head_chunks = 1;
    p->block = 256;
    p->nsplit = 1;
    p->split_tokens = (int32_t)S;
    const int64_t waves = B * Hq;
    p->grid = (int32_t)std::max<int64_t>(1, (waves + 3) / 4);
    return GQA_OK;
  }
  // Query-head chunks per kv-head: 8 heads per workgroup in the generic
  // kernel, 16 (one MFMA tile) in MFMA_QK, all G in MFMA_ALL.
  // MFMA_QK takes 16 heads per workgroup (4 waves) for G <= 16, 32 (8 waves
  // of two 16-head blocks) above.
  const int64_t qk_heads = G > 16 ? 32 : 16;
  p->head_chunks = p->kernel == GQA_KERNEL_GENERIC ? (int32_t)((G + kGenericHeadChunk - 1) / kGenericHeadChunk)
                   : p->kernel == GQA_KERNEL_MFMA_QK ? (int32_t)((G + qk_heads - 1) / qk_heads)
                                                     : 1;
  // Four waves per workgroup for every kernel but MFMA_QK on int8 / fp8
  // caches with G > 16 (two 16-head blocks per wave).  (For MFMA_QK, measured
  // on MI355X: one 4-wave workgroup per CU streams faster than 8- or 12-wave
  // workgroups or more, shorter splits -- fewer concurrent streams suit HBM.)
  p->block = p->kernel == GQA_KERNEL_MFMA_QK && G > 16 ? 512 : 256;
  // Caches (B, S, Hkv, D) hold a slot's kv-heads side by side: MFMA_QK then
  // gives the four waves of a workgroup four adjacent kv-heads over the same
  // slots (head-parallel), so the workgroup streams contiguous 1 KB row
  // segments instead of one head's 256 bytes per 2 KB row.
  if (p->kernel == GQA_KERNEL_MFMA_QK && G <= 16 && d->layout == GQA_LAYOUT_BSHD && Hkv % 4 == 0) p->hp = 4;
  const int64_t units = std::max<int64_t>(1, B * (Hkv / p->hp) * p->head_chunks);
  int64_t split_tokens;
  if (d->num_splits > 0) {
    const int64_t ns = std::min<int64_t>(d->num_splits, S);
    split_tokens = (S + ns - 1) / ns;
  } else {
    // Workgroups wanted: about one per CU for MFMA_QK (each wave streams its
    // own run of slots with a tile in flight), two per CU for MFMA_ALL (its
    // waves share LDS tiles; more splits would cost partials of G rows of
    // D + 2 floats each), three per CU for the generic kernel.  Splits are
    // equal and at least 256 slots long.
    const int64_t target = p->kernel == GQA_KERNEL_MFMA_QK ? cus : p->kernel == GQA_KERNEL_MFMA_ALL ? 2 * cus : 3 * cus;
    int64_t ns = std::max<int64_t>(1, (target + units / 2) / units);
    ns = std::min<int64_t>(ns, std::max<int64_t>(1, S / 256));
    split_tokens = (S + ns - 1) / ns;
  }
  split_tokens = std::max<int64_t>(split_tokens, (S + kMaxSplits - 1) / kMaxSplits);
  if (split_tokens >= S) split_tokens = S;
  const int64_t nsplit = (S + split_tokens - 1) / split_tokens;
  p->split_tokens = (int32_t)split_tokens;
  p->nsplit = (int32_t)nsplit;
  p->combine = nsplit > 1 ? 1 : 0;
  int64_t grid;
  if (!mul_ok(units, nsplit, &grid) || grid > INT32_MAX) return GQA_ERR_UNSUPPORTED;
  p->grid = (int32_t)grid;
  if (nsplit > 1) {
    const size_t nparts = (size_t)B * Hq * nsplit;
    p->off_m = align256(nparts * D * sizeof(float));
    p->off_l = p->off_m + align256(nparts * sizeof(float));
    p->workspace_bytes = p->off_l + align256(nparts * sizeof(float));
  }
  // More MFMA_QK work items (sequence, kv-head) than CUs and no forced split
  // count: balanced mode.  The work per item follows the sequence lengths, so
  // instead of one workgroup per item, one workgroup per CU takes an equal
  // contiguous range of the batch's units (16-slot tiles plus a per-item cost,
  // cut on the device from the lengths), and the items cut between workgroups
  // are merged by the balanced combine pass.  Its partials: two rows of G
  // heads per workgroup.  Not for huge batches (each workgroup scans the
  // lengths of the whole batch).  (On the large-group kernel the same mode
  // measured slower than its splits: the scan and the extra pieces cost more
  // than the balance gains there.)
  // Each item is charged a piece's fixed cost (start-up and merge: 2.5 us on
  // bf16 caches, 3.4 us on int8 ones, measured on MI355X) in tiles besides its
  // own tiles, so the cut gives workgroups holding many short items fewer tiles.
  // Less where a kv-head's slots are strided (BSHD): there how fast a tile
  // streams depends on the kv-head, which the charge does not see, and larger
  // charges measured slower.
  // MFMA_ALL on dense or slot-indexed caches without splits (whole-item
  // form): one 8-wave workgroup per (sequence, kv-head) item holding all G
  // heads, no partials and no combine pass -- when the items alone fill the
  // device (measured on MI355X: B = 256, G = 64 and 32, S = 2048, lengths in
  // [1024, 2048]: 41 and 38 us against 49-57 and 49 us with splits; with 128
  // items the split form stays ahead), or when one split is asked for.
  if (p->kernel == GQA_KERNEL_MFMA_ALL && !paged && (d->num_splits == 1 || (d->num_splits == 0 && B * Hkv >= cus))) {
    p->all8 = G > 32 ? 4 : 2;
    p->block = 512;
    p->grid = (int32_t)std::max<int64_t>(1, B * Hkv);
    p->nsplit = 1;
    p->split_tokens = (int32_t)S;
    p->combine = 0;
    p->workspace_bytes = 0;
    p->off_m = p->off_l = 0;
  }
  const bool i8 = quantized(d->kv_dtype);
  const int32_t cost = d->layout == GQA_LAYOUT_BHSD ? (i8 ? kBalancedCostI8 : kBalancedCostBf16)
                                                    : (i8 ? kBalancedCostI8Strided : kBalancedCostBf16Strided);
  int64_t units_max;
  if (p->kernel == GQA_KERNEL_MFMA_QK && G <= 16 && d->num_splits == 0 && B * Hkv > cus &&
      B <= kMaxBalancedBatch && mul_ok(B * Hkv, S / 16 + 1 + cost, &units_max) && units_max < INT32_MAX) {
    const size_t rows = (size_t)cus * 2 * G * p->hp;
    p->balanced = 1;
    p->bal_cost = cost;
    p->nsplit = 1;
    p->split_tokens = (int32_t)S;
    p->grid = (int32_t)cus;
    p->combine = 1;
    p->off_m = align256(rows * D * sizeof(float));
    p->off_l = p->off_m + align256(rows * sizeof(float));
    p->off_pre = p->off_l + align256(rows * sizeof(float));
    p->workspace_bytes = p->off_pre + align256((size_t)(B + 1) * sizeof(int32_t));
  }
  return GQA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, lo + bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

// Cache map (mapped entry points).  Shape fields first, then -- for B > 0 --
// the pointers and the whole host table (CLIKA groupQueryAttention page:
// slot rows in range and distinct; block entries -1 or in range, no block
// twice within a row).
gqa_status_t check_map(const gqa_decode_desc_t* d, const gqa_cache_map_t* m, const Plan& p) {
  if (m == nullptr) return GQA_ERR_INVALID_ARGUMENT;
  if ((m->kind != GQA_MAP_SLOTS && m->kind != GQA_MAP_PAGED) || m->num_rows < 1) return GQA_ERR_INVALID_ARGUMENT;
  int64_t t;
  if (m->kind == GQA_MAP_PAGED) {
    if (m->block_size < 1 || m->max_blocks < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (!mul_ok(m->max_blocks, m->block_size, &t) || t != d->capacity) return GQA_ERR_INVALID_ARGUMENT;
    if (!mul_ok(m->num_rows, d->num_kv_heads, &t) || !mul_ok(t, m->block_size, &t) || !mul_ok(t, d->head_dim, &t) ||
        !mul_ok(t, 4, &t))
      return GQA_ERR_UNSUPPORTED;
    if (!mul_ok(d->batch, m->max_blocks, &t)) return GQA_ERR_UNSUPPORTED;
    // The matrix-core kernels take one block per 16-slot tile; other block
    // sizes are planned on the generic kernel (plan_for).
    if (is_matrix_core(p.kernel) && m->block_size % 16 != 0) return GQA_ERR_INTERNAL;
  } else {
    if (!mul_ok(m->num_rows, d->num_kv_heads, &t) || !mul_ok(t, d->capacity, &t) || !mul_ok(t, d->head_dim, &t) ||
        !mul_ok(t, 4, &t))
      return GQA_ERR_UNSUPPORTED;
  }
  if (d->batch == 0) return GQA_OK;
  if (m->map == nullptr || m->map_host == nullptr || (reinterpret_cast<uintptr_t>(m->map) & 3) != 0)
    return GQA_ERR_INVALID_ARGUMENT;
  // One pass over the table: a per-thread stamp array (one word per cache row
  // or pool block, grown on demand and reused across calls) marks the entries
  // seen in the current group -- the whole slot map, or one table row -- so a
  // repeat is found in O(1) without sorting.
  thread_local std::vector<uint32_t> stamp;
  thread_local uint32_t epoch = 0;
  if (stamp.size() < (size_t)m->num_rows) stamp.assign((size_t)m->num_rows, 0u);
  auto next_epoch = [&]() {
    if (++epoch == 0) {  // wrapped: forget every old mark
      std::fill(stamp.begin(), stamp.end(), 0u);
      epoch = 1;
    }
  };
  const int32_t* h = m->map_host;
  if (m->kind == GQA_MAP_SLOTS) {
    next_epoch();
    for (int64_t b = 0; b < d->batch; ++b) {
      const int32_t x = h[b];
      if (x < 0 || x >= m->num_rows || stamp[x] == epoch) return GQA_ERR_INVALID_ARGUMENT;
      stamp[x] = epoch;
    }
  } else {
    for (int64_t b = 0; b < d->batch; ++b) {
      next_epoch();
      const int32_t* row = h + b * (int64_t)m->max_blocks;
      for (int64_t j = 0; j < m->max_blocks; ++j) {
        const int32_t x = row[j];
        if (x == -1) continue;
        if (x < 0 || x >= m->num_rows || stamp[x] == epoch) return GQA_ERR_INVALID_ARGUMENT;
        stamp[x] = epoch;
      }
    }
  }
  return GQA_OK;
}

// Elements of one cache tensor (K or V) and bytes of the device table.
size_t cache_elems(const gqa_decode_desc_t* d, const gqa_cache_map_t* m) {
  const size_t Hkv = d->num_kv_heads, S = d->capacity, D = d->head_dim;
  if (m == nullptr) return (size_t)d->batch * Hkv * S * D;
  if (m->kind == GQA_MAP_SLOTS) return (size_t)m->num_rows * Hkv * S * D;
  return (size_t)m->num_rows * Hkv * (size_t)m->block_size * D;
}
size_t map_bytes(const gqa_decode_desc_t* d, const gqa_cache_map_t* m) {
  if (m == nullptr) return 0;
  return (size_t)d->batch * (m->kind == GQA_MAP_SLOTS ? 1 : (size_t)m->max_blocks) * 4;
}

void fill_args(const gqa_decode_desc_t* d, const Plan& p, AttnArgs* a) {
  std::memset(a, 0, sizeof(*a));
  a->B = d->batch;
  a->Hq = d->num_q_heads;
  a->Hkv = d->num_kv_heads;
  a->D = d->head_dim;
  a->S = d->capacity;
  a->G = d->num_q_heads / d->num_kv_heads;
  const int64_t S = d->capacity, D = d->head_dim, Hkv = d->num_kv_heads;
  if (d->layout == GQA_LAYOUT_BHSD) {
    a->sb = Hkv * S * D;
    a->sh = S * D;
    a->st = D;
  } else {
    a->sb = S * Hkv * D;
    a->sh = D;
    a->st = Hkv * D;
  }
  a->nsplit = p.nsplit;
  a->split_tokens = p.split_tokens;
  a->head_chunks = p.head_chunks;
  a->hp = p.hp;
  a->kv_dtype = d->kv_dtype;
  a->qo_dtype = d->qo_dtype;
  a->scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d->head_dim));
}

// Map fields and pool strides of a mapped call (dense calls keep map_kind 0).
void fill_map(const gqa_decode_desc_t* d, const gqa_cache_map_t* m, AttnArgs* a) {
  if (m == nullptr) return;
  a->map = m->map;
  a->map_kind = m->kind;
  a->map_rows = m->num_rows;
  if (m->kind == GQA_MAP_PAGED) {
    const int64_t bs = m->block_size, D = d->head_dim, Hkv = d->num_kv_heads;
    a->bs = m->block_size;
    a->max_blocks = m->max_blocks;
    a->sblk = Hkv * bs * D;
    if (d->layout == GQA_LAYOUT_BHSD) {  // pool (blocks, Hkv, bs, D)
      a->sh = bs * D;
      a->st = D;
    } else {                             // pool (blocks, bs, Hkv, D)
      a->sh = D;
      a->st = Hkv * D;
    }
    a->sb = 0;
  }
}

// Pointer checks shared by attend and step.  `k_new`/`v_new` are null for attend.
gqa_status_t check_attend_ptrs(const gqa_decode_desc_t* d, const gqa_cache_map_t* m, const Plan& p, const void* q,
                               const void* kc, const void* vc, const void* kn, const void* vn,
                               const int32_t* lengths, const void* out, const void* ws, size_t ws_bytes,
                               bool step) {
  const size_t ekv = elem_bytes(d->kv_dtype), eqo = elem_bytes(d->qo_dtype);
  const size_t enew = quantized(d->kv_dtype) ? eqo : ekv;  // quantized caches take new K/V as activations
  if (!q || !kc || !vc || !lengths || !out) return GQA_ERR_INVALID_ARGUMENT;
  if (step && (!kn || !vn)) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(q, eqo) || !aligned(out, eqo) || !aligned(kc, ekv) || !aligned(vc, ekv) || !aligned(lengths, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  if (step && (!aligned(kn, enew) || !aligned(vn, enew))) return GQA_ERR_INVALID_ARGUMENT;
  if (is_matrix_core(p.kernel)) {
    // The matrix-core kernels read q, caches and new K/V with 16-byte loads.
    if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16)) return GQA_ERR_INVALID_ARGUMENT;
    if (step && (!aligned(kn, 16) || !aligned(vn, 16))) return GQA_ERR_INVALID_ARGUMENT;
  }
  if (p.workspace_bytes > 0) {
    if (ws_bytes < p.workspace_bytes) return GQA_ERR_WORKSPACE_TOO_SMALL;
    if (!ws || !aligned(ws, 256)) return GQA_ERR_INVALID_ARGUMENT;
  }
  const size_t B = d->batch, Hq = d->num_q_heads, Hkv = d->num_kv_heads, S = d->capacity, D = d->head_dim;
  const Span s_out = span(out, B * Hq * D * eqo);
  const Span s_q = span(q, B * Hq * D * eqo);
  (void)S;
  const Span s_kc = span(kc, cache_elems(d, m) * ekv);
  const Span s_vc = span(vc, cache_elems(d, m) * ekv);
  const Span s_len = span(lengths, B * 4);
  const Span s_ws = span(ws, p.workspace_bytes);
  const Span s_map = span(m ? m->map : nullptr, map_bytes(d, m));
  if (m != nullptr && (overlap(s_out, s_map) || (p.workspace_bytes > 0 && overlap(s_ws, s_map)) ||
                       (step && (overlap(s_kc, s_map) || overlap(s_vc, s_map)))))
    return GQA_ERR_INVALID_ARGUMENT;
  if (overlap(s_out, s_q) || overlap(s_out, s_kc) || overlap(s_out, s_vc) || overlap(s_out, s_len) ||
      (p.workspace_bytes > 0 && (overlap(s_out, s_ws) || overlap(s_ws, s_q) || overlap(s_ws, s_kc) ||
                                 overlap(s_ws, s_vc) || overlap(s_ws, s_len))))
    return GQA_ERR_INVALID_ARGUMENT;
  if (step) {
    const Span s_kn = span(kn, B * Hkv * D * enew), s_vn = span(vn, B * Hkv * D * enew);
    if (overlap(s_kc, s_vc) || overlap(s_kn, s_kc) || overlap(s_kn, s_vc) || overlap(s_vn, s_kc) ||
        overlap(s_vn, s_vc) || overlap(s_out, s_kn) || overlap(s_out, s_vn) || overlap(s_len, s_kc) ||
        overlap(s_len, s_vc) ||
        (p.workspace_bytes > 0 && (overlap(s_ws, s_kn) || overlap(s_ws, s_vn))))
      return GQA_ERR_INVALID_ARGUMENT;
  }
  return GQA_OK;
}

gqa_status_t run_attend(const gqa_decode_desc_t* d, const Plan& p, AttnArgs& a, hipStream_t s, void* workspace) {
  hipError_t e;
  if (p.balanced) {
    char* w = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(w);
    a.part_m = reinterpret_cast<float*>(w + p.off_m);
    a.part_l = reinterpret_cast<float*>(w + p.off_l);
    a.bal_pre = reinterpret_cast<int32_t*>(w + p.off_pre);
    a.bal_units = p.grid;
    a.bal_cost = p.bal_cost;
  }
  switch (p.kernel) {
    case GQA_KERNEL_MFMA_QK: e = launch_attend_mfma_qk(a, p, s); break;
    case GQA_KERNEL_MFMA_ALL: e = launch_attend_mfma_all(a, p, s); break;
    case GQA_KERNEL_SMALL: e = launch_attend_small(a, p, s); break;
    default: {
      const size_t ekv = elem_bytes(d->kv_dtype);
      const bool vec = (d->head_dim * ekv) % 16 == 0 && aligned(a.k_cache, 16) && aligned(a.v_cache, 16) &&
                       (a.k_new == nullptr || (aligned(a.k_new, 16) && aligned(a.v_new, 16)));
      e = launch_attend_generic(a, p, vec ? 1 : 0, s);
    }
  }
  if (e != hipSuccess) return GQA_ERR_HIP;
  if (p.combine) {
    e = launch_combine(a, p, s);
    if (e != hipSuccess) return GQA_ERR_HIP;
  }
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status_t gqa_decode_workspace_size(const gqa_decode_desc_t* desc, size_t* bytes) {
  try {
    if (bytes == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    Plan p;
    gqa_status_t st = make_plan(desc, &p);
    if (st != GQA_OK) return st;
    *bytes = p.workspace_bytes;
    return GQA_OK;
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_get_plan(const gqa_decode_desc_t* desc, gqa_decode_plan_t* plan) {
  try {
    if (plan == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    Plan p;
    gqa_status_t st = make_plan(desc, &p);
    if (st != GQA_OK) return st;
    plan->kernel = p.kernel;
    plan->num_splits = p.nsplit;
    plan->split_tokens = p.split_tokens;
    plan->grid = p.grid;
    plan->block = p.block;
    plan->combine = p.combine;
    plan->workspace_bytes = p.workspace_bytes;
    plan->balanced = p.balanced;
    plan->heads_per_item = p.hp;
    return GQA_OK;
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

}  // extern "C"

namespace {

// Int8 caches need their row scales and nothing else does; scales are 4-byte
// aligned float32 arrays with one entry per cache row (the cache's shape
// without the last axis, mapped caches included) that overlap no other buffer
// (`others`: the call's other spans).
gqa_status_t check_scales(const gqa_decode_desc_t* d, const gqa_kv_scales_t* sc) {
  if (quantized(d->kv_dtype) != (sc != nullptr)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}
gqa_status_t check_scale_ptrs(const gqa_decode_desc_t* d, const gqa_cache_map_t* map, const gqa_kv_scales_t* sc,
                              std::initializer_list<Span> others) {
  if (sc == nullptr) return GQA_OK;
  if (!sc->k_scale || !sc->v_scale || !aligned(sc->k_scale, 4) || !aligned(sc->v_scale, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  const size_t n = cache_elems(d, map) / d->head_dim * 4;
  const Span ks = span(sc->k_scale, n), vs = span(sc->v_scale, n);
  if (overlap(ks, vs)) return GQA_ERR_INVALID_ARGUMENT;
  for (const Span& o : others)
    if (overlap(ks, o) || overlap(vs, o)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}

// Rotary encoding: the descriptor-level rules (before the batch-0 early
// return), then the pointers (tables, positions, gains: read-only inputs that
// must not overlap anything the call writes, `written`).
gqa_status_t check_rope(const gqa_decode_desc_t* d, const gqa_rope_t* r) {
  if (r == nullptr) return GQA_OK;
  if (d->head_dim % 2 != 0 || r->max_pos < 1) return GQA_ERR_INVALID_ARGUMENT;
  if (r->mode != GQA_ROPE_HALF && r->mode != GQA_ROPE_INTERLEAVED) return GQA_ERR_INVALID_ARGUMENT;
  const bool gains = r->q_norm_gain != nullptr || r->k_norm_gain != nullptr;
  const bool eps = r->norm_eps >= 0.f && std::isfinite(r->norm_eps);
  if (gains != eps) return GQA_ERR_INVALID_ARGUMENT;
  if (gains && quantized(d->kv_dtype)) return GQA_ERR_UNSUPPORTED;
  int64_t t;
  if (!mul_ok(r->max_pos, d->head_dim, &t) || !mul_ok(t, 2, &t)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}
gqa_status_t check_rope_ptrs(const gqa_decode_desc_t* d, const gqa_rope_t* r, std::initializer_list<Span> written) {
  if (r == nullptr) return GQA_OK;
  if (!r->cos || !r->sin || !aligned(r->cos, 16) || !aligned(r->sin, 16)) return GQA_ERR_INVALID_ARGUMENT;
  if (!aligned(r->positions, 4) || !aligned(r->q_norm_gain, 4) || !aligned(r->k_norm_gain, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  const size_t tb = (size_t)r->max_pos * (d->head_dim / 2) * 4, gb = (size_t)d->head_dim * 4;
  const Span in[] = {span(r->cos, tb), span(r->sin, tb), span(r->positions, r->positions ? d->batch * 4 : 0),
                     span(r->q_norm_gain, r->q_norm_gain ? gb : 0), span(r->k_norm_gain, r->k_norm_gain ? gb : 0)};
  for (const Span& w : written)
    for (const Span& x : in)
      if (overlap(w, x)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}
void fill_rope(const gqa_rope_t* r, AttnArgs* a) {
  a->rope_cos = r->cos;
  a->rope_sin = r->sin;
  a->rope_pos = r->positions;
  a->q_gain = r->q_norm_gain;
  a->k_gain = r->k_norm_gain;
  a->rope_max_pos = r->max_pos;
  a->rope_mode = r->mode;
  a->norm_eps = r->norm_eps;
}

// Softmax variants: the values (before the batch-0 early return), then the
// device arrays, which must not overlap anything the call writes.
gqa_status_t check_softmax(const gqa_decode_desc_t* d, const gqa_softmax_t* v) {
  (void)d;
  if (v == nullptr) return GQA_OK;
  if (v->smooth != 0 && v->smooth != 1) return GQA_ERR_INVALID_ARGUMENT;
  if (v->smooth && v->sink != nullptr) return GQA_ERR_INVALID_ARGUMENT;
  if (!(v->softcap >= 0.f) || !std::isfinite(v->softcap)) return GQA_ERR_INVALID_ARGUMENT;
  if (v->window < 0 || v->kept_prefix < 0) return GQA_ERR_INVALID_ARGUMENT;
  if (v->window == 0 && (v->kept_prefix != 0 || v->kept_prefix_per_seq != nullptr)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}
gqa_status_t check_softmax_ptrs(const gqa_decode_desc_t* d, const gqa_softmax_t* v,
                                std::initializer_list<Span> written) {
  if (v == nullptr) return GQA_OK;
  if (!aligned(v->sink, 4) || !aligned(v->kept_prefix_per_seq, 4)) return GQA_ERR_INVALID_ARGUMENT;
  const Span in[] = {span(v->sink, v->sink ? (size_t)d->num_q_heads * 4 : 0),
                     span(v->kept_prefix_per_seq, v->kept_prefix_per_seq ? (size_t)d->batch * 4 : 0)};
  for (const Span& w : written)
    for (const Span& x : in)
      if (overlap(w, x)) return GQA_ERR_INVALID_ARGUMENT;
  return GQA_OK;
}
// Slots a sequence walks at most: with a window W and a kept prefix P known on
// the host, the virtual range is below W + P + 32 (0: no bound).
int64_t walk_span(const gqa_softmax_t* v) {
  if (v == nullptr || v->window <= 0 || v->kept_prefix < 0 || v->kept_prefix_per_seq != nullptr) return 0;
  return (int64_t)v->window + v->kept_prefix + 32;
}

void fill_softmax(const gqa_decode_desc_t* d, const gqa_softmax_t* v, AttnArgs* a) {
  if (v == nullptr) return;
  a->sink = v->sink;
  a->smooth = v->smooth;
  if (v->softcap > 0.f) {
    a->cap_T = (float)((double)v->softcap * std::sqrt((double)d->head_dim));
    a->cap_invT = (float)(1.0 / ((double)v->softcap * std::sqrt((double)d->head_dim)));
  }
  a->window = v->window;
  a->prefix = v->kept_prefix;
  a->prefix_seq = v->kept_prefix_per_seq;
}

const gqa_decode_opts_t kNoOpts = {nullptr, nullptr, nullptr, nullptr};

// The plan of an attend/step call with options: the descriptor's, over the
// window's span when one is known, and on the generic kernel for paged caches
// whose block size is not a multiple of the matrix-core kernels' 16-slot tile.
gqa_status_t plan_for(const gqa_decode_desc_t* d, const gqa_decode_opts_t* o, Plan* p) {
  const bool small = o->softmax == nullptr;
  gqa_status_t st = make_plan(d, p, walk_span(o->softmax), false, small);
  if (st != GQA_OK) return st;
  const gqa_cache_map_t* m = o->map;
  if (m != nullptr && m->kind == GQA_MAP_PAGED && m->block_size > 0 && m->block_size % 16 != 0 &&
      is_matrix_core(p->kernel))
    return make_plan(d, p, walk_span(o->softmax), true, small);
  // Paged caches: the large-group kernel's split form (tiles of 16-slot halves, one table entry each).
  if (m != nullptr && m->kind == GQA_MAP_PAGED && p->all8)
    return make_plan(d, p, walk_span(o->softmax), false, small, true);
  return st;
}

// Bytes of the rotated q a rotary step keeps after the plan's workspace.
size_t rope_q_offset(const Plan& p) { return align256(p.workspace_bytes); }
// MFMA_ALL rotates q and the new key itself on bf16 caches; the other paths
// (and int8 caches) read a rotated copy written by the rotary append.
bool rope_fused(const Plan& p, const gqa_decode_opts_t* o) {
  return p.kernel == GQA_KERNEL_MFMA_ALL && o->scales == nullptr;
}
size_t workspace_total(const gqa_decode_desc_t* d, const Plan& p, const gqa_decode_opts_t* o) {
  if (o->rope == nullptr || rope_fused(p, o)) return p.workspace_bytes;
  return rope_q_offset(p) + (size_t)d->batch * d->num_q_heads * d->head_dim * elem_bytes(d->qo_dtype);
}

gqa_status_t do_append(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, void* k_cache, void* v_cache,
                       const void* k_new, const void* v_new, const int32_t* lengths, void* stream) {
  gqa_status_t st = check_desc(desc);
  if (st != GQA_OK) return st;
  const gqa_decode_opts_t* o = opts ? opts : &kNoOpts;
  const gqa_cache_map_t* map = o->map;
  const gqa_kv_scales_t* sc = o->scales;
  if ((st = check_scales(desc, sc)) != GQA_OK) return st;
  if ((st = check_rope(desc, o->rope)) != GQA_OK) return st;
  if (o->softmax != nullptr) return GQA_ERR_INVALID_ARGUMENT;  // the append computes no softmax
  Plan p;
  std::memset(&p, 0, sizeof(p));
  p.kernel = GQA_KERNEL_GENERIC;  // the append kernel takes any block size
  p.nsplit = 1;
  if (map != nullptr && (st = check_map(desc, map, p)) != GQA_OK) return st;
  if (desc->batch == 0) return GQA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !lengths) return GQA_ERR_INVALID_ARGUMENT;
  const size_t e = elem_bytes(desc->kv_dtype);
  const size_t en = sc ? elem_bytes(desc->qo_dtype) : e;  // int8 caches take new K/V as activations
  if (!aligned(k_cache, e) || !aligned(v_cache, e) || !aligned(k_new, en) || !aligned(v_new, en) ||
      !aligned(lengths, 4))
    return GQA_ERR_INVALID_ARGUMENT;
  const size_t B = desc->batch, Hkv = desc->num_kv_heads, D = desc->head_dim;
  const Span s_kc = span(k_cache, cache_elems(desc, map) * e), s_vc = span(v_cache, cache_elems(desc, map) * e);
  const Span s_kn = span(k_new, B * Hkv * D * en), s_vn = span(v_new, B * Hkv * D * en);
  const Span s_len = span(lengths, B * 4);
  const Span s_map = span(map ? map->map : nullptr, map_bytes(desc, map));
  if (overlap(s_kc, s_vc) || overlap(s_kn, s_kc) || overlap(s_kn, s_vc) || overlap(s_vn, s_kc) ||
      overlap(s_vn, s_vc) || overlap(s_len, s_kc) || overlap(s_len, s_vc) || overlap(s_map, s_kc) ||
      overlap(s_map, s_vc))
    return GQA_ERR_INVALID_ARGUMENT;
  if ((st = check_scale_ptrs(desc, map, sc, {s_kc, s_vc, s_kn, s_vn, s_len, s_map})) != GQA_OK) return st;
  const size_t sb = sc ? cache_elems(desc, map) / D * 4 : 0;
  if ((st = check_rope_ptrs(desc, o->rope,
                            {s_kc, s_vc, span(sc ? sc->k_scale : nullptr, sb), span(sc ? sc->v_scale : nullptr, sb)})) !=
      GQA_OK)
    return st;
  AttnArgs a;
  fill_args(desc, p, &a);
  fill_map(desc, map, &a);
  a.k_new = k_new;
  a.v_new = v_new;
  a.lengths = lengths;
  if (sc != nullptr) {
    a.k_scale_w = sc->k_scale;
    a.v_scale_w = sc->v_scale;
  }
  hipError_t e2;
  if (o->rope != nullptr) {
    fill_rope(o->rope, &a);
    e2 = launch_rope_append(a, k_cache, v_cache, (hipStream_t)stream);
  } else if (sc != nullptr) {
    e2 = launch_append_q8(a, k_cache, v_cache, (hipStream_t)stream);
  } else {
    e2 = launch_append(a, k_cache, v_cache, (hipStream_t)stream);
  }
  return e2 == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

// Attend (step == false) or fused step (step == true), with options.
gqa_status_t do_attend(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, const void* q, void* k_cache,
                       void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths, void* out,
                       void* workspace, size_t workspace_bytes, void* stream, bool step) {
  const gqa_decode_opts_t* o = opts ? opts : &kNoOpts;
  Plan p;
  gqa_status_t st = plan_for(desc, o, &p);
  if (st != GQA_OK) return st;
  const gqa_cache_map_t* map = o->map;
  const gqa_kv_scales_t* sc = o->scales;
  const gqa_rope_t* rope = o->rope;
  if ((st = check_scales(desc, sc)) != GQA_OK) return st;
  if (rope != nullptr && !step) return GQA_ERR_INVALID_ARGUMENT;  // rotation belongs to the append
  if ((st = check_rope(desc, rope)) != GQA_OK) return st;
  if ((st = check_softmax(desc, o->softmax)) != GQA_OK) return st;
  if (map != nullptr && (st = check_map(desc, map, p)) != GQA_OK) return st;
  if (desc->batch == 0) return GQA_OK;
  Plan pw = p;  // the plan with the whole workspace the call needs (rotated q after the partials)
  pw.workspace_bytes = workspace_total(desc, p, o);
  st = check_attend_ptrs(desc, map, pw, q, k_cache, v_cache, step ? k_new : nullptr, step ? v_new : nullptr,
                         lengths, out, workspace, workspace_bytes, step);
  if (st != GQA_OK) return st;
  const size_t B = desc->batch, Hq = desc->num_q_heads, Hkv = desc->num_kv_heads, D = desc->head_dim;
  const size_t eqo = elem_bytes(desc->qo_dtype), ce = cache_elems(desc, map) * elem_bytes(desc->kv_dtype);
  if (sc != nullptr) {
    st = check_scale_ptrs(desc, map, sc,
                          {span(q, B * Hq * D * eqo), span(out, B * Hq * D * eqo), span(k_cache, ce),
                           span(v_cache, ce), span(lengths, B * 4), span(workspace, pw.workspace_bytes),
                           span(step ? k_new : nullptr, step ? B * Hkv * D * eqo : 0),
                           span(step ? v_new : nullptr, step ? B * Hkv * D * eqo : 0),
                           span(map ? map->map : nullptr, map_bytes(desc, map))});
    if (st != GQA_OK) return st;
  }
  if (rope != nullptr) {
    const size_t sb = sc ? cache_elems(desc, map) / D * 4 : 0;
    st = check_rope_ptrs(desc, rope,
                         {span(out, B * Hq * D * eqo), span(k_cache, ce), span(v_cache, ce),
                          span(workspace, pw.workspace_bytes), span(sc ? sc->k_scale : nullptr, sb),
                          span(sc ? sc->v_scale : nullptr, sb)});
    if (st != GQA_OK) return st;
  }
  if (o->softmax != nullptr) {
    const size_t sb = sc ? cache_elems(desc, map) / D * 4 : 0;
    st = check_softmax_ptrs(desc, o->softmax,
                            {span(out, B * Hq * D * eqo), span(workspace, pw.workspace_bytes),
                             span(step ? k_cache : nullptr, step ? ce : 0),
                             span(step ? v_cache : nullptr, step ? ce : 0),
                             span(step && sc ? sc->k_scale : nullptr, step ? sb : 0),
                             span(step && sc ? sc->v_scale : nullptr, step ? sb : 0)});
    if (st != GQA_OK) return st;
  }
  AttnArgs a;
  fill_args(desc, p, &a);
  fill_map(desc, map, &a);
  fill_softmax(desc, o->softmax, &a);
  if (sc != nullptr) {
    a.k_scale = sc->k_scale;
    a.v_scale = sc->v_scale;
  }
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.lengths = lengths;
  a.out = out;
  a.len_offset = step ? 1 : 0;
  if (p.nsplit > 1) {
    char* w = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(w);
    a.part_m = reinterpret_cast<float*>(w + p.off_m);
    a.part_l = reinterpret_cast<float*>(w + p.off_l);
  }
  if (step) {
    a.k_new = k_new;
    a.v_new = v_new;
    if (rope != nullptr && rope_fused(p, o)) {
      // Rotary step on MFMA_ALL: every workgroup rotates its q (all G heads of
      // its kv-head), the workgroup whose split holds slot lengths[b] rotates
      // the new key, attends it and stores it.  (On the G <= 16 kernel the
      // same fusion measured slower than the separate rotary append: its
      // single workgroup per CU pays the prologue's dependent loads in full.)
      fill_rope(rope, &a);
      if (sc != nullptr) {
        a.k_scale_w = sc->k_scale;
        a.v_scale_w = sc->v_scale;
      }
      a.k_cache_w = k_cache;
      a.v_cache_w = v_cache;
    } else if (rope != nullptr) {
      // Rotary step, other kernels: the rope append kernel writes the rotated key
      // (quantized for int8 caches) and the value at slot lengths[b] and the
      // rotated q into the workspace; attention over lengths[b] + 1 slots then
      // reads it.
      if (sc != nullptr) {
        a.k_scale_w = sc->k_scale;
        a.v_scale_w = sc->v_scale;
      }
      fill_rope(rope, &a);
      a.q_rot = static_cast<char*>(workspace) + rope_q_offset(p);
      if (launch_rope_append(a, k_cache, v_cache, (hipStream_t)stream) != hipSuccess) return GQA_ERR_HIP;
      a.q = a.q_rot;
      a.k_new = nullptr;
      a.v_new = nullptr;
      a.rope_cos = nullptr;  // the attention pass reads the rotated q and key as they are
    } else if (sc != nullptr && p.kernel == GQA_KERNEL_GENERIC) {
      // Int8 caches, generic path: the quantizing append, then attention over
      // lengths[b] + 1 slots (the new token is attended in its stored,
      // quantized form).
      a.k_scale_w = sc->k_scale;
      a.v_scale_w = sc->v_scale;
      if (launch_append_q8(a, k_cache, v_cache, (hipStream_t)stream) != hipSuccess) return GQA_ERR_HIP;
      a.k_new = nullptr;
      a.v_new = nullptr;
    } else if (sc != nullptr) {
      // Int8 caches, matrix-core paths: the workgroup whose split holds slot
      // lengths[b] quantizes the new rows itself, attends them in their
      // quantized form and stores codes and scales.
      a.k_scale_w = sc->k_scale;
      a.v_scale_w = sc->v_scale;
      a.k_cache_w = k_cache;
      a.v_cache_w = v_cache;
    } else {
      // Every kernel fuses the append: the workgroup whose split holds slot
      // lengths[b] takes the new K/V from k_new/v_new and writes it to the
      // cache (one head chunk of it); no other workgroup reads that slot.
      a.k_cache_w = k_cache;
      a.v_cache_w = v_cache;
    }
  }
  return run_attend(desc, p, a, (hipStream_t)stream, workspace);
}

}  // namespace

extern "C" {

gqa_status_t gqa_decode_append(const gqa_decode_desc_t* desc, void* k_cache, void* v_cache, const void* k_new,
                               const void* v_new, const int32_t* lengths, void* stream) {
  try {
    return do_append(desc, nullptr, k_cache, v_cache, k_new, v_new, lengths, stream);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_attend(const gqa_decode_desc_t* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* lengths, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  try {
    return do_attend(desc, nullptr, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), nullptr, nullptr,
                     lengths, out, workspace, workspace_bytes, stream, false);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_step(const gqa_decode_desc_t* desc, const void* q, void* k_cache, void* v_cache,
                             const void* k_new, const void* v_new, const int32_t* lengths, void* out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  try {
    return do_attend(desc, nullptr, q, k_cache, v_cache, k_new, v_new, lengths, out, workspace, workspace_bytes,
                     stream, true);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_append_mapped(const gqa_decode_desc_t* desc, const gqa_cache_map_t* map, void* k_cache,
                                      void* v_cache, const void* k_new, const void* v_new,
                                      const int32_t* lengths, void* stream) {
  try {
    if (map == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t o = {map, nullptr, nullptr, nullptr};
    return do_append(desc, &o, k_cache, v_cache, k_new, v_new, lengths, stream);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_attend_mapped(const gqa_decode_desc_t* desc, const gqa_cache_map_t* map, const void* q,
                                      const void* k_cache, const void* v_cache, const int32_t* lengths, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (map == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t o = {map, nullptr, nullptr, nullptr};
    return do_attend(desc, &o, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), nullptr, nullptr, lengths,
                     out, workspace, workspace_bytes, stream, false);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_step_mapped(const gqa_decode_desc_t* desc, const gqa_cache_map_t* map, const void* q,
                                    void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                    const int32_t* lengths, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  try {
    if (map == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t o = {map, nullptr, nullptr, nullptr};
    return do_attend(desc, &o, q, k_cache, v_cache, k_new, v_new, lengths, out, workspace, workspace_bytes, stream,
                     true);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_append_q8(const gqa_decode_desc_t* desc, const gqa_kv_scales_t* scales, void* k_cache,
                                  void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths,
                                  void* stream) {
  try {
    if (scales == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t o = {nullptr, scales, nullptr, nullptr};
    return do_append(desc, &o, k_cache, v_cache, k_new, v_new, lengths, stream);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_attend_q8(const gqa_decode_desc_t* desc, const gqa_kv_scales_t* scales, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* lengths, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (scales == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t o = {nullptr, scales, nullptr, nullptr};
    return do_attend(desc, &o, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), nullptr, nullptr, lengths,
                     out, workspace, workspace_bytes, stream, false);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_step_q8(const gqa_decode_desc_t* desc, const gqa_kv_scales_t* scales, const void* q,
                                void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                const int32_t* lengths, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  try {
    if (scales == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t o = {nullptr, scales, nullptr, nullptr};
    return do_attend(desc, &o, q, k_cache, v_cache, k_new, v_new, lengths, out, workspace, workspace_bytes, stream,
                     true);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_workspace_size_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts,
                                          size_t* bytes) {
  try {
    if (bytes == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t* o = opts ? opts : &kNoOpts;
    Plan p;
    gqa_status_t st = plan_for(desc, o, &p);
    if (st != GQA_OK) return st;
    if ((st = check_rope(desc, o->rope)) != GQA_OK) return st;
    if ((st = check_softmax(desc, o->softmax)) != GQA_OK) return st;
    *bytes = workspace_total(desc, p, o);
    return GQA_OK;
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_get_plan_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts,
                                    gqa_decode_plan_t* plan) {
  try {
    if (plan == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    const gqa_decode_opts_t* o = opts ? opts : &kNoOpts;
    Plan p;
    gqa_status_t st = plan_for(desc, o, &p);
    if (st != GQA_OK) return st;
    if ((st = check_rope(desc, o->rope)) != GQA_OK) return st;
    if ((st = check_softmax(desc, o->softmax)) != GQA_OK) return st;
    plan->kernel = p.kernel;
    plan->num_splits = p.nsplit;
    plan->split_tokens = p.split_tokens;
    plan->grid = p.grid;
    plan->block = p.block;
    plan->combine = p.combine;
    plan->workspace_bytes = workspace_total(desc, p, o);
    plan->balanced = p.balanced;
    plan->heads_per_item = p.hp;
    return GQA_OK;
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_append_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, void* k_cache,
                                  void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths,
                                  void* stream) {
  try {
    return do_append(desc, opts, k_cache, v_cache, k_new, v_new, lengths, stream);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_attend_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* lengths, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  try {
    return do_attend(desc, opts, q, const_cast<void*>(k_cache), const_cast<void*>(v_cache), nullptr, nullptr,
                     lengths, out, workspace, workspace_bytes, stream, false);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_step_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, const void* q,
                                void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                const int32_t* lengths, void* out, void* workspace, size_t workspace_bytes,
                                void* stream) {
  try {
    return do_attend(desc, opts, q, k_cache, v_cache, k_new, v_new, lengths, out, workspace, workspace_bytes,
                     stream, true);
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

gqa_status_t gqa_decode_check_lengths(const gqa_decode_desc_t* desc, const int32_t* lengths, int32_t mode,
                                      void* stream, int32_t* bad_count) {
  try {
    gqa_status_t st = check_desc(desc);
    if (st != GQA_OK) return st;
    if ((mode != 0 && mode != 1) || bad_count == nullptr) return GQA_ERR_INVALID_ARGUMENT;
    if (desc->batch == 0) {
      *bad_count = 0;
      return GQA_OK;
    }
    if (lengths == nullptr || (reinterpret_cast<uintptr_t>(lengths) & 3) != 0) return GQA_ERR_INVALID_ARGUMENT;
    const int32_t lo = mode == 0 ? 0 : 1;
    const int32_t hi = mode == 0 ? desc->capacity - 1 : desc->capacity;
    if (run_check_lengths(lengths, desc->batch, lo, hi, (hipStream_t)stream, bad_count) != hipSuccess)
      return GQA_ERR_HIP;
    return GQA_OK;
  } catch (...) {
    return GQA_ERR_INTERNAL;
  }
}

const char* gqa_decode_status_string(gqa_status_t s) {
  switch (s) {
    case GQA_OK: return "GQA_OK";
    case GQA_ERR_INVALID_ARGUMENT: return "GQA_ERR_INVALID_ARGUMENT";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED";
    case GQA_ERR_WORKSPACE_TOO_SMALL: return "GQA_ERR_WORKSPACE_TOO_SMALL";
    case GQA_ERR_HIP: return "GQA_ERR_HIP";
    case GQA_ERR_INTERNAL: return "GQA_ERR_INTERNAL";
  }
  return "GQA_ERR_UNKNOWN";
}

int32_t gqa_decode_version(void) { return kVersion; }

}  // extern "C"

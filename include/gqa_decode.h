/*
 * gqa_decode.h -- C ABI of the MI355X (gfx950) grouped-query attention decode step.
 *
 * One decode step of one attention layer for a batch of sequences:
 *   1. append: each sequence's new key/value (one per kv-head) is written in
 *      place at slot lengths[b] of a fixed-capacity cache;
 *   2. attend: every query head h reads cache head floor(h / G), G = Hq / Hkv,
 *      and returns softmax(q . K_j / sqrt(D)) weighted sums of V_j over the
 *      valid slots only.
 *
 * Sources of the semantics (web pages, cited by title and section):
 *   - TensorTonic, "KV cache decode step" problem page (CS336 L10): problem
 *     statement -- query (B,Hq,D), new key/value (B,Hkv,D), caches
 *     (B,Hkv,S,D); contiguous groups (query head hG+g of kv-head h); the new
 *     key/value take position S; the softmax runs over every cached position
 *     plus the new token; dtype is preserved.
 *   - TensorTonic, "Grouped-Query Decode Step" (JAX) problem page: problem
 *     statement and formulas -- caches (B,S,Hkv,D), query head h reads cache
 *     head floor(h/G), only slots j < lengths[b] are valid (the new token
 *     already among them), s_j = q.K_j/sqrt(D), softmax, o = sum w_j V_j;
 *     requirements -- stale slots get zero weight, bfloat16 caches are
 *     widened to float32 and scores/softmax/sums run in float32; constraints
 *     -- lengths is int32 (B,), each in [1,S].
 *   - CLIKA runtime, "groupQueryAttention" API page: the decode perf path
 *     appends the new K/V in place into the bound cache; a read-only attend is
 *     a separate call; malformed arguments are refused with INVALID_ARGUMENT
 *     once every argument has been checked, before any data is read.
 *   - Huawei CANN, "aclnnMlaPrologV3WeightNz" operator page: two-phase call
 *     convention (a size/validation phase, then execution), status-code
 *     returns, empty batch allowed with caches left untouched.
 *
 * Conventions shared by every entry point
 *   - All tensors are caller-owned, dense, row-major buffers in device memory
 *     of the current HIP device.  The library allocates nothing, keeps no
 *     pointer after returning and never writes `lengths`.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without synchronising:
 *     GQA_OK means "validated and enqueued"; a fault inside a kernel surfaces
 *     at the caller's next synchronisation.
 *   - Every condition the host can check is checked before anything is
 *     enqueued; on any error nothing has been enqueued or written.
 *   - `lengths` lives on the device and is never read by the host, so every
 *     call can be captured in a HIP graph.  Values outside the documented
 *     range do not fault: append skips the write, attend clamps the count to
 *     [0, capacity], and a sequence with no valid slot yields zeros; such
 *     outputs are outside the numerical contract.
 *   - Storage types: GQA_F32 = IEEE binary32, GQA_BF16 = bfloat16 (upper half of
 *     a binary32).  Scores, softmax and sums are float32 whatever the storage;
 *     a bf16 output is rounded to nearest-even from the float32 result.
 *   - Calls are deterministic: the same inputs give the same bits (no
 *     floating-point atomics; reductions have a fixed order).
 */
#ifndef GQA_DECODE_H
#define GQA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARGUMENT = 1,    /* malformed descriptor, null/misaligned/overlapping pointer */
  GQA_ERR_UNSUPPORTED = 2,         /* well-formed but not implemented (head_dim > 256, sizes
                                      beyond the limits in gqa_decode_desc_t)                    */
  GQA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below gqa_decode_workspace_size()         */
  GQA_ERR_HIP = 4,                 /* a HIP launch failed                                       */
  GQA_ERR_INTERNAL = 5             /* unexpected library error (no C++ exception crosses)       */
} gqa_status_t;

enum {
  GQA_F32 = 0,
  GQA_BF16 = 1,
  GQA_I8 = 2,  /* int8 codes with per-row scales: the _q8 calls (and _ex with scales) only            */
  GQA_FP8 = 3  /* OCP E4M3 codes with per-row scales: as GQA_I8; head_dim 128, bf16 q/out and
                  Hq/Hkv <= 64 only (GQA_ERR_UNSUPPORTED otherwise)                                    */
};
enum {
  GQA_LAYOUT_BHSD = 0,  /* caches (B, Hkv, S, D): KV cache decode step page            */
  GQA_LAYOUT_BSHD = 1   /* caches (B, S, Hkv, D): JAX Grouped-Query Decode Step page   */
};

typedef struct {
  int32_t batch;        /* B >= 0.  B == 0: the call validates the descriptor, returns GQA_OK
                           and enqueues nothing (pointers may then be NULL).               */
  int32_t num_q_heads;  /* Hq >= 1, a multiple of num_kv_heads                              */
  int32_t num_kv_heads; /* Hkv >= 1; Hkv * head_dim * 4 <= 2^32 - 1 (GQA_ERR_UNSUPPORTED
                           otherwise), as are caches beyond 2^63 bytes and B * Hq > 2^31 - 1 */
  int32_t head_dim;     /* D in [1, 256]; D > 256 is GQA_ERR_UNSUPPORTED                    */
  int32_t capacity;     /* S >= 1 slots per (sequence, kv-head) in both caches              */
  int32_t layout;       /* GQA_LAYOUT_BHSD or GQA_LAYOUT_BSHD, shared by both caches         */
  int32_t kv_dtype;     /* storage of k_cache, v_cache, k_new, v_new: GQA_F32 or GQA_BF16
                           (GQA_I8 or GQA_FP8 for the _q8 calls, whose k_new/v_new are in
                           qo_dtype)                                                          */
  int32_t qo_dtype;     /* storage of q and out: GQA_F32 or GQA_BF16                         */
  int32_t num_splits;   /* 0 = library's choice; n > 0 asks for n splits of the token axis
                           (the plan uses at most 64, and fewer when n would leave a split
                           empty; results agree within rounding for every n)                */
} gqa_decode_desc_t;

/* How a call with this descriptor runs (introspection for tests and tuning).
 * A pure function of the descriptor: never of `lengths` or of pointers. */
typedef struct {
  int32_t kernel;        /* GQA_KERNEL_* of the attention pass                              */
  int32_t num_splits;    /* splits of the token axis                                        */
  int32_t split_tokens;  /* slots per split (the last split may be shorter)                 */
  int32_t grid;          /* workgroups of the attention pass                                */
  int32_t block;         /* threads per workgroup of the attention pass                     */
  int32_t combine;       /* 1 if a combine pass follows the attention pass                  */
  size_t workspace_bytes;
  int32_t balanced;      /* 1 if each workgroup of the attention pass takes an equal share of
                            the batch's 16-slot tiles (each (b, kv-head) item also charged a
                            fixed cost in tiles), cut on the device from `lengths` (ragged
                            batches with more (b, kv-head) items than CUs); the combine pass
                            then merges the items cut between workgroups                   */
  int32_t heads_per_item; /* kv-heads one workgroup takes over the same slots: 1, or 4 when the
                             small-group matrix-core kernel reads a BSHD cache (its four waves
                             take four adjacent kv-heads, so the workgroup reads whole 1 KB
                             spans of each slot's row)                                       */
} gqa_decode_plan_t;

enum {
  GQA_KERNEL_GENERIC = 0,  /* vector ALU, any D <= 256, f32 or bf16 storage                  */
  GQA_KERNEL_MFMA_QK = 1,  /* bf16 caches with G <= 16, or int8 caches (bf16 q/out) with G <= 64;
                              D = 128: scores and V sum on MFMA, K/V rows loaded straight into
                              the MFMA operands                                                */
  GQA_KERNEL_MFMA_ALL = 2, /* bf16, D = 128, 16 < G <= 64: scores and V sum on MFMA; block 512:
                              one workgroup per (b, kv-head) item, no split (dense or slot-indexed
                              caches whose items fill the device, or one split asked for)        */
  GQA_KERNEL_SMALL = 3     /* f32 or bf16, D <= 16, capacity <= 512, no softmax variant and no
                              forced split: one wave per (sequence, query head)                 */
};

/* Phase one (CANN operator page, two-phase call convention): validate the
 * descriptor and report the workspace the attend/step calls need, in bytes
 * (0 when the token axis is not split and the plan is not balanced).  Returns GQA_ERR_INVALID_ARGUMENT or
 * GQA_ERR_UNSUPPORTED for a bad descriptor; *bytes is then untouched. */
gqa_status_t gqa_decode_workspace_size(const gqa_decode_desc_t* desc, size_t* bytes);

/* The execution plan for `desc` (see gqa_decode_plan_t). */
gqa_status_t gqa_decode_get_plan(const gqa_decode_desc_t* desc, gqa_decode_plan_t* plan);

/* In-place append (KV cache decode step page, problem statement: the new key
 * and value occupy the position after the cached ones; CLIKA
 * groupQueryAttention: in-place append into the bound cache).
 *   k_cache, v_cache : (B,Hkv,S,D) or (B,S,Hkv,D) per desc->layout, kv_dtype, written
 *   k_new, v_new     : (B, Hkv, D), kv_dtype, read
 *   lengths          : int32 (B,), device; lengths[b] = tokens held before the call.
 *                      Slot lengths[b] of every kv-head of sequence b receives a raw
 *                      copy of the new key/value bits; no other byte changes.
 *                      Contract: 0 <= lengths[b] < S (otherwise that sequence is skipped).
 * Pointers must be non-null and aligned to the element size; k_cache/v_cache
 * must not overlap each other or k_new/v_new. */
gqa_status_t gqa_decode_append(const gqa_decode_desc_t* desc, void* k_cache, void* v_cache,
                               const void* k_new, const void* v_new, const int32_t* lengths,
                               void* stream);

/* Read-only attend (JAX Grouped-Query Decode Step page, problem statement and
 * formulas; CLIKA groupQueryAttention: attention over the cache without
 * present outputs).
 *   q        : (B, Hq, D), qo_dtype, read
 *   k_cache, v_cache : per desc->layout, kv_dtype, read only
 *   lengths  : int32 (B,), device; lengths[b] = valid slots (the new token already
 *              stored among them).  Contract: 1 <= lengths[b] <= S.
 *   out      : (B, Hq, D), qo_dtype, written; out[b,h] = sum_{j<lengths[b]} w_j V_j of
 *              cache head h / (Hq/Hkv); must not overlap any other argument.
 *   workspace: device scratch of at least gqa_decode_workspace_size() bytes, 256-byte
 *              aligned (may be NULL when that size is 0).  It holds the split partials
 *              (balanced plans: the partials of cut items and the batch's tile
 *              offsets, written by the attention pass for the combine pass);
 *              its contents on entry do not matter, it needs no clearing and it may be
 *              reused by later calls with any descriptor.  Calls that run concurrently
 *              must not share one workspace.
 *              Split plans (num_splits > 1, not balanced) leave, for every (b, hq)
 *              whose valid slots reach more than one split, the partial of each split
 *              s holding valid slots ([s * split_tokens, min((s + 1) * split_tokens,
 *              n)), n = attended slots): with i = (b * Hq + hq) * num_splits + s,
 *              o = float32 [D] at byte offset 4 * i * D (the unnormalised weighted
 *              sum), m = float32 at byte offset off_m + 4 * i (the reference maximum
 *              in log2 units) and l = float32 at off_l + 4 * i (the denominator),
 *              with off_m = align256(4 * B * Hq * num_splits * D) and off_l = off_m +
 *              align256(4 * B * Hq * num_splits), align256(x) = x rounded up to a
 *              multiple of 256.  o / l is the softmax-weighted mean of V over the
 *              split's slots, in float32 before the output's rounding; the layout
 *              is exposed so tests can check that arithmetic, not as a data
 *              interface.
 * Pointers must be non-null and aligned to the element size; when the plan's
 * kernel is a matrix-core one (bf16 storage, head_dim 128, G <= 64), q, out and
 * the caches must be 16-byte aligned (GQA_ERR_INVALID_ARGUMENT otherwise). */
gqa_status_t gqa_decode_attend(const gqa_decode_desc_t* desc, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* lengths, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Fused decode step = append, then attend over lengths[b] + 1 slots (KV cache
 * decode step page: the softmax covers every cached position plus the new
 * token).  Arguments as in gqa_decode_append and gqa_decode_attend;
 * lengths[b] is the pre-append count (contract: 0 <= lengths[b] < S).  The
 * caller advances lengths itself afterwards (for example lengths += 1 on the
 * same stream).  On the matrix-core kernels k_new and v_new must be 16-byte
 * aligned as well. */
gqa_status_t gqa_decode_step(const gqa_decode_desc_t* desc, const void* q, void* k_cache,
                             void* v_cache, const void* k_new, const void* v_new,
                             const int32_t* lengths, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Mapped caches (CLIKA runtime, "groupQueryAttention" API page: the slot_ids
 * and paged block-table parameters).  The same decode step on caches that are
 * not indexed by batch row:
 *
 *   GQA_MAP_SLOTS  continuous cache of num_rows rows; batch row b appends to and
 *                  attends from cache row map[b].  Caches (num_rows, Hkv, S, D)
 *                  for GQA_LAYOUT_BHSD or (num_rows, S, Hkv, D) for BSHD, with
 *                  S = desc->capacity.  map: int32 [B], every entry in
 *                  [0, num_rows) and no two equal.
 *   GQA_MAP_PAGED  block pool of num_blocks blocks of block_size slots; token j
 *                  of batch row b lives in block map[b * max_blocks + j /
 *                  block_size] at slot j % block_size.  Pools (num_blocks, Hkv,
 *                  block_size, D) for BHSD or (num_blocks, block_size, Hkv, D)
 *                  for BSHD; desc->capacity must equal max_blocks * block_size.
 *                  map: int32 [B, max_blocks], every entry -1 (unused tail
 *                  pad) or in [0, num_blocks), and no block named twice within
 *                  one row.  Blocks holding slots below a row's length must not
 *                  be -1 (the device lengths are not checked, as above).
 *
 * The table is passed twice with the same entries: `map` in device memory for
 * the kernels and `map_host` in host memory, every entry of which is checked
 * before anything is enqueued (an out-of-range or repeated entry refuses
 * GQA_ERR_INVALID_ARGUMENT).  The device copy is trusted to match; entries it
 * holds out of range are clamped (reads) or skip the write (append), so a
 * mismatch cannot fault.  Rows of a paged table may share blocks for reading;
 * a step or append into a block shared by two rows races.
 * Matrix-core kernels serve paged caches whose block_size is a multiple of 16
 * (their 16-slot tiles then never straddle a block); calls with another block
 * size are planned on the generic kernel, whose plan (and workspace) can
 * differ from the descriptor's: size the workspace of a mapped call with
 * gqa_decode_workspace_size_ex (or read gqa_decode_get_plan_ex) with the map.
 * ------------------------------------------------------------------------- */
enum { GQA_MAP_SLOTS = 1, GQA_MAP_PAGED = 2 };
typedef struct {
  int32_t kind;              /* GQA_MAP_SLOTS or GQA_MAP_PAGED                              */
  int32_t num_rows;          /* SLOTS: cache rows; PAGED: pool blocks.  >= 1               */
  int32_t block_size;        /* PAGED: slots per block, >= 1 (ignored for SLOTS)            */
  int32_t max_blocks;        /* PAGED: table columns, >= 1 (ignored for SLOTS)              */
  const int32_t* map;        /* device table (4-byte aligned)                               */
  const int32_t* map_host;   /* host copy of the same entries                               */
} gqa_cache_map_t;

/* As gqa_decode_append / _attend / _step, with caches addressed through `map`.
 * The descriptor's batch, heads, head_dim, capacity, layout and dtypes keep
 * their meaning (capacity = slots per sequence); the workspace size and plan
 * are gqa_decode_workspace_size_ex / gqa_decode_get_plan_ex with the map (the
 * descriptor's own, unless the block size sends the call to the generic
 * kernel, or a paged map sends a large-group call planned without splits to
 * the split form of its kernel).  B == 0 validates and enqueues nothing. */
gqa_status_t gqa_decode_append_mapped(const gqa_decode_desc_t* desc, const gqa_cache_map_t* map, void* k_cache,
                                      void* v_cache, const void* k_new, const void* v_new,
                                      const int32_t* lengths, void* stream);
gqa_status_t gqa_decode_attend_mapped(const gqa_decode_desc_t* desc, const gqa_cache_map_t* map, const void* q,
                                      const void* k_cache, const void* v_cache, const int32_t* lengths, void* out,
                                      void* workspace, size_t workspace_bytes, void* stream);
gqa_status_t gqa_decode_step_mapped(const gqa_decode_desc_t* desc, const gqa_cache_map_t* map, const void* q,
                                    void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                    const int32_t* lengths, void* out, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---------------------------------------------------------------------------
 * Int8 caches with per-row scales (Huawei CANN "aclnnMlaPrologV3WeightNz"
 * operator page, dynamic-quantization formula: a row's dequantization scale is
 * its largest absolute value divided by 127 and its code the row divided by
 * that scale, rounded).  desc->kv_dtype = GQA_I8: the caches hold int8 codes in
 * the descriptor's layout, and every (sequence, kv-head, slot) row has a float32
 * scale; a cached value reads as code * scale.
 *   k_scale, v_scale : float32 (B, Hkv, S) for GQA_LAYOUT_BHSD, (B, S, Hkv) for
 *                      BSHD (mapped caches through gqa_decode_*_ex: the pool's
 *                      shape without the last axis); read by attend, the
 *                      appended rows written by append and step.
 *   k_new, v_new     : (B, Hkv, D) in desc->qo_dtype (the model's activations);
 *                      each row is quantized on the device: float32 widening,
 *                      scale = max|x| / 127 and code = round-half-even(x / scale)
 *                      with correctly rounded float32 divisions (a zero row has
 *                      scale 0 and codes 0).
 * desc->kv_dtype = GQA_FP8: the caches hold 8-bit floating-point codes in the
 * OCP E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals, largest finite magnitude 448; the pages define no fp8 format, so
 * the rule above is taken over with the code's largest value): scale =
 * max|x| / 448 and code = the E4M3 value nearest to x / scale clamped to
 * [-448, 448] (ties to even, the quotient's sign kept), correctly rounded
 * float32 divisions, a zero row with scale 0 and codes 0; a value reads as
 * decoded code * scale.  Served for head_dim 128, bf16 q/out and
 * num_q_heads / num_kv_heads <= 64 (GQA_ERR_UNSUPPORTED otherwise; the append
 * alone takes any shape).
 * Other arguments, contracts and errors as in the unquantized calls; the
 * unquantized calls refuse GQA_I8 and GQA_FP8 (GQA_ERR_INVALID_ARGUMENT).
 * Scale arrays must be 4-byte aligned and overlap no other argument.
 * ------------------------------------------------------------------------- */
typedef struct {
  float* k_scale;
  float* v_scale;
} gqa_kv_scales_t;

gqa_status_t gqa_decode_append_q8(const gqa_decode_desc_t* desc, const gqa_kv_scales_t* scales, void* k_cache,
                                  void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths,
                                  void* stream);
gqa_status_t gqa_decode_attend_q8(const gqa_decode_desc_t* desc, const gqa_kv_scales_t* scales, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* lengths, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);
gqa_status_t gqa_decode_step_q8(const gqa_decode_desc_t* desc, const gqa_kv_scales_t* scales, const void* q,
                                void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                const int32_t* lengths, void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---------------------------------------------------------------------------
 * Rotary position encoding fused into the append (CLIKA runtime,
 * "groupQueryAttention" API page, operator summary: q and the new k are rotated
 * with the rope planes and the post-rotation key is appended in place; optional
 * per-head RMS norm gains applied after the rotation, before the append; the
 * Huawei CANN "aclnnMlaPrologV3WeightNz" page rotates its query and key the
 * same way and gives the RmsNorm formula, epsilon inside the square root).
 *   cos, sin     : float32 (max_pos, D/2) tables in device memory, 16-byte aligned;
 *                  row p holds the angles of position p, column i the i-th rotation pair.
 *   mode         : GQA_ROPE_HALF pairs elements (i, i + D/2); GQA_ROPE_INTERLEAVED
 *                  pairs (2i, 2i + 1).  A pair (x1, x2) at position p becomes
 *                  (x1 c - x2 s, x2 c + x1 s), c = cos[p][i], s = sin[p][i], in float32
 *                  with each product and sum rounded separately (no fused
 *                  multiply-add), so a stored key is a reproducible rounding.
 *   positions    : int32 (B,) device, the new token's position per sequence, or NULL:
 *                  position lengths[b] (its cache slot).  Contract: 0 <= p < max_pos
 *                  (out-of-range positions are clamped into the table, memory-safe,
 *                  outside the numerical contract).
 *   q_norm_gain, k_norm_gain : float32 (D,) device, or NULL.  A gain normalizes the
 *                  rotated vector of every head: x / sqrt(mean(x^2) + norm_eps) * gain.
 *   norm_eps     : >= 0 when a gain is given; < 0 when neither is (a gain without
 *                  an epsilon, or an epsilon without a gain, is GQA_ERR_INVALID_ARGUMENT).
 * The step rotates q (every query head, at its sequence's position) and the new
 * key, appends the rotated key and the unchanged value at slot lengths[b], and
 * attends with the rotated q; the append alone rotates the key only.  The
 * rotated q is kept in the workspace (gqa_decode_workspace_size_ex), rounded to
 * qo_dtype.  D must be even.  Int8 caches take the rotation (the rotated key is
 * then quantized) but not the norm gains (GQA_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------- */
enum { GQA_ROPE_HALF = 0, GQA_ROPE_INTERLEAVED = 1 };

typedef struct {
  const float* cos;
  const float* sin;
  int32_t max_pos;
  int32_t mode;
  const int32_t* positions;
  const float* q_norm_gain;
  const float* k_norm_gain;
  float norm_eps;
} gqa_rope_t;

/* ---------------------------------------------------------------------------
 * Softmax variants (CLIKA runtime, "groupQueryAttention" API page, parameter
 * list and operator summary: head_sink, smooth_softmax, softcap,
 * sliding_window, kept_prefix).  For sequence b with n attended-valid slots
 * (lengths[b] + 1 for a step, lengths[b] for attend) the query is the newest
 * token, slot n - 1:
 *   window       : W > 0 keeps the slots j >= n - W (the last W, the new token's
 *                  own included) plus the kept prefix j < P; 0 keeps every slot.
 *   kept_prefix  : P >= 0 (negative: GQA_ERR_INVALID_ARGUMENT), used with a window
 *                  only (a prefix without a window is GQA_ERR_INVALID_ARGUMENT);
 *   kept_prefix_per_seq : int32 (B,) device, one P per sequence, or NULL (kept_prefix
 *                  for all); negative device values count as 0.
 *   softcap      : c > 0 maps each scaled score s = q.k / sqrt(D) to c tanh(s / c)
 *                  before the softmax; 0 leaves it.
 *   sink         : float32 (Hq,) device, a per-query-head logit added to the
 *                  softmax denominator only: w_j = e^(s_j) / (sum_i e^(s_i) + e^(sink));
 *                  NULL: none.
 *   smooth       : 1 adds a zero logit for every head (a sink of 0); not combined
 *                  with `sink` (GQA_ERR_INVALID_ARGUMENT).
 * With no attended slot the output is zeros.  Sink and prefix arrays must be
 * 4-byte aligned and overlap nothing the call writes.
 * ------------------------------------------------------------------------- */
typedef struct {
  const float* sink;
  int32_t smooth;
  float softcap;
  int32_t window;
  int32_t kept_prefix;
  const int32_t* kept_prefix_per_seq;
} gqa_softmax_t;

/* Options of the _ex calls; every member may be NULL (the plain behaviour).
 *   map     : mapped caches, as in the _mapped calls
 *   scales  : int8 caches (desc->kv_dtype = GQA_I8), as in the _q8 calls; with a
 *             map the scale arrays have the mapped caches' shape without the
 *             last axis ((num_rows, Hkv, S) / (num_rows, S, Hkv) for slot rows,
 *             (num_blocks, Hkv, block_size) / (num_blocks, block_size, Hkv) for
 *             a paged pool): the scale of a row sits at the row's index
 *   rope    : rotary encoding (append and step only)
 *   softmax : softmax variants (attend and step) */
typedef struct {
  const gqa_cache_map_t* map;
  const gqa_kv_scales_t* scales;
  const gqa_rope_t* rope;
  const gqa_softmax_t* softmax;
} gqa_decode_opts_t;

/* Workspace of an attend/step call with these options (the plain size plus the
 * rotated q when opts->rope is set).  opts may be NULL. */
gqa_status_t gqa_decode_workspace_size_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts,
                                          size_t* bytes);
/* The execution plan of an attend/step call with these options (the window's
 * span, the generic kernel for paged blocks the matrix-core kernels cannot
 * tile); workspace_bytes as gqa_decode_workspace_size_ex.  opts may be NULL. */
gqa_status_t gqa_decode_get_plan_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts,
                                    gqa_decode_plan_t* plan);
/* The append, attend and step calls with options; arguments, contracts and
 * errors as in the plain calls and the sections above.  opts may be NULL. */
gqa_status_t gqa_decode_append_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, void* k_cache,
                                  void* v_cache, const void* k_new, const void* v_new, const int32_t* lengths,
                                  void* stream);
gqa_status_t gqa_decode_attend_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, const void* q,
                                  const void* k_cache, const void* v_cache, const int32_t* lengths, void* out,
                                  void* workspace, size_t workspace_bytes, void* stream);
gqa_status_t gqa_decode_step_ex(const gqa_decode_desc_t* desc, const gqa_decode_opts_t* opts, const void* q,
                                void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                                const int32_t* lengths, void* out, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Debugging aid, not on the hot path: counts the entries of the device array
 * `lengths` (B = desc->batch entries) that lie outside the contract of a call
 * (JAX Grouped-Query Decode Step page, constraints: lengths in [1, S] for the
 * read-only attend; KV cache decode step page: the new token goes to slot
 * lengths[b], so 0 <= lengths[b] < S for append and step).
 *   mode      : 0 = append/step contract, 1 = attend contract
 *   bad_count : host pointer, receives the count
 * Synchronous: enqueues one small kernel on `stream`, copies the count back and
 * waits for the stream.  Calls are serialised inside the library (the count
 * lives in one device variable per GPU).  B == 0 gives 0 without a GPU call.
 * Errors: GQA_ERR_INVALID_ARGUMENT for a bad descriptor or mode, or a null
 * `bad_count` (or null `lengths` with B > 0); GQA_ERR_HIP if a HIP call fails. */
gqa_status_t gqa_decode_check_lengths(const gqa_decode_desc_t* desc, const int32_t* lengths, int32_t mode,
                                      void* stream, int32_t* bad_count);

/* Static, NUL-terminated name of a status code. */
const char* gqa_decode_status_string(gqa_status_t status);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gqa_decode_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_DECODE_H */

"""Float64 CPU oracle for the decode step on mapped caches.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.oracle``): only the tests, the
smoke check and the benchmark's CPU-baseline leg may use it; it shares no code
with the HIP library.

Source: CLIKA runtime, "groupQueryAttention" API page (the operator's
parameter notes on ``slot_ids`` and on the paged block table):

* Slot-indexed cache.  Batch row ``b`` appends to and attends from cache row
  ``slot_ids[b]`` of a continuous cache with ``R`` rows; every entry lies in
  ``[0, R)`` and no two batch rows share one.
* Paged cache.  A block table of shape ``(B, max_blocks)`` maps the tokens of
  batch row ``b`` to blocks of a pool: token ``j`` is slot ``j % bs`` of block
  ``table[b, j // bs]``.  Every entry of the table is checked before the
  caches are touched: ``-1`` (the pad of the unused tail) or a block index in
  ``[0, num_blocks)``, and no block appears twice in one row.

Everything else is the decode step of ``oracle.oracle`` (append at slot
``lengths[b]``, then attend over ``lengths[b] + 1`` slots, or attend over
``lengths[b]`` slots): the mapped functions only change *where* slot ``j`` of
(sequence ``b``, kv-head ``h``) is stored.

Storage layouts (raw buffers as NumPy arrays, float32 or uint16 bf16 bits):

* slots, ``"BHSD"``: ``(R, Hkv, S, D)``;  ``"BSHD"``: ``(R, S, Hkv, D)``.
* paged, ``"BHSD"``: ``(num_blocks, Hkv, bs, D)``;  ``"BSHD"``:
  ``(num_blocks, bs, Hkv, D)`` -- the block is the outer index, the rest is the
  dense layout with the block's ``bs`` slots as its slot axis.
"""

from __future__ import annotations

import numpy as np

from .oracle import attend_one, decode

__all__ = [
    "validate_slots",
    "validate_table",
    "slot_location",
    "mapped_rows",
    "append_mapped",
    "attend_mapped",
    "step_mapped",
    "append_q8_mapped",
    "attend_q8_mapped",
    "step_q8_mapped",
]

KINDS = ("slots", "paged")
LAYOUTS = ("BHSD", "BSHD")


def validate_slots(slot_ids, num_rows: int) -> None:
    """Raise ValueError unless every entry is in [0, num_rows) and none repeats."""
    s = np.asarray(slot_ids)
    if s.ndim != 1:
        raise ValueError("slot_ids is 1-D")
    for b, v in enumerate(s.tolist()):
        if not 0 <= v < num_rows:
            raise ValueError(f"slot_ids[{b}]={v} outside [0, {num_rows})")
    if len(set(s.tolist())) != s.size:
        raise ValueError("two batch rows share a cache row")


def validate_table(table, num_blocks: int) -> None:
    """Raise ValueError unless every entry is -1 or in [0, num_blocks) and no
    block appears twice within one row."""
    t = np.asarray(table)
    if t.ndim != 2:
        raise ValueError("the block table is 2-D")
    for b in range(t.shape[0]):
        seen = set()
        for j, v in enumerate(t[b].tolist()):
            if v == -1:
                continue
            if not 0 <= v < num_blocks:
                raise ValueError(f"table[{b}, {j}]={v} is neither -1 nor in [0, {num_blocks})")
            if v in seen:
                raise ValueError(f"table row {b} names block {v} twice")
            seen.add(v)


def slot_location(kind: str, layout: str, mapping, b: int, h: int, j: int, bs: int | None = None):
    """Index tuple, in the cache array, of slot ``j`` of kv-head ``h`` of batch row ``b``."""
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    if kind == "slots":
        row = int(mapping[b])
        return (row, h, j) if layout == "BHSD" else (row, j, h)
    if kind == "paged":
        blk = int(mapping[b][j // bs])
        if blk < 0:
            raise ValueError(f"token {j} of row {b} falls in an unmapped block")
        off = j % bs
        return (blk, h, off) if layout == "BHSD" else (blk, off, h)
    raise ValueError(f"unknown kind {kind!r}")


def mapped_rows(cache, kind: str, layout: str, mapping, b: int, h: int, n: int, bs: int | None = None):
    """The first ``n`` slots of (b, h), gathered one by one, shape (n, D)."""
    D = cache.shape[-1]
    rows = np.empty((n, D), dtype=cache.dtype)
    for j in range(n):
        rows[j] = cache[slot_location(kind, layout, mapping, b, h, j, bs)]
    return rows


def _dims(kind, cache, layout, mapping, bs):
    if kind not in KINDS:
        raise ValueError(f"unknown kind {kind!r}")
    if cache.ndim != 4:
        raise ValueError("a cache is 4-D")
    if layout == "BHSD":
        _, Hkv, inner, D = cache.shape
    elif layout == "BSHD":
        _, inner, Hkv, D = cache.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    m = np.asarray(mapping)
    if kind == "slots":
        validate_slots(m, cache.shape[0])
        B, S = m.shape[0], inner
    else:
        if bs is None or bs != inner:
            raise ValueError("block_size must match the pool's slot axis")
        validate_table(m, cache.shape[0])
        B, S = m.shape[0], m.shape[1] * bs
    return B, Hkv, S, D


def append_mapped(kind: str, k_cache, v_cache, k_new, v_new, lengths, layout: str, mapping, bs=None):
    """Expected caches after the in-place append at slot ``lengths[b]``."""
    B, Hkv, S, D = _dims(kind, k_cache, layout, mapping, bs)
    if v_cache.shape != k_cache.shape or k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D):
        raise ValueError("shape mismatch")
    lengths = np.asarray(lengths)
    k_out, v_out = k_cache.copy(), v_cache.copy()
    for b in range(B):
        pos = int(lengths[b])
        if not 0 <= pos < S:
            raise ValueError(f"lengths[{b}]={pos} leaves no free slot in capacity {S}")
        for h in range(Hkv):
            idx = slot_location(kind, layout, mapping, b, h, pos, bs)
            k_out[idx] = k_new[b, h]
            v_out[idx] = v_new[b, h]
    return k_out, v_out


def attend_mapped(kind: str, q, q_dtype: str, k_cache, v_cache, kv_dtype: str, lengths, layout: str,
                  num_q_heads: int, num_kv_heads: int, mapping, bs=None):
    """Length-masked GQA attention over mapped caches, float64 (B, Hq, D)."""
    B, Hkv, S, D = _dims(kind, k_cache, layout, mapping, bs)
    Hq = num_q_heads
    if num_kv_heads != Hkv or Hq % Hkv != 0 or q.shape != (B, Hq, D):
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    qf = decode(q, q_dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(lengths[b])
        if not 0 <= n <= S:
            raise ValueError(f"lengths[{b}]={n} outside [0, {S}]")
        for h in range(Hkv):
            K = decode(mapped_rows(k_cache, kind, layout, mapping, b, h, n, bs), kv_dtype)
            V = decode(mapped_rows(v_cache, kind, layout, mapping, b, h, n, bs), kv_dtype)
            for hq in range(h * G, (h + 1) * G):
                out[b, hq] = attend_one(qf[b, hq], K, V)
    return out


def step_mapped(kind: str, q, q_dtype: str, k_cache, v_cache, k_new, v_new, kv_dtype: str, lengths,
                layout: str, num_q_heads: int, num_kv_heads: int, mapping, bs=None):
    """Append at ``lengths[b]``, then attend over ``lengths[b] + 1`` slots.
    Returns ``(out, k_cache_after, v_cache_after)``."""
    k_out, v_out = append_mapped(kind, k_cache, v_cache, k_new, v_new, lengths, layout, mapping, bs)
    n_valid = np.asarray(lengths).astype(np.int64) + 1
    out = attend_mapped(kind, q, q_dtype, k_out, v_out, kv_dtype, n_valid, layout, num_q_heads, num_kv_heads,
                        mapping, bs)
    return out, k_out, v_out


# ---------------------------------------------------------------------------
# Int8 caches with per-row scales through a map: the CLIKA page lists kScale /
# vScale beside slot_ids and the block table as parameters of one operator.
# The scale arrays have the cache array's shape without the last axis (one
# float32 per stored row), so slot j of (b, h) has its scale at the same index
# tuple as its row; values read as code * scale, and an append quantizes the
# new row by the rule of ``oracle.quant`` (Huawei CANN aclnnMlaPrologV3WeightNz
# page, dynamic-quantization formula) and stores codes and scale there.
# ---------------------------------------------------------------------------
def append_q8_mapped(kind: str, k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_dtype: str, lengths,
                     layout: str, mapping, bs=None):
    """Expected quantized caches and scales (int8 or fp8 codes) after the quantizing append at slot
    ``lengths[b]``."""
    from .quant import code_format, quantize_row
    B, Hkv, S, D = _dims(kind, k_cache, layout, mapping, bs)
    fmt = code_format(k_cache)                 # int8 codes, or uint8 fp8 patterns
    if v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise ValueError("quantized caches of one code format and shape")
    if k_scale.shape != k_cache.shape[:3] or v_scale.shape != k_cache.shape[:3]:
        raise ValueError("scales have the caches' shape without the last axis")
    kn = decode(k_new, new_dtype).astype(np.float32)
    vn = decode(v_new, new_dtype).astype(np.float32)
    kc, vc, ks, vs = k_cache.copy(), v_cache.copy(), k_scale.copy(), v_scale.copy()
    lengths = np.asarray(lengths)
    for b in range(B):
        pos = int(lengths[b])
        if not 0 <= pos < S:
            raise ValueError(f"lengths[{b}]={pos} leaves no free slot in capacity {S}")
        for h in range(Hkv):
            idx = slot_location(kind, layout, mapping, b, h, pos, bs)
            kc[idx], ks[idx] = quantize_row(kn[b, h], fmt)
            vc[idx], vs[idx] = quantize_row(vn[b, h], fmt)
    return kc, vc, ks, vs


def attend_q8_mapped(kind: str, q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, lengths, layout: str,
                     num_q_heads: int, num_kv_heads: int, mapping, bs=None):
    """Length-masked GQA attention over mapped quantized rows read as code * scale, float64 (B, Hq, D)."""
    from .quant import dequantize
    B, Hkv, S, D = _dims(kind, k_cache, layout, mapping, bs)
    Hq = num_q_heads
    if num_kv_heads != Hkv or Hq % Hkv != 0 or q.shape != (B, Hq, D):
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    qf = decode(q, q_dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(lengths[b])
        if not 0 <= n <= S:
            raise ValueError(f"lengths[{b}]={n} outside [0, {S}]")
        for h in range(Hkv):
            at = [slot_location(kind, layout, mapping, b, h, j, bs) for j in range(n)]
            K = dequantize(np.array([k_cache[i] for i in at]).reshape(n, D),
                           np.array([k_scale[i] for i in at], dtype=np.float32))
            V = dequantize(np.array([v_cache[i] for i in at]).reshape(n, D),
                           np.array([v_scale[i] for i in at], dtype=np.float32))
            for hq in range(h * G, (h + 1) * G):
                out[b, hq] = attend_one(qf[b, hq], K, V)
    return out


def step_q8_mapped(kind: str, q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, k_new, v_new, lengths,
                   layout: str, num_q_heads: int, num_kv_heads: int, mapping, bs=None):
    """Quantizing append at ``lengths[b]`` (new rows stored as ``q_dtype``), then
    attend over ``lengths[b] + 1`` slots.  Returns (out, k_cache, v_cache,
    k_scale, v_scale) after the step."""
    kc, vc, ks, vs = append_q8_mapped(kind, k_cache, v_cache, k_scale, v_scale, k_new, v_new, q_dtype, lengths,
                                      layout, mapping, bs)
    n = np.asarray(lengths).astype(np.int64) + 1
    out = attend_q8_mapped(kind, q, q_dtype, kc, vc, ks, vs, n, layout, num_q_heads, num_kv_heads, mapping, bs)
    return out, kc, vc, ks, vs

"""Float64 CPU oracle for the grouped-query attention (GQA) decode step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it. It shares no code with the HIP library and imports
nothing from it.

What it computes, and where each piece is defined:

* Append (``append``): the new key and value of every (sequence, kv-head) are
  written at the position just after the cached tokens -- TensorTonic, "KV cache
  decode step" (CS336 L10 problem page), problem statement: the new key/value
  occupy position S after all cached positions and the caches come back
  extended.  With a fixed-capacity cache and per-sequence lengths that position
  is ``lengths[b]`` (the number of tokens held before the call).  The write is a
  raw copy of the stored bits: the same page asks that dtype be preserved, and
  its third worked example shows the appended key unchanged.

* Attend (``attend``): TensorTonic, "Grouped-Query Decode Step" (JAX problem
  page), problem statement and its three formulas:
  query head ``h`` reads cache head ``floor(h / G)`` with ``G = Hq / Hkv``;
  only slots ``j < lengths[b]`` hold real tokens; ``s_j = q . K_j / sqrt(D)``,
  ``w_j = exp(s_j) / sum_{m < lengths[b]} exp(s_m)``, ``o = sum_j w_j V_j``.
  Slots at or beyond the length get zero weight.  The same page's requirements
  ask for float32 scores/softmax/sums from bfloat16 caches; the oracle goes
  further and works in float64 throughout.

* Step (``step``): append, then attend over ``lengths[b] + 1`` slots, i.e.
  over every cached position plus the new token (KV-cache decode step page,
  problem statement: the new token's own position takes part in the
  softmax).

The attention here is the plain definition written out -- no tiling, no online
softmax, no split of the token axis.  The maximum score is subtracted before
exponentiating; that is an exact identity of the softmax (numerator and
denominator share the factor), done only so float64 does not overflow on
large logits.

Storage conventions (the caller's raw buffers, as NumPy arrays):

* ``"f32"`` data is a ``float32`` array; ``"bf16"`` data is a ``uint16`` array
  holding the bfloat16 bit patterns (the upper half of a float32).
* Layout ``"BHSD"`` is (B, Hkv, S, D) -- the KV-cache decode step page's cache
  shape; layout ``"BSHD"`` is (B, S, Hkv, D) -- the JAX page's cache shape.

Readings of points the pages leave open (each listed with its justification in
the design notes of the repository):

* scale is ``1/sqrt(D)`` (JAX page formula and its first example's 1/sqrt(2));
* grouping is contiguous: query head ``h`` uses kv-head ``h // G``;
* ``lengths`` for append/step is the pre-append count, for attend the valid
  count that already includes the new token;
* an attend row with zero valid slots produces zeros (outside both pages'
  constraints, which require at least one valid slot).
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode",
    "kv_index",
    "append",
    "attend",
    "attend_one",
    "softmax_weights",
    "step",
    "kv_rows",
]

DTYPES = ("f32", "bf16")
LAYOUTS = ("BHSD", "BSHD")


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.

    bfloat16 is the upper 16 bits of an IEEE binary32, so widening the bit
    pattern by 16 zero bits gives the float32 of equal value; float32 -> float64
    is exact.
    """
    if dtype == "f32":
        if x.dtype != np.float32:
            raise TypeError("f32 data must be a float32 array")
        return x.astype(np.float64)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 data must be a uint16 array of bit patterns")
        wide = x.astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):      # NaN patterns stay NaN
            return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _check_layout(layout: str) -> None:
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")


def _cache_dims(cache: np.ndarray, layout: str):
    """Return (B, Hkv, S, D) of a cache array in the given layout."""
    _check_layout(layout)
    if cache.ndim != 4:
        raise ValueError("a cache is 4-D")
    if layout == "BHSD":
        B, Hkv, S, D = cache.shape
    else:
        B, S, Hkv, D = cache.shape
    return B, Hkv, S, D


def kv_index(layout: str, b: int, h: int, j: int):
    """Index tuple of slot ``j`` of kv-head ``h`` of sequence ``b``."""
    _check_layout(layout)
    return (b, h, j) if layout == "BHSD" else (b, j, h)


def kv_rows(cache: np.ndarray, layout: str, b: int, h: int, n: int) -> np.ndarray:
    """The first ``n`` slots of kv-head ``h`` of sequence ``b``, shape (n, D).

    Only these rows are read; slots ``>= n`` are never touched, so whatever
    they hold cannot reach the result.
    """
    _check_layout(layout)
    if layout == "BHSD":
        return cache[b, h, :n, :]
    return cache[b, :n, h, :]


def append(k_cache, v_cache, k_new, v_new, lengths, layout: str):
    """Expected caches after the in-place append.

    ``k_cache``/``v_cache``: raw caches (float32 or uint16 bf16 bits) in
    ``layout``.  ``k_new``/``v_new``: (B, Hkv, D), same storage type.
    ``lengths``: int32 (B,), pre-append token counts, each in [0, S).
    Returns new arrays; the inputs are not modified.  Every byte outside slot
    ``lengths[b]`` of each (b, h) is the input's byte.
    """
    B, Hkv, S, D = _cache_dims(k_cache, layout)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache differ in shape")
    if k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D):
        raise ValueError("k_new/v_new must be (B, Hkv, D)")
    if k_new.dtype != k_cache.dtype or v_new.dtype != v_cache.dtype:
        raise TypeError("new K/V must have the caches' storage type")
    lengths = np.asarray(lengths)
    if lengths.shape != (B,):
        raise ValueError("lengths must be (B,)")
    k_out = k_cache.copy()
    v_out = v_cache.copy()
    for b in range(B):
        pos = int(lengths[b])
        if not 0 <= pos < S:
            raise ValueError(f"lengths[{b}]={pos} leaves no free slot in capacity {S}")
        for h in range(Hkv):
            idx = kv_index(layout, b, h, pos)
            k_out[idx] = k_new[b, h]
            v_out[idx] = v_new[b, h]
    return k_out, v_out


def softmax_weights(q_row: np.ndarray, k_rows: np.ndarray):
    """Scores and softmax weights of one query head over ``n`` valid slots.

    ``q_row`` is (D,) and ``k_rows`` is (n, D), float64.  Returns
    ``(s, w)`` with s_j = q.K_j / sqrt(D) and w_j = exp(s_j) / sum_m exp(s_m)
    (JAX "Grouped-Query Decode Step" page, problem statement formulas).
    """
    n, D = k_rows.shape
    if q_row.shape != (D,):
        raise ValueError("shape mismatch")
    scores = (k_rows @ q_row) / math.sqrt(D)          # s_j, j < n
    if n == 0:
        return scores, scores.copy()
    e = np.exp(scores - scores.max())                 # exact softmax identity
    return scores, e / e.sum()                        # w_j


def attend_one(q_row: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
    """Output of one query head over ``n`` valid slots, float64 in and out.

    ``q_row`` is (D,); ``k_rows``/``v_rows`` are (n, D) holding exactly the
    valid slots.  Implements o = sum_j w_j V_j with the weights above.
    """
    n, D = k_rows.shape
    if v_rows.shape != (n, D):
        raise ValueError("shape mismatch")
    if n == 0:
        return np.zeros(D, dtype=np.float64)
    _, w = softmax_weights(q_row, k_rows)
    return w @ v_rows                                 # o = sum_j w_j V_j


def attend(q, q_dtype: str, k_cache, v_cache, kv_dtype: str, lengths, layout: str,
           num_q_heads: int, num_kv_heads: int) -> np.ndarray:
    """Length-masked GQA attention, float64 (B, Hq, D).

    ``q`` is (B, Hq, D) in ``q_dtype`` storage; the caches are in ``kv_dtype``
    storage and ``layout``; ``lengths[b]`` is the number of valid slots of
    sequence ``b`` (the new token already among them), each in [0, S].
    """
    B, Hkv, S, D = _cache_dims(k_cache, layout)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache differ in shape")
    Hq = num_q_heads
    if num_kv_heads != Hkv or Hq < 1 or Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("head counts must satisfy Hq % Hkv == 0 and match the cache")
    if q.shape != (B, Hq, D):
        raise ValueError("q must be (B, Hq, D)")
    G = Hq // Hkv
    lengths = np.asarray(lengths)
    if lengths.shape != (B,):
        raise ValueError("lengths must be (B,)")
    qf = decode(q, q_dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        n = int(lengths[b])
        if not 0 <= n <= S:
            raise ValueError(f"lengths[{b}]={n} outside [0, {S}]")
        for h in range(Hkv):
            K = decode(kv_rows(k_cache, layout, b, h, n), kv_dtype)
            V = decode(kv_rows(v_cache, layout, b, h, n), kv_dtype)
            for hq in range(h * G, (h + 1) * G):       # the heads with hq // G == h
                out[b, hq] = attend_one(qf[b, hq], K, V)
    return out


def step(q, q_dtype: str, k_cache, v_cache, k_new, v_new, kv_dtype: str, lengths,
         layout: str, num_q_heads: int, num_kv_heads: int):
    """Append at ``lengths[b]``, then attend over ``lengths[b] + 1`` slots.

    Returns ``(out, k_cache_after, v_cache_after)``.
    """
    k_out, v_out = append(k_cache, v_cache, k_new, v_new, lengths, layout)
    n_valid = np.asarray(lengths).astype(np.int64) + 1
    out = attend(q, q_dtype, k_out, v_out, kv_dtype, n_valid, layout, num_q_heads, num_kv_heads)
    return out, k_out, v_out

"""Float64 CPU oracle for the decode step on int8 caches with per-row scales.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.oracle``).

Source of the quantization rule: Huawei CANN, "aclnnMlaPrologV3WeightNz"
operator page, the dynamic-quantization formula of its fifth path -- a row's
dequantization scale is its largest absolute value divided by 127, and the
stored code is the row divided by that scale, rounded.  Here the rule is
applied to every key and value row a step appends (one row = one slot of one
kv-head, D elements): the cache stores the int8 codes and a float32 scale per
row, and reads use ``value = code * scale``.

Readings (listed with their reasons in the repository's design notes):

* "round" is round-half-to-even;
* fp8 caches (a format the pages do not define; see ``oracle.fp8``) follow the
  same rule with the format's largest finite value in place of 127:
  ``scale = float32(max |x|) / 448``, ``code = encode(clamp(x / scale, -448,
  448))`` with a correctly rounded float32 division, the code the nearest
  E4M3 value (ties to even); a row of zeros has scale 0 and codes 0;
* the code is a decision float arithmetic takes, so it is taken in the
  kernel's precision: the new key/value (stored as ``new_dtype``) is widened
  to float32, ``scale = float32(max |x|) / 127`` and ``code = rne(x / scale)``
  with correctly rounded float32 divisions, codes clamped to [-127, 127]; a row
  of zeros has scale 0 and codes 0;
* attention then runs exactly as in ``oracle.oracle`` on the dequantized rows,
  in float64 (``code * scale`` is exact in float64).

Storage: caches are int8 arrays (int8 codes) or uint8 arrays (fp8 codes, as
bit patterns) in the dense layouts ("BHSD" (B, Hkv, S, D), "BSHD" (B, S, Hkv,
D)); the array's dtype selects the format.  Scales are float32 arrays of the
same layout without the last axis ((B, Hkv, S) or (B, S, Hkv)).
"""

from __future__ import annotations

import numpy as np

from .fp8 import E4M3_MAX, decode_e4m3, encode_e4m3
from .oracle import attend_one, decode, kv_index

__all__ = ["quantize_row", "dequantize", "append_q8", "attend_q8", "step_q8"]

CODE_DTYPES = {"i8": np.int8, "fp8": np.uint8}


def quantize_row(x32: np.ndarray, fmt: str = "i8"):
    """float32 row -> (codes, float32 scale) by the rule above; ``fmt`` "i8"
    gives int8 codes, "fp8" uint8 E4M3 codes."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax == 0 or not np.isfinite(amax):
        if amax == 0:
            return np.zeros(x32.shape, CODE_DTYPES[fmt]), np.float32(0)
        raise ValueError("non-finite row")
    if fmt == "fp8":
        scale = np.float32(amax / np.float32(E4M3_MAX))   # float32 division, correctly rounded
        q = np.clip(x32 / scale, -E4M3_MAX, E4M3_MAX)     # float32 division, then clamped
        return encode_e4m3(q), scale
    if fmt != "i8":
        raise ValueError(f"unknown code format {fmt!r}")
    scale = np.float32(amax / np.float32(127))            # float32 division, correctly rounded
    q = np.rint(x32 / scale).astype(np.float32)           # float32 division, then half-to-even
    return np.clip(q, -127, 127).astype(np.int8), scale


def code_format(codes: np.ndarray) -> str:
    """The code format of a cache array: int8 -> "i8", uint8 -> "fp8"."""
    for fmt, dt in CODE_DTYPES.items():
        if codes.dtype == dt:
            return fmt
    raise TypeError("codes are int8 (int8 codes) or uint8 (fp8 bit patterns)")


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes (..., D) (int8, or uint8 fp8 patterns) and scales (...) float32 ->
    float64 values ``code * scale`` (exact)."""
    vals = decode_e4m3(codes) if code_format(codes) == "fp8" else codes.astype(np.float64)
    return vals * scales.astype(np.float64)[..., None]


def _dims(cache, layout):
    if cache.ndim != 4:
        raise TypeError("a quantized cache is a 4-D array")
    code_format(cache)
    if layout == "BHSD":
        B, Hkv, S, D = cache.shape
    elif layout == "BSHD":
        B, S, Hkv, D = cache.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return B, Hkv, S, D


def append_q8(k_cache, v_cache, k_scale, v_scale, k_new, v_new, new_dtype: str, lengths, layout: str):
    """Quantize the new key/value rows and store them at slot ``lengths[b]``.

    Returns new (k_cache, v_cache, k_scale, v_scale); every other byte is kept."""
    B, Hkv, S, D = _dims(k_cache, layout)
    fmt = code_format(k_cache)
    if v_cache.dtype != k_cache.dtype:
        raise TypeError("k_cache and v_cache hold the same code format")
    kn = decode(k_new, new_dtype).astype(np.float32)        # exact: stored values widen to float32
    vn = decode(v_new, new_dtype).astype(np.float32)
    kc, vc, ks, vs = k_cache.copy(), v_cache.copy(), k_scale.copy(), v_scale.copy()
    for b in range(B):
        pos = int(lengths[b])
        if not 0 <= pos < S:
            raise ValueError(f"lengths[{b}]={pos} leaves no free slot in capacity {S}")
        for h in range(Hkv):
            idx = kv_index(layout, b, h, pos)
            kc[idx], ks[idx] = quantize_row(kn[b, h], fmt)
            vc[idx], vs[idx] = quantize_row(vn[b, h], fmt)
    return kc, vc, ks, vs


def attend_q8(q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, lengths, layout: str,
              num_q_heads: int, num_kv_heads: int) -> np.ndarray:
    """Length-masked GQA attention over dequantized rows, float64 (B, Hq, D)."""
    B, Hkv, S, D = _dims(k_cache, layout)
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
            if layout == "BHSD":
                K = dequantize(k_cache[b, h, :n], k_scale[b, h, :n])
                V = dequantize(v_cache[b, h, :n], v_scale[b, h, :n])
            else:
                K = dequantize(k_cache[b, :n, h], k_scale[b, :n, h])
                V = dequantize(v_cache[b, :n, h], v_scale[b, :n, h])
            for hq in range(h * G, (h + 1) * G):
                out[b, hq] = attend_one(qf[b, hq], K, V)
    return out


def step_q8(q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, k_new, v_new, lengths, layout: str,
            num_q_heads: int, num_kv_heads: int):
    """Quantizing append at ``lengths[b]`` (new K/V stored as ``q_dtype``), then
    attend over ``lengths[b] + 1`` slots.  Returns (out, k_cache, v_cache,
    k_scale, v_scale) after the step."""
    kc, vc, ks, vs = append_q8(k_cache, v_cache, k_scale, v_scale, k_new, v_new, q_dtype, lengths, layout)
    n = np.asarray(lengths).astype(np.int64) + 1
    out = attend_q8(q, q_dtype, kc, vc, ks, vs, n, layout, num_q_heads, num_kv_heads)
    return out, kc, vc, ks, vs

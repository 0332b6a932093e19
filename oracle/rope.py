"""CPU oracle for the decode step with rotary position encoding applied to the
new key and the query before the append -- TEST INFRASTRUCTURE ONLY (same rule
as ``oracle.oracle``).

Source: CLIKA runtime, "groupQueryAttention" API page (operator summary): the
operator rotates q and the new k with the rope planes ``rope_cos`` /
``rope_sin`` and appends the post-rotation key (and the value) in place into
the cache; when per-head gains are given, every head's rotated q and new-k
vector is then RMS-normalized with the gain (epsilon inside the square root,
as in the RmsNorm formula of the Huawei CANN "aclnnMlaPrologV3WeightNz" page)
before the append, so the cache holds rotated (and normalized) keys.  The
CANN page applies the same rotation to its query and key ("ROPE").

Readings (listed with their reasons in the repository's design notes):

* Tables: ``cos`` and ``sin`` are float32 arrays of shape (max_pos, D / 2);
  row p holds the angles of position p, column i the i-th rotation pair.
* Pairs: mode ``"half"`` rotates elements (i, i + D/2); mode ``"interleaved"``
  rotates (2i, 2i + 1).  For a pair (x1, x2) at position p:
  ``y1 = x1 cos - x2 sin`` and ``y2 = x2 cos + x1 sin`` -- the rotation of the
  complex number x1 + i x2 by the table's angle.
* Position of the new token: ``positions[b]`` when given, else its cache slot
  ``lengths[b]``; the query takes the same position (it is the new token's).
* Precision of the rotation: the stored key is a rounding of the rotated value,
  a decision taken in the kernel's precision -- float32, each product and sum
  rounded separately in the order written above (no fused multiply-add); the
  rotated key is then rounded to the cache's storage type (round to nearest
  even).  The query is used unrounded.
* Norm (optional): ``y = x / sqrt(mean(x^2) + eps) * gain`` over the head
  width, in float64 on the float32 rotation result; the normalized key is
  then rounded to the cache's storage type.  Gains are float32 (D,).
* The value is appended unchanged; attention is the plain definition of
  ``oracle.oracle`` over the appended cache (float64).
"""

from __future__ import annotations

import numpy as np

from .mapped import append_mapped, mapped_rows
from .oracle import append, attend_one, decode, kv_rows
from .quant import step_q8

__all__ = ["rope_rotate", "rms_norm", "encode", "rotate_new", "step_rope", "step_q8_rope"]

MODES = ("half", "interleaved")


def _pairs(D: int, mode: str):
    if D % 2:
        raise ValueError("rotary encoding needs an even head width")
    h = D // 2
    i = np.arange(h)
    if mode == "half":
        return i, i + h
    if mode == "interleaved":
        return 2 * i, 2 * i + 1
    raise ValueError(f"unknown mode {mode!r}")


def rope_rotate(x32, cos_row, sin_row, mode: str) -> np.ndarray:
    """Rotate one float32 vector (D,) with one table row (D/2,), in float32
    with each product and sum rounded separately."""
    x = np.asarray(x32, dtype=np.float32)
    c = np.asarray(cos_row, dtype=np.float32)
    s = np.asarray(sin_row, dtype=np.float32)
    i1, i2 = _pairs(x.shape[-1], mode)
    if c.shape[-1] != i1.size or s.shape[-1] != i1.size:
        raise ValueError("a table row holds D / 2 angles")
    x1, x2 = x[..., i1], x[..., i2]
    y = np.empty_like(x)
    y[..., i1] = (x1 * c) - (x2 * s)       # float32 operations, no fusion
    y[..., i2] = (x2 * c) + (x1 * s)
    return y


def rms_norm(x, gain, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gain over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gain, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def encode(x, dtype: str) -> np.ndarray:
    """Values -> storage: float32 (round to nearest even), or bf16 bit patterns
    rounded to nearest even from the float32 value."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        bits = f.view(np.uint32).astype(np.uint64)
        nan = np.isnan(f)
        r = ((bits + 0x7FFF + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
        r[nan] = ((bits[nan] >> 16) | 0x40).astype(np.uint16)
        return r
    raise ValueError(f"unknown dtype {dtype!r}")


def _check_tables(cos, sin, D):
    cos = np.asarray(cos)
    sin = np.asarray(sin)
    if cos.dtype != np.float32 or sin.dtype != np.float32 or cos.shape != sin.shape or cos.ndim != 2 \
            or cos.shape[1] != D // 2:
        raise ValueError("cos / sin are float32 tables of shape (max_pos, D / 2)")
    return cos, sin


def rotate_new(q, q_dtype: str, k_new, kv_dtype: str, pos, cos, sin, mode: str,
               q_gain=None, k_gain=None, eps=None):
    """The rotated (and normalized) query, float64 (B, Hq, D), and the stored
    new key in ``kv_dtype`` storage (B, Hkv, D)."""
    B, Hq, D = q.shape
    cos, sin = _check_tables(cos, sin, D)
    if (q_gain is not None or k_gain is not None) != (eps is not None):
        raise ValueError("the norm gains travel with an epsilon, and an epsilon with a gain")
    pos = np.asarray(pos)
    if pos.shape != (B,) or np.any(pos < 0) or np.any(pos >= cos.shape[0]):
        raise ValueError("positions index the tables")
    q32 = decode(q, q_dtype).astype(np.float32)          # exact: stored values widen to float32
    k32 = decode(k_new, kv_dtype).astype(np.float32)
    qr = np.empty(q.shape, np.float64)
    kr = np.empty(k_new.shape, k32.dtype if kv_dtype == "f32" else np.uint16)
    for b in range(B):
        p = int(pos[b])
        qb = rope_rotate(q32[b], cos[p], sin[p], mode).astype(np.float64)
        kb = rope_rotate(k32[b], cos[p], sin[p], mode).astype(np.float64)
        if q_gain is not None:
            qb = rms_norm(qb, q_gain, eps)
        if k_gain is not None:
            kb = rms_norm(kb, k_gain, eps)
        qr[b] = qb
        kr[b] = encode(kb, kv_dtype)
    return qr, kr


def step_rope(q, q_dtype: str, k_cache, v_cache, k_new, v_new, kv_dtype: str, lengths, layout: str,
              num_q_heads: int, num_kv_heads: int, cos, sin, mode: str, positions=None, q_gain=None,
              k_gain=None, eps=None, kind: str | None = None, mapping=None, bs=None):
    """Rotate (and normalize) q and the new key at the new token's position,
    append the stored key and the value at slot ``lengths[b]`` (dense caches,
    or ``kind`` "slots" / "paged" with ``mapping`` as in ``oracle.mapped``),
    then attend over ``lengths[b] + 1`` slots.

    Returns (out float64 (B, Hq, D), k_cache_after, v_cache_after)."""
    lengths = np.asarray(lengths)
    pos = lengths if positions is None else np.asarray(positions)
    qr, kr = rotate_new(q, q_dtype, k_new, kv_dtype, pos, cos, sin, mode, q_gain, k_gain, eps)
    if kind is None:
        kc, vc = append(k_cache, v_cache, kr, v_new, lengths, layout)
    else:
        kc, vc = append_mapped(kind, k_cache, v_cache, kr, v_new, lengths, layout, mapping, bs)
    B, Hq, D = q.shape
    Hkv = num_kv_heads
    if Hq != num_q_heads or Hq % Hkv:
        raise ValueError("head counts")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        n = int(lengths[b]) + 1
        for h in range(Hkv):
            if kind is None:
                Kr, Vr = kv_rows(kc, layout, b, h, n), kv_rows(vc, layout, b, h, n)
            else:
                Kr = mapped_rows(kc, kind, layout, mapping, b, h, n, bs)
                Vr = mapped_rows(vc, kind, layout, mapping, b, h, n, bs)
            K, V = decode(Kr, kv_dtype), decode(Vr, kv_dtype)
            for hq in range(h * G, (h + 1) * G):
                out[b, hq] = attend_one(qr[b, hq], K, V)
    return out, kc, vc


def step_q8_rope(q, q_dtype: str, k_cache, v_cache, k_scale, v_scale, k_new, v_new, lengths, layout: str,
                 num_q_heads: int, num_kv_heads: int, cos, sin, mode: str, positions=None):
    """Int8 caches (``oracle.quant``): the new key is rotated in float32 as above
    and then quantized by the per-row rule; q is rotated the same way and used
    unrounded.  Returns (out, k_cache, v_cache, k_scale, v_scale) after the step."""
    B, Hq, D = q.shape
    cos, sin = _check_tables(cos, sin, D)
    lengths = np.asarray(lengths)
    pos = lengths if positions is None else np.asarray(positions)
    if pos.shape != (B,) or np.any(pos < 0) or np.any(pos >= cos.shape[0]):
        raise ValueError("positions index the tables")
    q32 = decode(q, q_dtype).astype(np.float32)
    k32 = decode(k_new, q_dtype).astype(np.float32)
    qr = np.empty_like(q32)
    kr = np.empty_like(k32)
    for b in range(B):
        p = int(pos[b])
        qr[b] = rope_rotate(q32[b], cos[p], sin[p], mode)
        kr[b] = rope_rotate(k32[b], cos[p], sin[p], mode)
    vn = decode(v_new, q_dtype).astype(np.float32)            # exact
    return step_q8(qr, "f32", k_cache, v_cache, k_scale, v_scale, kr, vn, lengths, layout, num_q_heads,
                   num_kv_heads)

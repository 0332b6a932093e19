"""Float64 CPU oracle for the softmax variants of the decode step: attention
sink, smooth softmax, score soft-capping, sliding window with a kept prefix --
TEST INFRASTRUCTURE ONLY (same rule as ``oracle.oracle``).

Source: CLIKA runtime, "groupQueryAttention" API page (operator summary and
parameter list): ``head_sink`` is a per-query-head virtual logit folded into
the softmax denominator; ``smooth_softmax``; ``softcap``; ``sliding_window``;
``kept_prefix`` keeps each sequence's first P keys attended beside the sliding
window (one value for every sequence or one per sequence; a negative P is
refused): under the causal bound a key is attended when it lies in the first P
keys or inside the window, and without a kept prefix the window alone decides.

Readings (listed with their reasons in the repository's design notes):

* The query of a decode step is the newest token, at position n - 1 where n
  is the number of valid slots (lengths[b] + 1 for a step).  A window of W
  keeps the keys j with (n - 1) - j < W, i.e. the last W slots, the query's
  own key included; W >= n keeps everything.  The kept prefix adds the keys
  j < P.  Attended set: {j < n : j < P or j >= n - W}.
* Soft-capping applies to the scaled score: s = q.k / sqrt(D) becomes
  cap * tanh(s / cap), before the softmax (cap > 0).
* The sink is a logit in the same units as the (capped) scores, not capped
  itself, with no value row: w_j = exp(s_j) / (sum_i exp(s_i) + exp(sink)).
  Smooth softmax is the same with a zero logit for every head; the two are
  not combined.
* No attended key (n = 0) gives zeros.
"""

from __future__ import annotations

import math

import numpy as np

from .mapped import append_mapped, mapped_rows
from .oracle import append, decode, kv_rows
from .quant import append_q8, dequantize

__all__ = ["attended_slots", "attend_variant_one", "attend_variants", "step_variants"]


def attended_slots(n: int, window: int = 0, prefix: int = 0) -> np.ndarray:
    """Indices of the attended keys among n valid slots."""
    if prefix < 0 or window < 0:
        raise ValueError("window and kept prefix are >= 0")
    j = np.arange(n)
    if window == 0:
        return j
    return j[(j < prefix) | (j >= n - window)]


def attend_variant_one(q_row, k_rows, v_rows, sink=None, softcap: float = 0.0) -> np.ndarray:
    """One query head over the attended rows (float64 (D,))."""
    q = np.asarray(q_row, np.float64)
    K = np.asarray(k_rows, np.float64)
    V = np.asarray(v_rows, np.float64)
    D = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros(D)
    s = K @ q / math.sqrt(D)
    if softcap > 0:
        s = softcap * np.tanh(s / softcap)
    logits = s if sink is None else np.append(s, float(sink))
    m = np.max(logits)
    e = np.exp(logits - m)
    den = np.sum(e)
    return (e[: K.shape[0]] / den) @ V


def _sink_of(sink, smooth, hq):
    if sink is not None and smooth:
        raise ValueError("a sink and smooth softmax are not combined")
    if smooth:
        return 0.0
    return None if sink is None else float(sink[hq])


def _scale_rows(scale, layout, b, h, n):
    return scale[b, h, :n] if layout == "BHSD" else scale[b, :n, h]


def attend_variants(q, q_dtype: str, k_cache, v_cache, kv_dtype: str, lengths, layout: str, num_q_heads: int,
                    num_kv_heads: int, sink=None, smooth: bool = False, softcap: float = 0.0, window: int = 0,
                    prefix=0, kind: str | None = None, mapping=None, bs=None, scales=None) -> np.ndarray:
    """Length-masked GQA attention with the variants, float64 (B, Hq, D).
    ``prefix`` is one value or one per sequence; ``kind``/``mapping``/``bs``
    select a mapped cache as in ``oracle.mapped``; ``kv_dtype`` "i8" (or "fp8") takes
    int8 caches read as code * row scale with ``scales = (k_scale, v_scale)``
    (``oracle.quant`` storage)."""
    B, Hq, D = q.shape
    Hkv = num_kv_heads
    if Hq != num_q_heads or Hq % Hkv:
        raise ValueError("head counts")
    G = Hq // Hkv
    pre = np.broadcast_to(np.asarray(prefix), (B,))
    if np.any(pre < 0):
        raise ValueError("a negative kept prefix is refused")
    qf = decode(q, q_dtype)
    out = np.zeros((B, Hq, D), np.float64)
    for b in range(B):
        n = int(lengths[b])
        idx = attended_slots(n, window, int(pre[b]))
        for h in range(Hkv):
            if kind is None:
                Kr, Vr = kv_rows(k_cache, layout, b, h, n), kv_rows(v_cache, layout, b, h, n)
            else:
                Kr = mapped_rows(k_cache, kind, layout, mapping, b, h, n, bs)
                Vr = mapped_rows(v_cache, kind, layout, mapping, b, h, n, bs)
            if kv_dtype in ("i8", "fp8"):
                K = dequantize(Kr, _scale_rows(scales[0], layout, b, h, n))[idx]
                V = dequantize(Vr, _scale_rows(scales[1], layout, b, h, n))[idx]
            else:
                K, V = decode(Kr, kv_dtype)[idx], decode(Vr, kv_dtype)[idx]
            for hq in range(h * G, (h + 1) * G):
                out[b, hq] = attend_variant_one(qf[b, hq], K, V, _sink_of(sink, smooth, hq), softcap)
    return out


def step_variants(q, q_dtype: str, k_cache, v_cache, k_new, v_new, kv_dtype: str, lengths, layout: str,
                  num_q_heads: int, num_kv_heads: int, kind: str | None = None, mapping=None, bs=None, scales=None,
                  **variants):
    """Append at ``lengths[b]``, then attend with the variants over
    ``lengths[b] + 1`` slots.  Returns (out, k_cache_after, v_cache_after);
    int8 or fp8 caches ("i8" / "fp8", new rows in ``q_dtype``, ``scales = (k_scale, v_scale)``)
    return (out, k_cache, v_cache, k_scale, v_scale)."""
    if kv_dtype in ("i8", "fp8"):
        kc, vc, ks, vs = append_q8(k_cache, v_cache, scales[0], scales[1], k_new, v_new, q_dtype, lengths, layout)
        n = np.asarray(lengths).astype(np.int64) + 1
        out = attend_variants(q, q_dtype, kc, vc, kv_dtype, n, layout, num_q_heads, num_kv_heads, scales=(ks, vs),
                              **variants)
        return out, kc, vc, ks, vs
    if kind is None:
        kc, vc = append(k_cache, v_cache, k_new, v_new, lengths, layout)
    else:
        kc, vc = append_mapped(kind, k_cache, v_cache, k_new, v_new, lengths, layout, mapping, bs)
    n = np.asarray(lengths).astype(np.int64) + 1
    out = attend_variants(q, q_dtype, kc, vc, kv_dtype, n, layout, num_q_heads, num_kv_heads, kind=kind,
                          mapping=mapping, bs=bs, **variants)
    return out, kc, vc

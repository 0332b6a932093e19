"""Pins for the softmax-variant oracle (CLIKA runtime "groupQueryAttention"
API page: head sink, smooth softmax, softcap, sliding window, kept prefix).

Pins come from the mathematics and an independent library routine, not from
the oracle's own formula: reductions to the plain oracle (window covering all
slots, an infinitely negative sink, an unbounded cap), closed forms (a
one-slot window returns that value row; equal scores give a uniform average
diluted by the sink exactly as n / (n + e^(sink - s)); saturated caps make
unequal scores equal), the attended index sets written out by hand, and
scipy's softmax over an explicit -inf mask.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import variants as V


def rand_case(seed, B=3, Hq=4, Hkv=2, D=8, S=20):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    return q, kc, vc


def test_attended_sets_by_hand():
    assert V.attended_slots(10).tolist() == list(range(10))
    assert V.attended_slots(10, window=3).tolist() == [7, 8, 9]
    assert V.attended_slots(10, window=3, prefix=2).tolist() == [0, 1, 7, 8, 9]
    assert V.attended_slots(10, window=8, prefix=4).tolist() == list(range(10))      # overlap
    assert V.attended_slots(10, window=20).tolist() == list(range(10))
    assert V.attended_slots(10, window=1).tolist() == [9]
    assert V.attended_slots(0, window=3, prefix=2).tolist() == []
    with pytest.raises(ValueError):
        V.attended_slots(5, window=2, prefix=-1)


def test_reductions_to_the_plain_oracle():
    q, kc, vc = rand_case(1)
    L = np.array([20, 7, 1])
    ref = oracle.attend(q, "f32", kc, vc, "f32", L, "BHSD", 4, 2)
    for kw in (dict(), dict(window=20), dict(window=5, prefix=20), dict(sink=np.full(4, -np.inf)),
               dict(softcap=1e12)):
        got = V.attend_variants(q, "f32", kc, vc, "f32", L, "BHSD", 4, 2, **kw)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), kw


def test_one_slot_window_returns_the_last_value_row():
    q, kc, vc = rand_case(2)
    L = np.array([20, 9, 3])
    got = V.attend_variants(q, "f32", kc, vc, "f32", L, "BHSD", 4, 2, window=1)
    for b in range(3):
        for hq in range(4):
            assert np.array_equal(got[b, hq], vc[b, hq // 2, L[b] - 1].astype(np.float64))


def test_sink_dilutes_equal_scores_by_a_closed_form():
    """All keys equal -> every score is s; with a sink logit t the weights are
    e^s / (n e^s + e^t) each, so out = mean(V) * n / (n + e^(t - s))."""
    rng = np.random.default_rng(3)
    D, n = 4, 6
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    K = np.tile(k, (n, 1))
    Vv = rng.standard_normal((n, D))
    s = q @ k / 2.0
    for t in (-3.0, 0.0, 2.5):
        got = V.attend_variant_one(q, K, Vv, sink=t)
        assert np.allclose(got, Vv.mean(0) * n / (n + np.exp(t - s)), rtol=1e-13)
    # smooth softmax = a zero sink for every head
    qs = q.astype(np.float32)[None, None]
    Kc = K.astype(np.float32)[None, None]
    Vc = Vv.astype(np.float32)[None, None]
    a = V.attend_variants(qs, "f32", Kc, Vc, "f32", [n], "BHSD", 1, 1, smooth=True)
    b = V.attend_variants(qs, "f32", Kc, Vc, "f32", [n], "BHSD", 1, 1, sink=np.zeros(1))
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        V.attend_variants(qs, "f32", Kc, Vc, "f32", [n], "BHSD", 1, 1, smooth=True, sink=np.zeros(1))


def test_saturated_cap_equalizes_large_scores():
    """Two keys with scaled scores 1000 and 2000 under cap 1: both capped
    scores are 1 to double precision, so the weights are 1/2 each."""
    D = 4
    q = np.array([1.0, 0, 0, 0])
    K = np.array([[2000.0, 0, 0, 0], [4000.0, 0, 0, 0]])           # / sqrt(4) = 1000, 2000
    Vv = np.array([[1.0, 2, 3, 4], [5.0, 6, 7, 8]])
    assert np.allclose(V.attend_variant_one(q, K, Vv, softcap=1.0), Vv.mean(0), rtol=1e-15)
    # moderate cap: c tanh(s / c) written out for two keys
    K2 = np.array([[1.0, 0, 0, 0], [3.0, 0, 0, 0]])
    c = 0.7
    s = np.array([0.5, 1.5])
    w = np.exp(c * np.tanh(s / c))
    assert np.allclose(V.attend_variant_one(q, K2, Vv, softcap=c), (w / w.sum()) @ Vv, rtol=1e-14)


def test_against_scipy_softmax_over_a_masked_row():
    """Window + prefix + sink + cap together against scipy's softmax over the
    full row with -inf at the unattended slots and the sink appended."""
    q, kc, vc = rand_case(4, B=2, Hq=6, Hkv=3, D=16, S=40)
    L = np.array([40, 23])
    sink = np.array([0.3, -1.0, 2.0, 0.0, 1.5, -0.2])
    pre = np.array([3, 5])
    got = V.attend_variants(q, "f32", kc, vc, "f32", L, "BHSD", 6, 3, sink=sink, softcap=2.0, window=9, prefix=pre)
    for b in range(2):
        n = L[b]
        j = np.arange(n)
        keep = (j < pre[b]) | (j >= n - 9)
        for hq in range(6):
            h = hq // 2
            K = kc[b, h, :n].astype(np.float64)
            s = K @ q[b, hq].astype(np.float64) / 4.0
            s = 2.0 * np.tanh(s / 2.0)
            s = np.where(keep, s, -np.inf)
            w = softmax(np.append(s, sink[hq]))[:n]
            assert np.allclose(got[b, hq], w @ vc[b, h, :n].astype(np.float64), rtol=1e-12, atol=1e-14)


def test_step_appends_then_windows_over_the_new_token():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, S = 2, 4, 1, 8, 12
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    L = np.array([11, 4], np.int32)
    out, rk, rv = V.step_variants(q, "f32", kc, vc, kn, vn, "f32", L, "BHSD", Hq, Hkv, window=1)
    for b in range(B):
        assert np.array_equal(out[b], np.repeat(vn[b].astype(np.float64), Hq, axis=0))
    ref, ek, ev = oracle.step(q, "f32", kc, vc, kn, vn, "f32", L, "BHSD", Hq, Hkv)
    assert rk.tobytes() == ek.tobytes() and rv.tobytes() == ev.tobytes()


def test_int8_variants_reduce_to_the_int8_oracle():
    rng = np.random.default_rng(6)
    B, Hq, Hkv, D, S = 2, 4, 2, 8, 9
    q = (rng.standard_normal((B, Hq, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kc = rng.integers(-127, 128, (B, Hkv, S, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, S, D)).astype(np.int8)
    ks = rng.uniform(0.01, 0.03, (B, Hkv, S)).astype(np.float32)
    vs = rng.uniform(0.01, 0.03, (B, Hkv, S)).astype(np.float32)
    kn = (rng.standard_normal((B, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vn = (rng.standard_normal((B, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    L = np.array([3, 8], np.int32)
    got = V.step_variants(q, "bf16", kc, vc, kn, vn, "i8", L, "BHSD", Hq, Hkv, scales=(ks, vs), window=S)
    ref = oracle.step_q8(q, "bf16", kc, vc, ks, vs, kn, vn, L, "BHSD", Hq, Hkv)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-13, atol=1e-15) if a.dtype == np.float64 else np.array_equal(a, b)
    w1 = V.step_variants(q, "bf16", kc, vc, kn, vn, "i8", L, "BHSD", Hq, Hkv, scales=(ks, vs), window=1)[0]
    for b in range(B):
        row = oracle.dequantize(ref[2][b, :, L[b]], ref[4][b, :, L[b]])       # the appended value rows
        assert np.allclose(w1[b], np.repeat(row, Hq // Hkv, axis=0), rtol=1e-13)

"""Pins for the int8 (per-row scale) oracle.

The rule (CANN "aclnnMlaPrologV3WeightNz" page, dynamic-quantization formula):
scale = max|x| / 127, code = round(x / scale).  Pinned by hand-derived codes
on rows whose scale is a power of two (so every quotient is exact and the
rounding is visible: half-to-even, not half-away), the zero row, the error
bound |x - code * scale| <= scale / 2, and a reduction to the dense oracle on
caches whose dequantized values are exact in float32.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("row,scale,codes", [
    ([254.0, 1.0, 3.0, -5.0], 2.0, [127, 0, 2, -2]),         # 0.5 -> 0, 1.5 -> 2, -2.5 -> -2
    ([-127.0, 63.5, 0.5, -0.5], 1.0, [-127, 64, 0, 0]),       # 63.5 -> 64 (even), 0.5 -> 0
    ([31.75, 0.125, -0.375], 0.25, [127, 0, -2]),             # 0.5 -> 0, -1.5 -> -2
])
def test_quantize_closed_forms(row, scale, codes):
    q, s = oracle.quantize_row(np.array(row, np.float32))
    assert s == np.float32(scale)
    assert q.dtype == np.int8 and q.tolist() == codes


def test_zero_row():
    q, s = oracle.quantize_row(np.zeros(8, np.float32))
    assert s == 0 and not q.any()


def test_error_bound_and_full_range():
    rng = np.random.default_rng(3)
    for _ in range(200):
        x = (rng.standard_normal(64) * rng.uniform(0.01, 100)).astype(np.float32)
        q, s = oracle.quantize_row(x)
        deq = q.astype(np.float64) * np.float64(s)
        assert np.all(np.abs(x - deq) <= np.float64(s) * (0.5 + 1e-6))
        assert np.abs(q).max() == 127                         # the largest element maps to +-127


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_attend_reduces_to_dense_on_exact_values(layout):
    """Scales that are powers of two make code * scale exact in float32: the
    int8 oracle then equals the dense oracle on those float32 values."""
    rng = np.random.default_rng(8)
    B, Hq, Hkv, S, D = 2, 6, 2, 9, 16
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    kc = rng.integers(-127, 128, shape).astype(np.int8)
    vc = rng.integers(-127, 128, shape).astype(np.int8)
    ks = (2.0 ** rng.integers(-9, -3, shape[:3])).astype(np.float32)
    vs = (2.0 ** rng.integers(-9, -3, shape[:3])).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    n = np.array([9, 4])
    got = oracle.attend_q8(q, "f32", kc, vc, ks, vs, n, layout, Hq, Hkv)
    kf = (kc.astype(np.float32) * ks[..., None]).astype(np.float32)
    vf = (vc.astype(np.float32) * vs[..., None]).astype(np.float32)
    ref = oracle.attend(q, "f32", kf, vf, "f32", n, layout, Hq, Hkv)
    assert np.array_equal(got, ref)


def test_step_appends_one_row_and_ignores_stale_rows():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, S, D = 3, 4, 2, 6, 8
    kc = rng.integers(-127, 128, (B, Hkv, S, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, S, D)).astype(np.int8)
    ks = rng.uniform(0.01, 0.1, (B, Hkv, S)).astype(np.float32)
    vs = rng.uniform(0.01, 0.1, (B, Hkv, S)).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    L = np.array([0, 3, 5])
    out, kc2, vc2, ks2, vs2 = oracle.step_q8(q, "f32", kc, vc, ks, vs, kn, vn, L, "BHSD", Hq, Hkv)
    for b in range(B):
        for h in range(Hkv):
            for t in range(S):
                if t != L[b]:
                    assert kc2[b, h, t].tobytes() == kc[b, h, t].tobytes() and ks2[b, h, t] == ks[b, h, t]
                else:
                    qk, sk = oracle.quantize_row(kn[b, h])
                    assert kc2[b, h, t].tolist() == qk.tolist() and ks2[b, h, t] == sk
    # garbage in the slots past each length does not change the output
    kc3, vc3 = kc2.copy(), vc2.copy()
    ks3, vs3 = ks2.copy(), vs2.copy()
    for b in range(B):
        kc3[b, :, L[b] + 1:] = 127
        ks3[b, :, L[b] + 1:] = np.float32(1e30)
        vs3[b, :, L[b] + 1:] = np.float32(np.inf)
    out3 = oracle.attend_q8(q, "f32", kc3, vc3, ks3, vs3, L + 1, "BHSD", Hq, Hkv)
    assert np.array_equal(out3, out)
    # only the new token: the output is its dequantized value
    deq = vc2[0, :, 0].astype(np.float64) * vs2[0, :, 0, None]
    assert np.allclose(out[0], np.repeat(deq, Hq // Hkv, axis=0), rtol=0, atol=1e-12)

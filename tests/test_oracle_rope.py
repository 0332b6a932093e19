"""Pins for the rotary-encoding oracle (CLIKA runtime "groupQueryAttention" API
page: q and the new k rotated with the rope planes, optional post-rotation
per-head RMS norm with gains, the rotated key appended in place).

Each pin comes from the mathematics, not from the oracle's own formula:
hand-computed quarter turns, the complex-number form of the rotation, the
"rotate half" vector form, norm preservation, the relative-position property
of rotary encoding, the RmsNorm definition on constant vectors, bfloat16
rounding of hand-picked ties, and reductions to the plain step.
"""
import numpy as np
import pytest

import oracle
from oracle import rope


def table(max_pos, D, base=10000.0, dtype=np.float32):
    """Standard rotary angles p * base^(-2i/D), as float32 cos/sin tables."""
    i = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-2 * i / D)[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


# ---------------------------------------------------------------------------
# The rotation itself.
# ---------------------------------------------------------------------------
def test_quarter_turn_by_hand():
    x = np.array([1, 2, 3, 4], np.float32)
    c = np.zeros(2, np.float32)
    s = np.ones(2, np.float32)
    # half: pairs (0, 2) and (1, 3): (x1, x2) -> (-x2, x1)
    assert rope.rope_rotate(x, c, s, "half").tolist() == [-3, -4, 1, 2]
    # interleaved: pairs (0, 1) and (2, 3)
    assert rope.rope_rotate(x, c, s, "interleaved").tolist() == [-2, 1, -4, 3]
    # identity row and half turn
    assert rope.rope_rotate(x, np.ones(2, np.float32), np.zeros(2, np.float32), "half").tolist() == [1, 2, 3, 4]
    assert rope.rope_rotate(x, -np.ones(2, np.float32), np.zeros(2, np.float32), "interleaved").tolist() == \
        [-1, -2, -3, -4]


@pytest.mark.parametrize("mode", ["half", "interleaved"])
def test_rotation_is_complex_multiplication(mode):
    rng = np.random.default_rng(1)
    D = 16
    x = rng.standard_normal(D).astype(np.float32)
    th = rng.uniform(-np.pi, np.pi, D // 2)
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    y = rope.rope_rotate(x, c, s, mode).astype(np.float64)
    if mode == "half":
        z = x[: D // 2] + 1j * x[D // 2:].astype(np.float64)
        w = z * (c.astype(np.float64) + 1j * s)
        ref = np.concatenate([w.real, w.imag])
    else:
        z = x[0::2] + 1j * x[1::2].astype(np.float64)
        w = z * (c.astype(np.float64) + 1j * s)
        ref = np.stack([w.real, w.imag], axis=1).reshape(-1)
    assert np.allclose(y, ref, rtol=0, atol=4e-7 * np.abs(x).max())


def test_half_mode_is_rotate_half_form():
    """y = x * [cos, cos] + rotate_half(x) * [sin, sin], rotate_half(x) = [-x2, x1]."""
    rng = np.random.default_rng(2)
    D = 8
    x = rng.standard_normal((3, D)).astype(np.float32)
    c, s = table(5, D)
    y = rope.rope_rotate(x, c[4], s[4], "half").astype(np.float64)
    xd = x.astype(np.float64)
    rh = np.concatenate([-xd[:, D // 2:], xd[:, : D // 2]], axis=1)
    ref = xd * np.tile(c[4], 2) + rh * np.tile(s[4], 2)
    assert np.allclose(y, ref, atol=1e-6)


@pytest.mark.parametrize("mode", ["half", "interleaved"])
def test_rotation_preserves_norm_and_relative_position(mode):
    rng = np.random.default_rng(3)
    D = 64
    c, s = table(300, D)
    q = rng.standard_normal(D).astype(np.float32)
    k = rng.standard_normal(D).astype(np.float32)
    y = rope.rope_rotate(q, c[123], s[123], mode)
    assert abs(np.sum(y.astype(np.float64) ** 2) - np.sum(q.astype(np.float64) ** 2)) < 1e-4
    # q at p, k at p' : the dot product depends only on p - p'
    d1 = np.dot(rope.rope_rotate(q, c[200], s[200], mode).astype(np.float64),
                rope.rope_rotate(k, c[150], s[150], mode).astype(np.float64))
    d2 = np.dot(rope.rope_rotate(q, c[60], s[60], mode).astype(np.float64),
                rope.rope_rotate(k, c[10], s[10], mode).astype(np.float64))
    assert abs(d1 - d2) < 1e-4 * (1 + abs(d1))


def test_rotation_rounds_each_operation_in_float32():
    """x1 c - x2 s with x1 c and x2 s rounded to float32 first: values chosen
    so that a fused multiply-add would give a different float32."""
    x = np.array([1 + 2 ** -12, 1.0], np.float32)
    c = np.array([1 + 2 ** -12], np.float32)
    s = np.array([1.0], np.float32)
    y = rope.rope_rotate(x, c, s, "half")
    # exact x1*c = 1 + 2^-11 + 2^-24 -> float32 1 + 2^-11; minus 1 -> 2^-11
    assert y[0] == np.float32(2 ** -11)


# ---------------------------------------------------------------------------
# RmsNorm and bf16 rounding.
# ---------------------------------------------------------------------------
def test_rms_norm_on_constant_and_unit_vectors():
    x = np.full(8, -3.0)
    g = np.arange(1, 9, dtype=np.float32)
    assert np.allclose(rope.rms_norm(x, g, 0.0), -g)
    assert np.allclose(rope.rms_norm(x, np.ones(8), 7.0), -3 / 4.0)      # sqrt(9 + 7) = 4
    rng = np.random.default_rng(4)
    y = rope.rms_norm(rng.standard_normal(128) * 5, np.ones(128), 0.0)
    assert abs(np.mean(y * y) - 1) < 1e-12
    z = rng.standard_normal(16)
    assert np.allclose(rope.rms_norm(z, np.ones(16), 0.0), rope.rms_norm(1000 * z, np.ones(16), 0.0))


def test_bf16_encoding_rounds_to_nearest_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.0, 0.0, np.inf])
    assert rope.encode(vals, "bf16").tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x0000, 0x7F80]
    n = rope.encode(np.array([np.nan]), "bf16")
    assert (n[0] & 0x7F80) == 0x7F80 and (n[0] & 0x7F) != 0


# ---------------------------------------------------------------------------
# The step with rotation.
# ---------------------------------------------------------------------------
def _draw(rng, shape, dt):
    x = rng.standard_normal(shape).astype(np.float32)
    return x if dt == "f32" else (x.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("mode", ["half", "interleaved"])
def test_identity_row_reduces_to_plain_step(dt, mode):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, D, S = 3, 8, 2, 16, 12
    q, kc, vc = _draw(rng, (B, Hq, D), dt), _draw(rng, (B, Hkv, S, D), dt), _draw(rng, (B, Hkv, S, D), dt)
    kn, vn = _draw(rng, (B, Hkv, D), dt), _draw(rng, (B, Hkv, D), dt)
    L = np.array([0, 5, 11], np.int32)
    c = np.ones((1, D // 2), np.float32)
    s = np.zeros((1, D // 2), np.float32)
    out, rk, rv = rope.step_rope(q, dt, kc, vc, kn, vn, dt, L, "BHSD", Hq, Hkv, c, s, mode,
                                 positions=np.zeros(B, np.int32))
    ref, ek, ev = oracle.step(q, dt, kc, vc, kn, vn, dt, L, "BHSD", Hq, Hkv)
    assert np.array_equal(out, ref) and rk.tobytes() == ek.tobytes() and rv.tobytes() == ev.tobytes()


@pytest.mark.parametrize("mode", ["half", "interleaved"])
def test_shifting_every_position_leaves_the_step_unchanged(mode):
    """Cache keys rotated at their own positions j + delta, the new token at
    L + delta: the output does not depend on delta (relative positions)."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, D, S = 2, 4, 2, 32, 10
    c, s = table(64, D)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    raw = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    L = np.array([9, 4], np.int32)
    outs = []
    for delta in (0, 37):
        kc = np.empty_like(raw)
        for j in range(S):
            kc[:, :, j] = rope.rope_rotate(raw[:, :, j], c[j + delta], s[j + delta], mode)
        out, _, _ = rope.step_rope(q, "f32", kc, vc, kn, vn, "f32", L, "BHSD", Hq, Hkv, c, s, mode,
                                   positions=L + delta)
        outs.append(out)
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-5
    # and a wrong query position changes it
    kc = np.empty_like(raw)
    for j in range(S):
        kc[:, :, j] = rope.rope_rotate(raw[:, :, j], c[j], s[j], mode)
    bad, _, _ = rope.step_rope(q, "f32", kc, vc, kn, vn, "f32", L, "BHSD", Hq, Hkv, c, s, mode, positions=L + 3)
    assert np.max(np.abs(bad - outs[0])) > 1e-3


def test_default_position_is_the_new_slot_and_only_token_gives_v_new():
    rng = np.random.default_rng(7)
    B, Hq, Hkv, D, S = 2, 4, 1, 8, 6
    c, s = table(S, D)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, S, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    L = np.array([0, 3], np.int32)
    out, rk, _ = rope.step_rope(q, "f32", kc, vc, kn, vn, "f32", L, "BHSD", Hq, Hkv, c, s, "half")
    assert np.array_equal(out[0], np.repeat(vn[0].astype(np.float64), Hq, axis=0))
    assert np.array_equal(rk[1, 0, 3], rope.rope_rotate(kn[1, 0], c[3], s[3], "half"))
    assert np.array_equal(rk[0, 0, 0], kn[0, 0])                     # position 0: identity row


def test_norm_gains_scale_the_appended_key():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, S = 2, 4, 2, 64, 5
    c, s = table(S, D)
    q = _draw(rng, (B, Hq, D), "bf16")
    kc, vc = _draw(rng, (B, Hkv, S, D), "bf16"), _draw(rng, (B, Hkv, S, D), "bf16")
    kn, vn = _draw(rng, (B, Hkv, D), "bf16"), _draw(rng, (B, Hkv, D), "bf16")
    L = np.array([1, 4], np.int32)
    g = np.full(D, 2.0, np.float32)
    out, rk, _ = rope.step_rope(q, "bf16", kc, vc, kn, vn, "bf16", L, "BHSD", Hq, Hkv, c, s, "interleaved",
                                q_gain=np.ones(D, np.float32), k_gain=g, eps=1e-6)
    k = oracle.decode(rk[0, :, 1], "bf16")
    assert np.allclose(np.mean(k * k, axis=-1), 4.0, rtol=2e-2)      # gain 2 -> mean square 4
    with pytest.raises(ValueError):
        rope.step_rope(q, "bf16", kc, vc, kn, vn, "bf16", L, "BHSD", Hq, Hkv, c, s, "half", k_gain=g)
    with pytest.raises(ValueError):
        rope.step_rope(q, "bf16", kc, vc, kn, vn, "bf16", L, "BHSD", Hq, Hkv, c, s, "half", eps=1e-6)


def test_rejections():
    q = np.zeros((1, 1, 6), np.float32)
    c, s = table(4, 6)
    with pytest.raises(ValueError):
        rope.rotate_new(q, "f32", np.zeros((1, 1, 6), np.float32), "f32", np.array([4]), c, s, "half")
    with pytest.raises(ValueError):
        rope.rope_rotate(np.zeros(5, np.float32), c[0][:2], s[0][:2], "half")
    with pytest.raises(ValueError):
        rope.rope_rotate(np.zeros(6, np.float32), c[0], s[0], "spiral")


# ---------------------------------------------------------------------------
# Int8 caches: rotation, then the per-row quantization rule.
# ---------------------------------------------------------------------------
def _q8_inputs(rng, B, Hq, Hkv, D, S):
    q = (rng.standard_normal((B, Hq, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kc = rng.integers(-127, 128, (B, Hkv, S, D)).astype(np.int8)
    vc = rng.integers(-127, 128, (B, Hkv, S, D)).astype(np.int8)
    ks = rng.uniform(0.01, 0.03, (B, Hkv, S)).astype(np.float32)
    vs = rng.uniform(0.01, 0.03, (B, Hkv, S)).astype(np.float32)
    kn = (rng.standard_normal((B, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    vn = (rng.standard_normal((B, Hkv, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return q, kc, vc, ks, vs, kn, vn


def test_q8_identity_row_reduces_to_q8_step():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, D, S = 2, 4, 2, 16, 7
    q, kc, vc, ks, vs, kn, vn = _q8_inputs(rng, B, Hq, Hkv, D, S)
    L = np.array([0, 6], np.int32)
    c, s = np.ones((3, D // 2), np.float32), np.zeros((3, D // 2), np.float32)
    got = rope.step_q8_rope(q, "bf16", kc, vc, ks, vs, kn, vn, L, "BHSD", Hq, Hkv, c, s, "half",
                            positions=np.array([2, 1], np.int32))
    ref = oracle.step_q8(q, "bf16", kc, vc, ks, vs, kn, vn, L, "BHSD", Hq, Hkv)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


def test_q8_quarter_turn_permutes_codes_with_signs():
    """A quarter turn maps (x1, x2) to (-x2, x1) exactly; the row maximum is
    unchanged and rounding half to even is odd-symmetric, so the stored codes
    are the unrotated codes moved and negated, with the same scale."""
    rng = np.random.default_rng(10)
    B, Hq, Hkv, D, S = 1, 2, 1, 8, 3
    q, kc, vc, ks, vs, kn, vn = _q8_inputs(rng, B, Hq, Hkv, D, S)
    L = np.array([1], np.int32)
    c, s = np.zeros((1, D // 2), np.float32), np.ones((1, D // 2), np.float32)
    _, rk, _, rks, _ = rope.step_q8_rope(q, "bf16", kc, vc, ks, vs, kn, vn, L, "BHSD", Hq, Hkv, c, s, "half",
                                         positions=np.zeros(1, np.int32))
    codes, scale = oracle.quantize_row(oracle.decode(kn[0, 0], "bf16").astype(np.float32))
    h = D // 2
    assert rks[0, 0, 1] == scale
    assert rk[0, 0, 1].tolist() == (-codes[h:]).tolist() + codes[:h].tolist()

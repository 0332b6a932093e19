"""Pins for the float64 oracle, independent of the oracle itself.

Each test checks the oracle against something the pages or the mathematics fix:
the pages' worked examples (fixtures under tests/golden/, each citing its page),
closed forms, invariances of the definition, a library routine the definition
reduces to (torch's scaled-dot-product attention in float64 on the CPU), and
brute-force pure-Python loops on tiny inputs.  The comment on each test names
the mistake it is there to catch.
"""
import json
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _printed(strings):
    """Printed page values -> (float64 values, half a unit of the last printed digit)."""
    a = np.array(strings)
    vals = a.astype(np.float64)
    dec = np.vectorize(lambda s: len(s.split(".")[1]) if "." in s else 0)(a)
    return vals, 0.5 * 10.0 ** (-dec.astype(np.float64))


def f32(x):
    return np.array(x, dtype=np.float32)


def bf16_bits(x):
    """float values -> bf16 bit patterns, rounded to nearest even (via torch)."""
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ---------------------------------------------------------------------------
# Worked examples of the KV-cache decode step page (one step, caches extended).
# Catches: append at the wrong slot, attention that skips the new token,
# wrong grouping for Hq > Hkv, a softmax that is not normalised.
# ---------------------------------------------------------------------------
P1 = _load("kv_cache_decode_step_examples.json")


@pytest.mark.parametrize("case", P1["cases"], ids=[c["name"] for c in P1["cases"]])
def test_kv_cache_decode_step_page_examples(case):
    q = f32(case["query"])
    kc, vc = f32(case["key_cache"]), f32(case["value_cache"])    # (B, Hkv, S, D)
    B, Hkv, S, D = kc.shape
    # capacity S+1; the free slot holds garbage the append must overwrite
    kcap = np.full((B, Hkv, S + 1, D), 777.0, np.float32)
    vcap = np.full((B, Hkv, S + 1, D), -777.0, np.float32)
    kcap[:, :, :S] = kc
    vcap[:, :, :S] = vc
    lengths = np.full(B, S, np.int32)
    out, k_after, v_after = oracle.step(q, "f32", kcap, vcap, f32(case["new_key"]), f32(case["new_value"]),
                                        "f32", lengths, "BHSD", case["num_query_heads"], case["num_kv_heads"])
    exp, tol = _printed(case["output"])
    assert np.all(np.abs(out - exp) <= tol)
    # The printed outputs are exact closed forms (means, and weights 1/4, 3/4 for a
    # key gap of ln 3); the float32 storage of the inputs moves them by < 2e-8.
    assert np.max(np.abs(out - exp)) < 1e-7
    for got, key in ((k_after, "new_key_cache"), (v_after, "new_value_cache")):
        ev, et = _printed(case[key])
        assert got.shape == ev.shape
        assert np.all(np.abs(got.astype(np.float64) - ev) <= et)
    # slots < S keep their bits; slot S holds exactly the new key/value bits
    assert k_after[:, :, :S].tobytes() == kc.tobytes()
    assert v_after[:, :, :S].tobytes() == vc.tobytes()
    assert k_after[:, :, S].tobytes() == f32(case["new_key"]).tobytes()
    assert v_after[:, :, S].tobytes() == f32(case["new_value"]).tobytes()


# ---------------------------------------------------------------------------
# Worked examples of the JAX "Grouped-Query Decode Step" page.
# Catches: wrong scale (1/D instead of 1/sqrt(D)), stale slots with weight,
# wrong kv-head for a query head (h % Hkv instead of h // G), a (B,S,Hkv,D)
# cache indexed as (B,Hkv,S,D).
# ---------------------------------------------------------------------------
P2 = _load("gqa_decode_step_jax_examples.json")


@pytest.mark.parametrize("case", P2["cases"], ids=[c["name"] for c in P2["cases"]])
def test_gqa_jax_page_examples(case):
    q = f32(case["query"])
    kc, vc = f32(case["key_cache"]), f32(case["value_cache"])    # (B, S, Hkv, D)
    out = oracle.attend(q, "f32", kc, vc, "f32", np.array(case["lengths"], np.int32), "BSHD",
                        case["num_query_heads"], case["num_kv_heads"])
    exp, tol = _printed(case["output"])
    assert out.shape == exp.shape
    assert np.all(np.abs(out - exp) <= tol + 1e-7), np.abs(out - exp).max()


def test_jax_example1_scores_and_weights():
    """The page prints head 0's scores (1/sqrt(2) and 0) and weights."""
    case = P2["cases"][0]
    q = oracle.decode(f32(case["query"]), "f32")
    K = oracle.decode(oracle.kv_rows(f32(case["key_cache"]), "BSHD", 0, 0, 2), "f32")
    s, w = oracle.softmax_weights(q[0, 0], K)
    es, ts = _printed(case["head0_scores"])
    ew, tw = _printed(case["head0_weights"])
    assert np.all(np.abs(s - es) <= ts) and np.all(np.abs(w - ew) <= tw)
    assert s[0] == pytest.approx(1 / math.sqrt(2), abs=1e-15)


# ---------------------------------------------------------------------------
# Closed forms.
# ---------------------------------------------------------------------------
def test_identical_keys_give_mean_of_values():
    """Equal keys -> equal weights -> plain mean (catches a biased softmax)."""
    rng = np.random.default_rng(11)
    for n in (2, 3, 7):
        D = 8
        k = np.tile(rng.standard_normal(D).astype(np.float32), (n, 1))
        v = rng.standard_normal((n, D)).astype(np.float32)
        q = rng.standard_normal(D).astype(np.float32)
        cache_k = k[None, None]
        cache_v = v[None, None]
        out = oracle.attend(q[None, None], "f32", cache_k, cache_v, "f32", np.array([n], np.int32), "BHSD", 1, 1)
        np.testing.assert_allclose(out[0, 0], v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_log_gap_gives_ratio_weights_and_fixes_scale():
    """Scores log(c_j) give weights c_j / sum(c).  With D=4 and q = 2 e_0 the
    score is k_j[0] only if the scale is 1/sqrt(D) (1/D would halve it)."""
    D = 4
    c = np.array([1.0, 3.0, 0.5, 2.0])
    k = np.zeros((4, D), np.float32)
    k[:, 0] = np.log(c).astype(np.float32)
    k[:, 1:] = np.float32(5.0)        # orthogonal to q: must not matter
    v = np.eye(4, D, dtype=np.float32)  # output = weights
    q = np.array([2.0, 0.0, 0.0, 0.0], np.float32)
    out = oracle.attend(q[None, None], "f32", k[None, None], v[None, None], "f32", np.array([4], np.int32),
                        "BHSD", 1, 1)
    np.testing.assert_allclose(out[0, 0], c / c.sum(), rtol=0, atol=1e-7)
    # the ln 3 case: weights 1/4 and 3/4
    k2 = np.array([[0.0, 0, 0, 0], [math.log(3.0), 0, 0, 0]], np.float32)
    v2 = np.array([[2.0, 0, 0, 0], [6.0, 0, 0, 0]], np.float32)
    out2 = oracle.attend(q[None, None], "f32", k2[None, None], v2[None, None], "f32", np.array([2], np.int32),
                         "BHSD", 1, 1)
    assert out2[0, 0, 0] == pytest.approx(0.25 * 2 + 0.75 * 6, abs=1e-6)


def test_zero_query_gives_uniform_mean():
    rng = np.random.default_rng(12)
    k = rng.standard_normal((1, 1, 9, 16)).astype(np.float32) * 100
    v = rng.standard_normal((1, 1, 9, 16)).astype(np.float32)
    q = np.zeros((1, 1, 16), np.float32)
    out = oracle.attend(q, "f32", k, v, "f32", np.array([6], np.int32), "BHSD", 1, 1)
    np.testing.assert_allclose(out[0, 0], v[0, 0, :6].astype(np.float64).mean(0), rtol=0, atol=1e-14)


def test_single_valid_slot_returns_it_exactly():
    rng = np.random.default_rng(13)
    for dt in ("f32", "bf16"):
        kf = rng.standard_normal((2, 3, 5, 8)) * 30
        vf = rng.standard_normal((2, 3, 5, 8))
        k = f32(kf) if dt == "f32" else bf16_bits(kf)
        v = f32(vf) if dt == "f32" else bf16_bits(vf)
        q = f32(rng.standard_normal((2, 6, 8)))
        out = oracle.attend(q, "f32", k, v, dt, np.array([1, 1], np.int32), "BHSD", 6, 3)
        for b in range(2):
            for hq in range(6):
                assert np.array_equal(out[b, hq], oracle.decode(v[b, hq // 2, 0], dt))


def test_step_from_empty_returns_new_value_exactly():
    rng = np.random.default_rng(14)
    k = f32(rng.standard_normal((3, 2, 4, 8)) * 1e3)
    v = f32(rng.standard_normal((3, 2, 4, 8)) * 1e3)
    kn, vn = f32(rng.standard_normal((3, 2, 8))), f32(rng.standard_normal((3, 2, 8)))
    q = f32(rng.standard_normal((3, 4, 8)))
    out, _, _ = oracle.step(q, "f32", k, v, kn, vn, "f32", np.zeros(3, np.int32), "BHSD", 4, 2)
    for b in range(3):
        for hq in range(4):
            assert np.array_equal(out[b, hq], vn[b, hq // 2].astype(np.float64))


# ---------------------------------------------------------------------------
# Masking: whatever sits at slot >= lengths[b] cannot change the result.
# Catches reading one slot too many (j <= L instead of j < L).
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_stale_slots_never_matter(layout):
    rng = np.random.default_rng(15)
    B, Hq, Hkv, S, D = 3, 8, 2, 11, 16
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    k = f32(rng.standard_normal(shape))
    v = f32(rng.standard_normal(shape))
    q = f32(rng.standard_normal((B, Hq, D)))
    lengths = np.array([4, 11, 1], np.int32)
    ref = oracle.attend(q, "f32", k, v, "f32", lengths, layout, Hq, Hkv)
    for fill in (np.nan, np.inf, -np.inf, 1e30, 1e4):
        k2, v2 = k.copy(), v.copy()
        for b in range(B):
            for h in range(Hkv):
                for j in range(lengths[b], S):
                    k2[oracle.kv_index(layout, b, h, j)] = fill
                    v2[oracle.kv_index(layout, b, h, j)] = -fill
        out = oracle.attend(q, "f32", k2, v2, "f32", lengths, layout, Hq, Hkv)
        assert np.array_equal(out, ref)
    # ...while changing a valid slot does change it (the test above is not vacuous)
    k3 = k.copy()
    k3[oracle.kv_index(layout, 0, 0, 3)] += 1.0
    assert not np.array_equal(oracle.attend(q, "f32", k3, v, "f32", lengths, layout, Hq, Hkv), ref)


# ---------------------------------------------------------------------------
# A library routine the definition reduces to: torch's scaled_dot_product_attention
# in float64 on the CPU, with a boolean length mask and enable_gqa (query head i
# reads kv-head i // G).  Random shapes from the JAX page's constraint ranges.
# ---------------------------------------------------------------------------
def _sdpa(qf, kf, vf, n_valid, Hq, Hkv):
    """qf (B,Hq,D), kf/vf (B,Hkv,S,D) float64 -> (B,Hq,D)."""
    B, _, S, D = kf.shape
    mask = torch.arange(S)[None, :] < torch.as_tensor(n_valid)[:, None]     # (B,S)
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(qf)[:, :, None, :], torch.as_tensor(kf), torch.as_tensor(vf),
        attn_mask=mask[:, None, None, :], enable_gqa=(Hq != Hkv))
    return o[:, :, 0, :].numpy()


def test_against_torch_sdpa_on_page_domain():
    rng = np.random.default_rng(16)
    for trial in range(300):
        B = int(rng.integers(1, 4))
        S = int(rng.integers(3, 9))
        D = int(rng.integers(2, 5))
        Hq = int(rng.integers(2, 9))
        Hkv = int(rng.choice([h for h in range(1, Hq + 1) if Hq % h == 0]))
        layout = "BHSD" if trial % 2 else "BSHD"
        dt = "bf16" if trial % 3 == 0 else "f32"
        kf = rng.standard_normal((B, Hkv, S, D)) * 2
        vf = rng.standard_normal((B, Hkv, S, D))
        enc = (lambda x: f32(x)) if dt == "f32" else bf16_bits
        k_bhsd, v_bhsd = enc(kf), enc(vf)
        k_st = k_bhsd if layout == "BHSD" else np.ascontiguousarray(k_bhsd.transpose(0, 2, 1, 3))
        v_st = v_bhsd if layout == "BHSD" else np.ascontiguousarray(v_bhsd.transpose(0, 2, 1, 3))
        q = f32(rng.standard_normal((B, Hq, D)))
        n = rng.integers(1, S + 1, size=B).astype(np.int32)
        out = oracle.attend(q, "f32", k_st, v_st, dt, n, layout, Hq, Hkv)
        ref = _sdpa(q.astype(np.float64), oracle.decode(k_bhsd, dt), oracle.decode(v_bhsd, dt), n, Hq, Hkv)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_against_pure_python_brute_force():
    """Loops over python floats with math.exp/math.fsum -- no NumPy arithmetic."""
    rnd = random.Random(17)
    for _ in range(40):
        B, Hkv, G, S, D = rnd.randint(1, 2), rnd.randint(1, 3), rnd.randint(1, 3), rnd.randint(1, 5), rnd.randint(1, 4)
        Hq = Hkv * G
        k = [[[[rnd.uniform(-3, 3) for _ in range(D)] for _ in range(S)] for _ in range(Hkv)] for _ in range(B)]
        v = [[[[rnd.uniform(-3, 3) for _ in range(D)] for _ in range(S)] for _ in range(Hkv)] for _ in range(B)]
        q = [[[rnd.uniform(-3, 3) for _ in range(D)] for _ in range(Hq)] for _ in range(B)]
        n = [rnd.randint(1, S) for _ in range(B)]
        k32, v32, q32 = f32(k), f32(v), f32(q)
        out = oracle.attend(q32, "f32", k32, v32, "f32", np.array(n, np.int32), "BHSD", Hq, Hkv)
        for b in range(B):
            for hq in range(Hq):
                h = hq // G
                qq = [float(x) for x in q32[b, hq]]
                sc = [math.fsum(qq[d] * float(k32[b, h, j, d]) for d in range(D)) / math.sqrt(D) for j in range(n[b])]
                mx = max(sc)
                e = [math.exp(s - mx) for s in sc]
                z = math.fsum(e)
                for d in range(D):
                    ref = math.fsum(e[j] / z * float(v32[b, h, j, d]) for j in range(n[b]))
                    assert abs(out[b, hq, d] - ref) <= 1e-12


# ---------------------------------------------------------------------------
# Decode loop == causal attention (brainjuice "Reuse keys and values": earlier
# keys/values stay valid under a causal mask).  T steps from an empty cache give
# the rows of causal full attention, computed here by torch's SDPA(is_causal).
# Catches an append that lands one slot off, or a step that attends L instead
# of L+1 slots.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (6, 1)])
def test_decode_loop_equals_causal_attention(Hq, Hkv):
    g = torch.Generator().manual_seed(0)
    B, T, D = 2, 3, 4                      # the lesson's demo shape [2, 2, 3, 4]
    qs = torch.randn(B, Hq, T, D, generator=g).float()
    ks = torch.randn(B, Hkv, T, D, generator=g).float()
    vs = torch.randn(B, Hkv, T, D, generator=g).float()
    kc = np.full((B, Hkv, T, D), np.nan, np.float32)
    vc = np.full((B, Hkv, T, D), np.nan, np.float32)
    outs = []
    for t in range(T):
        out, kc, vc = oracle.step(qs[:, :, t].numpy(), "f32", kc, vc, ks[:, :, t].numpy().copy(),
                                  vs[:, :, t].numpy().copy(), "f32", np.full(B, t, np.int32), "BHSD", Hq, Hkv)
        outs.append(out)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qs.double(), ks.double(), vs.double(), is_causal=True, enable_gqa=(Hq != Hkv)).numpy()
    np.testing.assert_allclose(np.stack(outs, axis=2), ref, rtol=0, atol=1e-12)
    assert not np.isnan(kc).any() and not np.isnan(vc).any()


# ---------------------------------------------------------------------------
# Invariances of the definition.
# ---------------------------------------------------------------------------
def _rand_problem(rng, B=2, Hq=6, Hkv=3, S=9, D=8, layout="BHSD"):
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    # dyadic values: sums and shifts below are exact in float32
    k = f32(np.round(rng.standard_normal(shape) * 8) / 8)
    v = f32(np.round(rng.standard_normal(shape) * 8) / 8)
    q = f32(np.round(rng.standard_normal((B, Hq, D)) * 8) / 8)
    n = rng.integers(1, S + 1, size=B).astype(np.int32)
    return q, k, v, n


def test_permuting_valid_slots_jointly_changes_nothing():
    rng = np.random.default_rng(18)
    q, k, v, n = _rand_problem(rng)
    ref = oracle.attend(q, "f32", k, v, "f32", n, "BHSD", 6, 3)
    k2, v2 = k.copy(), v.copy()
    for b in range(2):
        p = rng.permutation(n[b])
        k2[b, :, :n[b]] = k[b, :, p].transpose(1, 0, 2)
        v2[b, :, :n[b]] = v[b, :, p].transpose(1, 0, 2)
    np.testing.assert_allclose(oracle.attend(q, "f32", k2, v2, "f32", n, "BHSD", 6, 3), ref, rtol=0, atol=1e-13)


def test_value_shift_and_scale():
    """Weights sum to one: out(V + c) = out(V) + c; out(2V) = 2 out(V)."""
    rng = np.random.default_rng(19)
    q, k, v, n = _rand_problem(rng)
    ref = oracle.attend(q, "f32", k, v, "f32", n, "BHSD", 6, 3)
    c = f32(np.arange(8) / 4 - 1)
    np.testing.assert_allclose(oracle.attend(q, "f32", k, v + c, "f32", n, "BHSD", 6, 3), ref + c.astype(np.float64),
                               rtol=0, atol=1e-12)
    np.testing.assert_array_equal(oracle.attend(q, "f32", k, 2 * v, "f32", n, "BHSD", 6, 3), 2 * ref)


def test_key_shift_changes_nothing():
    """K_j + c shifts every score of a head by q.c/sqrt(D): softmax unchanged."""
    rng = np.random.default_rng(20)
    q, k, v, n = _rand_problem(rng)
    ref = oracle.attend(q, "f32", k, v, "f32", n, "BHSD", 6, 3)
    c = f32(np.arange(8) / 8 - 0.5)
    np.testing.assert_allclose(oracle.attend(q, "f32", k + c, v, "f32", n, "BHSD", 6, 3), ref, rtol=0, atol=1e-12)


def test_layouts_agree():
    rng = np.random.default_rng(21)
    q, k, v, n = _rand_problem(rng)
    a = oracle.attend(q, "f32", k, v, "f32", n, "BHSD", 6, 3)
    b = oracle.attend(q, "f32", np.ascontiguousarray(k.transpose(0, 2, 1, 3)),
                      np.ascontiguousarray(v.transpose(0, 2, 1, 3)), "f32", n, "BSHD", 6, 3)
    assert np.array_equal(a, b)


def test_group_equals_mha_on_its_kv_head():
    """G = 1 is multi-head attention; a GQA head equals MHA over its own kv-head."""
    rng = np.random.default_rng(22)
    q, k, v, n = _rand_problem(rng)
    gqa = oracle.attend(q, "f32", k, v, "f32", n, "BHSD", 6, 3)
    krep, vrep = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)   # kv-head h -> query heads 2h, 2h+1
    mha = oracle.attend(q, "f32", krep, vrep, "f32", n, "BHSD", 6, 6)
    assert np.array_equal(gqa, mha)


def test_output_in_convex_hull_of_valid_values():
    rng = np.random.default_rng(23)
    q, k, v, n = _rand_problem(rng)
    out = oracle.attend(q, "f32", k * 4, v, "f32", n, "BHSD", 6, 3)
    for b in range(2):
        for hq in range(6):
            vv = v[b, hq // 2, :n[b]].astype(np.float64)
            assert np.all(out[b, hq] >= vv.min(0) - 1e-12) and np.all(out[b, hq] <= vv.max(0) + 1e-12)


# ---------------------------------------------------------------------------
# Storage decoding and the append's bytes.
# ---------------------------------------------------------------------------
def test_bf16_decode_matches_torch_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(ours, ref)     # NaNs compare equal here


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_append_touches_exactly_one_slot_per_head(layout, dt):
    rng = np.random.default_rng(24)
    B, Hkv, S, D = 3, 2, 6, 8
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    enc = (lambda x: f32(x)) if dt == "f32" else bf16_bits
    k, v = enc(rng.standard_normal(shape)), enc(rng.standard_normal(shape))
    kn, vn = enc(rng.standard_normal((B, Hkv, D))), enc(rng.standard_normal((B, Hkv, D)))
    L = np.array([0, 5, 2], np.int32)
    k2, v2 = oracle.append(k, v, kn, vn, L, layout)
    changed = set()
    for idx in np.argwhere(k2 != k):
        changed.add(tuple(idx[:3]))
    expect = {oracle.kv_index(layout, b, h, int(L[b])) for b in range(B) for h in range(Hkv)}
    assert changed <= expect and len(changed) == len(expect)
    for b in range(B):
        for h in range(Hkv):
            assert k2[oracle.kv_index(layout, b, h, int(L[b]))].tobytes() == kn[b, h].tobytes()
            assert v2[oracle.kv_index(layout, b, h, int(L[b]))].tobytes() == vn[b, h].tobytes()
    # slot lengths[b] in (B,Hkv,S,D) is the transpose of the same slot in (B,S,Hkv,D)
    if layout == "BSHD":
        kt, vt = oracle.append(np.ascontiguousarray(k.transpose(0, 2, 1, 3)),
                               np.ascontiguousarray(v.transpose(0, 2, 1, 3)), kn, vn, L, "BHSD")
        assert np.array_equal(kt.transpose(0, 2, 1, 3), k2) and np.array_equal(vt.transpose(0, 2, 1, 3), v2)


def test_out_of_contract_inputs_raise():
    k = np.zeros((1, 1, 4, 2), np.float32)
    kn = np.zeros((1, 1, 2), np.float32)
    q = np.zeros((1, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.append(k, k, kn, kn, np.array([4], np.int32), "BHSD")       # no free slot
    with pytest.raises(ValueError):
        oracle.attend(q, "f32", k, k, "f32", np.array([5], np.int32), "BHSD", 1, 1)
    with pytest.raises(ValueError):
        oracle.attend(np.zeros((1, 3, 2), np.float32), "f32", np.zeros((1, 2, 4, 2), np.float32),
                      np.zeros((1, 2, 4, 2), np.float32), "f32", np.array([1], np.int32), "BHSD", 3, 2)


def test_zero_valid_slots_reads_as_zeros():
    k = np.full((1, 1, 4, 2), np.nan, np.float32)
    q = np.ones((1, 2, 2), np.float32)
    out = oracle.attend(q, "f32", k, k, "f32", np.array([0], np.int32), "BHSD", 2, 1)
    assert np.array_equal(out, np.zeros((1, 2, 2)))

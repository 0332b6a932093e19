"""Pins for the mapped-cache oracle (slot-indexed rows, paged block pools).

The mapped functions only change where slot j of (sequence b, kv-head h) is
stored (CLIKA runtime "groupQueryAttention" API page, slot_ids and block-table
notes).  They are pinned to the pages' printed examples routed through
permuted rows / scattered blocks with NaN garbage everywhere else (a wrong
index reads NaN or a wrong value), to the dense oracle on the same logical
cache (a reduction the definition fixes), and to the page's validation rules.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _printed(strings):
    a = np.array(strings)
    vals = a.astype(np.float64)
    dec = np.vectorize(lambda s: len(s.split(".")[1]) if "." in s else 0)(a)
    return vals, 0.5 * 10.0 ** (-dec.astype(np.float64))


def f32(x):
    return np.array(x, dtype=np.float32)


def garbage_like(shape, dtype):
    """NaN everywhere (bf16 NaN bits for uint16 storage)."""
    if dtype == np.uint16:
        return np.full(shape, 0x7FC1, dtype=np.uint16)
    return np.full(shape, np.nan, dtype=np.float32)


def to_slots(dense, layout, slot_ids, num_rows):
    """Continuous cache with batch row b stored at row slot_ids[b], NaN elsewhere."""
    out = garbage_like((num_rows,) + dense.shape[1:], dense.dtype)
    for b, r in enumerate(slot_ids):
        out[r] = dense[b]
    return out


def to_pool(dense, layout, bs, rng, spare=3):
    """Scatter a dense (B, .., S, ..) cache into a block pool with a random
    table; unused blocks and the tail pads hold NaN.  Returns (pool, table)."""
    if layout == "BHSD":
        B, Hkv, S, D = dense.shape
    else:
        B, S, Hkv, D = dense.shape
    nb = -(-S // bs)
    total = B * nb + spare
    perm = rng.permutation(total)
    table = perm[: B * nb].reshape(B, nb).astype(np.int32)
    pool_shape = (total, Hkv, bs, D) if layout == "BHSD" else (total, bs, Hkv, D)
    pool = garbage_like(pool_shape, dense.dtype)
    for b in range(B):
        for j in range(S):
            blk, off = table[b, j // bs], j % bs
            for h in range(Hkv):
                src = dense[b, h, j] if layout == "BHSD" else dense[b, j, h]
                if layout == "BHSD":
                    pool[blk, h, off] = src
                else:
                    pool[blk, off, h] = src
    # one extra table column of -1 pads
    table = np.concatenate([table, -np.ones((B, 1), np.int32)], axis=1)
    return pool, table


# ---------------------------------------------------------------------------
# The JAX page's printed examples, routed through permuted rows and scattered
# blocks.  Catches: reading row b instead of slot_ids[b]; a wrong block or
# in-block offset; a pool layout with the head and slot axes swapped.
# ---------------------------------------------------------------------------
P2 = _load("gqa_decode_step_jax_examples.json")


@pytest.mark.parametrize("case", P2["cases"], ids=[c["name"] for c in P2["cases"]])
def test_jax_page_examples_through_slot_rows(case):
    q = f32(case["query"])
    kc, vc = f32(case["key_cache"]), f32(case["value_cache"])    # (B, S, Hkv, D)
    B = kc.shape[0]
    slots = list(range(2 * B - 1, -1, -2))                       # reversed, every other row
    ks, vs = to_slots(kc, "BSHD", slots, 2 * B), to_slots(vc, "BSHD", slots, 2 * B)
    out = oracle.attend_mapped("slots", q, "f32", ks, vs, "f32", np.array(case["lengths"]), "BSHD",
                               case["num_query_heads"], case["num_kv_heads"], np.array(slots, np.int32))
    exp, tol = _printed(case["output"])
    assert np.all(np.abs(out - exp) <= tol + 1e-7)


@pytest.mark.parametrize("bs", [1, 2])
@pytest.mark.parametrize("case", P2["cases"], ids=[c["name"] for c in P2["cases"]])
def test_jax_page_examples_through_paged_pool(case, bs):
    q = f32(case["query"])
    kc, vc = f32(case["key_cache"]), f32(case["value_cache"])
    S = kc.shape[1]
    if S % bs:
        pytest.skip("capacity not a multiple of the block size")
    rng = np.random.default_rng(5 + bs)
    kp, table = to_pool(kc, "BSHD", bs, rng)
    vp, table2 = to_pool(vc, "BSHD", bs, np.random.default_rng(5 + bs))
    assert np.array_equal(table, table2)
    table = table[:, :-1]                                        # capacity = columns * bs
    out = oracle.attend_mapped("paged", q, "f32", kp, vp, "f32", np.array(case["lengths"]), "BSHD",
                               case["num_query_heads"], case["num_kv_heads"], table, bs)
    exp, tol = _printed(case["output"])
    assert np.all(np.abs(out - exp) <= tol + 1e-7)


# ---------------------------------------------------------------------------
# The KV-cache decode step page's examples as a paged step: the output is the
# page's, and the new key/value land in block table[b][L // bs] at L % bs.
# ---------------------------------------------------------------------------
P1 = _load("kv_cache_decode_step_examples.json")


@pytest.mark.parametrize("case", P1["cases"], ids=[c["name"] for c in P1["cases"]])
def test_kv_cache_page_examples_as_paged_step(case):
    q = f32(case["query"])
    kc, vc = f32(case["key_cache"]), f32(case["value_cache"])    # (B, Hkv, S, D)
    B, Hkv, S, D = kc.shape
    kd = np.concatenate([kc, np.full((B, Hkv, 1, D), 7.0, np.float32)], axis=2)
    vd = np.concatenate([vc, np.full((B, Hkv, 1, D), 7.0, np.float32)], axis=2)
    kp, table = to_pool(kd, "BHSD", 1, np.random.default_rng(3))
    vp, _ = to_pool(vd, "BHSD", 1, np.random.default_rng(3))
    table = table[:, :-1]
    L = np.full(B, S, np.int32)
    out, kp2, vp2 = oracle.step_mapped("paged", q, "f32", kp, vp, f32(case["new_key"]), f32(case["new_value"]),
                                       "f32", L, "BHSD", case["num_query_heads"], Hkv, table, 1)
    exp, tol = _printed(case["output"])
    assert np.all(np.abs(out - exp) <= tol) and np.max(np.abs(out - exp)) < 1e-7
    for b in range(B):
        blk = table[b, S]
        assert np.array_equal(kp2[blk, :, 0], f32(case["new_key"])[b])
        assert np.array_equal(vp2[blk, :, 0], f32(case["new_value"])[b])


# ---------------------------------------------------------------------------
# Reduction to the dense oracle: the same logical cache, stored densely or
# through a map, gives identical float64 results (the mapping only moves
# bytes).  Catches any index slip in the gather for other shapes and layouts.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("bs", [1, 3, 4, 16])
def test_paged_equals_dense(layout, dt, bs):
    rng = np.random.default_rng(bs * 7 + (layout == "BSHD"))
    B, Hq, Hkv, D = 3, 6, 2, 8
    S = bs * 5
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)

    def draw(shp):
        x = rng.standard_normal(shp).astype(np.float32)
        if dt == "f32":
            return x
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    kc, vc, q = draw(shape), draw(shape), draw((B, Hq, D))
    kn, vn = draw((B, Hkv, D)), draw((B, Hkv, D))
    L = rng.integers(0, S, B).astype(np.int32)
    kp, table = to_pool(kc, layout, bs, np.random.default_rng(1))
    vp, _ = to_pool(vc, layout, bs, np.random.default_rng(1))
    table = table[:, :-1]
    ref, rk, rv = oracle.step(q, dt, kc, vc, kn, vn, dt, L, layout, Hq, Hkv)
    got, pk, pv = oracle.step_mapped("paged", q, dt, kp, vp, kn, vn, dt, L, layout, Hq, Hkv, table, bs)
    assert np.array_equal(got, ref)
    # the appended pool is the scatter of the appended dense cache; nothing else moved
    ek, _ = to_pool(rk, layout, bs, np.random.default_rng(1))
    ev, _ = to_pool(rv, layout, bs, np.random.default_rng(1))
    assert pk.tobytes() == ek.tobytes() and pv.tobytes() == ev.tobytes()
    # attend over the appended pool with lengths + 1 equals the step's output
    att = oracle.attend_mapped("paged", q, dt, pk, pv, dt, L + 1, layout, Hq, Hkv, table, bs)
    assert np.array_equal(att, ref)


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_slots_equal_dense(layout):
    rng = np.random.default_rng(21)
    B, Hq, Hkv, D, S, R = 4, 8, 2, 16, 9, 7
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    kc = rng.standard_normal(shape).astype(np.float32)
    vc = rng.standard_normal(shape).astype(np.float32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    L = np.array([0, 3, 8, 5], np.int32)
    slots = np.array([6, 0, 3, 4], np.int32)
    ks, vs = to_slots(kc, layout, slots, R), to_slots(vc, layout, slots, R)
    ref, rk, rv = oracle.step(q, "f32", kc, vc, kn, vn, "f32", L, layout, Hq, Hkv)
    got, sk, sv = oracle.step_mapped("slots", q, "f32", ks, vs, kn, vn, "f32", L, layout, Hq, Hkv, slots)
    assert np.array_equal(got, ref)
    ek, ev = to_slots(rk, layout, slots, R), to_slots(rv, layout, slots, R)
    assert sk.tobytes() == ek.tobytes() and sv.tobytes() == ev.tobytes()


# ---------------------------------------------------------------------------
# Validation rules of the page: -1 pads allowed, entries in range, no block
# twice in one row (two rows may share one), slot rows distinct and in range.
# ---------------------------------------------------------------------------
def test_table_validation():
    oracle.validate_table(np.array([[0, 1, -1], [2, 3, -1]]), 4)
    oracle.validate_table(np.array([[0, 1], [0, 1]]), 2)          # shared across rows: allowed
    for bad in ([[0, 4]], [[0, -2]], [[1, 1]], [[0, -1, 0]]):
        with pytest.raises(ValueError):
            oracle.validate_table(np.array(bad), 4)


def test_slot_validation():
    oracle.validate_slots(np.array([2, 0, 1]), 3)
    for bad in ([3], [-1], [1, 1]):
        with pytest.raises(ValueError):
            oracle.validate_slots(np.array(bad), 3)


def test_token_in_unmapped_block_raises():
    pool = np.zeros((2, 1, 2, 4), np.float32)
    q = np.zeros((1, 1, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attend_mapped("paged", q, "f32", pool, pool, "f32", np.array([3]), "BHSD", 1, 1,
                             np.array([[0, -1]], np.int32), 2)


# ---------------------------------------------------------------------------
# Int8 caches with per-row scales through a map (the CLIKA page lists kScale /
# vScale beside slot_ids and the block table).  Pins: the JAX page's printed
# examples, whose cached values are small integers, stored as codes with
# scales 1 or 1/2 (exact) in permuted rows / scattered blocks whose other
# scales are NaN; and equality with the dense int8 oracle on the same logical
# cache, appended codes and scales included.
# ---------------------------------------------------------------------------
def _q8_of(values):
    """Exact int8 codes and float32 scales for integer-valued rows: code = v and
    scale 1, or code = 2v and scale 1/2 where that fits."""
    v = np.asarray(values, dtype=np.float64)
    fits = (np.abs(v).max(axis=-1) * 2 <= 127)
    scale = np.where(fits, 0.5, 1.0).astype(np.float32)
    codes = np.rint(v / scale[..., None]).astype(np.int8)
    assert np.array_equal(codes.astype(np.float64) * scale[..., None], v)
    return codes, scale


def _scatter_q8(codes, scales, layout, kind, rng, bs=None):
    """Codes (B, .., D) and scales (B, ..) of a dense cache stored through a map.
    Unmapped rows / blocks: codes 127, scales NaN.  Returns (codes, scales, map)."""
    if layout == "BHSD":
        B, Hkv, S, D = codes.shape
    else:
        B, S, Hkv, D = codes.shape
    if kind == "slots":
        R = 2 * B + 1
        slot_ids = rng.permutation(R)[:B].astype(np.int32)
        c = np.full((R,) + codes.shape[1:], 127, np.int8)
        s = np.full((R,) + scales.shape[1:], np.nan, np.float32)
        c[slot_ids], s[slot_ids] = codes, scales
        return c, s, slot_ids
    nb = -(-S // bs)
    total = B * nb + 3
    table = rng.permutation(total)[: B * nb].reshape(B, nb).astype(np.int32)
    pshape = (total, Hkv, bs) if layout == "BHSD" else (total, bs, Hkv)
    c = np.full(pshape + (D,), 127, np.int8)
    s = np.full(pshape, np.nan, np.float32)
    for b in range(B):
        for j in range(S):
            for h in range(Hkv):
                src = (b, h, j) if layout == "BHSD" else (b, j, h)
                dst = oracle.slot_location("paged", layout, table, b, h, j, bs)
                c[dst], s[dst] = codes[src], scales[src]
    return c, s, table


@pytest.mark.parametrize("kind,bs", [("slots", None), ("paged", 1), ("paged", 3)])
@pytest.mark.parametrize("case", P2["cases"], ids=[c["name"] for c in P2["cases"]])
def test_jax_page_examples_int8_through_maps(case, kind, bs):
    q = f32(case["query"])
    kc, ks = _q8_of(case["key_cache"])                            # (B, S, Hkv, D) codes, (B, S, Hkv) scales
    vc, vs = _q8_of(case["value_cache"])
    S = kc.shape[1]
    if bs is not None and S % bs:
        pytest.skip("capacity not a multiple of the block size")
    kcm, ksm, m = _scatter_q8(kc, ks, "BSHD", kind, np.random.default_rng(17), bs)
    vcm, vsm, m2 = _scatter_q8(vc, vs, "BSHD", kind, np.random.default_rng(17), bs)
    assert np.array_equal(m, m2)
    out = oracle.attend_q8_mapped(kind, q, "f32", kcm, vcm, ksm, vsm, np.array(case["lengths"]), "BSHD",
                                  case["num_query_heads"], case["num_kv_heads"], m, bs)
    exp, tol = _printed(case["output"])
    assert np.all(np.abs(out - exp) <= tol + 1e-7)


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
@pytest.mark.parametrize("kind,bs", [("slots", None), ("paged", 1), ("paged", 4), ("paged", 16)])
def test_int8_mapped_step_equals_dense_int8_step(layout, kind, bs):
    rng = np.random.default_rng(23)
    B, Hkv, G, S, D = 3, 2, 3, 37, 8
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    kc = rng.integers(-127, 128, shape).astype(np.int8)
    vc = rng.integers(-127, 128, shape).astype(np.int8)
    ks = (rng.random(shape[:3]) + 0.5).astype(np.float32) / np.float32(40)
    vs = (rng.random(shape[:3]) + 0.5).astype(np.float32) / np.float32(40)
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float32)
    kn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    vn = rng.standard_normal((B, Hkv, D)).astype(np.float32)
    L = np.array([0, 17, S - 1], np.int32)
    want = oracle.step_q8(q, "f32", kc, vc, ks, vs, kn, vn, L, layout, Hkv * G, Hkv)
    S_map = S if bs is None else -(-S // bs) * bs
    if bs is not None and S_map != S:       # pad the logical capacity to whole blocks
        pad = [(0, 0)] * 4
        pad[2 if layout == "BHSD" else 1] = (0, S_map - S)
        kc, vc = np.pad(kc, pad), np.pad(vc, pad)
        ks, vs = np.pad(ks, pad[:3], constant_values=1.0), np.pad(vs, pad[:3], constant_values=1.0)
    kcm, ksm, m = _scatter_q8(kc, ks, layout, kind, np.random.default_rng(29), bs)
    vcm, vsm, _ = _scatter_q8(vc, vs, layout, kind, np.random.default_rng(29), bs)
    got = oracle.step_q8_mapped(kind, q, "f32", kcm, vcm, ksm, vsm, kn, vn, L, layout, Hkv * G, Hkv, m, bs)
    assert np.array_equal(got[0], want[0])
    for b in range(B):                       # the appended codes and scales sit at the mapped location
        for h in range(Hkv):
            src = (b, h, int(L[b])) if layout == "BHSD" else (b, int(L[b]), h)
            dst = oracle.slot_location(kind, layout, m, b, h, int(L[b]), bs)
            assert np.array_equal(got[1][dst], want[1][src]) and np.array_equal(got[2][dst], want[2][src])
            assert got[3][dst] == want[3][src] and got[4][dst] == want[4][src]

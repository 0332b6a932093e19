"""Pins of the oracle's fp8 (OCP E4M3) caches: the code itself, the quantizing
rule of its rows, and the attention over them.

The pages define no fp8 format; the reading (oracle/fp8.py) is the OCP E4M3
format with the pages' row rule (CANN "aclnnMlaPrologV3WeightNz" page,
dynamic-quantization formula) taken over with the format's largest value, 448,
in place of 127.  The code is pinned against an independent implementation of
the same format (torch.float8_e4m3fn: every code decoded, hundreds of
thousands of values encoded, every rounding tie) and against hand-derived
values; the row rule by exact rows and the rounding error bound; the attention
by reduction to the dense oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import E4M3_MAX, decode_e4m3, encode_e4m3
from oracle.quant import quantize_row

ALL = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    d, t = decode_e4m3(ALL), torch_decode(ALL)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    f = ~np.isnan(d)
    assert np.array_equal(d[f], t[f]) and np.array_equal(np.signbit(d[f]), np.signbit(t[f]))
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.sum(np.isnan(d)) == 2


def test_decode_closed_forms():
    cases = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x78: 256.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in cases.items():
        assert decode_e4m3(np.array([c], np.uint8))[0] == v, hex(c)
    z = decode_e4m3(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and np.signbit(z)


def test_encode_round_trips_every_finite_code():
    fin = ALL[~np.isnan(decode_e4m3(ALL))]
    assert np.array_equal(encode_e4m3(decode_e4m3(fin)), fin)


def test_encode_matches_torch_on_ties_and_random_values():
    mags = np.unique(np.abs(decode_e4m3(ALL)[~np.isnan(decode_e4m3(ALL))]))
    mids = (mags[1:] + mags[:-1]) / 2                       # every tie between neighbours (exact in f32)
    rng = np.random.default_rng(7)
    xs = [mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
          np.nextafter(mids.astype(np.float32), np.float32(1000)),
          rng.uniform(-448, 448, 200000), rng.uniform(-0.02, 0.02, 100000), rng.normal(0, 3, 100000)]
    x = np.clip(np.concatenate([np.asarray(a, np.float32) for a in xs]), -448, 448).astype(np.float32)
    assert np.array_equal(encode_e4m3(x), torch_encode(x))


def test_encode_ties_go_to_the_even_code_by_hand():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): the even code 0x38.
    # 1.1875 between 1.125 (0x39) and 1.25 (0x3A): 0x3A.  1.5 * 2^-9 between the
    # subnormals 1 and 2 (x 2^-9): code 0x02.  2^-10: halfway to zero: 0x00.
    x = np.array([1.0625, 1.1875, 1.5 * 2.0 ** -9, 2.0 ** -10, -1.0625, 432.0, 440.0], np.float32)
    assert encode_e4m3(x).tolist() == [0x38, 0x3A, 0x02, 0x00, 0xB8, 0x7E, 0x7E]
    # 432 is halfway between 416 (0x7D) and 448 (0x7E): even 0x7E; 440 nearer 448.


def test_encode_refuses_out_of_range():
    with pytest.raises(ValueError):
        encode_e4m3(np.array([448.5], np.float32))
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.nan], np.float32))


def test_quantize_row_fp8_exact_row():
    # amax 448 * 2^-3 gives scale 2^-3 exactly; every quotient is exact.
    s = 2.0 ** -3
    row = np.array([448, -448, 1, 0.5, 2.0 ** -6, 1.5 * 2.0 ** -9, 1.0625, 0, -0.0], np.float64) * s
    codes, scale = quantize_row(row.astype(np.float32), "fp8")
    assert scale == np.float32(s)
    assert codes.tolist() == [0x7E, 0xFE, 0x38, 0x30, 0x08, 0x02, 0x38, 0x00, 0x80]


def test_quantize_row_fp8_zero_row():
    codes, scale = quantize_row(np.zeros(16, np.float32), "fp8")
    assert scale == 0 and codes.dtype == np.uint8 and not codes.any()


def test_quantize_row_fp8_error_bound_and_row_maximum():
    rng = np.random.default_rng(11)
    for _ in range(200):
        x = (rng.normal(0, 1, 128) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        codes, scale = quantize_row(x, "fp8")
        q = np.abs(x.astype(np.float64) / np.float64(scale))
        # E4M3 spacing at magnitude q: 2^(floor(log2 q) - 3) for normals, 2^-9 below 2^-6.
        spacing = np.where(q >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3), 2.0 ** -9)
        err = np.abs(decode_e4m3(codes) * np.float64(scale) - x)
        assert np.all(err <= (0.5 * spacing * (1 + 1e-6) + 1e-7 * q) * scale)
        assert (codes[np.argmax(np.abs(x))] & 0x7F) == 0x7E      # the row maximum reads as 448


def _fp8_inputs(B, Hkv, G, S, D, layout, seed):
    rng = np.random.default_rng(seed)
    shape = (B, Hkv, S, D) if layout == "BHSD" else (B, S, Hkv, D)
    sshape = shape[:3]
    fin = ALL[~np.isnan(decode_e4m3(ALL))]
    kc = rng.choice(fin, size=shape).astype(np.uint8)
    vc = rng.choice(fin, size=shape).astype(np.uint8)
    ks = (2.0 ** rng.integers(-10, -6, size=sshape)).astype(np.float32)    # powers of two: exact products
    vs = (2.0 ** rng.integers(-10, -6, size=sshape)).astype(np.float32)
    q = rng.normal(0, 1, (B, Hkv * G, D)).astype(np.float32)
    return q, kc, vc, ks, vs


@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_attend_on_fp8_rows_equals_the_dense_oracle(layout):
    B, Hkv, G, S, D = 3, 2, 3, 9, 8
    q, kc, vc, ks, vs = _fp8_inputs(B, Hkv, G, S, D, layout, 3)
    L = np.array([9, 4, 1], np.int32)
    got = oracle.attend_q8(q, "f32", kc, vc, ks, vs, L, layout, Hkv * G, Hkv)
    kd = (decode_e4m3(kc) * ks[..., None]).astype(np.float32)            # exact in f32
    vd = (decode_e4m3(vc) * vs[..., None]).astype(np.float32)
    ref = oracle.attend(q, "f32", kd, vd, "f32", L, layout, Hkv * G, Hkv)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_fp8_step_changes_exactly_one_row_and_quantizes_it():
    B, Hkv, G, S, D = 2, 2, 2, 6, 8
    q, kc, vc, ks, vs = _fp8_inputs(B, Hkv, G, S, D, "BHSD", 5)
    rng = np.random.default_rng(6)
    kn = rng.normal(0, 2, (B, Hkv, D)).astype(np.float32)
    vn = rng.normal(0, 2, (B, Hkv, D)).astype(np.float32)
    L = np.array([2, 5], np.int32)
    out, k2, v2, ks2, vs2 = oracle.step_q8(q, "f32", kc, vc, ks, vs, kn, vn, L, "BHSD", Hkv * G, Hkv)
    for b in range(B):
        for h in range(Hkv):
            ck, sk = quantize_row(kn[b, h], "fp8")
            assert np.array_equal(k2[b, h, L[b]], ck) and ks2[b, h, L[b]] == sk
            mask = np.ones(S, bool)
            mask[L[b]] = False
            assert np.array_equal(k2[b, h, mask], kc[b, h, mask]) and np.array_equal(vs2[b, h, mask], vs[b, h, mask])
    assert np.all(np.isfinite(out))


def test_fp8_mapped_step_equals_the_dense_fp8_step():
    B, Hkv, G, S, D, bs = 2, 2, 2, 8, 8, 3
    q, kc, vc, ks, vs = _fp8_inputs(B, Hkv, G, S, D, "BHSD", 9)
    rng = np.random.default_rng(10)
    kn = rng.normal(0, 1, (B, Hkv, D)).astype(np.float32)
    vn = rng.normal(0, 1, (B, Hkv, D)).astype(np.float32)
    L = np.array([7, 3], np.int32)
    out, k2, v2, ks2, vs2 = oracle.step_q8(q, "f32", kc, vc, ks, vs, kn, vn, L, "BHSD", Hkv * G, Hkv)
    # The same logical caches in a pool of 3-slot blocks, rows of a sequence in a shuffled block order.
    mb = -(-S // bs)
    perm = rng.permutation(B * mb)
    table = perm.reshape(B, mb).astype(np.int32)
    pool = lambda c, fill: np.full((B * mb, Hkv, bs) + c.shape[3:], fill, c.dtype)
    pk, pv = pool(kc, 0x7F), pool(vc, 0x7F)                                # NaN codes where no row maps
    pks = np.full((B * mb, Hkv, bs), np.nan, np.float32)
    pvs = np.full((B * mb, Hkv, bs), np.nan, np.float32)
    for b in range(B):
        for j in range(mb * bs):
            if j >= S:
                continue
            blk, off = table[b, j // bs], j % bs
            pk[blk, :, off], pv[blk, :, off] = kc[b, :, j], vc[b, :, j]
            pks[blk, :, off], pvs[blk, :, off] = ks[b, :, j], vs[b, :, j]
    got = oracle.step_q8_mapped("paged", q, "f32", pk, pv, pks, pvs, kn, vn, L, "BHSD", Hkv * G, Hkv, table, bs)
    assert np.allclose(got[0], out, rtol=0, atol=1e-12)

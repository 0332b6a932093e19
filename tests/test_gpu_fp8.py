"""GPU parity for fp8 caches: OCP E4M3 codes with per-row float32 scales.

The pages define no fp8 format; the reading (oracle/fp8.py) takes the pages'
row rule (CANN "aclnnMlaPrologV3WeightNz" page, dynamic-quantization formula)
over to E4M3 codes with 448, the code's largest value, in place of 127.  The
library's _q8 calls on float8_e4m3fn caches against the float64 oracle on the
same stored bits: codes and scales of the appended rows byte-exact (the code is
an integer decision taken in float32 on both sides), every code decoded
exactly, outputs within the bf16 tolerance (1e-2 abs + rel).  Scales of the
slots past lengths[b] are NaN, so any read outside the valid slots shows up.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 1e-2}
DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_amd as lib
    lib.lib()
    return lib


def say(*a):
    print(*a, flush=True)


def np_of(t):
    return W.to_numpy_storage(t)


def assert_close(out_gpu, ref, qo_dtype, what=""):
    got = out_gpu.detach().float().cpu().double().numpy()
    tol = TOL[qo_dtype]
    err = np.abs(got - ref)
    bound = tol + tol * np.abs(ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst excess "
                           f"{np.max(err - bound):.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def assert_same_bytes(got, want, what):
    g_ = np_of(got)
    if g_.tobytes() != want.tobytes():
        bad = np.argwhere(g_.view(np.uint8).reshape(g_.shape + (-1,)) != want.view(np.uint8).reshape(g_.shape + (-1,)))
        raise AssertionError(f"{what}: {len(bad)} bytes differ, first at {bad[:3].tolist()}")


def codes_tensor(codes_u8):
    return torch.from_numpy(np.ascontiguousarray(codes_u8, dtype=np.uint8)).view(torch.float8_e4m3fn)


def test_fp8_every_code_decodes_exactly(g):
    """Attention over one valid slot returns that slot's value row: with scale 1
    each output element is the decoded code itself, exactly representable in
    bf16.  Two sequences x two kv-heads x 128 elements carry all 256 codes twice
    (the two NaN patterns replaced by +-0), so every code's decoding is compared
    exactly.  (The V sum starts from +0, so the code of -0 reads back as +0: an
    attention output's zero has no sign to compare.)"""
    B, Hkv, D, S = 2, 2, 128, 16
    codes = np.tile(np.arange(256, dtype=np.uint8), 2)
    codes[(codes & 0x7F) == 0x7F] &= 0x80
    w = W.custom(B, Hkv, Hkv, D, S, "BHSD", "fp8", "bf16", seed=51, stale="pm:1")
    L = torch.ones(B, dtype=torch.int32)
    inp = W.make_q8(w, DEV, lengths=L)
    vc = np_of(inp["v_cache"]).copy()
    vc[:, :, 0, :] = codes.reshape(B, Hkv, D)
    inp["v_cache"] = codes_tensor(vc).to(DEV)
    inp["v_scale"][:, :, 0] = 1.0
    desc = g.make_desc(B, Hkv, Hkv, D, S, "BHSD", g.FP8, g.BF16)
    assert g.get_plan(desc)["kernel"] == "mfma_qk"
    out = g.attend_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["lengths"],
                      layout="BHSD")
    torch.cuda.synchronize()
    want = torch.from_numpy(oracle.decode_e4m3(codes)).to(torch.bfloat16).reshape(B, Hkv, D)
    got = out.cpu()
    assert torch.equal(got.float(), want.float()), \
        [(int(c), float(a), float(b)) for c, a, b in zip(codes, got.flatten(), want.flatten()) if float(a) != float(b)][:8]


CASES = [
    # B, Hq, Hkv, D, S, layout, qo, num_splits
    (3, 32, 8, 128, 1500, "BHSD", "bf16", 0),      # Llama-like group of 4
    (3, 32, 8, 128, 900, "BSHD", "bf16", 0),       # four kv-heads per workgroup (BSHD)
    (2, 16, 2, 128, 700, "BSHD", "bf16", 3),       # G=8, forced splits
    (4, 16, 16, 128, 300, "BHSD", "bf16", 0),      # G=1
    (2, 64, 1, 128, 900, "BHSD", "bf16", 0),       # G=64: two 16-head blocks per wave, two head chunks
    (3, 48, 2, 128, 600, "BSHD", "bf16", 2),       # G=24: one partly used head block
    (2, 64, 1, 128, 700, "BHSD", "bf16", 3),       # G=64, forced splits
]


def _ids(c):
    return f"B{c[0]}Hq{c[1]}Hkv{c[2]}S{c[4]}{c[5]}n{c[7]}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_fp8_step_and_attend(g, case):
    B, Hq, Hkv, D, S, layout, qo, ns = case
    w = W.custom(B, Hq, Hkv, D, S, layout, "fp8", qo, seed=B * 100 + Hq + S, stale="pm:1")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(S + 11), dtype=torch.int32)
    L[0] = S - 1                          # a full sequence
    if B > 2:
        L[1] = 0                          # only the new token
    inp = W.make_q8(w, DEV, lengths=L)
    say(f"fp8 step {_ids(case)} plan {g.get_plan(g.make_desc(B, Hq, Hkv, D, S, layout, g.FP8, g.BF16, ns))}")
    ref, rk, rv, rks, rvs = oracle.step_q8(np_of(inp["q"]), qo, np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                           np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                           np_of(inp["v_new"]), L.numpy(), layout, Hq, Hkv)
    out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                    inp["v_new"], inp["lengths"], layout=layout, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, qo, "step")
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")
    n = (inp["lengths"] + 1).contiguous()
    out2 = g.attend_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], n, layout=layout,
                       num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out2, ref, qo, "attend")


# Row values whose quotient x / scale is exact (scale 1: the row's largest
# magnitude is 448) and lands on E4M3 rounding ties or special codes: 1.0625
# (tie of 0x38 / 0x39 -> 0x38), 1.1875 (-> 0x3A), 1.5 * 2^-9 (subnormal tie ->
# 0x02), 2^-10 (tie with zero -> 0x00), 432 (tie of 416 / 448 -> 0x7E), -0.0
# (-> 0x80), and their negations.
TIE = [448.0, 1.0625, 1.1875, 1.5 * 2.0 ** -9, 2.0 ** -10, 432.0, -0.0, -1.0625, -1.1875, -1.5 * 2.0 ** -9,
       -(2.0 ** -10), -432.0, 0.0, 3.0, -448.0, 2.0 ** -6]
TIE_CODES = [0x7E, 0x38, 0x3A, 0x02, 0x00, 0x7E, 0x80, 0xB8, 0xBA, 0x82, 0x80, 0xFE, 0x00, 0x44, 0xFE, 0x08]


@pytest.mark.parametrize("Hq", [8, 64], ids=["G4-one-head-block", "G32-two-head-blocks"])
def test_fp8_step_quantizes_ties_and_zero_rows_in_kernel(g, Hq):
    B, Hkv, D, S = 3, 2, 128, 200
    w = W.custom(B, Hq, Hkv, D, S, "BHSD", "fp8", "bf16", seed=53, stale="pm:1")
    L = torch.tensor([0, 57, S - 1], dtype=torch.int32)
    inp = W.make_q8(w, DEV, lengths=L)
    tie = torch.tensor(TIE, dtype=torch.float32).repeat(D // 16)
    inp["k_new"][0, 0] = tie.to(torch.bfloat16).to(DEV)
    inp["k_new"][1, 1] = (-tie).to(torch.bfloat16).to(DEV)
    inp["v_new"][2, 0] = 0
    inp["v_new"][1, 0] = tie.to(torch.bfloat16).to(DEV)
    ref, rk, rv, rks, rvs = oracle.step_q8(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                           np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                           np_of(inp["v_new"]), L.numpy(), "BHSD", Hq, Hkv)
    assert rks[0, 0, 0] == 1.0 and list(rk[0, 0, 0, :16]) == TIE_CODES       # the oracle's own rounding
    assert rvs[2, 0, S - 1] == 0.0 and not rv[2, 0, S - 1].any()
    out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                    inp["v_new"], inp["lengths"], layout="BHSD")
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "fp8 step")
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")


@pytest.mark.parametrize("qo,D", [("f32", 16), ("bf16", 16), ("bf16", 24)])
def test_fp8_append_alone_with_ties_and_zero_rows(g, qo, D):
    """The append entry point quantizes rows of any width (it runs no attention)."""
    w = W.custom(3, 4, 2, D, 20, "BHSD", "fp8", qo, seed=57, stale="pm:1")
    L = torch.tensor([0, 7, 19], dtype=torch.int32)
    inp = W.make_q8(w, DEV, lengths=L)
    tie = torch.tensor((TIE * 2)[:D], dtype=torch.float32)
    inp["k_new"][0, 0] = tie.to(inp["k_new"].dtype).to(DEV)
    inp["v_new"][0, 1] = 0
    inp["k_new"][1, 0] = (-tie).to(inp["k_new"].dtype).to(DEV)
    rk, rv, rks, rvs = oracle.append_q8(np_of(inp["k_cache"]), np_of(inp["v_cache"]), np_of(inp["k_scale"]),
                                        np_of(inp["v_scale"]), np_of(inp["k_new"]), np_of(inp["v_new"]), qo,
                                        L.numpy(), "BHSD")
    assert rks[0, 0, 0] == 1.0 and list(rk[0, 0, 0, :16]) == TIE_CODES
    g.append_q8(inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"], inp["v_new"],
                inp["lengths"], layout="BHSD")
    torch.cuda.synchronize()
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")


@pytest.mark.parametrize("kind,bs", [("paged", 16), ("slots", 0)])
def test_fp8_mapped_step(g, kind, bs):
    B, Hq, Hkv, D, S = 3, 32, 8, 128, 400
    w = W.custom(B, Hq, Hkv, D, S, "BSHD", "fp8", "bf16", seed=59, stale="pm:1")
    L = torch.tensor([S - 1, 0, 123], dtype=torch.int32)
    inp = W.make_q8(w, DEV, lengths=L)
    m = W.make_mapped(inp, w, kind, block_size=bs or 16)
    table = m["map"]
    host = {k: np_of(m[k]) for k in ("k_cache", "v_cache", "k_scale", "v_scale")}
    ref = oracle.step_q8_mapped(kind, np_of(inp["q"]), "bf16", host["k_cache"], host["v_cache"], host["k_scale"],
                                host["v_scale"], np_of(inp["k_new"]), np_of(inp["v_new"]), L.numpy(), "BSHD", Hq, Hkv,
                                table.cpu().numpy(), bs if kind == "paged" else None)
    out = g.step_ex(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout="BSHD",
                    table=table, kind=kind, table_host=table.cpu(), k_scale=m["k_scale"], v_scale=m["v_scale"])
    torch.cuda.synchronize()
    assert_close(out, ref[0], "bf16", f"fp8 {kind}")
    assert_same_bytes(m["k_cache"], ref[1], "k codes")
    assert_same_bytes(m["v_cache"], ref[2], "v codes")
    assert_same_bytes(m["k_scale"], ref[3], "k scales")
    assert_same_bytes(m["v_scale"], ref[4], "v scales")


@pytest.mark.parametrize("name", ["llama3_8b_layer", "ragged_batch", "long_context", "large_group"])
def test_fp8_full_size_workload(g, name):
    """A full-size workload on fp8 caches in the benchmark's launch
    configuration: every output against the oracle, and every byte of the code
    and scale caches against the oracle's quantizing append."""
    base = W.WORKLOADS[name]
    w = W.custom(base.B, base.Hq, base.Hkv, base.D, base.capacity, base.layout, "fp8", "bf16", seed=base.seed,
                 stale=base.stale, key_scale=base.key_scale)
    L = W.draw_lengths(base)
    inp = W.make_q8(w, DEV, lengths=L)
    desc = g.make_desc(w.B, w.Hq, w.Hkv, w.D, w.capacity, w.layout, g.FP8, g.BF16)
    say(f"fp8 full size {name}: plan {g.get_plan(desc)}")
    host = {k: np_of(v) for k, v in inp.items() if k != "lengths"}
    out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                    inp["v_new"], inp["lengths"], layout=w.layout)
    torch.cuda.synchronize()
    ref, rk, rv, rks, rvs = oracle.step_q8(host["q"], "bf16", host["k_cache"], host["v_cache"], host["k_scale"],
                                           host["v_scale"], host["k_new"], host["v_new"], L.numpy(), w.layout, w.Hq,
                                           w.Hkv)
    del host
    assert_close(out, ref, "bf16", f"fp8 {name}")
    assert torch.isfinite(out.float()).all()
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")

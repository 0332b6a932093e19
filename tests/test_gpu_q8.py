"""GPU parity for int8 caches with per-row scales (Huawei CANN
"aclnnMlaPrologV3WeightNz" page, dynamic-quantization formula).

The library's _q8 step/attend/append against the float64 int8 oracle on the
same stored bits: codes and scales of the appended rows byte-exact (the
quantization is an integer decision taken in float32 on both sides), outputs
within the dense tolerances (fp32 2e-5, bf16 1e-2, abs + rel).  Scales of the
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


CASES = [
    # B, Hq, Hkv, D, S, layout, qo, num_splits
    (3, 32, 8, 128, 1500, "BHSD", "bf16", 0),      # Llama-like group of 4
    (2, 16, 2, 128, 700, "BSHD", "bf16", 3),       # G=8, forced splits
    (2, 64, 1, 128, 900, "BHSD", "bf16", 0),       # G=64
    (3, 8, 2, 64, 300, "BHSD", "f32", 0),          # float32 activations
    (2, 6, 3, 24, 200, "BSHD", "f32", 2),          # D not a multiple of 16: element loads
    (2, 4, 1, 256, 100, "BHSD", "bf16", 0),        # largest head
    (4, 8, 8, 80, 64, "BSHD", "bf16", 0),          # G=1
    (2, 8, 2, 7, 50, "BHSD", "f32", 0),            # odd head_dim
    (3, 48, 2, 128, 600, "BSHD", "bf16", 2),       # G=24 on the large-group kernel (one partly used head block)
    (2, 64, 1, 128, 700, "BHSD", "bf16", 3),       # G=64, forced splits
]


def _ids(c):
    return f"B{c[0]}Hq{c[1]}Hkv{c[2]}D{c[3]}S{c[4]}{c[5]}{c[6]}n{c[7]}"


def _inputs(case, seed_extra=0):
    B, Hq, Hkv, D, S, layout, qo, ns = case
    w = W.custom(B, Hq, Hkv, D, S, layout, "i8", qo, seed=B * 100 + D + seed_extra, stale="pm:1")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(S + 7), dtype=torch.int32)
    L[0] = S - 1                          # a full sequence
    if B > 2:
        L[1] = 0                          # only the new token
    return w, L, W.make_q8(w, DEV, lengths=L)


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_q8_step_and_attend(g, case):
    B, Hq, Hkv, D, S, layout, qo, ns = case
    w, L, inp = _inputs(case)
    say(f"q8 step {_ids(case)}")
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


@pytest.mark.parametrize("qo", ["f32", "bf16"])
def test_q8_append_alone_with_ties_and_zero_rows(g, qo):
    """Rows built so that x / scale lands exactly on .5 (scale = 1 when the
    row's largest magnitude is 127), a zero row (scale 0, codes 0), and a row
    whose largest entry is negative; the other rows are random."""
    w = W.custom(3, 4, 2, 16, 20, "BHSD", "i8", qo, seed=41, stale="pm:1")
    L = torch.tensor([0, 7, 19], dtype=torch.int32)
    inp = W.make_q8(w, DEV, lengths=L)
    tie = torch.tensor([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 126.5, -126.5, 0, 4.5, 5.5, -3.5, 1, 2],
                       dtype=torch.float32)
    inp["k_new"][0, 0] = tie.to(inp["k_new"].dtype).to(DEV)
    inp["v_new"][0, 1] = 0
    inp["k_new"][1, 0] = (-tie).to(inp["k_new"].dtype).to(DEV)
    rk, rv, rks, rvs = oracle.append_q8(np_of(inp["k_cache"]), np_of(inp["v_cache"]), np_of(inp["k_scale"]),
                                        np_of(inp["v_scale"]), np_of(inp["k_new"]), np_of(inp["v_new"]), qo,
                                        L.numpy(), "BHSD")
    assert rks[0, 0, 0] == 1.0 and list(rk[0, 0, 0, :4]) == [127, 0, 2, 2]      # the oracle rounds half to even
    g.append_q8(inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"], inp["v_new"],
                inp["lengths"], layout="BHSD")
    torch.cuda.synchronize()
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")


@pytest.mark.parametrize("Hq", [8, 64], ids=["G4-one-head-block", "G32-two-head-blocks"])
def test_q8_step_quantizes_ties_and_zero_rows_in_kernel(g, Hq):
    """The matrix-core kernels quantize a step's new rows themselves: rows
    whose x / scale lands exactly on .5 (largest magnitude 127, so scale 1),
    their negation, and a zero value row (scale 0, codes 0) must give the
    oracle's codes and scales bit for bit, and the attention over them its
    output."""
    B, Hkv, D, S = 3, 2, 128, 200
    w = W.custom(B, Hq, Hkv, D, S, "BHSD", "i8", "bf16", seed=43, stale="pm:1")
    L = torch.tensor([0, 57, S - 1], dtype=torch.int32)
    inp = W.make_q8(w, DEV, lengths=L)
    tie = torch.tensor([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 126.5, -126.5, 0, 4.5, 5.5, -3.5, 1, 2],
                       dtype=torch.float32).repeat(D // 16)
    inp["k_new"][0, 0] = tie.to(torch.bfloat16).to(DEV)
    inp["k_new"][1, 1] = (-tie).to(torch.bfloat16).to(DEV)
    inp["v_new"][2, 0] = 0
    inp["v_new"][1, 0] = tie.to(torch.bfloat16).to(DEV)
    desc = g.make_desc(B, Hq, Hkv, D, S, "BHSD", g.I8, g.BF16)
    assert g.get_plan(desc)["kernel"] == "mfma_qk"
    assert g.get_plan(desc)["block"] == (256 if Hq // Hkv <= 16 else 512)
    ref, rk, rv, rks, rvs = oracle.step_q8(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                           np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                           np_of(inp["v_new"]), L.numpy(), "BHSD", Hq, Hkv)
    assert rks[0, 0, 0] == 1.0 and list(rk[0, 0, 0, :4]) == [127, 0, 2, 2]      # the oracle rounds half to even
    assert rvs[2, 0, S - 1] == 0.0
    out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                    inp["v_new"], inp["lengths"], layout="BHSD")
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "int8 step")
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")


@pytest.mark.parametrize("name", ["llama3_8b_layer", "ragged_batch", "long_context", "large_group"])
def test_q8_full_size_workload(g, name):
    """A full-size workload on int8 caches in the benchmark's launch
    configuration (the same shape, layout and lengths; codes and scales drawn by
    make_q8, NaN scales past each sequence's slots where the workload has a
    stale filler): every output against the oracle, and every byte of the code
    and scale caches against the oracle's quantizing append."""
    base = W.WORKLOADS[name]
    w = W.custom(base.B, base.Hq, base.Hkv, base.D, base.capacity, base.layout, "i8", "bf16", seed=base.seed,
                 stale=base.stale, key_scale=base.key_scale)
    L = W.draw_lengths(base)
    inp = W.make_q8(w, DEV, lengths=L)
    desc = g.make_desc(w.B, w.Hq, w.Hkv, w.D, w.capacity, w.layout, g.I8, g.BF16)
    say(f"int8 full size {name}: plan {g.get_plan(desc)}")
    host = {k: np_of(v) for k, v in inp.items() if k != "lengths"}
    out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                    inp["v_new"], inp["lengths"], layout=w.layout)
    torch.cuda.synchronize()
    ref, rk, rv, rks, rvs = oracle.step_q8(host["q"], "bf16", host["k_cache"], host["v_cache"], host["k_scale"],
                                           host["v_scale"], host["k_new"], host["v_new"], L.numpy(), w.layout, w.Hq,
                                           w.Hkv)
    del host
    assert_close(out, ref, "bf16", f"int8 {name}")
    assert torch.isfinite(out.float()).all()
    assert_same_bytes(inp["k_cache"], rk, "k codes")
    assert_same_bytes(inp["v_cache"], rv, "v codes")
    assert_same_bytes(inp["k_scale"], rks, "k scales")
    assert_same_bytes(inp["v_scale"], rvs, "v scales")

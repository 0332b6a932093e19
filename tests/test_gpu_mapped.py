"""GPU parity for mapped caches: slot-indexed rows and paged block pools
(CLIKA runtime "groupQueryAttention" API page, slot_ids and block-table notes).

The library's mapped step/attend/append against the float64 mapped oracle on
the same stored bits: outputs within the dense tolerances (fp32 2e-5, bf16 1e-2,
abs + rel), pools and slot caches byte-exact after the append.  Unmapped rows,
unmapped blocks and the slots past the capacity in each last block hold NaN, so
any read outside the mapped, valid slots shows up in the output.
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


CASES = [
    # B, Hq, Hkv, D, S, layout, kv, qo, kind, block_size, num_splits
    (3, 32, 8, 128, 1500, "BHSD", "bf16", "bf16", "paged", 16, 0),     # G=4 matrix-core kernel
    (3, 32, 8, 128, 1500, "BHSD", "bf16", "bf16", "paged", 64, 3),
    (2, 16, 2, 128, 700, "BSHD", "bf16", "bf16", "paged", 32, 0),      # G=8, (blocks, bs, Hkv, D) pool
    (2, 16, 1, 128, 500, "BSHD", "bf16", "bf16", "paged", 16, 5),      # G=16, several splits
    (2, 64, 1, 128, 900, "BHSD", "bf16", "bf16", "paged", 16, 0),      # G=64 shared-tile kernel
    (2, 48, 2, 128, 1000, "BSHD", "bf16", "bf16", "paged", 48, 2),     # G=24, block size 48
    (3, 8, 2, 64, 300, "BHSD", "f32", "f32", "paged", 7, 0),           # generic kernel, odd block size
    (2, 6, 3, 24, 200, "BSHD", "f32", "bf16", "paged", 1, 2),          # generic, one slot per block
    (2, 8, 2, 128, 333, "BHSD", "bf16", "f32", "paged", 8, 0),         # generic (f32 output), block 8
    (3, 32, 8, 128, 1500, "BHSD", "bf16", "bf16", "paged", 7, 0),      # matrix-core descriptor, block 7: generic
    (2, 16, 2, 128, 700, "BSHD", "bf16", "bf16", "paged", 24, 3),      # G=8, block 24: generic
    (2, 64, 1, 128, 900, "BHSD", "bf16", "bf16", "paged", 24, 0),      # G=64, block 24: generic
    (3, 32, 8, 128, 1500, "BHSD", "bf16", "bf16", "slots", None, 0),
    (2, 64, 1, 128, 900, "BSHD", "bf16", "bf16", "slots", None, 2),
    (3, 8, 2, 64, 300, "BHSD", "f32", "f32", "slots", None, 0),
]


def _ids(c):
    return f"{c[8]}{c[9] or ''}-B{c[0]}Hq{c[1]}Hkv{c[2]}D{c[3]}S{c[4]}{c[5]}{c[6]}{c[7]}n{c[10]}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_mapped_step_and_attend(g, case):
    B, Hq, Hkv, D, S, layout, kv, qo, kind, bs, ns = case
    w = W.custom(B, Hq, Hkv, D, S, layout, kv, qo, seed=B * 100 + D + (bs or 0), stale="pm:1000")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(S + 7), dtype=torch.int32)
    L[0] = S - 1                          # a full sequence
    if B > 2:
        L[1] = 0                          # only the new token
    inp = W.make_inputs(w, DEV, lengths=L)
    m = W.make_mapped(inp, w, kind, block_size=bs or 16)
    table = m["map"].cpu().numpy()
    say(f"mapped step {_ids(case)} capacity={m['capacity']}")
    pk, pv = np_of(m["k_cache"]), np_of(m["v_cache"])
    ref, rk, rv = oracle.step_mapped(kind, np_of(inp["q"]), qo, pk, pv, np_of(inp["k_new"]), np_of(inp["v_new"]), kv,
                                     L.numpy(), layout, Hq, Hkv, table, bs)
    out = g.step_mapped(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], m["map"],
                        kind=kind, layout=layout, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, qo, "step")
    assert np_of(m["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(m["v_cache"]).tobytes() == rv.tobytes()
    # attend over the appended caches with lengths + 1 gives the same softmax
    n = (inp["lengths"] + 1).contiguous()
    out2 = g.attend_mapped(inp["q"], m["k_cache"], m["v_cache"], n, m["map"], kind=kind, layout=layout,
                           num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out2, ref, qo, "attend")


@pytest.mark.parametrize("kind", ["slots", "paged"])
def test_mapped_append_alone(g, kind):
    w = W.custom(4, 8, 2, 40, 90, "BSHD", "f32", "f32", seed=77, stale="pm:1000")
    L = torch.tensor([0, 17, 89, 45], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    m = W.make_mapped(inp, w, kind, block_size=16)
    rk, rv = oracle.append_mapped(kind, np_of(m["k_cache"]), np_of(m["v_cache"]), np_of(inp["k_new"]),
                                  np_of(inp["v_new"]), L.numpy(), w.layout, m["map"].cpu().numpy(),
                                  m.get("block_size"))
    g.append_mapped(m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], m["map"], kind=kind,
                    layout=w.layout)
    torch.cuda.synchronize()
    assert np_of(m["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(m["v_cache"]).tobytes() == rv.tobytes()


def test_mapping_only_moves_bytes(g):
    """Two different block tables over the same logical caches give the same
    output bits (paged tiles start at multiples of 16 slots whatever the
    table); slot-indexed and dense runs agree within the tolerance."""
    w = W.custom(2, 32, 8, 128, 1024, "BHSD", "bf16", "bf16", seed=9)
    L = torch.tensor([1023, 400], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    outs = []
    for seed in (1, 2):
        mp = W.make_mapped(inp, w, "paged", block_size=64, seed=seed)
        outs.append(g.step_mapped(inp["q"], mp["k_cache"], mp["v_cache"], inp["k_new"], inp["v_new"],
                                  inp["lengths"], mp["map"], kind="paged", layout="BHSD"))
    ms = W.make_mapped(inp, w, "slots")
    slots = g.step_mapped(inp["q"], ms["k_cache"], ms["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                          ms["map"], kind="slots", layout="BHSD")
    dense = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                   layout="BHSD")
    torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    ref = dense.float().cpu().double().numpy()
    assert_close(outs[0], ref, "bf16", "paged vs dense")
    assert_close(slots, ref, "bf16", "slots vs dense")


def test_paged_full_size_llama_layer(g):
    """The Llama-like layer (B=32, 4096 cached + 1 new, bf16) on a 16-slot
    block pool, in the benchmark's launch configuration: sampled outputs
    against the oracle computed one head at a time, appended rows byte-exact."""
    w = W.WORKLOADS["llama3_8b_layer"]
    inp = W.make_inputs(w, DEV)
    m = W.make_mapped(inp, w, "paged", block_size=16)
    table = m["map"].cpu().numpy()
    out = g.step_mapped(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], m["map"],
                        kind="paged", layout=w.layout)
    torch.cuda.synchronize()
    L = inp["lengths"].cpu().numpy()
    q = oracle.decode(np_of(inp["q"]), "bf16")
    rng = np.random.default_rng(4)
    got = out.float().cpu().double().numpy()
    kpool, vpool = np_of(m["k_cache"]), np_of(m["v_cache"])
    knew = np_of(inp["k_new"])
    for _ in range(6):
        b, hq = int(rng.integers(w.B)), int(rng.integers(w.Hq))
        h = hq // (w.Hq // w.Hkv)
        n = int(L[b]) + 1
        # the appended row came from k_new/v_new; gather the logical rows from the pool after the step
        K = oracle.decode(oracle.mapped_rows(kpool, "paged", "BHSD", table, b, h, n, 16), "bf16")
        V = oracle.decode(oracle.mapped_rows(vpool, "paged", "BHSD", table, b, h, n, 16), "bf16")
        assert np.array_equal(K[-1], oracle.decode(knew[b, h], "bf16"))
        ref = oracle.attend_one(q[b, hq], K, V)
        err = np.abs(got[b, hq] - ref)
        assert np.all(err <= 1e-2 + 1e-2 * np.abs(ref)), (b, hq, err.max())


# ---------------------------------------------------------------------------
# Int8 caches with per-row scales through a map (the CLIKA page lists kScale /
# vScale beside slot_ids and the block table): codes and scales stored through
# the same map, the scales of stale, unmapped and padding rows NaN (so a read
# of any of them shows in the output); appended codes and scales byte-exact.
# ---------------------------------------------------------------------------
Q8_CASES = [
    # B, Hq, Hkv, S, layout, kind, block_size, num_splits, expected kernel
    (3, 32, 8, 1000, "BHSD", "paged", 16, 0, "mfma_qk"),     # one 16-head block per wave
    (2, 16, 2, 700, "BSHD", "paged", 32, 3, "mfma_qk"),
    (2, 64, 1, 900, "BHSD", "paged", 16, 0, "mfma_qk"),      # two 16-head blocks per wave
    (2, 48, 2, 600, "BSHD", "slots", None, 0, "mfma_qk"),
    (3, 32, 8, 500, "BHSD", "slots", None, 2, "mfma_qk"),
    (3, 32, 8, 500, "BHSD", "paged", 7, 0, "generic"),       # block size 7: the generic kernel
    (2, 8, 2, 300, "BSHD", "paged", 5, 0, "generic"),
]


def _q8_ids(c):
    return f"{c[5]}{c[6] or ''}-B{c[0]}Hq{c[1]}Hkv{c[2]}S{c[3]}{c[4]}n{c[7]}"


@pytest.mark.parametrize("case", Q8_CASES, ids=[_q8_ids(c) for c in Q8_CASES])
def test_int8_mapped_step_and_attend(g, case):
    import ctypes
    from gqa_decode_attention_amd import _lib
    B, Hq, Hkv, S, layout, kind, bs, ns, kernel = case
    w = W.custom(B, Hq, Hkv, 128, S, layout, "i8", "bf16", seed=B * 31 + Hq + (bs or 0), stale="pm:1")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(S + 11), dtype=torch.int32)
    L[0] = S - 1
    inp = W.make_q8(w, DEV, lengths=L)
    m = W.make_mapped(inp, w, kind, block_size=bs or 16)
    table = m["map"].cpu().numpy()
    say(f"int8 mapped step {_q8_ids(case)} capacity={m['capacity']}")
    desc, o, keep = _lib._opts((B, Hq, 128, g.I8, g.BF16, ns, None), table=m["map"], kind=kind,
                               k_scale=m["k_scale"], v_scale=m["v_scale"], k_cache=m["k_cache"], layout=layout)
    assert g.get_plan_ex(desc, o)["kernel"] == kernel
    host = {k: np_of(m[k]) for k in ("k_cache", "v_cache", "k_scale", "v_scale")}
    ref, rk, rv, rks, rvs = oracle.step_q8_mapped(kind, np_of(inp["q"]), "bf16", host["k_cache"], host["v_cache"],
                                                  host["k_scale"], host["v_scale"], np_of(inp["k_new"]),
                                                  np_of(inp["v_new"]), L.numpy(), layout, Hq, Hkv, table, bs)
    out = g.step_ex(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout=layout,
                    table=m["map"], kind=kind, k_scale=m["k_scale"], v_scale=m["v_scale"], num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "int8 mapped step")
    for name, want in (("k_cache", rk), ("v_cache", rv), ("k_scale", rks), ("v_scale", rvs)):
        assert np_of(m[name]).tobytes() == want.tobytes(), name
    n = (inp["lengths"] + 1).contiguous()
    out2 = g.attend_ex(inp["q"], m["k_cache"], m["v_cache"], n, layout=layout, table=m["map"], kind=kind,
                       k_scale=m["k_scale"], v_scale=m["v_scale"], num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out2, ref, "bf16", "int8 mapped attend")

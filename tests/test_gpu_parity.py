"""GPU parity: the HIP library against the float64 oracle, element by element.

Tolerances (abs + rel, elementwise): fp32 outputs |gpu - ref| <= 2e-5 + 2e-5 |ref|;
bf16 outputs <= 1e-2 + 1e-2 |ref|.  The append is compared byte for byte.
Inputs come from the seeded generators in workloads.py; the oracle gets the
same stored bits through workloads.to_numpy_storage.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = {"f32": 2e-5, "bf16": 1e-2}
DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_amd as lib
    lib.lib()           # raises if the HIP library is not built
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


def run_step(g, inp, w, num_splits=0):
    return g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                  layout=w.layout, num_splits=num_splits)


def oracle_step(inp, w):
    return oracle.step(np_of(inp["q"]), w.qo_dtype, np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                       np_of(inp["k_new"]), np_of(inp["v_new"]), w.kv_dtype, inp["lengths"].cpu().numpy(),
                       w.layout, w.Hq, w.Hkv)


def check_step_full(g, w, lengths=None, num_splits=0):
    """Step on the GPU vs the oracle: output within tolerance, caches byte-exact."""
    inp = W.make_inputs(w, DEV, lengths=lengths)
    ref_out, ref_k, ref_v = oracle_step(inp, w)         # oracle sees the caches before the append
    say(f"step {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.capacity} {w.layout} "
        f"kv={w.kv_dtype} qo={w.qo_dtype} splits={num_splits} plan={g.get_plan(g.desc_for(inp['q'], inp['k_cache'], w.layout, num_splits))}")
    out = run_step(g, inp, w, num_splits)
    torch.cuda.synchronize()
    assert_close(out, ref_out, w.qo_dtype, w.name)
    assert np_of(inp["k_cache"]).tobytes() == ref_k.tobytes()
    assert np_of(inp["v_cache"]).tobytes() == ref_v.tobytes()
    return inp, out


# ---------------------------------------------------------------------------
# The pages' worked examples, run through the library.
# ---------------------------------------------------------------------------
def test_kv_cache_decode_step_page_examples(g):
    cases = json.load(open(os.path.join(GOLDEN, "kv_cache_decode_step_examples.json")))["cases"]
    for c in cases:
        say("page example (KV cache decode step):", c["name"])
        q = torch.tensor(c["query"], dtype=torch.float32)
        kc = torch.tensor(c["key_cache"], dtype=torch.float32)
        vc = torch.tensor(c["value_cache"], dtype=torch.float32)
        B, Hkv, S, D = kc.shape
        kcap = torch.full((B, Hkv, S + 1, D), 777.0)
        vcap = torch.full((B, Hkv, S + 1, D), -777.0)
        kcap[:, :, :S] = kc
        vcap[:, :, :S] = vc
        kn = torch.tensor(c["new_key"], dtype=torch.float32)
        vn = torch.tensor(c["new_value"], dtype=torch.float32)
        L = torch.full((B,), S, dtype=torch.int32)
        ref, rk, rv = oracle.step(q.numpy(), "f32", kcap.numpy(), vcap.numpy(), kn.numpy(), vn.numpy(), "f32",
                                  L.numpy(), "BHSD", c["num_query_heads"], c["num_kv_heads"])
        qd, kd, vd, knd, vnd, Ld = (t.to(DEV) for t in (q, kcap, vcap, kn, vn, L))
        out = g.step(qd, kd, vd, knd, vnd, Ld, layout="BHSD")
        torch.cuda.synchronize()
        assert_close(out, ref, "f32", c["name"])
        printed = np.array(c["output"]).astype(np.float64)
        assert np.max(np.abs(out.cpu().double().numpy() - printed)) < 1e-6
        assert kd.cpu().numpy().tobytes() == rk.tobytes() and vd.cpu().numpy().tobytes() == rv.tobytes()


def test_gqa_jax_page_examples(g):
    cases = json.load(open(os.path.join(GOLDEN, "gqa_decode_step_jax_examples.json")))["cases"]
    for c in cases:
        say("page example (JAX Grouped-Query Decode Step):", c["name"])
        q = torch.tensor(c["query"], dtype=torch.float32)
        kc = torch.tensor(c["key_cache"], dtype=torch.float32)
        vc = torch.tensor(c["value_cache"], dtype=torch.float32)
        L = torch.tensor(c["lengths"], dtype=torch.int32)
        ref = oracle.attend(q.numpy(), "f32", kc.numpy(), vc.numpy(), "f32", L.numpy(), "BSHD",
                            c["num_query_heads"], c["num_kv_heads"])
        out = g.attend(q.to(DEV), kc.to(DEV), vc.to(DEV), L.to(DEV), layout="BSHD")
        torch.cuda.synchronize()
        assert_close(out, ref, "f32", c["name"])
        printed = np.array(c["output"]).astype(np.float64)
        dec = np.vectorize(lambda s: len(s.split(".")[1]) if "." in s else 0)(np.array(c["output"]))
        assert np.all(np.abs(out.cpu().double().numpy() - printed) <= 0.5 * 10.0 ** (-dec) + 1e-6)


def test_page_example_with_bf16_caches_and_f32_query(g):
    """JAX page requirement: bf16 caches widened to f32, f32 query and output."""
    c = json.load(open(os.path.join(GOLDEN, "gqa_decode_step_jax_examples.json")))["cases"][1]
    q = torch.tensor(c["query"], dtype=torch.float32)
    kc = torch.tensor(c["key_cache"], dtype=torch.float32).to(torch.bfloat16)   # small integers: exact
    vc = torch.tensor(c["value_cache"], dtype=torch.float32).to(torch.bfloat16)
    L = torch.tensor(c["lengths"], dtype=torch.int32)
    ref = oracle.attend(q.numpy(), "f32", np_of(kc), np_of(vc), "bf16", L.numpy(), "BSHD", 4, 2)
    out = g.attend(q.to(DEV), kc.to(DEV), vc.to(DEV), L.to(DEV), layout="BSHD")
    torch.cuda.synchronize()
    assert out.dtype == torch.float32
    assert_close(out, ref, "f32", "bf16 caches")


# ---------------------------------------------------------------------------
# The tiny workload, whole.
# ---------------------------------------------------------------------------
def test_tiny_workload_step(g):
    check_step_full(g, W.WORKLOADS["tiny"])


# ---------------------------------------------------------------------------
# Shapes that span several tiles and splits with ragged tails, every head
# width class, group sizes from 1 to 64, both layouts and storage types.
# ---------------------------------------------------------------------------
SHAPES = [
    # B, Hq, Hkv, D, S, layout, kv, qo, num_splits
    (2, 4, 2, 1, 37, "BHSD", "f32", "f32", 0),
    (2, 6, 3, 2, 50, "BSHD", "f32", "f32", 3),
    (3, 4, 4, 3, 41, "BHSD", "bf16", "bf16", 2),
    (2, 8, 2, 4, 300, "BSHD", "f32", "f32", 0),
    (2, 8, 2, 8, 333, "BHSD", "bf16", "f32", 4),
    (1, 12, 1, 16, 777, "BHSD", "f32", "bf16", 0),
    (2, 16, 2, 24, 513, "BSHD", "bf16", "bf16", 5),
    (2, 8, 8, 64, 1000, "BHSD", "f32", "f32", 0),
    (3, 16, 2, 100, 650, "BSHD", "f32", "f32", 2),
    (3, 32, 8, 128, 1500, "BHSD", "bf16", "bf16", 0),
    (2, 24, 2, 128, 1030, "BSHD", "bf16", "bf16", 3),
    (2, 16, 4, 128, 700, "BHSD", "f32", "f32", 0),
    (2, 16, 1, 128, 900, "BHSD", "bf16", "bf16", 0),
    (2, 64, 1, 128, 600, "BHSD", "bf16", "bf16", 0),
    (2, 128, 2, 128, 300, "BSHD", "bf16", "bf16", 2),
    (2, 8, 2, 256, 400, "BHSD", "bf16", "bf16", 0),
    (2, 4, 1, 256, 259, "BSHD", "f32", "f32", 2),
    (2, 8, 2, 136, 200, "BHSD", "bf16", "bf16", 0),
    (2, 48, 2, 128, 700, "BHSD", "bf16", "bf16", 0),     # G = 24: a partly used head block
    (3, 40, 1, 128, 333, "BSHD", "bf16", "bf16", 3),     # G = 40
    (2, 32, 1, 128, 1000, "BSHD", "bf16", "bf16", 0),    # G = 32
    (2, 80, 1, 128, 200, "BHSD", "bf16", "bf16", 0),     # G = 80: beyond the matrix-core kernels
    (2, 32, 8, 128, 2000, "BHSD", "bf16", "bf16", 24),   # many splits: the combine's second loop
    (2, 16, 2, 128, 1500, "BSHD", "f32", "f32", 64),     # 64 splits, float32 combine
    (2, 64, 1, 128, 3000, "BHSD", "bf16", "bf16", 13),   # G = 64, an odd split count above 8
    (3, 8, 2, 16, 500, "BSHD", "bf16", "bf16", 0),       # small-head-width kernel, several 64-slot chunks
    (2, 12, 3, 7, 130, "BHSD", "f32", "bf16", 0),        # small kernel, odd D, f32 caches with bf16 out
    (4, 8, 1, 2, 512, "BHSD", "f32", "f32", 0),          # small kernel at its largest capacity
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{s[0]}Hq{s[1]}Hkv{s[2]}D{s[3]}S{s[4]}{s[5]}{s[6]}{s[7]}n{s[8]}"
                                               for s in SHAPES])
def test_step_shapes(g, shape):
    B, Hq, Hkv, D, S, layout, kv, qo, ns = shape
    w = W.custom(B, Hq, Hkv, D, S, layout, kv, qo, seed=B * 1000 + D, stale="pm:1000")
    gen = torch.Generator().manual_seed(S)
    L = torch.randint(0, S, (B,), generator=gen, dtype=torch.int32)
    L[0] = S - 1                       # a full cache
    if B > 2:
        L[1] = 0                       # only the new token
    check_step_full(g, w, lengths=L, num_splits=ns)


@pytest.mark.parametrize("shape", SHAPES[::3], ids=[f"B{s[0]}Hq{s[1]}D{s[3]}S{s[4]}{s[5]}{s[6]}" for s in SHAPES[::3]])
def test_attend_shapes(g, shape):
    B, Hq, Hkv, D, S, layout, kv, qo, ns = shape
    w = W.custom(B, Hq, Hkv, D, S, layout, kv, qo, seed=7 + D, stale="pm:1000")
    gen = torch.Generator().manual_seed(S + 1)
    n = torch.randint(1, S + 1, (B,), generator=gen, dtype=torch.int32)
    n[0] = S
    inp = W.make_inputs(w, DEV, lengths=n)
    say(f"attend {shape}")
    ref = oracle.attend(np_of(inp["q"]), qo, np_of(inp["k_cache"]), np_of(inp["v_cache"]), kv, n.numpy(), layout,
                        Hq, Hkv)
    out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout=layout, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, qo, "attend")


@pytest.mark.parametrize("G", [4, 64])
@pytest.mark.parametrize("ns", [1, 2, 3, 7, 20, 0])
def test_split_count_does_not_change_the_result(g, ns, G):
    w = W.custom(3, 4 * G, 4, 128, 2100, "BHSD", "bf16", "bf16", seed=31, stale="pm:10000")
    L = torch.tensor([2099, 1, 1234], dtype=torch.int32)
    check_step_full(g, w, lengths=L, num_splits=ns)


# ---------------------------------------------------------------------------
# Properties the method fixes.
# ---------------------------------------------------------------------------
def test_stale_slots_never_read(g):
    """Refilling every slot past the attended range with NaN/Inf leaves the output bitwise equal."""
    w = W.custom(4, 32, 8, 128, 1200, "BSHD", "bf16", "bf16", seed=41, stale="pm:10000")
    L = torch.tensor([5, 1199, 640, 0], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    keep = {k: v.clone() for k, v in inp.items()}
    say("stale NaN refill")
    out1 = run_step(g, inp, w)
    slot = torch.arange(w.capacity, device=DEV)
    stale = slot[None, :] > L.to(DEV)[:, None]            # beyond the appended slot
    stale = stale[:, :, None, None]                        # (B, S, 1, 1) for BSHD
    for name, fill in (("k_cache", float("nan")), ("v_cache", float("inf"))):
        keep[name] = torch.where(stale, torch.tensor(fill, dtype=torch.bfloat16, device=DEV), keep[name])
    out2 = run_step(g, keep, w)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.isfinite(out1.float()).all()


def test_step_from_empty_cache_returns_new_value(g):
    for kv, qo in (("f32", "f32"), ("bf16", "bf16")):
        w = W.custom(3, 16, 4, 128, 64, "BHSD", kv, qo, seed=5, stale="const:1000")
        inp = W.make_inputs(w, DEV, lengths=torch.zeros(3, dtype=torch.int32))
        out = run_step(g, inp, w)
        torch.cuda.synchronize()
        expect = inp["v_new"].repeat_interleave(4, dim=1).to(out.dtype)
        assert torch.equal(out, expect)


def test_deterministic(g):
    w = W.custom(8, 32, 8, 128, 4097, "BHSD", "bf16", "bf16", seed=2)
    L = torch.full((8,), 4096, dtype=torch.int32)
    a = W.make_inputs(w, DEV, lengths=L)
    b = {k: v.clone() for k, v in a.items()}
    o1 = run_step(g, a, w)
    o2 = run_step(g, b, w)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_out_of_contract_lengths_are_memory_safe(g):
    """Append skips lengths outside [0, S); attend clamps the count to [0, S]."""
    w = W.custom(4, 8, 2, 64, 32, "BHSD", "f32", "f32", seed=9)
    L = torch.tensor([-1, 32, 40, 3], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=torch.tensor([0, 0, 0, 3], dtype=torch.int32))
    before_k = inp["k_cache"].clone()
    g.append(inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], L.to(DEV), layout="BHSD")
    torch.cuda.synchronize()
    diff = (inp["k_cache"] != before_k).any(dim=-1)        # (B, Hkv, S)
    assert not diff[:3].any()                               # skipped sequences untouched
    assert diff[3, :, 3].all() and diff[3].sum() == 2
    ref = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], torch.tensor([5, 32, 32, 3], dtype=torch.int32,
                                                                            device=DEV))
    out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], torch.tensor([0, 99, 33, -7], dtype=torch.int32,
                                                                            device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(out[0], torch.zeros_like(out[0])) and torch.equal(out[3], torch.zeros_like(out[3]))
    assert torch.equal(out[1], ref[1]) and torch.equal(out[2], ref[2])   # counts past S clamp to S = 32


def test_workspace_contents_do_not_matter(g):
    """A workspace full of garbage, reused across descriptors and calls, gives the clean result."""
    cases = [W.custom(4, 32, 8, 128, 3000, "BHSD", "bf16", "bf16", seed=51),
             W.custom(2, 128, 2, 128, 2500, "BSHD", "bf16", "bf16", seed=52),
             W.custom(3, 16, 2, 64, 900, "BHSD", "f32", "f32", seed=53)]
    ws = torch.randint(0, 256, (64 << 20,), generator=torch.Generator().manual_seed(5), dtype=torch.uint8).to(DEV)
    ws[: 16 << 20].fill_(0xFF)                                   # NaN floats
    ws[16 << 20: 32 << 20].view(torch.float32).fill_(float("inf"))
    for w in cases:
        L = torch.tensor([w.capacity - 1, 5, w.capacity // 2, 0][:w.B], dtype=torch.int32)
        a = W.make_inputs(w, DEV, lengths=L)
        b = {k: v.clone() for k, v in a.items()}
        desc = g.desc_for(a["q"], a["k_cache"], w.layout)
        assert g.workspace_size(desc) <= ws.numel()
        say(f"workspace reuse {w.name}: plan {g.get_plan(desc)}")
        clean = g.step(a["q"], a["k_cache"], a["v_cache"], a["k_new"], a["v_new"], a["lengths"], layout=w.layout,
                       workspace=torch.zeros_like(ws))
        for rep in range(3):
            got = g.step(b["q"], b["k_cache"], b["v_cache"], b["k_new"], b["v_new"], b["lengths"], layout=w.layout,
                         workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               clean.view(torch.int16) if clean.dtype == torch.bfloat16 else clean), (w.name, rep)


def test_empty_batch(g):
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.empty(0, 2, 16, 128, dtype=torch.bfloat16, device=DEV)
    L = torch.empty(0, dtype=torch.int32, device=DEV)
    out = g.attend(q, kc, kc.clone(), L)
    assert out.shape == (0, 8, 128)


def test_check_lengths_counts_out_of_contract_entries(g):
    S = 100
    vals = torch.tensor([-1, 0, 1, 5, S - 1, S, S + 1, 2 ** 31 - 1, -(2 ** 31)], dtype=torch.int32)
    lens = vals.to(DEV)
    want_step = int(((vals < 0) | (vals >= S)).sum())
    want_attend = int(((vals < 1) | (vals > S)).sum())
    assert g.check_lengths(lens, S, mode="step") == want_step == 5
    assert g.check_lengths(lens, S, mode="attend") == want_attend == 5
    big = torch.randint(-50, 3 * S, (5000,), generator=torch.Generator().manual_seed(11), dtype=torch.int32)
    assert g.check_lengths(big.to(DEV), S, mode="attend") == int(((big < 1) | (big > S)).sum())
    assert g.check_lengths(big.to(DEV), S, mode="append") == int(((big < 0) | (big >= S)).sum())
    # every workload's lengths are inside the contract
    for name in ("tiny", "ragged_batch", "large_group"):
        w = W.WORKLOADS[name]
        Lw = W.draw_lengths(w).to(DEV)
        assert g.check_lengths(Lw, w.capacity, mode="step") == 0


@pytest.mark.parametrize("B", [4, 40])
def test_graph_capture_replays(g, B):
    """The step has no host sync and no memset: it can be captured and
    replayed.  B = 4 splits the token axis (attention + combine); B = 40 has
    more (b, kv-head) items than CUs, so the balanced mode cuts the batch on
    the device from the lengths at run time.  Each replay runs on new lengths
    (written into the captured buffer) and matches an eager call on them."""
    w = W.custom(B, 32, 8, 128, 2048, "BHSD", "bf16", "bf16", seed=77)
    gen = torch.Generator().manual_seed(78)
    L = torch.randint(0, 2048, (B,), generator=gen, dtype=torch.int32)
    L[0] = 2047
    inp = W.make_inputs(w, DEV, lengths=L)
    desc = g.desc_for(inp["q"], inp["k_cache"], "BHSD")
    assert g.get_plan(desc)["balanced"] == (B == 40)
    ws = torch.empty(max(g.workspace_size(desc), 1), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(inp["q"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_step(g, {k: v.clone() for k, v in inp.items()}, w)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
               out=out, workspace=ws)
    caches = (inp["k_cache"].clone(), inp["v_cache"].clone())
    for r in range(4):
        Lr = torch.randint(0, 2048, (B,), generator=gen, dtype=torch.int32)
        inp["lengths"].copy_(Lr.to(DEV))
        inp["k_cache"].copy_(caches[0])
        inp["v_cache"].copy_(caches[1])
        eager = run_step(g, {k: v.clone() for k, v in inp.items()}, w)
        out.zero_()
        inp["q"].mul_(1.0)                                  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"


# ---------------------------------------------------------------------------
# Full-size workloads in the launch configuration the benchmark times: every
# (b, query head, d) output against the oracle, and every byte of both caches
# against the oracle's append.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["llama3_8b_layer", "ragged_batch", "long_context", "large_group"])
def test_full_size_workload(g, name):
    w = W.WORKLOADS[name]
    inp, out = check_step_full(g, w)
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("kind", ["dense", "paged", "int8", "fp8", "window"])
def test_balanced_mode_matches_oracle(g, kind):
    """More (b, kv-head) items than CUs: the plan switches to the balanced mode
    (equal tile ranges per workgroup, cut on the device from the lengths, and a
    combine of the items cut between workgroups).  Shuffled ragged lengths
    (including 0 and the full capacity) on dense, paged, int8 and fp8 caches and
    with a sliding window must match the oracle."""
    B, Hq, Hkv, D, S = 40, 32, 8, 128, 300
    kv = {"int8": "i8", "fp8": "fp8"}.get(kind, "bf16")
    w = W.custom(B, Hq, Hkv, D, S, "BHSD", kv, "bf16", seed=91, stale="pm:1")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(92), dtype=torch.int32)
    L[5], L[17], L[30] = 0, S - 1, S - 1
    desc = g.make_desc(B, Hq, Hkv, D, S, "BHSD", {"i8": g.I8, "fp8": g.FP8}.get(kv, g.BF16), g.BF16)
    assert g.get_plan(desc)["balanced"]
    say(f"balanced {kind}")
    if kv in ("i8", "fp8"):
        inp = W.make_q8(w, DEV, lengths=L)
        ref, rk, rv, rks, rvs = oracle.step_q8(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                               np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                               np_of(inp["v_new"]), L.numpy(), "BHSD", Hq, Hkv)
        out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                        inp["v_new"], inp["lengths"], layout="BHSD")
        torch.cuda.synchronize()
        assert_close(out, ref, "bf16", f"{kind} step")
        for name, want in (("k_cache", rk), ("v_cache", rv), ("k_scale", rks), ("v_scale", rvs)):
            assert np_of(inp[name]).tobytes() == want.tobytes(), name
        return
    inp = W.make_inputs(w, DEV, lengths=L)
    if kind == "paged":
        m = W.make_mapped(inp, w, "paged", block_size=16)
        ref, rk, rv = oracle.step_mapped("paged", np_of(inp["q"]), "bf16", np_of(m["k_cache"]), np_of(m["v_cache"]),
                                         np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), "BHSD", Hq,
                                         Hkv, m["map"].cpu().numpy(), 16)
        out = g.step_mapped(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                            m["map"], kind="paged", layout="BHSD")
        torch.cuda.synchronize()
        assert_close(out, ref, "bf16", "paged step")
        assert np_of(m["k_cache"]).tobytes() == rk.tobytes()
        return
    if kind == "window":
        sm = g.Softmax(window=50, kept_prefix=7)
        ref, rk, rv = oracle.step_variants(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                           np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), "BHSD", Hq,
                                           Hkv, window=50, prefix=7)
        out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                        layout="BHSD", softmax=sm)
    else:
        ref, rk, rv = oracle.step(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                  np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), "BHSD", Hq, Hkv)
        out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                     layout="BHSD")
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", f"{kind} step")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes() and np_of(inp["v_cache"]).tobytes() == rv.tobytes()


@pytest.mark.parametrize("kv", ["bf16", "i8"])
@pytest.mark.parametrize("layout", ["BHSD", "BSHD"])
def test_balanced_mode_largest_batch(g, kv, layout):
    """The largest batch the balanced mode takes (4096 sequences: 16 per
    thread of its on-device scan), with empty and full sequences among them:
    every output against the oracle, appended rows (codes and scales) byte
    for byte."""
    B, Hq, Hkv, S = 4096, 8, 1, 64
    w = W.custom(B, Hq, Hkv, 128, S, layout, kv, "bf16", seed=4096, stale="pm:100" if kv == "bf16" else "none")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(4097), dtype=torch.int32)
    L[0], L[1], L[4095] = S - 1, 0, S - 1
    desc = g.make_desc(B, Hq, Hkv, 128, S, layout, g.BF16 if kv == "bf16" else g.I8, g.BF16)
    plan = g.get_plan(desc)
    say(f"balanced largest batch {kv} {layout}: plan {plan}")
    assert plan["balanced"] and plan["kernel"] == "mfma_qk"
    if kv == "bf16":
        inp = W.make_inputs(w, DEV, lengths=L)
        ref, rk, rv = oracle_step(inp, w)
        out = run_step(g, inp, w)
        want = {"k_cache": rk, "v_cache": rv}
    else:
        inp = W.make_q8(w, DEV, lengths=L)
        ref, rk, rv, rks, rvs = oracle.step_q8(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                               np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                               np_of(inp["v_new"]), L.numpy(), layout, Hq, Hkv)
        out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                        inp["v_new"], inp["lengths"], layout=layout)
        want = {"k_cache": rk, "v_cache": rv, "k_scale": rks, "v_scale": rvs}
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", f"B={B} {kv} {layout}")
    for name, expect in want.items():
        assert np_of(inp[name]).tobytes() == expect.tobytes(), name


@pytest.mark.parametrize("seed", range(6))
def test_balanced_mode_random_shapes(g, seed):
    """Balanced mode on seeded random shapes: batch, group size, capacity,
    layout and cache dtype drawn at random (always more (b, kv-head) items than
    CUs), and lengths from one of three mixes (all short, heavy-tailed, or
    uniform with zeros and full sequences), so workgroup ranges start and end
    inside items' charged cost units, inside their tiles and on their edges."""
    rng = np.random.default_rng(1000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    B = int(rng.integers(256 // Hkv + 1, 256 // Hkv + 120))
    S = int(rng.integers(40, 1200))
    lay = str(rng.choice(["BHSD", "BSHD"]))
    kv = ("bf16", "i8", "fp8")[(seed // 3 + seed) % 3]
    mix = seed % 3
    if mix == 0:
        L = rng.integers(0, min(S, 48), B)
    elif mix == 1:
        L = np.minimum(S - 1, (rng.pareto(1.2, B) * 20).astype(np.int64))
    else:
        L = rng.integers(0, S, B)
        L[rng.integers(0, B, 3)] = 0
        L[rng.integers(0, B, 3)] = S - 1
    L = torch.from_numpy(L.astype(np.int32))
    Hq = Hkv * G
    say(f"balanced random seed={seed}: B={B} Hq={Hq} Hkv={Hkv} S={S} {lay} {kv} mix={mix}")
    desc = g.make_desc(B, Hq, Hkv, 128, S, lay, {"i8": g.I8, "fp8": g.FP8}.get(kv, g.BF16), g.BF16)
    assert g.get_plan(desc)["balanced"]
    w = W.custom(B, Hq, Hkv, 128, S, lay, kv, "bf16", seed=200 + seed, stale="pm:1")
    if kv in ("i8", "fp8"):
        inp = W.make_q8(w, DEV, lengths=L)
        ref, rk, rv, rks, rvs = oracle.step_q8(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                               np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                               np_of(inp["v_new"]), L.numpy(), lay, Hq, Hkv)
        out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                        inp["v_new"], inp["lengths"], layout=lay)
        torch.cuda.synchronize()
        assert_close(out, ref, "bf16", f"{kv} step")
        for name, want in (("k_cache", rk), ("v_cache", rv), ("k_scale", rks), ("v_scale", rvs)):
            assert np_of(inp[name]).tobytes() == want.tobytes(), name
        return
    inp = W.make_inputs(w, DEV, lengths=L)
    ref, rk, rv = oracle_step(inp, w)
    out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout=lay)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(inp["v_cache"]).tobytes() == rv.tobytes()


@pytest.mark.parametrize("case", ["one_long", "attend_empty", "sink_bshd", "one_long_bshd", "attend_empty_g4",
                                  "window"])
def test_balanced_mode_edge_cases(g, case):
    """Balanced-mode cases: one long sequence among many short ones (its item
    is cut across more than 64 workgroups, so the combine merges its partials
    in several rounds, an odd number of them in the last), attend with empty
    sequences (zero rows, never cut), a per-head sink on a (B, S, Hkv, D)
    cache, and a sliding window with a kept prefix."""
    if case == "one_long":
        B, Hq, Hkv, S, lay = 300, 16, 1, 28000, "BHSD"
        L = torch.randint(0, 40, (B,), generator=torch.Generator().manual_seed(93), dtype=torch.int32)
        L[123] = S - 1
        # The cut as the kernels make it (16-slot tiles, 12 cost units per item for bf16 BHSD caches,
        # 256 ranges): the long item must span more than 64 ranges, an odd number in the last round.
        units = 12 + np.maximum(1, -(-(L.numpy().astype(np.int64) + 1) // 16))
        pre = np.concatenate([[0], np.cumsum(units)])
        per = -(-int(pre[-1]) // 256)
        first, last = pre[123] + 12, pre[123 + 1] - 1
        pieces = int(last // per - first // per + 1)
        assert pieces > 64 and (pieces - 64) % 2 == 1, pieces
    elif case == "one_long_bshd":
        B, Hq, Hkv, S, lay = 150, 8, 2, 9000, "BSHD"
        L = torch.randint(0, 40, (B,), generator=torch.Generator().manual_seed(98), dtype=torch.int32)
        L[7] = S - 1
    elif case == "attend_empty":
        B, Hq, Hkv, S, lay = 70, 32, 4, 700, "BHSD"
        L = torch.randint(0, S + 1, (B,), generator=torch.Generator().manual_seed(94), dtype=torch.int32)
        L[0], L[9], L[69] = 0, 0, S
    elif case == "attend_empty_g4":
        B, Hq, Hkv, S, lay = 300, 4, 1, 700, "BSHD"
        L = torch.randint(0, S + 1, (B,), generator=torch.Generator().manual_seed(99), dtype=torch.int32)
        L[0], L[9], L[29] = 0, 0, S
    elif case == "window":
        B, Hq, Hkv, S, lay = 20, 64, 16, 1500, "BHSD"
        L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(100), dtype=torch.int32)
    else:
        B, Hq, Hkv, S, lay = 36, 64, 8, 520, "BSHD"
        L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(95), dtype=torch.int32)
    qo = "bf16"
    w = W.custom(B, Hq, Hkv, 128, S, lay, "bf16", qo, seed=96, stale="pm:100")
    inp = W.make_inputs(w, DEV, lengths=L)
    desc = g.make_desc(B, Hq, Hkv, 128, S, lay, g.BF16, g.BF16)
    assert g.get_plan(desc)["balanced"]
    say(f"balanced {case}: B={B} Hq={Hq} Hkv={Hkv} S={S} {lay}")
    args = (np_of(inp["q"]), qo, np_of(inp["k_cache"]), np_of(inp["v_cache"]))
    if case.startswith("attend_empty"):
        ref = oracle.attend(*args, "bf16", L.numpy(), lay, Hq, Hkv)
        out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout=lay)
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
        empty = L.numpy() == 0
        assert np.all(got[empty] == 0.0)
        assert_close(out[torch.from_numpy(~empty).to(DEV)], ref[~empty], qo, "balanced attend")
        return
    if case == "sink_bshd":
        sink = torch.randn(Hq, generator=torch.Generator().manual_seed(97)).to(DEV)
        ref, rk, rv = oracle.step_variants(*args, np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), lay,
                                           Hq, Hkv, sink=sink.cpu().numpy())
        out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                        layout=lay, softmax=g.Softmax(sink=sink))
    elif case == "window":
        ref, rk, rv = oracle.step_variants(*args, np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), lay,
                                           Hq, Hkv, window=300, prefix=20)
        out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                        layout=lay, softmax=g.Softmax(window=300, kept_prefix=20))
    else:
        ref, rk, rv = oracle.step(*args, np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), lay, Hq, Hkv)
        out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout=lay)
    torch.cuda.synchronize()
    assert_close(out, ref, qo, f"balanced {case}")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes() and np_of(inp["v_cache"]).tobytes() == rv.tobytes()

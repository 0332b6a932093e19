"""GPU parity for the large-group kernel's whole-item mode (16 < G <= 64, bf16).

In this mode one 8-wave workgroup covers a (sequence, kv-head) item and all
its query heads (two 16-head blocks for G <= 32, four above) over the whole
token axis, merging its sub-tile waves in LDS: no split partials and no
combine pass.  The planner takes this mode when the items fill the device, or
when one split is asked for.

Cases cover G in {17, 24, 32, 40, 48, 64} (partly used and empty head
blocks), capacities that are not multiples of a step (128 or 64 slots), both
layouts, step and attend (one valid slot, a full cache, zero valid slots),
the automatic choice at large batches, slot-indexed caches,
paged caches (planned on the split kernel instead), the softmax variants, the
rotary step, determinism and HIP-graph replay.  Outputs against the float64
oracle (bf16 1e-2, abs + rel), appended rows byte-exact.
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


def assert_close(out_gpu, ref, qo, what=""):
    got = out_gpu.detach().float().cpu().double().numpy()
    err = np.abs(got - ref)
    bound = TOL[qo] + TOL[qo] * np.abs(ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst excess "
                           f"{np.max(err - bound):.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def whole_plan(g, B, Hq, Hkv, S, layout, ns):
    """The whole-item plan: one 512-thread workgroup per (sequence, kv-head)."""
    desc = g.make_desc(B, Hq, Hkv, 128, S, layout, g.BF16, g.BF16, ns)
    plan = g.get_plan(desc)
    grid = B * Hkv
    assert plan["kernel"] == "mfma_all" and plan["num_splits"] == 1 and plan["block"] == 512, plan
    assert plan["grid"] == grid and not plan["combine"] and plan["workspace_bytes"] == 0, plan
    return plan


def lengths_for(B, S, seed, step):
    gen = torch.Generator().manual_seed(seed)
    if step:
        L = torch.randint(0, S, (B,), generator=gen, dtype=torch.int32)
        L[0] = S - 1                     # a full cache
        if B > 1:
            L[1] = 0                     # only the new token
    else:
        L = torch.randint(1, S + 1, (B,), generator=gen, dtype=torch.int32)
        L[0] = S
        if B > 1:
            L[1] = 1
    return L


SHAPES = [
    # B, Hq, Hkv, S, layout, num_splits (1: forced whole mode)
    (3, 64, 1, 1500, "BHSD", 1),     # four head blocks, several 64-slot steps
    (9, 64, 1, 700, "BSHD", 1),
    (5, 96, 2, 333, "BSHD", 1),      # G = 48: four head blocks, the last one empty
    (4, 48, 2, 333, "BHSD", 1),      # G = 24: two head blocks, the second partly used
    (2, 128, 4, 1030, "BSHD", 1),    # G = 32: two full head blocks, 128-slot steps
    (3, 17, 1, 257, "BHSD", 1),      # G = 17: one head in the second block
    (2, 80, 2, 2100, "BHSD", 1),     # G = 40, a ragged last step
    (300, 24, 1, 200, "BHSD", 0),    # chosen automatically: 300 items fill the device
    (260, 64, 1, 300, "BSHD", 0),    # chosen automatically, G = 64
    (270, 48, 1, 150, "BHSD", 0),    # chosen automatically, G = 48
]


def _id(s):
    return f"B{s[0]}Hq{s[1]}Hkv{s[2]}S{s[3]}{s[4]}n{s[5]}"


@pytest.mark.parametrize("shape", SHAPES, ids=[_id(s) for s in SHAPES])
def test_whole_mode_step(g, shape):
    B, Hq, Hkv, S, layout, ns = shape
    whole_plan(g, B, Hq, Hkv, S, layout, ns)
    w = W.custom(B, Hq, Hkv, 128, S, layout, "bf16", "bf16", seed=B * 31 + Hq, stale="pm:1000")
    L = lengths_for(B, S, S + Hq, True)
    inp = W.make_inputs(w, DEV, lengths=L)
    say(f"whole step {_id(shape)}")
    ref, rk, rv = oracle.step(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                              np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), layout, Hq, Hkv)
    out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                 layout=layout, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(inp["v_cache"]).tobytes() == rv.tobytes()


@pytest.mark.parametrize("shape", SHAPES[::2], ids=[_id(s) for s in SHAPES[::2]])
def test_whole_mode_attend(g, shape):
    B, Hq, Hkv, S, layout, ns = shape
    w = W.custom(B, Hq, Hkv, 128, S, layout, "bf16", "bf16", seed=B + Hq + 5, stale="pm:1000")
    n = lengths_for(B, S, S + 7, False)
    inp = W.make_inputs(w, DEV, lengths=n)
    say(f"whole attend {_id(shape)}")
    ref = oracle.attend(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]), "bf16", n.numpy(),
                        layout, Hq, Hkv)
    out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout=layout, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "attend")


def test_whole_mode_attend_with_no_valid_slot(g):
    """An attend call whose sequence holds no valid slot writes zeros for it
    (no softmax exists); the others are unaffected."""
    B, Hq, Hkv, S = 3, 64, 1, 400
    w = W.custom(B, Hq, Hkv, 128, S, "BHSD", "bf16", "bf16", seed=4, stale="pm:1000")
    n = torch.tensor([400, 0, 129], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=n)
    out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout="BHSD", num_splits=1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[1]).item() == 0
    keep = np.array([0, 2])
    ref = oracle.attend(np_of(inp["q"])[keep], "bf16", np_of(inp["k_cache"])[keep], np_of(inp["v_cache"])[keep],
                        "bf16", n.numpy()[keep], "BHSD", Hq, Hkv)
    assert_close(out[keep], ref, "bf16", "attend")


def test_whole_mode_matches_split_mode(g):
    """Whole-item and split mode compute the same softmax: their outputs agree
    within bf16 rounding (keys scaled x3 stress the running maximum)."""
    B, Hq, Hkv, S = 4, 64, 1, 2100
    w = W.custom(B, Hq, Hkv, 128, S, "BHSD", "bf16", "bf16", seed=8, stale="pm:1000", key_scale=3.0)
    L = torch.tensor([2099, 0, 1500, 127], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    outs = []
    for ns in (1, 4):
        c = {k: v.clone() for k, v in inp.items()}
        outs.append(g.step(c["q"], c["k_cache"], c["v_cache"], c["k_new"], c["v_new"], c["lengths"], layout="BHSD",
                           num_splits=ns).float())
    torch.cuda.synchronize()
    d = (outs[0] - outs[1]).abs()
    assert float(d.max()) <= 2 * 2.0 ** -8 * float(outs[1].abs().max()) + 1e-6


def test_whole_mode_deterministic(g):
    w = W.custom(3, 64, 1, 128, 900, "BSHD", "bf16", "bf16", seed=9)
    L = torch.tensor([899, 3, 450], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    runs = []
    for _ in range(3):
        c = {k: v.clone() for k, v in inp.items()}
        runs.append(g.step(c["q"], c["k_cache"], c["v_cache"], c["k_new"], c["v_new"], c["lengths"], layout="BSHD",
                           num_splits=1))
    torch.cuda.synchronize()
    for r in runs[1:]:
        assert torch.equal(r.view(torch.int16), runs[0].view(torch.int16))


@pytest.mark.parametrize("kind", ["slots", "paged"])
def test_whole_mode_on_mapped_caches(g, kind):
    """Slot-indexed caches run the whole-item mode; paged ones the split
    kernel (one split per item), both against the oracle with unmapped rows
    holding NaN."""
    B, Hq, Hkv, S, layout = 3, 64, 1, 600, "BSHD"
    w = W.custom(B, Hq, Hkv, 128, S, layout, "bf16", "bf16", seed=21, stale="pm:1000")
    L = lengths_for(B, S, 22, True)
    inp = W.make_inputs(w, DEV, lengths=L)
    m = W.make_mapped(inp, w, kind, block_size=32)
    table = m["map"]
    ref, rk, rv = oracle.step_variants(np_of(inp["q"]), "bf16", np_of(m["k_cache"]), np_of(m["v_cache"]),
                                       np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), layout, Hq, Hkv,
                                       kind=kind, mapping=table.cpu().numpy(), bs=m.get("block_size"))
    out = g.step_mapped(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], table,
                        kind=kind, layout=layout, num_splits=1)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", kind)
    assert np_of(m["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(m["v_cache"]).tobytes() == rv.tobytes()


VARIANTS = [
    ("winpre", dict(window=70, kept_prefix=37)),
    ("win1", dict(window=1)),
    ("cap", dict(softcap=1.5)),
    ("sink", dict(sink=True)),
    ("smooth", dict(smooth=True)),
    ("all", dict(window=200, kept_prefix=16, softcap=2.0, sink=True)),
]


@pytest.mark.parametrize("vname", [v for v, _ in VARIANTS])
@pytest.mark.parametrize("shape", [(3, 64, 1, 900, "BHSD"), (2, 48, 2, 500, "BSHD"), (260, 64, 1, 300, "BHSD")],
                         ids=["G64", "G24", "G64-auto"])
def test_whole_mode_variants(g, vname, shape):
    B, Hq, Hkv, S, layout = shape
    v = dict(VARIANTS)[vname]
    say(f"whole variants {vname} {shape}")
    w = W.custom(B, Hq, Hkv, 128, S, layout, "bf16", "bf16", seed=B + Hq + len(vname), stale="pm:1000")
    L = lengths_for(B, S, S + len(vname), True)
    inp = W.make_inputs(w, DEV, lengths=L)
    gen = torch.Generator().manual_seed(3 + len(vname))
    sink = (torch.randn(Hq, generator=gen) * 2).to(DEV) if v.get("sink") else None
    sm = g.Softmax(sink=sink, smooth=v.get("smooth", False), softcap=v.get("softcap", 0.0), window=v.get("window", 0),
                   kept_prefix=v.get("kept_prefix", 0))
    ref, rk, rv = oracle.step_variants(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                       np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), layout, Hq, Hkv,
                                       sink=None if sink is None else sink.cpu().numpy(),
                                       smooth=v.get("smooth", False), softcap=v.get("softcap", 0.0),
                                       window=v.get("window", 0), prefix=v.get("kept_prefix", 0))
    out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                    layout=layout, softmax=sm, num_splits=1)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(inp["v_cache"]).tobytes() == rv.tobytes()


@pytest.mark.parametrize("B", [3, 260], ids=["forced", "auto"])
@pytest.mark.parametrize("mode", ["half", "interleaved"])
def test_whole_mode_rotary_step(g, mode, B):
    """The rotary step fused into the whole-item mode: q and the new key
    rotated in the kernel (with norm gains in half mode); outputs against the
    oracle, the appended key within one bf16 rounding step (a normalized
    key) or byte-exact, the value byte-exact."""
    Hq, Hkv, S, layout = 64, 1, 300, "BHSD"
    norm = mode == "half"
    w = W.custom(B, Hq, Hkv, 128, S, layout, "bf16", "bf16", seed=41, stale="pm:1000")
    L = lengths_for(B, S, 42, True)
    inp = W.make_inputs(w, DEV, lengths=L)
    cos, sin = W.rope_tables(S + 50, 128, DEV)
    gq = gk = eps = None
    if norm:
        gen = torch.Generator().manual_seed(5)
        gq = (torch.rand(128, generator=gen) + 0.5).to(DEV)
        gk = (torch.rand(128, generator=gen) + 0.5).to(DEV)
        eps = 1e-5
    rope = g.Rope(cos, sin, mode, q_gain=gq, k_gain=gk, eps=eps)
    ref, rk, rv = oracle.step_rope(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                   np_of(inp["k_new"]), np_of(inp["v_new"]), "bf16", L.numpy(), layout, Hq, Hkv,
                                   cos.cpu().numpy(), sin.cpu().numpy(), mode,
                                   q_gain=None if gq is None else gq.cpu().numpy(),
                                   k_gain=None if gk is None else gk.cpu().numpy(), eps=eps)
    out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                    layout=layout, rope=rope, num_splits=1)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    got_k, want_k = np_of(inp["k_cache"]), rk
    rows = [(b, 0, int(L[b])) for b in range(B)]
    for b, h, t in rows:
        a_, b_ = oracle.decode(got_k[b, h, t], "bf16"), oracle.decode(want_k[b, h, t], "bf16")
        if norm:
            assert np.all(np.abs(a_ - b_) <= 2.0 ** -7 * np.abs(b_) + 1e-30)
        else:
            assert got_k[b, h, t].tobytes() == want_k[b, h, t].tobytes()
        got_k[b, h, t] = want_k[b, h, t]
    assert got_k.tobytes() == want_k.tobytes(), "bytes outside the appended rows changed"
    assert np_of(inp["v_cache"]).tobytes() == rv.tobytes()


def test_whole_mode_graph_replays(g):
    """Captured once, replayed on new lengths: every replay equals an eager
    call on the same lengths."""
    B, Hq, Hkv, S = 260, 64, 1, 600
    w = W.custom(B, Hq, Hkv, 128, S, "BHSD", "bf16", "bf16", seed=51)
    gen = torch.Generator().manual_seed(52)
    L = torch.randint(0, S, (B,), generator=gen, dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    whole_plan(g, B, Hq, Hkv, S, "BHSD", 0)
    out = torch.empty_like(inp["q"])

    def eager():
        c = {k: v.clone() for k, v in inp.items()}
        return g.step(c["q"], c["k_cache"], c["v_cache"], c["k_new"], c["v_new"], c["lengths"], layout="BHSD")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eager()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    caches = (inp["k_cache"].clone(), inp["v_cache"].clone())
    with torch.cuda.graph(graph):
        g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], out=out)
    for r in range(3):
        inp["lengths"].copy_(torch.randint(0, S, (B,), generator=gen, dtype=torch.int32).to(DEV))
        inp["k_cache"].copy_(caches[0])
        inp["v_cache"].copy_(caches[1])
        want = eager()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {r}"


def test_large_group_full_size_split_mode(g):
    """The large-group workload at full size on the split kernel (four splits
    and the combine pass, as for smaller batches): every output against the
    oracle, both caches byte-exact."""
    w = W.WORKLOADS["large_group"]
    inp = W.make_inputs(w, DEV)
    desc = g.desc_for(inp["q"], inp["k_cache"], w.layout, 4)
    plan = g.get_plan(desc)
    assert plan["num_splits"] == 4 and plan["combine"], plan
    say(f"large group split mode plan {plan}")
    ref, rk, rv = oracle.step(np_of(inp["q"]), w.qo_dtype, np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                              np_of(inp["k_new"]), np_of(inp["v_new"]), w.kv_dtype, inp["lengths"].cpu().numpy(),
                              w.layout, w.Hq, w.Hkv)
    out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                 layout=w.layout, num_splits=4)
    torch.cuda.synchronize()
    assert_close(out, ref, w.qo_dtype, "large_group split")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(inp["v_cache"]).tobytes() == rv.tobytes()


@pytest.mark.parametrize("ns", [1, 0], ids=["whole-item", "split"])
def test_rows_beyond_buffer_offsets(g, ns):
    """Rows of a kv-head spanning more than 2^31 bytes (BSHD, 64 kv-heads of 128
    bf16 elements: a 16 KB slot stride, capacity 131072) are loaded with
    per-row addresses instead of buffer resources, in both forms of the
    large-group kernel.  The output against the oracle on the first slots (the
    only attended ones), the appended row and those slots byte-exact."""
    B, Hkv, G, S, keep = 1, 64, 17, 131072, 320
    Hq = Hkv * G
    assert S * Hkv * 128 * 2 > 2 ** 31 - 1
    w = W.custom(B, Hq, Hkv, 128, S, "BSHD", "bf16", "bf16", seed=61)
    L = torch.tensor([300], dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    kc, vc = inp["k_cache"][:, :keep].contiguous(), inp["v_cache"][:, :keep].contiguous()
    ref, rk, rv = oracle.step(np_of(inp["q"]), "bf16", np_of(kc), np_of(vc), np_of(inp["k_new"]), np_of(inp["v_new"]),
                              "bf16", L.numpy(), "BSHD", Hq, Hkv)
    plan = g.get_plan(g.desc_for(inp["q"], inp["k_cache"], "BSHD", ns))
    say(f"large stride ns={ns}: plan {plan}")
    assert plan["kernel"] == "mfma_all" and (plan["block"] == 512) == (ns == 1)
    out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout="BSHD",
                 num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    assert np_of(inp["k_cache"][:, :keep].contiguous()).tobytes() == rk.tobytes()
    assert np_of(inp["v_cache"][:, :keep].contiguous()).tobytes() == rv.tobytes()

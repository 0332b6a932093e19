"""GPU parity for the softmax variants (CLIKA runtime "groupQueryAttention"
API page: head sink, smooth softmax, softcap, sliding window with a kept
prefix) on every attention kernel, dense and mapped caches, one split and
several (the split combine applies the sink and walks the window's slots),
and together with the rotary step in one call.

Outputs against the float64 variant oracle within the dense tolerances (fp32
2e-5, bf16 1e-2, abs + rel); the appended rows byte-exact.  Stale slots hold
+-1e3 (int8: NaN scales) and unmapped rows NaN, so a read outside the valid
slots shows up; slots inside the valid range that the window skips hold real
values and must get weight 0.
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


# Shapes: one per kernel family.
SHAPES = {
    "qk4": (3, 32, 8, 128, 900, "BHSD", "bf16", "bf16"),     # G <= 16 matrix-core kernel
    "qk16": (2, 32, 2, 128, 700, "BSHD", "bf16", "bf16"),
    "all64": (2, 64, 1, 128, 600, "BHSD", "bf16", "bf16"),   # 16 < G <= 64 matrix-core kernel
    "gen32": (3, 8, 2, 64, 300, "BHSD", "f32", "f32"),       # generic kernel
    "genbf": (2, 12, 3, 40, 250, "BSHD", "bf16", "f32"),
}
# Variant sets: (name, dict)
VARIANTS = [
    ("win", dict(window=100)),
    ("win1", dict(window=1)),
    ("winpre", dict(window=70, kept_prefix=37)),
    ("winpreseq", dict(window=40, prefix_seq=True)),
    ("cap", dict(softcap=1.5)),
    ("sink", dict(sink=True)),
    ("smooth", dict(smooth=True)),
    ("all", dict(window=64, kept_prefix=16, softcap=2.0, sink=True)),
]


def _softmax(g, v, B, Hq, seed):
    gen = torch.Generator().manual_seed(seed)
    sink = (torch.randn(Hq, generator=gen) * 2).to(DEV) if v.get("sink") else None
    pseq = torch.randint(0, 60, (B,), generator=gen, dtype=torch.int32).to(DEV) if v.get("prefix_seq") else None
    sm = g.Softmax(sink=sink, smooth=v.get("smooth", False), softcap=v.get("softcap", 0.0),
                   window=v.get("window", 0), kept_prefix=v.get("kept_prefix", 0), kept_prefix_per_seq=pseq)
    okw = dict(sink=None if sink is None else sink.cpu().numpy(), smooth=v.get("smooth", False),
               softcap=v.get("softcap", 0.0), window=v.get("window", 0),
               prefix=pseq.cpu().numpy() if pseq is not None else v.get("kept_prefix", 0))
    return sm, okw


def _lengths(B, S, seed):
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(seed), dtype=torch.int32)
    L[0] = S - 1
    if B > 2:
        L[1] = 0
    return L


CASES = [(s, vn, ns) for s in SHAPES for vn, _ in VARIANTS for ns in (0, 3)
         if not (ns == 3 and vn in ("win1", "smooth"))]
# The large-group kernel's whole-item mode (one split).
CASES += [("all64", vn, 1) for vn, _ in VARIANTS]


@pytest.mark.parametrize("case", CASES, ids=[f"{s}-{v}-n{n}" for s, v, n in CASES])
def test_variants_step_and_attend(g, case):
    shape, vname, ns = case
    B, Hq, Hkv, D, S, layout, kv, qo = SHAPES[shape]
    v = dict(VARIANTS)[vname]
    say(f"variants {shape} {vname} splits={ns}")
    w = W.custom(B, Hq, Hkv, D, S, layout, kv, qo, seed=B + D + Hq + len(vname), stale="pm:1000")
    L = _lengths(B, S, S + len(vname))
    inp = W.make_inputs(w, DEV, lengths=L)
    sm, okw = _softmax(g, v, B, Hq, 3 + len(vname))
    ref, rk, rv = oracle.step_variants(np_of(inp["q"]), qo, np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                       np_of(inp["k_new"]), np_of(inp["v_new"]), kv, L.numpy(), layout, Hq, Hkv,
                                       **okw)
    out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                    layout=layout, softmax=sm, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, qo, "step")
    assert np_of(inp["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(inp["v_cache"]).tobytes() == rv.tobytes()
    n = (inp["lengths"] + 1).contiguous()
    out2 = g.attend_ex(inp["q"], inp["k_cache"], inp["v_cache"], n, layout=layout, softmax=sm, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out2, ref, qo, "attend")


MAPPED = [
    ("qk4", "paged", "winpre"), ("qk4", "paged", "all"), ("all64", "paged", "winpre"), ("all64", "paged", "all"),
    ("qk16", "slots", "all"), ("gen32", "paged", "all"), ("qk4", "paged", "win1"), ("all64", "slots", "all"),
]


@pytest.mark.parametrize("case", MAPPED, ids=["-".join(c) for c in MAPPED])
@pytest.mark.parametrize("ns", [0, 1, 4])
def test_variants_on_mapped_caches(g, case, ns):
    shape, kind, vname = case
    B, Hq, Hkv, D, S, layout, kv, qo = SHAPES[shape]
    v = dict(VARIANTS)[vname]
    say(f"variants mapped {case} splits={ns}")
    w = W.custom(B, Hq, Hkv, D, S, layout, kv, qo, seed=B * 3 + D + Hq, stale="pm:1000")
    L = _lengths(B, S, S + 1)
    inp = W.make_inputs(w, DEV, lengths=L)
    m = W.make_mapped(inp, w, kind, block_size=16)
    table = m["map"]
    sm, okw = _softmax(g, v, B, Hq, 9)
    ref, rk, rv = oracle.step_variants(np_of(inp["q"]), qo, np_of(m["k_cache"]), np_of(m["v_cache"]),
                                       np_of(inp["k_new"]), np_of(inp["v_new"]), kv, L.numpy(), layout, Hq, Hkv,
                                       kind=kind, mapping=table.cpu().numpy(), bs=m.get("block_size"), **okw)
    out = g.step_ex(inp["q"], m["k_cache"], m["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout=layout,
                    table=table, kind=kind, table_host=table.cpu(), softmax=sm, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, qo, "step")
    assert np_of(m["k_cache"]).tobytes() == rk.tobytes()
    assert np_of(m["v_cache"]).tobytes() == rv.tobytes()


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("vname", ["winpre", "all", "cap", "sink"])
@pytest.mark.parametrize("ns", [0, 3])
@pytest.mark.parametrize("shape", [(3, 32, 8), (2, 64, 1)], ids=["G4", "G64"])
def test_variants_on_quantized_caches(g, vname, ns, shape, kv):
    """Int8 and fp8 (E4M3) caches with per-row scales under every softmax
    variant: outputs within the bf16 tolerance, appended codes and scales
    byte-exact."""
    B, Hq, Hkv = shape
    D, S, layout = 128, 800, "BHSD"
    v = dict(VARIANTS)[vname]
    say(f"variants {kv} {vname} splits={ns} shape={shape}")
    w = W.custom(B, Hq, Hkv, D, S, layout, kv, "bf16", seed=77, stale="pm:1")
    L = _lengths(B, S, 5)
    inp = W.make_q8(w, DEV, lengths=L)
    sm, okw = _softmax(g, v, B, Hq, 21)
    ref, rk, rv, rks, rvs = oracle.step_variants(np_of(inp["q"]), "bf16", np_of(inp["k_cache"]),
                                                 np_of(inp["v_cache"]), np_of(inp["k_new"]), np_of(inp["v_new"]),
                                                 kv, L.numpy(), layout, Hq, Hkv,
                                                 scales=(np_of(inp["k_scale"]), np_of(inp["v_scale"])), **okw)
    out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                    layout=layout, k_scale=inp["k_scale"], v_scale=inp["v_scale"], softmax=sm, num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    for name, want in (("k_cache", rk), ("v_cache", rv), ("k_scale", rks), ("v_scale", rvs)):
        assert np_of(inp[name]).tobytes() == want.tobytes(), name


def test_window_skips_the_middle_of_a_long_sequence(g):
    """A 64-slot window plus a 16-slot prefix over 100k cached slots, long
    context shape: sampled heads against the oracle, and the step runs in a
    small fraction of the full-context step's time (the skipped slots are not
    read)."""
    B, Hq, Hkv, D, S = 2, 32, 8, 128, 100_001
    w = W.custom(B, Hq, Hkv, D, S, "BHSD", "bf16", "bf16", seed=12)
    L = torch.full((B,), S - 1, dtype=torch.int32)
    inp = W.make_inputs(w, DEV, lengths=L)
    sm = g.Softmax(window=64, kept_prefix=16)
    out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                    layout="BHSD", softmax=sm)
    torch.cuda.synchronize()
    q = oracle.decode(np_of(inp["q"]), "bf16")
    got = out.float().cpu().double().numpy()
    n = S
    idx = oracle.attended_slots(n, 64, 16)
    for b, hq in ((0, 0), (1, 17), (0, 31)):
        h = hq // 4
        K = oracle.decode(np_of(inp["k_cache"][b, h, idx]), "bf16")
        Vv = oracle.decode(np_of(inp["v_cache"][b, h, idx]), "bf16")
        ref = oracle.attend_variant_one(q[b, hq], K, Vv)
        assert np.all(np.abs(got[b, hq] - ref) <= 1e-2 + 1e-2 * np.abs(ref))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for _ in range(20):
        g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                  layout="BHSD", softmax=sm)
    ev[1].record()
    for _ in range(20):
        g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"], layout="BHSD")
    ev[2].record()
    torch.cuda.synchronize()
    t_win, t_full = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    say(f"window step {t_win / 20 * 1e3:.1f} us, full step {t_full / 20 * 1e3:.1f} us")
    assert t_win < 0.25 * t_full


# Rotary step and softmax variants in one call, on each kernel family that
# takes both (the options combine in one gqa_decode_opts_t).  The reference
# composes the two oracles: q and the new key rotated first (rope oracle), then
# the variant softmax over the appended cache with the rotated query.
COMBINED = [
    # B, Hq, Hkv, S, layout, kv/qo, num_splits, map kind
    (3, 32, 8, 700, "BHSD", "bf16", 0, None),     # G = 4, register-operand kernel (rotated copy of q)
    (2, 64, 1, 900, "BSHD", "bf16", 0, None),     # G = 64, split form (rotation fused)
    (260, 64, 1, 200, "BHSD", "bf16", 0, None),   # G = 64, whole-item form
    (3, 48, 2, 500, "BSHD", "bf16", 1, "slots"),  # G = 24, whole-item form on slot-indexed rows
    (3, 8, 2, 300, "BHSD", "f32", 3, None),       # D = 64 below: generic kernel
]


@pytest.mark.parametrize("case", COMBINED, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}{c[4]}-{c[5]}-n{c[6]}-{c[7]}" for c in COMBINED])
def test_rotary_step_with_variants(g, case):
    B, Hq, Hkv, S, layout, dt, ns, kind = case
    D = 64 if dt == "f32" else 128
    say(f"rope + variants {case}")
    w = W.custom(B, Hq, Hkv, D, S, layout, dt, dt, seed=B + Hq + S, stale="pm:1000")
    L = _lengths(B, S, S + 11)
    inp = W.make_inputs(w, DEV, lengths=L)
    cos, sin = W.rope_tables(S + 8, D, DEV)
    rope = g.Rope(cos, sin, "half")
    gen = torch.Generator().manual_seed(12)
    sink = (torch.randn(Hq, generator=gen) * 2).to(DEV)
    sm = g.Softmax(sink=sink, softcap=2.0, window=90, kept_prefix=16)
    qr, kr = oracle.rotate_new(np_of(inp["q"]), dt, np_of(inp["k_new"]), dt, L.numpy(), cos.cpu().numpy(),
                               sin.cpu().numpy(), "half")
    kc, vc, table, okw = inp["k_cache"], inp["v_cache"], None, {}
    if kind is not None:
        m = W.make_mapped(inp, w, kind)
        kc, vc, table = m["k_cache"], m["v_cache"], m["map"]
        okw = dict(kind=kind, mapping=table.cpu().numpy(), bs=m.get("block_size"))
    ref, rk, rv = oracle.step_variants(qr.astype(np.float32), "f32", np_of(kc), np_of(vc), kr, np_of(inp["v_new"]), dt,
                                       L.numpy(), layout, Hq, Hkv, sink=sink.cpu().numpy(), softcap=2.0, window=90,
                                       prefix=16, **okw)
    out = g.step_ex(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], layout=layout, table=table,
                    kind=kind, table_host=None if table is None else table.cpu(), rope=rope, softmax=sm,
                    num_splits=ns)
    torch.cuda.synchronize()
    assert_close(out, ref, dt, "step")
    assert np_of(kc).tobytes() == rk.tobytes()
    assert np_of(vc).tobytes() == rv.tobytes()


@pytest.mark.parametrize("kv", ["i8", "fp8"])
@pytest.mark.parametrize("shape", [(3, 32, 8, 700, "BHSD"), (2, 64, 1, 600, "BSHD")], ids=["G4", "G64"])
def test_rotary_step_with_variants_on_quantized_caches(g, shape, kv):
    """The same on int8 and fp8 caches with row scales: the rotated new key
    (bf16) quantized into the cache, codes and scales byte-exact."""
    B, Hq, Hkv, S, layout = shape
    say(f"rope + variants {kv} {shape}")
    w = W.custom(B, Hq, Hkv, 128, S, layout, kv, "bf16", seed=B + Hq + 5)
    L = _lengths(B, S, S + 13)
    inp = W.make_q8(w, DEV, lengths=L)
    cos, sin = W.rope_tables(S + 8, 128, DEV)
    rope = g.Rope(cos, sin, "interleaved")
    gen = torch.Generator().manual_seed(14)
    sink = (torch.randn(Hq, generator=gen) * 2).to(DEV)
    sm = g.Softmax(sink=sink, softcap=2.0, window=90, kept_prefix=16)
    # As the quantized rotary oracle composes it: q and the new key rotated in
    # float32 (the key quantized from there, q used unrounded), the value exact.
    cs, sn = cos.cpu().numpy(), sin.cpu().numpy()
    q32 = oracle.decode(np_of(inp["q"]), "bf16").astype(np.float32)
    k32 = oracle.decode(np_of(inp["k_new"]), "bf16").astype(np.float32)
    qr, kr = np.empty_like(q32), np.empty_like(k32)
    for b in range(B):
        p = int(L[b])
        qr[b] = oracle.rope_rotate(q32[b], cs[p], sn[p], "interleaved")
        kr[b] = oracle.rope_rotate(k32[b], cs[p], sn[p], "interleaved")
    vn = oracle.decode(np_of(inp["v_new"]), "bf16").astype(np.float32)
    ref, rk, rv, rks, rvs = oracle.step_variants(qr, "f32", np_of(inp["k_cache"]), np_of(inp["v_cache"]), kr, vn, kv,
                                                 L.numpy(), layout, Hq, Hkv,
                                                 scales=(np_of(inp["k_scale"]), np_of(inp["v_scale"])),
                                                 sink=sink.cpu().numpy(), softcap=2.0, window=90, prefix=16)
    out = g.step_ex(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                    layout=layout, k_scale=inp["k_scale"], v_scale=inp["v_scale"], rope=rope, softmax=sm)
    torch.cuda.synchronize()
    assert_close(out, ref, "bf16", "step")
    for name, want in (("k_cache", rk), ("v_cache", rv), ("k_scale", rks), ("v_scale", rvs)):
        assert np_of(inp[name]).tobytes() == want.tobytes(), name

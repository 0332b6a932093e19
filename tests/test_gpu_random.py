"""GPU parity on seeded random shapes and options.

Each case draws a kernel family (small-head, generic, register-operand,
large-group split or whole-item, 8-bit caches, balanced mode), then a batch, group size, head
width, capacity, layout, cache and q/out storage types, a forced split count
(or the plan's), a step or an attend call, and ragged lengths that include a
full sequence and (for B > 1) one attending a single slot (a step from an
empty cache, or an attend over one valid slot).  Only combinations the library
serves are drawn (fp8 caches: head width 128, bf16 q/out, G <= 64), so the
plan the library picks -- small, generic, register-operand or large-group
kernel, split or balanced, with or without a combine pass -- must run and
match the float64 oracle: outputs
within the dtype's tolerance (f32 2e-5, bf16 1e-2, abs + rel), appended cache
rows, codes and scales byte-exact.  Stale slots hold finite values of
magnitude 100, which a read of them would show.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-5, "bf16": 1e-2}
DEV = "cuda"
CODE = {"f32": 0, "bf16": 1, "i8": 2, "fp8": 3}


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_amd as lib
    lib.lib()
    return lib


def np_of(t):
    return W.to_numpy_storage(t)


def assert_close(out_gpu, ref, qo, what):
    got = out_gpu.detach().float().cpu().double().numpy()
    err = np.abs(got - ref)
    bound = TOL[qo] + TOL[qo] * np.abs(ref)
    bad = ~(err <= bound)
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst excess "
                           f"{np.max(err - bound):.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def draw(seed):
    """One case: a kernel family first (so every kernel and mode is drawn
    often), then the shape and options within it."""
    rng = np.random.default_rng(7000 + seed)
    fam = ["small", "generic", "qk", "all", "q8", "balanced", "whole"][seed % 7]
    Hkv = int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 5))
    S = int(rng.integers(1, 420))
    qo = str(rng.choice(["f32", "bf16"]))
    if fam == "small":                       # f32 / bf16 caches, head width <= 16, capacity <= 512
        kv, D, G = str(rng.choice(["f32", "bf16"])), int(rng.choice([1, 2, 4, 8, 16])), int(rng.choice([1, 2, 3, 4, 8]))
    elif fam == "generic":                   # any head width up to 256
        kv, D, G = str(rng.choice(["f32", "bf16"])), int(rng.choice([24, 64, 100, 128, 256])), int(rng.choice([1, 2, 5, 8, 12]))
        if kv == "bf16" and qo == "bf16" and D == 128:
            qo = "f32"                       # (bf16 / bf16 / 128 is a matrix-core shape)
    elif fam == "qk":                        # G <= 16 on the register-operand kernel
        kv, qo, D, G = "bf16", "bf16", 128, int(rng.choice([1, 2, 4, 8, 12, 16]))
    elif fam == "all":                       # 16 < G <= 64 on the large-group kernel
        kv, qo, D, G, Hkv = "bf16", "bf16", 128, int(rng.choice([20, 24, 32, 40, 48, 64])), int(rng.choice([1, 2]))
    elif fam == "q8":                        # int8 or fp8 codes with row scales
        kv, qo, D, G = str(rng.choice(["i8", "fp8"])), "bf16", 128, int(rng.choice([1, 4, 8, 16, 24, 32, 64]))
        Hkv = min(Hkv, 2)
    elif fam == "balanced":                  # more (sequence, kv-head) items than CUs: balanced mode
        kv, qo, D, G = str(rng.choice(["bf16", "i8", "fp8"])), "bf16", 128, int(rng.choice([1, 2, 4, 8]))
        Hkv, B, S = 8, int(rng.integers(33, 48)), int(rng.integers(1, 120))
    else:                                    # 16 < G <= 64 with items filling the CUs: whole-item form
        kv, qo, D, G = "bf16", "bf16", 128, int(rng.choice([17, 24, 32, 40, 48, 64]))
        Hkv = int(rng.choice([1, 2]))
        B, S = int(rng.integers(256, 300)) // Hkv, int(rng.integers(1, 200))
    layout = str(rng.choice(["BHSD", "BSHD"]))
    ns = 0 if fam in ("balanced", "whole") else int(rng.choice([0, 0, 0, 1, 2, 3, 7]))
    mode = str(rng.choice(["step", "attend"]))
    if mode == "step":
        L = rng.integers(0, S, B)             # pre-append counts in [0, S - 1]
        L[0] = S - 1
        if B > 1:
            L[1] = 0                          # only the new token
    else:
        L = rng.integers(1, S + 1, B)         # valid counts in [1, S]
        L[0] = S
        if B > 1:
            L[1] = 1
    return dict(seed=7000 + seed, fam=fam, kv=kv, qo=qo, B=B, Hq=Hkv * G, Hkv=Hkv, D=D, S=S, layout=layout,
                ns=ns, mode=mode, L=torch.from_numpy(L.astype(np.int32)))


CASES = [draw(s) for s in range(56)]


def _id(c):
    return (f"{c['seed']}-{c['fam']}-{c['mode']}-B{c['B']}Hq{c['Hq']}Hkv{c['Hkv']}D{c['D']}S{c['S']}{c['layout']}"
            f"-{c['kv']}-{c['qo']}-n{c['ns']}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_case(g, case):
    c = case
    w = W.custom(c["B"], c["Hq"], c["Hkv"], c["D"], c["S"], c["layout"], c["kv"], c["qo"],
                 seed=c["seed"], stale="pm:100")
    desc = g.make_desc(c["B"], c["Hq"], c["Hkv"], c["D"], c["S"], c["layout"], CODE[c["kv"]], CODE[c["qo"]], c["ns"])
    print(f"random {_id(c)} plan {g.get_plan(desc)}", flush=True)
    q8 = c["kv"] in ("i8", "fp8")
    L = c["L"]
    inp = W.make_q8(w, DEV, lengths=L) if q8 else W.make_inputs(w, DEV, lengths=L)
    args = (np_of(inp["q"]), c["qo"])
    Ln = L.numpy()
    if c["mode"] == "step":
        if q8:
            ref, rk, rv, rks, rvs = oracle.step_q8(*args, np_of(inp["k_cache"]), np_of(inp["v_cache"]),
                                                   np_of(inp["k_scale"]), np_of(inp["v_scale"]), np_of(inp["k_new"]),
                                                   np_of(inp["v_new"]), Ln, c["layout"], c["Hq"], c["Hkv"])
            out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                            inp["v_new"], inp["lengths"], layout=c["layout"], num_splits=c["ns"])
            want = {"k_cache": rk, "v_cache": rv, "k_scale": rks, "v_scale": rvs}
        else:
            ref, rk, rv = oracle.step(*args, np_of(inp["k_cache"]), np_of(inp["v_cache"]), np_of(inp["k_new"]),
                                      np_of(inp["v_new"]), c["kv"], Ln, c["layout"], c["Hq"], c["Hkv"])
            out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                         layout=c["layout"], num_splits=c["ns"])
            want = {"k_cache": rk, "v_cache": rv}
    else:
        if q8:
            ref = oracle.attend_q8(*args, np_of(inp["k_cache"]), np_of(inp["v_cache"]), np_of(inp["k_scale"]),
                                   np_of(inp["v_scale"]), Ln, c["layout"], c["Hq"], c["Hkv"])
            out = g.attend_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"],
                              inp["lengths"], layout=c["layout"], num_splits=c["ns"])
        else:
            ref = oracle.attend(*args, np_of(inp["k_cache"]), np_of(inp["v_cache"]), c["kv"], Ln, c["layout"],
                                c["Hq"], c["Hkv"])
            out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout=c["layout"],
                           num_splits=c["ns"])
        want = {}
    torch.cuda.synchronize()
    assert_close(out, ref, c["qo"], _id(c))
    for name, expect in want.items():
        assert np_of(inp[name]).tobytes() == expect.tobytes(), name

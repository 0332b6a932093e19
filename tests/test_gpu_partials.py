"""Float32 arithmetic of the attention passes, below the output's rounding.

JAX "Grouped-Query Decode Step" page, requirements: scores, softmax and the
weighted sum are float32.  A bf16 output (rounding 2^-9) hides whether the
weights entered the V sum at bf16 or at float32 precision, so these tests
force a split of the token axis and read the float32 split partials (m, l, o)
the attention pass leaves in the caller's workspace (layout documented with
gqa_decode_attend in include/gqa_decode.h).  For every (b, query head, split)
with valid slots, o / l is the softmax-weighted mean of V over that split's
slots, and must match the oracle restricted to those slots within the float32
tolerance, 2e-5 + 2e-5 |ref| elementwise.  Weights rounded to bf16 alone would
miss it by about 1e-4 on these inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = 2e-5


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_amd as lib
    lib.lib()
    return lib


def align256(x):
    return (x + 255) // 256 * 256


CASES = {
    # name: (B, Hq, Hkv, S, layout, kv, qo, num_splits, key_scale, attended counts, kernel)
    "mfma_qk_g4": (3, 32, 8, 2100, "BHSD", "bf16", "bf16", 4, 1.0, [2100, 1500, 700], "mfma_qk"),
    "mfma_qk_g8_bshd_keys3": (2, 16, 2, 1900, "BSHD", "bf16", "bf16", 3, 3.0, [1900, 1000], "mfma_qk"),
    "mfma_qk_g16_int8": (2, 32, 2, 1700, "BHSD", "i8", "bf16", 3, 1.0, [1700, 1200], "mfma_qk"),
    "mfma_all_g64": (2, 64, 1, 2100, "BHSD", "bf16", "bf16", 4, 1.0, [2100, 1300], "mfma_all"),
    "mfma_all_g32_keys3": (2, 64, 2, 1600, "BSHD", "bf16", "bf16", 3, 3.0, [1600, 900], "mfma_all"),
    "mfma_qk_g64_int8": (2, 64, 1, 1800, "BHSD", "i8", "bf16", 3, 1.0, [1800, 1100], "mfma_qk"),
    "mfma_qk_g24_int8_bshd": (2, 48, 2, 1500, "BSHD", "i8", "bf16", 3, 1.0, [1500, 900], "mfma_qk"),
    "mfma_qk_g8_fp8": (2, 32, 4, 1700, "BHSD", "fp8", "bf16", 3, 1.0, [1700, 1200], "mfma_qk"),
    "mfma_qk_g16_fp8_bshd_four_heads": (2, 64, 4, 1500, "BSHD", "fp8", "bf16", 3, 1.0, [1500, 700], "mfma_qk"),
    "mfma_qk_g4_bshd_four_heads": (2, 32, 8, 1900, "BSHD", "bf16", "bf16", 3, 1.0, [1900, 1000], "mfma_qk"),
    "mfma_qk_g16_int8_bshd_four_heads": (2, 64, 4, 1500, "BSHD", "i8", "bf16", 3, 1.0, [1500, 700], "mfma_qk"),
    "generic_bf16_caches_f32_out": (2, 16, 4, 1500, "BHSD", "bf16", "f32", 3, 1.0, [1500, 800], "generic"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_split_partials_are_float32_accurate(g, case):
    B, Hq, Hkv, S, lay, kv, qo, ns, ks, n_att, kernel = CASES[case]
    D = 128
    w = W.custom(B, Hq, Hkv, D, S, lay, kv, qo, seed=400 + Hq + S, key_scale=ks)
    n = torch.tensor(n_att, dtype=torch.int32)
    code = {"bf16": g.BF16, "f32": g.F32, "i8": g.I8, "fp8": g.FP8}
    desc = g.make_desc(B, Hq, Hkv, D, S, lay, code[kv], code[qo], ns)
    plan = g.get_plan(desc)
    print(f"partials {case}: plan {plan}", flush=True)
    assert plan["kernel"] == kernel and not plan["balanced"] and plan["num_splits"] == ns
    assert plan["heads_per_item"] == (4 if case.endswith("four_heads") else 1)
    st = plan["split_tokens"]
    ws = torch.full((plan["workspace_bytes"],), 0xFF, dtype=torch.uint8, device=DEV)
    if kv in ("i8", "fp8"):
        inp = W.make_q8(w, DEV, lengths=n)
        g.attend_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["lengths"],
                    layout=lay, workspace=ws, num_splits=ns)
    else:
        inp = W.make_inputs(w, DEV, lengths=n)
        g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout=lay, workspace=ws, num_splits=ns)
    torch.cuda.synchronize()
    rows = B * Hq * ns
    off_m = align256(4 * rows * D)
    off_l = off_m + align256(4 * rows)
    wsh = ws.cpu()
    part_o = wsh[: 4 * rows * D].view(torch.float32).double().numpy().reshape(B, Hq, ns, D)
    part_m = wsh[off_m: off_m + 4 * rows].view(torch.float32).double().numpy().reshape(B, Hq, ns)
    part_l = wsh[off_l: off_l + 4 * rows].view(torch.float32).double().numpy().reshape(B, Hq, ns)
    q = oracle.decode(W.to_numpy_storage(inp["q"]), qo)
    G = Hq // Hkv
    checked = 0
    for b in range(B):
        nb = int(n_att[b])
        nact = min(ns, -(-nb // st))
        if nact <= 1:
            continue
        for h in range(Hkv):
            idx = (lambda j0, j1: (b, h, slice(j0, j1))) if lay == "BHSD" else (lambda j0, j1: (b, slice(j0, j1), h))
            for s in range(nact):
                t0, t1 = s * st, min((s + 1) * st, nb)
                if kv in ("i8", "fp8"):
                    sl = idx(t0, t1)
                    K = oracle.dequantize(W.to_numpy_storage(inp["k_cache"][sl]), inp["k_scale"][sl].cpu().numpy())
                    V = oracle.dequantize(W.to_numpy_storage(inp["v_cache"][sl]), inp["v_scale"][sl].cpu().numpy())
                else:
                    K = oracle.decode(W.to_numpy_storage(inp["k_cache"][idx(t0, t1)]), kv)
                    V = oracle.decode(W.to_numpy_storage(inp["v_cache"][idx(t0, t1)]), kv)
                for hq in range(h * G, (h + 1) * G):
                    ref = oracle.attend_one(q[b, hq], K, V)
                    assert np.isfinite(part_m[b, hq, s]) and part_l[b, hq, s] > 0, (b, hq, s)
                    got = part_o[b, hq, s] / part_l[b, hq, s]
                    err = np.abs(got - ref)
                    bound = TOL + TOL * np.abs(ref)
                    assert np.all(err <= bound), (case, b, hq, s, float(np.max(err - bound)), float(err.max()))
                    checked += 1
    assert checked > 0

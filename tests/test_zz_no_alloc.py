"""The decode step without a caller workspace (include/gqa_decode_static.h),
for callers that cannot allocate: called through the C ABI and compared with
gqa_decode_step on the same inputs -- the same kernels and plan, so the outputs
and appended caches must be bitwise equal -- on two calls in a row, the second
with a smaller batch, over split plans (large group, long context) and a
balanced plan (ragged batch)."""
import ctypes

import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_decode_attention_amd as lib
    L = lib.lib()
    P = ctypes.c_void_p
    L.gqa_decode_step_static.argtypes = [ctypes.POINTER(lib.Desc), P, P, P, P, P, P, P, P]
    L.gqa_decode_step_static.restype = ctypes.c_int
    return lib


def step_static(g, inp, layout, num_splits=0):
    desc = g.desc_for(inp["q"], inp["k_cache"], layout, num_splits)
    out = torch.empty_like(inp["q"])
    st = g.lib().gqa_decode_step_static(ctypes.byref(desc), inp["q"].data_ptr(), inp["k_cache"].data_ptr(),
                                        inp["v_cache"].data_ptr(), inp["k_new"].data_ptr(), inp["v_new"].data_ptr(),
                                        inp["lengths"].data_ptr(), out.data_ptr(),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, g.GqaError(st, "gqa_decode_step_static")
    return out


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


CASES = [
    # (B, Hq, Hkv, S, layout, smaller B, num_splits): plans with a workspace
    (96, 64, 1, 2048, "BHSD", 40, 0),       # large group: split partials
    (4, 32, 8, 20000, "BHSD", 2, 0),        # long context: split partials
    (48, 64, 8, 3000, "BSHD", 36, 0),       # ragged: balanced tile offsets and partials
    (3, 32, 8, 2500, "BHSD", 2, 7),         # forced splits
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}Hq{c[1]}Hkv{c[2]}S{c[3]}{c[4]}n{c[6]}" for c in CASES])
def test_static_step_matches_step(g, case):
    B, Hq, Hkv, S, lay, B2, ns = case
    for rep, nb in enumerate((B, B2)):
        w = W.custom(nb, Hq, Hkv, 128, S, lay, "bf16", "bf16", seed=600 + rep + B, stale="pm:100")
        L = torch.randint(0, S, (nb,), generator=torch.Generator().manual_seed(601 + rep), dtype=torch.int32)
        inp = W.make_inputs(w, DEV, lengths=L)
        ref_inp = {k: v.clone() for k, v in inp.items()}
        desc = g.desc_for(inp["q"], inp["k_cache"], lay, ns)
        plan = g.get_plan(desc)
        print(f"static step {case} call {rep}: B={nb} plan {plan}", flush=True)
        assert plan["workspace_bytes"] > 0
        got = step_static(g, inp, lay, ns)
        want = g.step(ref_inp["q"], ref_inp["k_cache"], ref_inp["v_cache"], ref_inp["k_new"], ref_inp["v_new"],
                      ref_inp["lengths"], layout=lay, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(want)), f"call {rep}"
        assert torch.equal(bits(inp["k_cache"]), bits(ref_inp["k_cache"]))
        assert torch.equal(bits(inp["v_cache"]), bits(ref_inp["v_cache"]))


def test_static_step_refuses_plans_beyond_its_scratch(g):
    # 4096 sequences x 64 heads x 64 forced splits of partials need far more than 32 MiB.
    desc = g.make_desc(4096, 64, 1, 128, 8192, "BHSD", g.BF16, g.BF16, 64)
    assert g.workspace_size(desc) > (32 << 20)
    st = g.lib().gqa_decode_step_static(ctypes.byref(desc), None, None, None, None, None, None, None, None)
    assert st == 3   # GQA_ERR_WORKSPACE_TOO_SMALL, before anything is enqueued

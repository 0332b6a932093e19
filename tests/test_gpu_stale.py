"""Stale slots are never loaded, on every kernel family.

JAX "Grouped-Query Decode Step" page, requirements: slots at or beyond a
sequence's valid count get zero weight whatever they hold.  A stronger check
than a tolerance: each case runs the same call twice, the second time with
every slot past the attended range refilled with NaN (keys) and +Inf (values)
-- for mapped caches also every pool row or block no sequence maps -- and the
two outputs must be bitwise equal and finite.  A kernel that loaded a stale
row and gave it weight 0 would turn the output into NaN (0 * Inf, NaN * 0).

Cases cover the small-group matrix-core kernel (split mode, both layouts,
forced splits, attend, four kv-heads per workgroup on BSHD caches; int8
caches with two 16-head blocks per wave), the
large-group matrix-core kernel (G = 24 and 64, split and whole-item mode), the generic vector kernel
(float32 and bf16 storage, D = 64 and G = 80), the small-head-width kernel
(D = 4 and 16), the balanced mode, and paged / slot-indexed caches, int8 and fp8 caches.  Int8 codes cannot hold NaN:
there the refill puts NaN in the stale slots' scales and -127 in their codes;
fp8 refills put NaN in both (the E4M3 NaN code 0x7F).
"""
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
    lib.lib()
    return lib


CASES = {
    # name: (B, Hq, Hkv, D, S, layout, kv, qo, num_splits, map, block_size, expected kernel, balanced)
    "mfma_qk_bhsd": (4, 32, 8, 128, 1200, "BHSD", "bf16", "bf16", 0, None, 0, "mfma_qk", False),
    "mfma_qk_bhsd_splits3": (4, 32, 8, 128, 1200, "BHSD", "bf16", "bf16", 3, None, 0, "mfma_qk", False),
    "mfma_qk_bshd_g16": (3, 32, 2, 128, 900, "BSHD", "bf16", "bf16", 0, None, 0, "mfma_qk", False),
    "mfma_all_g64": (3, 64, 1, 128, 1500, "BHSD", "bf16", "bf16", 0, None, 0, "mfma_all", False),
    "mfma_all_g24_bshd_splits3": (2, 48, 2, 128, 700, "BSHD", "bf16", "bf16", 3, None, 0, "mfma_all", False),
    "generic_f32_d64": (3, 16, 4, 64, 900, "BHSD", "f32", "f32", 0, None, 0, "generic", False),
    "generic_bf16_d64_bshd": (3, 16, 2, 64, 700, "BSHD", "bf16", "bf16", 2, None, 0, "generic", False),
    "generic_bf16_g80": (2, 80, 1, 128, 400, "BHSD", "bf16", "bf16", 0, None, 0, "generic", False),
    "generic_f32_d128_f32_out": (2, 16, 4, 128, 600, "BSHD", "f32", "f32", 3, None, 0, "generic", False),
    "balanced_bhsd": (40, 32, 8, 128, 600, "BHSD", "bf16", "bf16", 0, None, 0, "mfma_qk", True),
    "balanced_bshd": (40, 32, 8, 128, 600, "BSHD", "bf16", "bf16", 0, None, 0, "mfma_qk", True),
    "paged16_mfma_qk": (3, 32, 8, 128, 800, "BHSD", "bf16", "bf16", 0, "paged", 16, "mfma_qk", False),
    "paged32_mfma_all": (2, 64, 1, 128, 900, "BSHD", "bf16", "bf16", 0, "paged", 32, "mfma_all", False),
    "paged7_generic_f32": (3, 8, 2, 64, 300, "BHSD", "f32", "f32", 0, "paged", 7, "generic", False),
    "slots_mfma_qk": (3, 32, 8, 128, 700, "BSHD", "bf16", "bf16", 0, "slots", 0, "mfma_qk", False),
    "mfma_qk_bshd_four_heads_splits3": (3, 32, 8, 128, 900, "BSHD", "bf16", "bf16", 3, None, 0, "mfma_qk", False),
    "mfma_qk_int8_bshd_four_heads": (3, 64, 4, 128, 900, "BSHD", "i8", "bf16", 0, None, 0, "mfma_qk", False),
    "paged16_bshd_four_heads": (3, 32, 8, 128, 800, "BSHD", "bf16", "bf16", 0, "paged", 16, "mfma_qk", False),
    "small_f32_d4": (3, 4, 2, 4, 200, "BHSD", "f32", "f32", 0, None, 0, "small", False),
    "small_bf16_d16_paged5": (3, 8, 2, 16, 200, "BSHD", "bf16", "bf16", 0, "paged", 5, "small", False),
    "mfma_qk_g32_two_blocks_int8": (3, 64, 2, 128, 900, "BHSD", "i8", "bf16", 0, None, 0, "mfma_qk", False),
    "mfma_qk_g64_two_blocks_int8": (2, 64, 1, 128, 1100, "BSHD", "i8", "bf16", 3, None, 0, "mfma_qk", False),
    "mfma_qk_fp8_bhsd": (3, 32, 8, 128, 900, "BHSD", "fp8", "bf16", 0, None, 0, "mfma_qk", False),
    "mfma_qk_fp8_bshd_four_heads_splits3": (3, 32, 8, 128, 900, "BSHD", "fp8", "bf16", 3, None, 0, "mfma_qk", False),
    "mfma_qk_fp8_g64_two_blocks": (2, 64, 1, 128, 1100, "BHSD", "fp8", "bf16", 0, None, 0, "mfma_qk", False),
    "paged16_fp8": (3, 32, 8, 128, 800, "BHSD", "fp8", "bf16", 0, "paged", 16, "mfma_qk", False),
    # the large-group kernel's whole-item mode (one split: no partials, sub-tile waves merged in LDS)
    "mfma_all_whole_g64": (3, 64, 1, 128, 1500, "BHSD", "bf16", "bf16", 1, None, 0, "mfma_all", False),
    "mfma_all_whole_g24_bshd": (2, 48, 2, 128, 700, "BSHD", "bf16", "bf16", 1, None, 0, "mfma_all", False),
    "slots_mfma_all_whole": (3, 64, 1, 128, 700, "BSHD", "bf16", "bf16", 1, "slots", 0, "mfma_all", False),
    "paged32_mfma_all_one_split": (2, 64, 1, 128, 900, "BSHD", "bf16", "bf16", 1, "paged", 32, "mfma_all", False),
    "mfma_all_whole_four_blocks": (260, 64, 1, 128, 200, "BHSD", "bf16", "bf16", 0, None, 0, "mfma_all", False),
}


def refill(inp, w, n_att):
    """Copies of the caches with every slot j >= n_att[b] set to NaN (K) / +Inf (V);
    int8 caches: NaN scales and codes of -127 there; fp8 caches: NaN scales and NaN codes."""
    slot = torch.arange(w.capacity, device=DEV)
    stale = slot[None, :] >= n_att.to(DEV).long()[:, None]
    row = stale[:, None, :] if w.layout == "BHSD" else stale[:, :, None]   # the scales' shape
    stale = row[..., None]                                                 # the caches' shape
    out = dict(inp)
    if w.kv_dtype == "fp8":
        for name in ("k_cache", "v_cache"):
            c = inp[name].view(torch.uint8)
            out[name] = torch.where(stale, torch.tensor(0x7F, dtype=torch.uint8, device=DEV), c).view(torch.float8_e4m3fn)
        for name in ("k_scale", "v_scale"):
            out[name] = torch.where(row, torch.tensor(float("nan"), device=DEV), inp[name])
        return out
    if w.kv_dtype == "i8":
        for name in ("k_cache", "v_cache"):
            out[name] = torch.where(stale, torch.tensor(-127, dtype=torch.int8, device=DEV), inp[name])
        for name in ("k_scale", "v_scale"):
            out[name] = torch.where(row, torch.tensor(float("nan"), device=DEV), inp[name])
        return out
    for name, fill in (("k_cache", float("nan")), ("v_cache", float("inf"))):
        c = inp[name]
        out[name] = torch.where(stale, torch.tensor(fill, dtype=c.dtype, device=DEV), c)
    return out


def same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("call", ["step", "attend"])
def test_stale_slots_never_loaded(g, case, call):
    B, Hq, Hkv, D, S, lay, kv, qo, ns, kind, bs, kernel, balanced = CASES[case]
    quant = kv in ("i8", "fp8")
    w = W.custom(B, Hq, Hkv, D, S, lay, kv, qo, seed=300 + B + Hq, stale="none" if quant else "pm:1000")
    L = torch.randint(0, S, (B,), generator=torch.Generator().manual_seed(S + B), dtype=torch.int32)
    L[0] = S - 1 if call == "step" else S
    L[1] = 0 if call == "step" else 1
    if call == "attend":
        L = L.clamp(min=1)
    code = {"f32": g.F32, "bf16": g.BF16, "i8": g.I8, "fp8": g.FP8}
    desc = g.make_desc(B, Hq, Hkv, D, S, lay, code[kv], code[qo], ns)
    plan = g.get_plan(desc)
    print(f"stale refill {case} {call}: plan {plan}", flush=True)
    assert plan["kernel"] == kernel and plan["balanced"] == balanced
    n_att = L + 1 if call == "step" else L
    base = W.make_q8(w, DEV, lengths=L) if quant else W.make_inputs(w, DEV, lengths=L)
    runs = []
    for inp in (base, refill(base, w, n_att)):
        inp = {k: v.clone() for k, v in inp.items()}
        if kind is not None:
            m = W.make_mapped(inp, w, kind, block_size=bs or 16)    # same seed: the same table both times
            kc, vc, table = m["k_cache"], m["v_cache"], m["map"]
            if quant:
                sc = dict(k_scale=m["k_scale"], v_scale=m["v_scale"], table=table, kind=kind, table_host=table.cpu(),
                          layout=lay, num_splits=ns)
                out = (g.step_ex(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], **sc) if call == "step"
                       else g.attend_ex(inp["q"], kc, vc, inp["lengths"], **sc))
            elif call == "step":
                out = g.step_mapped(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], table, kind=kind,
                                    layout=lay, num_splits=ns)
            else:
                out = g.attend_mapped(inp["q"], kc, vc, inp["lengths"], table, kind=kind, layout=lay,
                                      num_splits=ns)
        elif quant and call == "step":
            out = g.step_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"], inp["k_new"],
                            inp["v_new"], inp["lengths"], layout=lay, num_splits=ns)
        elif quant:
            out = g.attend_q8(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_scale"], inp["v_scale"],
                              inp["lengths"], layout=lay, num_splits=ns)
        elif call == "step":
            out = g.step(inp["q"], inp["k_cache"], inp["v_cache"], inp["k_new"], inp["v_new"], inp["lengths"],
                         layout=lay, num_splits=ns)
        else:
            out = g.attend(inp["q"], inp["k_cache"], inp["v_cache"], inp["lengths"], layout=lay, num_splits=ns)
        runs.append(out)
    torch.cuda.synchronize()
    assert torch.isfinite(runs[0].float()).all() and torch.isfinite(runs[1].float()).all()
    assert same_bits(runs[0], runs[1])

"""C-ABI checks that need no GPU.

The library must load and export every function include/gqa_decode.h
declares; every malformed call must return its status before any HIP call.
Only calls that are invalid (or have batch 0) are made here: pointers are
fake host integers that the library never dereferences on these paths.
"""
import ctypes
import os
import re

import pytest

import torch

import gqa_decode_attention_amd as g
from gqa_decode_attention_amd import _lib

# The calls below pass fake pointers that must never reach a real device: a
# test bug that made one of them valid would launch a kernel on them.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-pointer ABI tests run only where no GPU is visible")

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "gqa_decode.h")
OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3

FAKE = 1 << 40          # 256-byte aligned fake device address: never dereferenced on error paths
GAP = 1 << 34           # spacing that keeps fake buffers disjoint


def header_functions(path=HEADER):
    text = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:gqa_status_t|const char\*|int32_t)\s+(gqa_decode_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    L = g.lib()
    names = header_functions()
    assert len(names) >= 7
    assert set(names) == set(_lib.EXPORTS)
    headers = sorted(f for f in os.listdir(INCLUDE) if f.endswith(".h"))
    for h in headers:
        for n in header_functions(os.path.join(INCLUDE, h)):
            assert hasattr(L, n), (h, n)


def test_status_strings_and_version():
    L = g.lib()
    for code, name in _lib.STATUS_NAMES.items():
        assert L.gqa_decode_status_string(code).decode() == name
    assert L.gqa_decode_status_string(99).decode() == "GQA_ERR_UNKNOWN"
    assert L.gqa_decode_version() >= 100


def desc(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, capacity=4096, layout="BHSD",
                kv_dtype=g.BF16, qo_dtype=g.BF16, num_splits=0)
    base.update(kw)
    return g.make_desc(**base)


BAD_DESCS = [
    (dict(batch=-1), INVALID),
    (dict(num_q_heads=0), INVALID),
    (dict(num_kv_heads=0), INVALID),
    (dict(num_q_heads=6, num_kv_heads=4), INVALID),     # Hq not a multiple of Hkv
    (dict(head_dim=0), INVALID),
    (dict(capacity=0), INVALID),
    (dict(kv_dtype=7), INVALID),
    (dict(qo_dtype=-1), INVALID),
    (dict(num_splits=-2), INVALID),
    (dict(head_dim=257), UNSUPPORTED),
    (dict(batch=1 << 30, capacity=1 << 30), UNSUPPORTED),   # byte count past 2^62
    (dict(batch=1, num_q_heads=1 << 23, num_kv_heads=1 << 23, head_dim=128, capacity=1),
     UNSUPPORTED),                                          # slot stride past 2^32 bytes
]


@pytest.mark.parametrize("kw,status", BAD_DESCS)
def test_bad_descriptor_rejected_everywhere(kw, status):
    L = g.lib()
    d = desc(**kw)
    n = ctypes.c_size_t(12345)
    assert L.gqa_decode_workspace_size(ctypes.byref(d), ctypes.byref(n)) == status
    assert n.value == 12345                                   # untouched on error
    p = _lib.PlanT()
    assert L.gqa_decode_get_plan(ctypes.byref(d), ctypes.byref(p)) == status
    ptrs = [FAKE + i * GAP for i in range(8)]
    assert L.gqa_decode_attend(ctypes.byref(d), ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], 1 << 30,
                               None) == status
    assert L.gqa_decode_step(ctypes.byref(d), ptrs[0], ptrs[1], ptrs[2], ptrs[6], ptrs[7], ptrs[3], ptrs[4],
                             ptrs[5], 1 << 30, None) == status
    assert L.gqa_decode_append(ctypes.byref(d), ptrs[1], ptrs[2], ptrs[6], ptrs[7], ptrs[3], None) == status


def test_fp8_caches_plan_the_matrix_core_kernel_or_are_refused():
    """fp8 (E4M3) caches run on the small-group matrix-core kernel (head width
    128, bf16 q/out, up to 64 query heads per kv-head, dense or mapped with
    16-slot blocks); any other shape is refused with UNSUPPORTED before anything
    is enqueued, and the plain (unquantized) calls refuse the type outright."""
    L = g.lib()
    for kw in (dict(), dict(num_q_heads=64, num_kv_heads=1), dict(layout="BSHD", num_q_heads=32, num_kv_heads=8),
               dict(num_q_heads=48, num_kv_heads=2, num_splits=3)):
        p = g.get_plan(desc(kv_dtype=g.FP8, **kw))
        assert p["kernel"] == "mfma_qk", (kw, p)
    for kw in (dict(head_dim=64), dict(qo_dtype=g.F32), dict(num_q_heads=80, num_kv_heads=1)):
        d = desc(kv_dtype=g.FP8, **kw)
        pt = _lib.PlanT()
        assert L.gqa_decode_get_plan(ctypes.byref(d), ctypes.byref(pt)) == UNSUPPORTED, kw
        n = ctypes.c_size_t(7)
        assert L.gqa_decode_workspace_size(ctypes.byref(d), ctypes.byref(n)) == UNSUPPORTED and n.value == 7
    d = desc(kv_dtype=g.FP8)
    ptrs = [FAKE + i * GAP for i in range(8)]
    assert L.gqa_decode_attend(ctypes.byref(d), ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4], ptrs[5], 1 << 30,
                               None) == INVALID       # no scales: the plain call refuses quantized caches


def test_null_desc_and_null_outputs():
    L = g.lib()
    assert L.gqa_decode_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == INVALID
    d = desc()
    assert L.gqa_decode_workspace_size(ctypes.byref(d), None) == INVALID
    assert L.gqa_decode_get_plan(ctypes.byref(d), None) == INVALID


def test_empty_batch_is_a_noop():
    """Batch 0 validates the descriptor and returns OK without touching pointers (all NULL)."""
    L = g.lib()
    d = desc(batch=0)
    assert L.gqa_decode_attend(ctypes.byref(d), None, None, None, None, None, None, 0, None) == OK
    assert L.gqa_decode_step(ctypes.byref(d), None, None, None, None, None, None, None, None, 0, None) == OK
    assert L.gqa_decode_append(ctypes.byref(d), None, None, None, None, None, None) == OK
    n = ctypes.c_size_t(1)
    assert L.gqa_decode_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK and n.value == 0


def test_check_lengths_argument_errors():
    """Every refusal happens before any HIP call (no GPU is touched here)."""
    L = g.lib()
    d = desc()
    n = ctypes.c_int32(-7)
    assert L.gqa_decode_check_lengths(ctypes.byref(d), FAKE, 2, None, ctypes.byref(n)) == INVALID   # bad mode
    assert L.gqa_decode_check_lengths(ctypes.byref(d), FAKE, 0, None, None) == INVALID              # no result
    assert L.gqa_decode_check_lengths(ctypes.byref(d), None, 0, None, ctypes.byref(n)) == INVALID   # no lengths
    assert L.gqa_decode_check_lengths(ctypes.byref(d), FAKE + 2, 1, None, ctypes.byref(n)) == INVALID  # misaligned
    assert L.gqa_decode_check_lengths(None, FAKE, 0, None, ctypes.byref(n)) == INVALID
    assert n.value == -7
    d0 = desc(batch=0)
    assert L.gqa_decode_check_lengths(ctypes.byref(d0), None, 1, None, ctypes.byref(n)) == OK
    assert n.value == 0


def _attend_ptrs():
    return dict(q=FAKE, kc=FAKE + GAP, vc=FAKE + 2 * GAP, lens=FAKE + 3 * GAP, out=FAKE + 4 * GAP,
                ws=FAKE + 5 * GAP, kn=FAKE + 6 * GAP, vn=FAKE + 7 * GAP)


def _attend(d, p, wsb):
    return g.lib().gqa_decode_attend(ctypes.byref(d), p["q"], p["kc"], p["vc"], p["lens"], p["out"], p["ws"], wsb,
                                     None)


def _step(d, p, wsb):
    return g.lib().gqa_decode_step(ctypes.byref(d), p["q"], p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], p["out"],
                                   p["ws"], wsb, None)


@pytest.mark.parametrize("call", [_attend, _step])
@pytest.mark.parametrize("field", ["q", "kc", "vc", "lens", "out"])
def test_null_pointer_rejected(call, field):
    d = desc()
    p = _attend_ptrs()
    p[field] = None
    assert call(d, p, 1 << 30) == INVALID


def test_step_null_new_kv_rejected():
    d = desc()
    for f in ("kn", "vn"):
        p = _attend_ptrs()
        p[f] = None
        assert _step(d, p, 1 << 30) == INVALID


@pytest.mark.parametrize("call", [_attend, _step])
def test_workspace_too_small(call):
    d = desc()
    need = g.workspace_size(d)
    assert need > 0
    assert call(d, _attend_ptrs(), need - 1) == WS_SMALL
    p = _attend_ptrs()
    p["ws"] = None
    assert call(d, p, need) == INVALID
    p = _attend_ptrs()
    p["ws"] += 16                                             # not 256-byte aligned
    assert call(d, p, need) == INVALID


@pytest.mark.parametrize("call", [_attend, _step])
@pytest.mark.parametrize("field,shift", [("q", 1), ("out", 1), ("kc", 1), ("vc", 1), ("lens", 2)])
def test_misaligned_pointer_rejected(call, field, shift):
    d = desc(kv_dtype=g.F32, qo_dtype=g.F32, head_dim=4)
    p = _attend_ptrs()
    p[field] += shift
    assert call(d, p, 1 << 30) == INVALID


@pytest.mark.parametrize("call", [_attend, _step])
@pytest.mark.parametrize("other", ["q", "kc", "vc", "lens", "ws"])
def test_output_overlapping_an_input_rejected(call, other):
    d = desc()
    p = _attend_ptrs()
    p["out"] = p[other]
    assert call(d, p, 1 << 30) == INVALID
    p = _attend_ptrs()
    p["out"] = p[other] - 256          # out's span reaches into the other buffer
    assert call(d, p, 1 << 30) == INVALID


def test_step_and_append_reject_aliased_caches():
    d = desc()
    p = _attend_ptrs()
    p["vc"] = p["kc"] + 512
    assert _step(d, p, 1 << 30) == INVALID
    assert g.lib().gqa_decode_append(ctypes.byref(d), p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], None) == INVALID
    p = _attend_ptrs()
    p["kn"] = p["vc"] + 1024
    assert _step(d, p, 1 << 30) == INVALID
    assert g.lib().gqa_decode_append(ctypes.byref(d), p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], None) == INVALID


def test_append_null_and_misaligned():
    L = g.lib()
    d = desc()
    p = _attend_ptrs()
    for f in ("kc", "vc", "kn", "vn", "lens"):
        q = dict(p)
        q[f] = None
        assert L.gqa_decode_append(ctypes.byref(d), q["kc"], q["vc"], q["kn"], q["vn"], q["lens"], None) == INVALID
        q = dict(p)
        q[f] += 1
        assert L.gqa_decode_append(ctypes.byref(d), q["kc"], q["vc"], q["kn"], q["vn"], q["lens"], None) == INVALID


def test_plan_is_a_function_of_the_descriptor_only():
    """Same descriptor -> same plan and workspace; the plan has no lengths input at all."""
    for kw in (dict(), dict(layout="BSHD"), dict(batch=64, num_q_heads=64, num_kv_heads=8, capacity=8192),
               dict(batch=4, num_q_heads=32, num_kv_heads=8, capacity=131073),
               dict(batch=128, num_q_heads=64, num_kv_heads=1, capacity=2048),
               dict(batch=2, num_q_heads=4, num_kv_heads=2, head_dim=4, capacity=8, kv_dtype=g.F32, qo_dtype=g.F32)):
        d = desc(**kw)
        p1, p2 = g.get_plan(d), g.get_plan(d)
        assert p1 == p2
        assert p1["workspace_bytes"] == g.workspace_size(d)
        assert p1["num_splits"] * p1["split_tokens"] >= d.capacity
        assert (p1["num_splits"] - 1) * p1["split_tokens"] < d.capacity     # no empty split
        assert p1["combine"] == (p1["num_splits"] > 1 or p1["balanced"])
        assert p1["num_splits"] <= 64
        # the workspace holds split partials, or the balanced mode's partials and tile offsets
        assert (p1["workspace_bytes"] == 0) == (p1["num_splits"] == 1 and not p1["balanced"])
        if p1["balanced"]:
            # more (b, kv-head) items than CUs: one workgroup per CU, two partial rows of G heads each
            assert p1["kernel"] == "mfma_qk" and p1["grid"] == 256 and p1["num_splits"] == 1
            assert d.batch * d.num_kv_heads > 256
            G = d.num_q_heads // d.num_kv_heads
            hp = p1["heads_per_item"]
            assert p1["workspace_bytes"] >= 256 * 2 * G * hp * (d.head_dim + 2) * 4 + (d.batch + 1) * 4


def test_balanced_mode_only_where_items_outnumber_cus():
    """The balanced mode replaces one workgroup per (b, kv-head) item on the
    G <= 16 kernel only when the items outnumber the CUs, no split count is
    forced and the batch fits the kernel's on-device scan (4096 sequences);
    the large-group kernel keeps its splits."""
    assert not g.get_plan(desc(batch=128, num_q_heads=64, num_kv_heads=1, capacity=2048))["balanced"]
    assert not g.get_plan(desc(batch=300, num_q_heads=64, num_kv_heads=1, capacity=2048))["balanced"]
    assert not g.get_plan(desc(batch=32, num_q_heads=32, num_kv_heads=8, capacity=4097))["balanced"]   # 256 items
    assert g.get_plan(desc(batch=33, num_q_heads=32, num_kv_heads=8, capacity=4097))["balanced"]
    assert g.get_plan(desc(batch=64, num_q_heads=64, num_kv_heads=8, capacity=8192, layout="BSHD"))["balanced"]
    assert not g.get_plan(desc(batch=64, num_q_heads=64, num_kv_heads=8, capacity=8192, num_splits=1))["balanced"]
    assert g.get_plan(desc(batch=4096, num_q_heads=8, num_kv_heads=1, capacity=64))["balanced"]
    assert not g.get_plan(desc(batch=4097, num_q_heads=8, num_kv_heads=1, capacity=64))["balanced"]
    assert not g.get_plan(desc(batch=300, num_q_heads=8, num_kv_heads=1, kv_dtype=g.F32, qo_dtype=g.F32))["balanced"]


def test_large_group_whole_item_mode_plan():
    """The large-group kernel (bf16, D = 128, 16 < G <= 64) runs without
    splits -- one 512-thread workgroup per (sequence, kv-head) item, no
    partials, no combine pass -- when the items fill the 256 CUs or when one
    split is forced; otherwise it splits the token axis.  Paged caches keep
    the split form (256-thread workgroups over its own split count)."""
    def plan(**kw):
        return g.get_plan(desc(head_dim=128, **kw))
    for kw in (dict(batch=256, num_q_heads=64, num_kv_heads=1, capacity=2048),
               dict(batch=300, num_q_heads=48, num_kv_heads=1, capacity=2048),
               dict(batch=256, num_q_heads=24, num_kv_heads=1, capacity=900),
               dict(batch=100, num_q_heads=144, num_kv_heads=3, capacity=900),
               dict(batch=128, num_q_heads=64, num_kv_heads=1, num_splits=1),
               dict(batch=3, num_q_heads=48, num_kv_heads=2, num_splits=1)):
        p = plan(**kw)
        grid = kw["batch"] * kw["num_kv_heads"]
        assert (p["kernel"], p["num_splits"], p["block"], p["grid"], p["combine"], p["workspace_bytes"]) == \
            ("mfma_all", 1, 512, grid, False, 0), (kw, p)
    for kw in (dict(batch=128, num_q_heads=64, num_kv_heads=1, capacity=2048),   # 128 items: splits
               dict(batch=128, num_q_heads=32, num_kv_heads=1, capacity=2048),
               dict(batch=300, num_q_heads=64, num_kv_heads=1, num_splits=4)):
        p = plan(**kw)
        assert p["kernel"] == "mfma_all" and p["block"] == 256 and p["num_splits"] > 1 and p["combine"], (kw, p)
    d = desc(batch=300, num_q_heads=64, num_kv_heads=1, capacity=2048)
    m, keep = _map("paged", 600, [[2 * b, 2 * b + 1] for b in range(300)], block_size=1024, max_blocks=2)
    p = g.get_plan_ex(d, _lib.OptsT(ctypes.pointer(m), None, None, None))
    assert (p["kernel"], p["block"], p["grid"]) == ("mfma_all", 256, 300 * p["num_splits"]), p


def test_head_parallel_items_on_bshd_caches():
    """The small-group matrix-core kernel takes four adjacent kv-heads per
    workgroup (one per wave, over the same slots) on BSHD caches whose kv-head
    count is a multiple of 4; every other plan keeps one kv-head per item."""
    bshd = dict(layout="BSHD", num_q_heads=32, num_kv_heads=8)
    four = [bshd, dict(bshd, batch=64, num_q_heads=64, capacity=8192), dict(bshd, num_splits=3),
            dict(bshd, batch=40, capacity=600), dict(bshd, num_q_heads=64, num_kv_heads=4),
            dict(bshd, num_q_heads=64, num_kv_heads=4, kv_dtype=g.I8)]
    one = [dict(bshd, layout="BHSD"), dict(bshd, num_q_heads=16, num_kv_heads=2),
           dict(bshd, num_q_heads=96, num_kv_heads=4, kv_dtype=g.I8),     # G = 24: two 16-head blocks a wave
           dict(bshd, num_q_heads=128, num_kv_heads=4),                    # G = 32: large-group kernel
           dict(bshd, head_dim=64), dict(bshd, kv_dtype=g.F32, qo_dtype=g.F32)]
    for kw in four:
        p = g.get_plan(desc(**kw))
        assert p["kernel"] == "mfma_qk" and p["heads_per_item"] == 4, (kw, p)
    for kw in one:
        p = g.get_plan(desc(**kw))
        assert p["heads_per_item"] == 1, (kw, p)


@pytest.mark.parametrize("ns", [1, 2, 3, 7, 64, 10_000])
def test_forced_split_count(ns):
    d = desc(num_splits=ns, capacity=4097)
    p = g.get_plan(d)
    assert 1 <= p["num_splits"] <= min(ns, 4097)
    assert p["num_splits"] * p["split_tokens"] >= 4097
    if ns == 1:
        assert p["workspace_bytes"] == 0 and not p["combine"]


@pytest.mark.parametrize("ns", [0, 2, 5])
def test_workspace_bytes_cover_partials(ns):
    d = desc(batch=32, num_q_heads=32, num_kv_heads=8, capacity=4097, num_splits=ns)
    p = g.get_plan(d)
    if p["num_splits"] == 1:
        assert p["workspace_bytes"] == 0
    else:
        assert p["workspace_bytes"] >= 32 * 32 * p["num_splits"] * (128 + 2) * 4


def test_block_shapes():
    """Kernels run 4-wave workgroups (8 for int8 caches with G > 16); MFMA_QK aims at about one workgroup per CU."""
    for kw in (dict(num_q_heads=8, num_kv_heads=2), dict(num_q_heads=32, num_kv_heads=2),
               dict(num_q_heads=64, num_kv_heads=1), dict(kv_dtype=g.F32, qo_dtype=g.F32)):
        assert g.get_plan(desc(**kw))["block"] == 256
    # int8 caches with more than 16 heads per kv-head: 8 waves of two 16-head blocks
    assert g.get_plan(desc(num_q_heads=64, num_kv_heads=1, kv_dtype=g.I8))["block"] == 512
    p = g.get_plan(desc(batch=32, num_q_heads=32, num_kv_heads=8, capacity=4097))
    assert p["kernel"] == "mfma_qk" and p["grid"] == 256 and p["num_splits"] == 1


# ---------------------------------------------------------------------------
# Mapped caches: every refusal of the CLIKA groupQueryAttention page's rules
# (slot rows in range and distinct; block entries -1 or in range, no block
# twice within one row) and of the map's shape fields happens on the host,
# before any HIP call.
# ---------------------------------------------------------------------------
import numpy as np  # noqa: E402


def _map(kind, num_rows, table, block_size=0, max_blocks=0, dev=FAKE + 8 * GAP):
    host = np.ascontiguousarray(np.asarray(table, dtype=np.int32))
    m = _lib.MapT(_lib.MAP_KINDS[kind], num_rows, block_size, max_blocks, dev, host.ctypes.data)
    return m, host


def _mapped_calls(d, m):
    L = g.lib()
    p = _attend_ptrs()
    return [
        L.gqa_decode_attend_mapped(ctypes.byref(d), ctypes.byref(m), p["q"], p["kc"], p["vc"], p["lens"], p["out"],
                                   p["ws"], 1 << 30, None),
        L.gqa_decode_step_mapped(ctypes.byref(d), ctypes.byref(m), p["q"], p["kc"], p["vc"], p["kn"], p["vn"],
                                 p["lens"], p["out"], p["ws"], 1 << 30, None),
        L.gqa_decode_append_mapped(ctypes.byref(d), ctypes.byref(m), p["kc"], p["vc"], p["kn"], p["vn"], p["lens"],
                                   None),
    ]


BAD_SLOTS = [
    ([0, 4], 4),      # out of range
    ([-1, 0], 4),     # negative
    ([2, 2], 4),      # two rows share a cache row
]


@pytest.mark.parametrize("table,rows", BAD_SLOTS)
def test_bad_slot_map_refused(table, rows):
    m, keep = _map("slots", rows, table)
    assert _mapped_calls(desc(), m) == [INVALID] * 3


BAD_TABLES = [
    [[0, 1, 2, 3], [4, 5, 6, 99]],    # entry past num_blocks
    [[0, 1, 2, 3], [4, 5, -2, -1]],   # negative other than the -1 pad
    [[0, 1, 0, -1], [4, 5, 6, 7]],    # block named twice within one row
    [[0, -1, 3, 3], [4, 5, 6, 7]],    # repeat after a pad
]


@pytest.mark.parametrize("table", BAD_TABLES)
def test_bad_block_table_refused(table):
    m, keep = _map("paged", 16, table, block_size=1024, max_blocks=4)
    assert _mapped_calls(desc(), m) == [INVALID] * 3


@pytest.mark.parametrize("field,value", [("kind", 0), ("kind", 3), ("num_rows", 0), ("block_size", 0),
                                         ("max_blocks", 0), ("block_size", 512)])   # 512 * 4 != capacity 4096
def test_bad_map_shape_refused(field, value):
    m, keep = _map("paged", 16, [[0, 1, 2, 3], [4, 5, 6, 7]], block_size=1024, max_blocks=4)
    setattr(m, field, value)
    assert _mapped_calls(desc(), m) == [INVALID] * 3


def test_missing_or_misaligned_map_refused():
    L = g.lib()
    d = desc()
    for dev, host_ok in ((0, True), (FAKE + 8 * GAP + 2, True), (FAKE + 8 * GAP, False)):
        m, keep = _map("slots", 4, [1, 2], dev=dev)
        if not host_ok:
            m.map_host = None
        assert _mapped_calls(d, m) == [INVALID] * 3
    p = _attend_ptrs()
    assert L.gqa_decode_attend_mapped(ctypes.byref(d), None, p["q"], p["kc"], p["vc"], p["lens"], p["out"], p["ws"],
                                      1 << 30, None) == INVALID


def test_paged_blocks_not_multiple_of_16_plan_the_generic_kernel():
    """bf16, D = 128, G = 4 is a matrix-core descriptor: paged caches with a
    block size that is a multiple of 16 keep the matrix-core plan, any other
    block size is planned on the generic kernel, and the workspace the call
    needs is that plan's."""
    d = desc()
    assert g.get_plan(d)["kernel"] == "mfma_qk"
    for bs, kernel in ((16, "mfma_qk"), (48, "mfma_qk"), (8, "generic"), (7, "generic"), (24, "generic")):
        mb = -(-4096 // bs)
        dd = desc(capacity=mb * bs)
        m, keep = _map("paged", 2 * mb, [list(range(0, mb)), list(range(mb, 2 * mb))], block_size=bs, max_blocks=mb)
        opts = _lib.OptsT(ctypes.pointer(m), None, None, None)
        plan = g.get_plan_ex(dd, opts)
        assert plan["kernel"] == kernel, (bs, plan)
        assert g.workspace_size_ex(dd, opts) == plan["workspace_bytes"]
        if kernel == "mfma_qk":
            assert plan == g.get_plan(dd)
    # int8 caches and large groups fall back the same way
    for kw in (dict(kv_dtype=g.I8), dict(num_q_heads=64, num_kv_heads=1)):
        m, keep = _map("paged", 1024, [list(range(0, 512)), list(range(512, 1024))], block_size=8, max_blocks=512)
        assert g.get_plan_ex(desc(**kw), _lib.OptsT(ctypes.pointer(m), None, None, None))["kernel"] == "generic"


def test_map_overlapping_output_or_caches_refused():
    L = g.lib()
    p = _attend_ptrs()
    d = desc()
    m, keep = _map("slots", 4, [1, 2], dev=p["out"])
    assert L.gqa_decode_attend_mapped(ctypes.byref(d), ctypes.byref(m), p["q"], p["kc"], p["vc"], p["lens"], p["out"],
                                      p["ws"], 1 << 30, None) == INVALID
    m, keep = _map("slots", 4, [1, 2], dev=p["kc"])       # the step and the append write the caches
    assert L.gqa_decode_step_mapped(ctypes.byref(d), ctypes.byref(m), p["q"], p["kc"], p["vc"], p["kn"], p["vn"],
                                    p["lens"], p["out"], p["ws"], 1 << 30, None) == INVALID
    assert L.gqa_decode_append_mapped(ctypes.byref(d), ctypes.byref(m), p["kc"], p["vc"], p["kn"], p["vn"], p["lens"],
                                      None) == INVALID


def test_mapped_empty_batch_is_a_noop():
    L = g.lib()
    d = desc(batch=0)
    m = _lib.MapT(_lib.MAP_KINDS["paged"], 4, 1024, 4, None, None)
    assert L.gqa_decode_attend_mapped(ctypes.byref(d), ctypes.byref(m), None, None, None, None, None, None, 0,
                                      None) == OK
    assert L.gqa_decode_step_mapped(ctypes.byref(d), ctypes.byref(m), None, None, None, None, None, None, None, None,
                                    0, None) == OK
    assert L.gqa_decode_append_mapped(ctypes.byref(d), ctypes.byref(m), None, None, None, None, None, None) == OK


# ---------------------------------------------------------------------------
# Int8 caches (CANN dynamic-quantization rule): the _q8 calls need an int8
# descriptor and both scale arrays; every other call refuses int8 caches.
# ---------------------------------------------------------------------------
def _q8_calls(d, sc, p=None):
    L = g.lib()
    p = p or _attend_ptrs()
    scp = ctypes.byref(sc) if sc is not None else None
    return [
        L.gqa_decode_attend_q8(ctypes.byref(d), scp, p["q"], p["kc"], p["vc"], p["lens"], p["out"], p["ws"], 1 << 30,
                               None),
        L.gqa_decode_step_q8(ctypes.byref(d), scp, p["q"], p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], p["out"],
                             p["ws"], 1 << 30, None),
        L.gqa_decode_append_q8(ctypes.byref(d), scp, p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], None),
    ]


def _scales(k=FAKE + 9 * GAP, v=FAKE + 10 * GAP):
    return _lib.ScalesT(k, v)


def test_unquantized_calls_refuse_int8_caches():
    L = g.lib()
    d = desc(kv_dtype=g.I8)
    p = _attend_ptrs()
    assert _attend(d, p, 1 << 30) == INVALID
    assert _step(d, p, 1 << 30) == INVALID
    assert L.gqa_decode_append(ctypes.byref(d), p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], None) == INVALID
    m, keep = _map("slots", 4, [1, 2])
    assert _mapped_calls(d, m) == [INVALID] * 3


def test_q8_calls_refuse_other_cache_dtypes_and_missing_scales():
    for kv in (g.BF16, g.F32):
        assert _q8_calls(desc(kv_dtype=kv), _scales()) == [INVALID] * 3
    d = desc(kv_dtype=g.I8)
    assert _q8_calls(d, None) == [INVALID] * 3
    assert _q8_calls(d, _scales(k=0)) == [INVALID] * 3
    assert _q8_calls(d, _scales(v=0)) == [INVALID] * 3
    assert _q8_calls(d, _scales(k=FAKE + 9 * GAP + 2)) == [INVALID] * 3     # not 4-byte aligned
    assert _q8_calls(desc(kv_dtype=g.I8, qo_dtype=g.I8), _scales()) == [INVALID] * 3   # q/out are activations


def test_q8_scales_overlapping_anything_refused():
    d = desc(kv_dtype=g.I8)
    p = _attend_ptrs()
    n = 2 * 2 * 4096 * 4                                   # B * Hkv * S float32 scales
    assert _q8_calls(d, _scales(k=FAKE + 9 * GAP, v=FAKE + 9 * GAP + n - 4)) == [INVALID] * 3
    for other in ("kc", "vc", "lens"):
        assert _q8_calls(d, _scales(k=p[other]), p) == [INVALID] * 3, other
    for other in ("kn", "vn"):                             # attend does not take these
        assert _q8_calls(d, _scales(k=p[other]), p)[1:] == [INVALID] * 2, other
    for other in ("q", "out", "ws"):                       # append does not take these
        assert _q8_calls(d, _scales(v=p[other]), p)[:2] == [INVALID] * 2, other


def test_q8_new_rows_aligned_for_their_activation_dtype():
    """k_new/v_new of the _q8 calls are in qo_dtype: 2-byte alignment for
    bf16, 4-byte for float32; int8 caches need none."""
    for qo, shift, want in ((g.BF16, 1, INVALID), (g.F32, 2, INVALID)):
        d = desc(kv_dtype=g.I8, qo_dtype=qo)
        p = _attend_ptrs()
        p["kn"] += shift
        assert _q8_calls(d, _scales(), p)[1:] == [want] * 2


def test_q8_empty_batch_is_a_noop_and_plans_int8():
    L = g.lib()
    d = desc(batch=0, kv_dtype=g.I8)
    sc = _scales()
    assert L.gqa_decode_attend_q8(ctypes.byref(d), ctypes.byref(sc), None, None, None, None, None, None, 0,
                                  None) == OK
    assert L.gqa_decode_step_q8(ctypes.byref(d), ctypes.byref(sc), None, None, None, None, None, None, None, None,
                                0, None) == OK
    assert L.gqa_decode_append_q8(ctypes.byref(d), ctypes.byref(sc), None, None, None, None, None, None) == OK
    p = g.get_plan(desc(kv_dtype=g.I8))
    assert p["block"] == 256 and p["workspace_bytes"] == g.workspace_size(desc(kv_dtype=g.I8))


# ---------------------------------------------------------------------------
# Options (_ex calls) and rotary encoding: refusals before any launch.
# ---------------------------------------------------------------------------
def _rope(**kw):
    base = dict(cos=FAKE + 11 * GAP, sin=FAKE + 12 * GAP, max_pos=4096, mode=0, positions=None, q_norm_gain=None,
                k_norm_gain=None, norm_eps=-1.0)
    base.update(kw)
    return _lib.RopeT(base["cos"], base["sin"], base["max_pos"], base["mode"], base["positions"],
                      base["q_norm_gain"], base["k_norm_gain"], base["norm_eps"])


def _ex_calls(d, o, p=None):
    L = g.lib()
    p = p or _attend_ptrs()
    op = ctypes.byref(o) if o is not None else None
    return [
        L.gqa_decode_step_ex(ctypes.byref(d), op, p["q"], p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], p["out"],
                             p["ws"], 1 << 30, None),
        L.gqa_decode_append_ex(ctypes.byref(d), op, p["kc"], p["vc"], p["kn"], p["vn"], p["lens"], None),
    ]


BAD_ROPES = [
    (dict(mode=2), INVALID),
    (dict(max_pos=0), INVALID),
    (dict(cos=0), INVALID),
    (dict(sin=FAKE + 12 * GAP + 2), INVALID),                        # misaligned table
    (dict(cos=FAKE + 11 * GAP + 4), INVALID),                        # tables are 16-byte aligned
    (dict(positions=FAKE + 13 * GAP + 1), INVALID),
    (dict(q_norm_gain=FAKE + 13 * GAP), INVALID),                    # a gain without an epsilon
    (dict(norm_eps=1e-6), INVALID),                                  # an epsilon without a gain
    (dict(k_norm_gain=FAKE + 13 * GAP, norm_eps=float("nan")), INVALID),
    (dict(cos=FAKE + GAP), INVALID),                                 # table inside the K cache (written)
]


@pytest.mark.parametrize("kw,status", BAD_ROPES)
def test_bad_rope_refused(kw, status):
    r = _rope(**kw)
    o = _lib.OptsT(None, None, ctypes.pointer(r), None)
    assert _ex_calls(desc(), o) == [status, status]


def test_rope_needs_even_head_dim_and_no_norm_on_int8():
    r = _rope()
    o = _lib.OptsT(None, None, ctypes.pointer(r), None)
    assert _ex_calls(desc(head_dim=7, kv_dtype=g.F32, qo_dtype=g.F32), o) == [INVALID, INVALID]
    sc = _scales()
    r = _rope(k_norm_gain=FAKE + 13 * GAP, norm_eps=1e-6)
    o = _lib.OptsT(None, ctypes.pointer(sc), ctypes.pointer(r), None)
    assert _ex_calls(desc(kv_dtype=g.I8), o) == [UNSUPPORTED, UNSUPPORTED]


def test_attend_refuses_rope_and_ex_matches_plain_refusals():
    L = g.lib()
    r = _rope()
    o = _lib.OptsT(None, None, ctypes.pointer(r), None)
    p = _attend_ptrs()
    d = desc()
    assert L.gqa_decode_attend_ex(ctypes.byref(d), ctypes.byref(o), p["q"], p["kc"], p["vc"], p["lens"], p["out"],
                                  p["ws"], 1 << 30, None) == INVALID
    # NULL options = the plain calls: int8 without scales, bad descriptors
    assert _ex_calls(desc(kv_dtype=g.I8), None) == [INVALID, INVALID]
    assert _ex_calls(desc(num_q_heads=6, num_kv_heads=4), None) == [INVALID, INVALID]


def test_workspace_size_ex_adds_the_rotated_q():
    """MFMA_ALL rotates q in registers (no extra workspace); the other kernels
    read a rotated copy kept after the plan's partials."""
    L = g.lib()
    for kw in (dict(), dict(batch=32, num_q_heads=32, num_kv_heads=8, capacity=131073),
               dict(kv_dtype=g.F32, qo_dtype=g.F32, head_dim=64), dict(kv_dtype=g.BF16, qo_dtype=g.F32),
               dict(batch=128, num_q_heads=64, num_kv_heads=1, capacity=2048)):
        d = desc(**kw)
        plain = g.workspace_size(d)
        generic = g.get_plan(d)["kernel"] != "mfma_all"
        n = ctypes.c_size_t(0)
        assert L.gqa_decode_workspace_size_ex(ctypes.byref(d), None, ctypes.byref(n)) == OK and n.value == plain
        r = _rope()
        o = _lib.OptsT(None, None, ctypes.pointer(r), None)
        assert L.gqa_decode_workspace_size_ex(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)) == OK
        eqo = 4 if d.qo_dtype == g.F32 else 2
        extra = d.batch * d.num_q_heads * d.head_dim * eqo if generic else 0
        assert n.value == (-(-plain // 256) * 256 + extra if generic else plain)
        if n.value == 0:
            continue
        # a workspace one byte short of that is refused
        p = _attend_ptrs()
        assert L.gqa_decode_step_ex(ctypes.byref(d), ctypes.byref(o), p["q"], p["kc"], p["vc"], p["kn"], p["vn"],
                                    p["lens"], p["out"], p["ws"], n.value - 1, None) == WS_SMALL


def test_ex_empty_batch_is_a_noop():
    L = g.lib()
    d = desc(batch=0)
    r = _rope()
    o = _lib.OptsT(None, None, ctypes.pointer(r), None)
    assert L.gqa_decode_step_ex(ctypes.byref(d), ctypes.byref(o), None, None, None, None, None, None, None, None, 0,
                                None) == OK
    assert L.gqa_decode_append_ex(ctypes.byref(d), ctypes.byref(o), None, None, None, None, None, None) == OK


# ---------------------------------------------------------------------------
# Softmax variants: refusals before any launch.
# ---------------------------------------------------------------------------
def _smx(**kw):
    base = dict(sink=None, smooth=0, softcap=0.0, window=0, kept_prefix=0, kept_prefix_per_seq=None)
    base.update(kw)
    return _lib.SoftmaxT(base["sink"], base["smooth"], base["softcap"], base["window"], base["kept_prefix"],
                         base["kept_prefix_per_seq"])


def _attend_step_ex(d, o, p=None):
    L = g.lib()
    p = p or _attend_ptrs()
    return [
        L.gqa_decode_attend_ex(ctypes.byref(d), ctypes.byref(o), p["q"], p["kc"], p["vc"], p["lens"], p["out"],
                               p["ws"], 1 << 30, None),
        L.gqa_decode_step_ex(ctypes.byref(d), ctypes.byref(o), p["q"], p["kc"], p["vc"], p["kn"], p["vn"], p["lens"],
                             p["out"], p["ws"], 1 << 30, None),
    ]


BAD_SOFTMAX = [
    dict(smooth=2),
    dict(smooth=1, sink=FAKE + 14 * GAP),            # a sink and smooth softmax together
    dict(softcap=-1.0),
    dict(softcap=float("nan")),
    dict(softcap=float("inf")),
    dict(window=-3),
    dict(window=8, kept_prefix=-1),
    dict(kept_prefix=4),                              # a prefix without a window
    dict(kept_prefix_per_seq=FAKE + 15 * GAP),
    dict(sink=FAKE + 14 * GAP + 2),                   # misaligned
    dict(window=8, kept_prefix_per_seq=FAKE + 15 * GAP + 1),
    dict(sink=FAKE + 4 * GAP),                        # the sink inside the output
    dict(window=4, kept_prefix_per_seq=FAKE + 5 * GAP),  # the prefixes inside the workspace
]


@pytest.mark.parametrize("kw", BAD_SOFTMAX, ids=[str(k) for k in BAD_SOFTMAX])
def test_bad_softmax_refused(kw):
    v = _smx(**kw)
    o = _lib.OptsT(None, None, None, ctypes.pointer(v))
    assert _attend_step_ex(desc(), o) == [INVALID, INVALID]


def test_softmax_arrays_may_share_read_only_inputs_but_not_written_caches():
    """A sink stored inside the K cache is refused by the step, which writes
    the cache (attend, which only reads it, would accept it)."""
    L = g.lib()
    v = _smx(sink=FAKE + GAP)
    o = _lib.OptsT(None, None, None, ctypes.pointer(v))
    p = _attend_ptrs()
    d = desc()
    assert L.gqa_decode_step_ex(ctypes.byref(d), ctypes.byref(o), p["q"], p["kc"], p["vc"], p["kn"], p["vn"],
                                p["lens"], p["out"], p["ws"], 1 << 30, None) == INVALID


def test_append_refuses_softmax_options_and_empty_batch_is_a_noop():
    L = g.lib()
    v = _smx(window=4)
    o = _lib.OptsT(None, None, None, ctypes.pointer(v))
    p = _attend_ptrs()
    assert L.gqa_decode_append_ex(ctypes.byref(desc()), ctypes.byref(o), p["kc"], p["vc"], p["kn"], p["vn"],
                                  p["lens"], None) == INVALID
    d0 = desc(batch=0)
    assert L.gqa_decode_attend_ex(ctypes.byref(d0), ctypes.byref(o), None, None, None, None, None, None, 0,
                                  None) == OK
    assert L.gqa_decode_step_ex(ctypes.byref(d0), ctypes.byref(o), None, None, None, None, None, None, None, None, 0,
                                None) == OK


def test_window_plans_splits_over_its_span():
    """With a host-known window and prefix the splits cover W + P + 32 slots,
    not the capacity: the workspace follows that plan."""
    L = g.lib()
    d = desc(batch=4, num_q_heads=32, num_kv_heads=8, capacity=131073)
    plain = g.workspace_size(d)
    n = ctypes.c_size_t(0)
    for W_, P_ in ((4096, 4), (64, 0), (200000, 0)):
        v = _smx(window=W_, kept_prefix=P_)
        o = _lib.OptsT(None, None, None, ctypes.pointer(v))
        assert L.gqa_decode_workspace_size_ex(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)) == OK
        if W_ == 64:
            assert n.value == 0                    # one split
        elif W_ == 4096:
            assert 0 < n.value
        else:
            assert n.value == plain                # the window spans the capacity
    v = _smx(window=64, kept_prefix_per_seq=FAKE + 15 * GAP)  # prefixes on the device: no bound
    o = _lib.OptsT(None, None, None, ctypes.pointer(v))
    assert L.gqa_decode_workspace_size_ex(ctypes.byref(d), ctypes.byref(o), ctypes.byref(n)) == OK
    assert n.value == plain

"""ctypes binding of libgqa_decode.so (the C ABI declared in include/gqa_decode.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  torch tensors supply device memory and the current HIP stream.  If
the library is not built, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_decode.so")

GQA_OK = 0
STATUS_NAMES = {
    0: "GQA_OK",
    1: "GQA_ERR_INVALID_ARGUMENT",
    2: "GQA_ERR_UNSUPPORTED",
    3: "GQA_ERR_WORKSPACE_TOO_SMALL",
    4: "GQA_ERR_HIP",
    5: "GQA_ERR_INTERNAL",
}
F32, BF16, I8, FP8 = 0, 1, 2, 3
LAYOUTS = {"BHSD": 0, "BSHD": 1}
KERNEL_NAMES = {0: "generic", 1: "mfma_qk", 2: "mfma_all", 3: "small"}


class GqaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)}")


class Desc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("layout", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("qo_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
    ]


class PlanT(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("combine", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("balanced", ctypes.c_int32),
        ("heads_per_item", ctypes.c_int32),
    ]


MAP_KINDS = {"slots": 1, "paged": 2}


class MapT(ctypes.Structure):
    """gqa_cache_map_t."""
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("map", ctypes.c_void_p),
        ("map_host", ctypes.c_void_p),
    ]


class ScalesT(ctypes.Structure):
    """gqa_kv_scales_t."""
    _fields_ = [("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


ROPE_MODES = {"half": 0, "interleaved": 1}


class RopeT(ctypes.Structure):
    """gqa_rope_t."""
    _fields_ = [
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("max_pos", ctypes.c_int32),
        ("mode", ctypes.c_int32),
        ("positions", ctypes.c_void_p),
        ("q_norm_gain", ctypes.c_void_p),
        ("k_norm_gain", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
    ]


class SoftmaxT(ctypes.Structure):
    """gqa_softmax_t."""
    _fields_ = [
        ("sink", ctypes.c_void_p),
        ("smooth", ctypes.c_int32),
        ("softcap", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("kept_prefix", ctypes.c_int32),
        ("kept_prefix_per_seq", ctypes.c_void_p),
    ]


class OptsT(ctypes.Structure):
    """gqa_decode_opts_t."""
    _fields_ = [
        ("map", ctypes.POINTER(MapT)),
        ("scales", ctypes.POINTER(ScalesT)),
        ("rope", ctypes.POINTER(RopeT)),
        ("softmax", ctypes.POINTER(SoftmaxT)),
    ]


EXPORTS = (
    "gqa_decode_workspace_size",
    "gqa_decode_get_plan",
    "gqa_decode_append",
    "gqa_decode_attend",
    "gqa_decode_step",
    "gqa_decode_append_mapped",
    "gqa_decode_attend_mapped",
    "gqa_decode_step_mapped",
    "gqa_decode_append_q8",
    "gqa_decode_attend_q8",
    "gqa_decode_step_q8",
    "gqa_decode_workspace_size_ex",
    "gqa_decode_get_plan_ex",
    "gqa_decode_append_ex",
    "gqa_decode_attend_ex",
    "gqa_decode_step_ex",
    "gqa_decode_check_lengths",
    "gqa_decode_status_string",
    "gqa_decode_version",
)

_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gqa_decode_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, S, I32P = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    DP = ctypes.POINTER(Desc)
    L.gqa_decode_workspace_size.argtypes = [DP, ctypes.POINTER(ctypes.c_size_t)]
    L.gqa_decode_get_plan.argtypes = [DP, ctypes.POINTER(PlanT)]
    L.gqa_decode_append.argtypes = [DP, P, P, P, P, I32P, P]
    L.gqa_decode_attend.argtypes = [DP, P, P, P, I32P, P, P, S, P]
    L.gqa_decode_step.argtypes = [DP, P, P, P, P, P, I32P, P, P, S, P]
    L.gqa_decode_check_lengths.argtypes = [DP, I32P, ctypes.c_int32, P, ctypes.POINTER(ctypes.c_int32)]
    MP = ctypes.POINTER(MapT)
    L.gqa_decode_append_mapped.argtypes = [DP, MP, P, P, P, P, I32P, P]
    L.gqa_decode_attend_mapped.argtypes = [DP, MP, P, P, P, I32P, P, P, S, P]
    L.gqa_decode_step_mapped.argtypes = [DP, MP, P, P, P, P, P, I32P, P, P, S, P]
    SP = ctypes.POINTER(ScalesT)
    L.gqa_decode_append_q8.argtypes = [DP, SP, P, P, P, P, I32P, P]
    L.gqa_decode_attend_q8.argtypes = [DP, SP, P, P, P, I32P, P, P, S, P]
    L.gqa_decode_step_q8.argtypes = [DP, SP, P, P, P, P, P, I32P, P, P, S, P]
    OP = ctypes.POINTER(OptsT)
    L.gqa_decode_workspace_size_ex.argtypes = [DP, OP, ctypes.POINTER(ctypes.c_size_t)]
    L.gqa_decode_get_plan_ex.argtypes = [DP, OP, ctypes.POINTER(PlanT)]
    L.gqa_decode_append_ex.argtypes = [DP, OP, P, P, P, P, I32P, P]
    L.gqa_decode_attend_ex.argtypes = [DP, OP, P, P, P, I32P, P, P, S, P]
    L.gqa_decode_step_ex.argtypes = [DP, OP, P, P, P, P, P, I32P, P, P, S, P]
    for name in ("gqa_decode_workspace_size", "gqa_decode_get_plan", "gqa_decode_append", "gqa_decode_attend",
                 "gqa_decode_step", "gqa_decode_check_lengths", "gqa_decode_append_mapped",
                 "gqa_decode_attend_mapped", "gqa_decode_step_mapped", "gqa_decode_append_q8",
                 "gqa_decode_attend_q8", "gqa_decode_step_q8", "gqa_decode_workspace_size_ex", "gqa_decode_get_plan_ex",
                 "gqa_decode_append_ex", "gqa_decode_attend_ex", "gqa_decode_step_ex"):
        getattr(L, name).restype = ctypes.c_int
    L.gqa_decode_status_string.argtypes = [ctypes.c_int]
    L.gqa_decode_status_string.restype = ctypes.c_char_p
    L.gqa_decode_version.argtypes = []
    L.gqa_decode_version.restype = ctypes.c_int32
    _lib = L
    return L


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    if t == torch.int8:
        return I8
    if t == torch.float8_e4m3fn:
        return FP8
    raise ValueError(f"unsupported dtype {t}; float32, bfloat16, or int8 / float8_e4m3fn (caches only)")


def make_desc(batch, num_q_heads, num_kv_heads, head_dim, capacity, layout="BHSD", kv_dtype=BF16, qo_dtype=BF16,
              num_splits=0) -> Desc:
    return Desc(batch, num_q_heads, num_kv_heads, head_dim, capacity, LAYOUTS[layout], kv_dtype, qo_dtype,
                num_splits)


def desc_for(q: torch.Tensor, k_cache: torch.Tensor, layout: str, num_splits: int = 0) -> Desc:
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q is (B, Hq, D); caches are 4-D")
    B, Hq, D = q.shape
    if layout == "BHSD":
        Bc, Hkv, S, Dc = k_cache.shape
    else:
        Bc, S, Hkv, Dc = k_cache.shape
    if Bc != B or Dc != D:
        raise ValueError("q and cache disagree on batch or head_dim")
    return make_desc(B, Hq, Hkv, D, S, layout, _dtype_code(k_cache.dtype), _dtype_code(q.dtype), num_splits)


def check(status: int, what: str) -> None:
    if status != GQA_OK:
        raise GqaError(status, what)


def workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    check(lib().gqa_decode_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "gqa_decode_workspace_size")
    return n.value


def get_plan(desc: Desc) -> dict:
    p = PlanT()
    check(lib().gqa_decode_get_plan(ctypes.byref(desc), ctypes.byref(p)), "gqa_decode_get_plan")
    return _plan_dict(p)


def get_plan_ex(desc: Desc, opts) -> dict:
    """The plan of an attend/step call with options (an OptsT, or None)."""
    p = PlanT()
    check(lib().gqa_decode_get_plan_ex(ctypes.byref(desc), None if opts is None else ctypes.byref(opts),
                                       ctypes.byref(p)), "gqa_decode_get_plan_ex")
    return _plan_dict(p)


def _plan_dict(p: PlanT) -> dict:
    return dict(kernel=KERNEL_NAMES.get(p.kernel, p.kernel), num_splits=p.num_splits, split_tokens=p.split_tokens,
                grid=p.grid, block=p.block, combine=bool(p.combine), workspace_bytes=p.workspace_bytes,
                balanced=bool(p.balanced), heads_per_item=p.heads_per_item)


def _dev(tensors, lengths):
    dev = tensors[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for t in tensors:
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if lengths.dtype != torch.int32 or lengths.device != dev or not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous int32 tensor on the same device")
    return dev


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(desc: Desc, dev, workspace):
    need = workspace_size(desc)
    if need == 0:
        return workspace, None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def append(k_cache, v_cache, k_new, v_new, lengths, *, layout="BHSD"):
    """In-place append of k_new/v_new (B, Hkv, D) at slot lengths[b] of the caches."""
    dev = _dev([k_cache, v_cache, k_new, v_new], lengths)
    B, Hkv, D = k_new.shape
    S = k_cache.shape[2] if layout == "BHSD" else k_cache.shape[1]
    desc = make_desc(B, Hkv, Hkv, D, S, layout, _dtype_code(k_cache.dtype), _dtype_code(k_cache.dtype))
    check(lib().gqa_decode_append(ctypes.byref(desc), k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(),
                                  v_new.data_ptr(), lengths.data_ptr(), _stream(dev)), "gqa_decode_append")


def attend(q, k_cache, v_cache, lengths, *, layout="BHSD", out=None, workspace=None, num_splits=0):
    """Read-only length-masked GQA attention; lengths[b] = valid slots. Returns out (B, Hq, D)."""
    dev = _dev([q, k_cache, v_cache], lengths)
    desc = desc_for(q, k_cache, layout, num_splits)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace(desc, dev, workspace)
    check(lib().gqa_decode_attend(ctypes.byref(desc), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                  lengths.data_ptr(), out.data_ptr(), wptr, wbytes, _stream(dev)),
          "gqa_decode_attend")
    return out


def step(q, k_cache, v_cache, k_new, v_new, lengths, *, layout="BHSD", out=None, workspace=None, num_splits=0):
    """Fused decode step: append at lengths[b], then attend lengths[b] + 1 slots. Returns out."""
    dev = _dev([q, k_cache, v_cache, k_new, v_new], lengths)
    desc = desc_for(q, k_cache, layout, num_splits)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace(desc, dev, workspace)
    check(lib().gqa_decode_step(ctypes.byref(desc), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(), out.data_ptr(), wptr, wbytes,
                                _stream(dev)), "gqa_decode_step")
    return out


def check_lengths(lengths, capacity, *, mode="step"):
    """Number of lengths[b] outside the contract of `mode` ("step"/"append": 0 <= L < capacity,
    "attend": 1 <= L <= capacity). Synchronous debugging aid."""
    if mode not in ("step", "append", "attend"):
        raise ValueError(f"mode {mode!r}: 'step', 'append' or 'attend'")
    if lengths.dtype != torch.int32 or lengths.dim() != 1 or not lengths.is_contiguous() or not lengths.is_cuda:
        raise ValueError("lengths must be a contiguous 1-D int32 CUDA tensor")
    B = lengths.numel()
    desc = make_desc(B, 1, 1, 1, capacity)
    n = ctypes.c_int32(-1)
    check(lib().gqa_decode_check_lengths(ctypes.byref(desc), lengths.data_ptr(), 1 if mode == "attend" else 0,
                                         _stream(lengths.device), ctypes.byref(n)), "gqa_decode_check_lengths")
    return int(n.value)


def _mapped_desc(q_like_B, Hq, D, kv_dtype, qo_dtype, k_cache, kind, layout, table, num_splits, Hkv=None,
                 table_host=None):
    """Descriptor and gqa_cache_map_t for a mapped call (kept alive by the caller).

    ``table`` is the device table the kernels read; ``table_host`` the same
    entries in host memory, which the library validates.  Without
    ``table_host`` the binding copies ``table`` to the host, which waits for the
    stream: pass the host copy in a decode loop."""
    if kind not in MAP_KINDS:
        raise ValueError(f"kind must be one of {list(MAP_KINDS)}")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {list(LAYOUTS)}")
    if k_cache.dim() != 4:
        raise ValueError("caches are 4-D")
    rows = k_cache.shape[0]
    if layout == "BHSD":
        _, Hc, inner, Dc = k_cache.shape
    else:
        _, inner, Hc, Dc = k_cache.shape
    if Dc != D or (Hkv is not None and Hkv != Hc):
        raise ValueError("cache disagrees on head_dim or kv-heads")
    if table.dtype != torch.int32:
        raise ValueError("the map is int32")
    if table_host is None:
        host = table.detach().to("cpu").contiguous()
    else:
        host = torch.as_tensor(table_host, dtype=torch.int32).contiguous()
        if host.device.type != "cpu" or host.shape != table.shape:
            raise ValueError("table_host must be a host copy of table")
    if table.device != k_cache.device or not table.is_contiguous():
        raise ValueError("table must be contiguous on the caches' device")
    dev_t = table
    if kind == "slots":
        if host.dim() != 1 or host.shape[0] != q_like_B:
            raise ValueError("slot map is (B,)")
        S, bs, mb = inner, 0, 0
    else:
        if host.dim() != 2 or host.shape[0] != q_like_B:
            raise ValueError("block table is (B, max_blocks)")
        bs, mb = inner, host.shape[1]
        S = bs * mb
    desc = make_desc(q_like_B, Hq, Hc, D, S, layout, kv_dtype, qo_dtype, num_splits)
    m = MapT(MAP_KINDS[kind], rows, bs, mb, dev_t.data_ptr(), host.data_ptr())
    return desc, m, (host, dev_t)


def append_mapped(k_cache, v_cache, k_new, v_new, lengths, table, *, kind, layout="BHSD", table_host=None):
    """In-place append at slot lengths[b] of a slot-indexed cache or a block pool."""
    dev = _dev([k_cache, v_cache, k_new, v_new], lengths)
    B, Hkv, D = k_new.shape
    code = _dtype_code(k_cache.dtype)
    desc, m, keep = _mapped_desc(B, Hkv, D, code, code, k_cache, kind, layout, table, 0, Hkv, table_host)
    check(lib().gqa_decode_append_mapped(ctypes.byref(desc), ctypes.byref(m), k_cache.data_ptr(), v_cache.data_ptr(),
                                         k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(), _stream(dev)),
          "gqa_decode_append_mapped")
    del keep


def attend_mapped(q, k_cache, v_cache, lengths, table, *, kind, layout="BHSD", out=None, workspace=None,
                  num_splits=0, table_host=None):
    """Read-only attention over a slot-indexed cache or a block pool. Returns out (B, Hq, D)."""
    dev = _dev([q, k_cache, v_cache], lengths)
    B, Hq, D = q.shape
    desc, m, keep = _mapped_desc(B, Hq, D, _dtype_code(k_cache.dtype), _dtype_code(q.dtype), k_cache, kind, layout,
                                 table, num_splits, None, table_host)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace_ex(desc, OptsT(ctypes.pointer(m), None, None, None), dev, workspace)
    check(lib().gqa_decode_attend_mapped(ctypes.byref(desc), ctypes.byref(m), q.data_ptr(), k_cache.data_ptr(),
                                         v_cache.data_ptr(), lengths.data_ptr(), out.data_ptr(), wptr, wbytes,
                                         _stream(dev)), "gqa_decode_attend_mapped")
    del keep
    return out


def step_mapped(q, k_cache, v_cache, k_new, v_new, lengths, table, *, kind, layout="BHSD", out=None, workspace=None,
                num_splits=0, table_host=None):
    """Fused decode step on a slot-indexed cache or a block pool. Returns out (B, Hq, D)."""
    dev = _dev([q, k_cache, v_cache, k_new, v_new], lengths)
    B, Hq, D = q.shape
    desc, m, keep = _mapped_desc(B, Hq, D, _dtype_code(k_cache.dtype), _dtype_code(q.dtype), k_cache, kind, layout,
                                 table, num_splits, k_new.shape[1], table_host)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace_ex(desc, OptsT(ctypes.pointer(m), None, None, None), dev, workspace)
    check(lib().gqa_decode_step_mapped(ctypes.byref(desc), ctypes.byref(m), q.data_ptr(), k_cache.data_ptr(),
                                       v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(),
                                       out.data_ptr(), wptr, wbytes, _stream(dev)), "gqa_decode_step_mapped")
    del keep
    return out


def _scales(k_cache, k_scale, v_scale, layout):
    """gqa_kv_scales_t for int8 or fp8 (float8_e4m3fn) caches; scales are float32 of the
    cache's shape without D."""
    if k_cache.dtype not in (torch.int8, torch.float8_e4m3fn):
        raise ValueError("the _q8 calls take int8 or float8_e4m3fn caches")
    for t in (k_scale, v_scale):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(k_cache.shape[:3]):
            raise ValueError(f"scales are float32 of shape {tuple(k_cache.shape[:3])} for {layout} caches")
    return ScalesT(k_scale.data_ptr(), v_scale.data_ptr())


def append_q8(k_cache, v_cache, k_scale, v_scale, k_new, v_new, lengths, *, layout="BHSD"):
    """Quantize k_new/v_new (B, Hkv, D; float32 or bfloat16) row by row and store
    codes and scales at slot lengths[b] of the int8 or fp8 caches."""
    dev = _dev([k_cache, v_cache, k_scale, v_scale, k_new, v_new], lengths)
    B, Hkv, D = k_new.shape
    S = k_cache.shape[2] if layout == "BHSD" else k_cache.shape[1]
    desc = make_desc(B, Hkv, Hkv, D, S, layout, _dtype_code(k_cache.dtype), _dtype_code(k_new.dtype))
    sc = _scales(k_cache, k_scale, v_scale, layout)
    check(lib().gqa_decode_append_q8(ctypes.byref(desc), ctypes.byref(sc), k_cache.data_ptr(), v_cache.data_ptr(),
                                     k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(), _stream(dev)),
          "gqa_decode_append_q8")


def attend_q8(q, k_cache, v_cache, k_scale, v_scale, lengths, *, layout="BHSD", out=None, workspace=None,
              num_splits=0):
    """Attention over int8 or fp8 caches read as code * scale; lengths[b] = valid slots."""
    dev = _dev([q, k_cache, v_cache, k_scale, v_scale], lengths)
    desc = desc_for(q, k_cache, layout, num_splits)
    sc = _scales(k_cache, k_scale, v_scale, layout)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace(desc, dev, workspace)
    check(lib().gqa_decode_attend_q8(ctypes.byref(desc), ctypes.byref(sc), q.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), lengths.data_ptr(), out.data_ptr(), wptr, wbytes,
                                     _stream(dev)), "gqa_decode_attend_q8")
    return out


def step_q8(q, k_cache, v_cache, k_scale, v_scale, k_new, v_new, lengths, *, layout="BHSD", out=None,
            workspace=None, num_splits=0):
    """Quantizing append at lengths[b], then attention over lengths[b] + 1 slots."""
    dev = _dev([q, k_cache, v_cache, k_scale, v_scale, k_new, v_new], lengths)
    desc = desc_for(q, k_cache, layout, num_splits)
    sc = _scales(k_cache, k_scale, v_scale, layout)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace(desc, dev, workspace)
    check(lib().gqa_decode_step_q8(ctypes.byref(desc), ctypes.byref(sc), q.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(),
                                   out.data_ptr(), wptr, wbytes, _stream(dev)), "gqa_decode_step_q8")
    return out


# ---------------------------------------------------------------------------
# Calls with options: any combination of a cache map, int8 scales and rotary
# encoding (gqa_decode_opts_t).
# ---------------------------------------------------------------------------
class Rope:
    """Rotary encoding of q and the new key (gqa_rope_t).

    cos, sin: float32 (max_pos, D/2) device tensors; mode "half" or
    "interleaved"; positions: int32 (B,) device tensor or None (the new slot
    lengths[b]); q_gain / k_gain: float32 (D,) device tensors or None, with eps
    (>= 0) exactly when a gain is given."""

    def __init__(self, cos, sin, mode="half", positions=None, q_gain=None, k_gain=None, eps=None):
        if mode not in ROPE_MODES:
            raise ValueError(f"mode must be one of {list(ROPE_MODES)}")
        for t in (cos, sin, q_gain, k_gain):
            if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda):
                raise ValueError("rope tables and gains are contiguous float32 device tensors")
        if positions is not None and (positions.dtype != torch.int32 or not positions.is_contiguous()):
            raise ValueError("positions is a contiguous int32 tensor")
        if cos.dim() != 2 or cos.shape != sin.shape:
            raise ValueError("cos / sin are (max_pos, D/2)")
        self.cos, self.sin, self.mode, self.positions = cos, sin, mode, positions
        self.q_gain, self.k_gain, self.eps = q_gain, k_gain, eps

    def struct(self) -> RopeT:
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        return RopeT(self.cos.data_ptr(), self.sin.data_ptr(), self.cos.shape[0], ROPE_MODES[self.mode],
                     ptr(self.positions), ptr(self.q_gain), ptr(self.k_gain),
                     -1.0 if self.eps is None else float(self.eps))


class Softmax:
    """Softmax variants (gqa_softmax_t): sink = float32 (Hq,) device logits or
    None; smooth = a zero logit for every head; softcap > 0 caps the scaled
    scores; window > 0 keeps the last `window` slots plus the kept prefix
    (kept_prefix for every sequence, or kept_prefix_per_seq: int32 (B,) device)."""

    def __init__(self, sink=None, smooth=False, softcap=0.0, window=0, kept_prefix=0, kept_prefix_per_seq=None):
        if sink is not None and (sink.dtype != torch.float32 or not sink.is_contiguous() or not sink.is_cuda):
            raise ValueError("sink is a contiguous float32 device tensor")
        if kept_prefix_per_seq is not None and (kept_prefix_per_seq.dtype != torch.int32
                                                or not kept_prefix_per_seq.is_contiguous()):
            raise ValueError("kept_prefix_per_seq is a contiguous int32 tensor")
        self.sink, self.smooth, self.softcap = sink, bool(smooth), float(softcap)
        self.window, self.kept_prefix, self.kept_prefix_per_seq = int(window), int(kept_prefix), kept_prefix_per_seq

    def struct(self) -> SoftmaxT:
        ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
        return SoftmaxT(ptr(self.sink), int(self.smooth), self.softcap, self.window, self.kept_prefix,
                        ptr(self.kept_prefix_per_seq))


def _opts(desc_args, *, table=None, kind=None, table_host=None, k_scale=None, v_scale=None, k_cache=None,
          layout="BHSD", rope=None, softmax=None):
    """(desc, opts, keep-alive) for an _ex call; desc_args = (B, Hq, D, kv_code, qo_code, num_splits, Hkv)."""
    B, Hq, D, kv_code, qo_code, ns, Hkv = desc_args
    keep = []
    o = OptsT()
    if table is not None:
        desc, m, k = _mapped_desc(B, Hq, D, kv_code, qo_code, k_cache, kind, layout, table, ns, Hkv, table_host)
        keep += [m, k]
        o.map = ctypes.pointer(m)
    else:
        if layout == "BHSD":
            Bc, Hc, S, Dc = k_cache.shape
        else:
            Bc, S, Hc, Dc = k_cache.shape
        if Bc != B or Dc != D or (Hkv is not None and Hc != Hkv):
            raise ValueError("cache shape disagrees with q / new rows")
        desc = make_desc(B, Hq, Hc, D, S, layout, kv_code, qo_code, ns)
    if k_scale is not None:
        sc = _scales(k_cache, k_scale, v_scale, layout)
        keep.append(sc)
        o.scales = ctypes.pointer(sc)
    if rope is not None:
        r = rope.struct()
        keep.append(r)
        o.rope = ctypes.pointer(r)
    if softmax is not None:
        v = softmax.struct()
        keep.append(v)
        o.softmax = ctypes.pointer(v)
    return desc, o, keep


def workspace_size_ex(desc: Desc, opts: OptsT) -> int:
    n = ctypes.c_size_t(0)
    check(lib().gqa_decode_workspace_size_ex(ctypes.byref(desc), ctypes.byref(opts), ctypes.byref(n)),
          "gqa_decode_workspace_size_ex")
    return n.value


def _workspace_ex(desc, opts, dev, workspace):
    need = workspace_size_ex(desc, opts)
    if need == 0:
        return workspace, None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def append_ex(k_cache, v_cache, k_new, v_new, lengths, *, layout="BHSD", table=None, kind=None, table_host=None,
              k_scale=None, v_scale=None, rope=None, qo_dtype=None):
    """In-place append with options (map, int8 scales, rotary encoding of the key).
    For int8 caches the new rows are activations (float32 or bfloat16)."""
    tens = [k_cache, v_cache, k_new, v_new] + ([k_scale, v_scale] if k_scale is not None else [])
    dev = _dev(tens, lengths)
    B, Hkv, D = k_new.shape
    kv = _dtype_code(k_cache.dtype)
    qo = _dtype_code(k_new.dtype) if kv in (I8, FP8) else (kv if qo_dtype is None else _dtype_code(qo_dtype))
    desc, o, keep = _opts((B, Hkv, D, kv, qo, 0, Hkv), table=table, kind=kind, table_host=table_host,
                          k_scale=k_scale, v_scale=v_scale, k_cache=k_cache, layout=layout, rope=rope)
    check(lib().gqa_decode_append_ex(ctypes.byref(desc), ctypes.byref(o), k_cache.data_ptr(), v_cache.data_ptr(),
                                     k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(), _stream(dev)),
          "gqa_decode_append_ex")
    del keep


def attend_ex(q, k_cache, v_cache, lengths, *, layout="BHSD", table=None, kind=None, table_host=None, k_scale=None,
              v_scale=None, softmax=None, out=None, workspace=None, num_splits=0):
    """Read-only attention with options (map, int8 scales, softmax variants)."""
    tens = [q, k_cache, v_cache] + ([k_scale, v_scale] if k_scale is not None else [])
    dev = _dev(tens, lengths)
    B, Hq, D = q.shape
    desc, o, keep = _opts((B, Hq, D, _dtype_code(k_cache.dtype), _dtype_code(q.dtype), num_splits, None),
                          table=table, kind=kind, table_host=table_host, k_scale=k_scale, v_scale=v_scale,
                          k_cache=k_cache, layout=layout, softmax=softmax)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace_ex(desc, o, dev, workspace)
    check(lib().gqa_decode_attend_ex(ctypes.byref(desc), ctypes.byref(o), q.data_ptr(), k_cache.data_ptr(),
                                     v_cache.data_ptr(), lengths.data_ptr(), out.data_ptr(), wptr, wbytes,
                                     _stream(dev)), "gqa_decode_attend_ex")
    del keep
    return out


def step_ex(q, k_cache, v_cache, k_new, v_new, lengths, *, layout="BHSD", table=None, kind=None, table_host=None,
            k_scale=None, v_scale=None, rope=None, softmax=None, out=None, workspace=None, num_splits=0):
    """Decode step with options (map, int8 scales, rotary encoding, softmax variants). Returns out."""
    tens = [q, k_cache, v_cache, k_new, v_new] + ([k_scale, v_scale] if k_scale is not None else [])
    dev = _dev(tens, lengths)
    B, Hq, D = q.shape
    desc, o, keep = _opts((B, Hq, D, _dtype_code(k_cache.dtype), _dtype_code(q.dtype), num_splits, None),
                          table=table, kind=kind, table_host=table_host, k_scale=k_scale, v_scale=v_scale,
                          k_cache=k_cache, layout=layout, rope=rope, softmax=softmax)
    if out is None:
        out = torch.empty_like(q)
    workspace, wptr, wbytes = _workspace_ex(desc, o, dev, workspace)
    check(lib().gqa_decode_step_ex(ctypes.byref(desc), ctypes.byref(o), q.data_ptr(), k_cache.data_ptr(),
                                   v_cache.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), lengths.data_ptr(),
                                   out.data_ptr(), wptr, wbytes, _stream(dev)), "gqa_decode_step_ex")
    del keep
    return out

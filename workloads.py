"""Seeded synthetic inputs for the GQA decode step.

Shared by the tests, the smoke check and the benchmark, and fed identically to
the HIP library and to the float64 oracle.  This module holds no attention
arithmetic: it only draws random numbers, casts them to the storage type and
writes the stale-slot filler.

The five workloads follow the shapes, distributions and length mixes given for
this decode step (tiny, Llama-3-8B-like layer, ragged batch, long context,
large group).  ``lengths`` is always the number of tokens held *before* the
step's append (the step writes the new key/value at slot ``lengths[b]`` and
then attends ``lengths[b] + 1`` slots); slots ``>= lengths[b]`` start out
holding the workload's stale filler, or the plain random draw where none is
given.

Draw order (one ``torch.Generator`` seeded with the workload's seed, on the
device the tensors are made on): q, K cache, V cache, new K, new V, stale
signs.  ``lengths`` comes from a CPU generator with the same seed so it does not
depend on the device.  fp32 draws are rounded to bf16 to nearest-even by
``Tensor.to``.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    capacity: int
    layout: str            # "BHSD" = (B, Hkv, S, D); "BSHD" = (B, S, Hkv, D)
    kv_dtype: str          # "f32" | "bf16" | "i8" / "fp8" (int8 / E4M3 codes + per-row scales: make_q8)
    qo_dtype: str          # "f32" | "bf16"
    len_lo: int            # pre-append length range, inclusive
    len_hi: int
    key_scale: float = 1.0
    stale: str = "none"    # "none" | "const:<v>" | "pm:<v>" (random sign)
    note: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 1, B=2, Hq=4, Hkv=2, D=4, capacity=8, layout="BHSD", kv_dtype="f32", qo_dtype="f32",
                 len_lo=1, len_hi=7, stale="const:1000",
                 note="B=2 Hq=4 Hkv=2 D=4 cap=8 fp32, lengths U[1,7], stale 1e3"),
        Workload("llama3_8b_layer", 2, B=32, Hq=32, Hkv=8, D=128, capacity=4097, layout="BHSD", kv_dtype="bf16",
                 qo_dtype="bf16", len_lo=4096, len_hi=4096,
                 note="B=32 Hq=32 Hkv=8 D=128, 4096 cached + 1 new, bf16"),
        Workload("ragged_batch", 3, B=64, Hq=64, Hkv=8, D=128, capacity=8192, layout="BSHD", kv_dtype="bf16",
                 qo_dtype="bf16", len_lo=0, len_hi=8191, stale="pm:10000",
                 note="B=64 Hq=64 Hkv=8 D=128 cap=8192 (B,S,Hkv,D), attended counts U[1,8192], stale +-1e4"),
        Workload("long_context", 4, B=4, Hq=32, Hkv=8, D=128, capacity=131073, layout="BHSD", kv_dtype="bf16",
                 qo_dtype="bf16", len_lo=131072, len_hi=131072, key_scale=3.0,
                 note="B=4 Hq=32 Hkv=8 D=128, 131072 cached + 1 new, keys x3"),
        Workload("large_group", 5, B=128, Hq=64, Hkv=1, D=128, capacity=2048, layout="BHSD", kv_dtype="bf16",
                 qo_dtype="bf16", len_lo=1023, len_hi=2047,
                 note="B=128 Hq=64 Hkv=1 D=128 cap=2048, attended counts U[1024,2048]"),
    ]
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def cache_shape(w: Workload, capacity: int | None = None):
    S = w.capacity if capacity is None else capacity
    return (w.B, w.Hkv, S, w.D) if w.layout == "BHSD" else (w.B, S, w.Hkv, w.D)


def draw_lengths(w: Workload) -> torch.Tensor:
    g = torch.Generator().manual_seed(w.seed)
    return torch.randint(w.len_lo, w.len_hi + 1, (w.B,), generator=g, dtype=torch.int64).to(torch.int32)


def make_inputs(w: Workload, device="cpu", lengths: torch.Tensor | None = None) -> dict:
    """Seeded inputs of workload ``w`` as torch tensors on ``device``.

    Returns a dict with q (B,Hq,D), k_cache / v_cache (layout), k_new / v_new
    (B,Hkv,D), lengths int32 (B,) (pre-append counts).
    """
    g = torch.Generator(device=device).manual_seed(w.seed)
    L = draw_lengths(w) if lengths is None else lengths.to(torch.int32).cpu()
    kvt, qot = TORCH_DTYPE[w.kv_dtype], TORCH_DTYPE[w.qo_dtype]

    def randn(shape, scale=1.0):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        return x

    q = randn((w.B, w.Hq, w.D)).to(qot)
    k_cache = randn(cache_shape(w), w.key_scale).to(kvt)
    v_cache = randn(cache_shape(w)).to(kvt)
    k_new = randn((w.B, w.Hkv, w.D), w.key_scale).to(kvt)
    v_new = randn((w.B, w.Hkv, w.D)).to(kvt)
    if w.stale != "none":
        kind, val = w.stale.split(":")
        val = float(val)
        S = w.capacity
        slot = torch.arange(S, device=device)
        stale = slot[None, :] >= L.to(device)[:, None].to(torch.int64)          # (B, S)
        stale = stale[:, None, :, None] if w.layout == "BHSD" else stale[:, :, None, None]
        for cache in (k_cache, v_cache):
            if kind == "const":
                fill = torch.full(cache.shape, val, device=device, dtype=torch.float32)
            else:
                sign = torch.randint(0, 2, cache.shape, generator=g, device=device, dtype=torch.int8)
                fill = (sign.to(torch.float32) * 2 - 1) * val
            cache.copy_(torch.where(stale, fill.to(kvt), cache))
            del fill
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, k_new=k_new, v_new=v_new,
                lengths=L.to(device))


def make_mapped(inp: dict, w: Workload, kind: str, *, block_size: int = 16, num_rows: int | None = None,
                spare_blocks: int = 7, seed: int = 0, shuffle: bool = True) -> dict:
    """The same logical caches stored through a map (data movement only).

    ``kind == "slots"``: a continuous cache of ``num_rows`` rows (default 2B+1);
    batch row b lives at row ``map[b]`` of a seeded permutation.  ``"paged"``:
    a pool of ``B * ceil(S / block_size) + spare_blocks`` blocks; the table maps
    each sequence's blocks to a seeded permutation of the pool (``shuffle=False``:
    to consecutive blocks in order).  Cache rows or blocks that no sequence
    maps, and the slots past the capacity in the last block, hold NaN bit
    patterns (int8 codes: 127, with NaN scales).  Int8 inputs (``k_scale`` /
    ``v_scale`` present) have their scale arrays stored through the same map,
    in the mapped caches' shape without the last axis.  Returns a dict like
    ``inp`` with the caches (and scales) replaced, plus ``map`` (int32, same
    device) and, for a paged cache, ``block_size`` and the mapped capacity (a
    multiple of it).
    """
    gen = torch.Generator().manual_seed(1000 + w.seed * 17 + seed)
    dev = inp["k_cache"].device
    B, Hkv, D, S = w.B, w.Hkv, w.D, w.capacity

    def garbage(shape, like):
        if like.dtype == torch.int8:
            return torch.full(shape, 127, dtype=torch.int8, device=dev)
        if like.dtype == torch.float8_e4m3fn:       # the E4M3 NaN pattern
            return torch.full(shape, 0x7F, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
        if like.dtype == torch.bfloat16:
            return torch.full(shape, 0x7FC1, dtype=torch.int16, device=dev).view(torch.bfloat16)
        return torch.full(shape, 0x7FC00001, dtype=torch.int32, device=dev).view(torch.float32)

    names = [("k_cache", False), ("v_cache", False)]
    if "k_scale" in inp:
        names += [("k_scale", True), ("v_scale", True)]
    out = dict(inp)
    if kind == "slots":
        R = num_rows if num_rows is not None else 2 * B + 1
        slot_ids = torch.randperm(R, generator=gen)[:B].to(torch.int32)
        for name, _ in names:
            c = inp[name]
            m = garbage((R,) + tuple(c.shape[1:]), c)
            m[slot_ids.to(dev).long()] = c
            out[name] = m
        out["map"] = slot_ids.to(dev)
        out["capacity"] = S
        return out
    if kind != "paged":
        raise ValueError(kind)
    bs = block_size
    nb = -(-S // bs)
    total = B * nb + spare_blocks
    order = torch.randperm(total, generator=gen) if shuffle else torch.arange(total)
    table = order[: B * nb].to(torch.int32).view(B, nb)
    idx = table.to(dev).long().flatten()
    pad = nb * bs - S
    for name, is_scale in names:
        c = inp[name].unsqueeze(-1) if is_scale else inp[name]   # scales: a trailing axis of 1
        E = c.shape[-1]
        if w.layout == "BHSD":                                   # (B, Hkv, S, E) -> blocks (B*nb, Hkv, bs, E)
            full = torch.cat([c, garbage((B, Hkv, pad, E), c)], dim=2) if pad else c
            blocks = full.view(B, Hkv, nb, bs, E).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, bs, E)
            pool = garbage((total, Hkv, bs, E), c)
        else:                                                    # (B, S, Hkv, E) -> blocks (B*nb, bs, Hkv, E)
            full = torch.cat([c, garbage((B, pad, Hkv, E), c)], dim=1) if pad else c
            blocks = full.view(B, nb, bs, Hkv, E).reshape(B * nb, bs, Hkv, E)
            pool = garbage((total, bs, Hkv, E), c)
        pool[idx] = blocks
        out[name] = pool.squeeze(-1) if is_scale else pool
    out["map"] = table.to(dev)
    out["block_size"] = bs
    out["capacity"] = nb * bs
    return out


def make_q8(w: Workload, device="cpu", lengths: torch.Tensor | None = None) -> dict:
    """Seeded inputs for int8 (``w.kv_dtype == "i8"``) or fp8 (``"fp8"``, E4M3
    codes as torch.float8_e4m3fn) caches with per-row float32 scales.

    Int8 caches hold codes drawn uniformly from [-127, 127] and the scales are
    drawn uniformly from [0.5, 1.5] * 3 * key_scale / 127 (keys) or
    [0.5, 1.5] * 3 / 127 (values), so cached values span about +-3 like the
    normal draws of ``make_inputs``.  Fp8 caches hold bytes drawn uniformly
    over all codes, the two NaN patterns replaced by +-0 (so every finite code,
    subnormals included, occurs), with 448 in place of 127 in the scales.  q and the new key/value rows are normal
    draws stored as ``w.qo_dtype`` (the step quantizes the new rows itself).
    With ``w.stale != "none"`` the scales of slots >= lengths[b] are NaN, so a
    read past the valid slots shows up in the output.  Draw order (one
    generator seeded with ``w.seed + 5000``): q, K codes, V codes, K scales,
    V scales, new K, new V.  Returns q, k_cache, v_cache, k_scale, v_scale,
    k_new, v_new, lengths.
    """
    g = torch.Generator(device=device).manual_seed(w.seed + 5000)
    L = draw_lengths(w) if lengths is None else lengths.to(torch.int32).cpu()
    qot = TORCH_DTYPE[w.qo_dtype]
    shape = cache_shape(w)
    sshape = shape[:3]

    def randn(shp, scale=1.0):
        x = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        return x.mul_(scale) if scale != 1.0 else x

    q = randn((w.B, w.Hq, w.D)).to(qot)
    fp8 = w.kv_dtype == "fp8"
    if fp8:
        def codes():
            c = torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32)
            c = torch.where((c & 0x7F) == 0x7F, c & 0x80, c)           # NaN patterns -> +-0
            return c.to(torch.uint8).view(torch.float8_e4m3fn)
        k_cache, v_cache = codes(), codes()
    else:
        k_cache = torch.randint(-127, 128, shape, generator=g, device=device, dtype=torch.int8)
        v_cache = torch.randint(-127, 128, shape, generator=g, device=device, dtype=torch.int8)
    qmax = 448.0 if fp8 else 127.0
    k_scale = (torch.rand(sshape, generator=g, device=device) + 0.5).mul_(3.0 * w.key_scale / qmax)
    v_scale = (torch.rand(sshape, generator=g, device=device) + 0.5).mul_(3.0 / qmax)
    k_new = randn((w.B, w.Hkv, w.D), w.key_scale).to(qot)
    v_new = randn((w.B, w.Hkv, w.D)).to(qot)
    if w.stale != "none":
        slot = torch.arange(w.capacity, device=device)
        stale = slot[None, :] >= L.to(device)[:, None].to(torch.int64)          # (B, S)
        stale = stale[:, None, :] if w.layout == "BHSD" else stale[:, :, None]
        for sc in (k_scale, v_scale):
            sc.masked_fill_(stale.expand(sshape), float("nan"))
    return dict(q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale, k_new=k_new, v_new=v_new,
                lengths=L.to(device))


def to_numpy_storage(t: torch.Tensor) -> np.ndarray:
    """A tensor's stored bits as the oracle takes them: float32, int8, uint16 bf16
    patterns, or uint8 E4M3 patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    if t.dtype in (torch.float32, torch.int8):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def algorithmic_bytes(w: Workload, lengths, window: int = 0, prefix: int = 0) -> int:
    """Bytes one step must move at minimum: valid K+V read (the new token
    included), Q read, new K/V write, output write.  Int8 and fp8 caches move a
    float32 scale with every row and take the new rows in the q/out dtype.  A
    sliding window (with a kept prefix) reads only the slots it attends."""
    e_qo = 4 if w.qo_dtype == "f32" else 2
    n = np.asarray(lengths, dtype=np.int64) + 1
    if window > 0:
        wv = np.minimum(n, window)
        n = wv + np.minimum(prefix, n - wv)
    if w.kv_dtype in ("i8", "fp8"):
        row = w.D + 4
        kv_read = int(n.sum()) * w.Hkv * row * 2
        return kv_read + 2 * w.B * w.Hq * w.D * e_qo + 2 * w.B * w.Hkv * (w.D * e_qo + row)
    e_kv = 4 if w.kv_dtype == "f32" else 2
    kv_read = int(n.sum()) * w.Hkv * w.D * 2 * e_kv
    return kv_read + 2 * w.B * w.Hq * w.D * e_qo + 2 * w.B * w.Hkv * w.D * e_kv


def custom(B, Hq, Hkv, D, capacity, layout="BHSD", kv_dtype="bf16", qo_dtype="bf16", seed=0, stale="none",
           key_scale=1.0) -> Workload:
    """A workload of any shape (lengths are passed to ``make_inputs``)."""
    return Workload(f"custom{seed}", seed, B=B, Hq=Hq, Hkv=Hkv, D=D, capacity=capacity, layout=layout,
                    kv_dtype=kv_dtype, qo_dtype=qo_dtype, len_lo=0, len_hi=max(capacity - 1, 0),
                    key_scale=key_scale, stale=stale)


def rope_tables(max_pos: int, D: int, device="cpu", base: float = 10000.0):
    """Rotary planes as a caller would pass them: float32 cos / sin tables of
    shape (max_pos, D/2) for the angles p * base^(-2i/D) (an input of the
    rotary step, computed in float64 and rounded once)."""
    i = torch.arange(D // 2, dtype=torch.float64)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * base ** (-2.0 * i / D)[None, :]
    return ang.cos().to(torch.float32).to(device), ang.sin().to(torch.float32).to(device)

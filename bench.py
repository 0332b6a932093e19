"""Benchmark of the GQA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one gqa_decode_step call (in-place append + length-masked GQA
attention over every sequence of the batch, i.e. one layer's decode) on
seeded synthetic inputs already resident in HBM.  W untimed steps, then K
timed back-to-back on one stream between HIP events, replayed from one HIP
graph that holds the K steps (--no-graph: launched one by one).  The cache tensors
rotate over R copies so the bytes one rotation touches exceed the 256 MB
Infinity Cache and every step reads K/V from HBM.

Prints ONE JSON line: value = achieved HBM GB/s over the algorithmic bytes
(valid K+V read incl. the new token, Q read, new K/V write, output write),
plus steps/s, the fraction of the 8 TB/s peak, and the float64 oracle timed on
this host's cores over a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "achieved HBM GB/s (% of MI355X peak) + decode steps/sec per config"
PROFILES = os.path.join(ROOT, "profiles")
# Every source the library is built from: the recorded traffic counts only
# while none of them has changed since the counters were taken.
KERNEL_SOURCES = sorted(
    [os.path.join("gqa_decode_attention_amd/csrc", f) for f in os.listdir(os.path.join(ROOT, "gqa_decode_attention_amd/csrc"))
     if f.endswith((".hip", ".cpp", ".h"))]) + ["include/gqa_decode.h", "gqa_decode_attention_amd/build.py"]


PER_CONFIG_PAUSE_S = 3.0  # idle time before each per_config measurement


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernels as they are now; otherwise None."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, budget_s=12.0, rope=None, variants=None, window=0, prefix=0):
    """The float64 oracle on this host's cores over a bounded sample of the same
    inputs: whole sequences (all query heads), repeated until about budget_s
    seconds of CPU work, scaled to GB/s with the same byte formula."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    L = inp["lengths"].cpu().numpy()
    q8 = w.kv_dtype in ("i8", "fp8")
    names = ("q", "k_cache", "v_cache", "k_new", "v_new") + (("k_scale", "v_scale") if q8 else ())

    def host(nb):
        return {k: W.to_numpy_storage(inp[k][:nb]) for k in names}

    def run(st, nb):
        t0 = time.perf_counter()
        if variants is not None and rope is None:
            oracle.step_variants(st["q"], w.qo_dtype, st["k_cache"], st["v_cache"], st["k_new"], st["v_new"],
                                 w.kv_dtype, L[:nb], w.layout, w.Hq, w.Hkv,
                                 scales=(st["k_scale"], st["v_scale"]) if q8 else None, **variants)
        elif rope is not None and q8:
            oracle.step_q8_rope(st["q"], w.qo_dtype, st["k_cache"], st["v_cache"], st["k_scale"], st["v_scale"],
                                st["k_new"], st["v_new"], L[:nb], w.layout, w.Hq, w.Hkv, *rope)
        elif rope is not None:
            oracle.step_rope(st["q"], w.qo_dtype, st["k_cache"], st["v_cache"], st["k_new"], st["v_new"], w.kv_dtype,
                             L[:nb], w.layout, w.Hq, w.Hkv, *rope)
        elif q8:
            oracle.step_q8(st["q"], w.qo_dtype, st["k_cache"], st["v_cache"], st["k_scale"], st["v_scale"],
                           st["k_new"], st["v_new"], L[:nb], w.layout, w.Hq, w.Hkv)
        else:
            oracle.step(st["q"], w.qo_dtype, st["k_cache"], st["v_cache"], st["k_new"], st["v_new"], w.kv_dtype,
                        L[:nb], w.layout, w.Hq, w.Hkv)
        return time.perf_counter() - t0

    st1 = host(1)
    t1 = run(st1, 1)                      # one sequence, to size the sample
    nb = int(max(1, min(w.B, budget_s / max(t1, 1e-9))))
    st = host(nb)
    reps, t = 0, 0.0
    while t < budget_s and reps < 100000:
        t += run(st, nb)
        reps += 1
    sub = W.Workload(**{**w.__dict__, "B": nb})
    nbytes = W.algorithmic_bytes(sub, L[:nb], window, prefix) * reps
    gbs = nbytes / t / 1e9
    fn = ("step_q8" if q8 else "step") if rope is None else ("step_q8_rope" if q8 else "step_rope")
    if variants is not None and rope is None:
        fn = "step_variants"
    sample = (f"oracle.{fn} over sequences 0..{nb - 1} of {w.B} (all {w.Hq} query heads) of the same inputs, "
              f"{reps} repetition(s), {t:.1f} s")
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "kind": "oracle", "sample": sample,
            "steps_per_sec_equiv": round(gbs * 1e9 / W.algorithmic_bytes(w, L, window, prefix), 6),
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}


def calibration_copy(mib: int, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters of a profile run: each launch reads and writes mib MiB."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_per_launch": mib << 20, "launches": reps}), flush=True)


def time_replay(step, steps: int, warmup: int, graph: bool = True) -> float:
    """Mean milliseconds per step over `steps` steps after `warmup` untimed ones:
    the timed steps are captured once in a HIP graph and replayed (graph=False:
    launched one by one), between HIP events on the stream they run on."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = None
    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                step(i)
        torch.cuda.synchronize()
        g.replay()  # untimed: the graph's own first launch
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    if g is not None:
        g.replay()
    else:
        for i in range(steps):
            step(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure_plain(name: str, steps: int, warmup: int, graph: bool = True) -> dict:
    """One workload's plain step (dense caches in its own storage type, no
    options), timed as the headline is: the per-config entry of the JSON line."""
    import torch
    import gqa_decode_attention_amd as g
    import workloads as W
    w = W.WORKLOADS[name]
    inp = W.make_inputs(w, "cuda")
    L = inp["lengths"].cpu().numpy()
    nbytes = W.algorithmic_bytes(w, L)
    kv_bytes = 2 * inp["k_cache"].numel() * inp["k_cache"].element_size()
    R = min(16, math.ceil(3 * MALL_BYTES / kv_bytes)) if 16 * kv_bytes >= MALL_BYTES else 1
    caches = [(inp["k_cache"], inp["v_cache"])] + [(inp["k_cache"].clone(), inp["v_cache"].clone())
                                                   for _ in range(R - 1)]
    desc = g.desc_for(inp["q"], inp["k_cache"], w.layout)
    plan = g.get_plan(desc)
    ws = torch.empty(max(plan["workspace_bytes"], 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(inp["q"])

    def step(i):
        kc, vc = caches[i % R]
        g.step(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], layout=w.layout, out=out, workspace=ws)

    ms = time_replay(step, steps, warmup, graph)
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = traffic_from_profiles(name)
    entry = {"us_per_step": round(ms * 1e3, 3), "steps_per_sec": round(1000.0 / ms, 1), "gbs": round(gbs, 1),
             "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_step": nbytes, "cache_rotation": R,
             "plan": plan, "traffic_ratio": None if traffic is None else round(traffic / nbytes, 4)}
    if name == "tiny":
        entry["note"] = "launch-latency bound (at most 1.4 KB per step); frac shown, not meaningful"
    del caches, inp, ws, out
    torch.cuda.empty_cache()
    return entry


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_layer")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = the library's plan")
    ap.add_argument("--batch", type=int, default=0,
                    help="run the workload with this many sequences instead of its own (lengths drawn the same "
                         "way; the workload is then named <workload>_b<batch>)")
    ap.add_argument("--cache", default="dense",
                    help="dense (default), slots (slot-indexed rows), pagedN (pool of N-slot blocks in a "
                         "seeded random order) or pagedNseq (blocks in pool order)")
    ap.add_argument("--kv", default="native", choices=["native", "int8", "fp8"],
                    help="native: the workload's cache dtype; int8 / fp8: int8 or fp8 (E4M3) codes with "
                         "per-row float32 scales (the step quantizes the new rows)")
    ap.add_argument("--rope", default="none", choices=["none", "half", "interleaved"],
                    help="rotate q and the new key with rotary planes in the append (positions = lengths)")
    ap.add_argument("--window", type=int, default=0, help="sliding window of the softmax (0: none)")
    ap.add_argument("--kept-prefix", type=int, default=0, help="slots kept beside the window")
    ap.add_argument("--softcap", type=float, default=0.0, help="cap of the scaled scores (0: none)")
    ap.add_argument("--sink", action="store_true", help="a per-query-head sink logit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps one by one instead of replaying them from one HIP graph")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip the per_config timings of the five workloads' plain steps")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_decode_attention_amd as g
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibration_copy_mib > 0:
        calibration_copy(args.calibration_copy_mib)
        return
    g.lib()
    w = W.WORKLOADS[args.workload]
    if args.batch > 0 and args.batch != w.B:
        w = W.Workload(**{**w.__dict__, "B": args.batch, "name": f"{w.name}_b{args.batch}"})
    dev = "cuda"
    q8 = args.kv in ("int8", "fp8")
    if q8:
        if args.cache != "dense":
            raise SystemExit("--kv int8/fp8 takes dense caches")
        w = W.Workload(**{**w.__dict__, "kv_dtype": "i8" if args.kv == "int8" else "fp8"})
        inp = W.make_q8(w, dev)
    else:
        inp = W.make_inputs(w, dev)
    L = inp["lengths"].cpu().numpy()
    nbytes = W.algorithmic_bytes(w, L, args.window, args.kept_prefix)
    n_att = L.astype("int64") + 1
    if args.window > 0:
        wv = n_att.clip(max=args.window)
        n_att = wv + (n_att - wv).clip(max=args.kept_prefix)
    smx, smx_np = None, None
    if args.window or args.softcap or args.sink:
        sink = torch.randn(w.Hq, generator=torch.Generator().manual_seed(1)).to(dev) if args.sink else None
        smx = g.Softmax(sink=sink, softcap=args.softcap, window=args.window, kept_prefix=args.kept_prefix)
        smx_np = dict(sink=None if sink is None else sink.cpu().numpy(), softcap=args.softcap, window=args.window,
                      prefix=args.kept_prefix)
    desc = g.desc_for(inp["q"], inp["k_cache"], w.layout, args.num_splits)
    plan = g.get_plan(desc)
    if args.window > 0:
        # With a window known on the host the library plans its splits over the
        # slots a sequence can walk (window + kept prefix + 32), not the
        # capacity: that plan is the one of a descriptor of that capacity.
        span = min(desc.capacity, args.window + args.kept_prefix + 32)
        plan = dict(g.get_plan(g.make_desc(desc.batch, desc.num_q_heads, desc.num_kv_heads, desc.head_dim, span,
                                           w.layout, desc.kv_dtype, desc.qo_dtype, args.num_splits)),
                    planned_span=span)
    kind, table = None, None
    inp_dense = inp
    if args.cache != "dense":
        # The same logical caches stored through a map (slot-indexed rows or a
        # block pool); the bytes the step must move are the same.
        if args.cache == "slots":
            kind, m = "slots", W.make_mapped(inp, w, "slots")
        elif args.cache.startswith("paged"):
            seq = args.cache.endswith("seq")          # pagedNseq: blocks in pool order
            bs = int(args.cache[5:-3] if seq else args.cache[5:])
            kind, m = "paged", W.make_mapped(inp, w, "paged", block_size=bs, shuffle=not seq)
        else:
            raise SystemExit(f"--cache {args.cache}: dense, slots or pagedN")
        inp = {**inp, "k_cache": m["k_cache"], "v_cache": m["v_cache"]}
        table = m["map"]
        table_host = table.cpu()      # the host copy the library validates, made once
    kv_bytes = 2 * inp["k_cache"].numel() * inp["k_cache"].element_size()
    if q8:
        kv_bytes += 2 * inp["k_scale"].numel() * 4
    # Rotate over R cache copies so one rotation touches over 3x the Infinity
    # Cache; a workload too small to matter (16 copies would still fit) uses one.
    R = min(16, math.ceil(3 * MALL_BYTES / kv_bytes)) if 16 * kv_bytes >= MALL_BYTES else 1
    names = ("k_cache", "v_cache") + (("k_scale", "v_scale") if q8 else ())
    caches = [tuple(inp[n] for n in names)] + [tuple(inp[n].clone() for n in names) for _ in range(R - 1)]
    rope = None
    wsb = plan["workspace_bytes"]
    if args.rope != "none":
        cos, sin = W.rope_tables(w.capacity, w.D, dev)
        rope = g.Rope(cos, sin, args.rope)
    if rope is not None or smx is not None:
        import ctypes
        rs = rope.struct() if rope is not None else None
        ss = smx.struct() if smx is not None else None
        from gqa_decode_attention_amd import _lib
        sc = _lib._scales(inp["k_cache"], inp["k_scale"], inp["v_scale"], w.layout) if q8 else None
        wsb = g.workspace_size_ex(desc, g.OptsT(None, ctypes.pointer(sc) if sc is not None else None,
                                                ctypes.pointer(rs) if rs is not None else None,
                                                ctypes.pointer(ss) if ss is not None else None))
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])

    def step(i):
        kc, vc = caches[i % R][:2]
        if rope is not None or smx is not None:
            ks, vs = caches[i % R][2:] if q8 else (None, None)
            g.step_ex(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], layout=w.layout, table=table,
                      kind=kind, table_host=table_host if kind else None, k_scale=ks, v_scale=vs, rope=rope,
                      softmax=smx, out=out, workspace=ws, num_splits=args.num_splits)
        elif q8:
            ks, vs = caches[i % R][2:]
            g.step_q8(inp["q"], kc, vc, ks, vs, inp["k_new"], inp["v_new"], inp["lengths"], layout=w.layout, out=out,
                      workspace=ws, num_splits=args.num_splits)
        elif kind is None:
            g.step(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], layout=w.layout, out=out,
                   workspace=ws, num_splits=args.num_splits)
        else:
            g.step_mapped(inp["q"], kc, vc, inp["k_new"], inp["v_new"], inp["lengths"], table, kind=kind,
                          layout=w.layout, out=out, workspace=ws, num_splits=args.num_splits, table_host=table_host)

    # The K timed steps (cache copies rotating as in the eager loop) are
    # captured once into a HIP graph and replayed: the library launches only
    # kernels (no host sync, no memset), so the replay is the same work without
    # the per-call host marshalling and launch latency.
    t0 = time.perf_counter()
    ms = time_replay(step, args.steps, args.warmup, graph=not args.no_graph)
    wall = time.perf_counter() - t0
    gbs = nbytes / (ms * 1e-3) / 1e9
    del caches
    torch.cuda.empty_cache()

    # Every workload's plain step, timed the same way in the same run.  Each
    # starts after an idle pause: straight after another workload's sustained
    # stream the GPU measured up to 6 % slow (long context: 322 vs 303 us).
    per_config = None
    if not args.no_per_config:
        per_config = {}
        for name in ("tiny", "llama3_8b_layer", "ragged_batch", "long_context", "large_group"):
            time.sleep(PER_CONFIG_PAUSE_S)
            per_config[name] = measure_plain(name, args.steps, args.warmup, graph=not args.no_graph)
            print(json.dumps({"per_config": name, **per_config[name]}), file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        rope_np = None if rope is None else (rope.cos.cpu().numpy(), rope.sin.cpu().numpy(), args.rope)
        cpu = cpu_baseline(w, inp_dense, rope=rope_np, variants=smx_np, window=args.window,
                           prefix=args.kept_prefix)   # the dense oracle on the same logical caches

    kv = {"bf16": "bf16", "f32": "f32", "i8": "i8+f32 row scales", "fp8": "fp8 e4m3+f32 row scales"}[w.kv_dtype]
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_detail": ("scores, softmax and sums in float32; on the matrix-core kernels each softmax weight "
                         "enters the V-sum MFMA as a bf16 hi + lo pair (about 16 significant bits) with float32 "
                         "accumulation"),
        "storage_dtype": kv,
        "data": "synthetic",
        "steps_per_sec": round(1000.0 / ms, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "config": {"workload": w.name, "launch": "eager" if args.no_graph else "hip_graph", "cache": args.cache, "rope": args.rope, "window": args.window,
                   "kept_prefix": args.kept_prefix, "softcap": args.softcap, "sink": args.sink, "batch": w.B, "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.D,
                   "capacity": w.capacity, "layout": w.layout, "kv_dtype": w.kv_dtype, "qo_dtype": w.qo_dtype,
                   "tokens_attended": int(n_att.sum()), "algorithmic_bytes_per_step": nbytes,
                   "cache_rotation": R, "plan": plan},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profiles(w.name)
                     if args.cache == "dense" and not q8 and rope is None and smx is None else None,
                     "per": "one gqa_decode_step call (attention kernel + split combine), HIP events over the "
                            "timed region on the stream the steps run on"},
        "cpu_baseline": cpu,
        "per_config": per_config,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

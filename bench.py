#!/usr/bin/env python3
"""Benchmark of the fused add + RMSNorm + FP8/NVFP4 tail (and the Q/K norm +
RoPE + FP8 store) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 1..5] [--no-sweep] [--no-cpu] [--no-ab]

A step is one call of the fused op on one batch of the workload's seeded
synthetic inputs, already resident in HBM. Inputs and outputs rotate over
enough buffer sets (>= 1 GiB in total) that every call streams from HBM rather
than from the 256 MB last-level cache. The timed region replays a HIP graph
holding K calls, bracketed by device synchronisation; kernel time comes from
HIP events on the launch stream. Eager (host-launched) time per call is
reported beside it.

Prints ONE JSON line. `value` is achieved algorithmic HBM throughput in GB/s
on the headline workload (fp16 [64, 8192] add + RMSNorm + NVFP4, the shape the
pages measure: 0.039 ms on an RTX 5060 Ti, TensorRT-LLM issue #17900,
Performance result). `all_workloads` holds the same figures for every shape.
`kv_store` times the Q/K op with its KV-cache store epilogue (SGLang PR
#32975) on the Q/K workload, writing K|V codes into a shuffled paged pool.
`sf_swizzled` times the NVFP4 op writing its block scales in the 128x4-tiled
GEMM layout. `fusion_ab` times the separated tail (add_rmsnorm, then quant_fp8 or
quant_nvfp4: two kernels and a T-rounded norm tensor between them) against the
fused kernel on the tail workloads, the comparison the pages make (0.103 ms
separated vs 0.039 ms fused, 2.64x).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused add+RMSNorm+FP8/NVFP4 quant: µs/call and achieved HBM GB/s (% peak)"
PEAK_GBS = 8000.0                      # MI355X HBM3E
PAGES_US = {2: 39.0}                   # the pages' fused-tail latency for this exact workload
PAGES_SEPARATED_US = {2: 103.0}        # ... and their separated (two-kernel) latency
AB_WORKLOADS = (2, 3, 4)
ROTATE_BYTES = 1 << 30
SCALARS = os.path.join(ROOT, "tests", "golden", "workload_scalars.json")
TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "nvfp4_quantization_place_amd", "csrc")


def algorithmic_bytes(inp) -> int:
    """Bytes the method must move per call (gamma and scales counted once)."""
    import workloads as W
    if isinstance(inp, W.QKInputs):
        D = inp.head_dim
        C = (inp.nq + inp.nk + inp.nv) * D
        return inp.tokens * C * 3 + inp.tokens * (4 * D + 8) + 4 * D + 4
    M, H = inp.tokens, inp.hidden
    if inp.op == "gated":  # reads x and z, writes codes and scales; no residual
        return int(round(M * H * (2 + 2 + 0.5 + 1 / 16))) + 2 * H + 4
    per = 2 + 2 + 2 + (1 if inp.op == "fp8" else 0.5 + 1 / 16) + (2 if inp.norm_out else 0)
    return int(round(M * H * per)) + 2 * H + 4


def source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Workload:
    """Device-resident inputs and outputs of one workload, in R rotating sets."""

    def __init__(self, k: int, scalars: dict, steps: int, separated: bool = False,
                 kv_store: bool = False, swizzled: bool = False):
        import numpy as np
        import torch

        import workloads as W
        self.k = k
        self.separated = separated
        self.kv_store = kv_store
        self.swizzled = swizzled
        self.inp = W.make_config(k)
        self.bytes = algorithmic_bytes(self.inp) + (self.inp.tokens * 8 if kv_store else 0)
        # a graph of `steps` calls only ever touches `steps` sets
        self.sets = max(2, min(math.ceil(ROTATE_BYTES / self.bytes), steps))
        dev = "cuda"
        inp = self.inp
        if isinstance(inp, W.QKInputs):
            self.kind = "qk"
            qkv = inp.qkv.to(dev)
            self.qkv = [qkv] + [qkv.clone() for _ in range(self.sets - 1)]
            self.out = [torch.empty(qkv.shape, dtype=torch.uint8, device=dev) for _ in range(self.sets)]
            self.gq, self.gk = inp.gamma_q.to(dev), inp.gamma_k.to(dev)
            self.pos = inp.positions.to(dev)
            self.cs = torch.from_numpy(inp.cos_sin).to(dev)
            self.scale = torch.tensor([inp.scale], dtype=torch.float32, device=dev)
            self.dtype = inp.dtype
            self.name = inp.name
            if kv_store:  # pool of 1.25x the tokens' slots, shuffled; Q codes dense
                D = inp.head_dim
                nslots = inp.tokens * 5 // 4
                rng = np.random.default_rng(k)
                self.slots = torch.from_numpy(rng.permutation(nslots)[:inp.tokens].astype(np.int64)).to(dev)
                self.pool = [torch.zeros(nslots, (inp.nk + inp.nv) * D, dtype=torch.uint8, device=dev)
                             for _ in range(self.sets)]
                self.out = [torch.empty(inp.tokens, inp.nq * D, dtype=torch.uint8, device=dev)
                            for _ in range(self.sets)]
                self.name = inp.name + "_kv_store"
            return
        self.kind = inp.op
        self.name = inp.name
        self.dtype = inp.dtype
        x, r = inp.x.to(dev), inp.residual.to(dev)
        self.x = [x] + [x.clone() for _ in range(self.sets - 1)]
        self.res = [r] + [r.clone() for _ in range(self.sets - 1)]
        self.g = inp.gamma.to(dev)
        if inp.op == "fp8":
            s = inp.scale
        else:
            s = scalars[str(k)]["global_scale"]
        self.scale = torch.tensor([s], dtype=torch.float32, device=dev)
        M, H = inp.tokens, inp.hidden
        qcols = H if inp.op == "fp8" else H // 2
        self.q = [torch.empty(M, qcols, dtype=torch.uint8, device=dev) for _ in range(self.sets)]
        sf_shape = (M, H // 16)
        if swizzled:
            import nvfp4_quantization_place_amd as A
            sf_shape = A.nvfp4_swizzled_sf_shape(M, H)
            self.name = inp.name + "_sf_swizzled"
        self.sf = ([torch.empty(*sf_shape, dtype=torch.uint8, device=dev) for _ in range(self.sets)]
                   if inp.op in ("nvfp4", "gated") else None)
        # the separated path always materialises the norm (the quantiser's input)
        self.norm = ([torch.empty_like(x) for _ in range(self.sets)]
                     if inp.norm_out or separated else None)

    def call(self, i: int):
        import nvfp4_quantization_place_amd as A
        j = i % self.sets
        inp = self.inp
        if self.separated:
            n = A.add_rmsnorm(self.x[j], self.res[j], self.g, inp.eps, norm=self.norm[j])
            if self.kind == "fp8":
                A.quant_fp8(n, self.scale, q=self.q[j])
            else:
                A.quant_nvfp4(n, self.scale, q=self.q[j], sf=self.sf[j])
        elif self.kv_store:
            A.qk_norm_rope_fp8_kv_store(self.qkv[j], self.gq, self.gk, self.pos, self.cs, self.scale,
                                        inp.eps, inp.nq, inp.nk, inp.nv, inp.head_dim, self.slots,
                                        self.pool[j], q_out=self.out[j])
        elif self.kind == "qk":
            A.qk_norm_rope_fp8(self.qkv[j], self.gq, self.gk, self.pos, self.cs, self.scale, inp.eps,
                               inp.nq, inp.nk, inp.nv, inp.head_dim, out=self.out[j])
        elif self.swizzled:
            A.add_rmsnorm_quant_nvfp4_swizzled(self.x[j], self.res[j], self.g, self.scale, inp.eps,
                                               q=self.q[j], sf=self.sf[j],
                                               norm=self.norm[j] if self.norm else None)
        elif self.kind == "gated":
            A.gated_rmsnorm_quant_nvfp4(self.x[j], self.res[j], self.g, self.scale, inp.eps,
                                        group=inp.meta["group"], q=self.q[j], sf=self.sf[j])
        elif self.kind == "fp8":
            A.add_rmsnorm_quant_fp8(self.x[j], self.res[j], self.g, self.scale, inp.eps,
                                    q=self.q[j], norm=self.norm[j] if self.norm else None)
        elif self.kind == "nvfp4":
            A.add_rmsnorm_quant_nvfp4(self.x[j], self.res[j], self.g, self.scale, inp.eps,
                                      q=self.q[j], sf=self.sf[j],
                                      norm=self.norm[j] if self.norm else None)
        else:
            raise ValueError(f"no call for workload kind {self.kind!r}")


SPREAD_REPLAYS = 10
GRAPH_WARM_S = 0.025


def time_workload(w: Workload, steps: int, warmup: int, eager: bool = True,
                  spread: bool = True) -> dict:
    import torch
    for i in range(warmup):
        w.call(i)
    torch.cuda.synchronize()
    # eager: host-launched calls, wall clock
    eager_us = None
    if eager:
        t0 = time.perf_counter()
        for i in range(steps):
            w.call(i)
        torch.cuda.synchronize()
        eager_us = round((time.perf_counter() - t0) / steps * 1e6, 3)
    # graph of `steps` calls, replayed
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(2):
            w.call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            w.call(i)
    # warm the graph until the GPU has run it for >= GRAPH_WARM_S (at least 2
    # replays), so the timed replay runs at settled clocks; profiler runs
    # (spread off) keep to 2 replays so their traces stay small
    warm_s = GRAPH_WARM_S if spread else 0.0
    t_w = time.perf_counter()
    reps = 0
    while reps < 2 or time.perf_counter() - t_w < warm_s:
        g.replay()
        torch.cuda.synchronize()
        reps += 1
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    dev_us = ev0.elapsed_time(ev1) * 1e3 / steps
    gbs = w.bytes / (dev_us * 1e-6) / 1e9
    r = dict(workload=w.name, io_dtype=w.dtype, bytes_per_call=w.bytes, rotating_sets=w.sets,
             us_per_call=round(dev_us, 3), eager_us_per_call=eager_us,
             wall_ms_timed=round(wall_s * 1e3, 3), gbs=round(gbs, 1),
             frac_of_peak=round(gbs / PEAK_GBS, 4))
    if not spread:
        return r
    # spread: the per-call average of SPREAD_REPLAYS further replays of the same graph
    per = []
    for _ in range(SPREAD_REPLAYS):
        ev0.record()
        g.replay()
        ev1.record()
        torch.cuda.synchronize()
        per.append(ev0.elapsed_time(ev1) * 1e3 / steps)
    per.sort()
    pick = lambda q: round(per[int(round(q * (len(per) - 1)))], 3)
    # hot: the same calls on one buffer set, so inputs that fit stay in the last-level cache
    gh = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gh):
        for _ in range(steps):
            w.call(0)
    gh.replay()
    torch.cuda.synchronize()
    ev0.record()
    gh.replay()
    ev1.record()
    torch.cuda.synchronize()
    hot_us = ev0.elapsed_time(ev1) * 1e3 / steps
    del g, gh
    r["spread_us"] = {"replays": SPREAD_REPLAYS, "p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}
    r["hot_us_per_call"] = round(hot_us, 3)
    return r


def cpu_baseline(k: int, scalars: dict, budget_s: float = 10.0) -> dict:
    """The oracle as it stands, single process, on a bounded sample of the
    same workload: whole calls for small workloads, a fixed slice of rows
    (tokens) for large ones, repeated until about budget_s of CPU time."""
    import oracle as O
    import workloads as W
    inp = W.make_config(k)
    if isinstance(inp, W.QKInputs):
        rows = min(inp.tokens, 64)
        sub = W.QKInputs(**{**inp.__dict__, "tokens": rows, "qkv": inp.qkv[:rows],
                            "positions": inp.positions[:rows]})
        args = (W.bits(sub.qkv), W.bits(sub.gamma_q), W.bits(sub.gamma_k), sub.positions.numpy(),
                sub.cos_sin, sub.scale, sub.eps, sub.nq, sub.nk, sub.nv, sub.head_dim, sub.dtype)
        fn = lambda: O.qk_norm_rope_fp8(*args)  # noqa: E731
        nbytes = algorithmic_bytes(sub)
        sample = f"{rows} of {inp.tokens} tokens per pass"
    else:
        rows = min(inp.tokens, max(1, (64 * 8192) // inp.hidden))
        xb, rb, gb = W.bits(inp.x)[:rows], W.bits(inp.residual)[:rows], W.bits(inp.gamma)
        if inp.op == "fp8":
            fn = lambda: O.add_rmsnorm_quant_fp8(xb, rb, gb, inp.dtype, inp.scale, inp.eps,  # noqa
                                                 inp.norm_out)
        elif inp.op == "gated":
            G = scalars[str(k)]["global_scale"]
            fn = lambda: O.gated_rmsnorm_quant_nvfp4(xb, rb, gb, inp.dtype,  # noqa
                                                     inp.meta["group"], G, inp.eps)
        else:
            G = scalars[str(k)]["global_scale"]
            fn = lambda: O.add_rmsnorm_quant_nvfp4(xb, rb, gb, inp.dtype, G, inp.eps,  # noqa
                                                   inp.norm_out)
        sub = W.TailInputs(**{**inp.__dict__, "tokens": rows})
        nbytes = algorithmic_bytes(sub)
        sample = f"{rows} of {inp.tokens} rows per pass"
    passes, t0 = 0, time.perf_counter()
    while True:
        fn()
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": round(nbytes * passes / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": f"{sample}, {passes} passes in {el:.1f} s",
            "us_per_call_equiv": round(el / passes * (inp.tokens / rows) * 1e6, 1)}


def copy_calibration(steps: int, warmup: int, nbytes: int = 1 << 30) -> dict:
    """A plain 1 GiB device-to-device copy (HIP's copy kernel), read + write
    bytes over event time: the streaming rate this GPU reaches in practice."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        dst.copy_(src)
    ev1.record()
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / steps
    return {"copy_bytes": nbytes, "us_per_copy": round(us, 2),
            "gbs_read_plus_write": round(2 * nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / (us * 1e-6) / 1e9 / PEAK_GBS, 4)}


def load_traffic(k: int, bytes_per_call: int):
    """HBM bytes per call measured by rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE), if they were taken on the current kernel sources."""
    try:
        with open(TRAFFIC) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(str(k))
    if not e or t.get("source_hash") != source_hash():
        return None
    return e.get("bytes_per_call")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--no-sweep", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip the fused vs separated (two-kernel) comparison and the KV-store timing")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip the eager timing (so a kernel trace holds graph launches only)")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the spread replays and the hot (same buffers) graph, so a kernel "
                    "trace holds only the timed graph's launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device-to-device copy of 1 GiB instead (practical "
                    "streaming ceiling; the same copy calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused tail is row-parallel (a split of the "
              "tokens needs no exchange), so one GPU's share is the whole measurement; "
              "rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import nvfp4_quantization_place_amd as A
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    A.lib()
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.steps, args.warmup)), flush=True)
        return
    with open(SCALARS) as fh:
        scalars = json.load(fh)

    todo = [args.workload] + ([] if args.no_sweep else
                              [k for k in (1, 2, 3, 4, 5, 6) if k != args.workload])
    results = {}
    for k in todo:
        w = Workload(k, scalars, args.steps)
        r = time_workload(w, args.steps, args.warmup, eager=not args.no_eager,
                          spread=not args.no_spread)
        r["traffic_bytes_per_call"] = load_traffic(k, w.bytes)
        results[k] = r
        extra = ""
        if "spread_us" in r:
            sp = r["spread_us"]
            extra = (f"; p10/p50/p90 {sp['p10']}/{sp['p50']}/{sp['p90']}; hot, same buffers "
                     f"{r['hot_us_per_call']}")
        print(f"# workload {k} {r['workload']}: {r['us_per_call']} us/call (graph{extra}), "
              f"{r['eager_us_per_call']} us/call (eager), {r['gbs']} GB/s", file=sys.stderr, flush=True)
        del w
        torch.cuda.empty_cache()

    ab = {}
    if not args.no_ab:
        for k in AB_WORKLOADS:
            w = Workload(k, scalars, args.steps, separated=True)
            r = time_workload(w, args.steps, args.warmup, eager=False)
            fused = results[k]["us_per_call"] if k in results else None
            e = {"workload": r["workload"], "separated_us": r["us_per_call"], "fused_us": fused,
                 "speedup": round(r["us_per_call"] / fused, 3) if fused else None}
            if k in PAGES_US:
                e["pages_separated_us"] = PAGES_SEPARATED_US[k]
                e["pages_fused_us"] = PAGES_US[k]
                e["pages_speedup"] = round(PAGES_SEPARATED_US[k] / PAGES_US[k], 3)
            ab[str(k)] = e
            print(f"# separated {k} {r['workload']}: {r['us_per_call']} us/call (graph)",
                  file=sys.stderr, flush=True)
            del w
            torch.cuda.empty_cache()

    kv = None
    if not args.no_ab:
        w = Workload(5, scalars, args.steps, kv_store=True)
        r = time_workload(w, args.steps, args.warmup, eager=False)
        kv = {"workload": r["workload"], "us_per_call": r["us_per_call"],
              "bytes_per_call": r["bytes_per_call"], "gbs": r["gbs"],
              "frac_of_peak": r["frac_of_peak"],
              "plain_us_per_call": results[5]["us_per_call"] if 5 in results else None}
        print(f"# kv store 5 {r['workload']}: {r['us_per_call']} us/call (graph), {r['gbs']} GB/s",
              file=sys.stderr, flush=True)
        del w
        torch.cuda.empty_cache()

    swz = {}
    if not args.no_ab:
        for k in (2, 4):
            w = Workload(k, scalars, args.steps, swizzled=True)
            r = time_workload(w, args.steps, args.warmup, eager=False)
            swz[str(k)] = {"workload": r["workload"], "us_per_call": r["us_per_call"],
                           "linear_us_per_call": results[k]["us_per_call"] if k in results else None}
            print(f"# swizzled scales {k} {r['workload']}: {r['us_per_call']} us/call (graph)",
                  file=sys.stderr, flush=True)
            del w
            torch.cuda.empty_cache()

    head = results[args.workload]
    inp_dtype = head["io_dtype"]
    traffic = head["traffic_bytes_per_call"]
    line = {
        "metric": METRIC,
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(head["gbs"] / (head["bytes_per_call"] / PAGES_US[args.workload] / 1e3), 2)
                        if args.workload in PAGES_US else None),
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "io_dtype": inp_dtype,
                   "us_per_call": head["us_per_call"], "eager_us_per_call": head["eager_us_per_call"],
                   "bytes_per_call": head["bytes_per_call"], "spread_us": head.get("spread_us"),
                   "hot_us_per_call": head.get("hot_us_per_call"), "timing": "HIP graph of steps calls, "
                   "HIP events on the launch stream; inputs rotate over >= 1 GiB of buffers; "
                   "spread_us over further replays of that graph; hot_us_per_call on one buffer set"},
        "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": head["frac_of_peak"],
                     "traffic": (round(traffic / (head["us_per_call"] * 1e-6) / 1e9, 1)
                                 if traffic else None)},
        "all_workloads": {str(k): v for k, v in results.items()},
    }
    if ab:
        line["fusion_ab"] = ab
    if kv:
        line["kv_store"] = kv
    if swz:
        line["sf_swizzled"] = swz
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(args.workload, scalars)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the fused add + RMSNorm + FP8/NVFP4 tail (and the Q/K norm +
RoPE + FP8 store) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 1..7] [--no-sweep] [--no-cpu]
                    [--no-ab] [--no-eager] [--no-spread] [--split-rows] [--copy-calibration]

A step is one call of the fused op on one batch of the workload's seeded
synthetic inputs, already resident in HBM. Every workload's inputs and outputs
rotate over enough buffer sets that they span at least 1 GiB, whatever K is:
the calls are captured into HIP graphs of exactly K calls each, one graph per
K consecutive sets, and the graphs are replayed in order, so when a graph is
timed its buffers were last touched a full rotation (>= 1 GiB of traffic)
earlier and come from HBM, not from the 256 MB last-level cache. A call so
small that this would take more than 64 graphs (workload 1, 14.6 KB) runs one
graph of K calls on K sets, after a 1 GiB read of other memory that evicts the
cache. The timed region is one replay of one graph (K calls) between HIP
events on the launch stream, bracketed by device synchronisation.

Prints ONE JSON line. `value` is achieved algorithmic HBM throughput in GB/s
on the headline workload (fp16 [64, 8192] add + RMSNorm + NVFP4, the shape the
pages measure: 0.039 ms on an RTX 5060 Ti, TensorRT-LLM issue #17900,
Performance result). Beside it:
  all_workloads  the same figures for every workload, each with its parity
                 against the oracle (every output byte of one fresh call,
                 digested and compared with tests/golden/workload_digests.json)
                 and a calibration: the no-arithmetic stream kernel
                 (anq_stream_rw) moving the same read and write bytes, timed
                 the same way (the practical ceiling of that byte mix)
  fusion_ab      the separated tail (add_rmsnorm, then the quantiser) against
                 the fused kernel, the pages' comparison (2.64x at [64, 8192])
  kv_store       the Q/K op with its uniform FP8 pool store
  sf_swizzled    NVFP4 with the 128x4-tiled block scales
  split_rows     the headline's bytes as shorter rows ([128, 4096] ... [1024,
                 512]): the most that splitting a row over several CUs can gain
  cpu_baseline   the oracle timed on this host, one process and one process
                 per core (rows split among them), for every workload, with
                 the core count and CPU model
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused add+RMSNorm+FP8/NVFP4 quant: µs/call and achieved HBM GB/s (% peak)"
PEAK_GBS = 8000.0                      # MI355X HBM3E
PAGES_US = {2: 39.0}                   # the pages' fused-tail latency for this exact workload
PAGES_SEPARATED_US = {2: 103.0}        # ... and their separated (two-kernel) latency
WORKLOADS = (1, 2, 3, 4, 5, 6, 7)
AB_WORKLOADS = (2, 3, 4)
ROTATE_BYTES = 1 << 30
MAX_GRAPHS = 64                        # past this, one graph and a cache flush instead (below)
FLUSH_BYTES = 1 << 30
SCALARS = os.path.join(ROOT, "tests", "golden", "workload_scalars.json")
DIGESTS = os.path.join(ROOT, "tests", "golden", "workload_digests.json")
TRAFFIC = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "nvfp4_quantization_place_amd", "csrc")
SPLIT_SHAPES = ((64, 8192), (128, 4096), (256, 2048), (512, 1024), (1024, 512))
CPU_BUDGET_S = 1.5                     # oracle time per workload and mode (single, all cores)
CPU_HEAD_BUDGET_S = 10.0               # the same for the workload the line reports
MAX_CPU_PROCS = 16                     # worker processes at most: a host's cores per GPU


# ---------------------------------------------------------------- byte counts

def rw_bytes(inp, kind: str = "fused", stored: int | None = None) -> tuple[int, int]:
    """(read, write) algorithmic bytes per call: what the method must move,
    gamma and scales counted once; with a KV store, each token's slot index is
    read and the pool row written for the `stored` tokens whose slot is in the
    pool (all tokens if not given).

    fused tail  reads x, residual (2 + 2 B/element), gamma (2H) and the scale;
                writes residual 2, codes (FP8 1 | NVFP4 0.5 + 1/16), norm 2 if asked
    gated       reads x, z; writes NVFP4 codes and scales
    separated   add_rmsnorm (reads 4, writes residual 2 + norm 2) plus the
                quantiser (reads norm 2, writes codes)
    Q/K         reads qkv (2 B/element), positions (8 B/token), the cos|sin row
                (4R B/token), gamma_q and gamma_k (2D each), the scale; writes
                codes (1 B/element: Q for every token, K and V for the stored
                ones), the mixed pool's rotated K part 2 B/element"""
    import workloads as W
    if isinstance(inp, W.QKInputs):
        D, R, T = inp.head_dim, inp.rotary_dim, inp.tokens
        C = (inp.nq + inp.nk + inp.nv) * D
        kv = kind in ("kv_store", "kv_mixed")
        read = T * C * 2 + T * (4 * R + 8) + 4 * D + 4 + (T * 8 if kv else 0)
        if not kv:
            return read, T * C
        st = T if stored is None else stored
        pool_row = (inp.nk + inp.nv) * D + (inp.nk * R if kind == "kv_mixed" else 0)
        return read, T * inp.nq * D + st * pool_row
    M, H = inp.tokens, inp.hidden
    n = M * H
    codes = n if inp.op == "fp8" else n // 2 + n // 16
    if inp.op == "gated":
        return 4 * n + 2 * H + 4, codes
    if kind == "separated":
        return 4 * n + 2 * H + 2 * n + 4, 4 * n + codes
    return 4 * n + 2 * H + 4, 2 * n + codes + (2 * n if inp.norm_out else 0)


def _code_text(name: str, text: str) -> str:
    """A source file's text without comments and with runs of whitespace
    collapsed, so that editing a comment keeps measured counters valid."""
    if name.endswith((".hip", ".h", ".cpp", ".c")):
        text = re.sub(r"//[^\n]*|/\*.*?\*/", " ", text, flags=re.S)
    elif name.endswith(".py"):
        text = re.sub(r"#[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash() -> str:
    """Hash of the kernel sources (comments and layout ignored): the counter
    bytes of profiles/hbm_traffic.json apply only while it matches."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        path = os.path.join(CSRC, f)
        if not os.path.isfile(path):
            continue
        with open(path, encoding="utf-8") as fh:
            h.update(f.encode() + _code_text(f, fh.read()).encode())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------- CPU baseline

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rows(task):
    """`reps` oracle passes over a slice of a workload (runs in a worker or
    here). task = (op, arrays, params, reps); returns the rows done."""
    op, a, prm, reps = task
    for _ in range(reps):
        _oracle_pass(op, a, prm)
    return reps * len(a["x"] if "x" in a else a["qkv"])


def _oracle_pass(op, a, prm):
    import oracle as O
    if op == "fp8":
        O.add_rmsnorm_quant_fp8(a["x"], a["r"], a["g"], prm["dtype"], prm["scale"], prm["eps"],
                                prm["norm_out"])
    elif op == "nvfp4":
        O.add_rmsnorm_quant_nvfp4(a["x"], a["r"], a["g"], prm["dtype"], prm["scale"], prm["eps"],
                                  prm["norm_out"])
    elif op == "gated":
        O.gated_rmsnorm_quant_nvfp4(a["x"], a["r"], a["g"], prm["dtype"], prm["group"],
                                    prm["scale"], prm["eps"])
    elif op == "qk":
        O.qk_norm_rope_fp8(a["qkv"], a["gq"], a["gk"], a["pos"], a["cs"], prm["scale"], prm["eps"],
                           prm["nq"], prm["nk"], prm["nv"], prm["D"], prm["dtype"],
                           rotary_dim=prm["R"])
    elif op == "qk_mixed":
        O.qk_norm_rope_kv_store_mixed(a["qkv"], a["gq"], a["gk"], a["pos"], a["cs"], prm["scale"],
                                      prm["eps"], prm["nq"], prm["nk"], prm["nv"], prm["D"],
                                      prm["R"], prm["dtype"], a["slots"], a["pool"])
    else:
        raise ValueError(op)


def _oracle_task(k: int, inp, scalars: dict, r0: int, r1: int, reps: int = 1):
    """The oracle call of rows [r0, r1) of workload k (inputs as raw bits)."""
    import numpy as np

    import workloads as W
    if isinstance(inp, W.QKInputs):
        prm = dict(scale=inp.scale, eps=inp.eps, nq=inp.nq, nk=inp.nk, nv=inp.nv, D=inp.head_dim,
                   R=inp.rotary_dim, dtype=inp.dtype)
        a = dict(qkv=W.bits(inp.qkv)[r0:r1], gq=W.bits(inp.gamma_q), gk=W.bits(inp.gamma_k),
                 pos=inp.positions.numpy()[r0:r1], cs=inp.cos_sin)
        if inp.name.startswith("qk_norm_rope_kv_mixed"):
            import oracle as O
            n = r1 - r0
            a["slots"] = np.arange(n, dtype=np.int64)
            a["pool"] = np.zeros((n, O.mixed_kv_row_bytes(inp.nk, inp.nv, inp.head_dim,
                                                           inp.rotary_dim)), np.uint8)
            return ("qk_mixed", a, prm, reps)
        return ("qk", a, prm, reps)
    scale = inp.scale if inp.op == "fp8" else scalars[str(k)]["global_scale"]
    prm = dict(dtype=inp.dtype, scale=scale, eps=inp.eps, norm_out=inp.norm_out,
               group=inp.meta.get("group"))
    a = dict(x=W.bits(inp.x)[r0:r1], r=W.bits(inp.residual)[r0:r1], g=W.bits(inp.gamma))
    return (inp.op, a, prm, reps)


def cpu_baseline(workloads: list, scalars: dict, budget_s: float, head_budget_s: float) -> dict:
    """The oracle as it stands, on bounded samples of each workload: one
    process, then one process per core with the rows split among them (rows
    are independent). Runs before any GPU work; the worker pool is closed
    when it returns. GB/s = the sample's algorithmic bytes / wall time. The
    first workload (the one the line reports) gets head_budget_s per mode,
    the others budget_s."""
    import multiprocessing as mp

    import workloads as W
    cores = min(len(os.sched_getaffinity(0)), MAX_CPU_PROCS)
    out = {"cores": cores, "cpu_model": _cpu_model(), "kind": "oracle", "per_workload": {}}
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        pool.map(_noop, range(cores))           # start every worker before timing
        for wi, k in enumerate(workloads):
            budget = head_budget_s if wi == 0 else budget_s
            inp = W.make_config(k)
            rows_total = inp.tokens
            # rows for about `budget` seconds in one process: a timed probe, then scale
            probe = max(1, min(rows_total, 8))
            t0 = time.perf_counter()
            _oracle_rows(_oracle_task(k, inp, scalars, 0, probe))
            per_row = max((time.perf_counter() - t0) / probe, 1e-7)
            rows = max(1, min(rows_total, int(budget / per_row)))
            task = _oracle_task(k, inp, scalars, 0, rows)
            reps, t0 = 0, time.perf_counter()
            while True:
                _oracle_rows(task)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
            single_rows_s = rows * reps / el
            # all cores: the rows split among the processes (up to all of the
            # workload's), each process repeating its share until it has done
            # about the single run's rows
            n_all = min(rows_total, rows * cores)
            bounds = [(i * n_all // cores, (i + 1) * n_all // cores) for i in range(cores)]
            tasks = [_oracle_task(k, inp, scalars, a, b, max(1, round(rows * reps / (b - a))))
                     for a, b in bounds if b > a]
            t0 = time.perf_counter()
            done = sum(pool.map(_oracle_rows, tasks))
            el_all = time.perf_counter() - t0
            all_rows_s = done / el_all
            # the sample stores every row of the mixed workload's pool
            rd, wr = rw_bytes(inp, "kv_mixed" if inp.name.startswith("qk_norm_rope_kv_mixed")
                              else "fused")
            per_row_bytes = (rd + wr) / rows_total
            out["per_workload"][str(k)] = {
                "workload": inp.name,
                "single": {"rows_per_s": round(single_rows_s, 1),
                           "gbs": round(single_rows_s * per_row_bytes / 1e9, 4),
                           "us_per_call_equiv": round(rows_total / single_rows_s * 1e6, 1),
                           "sample": f"{rows} of {rows_total} rows x {reps} passes in {el:.2f} s"},
                "all_cores": {"rows_per_s": round(all_rows_s, 1),
                              "gbs": round(all_rows_s * per_row_bytes / 1e9, 4),
                              "us_per_call_equiv": round(rows_total / all_rows_s * 1e6, 1),
                              "sample": f"{n_all} of {rows_total} rows split over {len(tasks)} "
                                        f"processes, {done} rows done in {el_all:.2f} s"},
            }
            print(f"# cpu oracle {k} {inp.name}: {single_rows_s:.0f} rows/s one process, "
                  f"{all_rows_s:.0f} rows/s on {cores}", file=sys.stderr, flush=True)
    return out


def _noop(_):
    return 0


# ---------------------------------------------------------------- GPU timing

def rotating_sets(bytes_per_call: int, steps: int) -> int:
    """Buffer sets for >= 1 GiB of rotation (at least 2); past one graph's
    worth, a multiple of the calls per graph, so the graphs partition the sets
    and every set is touched once per rotation. A call so small that this
    would take more than MAX_GRAPHS graphs gets `steps` sets (one graph) and a
    cache flush before each timed replay instead: thousands of graph
    executables of such calls measured many times slower per call than the
    one-graph, flushed timing (workload 1: 27 against 3.2 us)."""
    s = max(2, math.ceil(ROTATE_BYTES / bytes_per_call))
    if s <= steps:
        return s
    if math.ceil(s / steps) > MAX_GRAPHS:
        return max(2, steps)
    return math.ceil(s / steps) * steps


class Workload:
    """Device-resident inputs and outputs of one workload in S rotating sets
    (rotating_sets), each tensor role one allocation of S slices."""

    def __init__(self, k: int, scalars: dict, steps: int, kind: str = "fused", inp=None):
        import torch

        import workloads as W
        import nvfp4_quantization_place_amd as A
        self.inp = inp if inp is not None else W.make_config(k)
        self.name = self.inp.name + ("" if kind == "fused" else "_" + kind)
        if self.inp.name.startswith("qk_norm_rope_kv_mixed") and kind == "fused":
            kind = "kv_mixed"  # this workload is the op with its mixed pool store
        self.k, self.kind = k, kind
        slots = None
        if kind in ("kv_store", "kv_mixed"):
            T = self.inp.tokens
            slots = W.kv_slots(k, T, T * W.KV_POOL_FACTOR[0] // W.KV_POOL_FACTOR[1])
        rd, wr = rw_bytes(self.inp, kind, None if slots is None else int((slots >= 0).sum()))
        self.read_bytes, self.write_bytes = rd, wr
        self.bytes = rd + wr
        self.sets = rotating_sets(self.bytes, steps)
        dev, S, inp = "cuda", self.sets, self.inp

        def rep(t):  # S copies of a CPU tensor, as one allocation
            return t.to(dev).unsqueeze(0).repeat(S, *([1] * t.dim()))

        def u8(*shape):
            return torch.empty(S, *shape, dtype=torch.uint8, device=dev)

        self.dtype = inp.dtype
        if isinstance(inp, W.QKInputs):
            D, R = inp.head_dim, inp.rotary_dim
            self.qkv = rep(inp.qkv)
            self.gq, self.gk = inp.gamma_q.to(dev), inp.gamma_k.to(dev)
            self.pos = inp.positions.to(dev)
            self.cs = torch.from_numpy(inp.cos_sin).to(dev)
            self.scale = torch.tensor([inp.scale], dtype=torch.float32, device=dev)
            T = inp.tokens
            if kind in ("kv_store", "kv_mixed"):
                nslots = T * W.KV_POOL_FACTOR[0] // W.KV_POOL_FACTOR[1]
                self.slots = torch.from_numpy(slots).to(dev)
                width = (A.mixed_kv_row_bytes(inp.nk, inp.nv, D, R) if kind == "kv_mixed"
                         else (inp.nk + inp.nv) * D)
                self.pool = torch.zeros(S, nslots, width, dtype=torch.uint8, device=dev)
                self.out = u8(T, inp.nq * D)
            else:
                self.out = u8(*inp.qkv.shape)
            return
        self.x, self.res = rep(inp.x), rep(inp.residual)
        self.g = inp.gamma.to(dev)
        s = inp.scale if inp.op == "fp8" else scalars[str(k)]["global_scale"]
        self.scale = torch.tensor([s], dtype=torch.float32, device=dev)
        M, H = inp.tokens, inp.hidden
        self.q = u8(M, H if inp.op == "fp8" else H // 2)
        self.sf = None
        if inp.op in ("nvfp4", "gated"):
            self.sf = u8(*(A.nvfp4_swizzled_sf_shape(M, H) if kind == "swizzled" else (M, H // 16)))
        # the separated path always materialises the norm (the quantiser's input)
        self.norm = (torch.empty(S, M, H, dtype=self.x.dtype, device=dev)
                     if inp.norm_out or kind == "separated" else None)

    def call(self, i: int):
        """One call on buffer set i mod sets. The per-set tensor views and
        arguments are built once, so an eager call times the binding and the
        launch, not the slicing of the rotation buffers."""
        calls = self.__dict__.get("_calls")
        if calls is None:
            calls = self._calls = [self._make_call(j) for j in range(self.sets)]
        calls[i % self.sets]()

    def prepared(self):
        """The calls of every buffer set as prepared calls (the binding's
        checks done once), or None where a call is two library calls."""
        import nvfp4_quantization_place_amd as A
        if self.kind == "separated":
            return None
        out = []
        for j in range(self.sets):
            fn, args, kw = self._spec(j)
            out.append(A.prepare(fn, *args, **kw))
        return out

    def _make_call(self, j: int):
        import functools

        import nvfp4_quantization_place_amd as A
        if self.kind == "separated":
            inp = self.inp
            x, res, q = self.x[j], self.res[j], self.q[j]
            norm = self.norm[j]
            sf = self.sf[j] if self.sf is not None else None

            def sep():
                n = A.add_rmsnorm(x, res, self.g, inp.eps, norm=norm)
                if inp.op == "fp8":
                    A.quant_fp8(n, self.scale, q=q)
                else:
                    A.quant_nvfp4(n, self.scale, q=q, sf=sf)
            return sep
        fn, args, kw = self._spec(j)
        return functools.partial(fn, *args, **kw)

    def _spec(self, j: int):
        """(op, args, kwargs) of the one binding call on buffer set j."""
        import nvfp4_quantization_place_amd as A
        inp = self.inp
        if hasattr(self, "qkv"):
            args = (self.qkv[j], self.gq, self.gk, self.pos, self.cs, self.scale, inp.eps, inp.nq,
                    inp.nk, inp.nv, inp.head_dim)
            if self.kind == "kv_mixed":
                return (A.qk_norm_rope_kv_store_mixed, args + (inp.rotary_dim, self.slots,
                                                               self.pool[j]),
                        dict(q_out=self.out[j]))
            if self.kind == "kv_store":
                return (A.qk_norm_rope_fp8_kv_store, args + (self.slots, self.pool[j]),
                        dict(q_out=self.out[j], rotary_dim=inp.rotary_dim))
            return A.qk_norm_rope_fp8, args, dict(rotary_dim=inp.rotary_dim, out=self.out[j])
        x, res = self.x[j], self.res[j]
        norm = self.norm[j] if self.norm is not None else None
        q = self.q[j]
        sf = self.sf[j] if self.sf is not None else None
        base = (x, res, self.g, self.scale, inp.eps)
        if self.kind == "swizzled":
            return A.add_rmsnorm_quant_nvfp4_swizzled, base, dict(q=q, sf=sf, norm=norm)
        if inp.op == "gated":
            return A.gated_rmsnorm_quant_nvfp4, base, dict(group=inp.meta["group"], q=q, sf=sf)
        if inp.op == "fp8":
            return A.add_rmsnorm_quant_fp8, base, dict(q=q, norm=norm)
        return A.add_rmsnorm_quant_nvfp4, base, dict(q=q, sf=sf, norm=norm)


class StreamCalib:
    """The calibration stream with a workload's read and write bytes, in the
    same rotation (anq_stream_rw: one pass, 16-byte accesses, non-temporal)."""

    def __init__(self, name: str, read_bytes: int, write_bytes: int, steps: int):
        import torch
        self.name = name + "_stream"
        self.read_bytes = read_bytes // 16 * 16
        self.write_bytes = max(16, write_bytes // 16 * 16)
        self.bytes = self.read_bytes + self.write_bytes
        self.sets = rotating_sets(self.bytes, steps)
        self.src = torch.zeros(self.sets, self.read_bytes, dtype=torch.uint8, device="cuda")
        self.dst = torch.empty(self.sets, self.write_bytes, dtype=torch.uint8, device="cuda")
        self.dtype = "u8"

    def call(self, i: int):
        import nvfp4_quantization_place_amd as A
        j = i % self.sets
        A.stream_rw(self.src[j], self.read_bytes, self.dst[j], self.write_bytes)


SPREAD_REPLAYS = 10
GRAPH_WARM_S = 0.025
# a spin kernel of this many GPU cycles (~0.1 ms) runs before each timed
# replay, so the host has submitted the graph by the time the start event is
# reached: the events then bracket the GPU's work on the K calls, not the
# host's submission of the graph
LEAD_CYCLES = 250_000


def time_workload(w, steps: int, warmup: int, eager: bool = True, spread: bool = True) -> dict:
    """Device time per call: one graph of `steps` calls on consecutive sets,
    timed with HIP events after every other graph (the rest of the rotation)
    has replayed since its buffers were last touched."""
    import torch
    for i in range(warmup):
        w.call(i)
    torch.cuda.synchronize()
    eager_us = prepared_us = None
    if eager:  # host-launched calls, wall clock: through the binding, then prepared calls
        t0 = time.perf_counter()
        for i in range(steps):
            w.call(i)
        torch.cuda.synchronize()
        eager_us = round((time.perf_counter() - t0) / steps * 1e6, 3)
        prep = w.prepared() if hasattr(w, "prepared") else None
        if prep:
            for i in range(min(steps, 5)):
                prep[i % len(prep)]()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                prep[i % len(prep)]()
            torch.cuda.synchronize()
            prepared_us = round((time.perf_counter() - t0) / steps * 1e6, 3)
            del prep
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(2):
            w.call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    n_graphs = max(1, math.ceil(w.sets / steps))
    graphs = []
    for gi in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                w.call(gi * steps + i)
        graphs.append(g)
    cursor = [0]
    # small calls (rotation below 1 GiB): a read of FLUSH_BYTES of other memory
    # before each timed replay evicts the last-level cache without leaving
    # dirty lines to write back during the timed region
    flush = None
    if w.sets * w.bytes < ROTATE_BYTES:
        flush = torch.ones(FLUSH_BYTES // 8, dtype=torch.int64, device="cuda")

    def replay_next():
        g = graphs[cursor[0] % n_graphs]
        cursor[0] += 1
        g.replay()

    def rotate_rest():  # every graph but the next one, so the next one's buffers are cold
        for _ in range(n_graphs - 1):
            replay_next()

    # warm the graphs until the GPU has run them for >= GRAPH_WARM_S (at least
    # one full rotation), so the timed replay runs at settled clocks
    t_w = time.perf_counter()
    reps = 0
    while reps < max(2, n_graphs) or (spread and time.perf_counter() - t_w < GRAPH_WARM_S):
        replay_next()
        torch.cuda.synchronize()
        reps += 1
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed() -> float:
        rotate_rest()
        if flush is not None:
            assert int(flush.sum()) == flush.numel()
        torch.cuda.synchronize()
        torch.cuda._sleep(LEAD_CYCLES)
        ev0.record()
        replay_next()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / steps

    # the timed sequence once, discarded: the first replay after the warm-up
    # loop measured up to 12% slower than every later one (workload 2 with
    # hinted code stores: 4.44 against 3.93-4.04 us per call)
    timed()
    t0 = time.perf_counter()
    dev_us = timed()
    wall_s = time.perf_counter() - t0
    gbs = w.bytes / (dev_us * 1e-6) / 1e9
    r = dict(workload=w.name, io_dtype=w.dtype, bytes_per_call=w.bytes,
             read_bytes=w.read_bytes, write_bytes=w.write_bytes, rotating_sets=w.sets,
             rotating_bytes=w.sets * w.bytes, graphs=n_graphs, calls_per_graph=steps,
             flush_bytes=FLUSH_BYTES if flush is not None else 0,
             us_per_call=round(dev_us, 3), eager_us_per_call=eager_us,
             eager_prepared_us_per_call=prepared_us,
             wall_ms_timed=round(wall_s * 1e3, 3), gbs=round(gbs, 1),
             frac_of_peak=round(gbs / PEAK_GBS, 4))
    if not spread:
        del graphs, flush
        return r
    per = sorted(timed() for _ in range(SPREAD_REPLAYS))
    pick = lambda q: round(per[int(round(q * (len(per) - 1)))], 3)  # noqa: E731
    # hot: the same calls on one buffer set, so inputs that fit stay in the last-level cache
    gh = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gh):
        for _ in range(steps):
            w.call(0)
    gh.replay()
    torch.cuda.synchronize()
    torch.cuda._sleep(LEAD_CYCLES)
    ev0.record()
    gh.replay()
    ev1.record()
    torch.cuda.synchronize()
    hot_us = ev0.elapsed_time(ev1) * 1e3 / steps
    del graphs, gh, flush
    r["spread_us"] = {"replays": SPREAD_REPLAYS, "p10": pick(0.1), "p50": pick(0.5),
                      "p90": pick(0.9)}
    r["hot_us_per_call"] = round(hot_us, 3)
    return r


# ---------------------------------------------------------------- parity

def parity(k: int, kind: str, digests: dict) -> dict:
    """Every output byte of one call on fresh inputs against the oracle's
    digests (whole tensor and runs of rows)."""
    import workloads as W
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from runners import gpu_full_workload
    entry = digests[str(k)]
    got = gpu_full_workload(k, kind)
    bad, n = 0, 0
    for name, a in got.items():
        want = entry["outputs"][name]
        d = W.row_chunk_digests(a, want["chunk_rows"])
        n += 1
        if d["sha256"] != want["sha256"]:
            bad += sum(x != y for x, y in zip(d["chunks"], want["chunks"])) or 1
    return {"rows": entry["rows"], "outputs": sorted(got), "bit_exact": bad == 0,
            "mismatched_chunks": bad,
            **({"norm_out_max_abs_err": 0.0, "codes_identical_frac": 1.0} if bad == 0 else {})}


def load_traffic(k: int):
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


def copy_calibration(steps: int, warmup: int, nbytes: int = 1 << 30) -> dict:
    """A plain 1 GiB device-to-device copy (HIP's copy kernel), read + write
    bytes over event time; the same copy calibrates the HBM byte counters."""
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


def _log(r: dict, what: str):
    extra = ""
    if "spread_us" in r:
        sp = r["spread_us"]
        extra = (f"; p10/p50/p90 {sp['p10']}/{sp['p50']}/{sp['p90']}; hot, same buffers "
                 f"{r['hot_us_per_call']}")
    print(f"# {what} {r['workload']}: {r['us_per_call']} us/call (graph{extra}), "
          f"{r['gbs']} GB/s, {r['rotating_sets']} sets in {r['graphs']} graphs",
          file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=list(WORKLOADS))
    ap.add_argument("--no-sweep", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-ab", action="store_true",
                    help="skip the separated, KV-store, swizzled and split-row timings")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip the eager timing (so a kernel trace holds graph launches only)")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the spread replays and the hot (same buffers) graph")
    ap.add_argument("--no-parity", action="store_true", help="skip the per-workload parity check")
    ap.add_argument("--no-calib", action="store_true", help="skip the same-mix stream calibration")
    ap.add_argument("--split-rows", action="store_true",
                    help="time only the headline's bytes as shorter rows (split-row bound)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device-to-device copy of 1 GiB instead")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused tail is row-parallel (a split of the "
              "tokens needs no exchange), so one GPU's share is the whole measurement; "
              "rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    with open(SCALARS) as fh:
        scalars = json.load(fh)
    todo = [args.workload] + ([] if args.no_sweep else [k for k in WORKLOADS if k != args.workload])

    # the oracle on the host cores first: its worker pool is closed before any GPU work
    cpu = None
    if not (args.no_cpu or args.copy_calibration or args.split_rows):
        cpu = cpu_baseline(todo, scalars, CPU_BUDGET_S, CPU_HEAD_BUDGET_S)

    import torch

    import nvfp4_quantization_place_amd as A
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    A.lib()
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.steps, args.warmup)), flush=True)
        return
    spread = not args.no_spread

    def split_rows() -> dict:
        res = {}
        for M, H in SPLIT_SHAPES:
            inp = W.make_tail(2, "nvfp4", "f16", M, H, scale=None, name=f"nvfp4_f16_{M}x{H}")
            w = Workload(2, scalars, args.steps, inp=inp)
            r = time_workload(w, args.steps, args.warmup, eager=False, spread=spread)
            _log(r, "split rows")
            res[f"{M}x{H}"] = {"us_per_call": r["us_per_call"], "gbs": r["gbs"],
                               "spread_us": r.get("spread_us")}
            del w
            torch.cuda.empty_cache()
        return res

    if args.split_rows:
        print(json.dumps({"split_rows": split_rows()}), flush=True)
        return
    with open(DIGESTS) as fh:
        digests = json.load(fh)

    results = {}
    for k in todo:
        w = Workload(k, scalars, args.steps)
        r = time_workload(w, args.steps, args.warmup, eager=not args.no_eager, spread=spread)
        r["traffic_bytes_per_call"] = load_traffic(k)
        _log(r, f"workload {k}")
        rd, wr = w.read_bytes, w.write_bytes
        name, kind = w.name, w.kind
        del w
        torch.cuda.empty_cache()
        if not args.no_calib:
            c = StreamCalib(name, rd, wr, args.steps)
            rc = time_workload(c, args.steps, args.warmup, eager=False, spread=False)
            r["calibration"] = {"kernel": "anq_stream_rw", "read_bytes": c.read_bytes,
                                "write_bytes": c.write_bytes, "us_per_call": rc["us_per_call"],
                                "gbs": rc["gbs"], "frac_of_peak": rc["frac_of_peak"],
                                "kernel_over_stream": round(r["us_per_call"] / rc["us_per_call"], 3)}
            print(f"#   same-mix stream: {rc['us_per_call']} us ({rc['gbs']} GB/s)",
                  file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
        if not args.no_parity:
            r["parity"] = parity(k, "kv_mixed" if kind == "kv_mixed" else "fused", digests)
        results[k] = r

    ab, kv, swz, split = {}, None, {}, None
    if not args.no_ab:
        for k in AB_WORKLOADS:
            w = Workload(k, scalars, args.steps, kind="separated")
            r = time_workload(w, args.steps, args.warmup, eager=False, spread=spread)
            _log(r, "separated")
            fused = results[k]["us_per_call"] if k in results else None
            e = {"workload": r["workload"], "separated_us": r["us_per_call"], "fused_us": fused,
                 "speedup": round(r["us_per_call"] / fused, 3) if fused else None}
            if not args.no_parity:
                e["parity"] = parity(k, "separated", digests)
            if k in PAGES_US:
                e["pages_separated_us"] = PAGES_SEPARATED_US[k]
                e["pages_fused_us"] = PAGES_US[k]
                e["pages_speedup"] = round(PAGES_SEPARATED_US[k] / PAGES_US[k], 3)
            ab[str(k)] = e
            del w
            torch.cuda.empty_cache()
        w = Workload(5, scalars, args.steps, kind="kv_store")
        r = time_workload(w, args.steps, args.warmup, eager=False, spread=spread)
        _log(r, "kv store")
        kv = {"workload": r["workload"], "us_per_call": r["us_per_call"],
              "bytes_per_call": r["bytes_per_call"], "gbs": r["gbs"],
              "frac_of_peak": r["frac_of_peak"],
              "plain_us_per_call": results[5]["us_per_call"] if 5 in results else None}
        if not args.no_parity:
            kv["parity"] = parity(5, "kv_store", digests)
        del w
        torch.cuda.empty_cache()
        for k in (2, 4):
            w = Workload(k, scalars, args.steps, kind="swizzled")
            r = time_workload(w, args.steps, args.warmup, eager=False, spread=spread)
            _log(r, "swizzled scales")
            swz[str(k)] = {"workload": r["workload"], "us_per_call": r["us_per_call"],
                           "linear_us_per_call": results[k]["us_per_call"] if k in results else None}
            if not args.no_parity:
                swz[str(k)]["parity"] = parity(k, "swizzled", digests)
            del w
            torch.cuda.empty_cache()
        split = split_rows()

    head = results[args.workload]
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
        "config": {"workload": head["workload"], "io_dtype": head["io_dtype"],
                   "us_per_call": head["us_per_call"], "eager_us_per_call": head["eager_us_per_call"],
                   "eager_prepared_us_per_call": head["eager_prepared_us_per_call"],
                   "bytes_per_call": head["bytes_per_call"], "spread_us": head.get("spread_us"),
                   "hot_us_per_call": head.get("hot_us_per_call"),
                   "rotating_sets": head["rotating_sets"], "rotating_bytes": head["rotating_bytes"],
                   "timing": f"HIP graphs of exactly {args.steps} calls each over "
                             f"{head['rotating_sets']} rotating buffer sets "
                             f"({head['rotating_bytes'] / 2 ** 30:.2f} GiB) in {head['graphs']} "
                             "graphs replayed in turn, so a timed graph's buffers were last "
                             "touched a full rotation earlier (calls too small for that: one "
                             "graph after a 1 GiB read that evicts the cache, flush_bytes); HIP "
                             "events on the launch stream around one replay; spread_us over "
                             "further replays; hot_us_per_call on one buffer set"},
        "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": head["frac_of_peak"],
                     "traffic": (round(traffic / (head["us_per_call"] * 1e-6) / 1e9, 1)
                                 if traffic else None)},
        "parity": {str(k): v["parity"]["bit_exact"] for k, v in results.items() if "parity" in v},
        "all_workloads": {str(k): v for k, v in results.items()},
    }
    if ab:
        line["fusion_ab"] = ab
    if kv:
        line["kv_store"] = kv
    if swz:
        line["sf_swizzled"] = swz
    if split:
        line["split_rows"] = split
    if cpu:
        h = cpu["per_workload"].get(str(args.workload))
        line["cpu_baseline"] = {
            "value": h["all_cores"]["gbs"], "unit": "GB/s", "cores": cpu["cores"],
            "kind": "oracle", "cpu_model": cpu["cpu_model"],
            "sample": h["all_cores"]["sample"],
            "single_process": h["single"],
            "per_workload": cpu["per_workload"],
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

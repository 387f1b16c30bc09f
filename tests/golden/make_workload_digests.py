"""Write tests/golden/workload_digests.json: SHA-256 digests of every output
the oracle computes for the six full-size workloads (and for the variants the
benchmark times on them: the separated two-kernel tail, the swizzled block
scales, the KV-cache store), whole and per run of rows.

The full outputs are hundreds of MB, too large to store; their digests let a
GPU test compare every byte of a full-size launch with the oracle, and a
mismatching chunk names the rows to recompute. Calls only the oracle and the
input generator (the NVFP4 global scales come from workload_scalars.json,
written by make_workload_scalars.py, which calls only the oracle too).

    python tests/golden/make_workload_digests.py [--procs N]

Row chunks are computed in worker processes (rows are independent); the
result does not depend on N.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "workload_digests.json")
SCALARS = os.path.join(HERE, "workload_scalars.json")

KV_SENTINEL = 0xA5          # initial byte of every KV-pool row
SEPARATED = (2, 3, 4)       # workloads the separated (two-kernel) tail is timed on
SWIZZLED = (2, 4)           # workloads the swizzled block-scale layout is timed on

_W = {}


def _init(k: int):
    import workloads as W
    _W["k"] = k
    _W["inp"] = W.make_config(k)
    with open(SCALARS) as fh:
        _W["scalars"] = json.load(fh)


def _rows(r0: int, r1: int) -> dict:
    """Oracle outputs of rows [r0, r1) of workload _W["k"]."""
    import numpy as np

    import oracle as O
    import workloads as W
    k, inp = _W["k"], _W["inp"]
    if isinstance(inp, W.QKInputs):
        out = O.qk_norm_rope_fp8(W.bits(inp.qkv)[r0:r1], W.bits(inp.gamma_q), W.bits(inp.gamma_k),
                                 inp.positions.numpy()[r0:r1], inp.cos_sin, inp.scale, inp.eps,
                                 inp.nq, inp.nk, inp.nv, inp.head_dim, inp.dtype,
                                 rotary_dim=inp.rotary_dim)["out"]
        return {"out": out}
    xb, rb, gb = W.bits(inp.x)[r0:r1], W.bits(inp.residual)[r0:r1], W.bits(inp.gamma)
    if inp.op == "gated":
        G = _W["scalars"][str(k)]["global_scale"]
        r = O.gated_rmsnorm_quant_nvfp4(xb, rb, gb, inp.dtype, inp.meta["group"], G, inp.eps)
        return {"q": r["q"], "sf": r["sf"]}
    if inp.op == "fp8":
        r = O.add_rmsnorm_quant_fp8(xb, rb, gb, inp.dtype, inp.scale, inp.eps, norm_out=True)
        out = {"residual": r["residual"], "q": r["q"]}
    else:
        G = _W["scalars"][str(k)]["global_scale"]
        r = O.add_rmsnorm_quant_nvfp4(xb, rb, gb, inp.dtype, G, inp.eps, norm_out=True)
        out = {"residual": r["residual"], "q": r["q"], "sf": r["sf"]}
    if inp.norm_out:
        out["norm_out"] = r["norm_out"]
    if k in SEPARATED:
        # the separated tail quantises the norm tensor its first kernel writes in T
        nt = O.t_decode(r["norm_out"], inp.dtype)
        if inp.op == "fp8":
            out["q_separated"] = O.quant_fp8(nt, inp.scale)
        else:
            out["q_separated"], out["sf_separated"] = O.quant_nvfp4(nt, G)
    return out


def _digests(arrays: dict) -> dict:
    import workloads as W
    return {name: W.row_chunk_digests(a, W.chunk_rows_for(a.shape[0]))
            for name, a in arrays.items()}


def workload(k: int, procs: int) -> dict:
    import numpy as np

    import oracle as O
    import workloads as W
    _init(k)
    inp = _W["inp"]
    rows = inp.tokens
    step = max(1, -(-rows // (4 * procs)))
    spans = [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)]
    if procs > 1:
        ctx = mp.get_context("spawn")
        with ctx.Pool(procs, initializer=_init, initargs=(k,)) as pool:
            parts = pool.starmap(_rows, spans)
    else:
        parts = [_rows(r0, r1) for r0, r1 in spans]
    full = {name: np.concatenate([p[name] for p in parts]) for name in parts[0]}
    e = {"name": inp.name, "rows": rows}
    if isinstance(inp, W.QKInputs):
        D, R = inp.head_dim, inp.rotary_dim
        num_slots = rows * W.KV_POOL_FACTOR[0] // W.KV_POOL_FACTOR[1]
        slots = W.kv_slots(k, rows, num_slots)
        args = (W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
                inp.cos_sin, inp.scale, inp.eps, inp.nq, inp.nk, inp.nv, D)
        if inp.name.startswith("qk_norm_rope_kv_mixed"):   # the mixed pool
            pool0 = np.full((num_slots, O.mixed_kv_row_bytes(inp.nk, inp.nv, D, R)), KV_SENTINEL,
                            np.uint8)
            st = O.qk_norm_rope_kv_store_mixed(*args, R, inp.dtype, slots, pool0)
            prefix = "kv_mixed"
        else:                                               # the uniform FP8 pool
            pool0 = np.full((num_slots, (inp.nk + inp.nv) * D), KV_SENTINEL, np.uint8)
            st = O.qk_norm_rope_fp8_kv_store(*args, inp.dtype, slots, pool0, rotary_dim=R)
            prefix = "kv_store"
        assert np.array_equal(st["q"], full["out"][:, :inp.nq * D])
        full[prefix + "_q"] = st["q"]
        full[prefix + "_pool"] = st["kv"]
        e["kv_store"] = {"num_slots": num_slots, "slots": "workloads.kv_slots(%d, %d, %d)"
                         % (k, rows, num_slots), "sentinel": KV_SENTINEL, "rotary_dim": R}
    if k in SWIZZLED:
        full["sf_swizzled"] = O.swizzle_block_scales(full["sf"])
    e["outputs"] = _digests(full)
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--procs", type=int, default=min(os.cpu_count() or 1, 16))
    args = ap.parse_args()
    import workloads as W
    res = {"_about": "Written by make_workload_digests.py from the oracle; do not edit by hand. "
                     "Each output: sha256 of its bytes, and sha256[:16] of each run of "
                     "chunk_rows rows."}
    for k in sorted(W.CONFIGS):
        t0 = time.time()
        res[str(k)] = workload(k, args.procs)
        print(f"workload {k}: {len(res[str(k)]['outputs'])} outputs, {time.time() - t0:.1f} s",
              flush=True)
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")


if __name__ == "__main__":
    main()

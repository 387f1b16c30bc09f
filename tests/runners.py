"""Run one workload through the HIP library (via the Python binding) and
through the CPU oracle, on the same seeded inputs, and hand back numpy arrays
of raw bits for the comparators."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import workloads as W


def _np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_global_scale(inp: W.TailInputs) -> np.float32:
    n = O.rmsnorm_f32(W.bits(inp.x), W.bits(inp.residual), W.bits(inp.gamma), inp.dtype, inp.eps)
    return O.nvfp4_global_scale(n)


def gpu_tail(inp: W.TailInputs, scale: float, dev="cuda", stream=None) -> dict:
    import nvfp4_quantization_place_amd as A
    x = inp.x.to(dev)
    res = inp.residual.to(dev)
    g = inp.gamma.to(dev)
    s = torch.tensor([scale], dtype=torch.float32, device=dev)
    if inp.op == "fp8":
        q, norm = A.add_rmsnorm_quant_fp8(x, res, g, s, inp.eps, norm_out=inp.norm_out, stream=stream)
        out = dict(q=q)
    else:
        q, sf, norm = A.add_rmsnorm_quant_nvfp4(x, res, g, s, inp.eps, norm_out=inp.norm_out,
                                                stream=stream)
        out = dict(q=q, sf=sf)
    torch.cuda.synchronize()
    out["residual"] = res
    if norm is not None:
        out["norm_out"] = norm
    return {k: _np(v) for k, v in out.items()}


def oracle_tail(inp: W.TailInputs, scale: float, rows=None) -> dict:
    sel = slice(None) if rows is None else rows
    xb = W.bits(inp.x)[sel]
    rb = W.bits(inp.residual)[sel]
    gb = W.bits(inp.gamma)
    if inp.op == "fp8":
        return O.add_rmsnorm_quant_fp8(xb, rb, gb, inp.dtype, scale, inp.eps, inp.norm_out)
    return O.add_rmsnorm_quant_nvfp4(xb, rb, gb, inp.dtype, scale, inp.eps, inp.norm_out)


def gpu_qk(inp: W.QKInputs, dev="cuda", stream=None) -> np.ndarray:
    import nvfp4_quantization_place_amd as A
    out = A.qk_norm_rope_fp8(inp.qkv.to(dev), inp.gamma_q.to(dev), inp.gamma_k.to(dev),
                             inp.positions.to(dev), torch.from_numpy(inp.cos_sin).to(dev),
                             torch.tensor([inp.scale], dtype=torch.float32, device=dev), inp.eps,
                             inp.nq, inp.nk, inp.nv, inp.head_dim, stream=stream)
    torch.cuda.synchronize()
    return _np(out)


def oracle_qk(inp: W.QKInputs, tokens=None) -> np.ndarray:
    sel = slice(None) if tokens is None else tokens
    return O.qk_norm_rope_fp8(W.bits(inp.qkv)[sel], W.bits(inp.gamma_q), W.bits(inp.gamma_k),
                              inp.positions.numpy()[sel], inp.cos_sin, inp.scale, inp.eps, inp.nq,
                              inp.nk, inp.nv, inp.head_dim, inp.dtype)["out"]


def gpu_full_workload(k: int, variant: str = "fused") -> dict:
    """Outputs of one full-size launch of workload k on fresh inputs, as 2-D
    numpy arrays named like the oracle digests in tests/golden/workload_digests.json.

    variant: "fused" (the workload's own op), "separated" (add_rmsnorm, then the
    standalone quantiser on its T norm output), "swizzled" (NVFP4 with the
    128x4-tiled block scales), "kv_store" (the Q/K op into a uniform FP8 pool)
    or "kv_mixed" (the Q/K op into the mixed FP8 / bf16 pool)."""
    import json
    import os

    import nvfp4_quantization_place_amd as A
    golden = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    with open(os.path.join(golden, "workload_scalars.json")) as fh:
        scalars = json.load(fh)
    inp = W.make_config(k)
    dev = "cuda"
    if isinstance(inp, W.QKInputs):
        args = (inp.qkv.to(dev), inp.gamma_q.to(dev), inp.gamma_k.to(dev), inp.positions.to(dev),
                torch.from_numpy(inp.cos_sin).to(dev),
                torch.tensor([inp.scale], dtype=torch.float32, device=dev), inp.eps, inp.nq,
                inp.nk, inp.nv, inp.head_dim)
        R = inp.rotary_dim
        if variant == "fused":
            out = {"out": A.qk_norm_rope_fp8(*args, rotary_dim=R)}
        elif variant in ("kv_store", "kv_mixed"):
            with open(os.path.join(golden, "workload_digests.json")) as fh:
                kv = json.load(fh)[str(k)]["kv_store"]
            slots = torch.from_numpy(W.kv_slots(k, inp.tokens, kv["num_slots"])).to(dev)
            width = (A.mixed_kv_row_bytes(inp.nk, inp.nv, inp.head_dim, R) if variant == "kv_mixed"
                     else (inp.nk + inp.nv) * inp.head_dim)
            pool = torch.full((kv["num_slots"], width), kv["sentinel"], dtype=torch.uint8, device=dev)
            if variant == "kv_mixed":
                q = A.qk_norm_rope_kv_store_mixed(*args, R, slots, pool)
            else:
                q = A.qk_norm_rope_fp8_kv_store(*args, slots, pool, rotary_dim=R)
            out = {variant + "_q": q, variant + "_pool": pool}
        else:
            raise ValueError(variant)
        torch.cuda.synchronize()
        return {n: _np(v) for n, v in out.items()}
    x, res, g = inp.x.to(dev), inp.residual.to(dev), inp.gamma.to(dev)
    s = float(inp.scale) if inp.op == "fp8" else scalars[str(k)]["global_scale"]
    st = torch.tensor([s], dtype=torch.float32, device=dev)
    if inp.op == "gated":
        q, sf = A.gated_rmsnorm_quant_nvfp4(x, res, g, st, inp.eps, group=inp.meta["group"])
        out = {"q": q, "sf": sf}
    elif variant == "separated":
        norm = A.add_rmsnorm(x, res, g, inp.eps)
        if inp.op == "fp8":
            out = {"q_separated": A.quant_fp8(norm, st)}
        else:
            q, sf = A.quant_nvfp4(norm, st)
            out = {"q_separated": q, "sf_separated": sf}
        out["residual"] = res
        if inp.norm_out:
            out["norm_out"] = norm
    elif variant == "swizzled":
        q, sf, norm = A.add_rmsnorm_quant_nvfp4_swizzled(x, res, g, st, inp.eps,
                                                         norm_out=inp.norm_out)
        out = {"residual": res, "q": q, "sf_swizzled": sf}
        if norm is not None:
            out["norm_out"] = norm
    elif variant == "fused":
        if inp.op == "fp8":
            q, norm = A.add_rmsnorm_quant_fp8(x, res, g, st, inp.eps, norm_out=inp.norm_out)
            out = {"q": q}
        else:
            q, sf, norm = A.add_rmsnorm_quant_nvfp4(x, res, g, st, inp.eps, norm_out=inp.norm_out)
            out = {"q": q, "sf": sf}
        out["residual"] = res
        if norm is not None:
            out["norm_out"] = norm
    else:
        raise ValueError(variant)
    torch.cuda.synchronize()
    return {n: _np(v) for n, v in out.items()}

"""Seeded synthetic inputs for the fused residual-add + RMSNorm + FP8/NVFP4 tail
and for the Q/K per-head RMSNorm + RoPE + FP8 store.

This module only draws random numbers and lays them out as the inputs of the
five workload shapes. It holds none of the method's arithmetic: no residual
add, no norm, no quantisation. The same arrays are handed to the CPU oracle and
to the HIP library, so both sides always see bit-identical inputs.

Generator (stated once so any reader can re-derive every input):
  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): output i of stream k is mix(k + (i+1)*0x9E3779B97F4A7C15),
    mix(z) = z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27; z *= 0x94D049BB133111EB; z ^= z>>31.
    The stream key is (seed << 32) | tensor_id.
  * uniform(0,1): top 53 bits of an output times 2**-53.
  * normal: Box-Muller in float64 on consecutive uniform pairs (u1, u2),
    r = sqrt(-2 ln(1-u1)), z0 = r cos(2 pi u2), z1 = r sin(2 pi u2); both are used.
  * each float64 draw is converted to fp16 / bf16 by torch's CPU conversion.

Tensor ids: x = 0, residual = 1, gamma (gamma_q) = 2, outlier mask = 3, qkv = 4, gamma_k = 5,
KV-cache slot order = 6.

Workload shapes follow the fused NVFP4 tail of TensorRT-LLM issue #17900
("Performance result" and "Correctness" sections: FP16 [64, 8192]; hidden
128/7168 x seq 16/256/8192), the 64 x 1024-token prefill of TensorRT-LLM PR
#17288 ("Benchmark" section) and the norm + RoPE + uniform FP8 store of SGLang
PR #32975. Model dimensions the pages do not give (hidden 1024, 16/8/8 heads of
128) are fixed here.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field

import numpy as np
import torch

_GOLDEN = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

TID_X, TID_RES, TID_GAMMA, TID_MASK, TID_QKV, TID_GAMMA_K, TID_SLOTS = 0, 1, 2, 3, 4, 5, 6


def _s64(v: int) -> int:
    v &= (1 << 64) - 1
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64(seed: int, tid: int, n: int) -> np.ndarray:
    """Outputs 0..n-1 of the SplitMix64 stream keyed by (seed, tid), as uint64."""
    key = ((seed & 0xFFFFFFFF) << 32) | (tid & 0xFFFFFFFF)
    z = torch.arange(1, n + 1, dtype=torch.int64)
    z.mul_(_s64(_GOLDEN)).add_(_s64(key))
    z ^= _lsr(z, 30)
    z.mul_(_s64(_M1))
    z ^= _lsr(z, 27)
    z.mul_(_s64(_M2))
    z ^= _lsr(z, 31)
    return z.numpy().view(np.uint64)


def uniform(seed: int, tid: int, n: int) -> np.ndarray:
    z = torch.from_numpy(splitmix64(seed, tid, n).view(np.int64))
    return (_lsr(z, 11).to(torch.float64) * (2.0 ** -53)).numpy()


def normal(seed: int, tid: int, n: int) -> np.ndarray:
    m = (n + 1) // 2
    u = torch.from_numpy(uniform(seed, tid, 2 * m))
    u1, u2 = u[0::2], u[1::2]
    r = torch.sqrt(-2.0 * torch.log1p(-u1))
    th = (2.0 * math.pi) * u2
    out = torch.empty(2 * m, dtype=torch.float64)
    out[0::2] = r * torch.cos(th)
    out[1::2] = r * torch.sin(th)
    return out[:n].numpy()


_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_dtype(a64: np.ndarray, dtype: str) -> torch.Tensor:
    """float64 draws -> fp16/bf16 CPU tensor (torch's own conversion)."""
    return torch.from_numpy(np.ascontiguousarray(a64)).to(_TORCH_DT[dtype])


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of an fp16/bf16 CPU tensor (what the oracle reads)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def rope_table(max_pos: int, width: int, theta: float) -> np.ndarray:
    """cos | sin table [max_pos, width] float32 of a NeoX rotation over `width`
    elements (the head, or its rotated part): frequencies theta**(-2k/width)
    for k < width/2, evaluated in float64 and rounded once. It is an input of
    the Q/K kernel, identical on both sides."""
    half = width // 2
    k = np.arange(half, dtype=np.float64)
    inv = theta ** (-2.0 * k / width)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    tab = np.empty((max_pos, width), dtype=np.float64)
    tab[:, :half] = np.cos(ang)
    tab[:, half:] = np.sin(ang)
    return tab.astype(np.float32)


@dataclass
class TailInputs:
    """Inputs of one add + RMSNorm + quant call. Tensors are CPU, contiguous."""
    name: str
    op: str                 # "fp8", "nvfp4", or "gated" (residual then holds the gate z)
    dtype: str              # "f16" or "bf16"
    tokens: int
    hidden: int
    x: torch.Tensor
    residual: torch.Tensor
    gamma: torch.Tensor
    eps: float
    scale: float | None     # fp8 dequant scale s (q = E4M3(n / s)); None for nvfp4
    norm_out: bool
    meta: dict = field(default_factory=dict)


@dataclass
class QKInputs:
    name: str
    dtype: str
    tokens: int
    nq: int
    nk: int
    nv: int
    head_dim: int
    qkv: torch.Tensor
    gamma_q: torch.Tensor
    gamma_k: torch.Tensor
    positions: torch.Tensor  # int64 [tokens]
    cos_sin: np.ndarray      # float32 [max_pos, rotary_dim]
    eps: float
    scale: float
    rotary_dim: int = 0      # rotated width at the end of each Q/K head (0: the whole head)


# The workloads. "sizes" are the shapes the pages name or that are fixed here.
CONFIGS = {
    1: dict(name="fp8_f16_16x128", op="fp8", dtype="f16", tokens=16, hidden=128,
            x=("normal", 1.0), res=("normal", 1.0), gamma=("one_plus", 0.1),
            eps=1e-6, scale=0.02, norm_out=False, outliers=0.0),
    2: dict(name="nvfp4_f16_64x8192", op="nvfp4", dtype="f16", tokens=64, hidden=8192,
            x=("normal", 1.0), res=("normal", 1.0), gamma=("one_plus", 0.1),
            eps=1e-6, scale=None, norm_out=False, outliers=0.0),
    3: dict(name="fp8_bf16_65536x1024_normout", op="fp8", dtype="bf16", tokens=65536, hidden=1024,
            x=("normal", 1.0), res=("normal", 2.0), gamma=("uniform", 0.5, 1.5),
            eps=1e-6, scale=0.01, norm_out=True, outliers=0.0),
    4: dict(name="nvfp4_bf16_8192x7168_normout", op="nvfp4", dtype="bf16", tokens=8192, hidden=7168,
            x=("normal", 1.0), res=("normal", 1.0), gamma=("one_plus", 0.1),
            eps=1e-5, scale=None, norm_out=True, outliers=0.001),
    5: dict(name="qk_norm_rope_fp8_bf16_4096x32x128", op="qk", dtype="bf16", tokens=4096,
            nq=16, nk=8, nv=8, head_dim=128, theta=1e6, eps=1e-6, scale=0.05),
    # gated RMSNorm + NVFP4 at a Mamba-2 mixer's shape (inner width 8192, 8 groups);
    # the pages name the op but no workload for it
    6: dict(name="gated_nvfp4_bf16_8192x8192_g1024", op="gated", dtype="bf16", tokens=8192,
            hidden=8192, group=1024, x=("normal", 1.0), z=("normal", 2.0),
            gamma=("one_plus", 0.1), eps=1e-5),
    # the Q/K op storing K into the mixed pool (FP8 unrotated part, bf16 rotated part) with the
    # last 64 of 128 elements rotated; the pages give no shape, so workload 5's layout is kept
    7: dict(name="qk_norm_rope_kv_mixed_bf16_4096x32x128_rot64", op="qk_mixed", dtype="bf16",
            tokens=4096, nq=16, nk=8, nv=8, head_dim=128, rotary_dim=64, theta=1e6, eps=1e-6,
            scale=0.05),
}

KV_POOL_FACTOR = (5, 4)   # KV-store workloads: a pool of tokens * 5 / 4 slots, tokens shuffled in


def _draw(spec, seed: int, tid: int, n: int) -> np.ndarray:
    kind = spec[0]
    if kind == "normal":
        return spec[1] * normal(seed, tid, n)
    if kind == "one_plus":
        return 1.0 + spec[1] * normal(seed, tid, n)
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        return lo + (hi - lo) * uniform(seed, tid, n)
    raise ValueError(kind)


def make_tail(seed: int, op: str, dtype: str, tokens: int, hidden: int, *,
              x=("normal", 1.0), res=("normal", 1.0), gamma=("one_plus", 0.1),
              eps: float = 1e-6, scale: float | None = 0.02, norm_out: bool = False,
              outliers: float = 0.0, name: str = "custom") -> TailInputs:
    """Draw the inputs of one add + RMSNorm + quant call.

    outliers: each x entry is multiplied by 50 with this independent
    probability (mask drawn from its own stream)."""
    n = tokens * hidden
    xv = _draw(x, seed, TID_X, n)
    if outliers > 0.0:
        mask = uniform(seed, TID_MASK, n) < outliers
        xv = np.where(mask, 50.0 * xv, xv)
    rv = _draw(res, seed, TID_RES, n)
    gv = _draw(gamma, seed, TID_GAMMA, hidden)
    return TailInputs(
        name=name, op=op, dtype=dtype, tokens=tokens, hidden=hidden,
        x=to_dtype(xv, dtype).reshape(tokens, hidden),
        residual=to_dtype(rv, dtype).reshape(tokens, hidden),
        gamma=to_dtype(gv, dtype), eps=eps, scale=scale, norm_out=norm_out)


def make_qk(seed: int, dtype: str, tokens: int, nq: int, nk: int, nv: int, head_dim: int, *,
            theta: float = 1e6, eps: float = 1e-6, scale: float = 0.05,
            max_pos: int | None = None, positions: np.ndarray | None = None,
            rotary_dim: int | None = None, name: str = "custom") -> QKInputs:
    """Inputs of one Q/K call. rotary_dim R (default head_dim): the cos|sin
    table is [max_pos, R], with the NeoX frequencies of an R-wide rotation."""
    cols = (nq + nk + nv) * head_dim
    qkv = to_dtype(normal(seed, TID_QKV, tokens * cols), dtype).reshape(tokens, cols)
    gq = to_dtype(1.0 + 0.1 * normal(seed, TID_GAMMA, head_dim), dtype)
    gk = to_dtype(1.0 + 0.1 * normal(seed, TID_GAMMA_K, head_dim), dtype)
    if positions is None:
        positions = np.arange(tokens, dtype=np.int64)
    if max_pos is None:
        max_pos = max(int(positions.max()) + 1 if tokens else 1, 1)
    R = head_dim if rotary_dim is None else rotary_dim
    return QKInputs(name=name, dtype=dtype, tokens=tokens, nq=nq, nk=nk, nv=nv,
                    head_dim=head_dim, qkv=qkv, gamma_q=gq, gamma_k=gk,
                    positions=torch.from_numpy(np.ascontiguousarray(positions, dtype=np.int64)),
                    cos_sin=rope_table(max_pos, R, theta), eps=eps, scale=scale, rotary_dim=R)


def make_gated(seed: int, dtype: str, tokens: int, hidden: int, group: int, *,
               x=("normal", 1.0), z=("normal", 2.0), gamma=("one_plus", 0.1),
               eps: float = 1e-5, name: str = "custom") -> TailInputs:
    """Inputs of one gated RMSNorm + NVFP4 call: x, the gate z (in `residual`),
    gamma; meta["group"] is the normalisation group width."""
    n = tokens * hidden
    return TailInputs(
        name=name, op="gated", dtype=dtype, tokens=tokens, hidden=hidden,
        x=to_dtype(_draw(x, seed, TID_X, n), dtype).reshape(tokens, hidden),
        residual=to_dtype(_draw(z, seed, TID_RES, n), dtype).reshape(tokens, hidden),
        gamma=to_dtype(_draw(gamma, seed, TID_GAMMA, hidden), dtype), eps=eps, scale=None,
        norm_out=False, meta={"group": group})


def make_config(k: int):
    """Inputs of workload k (1..7), seed k. NVFP4 global scales are not drawn:
    they are derived from the normed tensor and stored beside the tests."""
    c = dict(CONFIGS[k])
    if c["op"] == "gated":
        return make_gated(k, c["dtype"], c["tokens"], c["hidden"], c["group"], x=c["x"], z=c["z"],
                          gamma=c["gamma"], eps=c["eps"], name=c["name"])
    if c["op"] in ("qk", "qk_mixed"):
        return make_qk(k, c["dtype"], c["tokens"], c["nq"], c["nk"], c["nv"], c["head_dim"],
                       theta=c["theta"], eps=c["eps"], scale=c["scale"],
                       rotary_dim=c.get("rotary_dim"), name=c["name"])
    return make_tail(k, c["op"], c["dtype"], c["tokens"], c["hidden"], x=c["x"], res=c["res"],
                     gamma=c["gamma"], eps=c["eps"], scale=c["scale"], norm_out=c["norm_out"],
                     outliers=c["outliers"], name=c["name"])


def kv_slots(seed: int, tokens: int, num_slots: int, pad_every: int = 16) -> np.ndarray:
    """Distinct KV-cache slots for `tokens` tokens in a pool of num_slots rows:
    the first `tokens` entries of the permutation that sorts num_slots uniform
    draws (stable sort), with every pad_every-th token (index % pad_every ==
    pad_every - 1) set to -1, a padding token that stores nothing."""
    order = np.argsort(uniform(seed, TID_SLOTS, num_slots), kind="stable")[:tokens]
    s = order.astype(np.int64)
    if pad_every > 0:
        s[pad_every - 1::pad_every] = -1
    return s


MEMBERS_PER_DIGEST = 64


def row_chunk_digests(a, chunk_rows: int) -> dict:
    """SHA-256 of a 2-D array's bytes (whole, 64 hex digits) and of each run of
    chunk_rows consecutive rows (16 hex digits each): a stored expected output
    is compared without storing it, and a mismatch names the rows it is in."""
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().contiguous()
        a = a.view(torch.uint8).numpy() if a.dtype != torch.uint8 else a.numpy()
    a = np.ascontiguousarray(a)
    if a.ndim != 2:
        raise ValueError("row_chunk_digests takes a 2-D array")
    raw = a.view(np.uint8).reshape(a.shape[0], -1)
    whole = hashlib.sha256()
    chunks = []
    for r0 in range(0, raw.shape[0], chunk_rows):
        b = raw[r0:r0 + chunk_rows].tobytes()
        whole.update(b)
        chunks.append(hashlib.sha256(b).hexdigest()[:16])
    return {"sha256": whole.hexdigest(), "chunk_rows": chunk_rows, "chunks": chunks}


def chunk_rows_for(rows: int) -> int:
    """Rows per digest chunk: about MEMBERS_PER_DIGEST chunks per tensor."""
    return max(1, -(-rows // MEMBERS_PER_DIGEST))


def checksum(t) -> str:
    if isinstance(t, torch.Tensor):
        b = t.contiguous().view(torch.uint8).numpy().tobytes()
    else:
        b = np.ascontiguousarray(t).tobytes()
    return hashlib.sha256(b).hexdigest()[:16]

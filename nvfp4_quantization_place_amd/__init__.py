"""Python binding of libaddnormq.so, the MI355X (gfx950) fused local tail:
residual add + RMSNorm + FP8 E4M3 / NVFP4 quantisation, and the Q/K per-head
RMSNorm + NeoX RoPE + FP8 store.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (include/addnormq.h). PyTorch provides device memory
and the current stream. There is no CPU path: without the built library, or
without a GPU, every call raises.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os

import torch  # loads the HIP runtime the library binds to

__all__ = ["add_rmsnorm_quant_fp8", "add_rmsnorm_quant_nvfp4", "qk_norm_rope_fp8",
           "qk_norm_rope_fp8_kv_store", "qk_norm_rope_kv_store_mixed", "mixed_kv_row_bytes",
           "add_rmsnorm_quant_nvfp4_swizzled",
           "gated_rmsnorm_quant_nvfp4", "silu_gate_f32",
           "quant_nvfp4_swizzled", "nvfp4_swizzled_sf_shape", "add_rmsnorm", "quant_fp8", "quant_nvfp4",
           "nvfp4_shape", "status_string", "selfcheck_arith", "stream_rw", "prepare", "Prepared",
           "lib", "AnqError",
           "LIB_PATH", "ANQ_F16", "ANQ_BF16", "STATUS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaddnormq.so")

ANQ_F16, ANQ_BF16 = 0, 1
STATUS = {0: "ANQ_OK", 1: "ANQ_ERR_NULL", 2: "ANQ_ERR_SHAPE", 3: "ANQ_ERR_DTYPE",
          4: "ANQ_ERR_ALIGN", 5: "ANQ_ERR_ALIAS", 6: "ANQ_ERR_UNSUPPORTED", 7: "ANQ_ERR_LAUNCH",
          8: "ANQ_ERR_VALUE", 9: "ANQ_ERR_CONFIG"}

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SIGS = {
    "add_rmsnorm_quant_fp8": [_P, _P, _P, _P, _F, _I64, _I64, ctypes.c_int, _P, _P, _P],
    "add_rmsnorm_quant_nvfp4": [_P, _P, _P, _P, _F, _I64, _I64, ctypes.c_int, _P, _P, _P, _P],
    "qk_norm_rope_fp8": [_P, _P, _P, _P, _P, _I64, _P, _F, _I64, _I32, _I32, _I32, _I32, _I32,
                         ctypes.c_int, _P, _P],
    "qk_norm_rope_fp8_kv_store": [_P, _P, _P, _P, _P, _I64, _P, _F, _I64, _I32, _I32, _I32, _I32,
                                  _I32, ctypes.c_int, _P, _I64, _P, _P, _P],
    "qk_norm_rope_kv_store_mixed": [_P, _P, _P, _P, _P, _I64, _P, _F, _I64, _I32, _I32, _I32,
                                    _I32, _I32, ctypes.c_int, _P, _I64, _P, _P, _P],
    "add_rmsnorm": [_P, _P, _P, _F, _I64, _I64, ctypes.c_int, _P, _P],
    "quant_fp8": [_P, _P, _I64, _I64, ctypes.c_int, _P, _P],
    "quant_nvfp4": [_P, _P, _I64, _I64, ctypes.c_int, _P, _P, _P],
    "add_rmsnorm_quant_nvfp4_swizzled": [_P, _P, _P, _P, _F, _I64, _I64, ctypes.c_int, _P, _P, _P,
                                         _P],
    "quant_nvfp4_swizzled": [_P, _P, _I64, _I64, ctypes.c_int, _P, _P, _P],
    "gated_rmsnorm_quant_nvfp4": [_P, _P, _P, _P, _F, _I64, _I64, _I64, ctypes.c_int, _P, _P, _P],
    "silu_gate_f32": [_P, _P, _I64, ctypes.c_int, _P, _P],
    "anq_selfcheck_arith": [_P, _P],
    "anq_nvfp4_swizzled_sf_shape": [_I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
    "anq_nvfp4_shape": [_I64, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)],
    "anq_status_string": [ctypes.c_int],
    "anq_stream_rw": [_P, _I64, _P, _I64, ctypes.c_int, _P],
}

_lib = None


class AnqError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn}: {STATUS.get(code, code)} ({status_string(code)})")


def load(path: str) -> ctypes.CDLL:
    """Open a build of the C ABI at `path` and declare its signatures."""
    L = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "anq_status_string" else ctypes.c_int
    return L


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m nvfp4_quantization_place_amd.build`")
        _lib = load(LIB_PATH)
    return _lib


def status_string(code: int) -> str:
    return lib().anq_status_string(code).decode()


@functools.lru_cache(maxsize=1024)
def nvfp4_shape(tokens: int, hidden: int) -> tuple[int, int]:
    """(q_cols, sf_cols) of the NVFP4 outputs, from the library's one shape
    helper (anq_nvfp4_shape): hidden/2 packed bytes and hidden/16 scales per
    row. Raises AnqError (ANQ_ERR_SHAPE) for a hidden size the ops reject."""
    q, s = _I64(), _I64()
    st = lib().anq_nvfp4_shape(tokens, hidden, ctypes.byref(q), ctypes.byref(s))
    if st:
        raise AnqError("anq_nvfp4_shape", st)
    return q.value, s.value


@functools.lru_cache(maxsize=1024)
def nvfp4_swizzled_sf_shape(tokens: int, hidden: int) -> tuple[int, int]:
    """(rows, cols) of the swizzled block-scale buffer: tokens padded to 128,
    hidden/16 padded to 4."""
    r, c = _I64(), _I64()
    st = lib().anq_nvfp4_swizzled_sf_shape(tokens, hidden, ctypes.byref(r), ctypes.byref(c))
    if st:
        raise AnqError("anq_nvfp4_swizzled_sf_shape", st)
    return r.value, c.value


_DT = {torch.float16: ANQ_F16, torch.bfloat16: ANQ_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def _check_gpu(*ts) -> int:
    """The one GPU (ordinal) all given tensors live on; they must be contiguous."""
    dev = -1
    for t in ts:
        if t is None:
            continue
        d = t.get_device()  # -1 for a CPU tensor
        if d < 0:
            raise ValueError("all tensors must live on the GPU (there is no CPU path)")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev < 0:
            dev = d
        elif d != dev:
            raise ValueError("all tensors must be on one device")
    return dev


# the current stream's raw handle without building a Stream object (torch's own
# launchers read it this way); the public API where the installed torch lacks it
_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: int, stream) -> int:
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is not None:
        return _RAW_STREAM(dev)
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


# While prepare() runs an op, the op's one library call is recorded here
# instead of made.
_record = None


def _call(name: str, *args) -> int:
    if _record is not None:
        _record.append((name, args))
        return 0
    return getattr(lib(), name)(*args)


class Prepared:
    """One op's library call with its arguments fixed: the checks of the
    Python binding ran once when it was prepared, and each call of this
    object makes the library call alone (which still validates its arguments
    on the host and enqueues the kernel). It holds its tensors, so their
    memory stays valid; the results land in the same output tensors
    (`outputs`, what the op returned) at every call, computed from the
    inputs' contents at that time. Without an explicit stream it enqueues on
    the current stream at each call. The tensors it holds must keep their
    storage (no resize_ or set_ on them)."""

    __slots__ = ("name", "outputs", "_fn", "_args", "_dev", "_current", "_keep")

    def __call__(self):
        args = self._args
        if self._current:
            args = args[:-1] + (_stream(self._dev, None),)
        st = self._fn(*args)
        if st:
            raise AnqError(self.name, st)
        return self.outputs


def prepare(op, *args, **kwargs) -> Prepared:
    """Run op(*args, **kwargs) through the binding's checks without launching
    it, and return the Prepared call that launches it. For loops that call
    one op on fixed buffers: each call then skips the per-call tensor checks
    of the binding. Output tensors the op would allocate are allocated here
    once; pass them in to reuse buffers of your own. Not thread-safe: prepare
    from one thread at a time."""
    global _record
    rec = []
    _record = rec
    try:
        outputs = op(*args, **kwargs)
    finally:
        _record = None
    if len(rec) != 1:
        raise ValueError(f"{getattr(op, '__name__', op)} does not make exactly one library call")
    name, cargs = rec[0]
    p = Prepared()
    p.name, p.outputs, p._fn, p._args = name, outputs, getattr(lib(), name), cargs
    tensors = [a for a in list(args) + list(kwargs.values()) if isinstance(a, torch.Tensor)]
    p._dev = tensors[0].get_device() if tensors else torch.cuda.current_device()
    try:  # the stream argument however it was passed
        given = inspect.signature(op).bind(*args, **kwargs).arguments.get("stream")
    except (TypeError, ValueError):
        given = kwargs.get("stream")
    p._current = given is None
    p._keep = (args, kwargs, outputs)
    return p


def _rows(x: torch.Tensor) -> tuple[int, int]:
    hidden = x.shape[-1]
    return (x.numel() // hidden if hidden else 0), hidden


def _scalar(s: torch.Tensor, name: str):
    if s.dtype != torch.float32 or s.numel() != 1:
        raise ValueError(f"{name} must be a one-element float32 device tensor")


def _need(t, numel: int, dtype, name: str):
    """t (if given) holds exactly numel elements of dtype. The library takes
    pointers and sizes and trusts the sizes, so every tensor is checked here,
    before any launch."""
    if t is not None and (t.dtype != dtype or t.numel() != numel):
        raise ValueError(f"{name} must hold {numel} elements of {dtype}, "
                         f"got {t.numel()} of {t.dtype}")


def _tail_shapes(x, residual, gamma, norm, other: str = "residual"):
    """x and `other` share dtype and shape; gamma [hidden] and norm like x."""
    tokens, hidden = _rows(x)
    if residual.dtype != x.dtype or gamma.dtype != x.dtype or residual.shape != x.shape:
        raise ValueError(f"x, {other} and gamma must share the dtype; x and {other} the shape")
    _need(gamma, hidden, x.dtype, "gamma")
    _need(norm, x.numel(), x.dtype, "norm")
    return tokens, hidden


def _nvfp4_outs(q, sf, lead: tuple, tokens: int, hidden: int, dev: int, swizzled: bool = False):
    """The NVFP4 outputs of a call: q [.., q_cols] and sf [.., sf_cols] uint8
    (or the padded swizzled sf buffer), the caller's after a size check or new
    ones, with every shape from the library's shape helpers."""
    qc, sc = nvfp4_shape(tokens, hidden)
    _need(q, tokens * qc, torch.uint8, "q")
    if q is None:
        q = torch.empty(*lead, qc, dtype=torch.uint8, device=dev)
    if swizzled:
        r, c = nvfp4_swizzled_sf_shape(tokens, hidden)
        _need(sf, r * c, torch.uint8, "sf (swizzled)")
        if sf is None:
            sf = torch.empty(r, c, dtype=torch.uint8, device=dev)
    else:
        _need(sf, tokens * sc, torch.uint8, "sf")
        if sf is None:
            sf = torch.empty(*lead, sc, dtype=torch.uint8, device=dev)
    return q, sf


def add_rmsnorm_quant_fp8(x, residual, gamma, scale, eps: float, norm_out: bool = False,
                          q=None, norm=None, stream=None):
    """residual += x (in place, rounded to T); n = RMSNorm(residual) * gamma;
    returns (q, norm_out): q uint8 E4M3 codes of n / scale, norm_out n in T or None."""
    dev = _check_gpu(x, residual, gamma, scale, q, norm)
    _scalar(scale, "scale")
    tokens, hidden = _tail_shapes(x, residual, gamma, norm)
    _need(q, x.numel(), torch.uint8, "q")
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    if norm_out and norm is None:
        norm = torch.empty_like(x)
    st = _call("add_rmsnorm_quant_fp8", _ptr(x), _ptr(residual), _ptr(gamma), _ptr(scale), eps,
                                     tokens, hidden, _dtype_code(x), _ptr(q), _ptr(norm),
                                     _stream(dev, stream))
    if st:
        raise AnqError("add_rmsnorm_quant_fp8", st)
    return q, norm


def add_rmsnorm_quant_nvfp4(x, residual, gamma, global_scale, eps: float, norm_out: bool = False,
                            q=None, sf=None, norm=None, stream=None):
    """residual += x; n = RMSNorm(residual) * gamma; returns (q, sf, norm_out):
    q [.., hidden/2] packed E2M1, sf [.., hidden/16] E4M3 block scales under
    the global scale G, norm_out n in T or None."""
    dev = _check_gpu(x, residual, gamma, global_scale, q, sf, norm)
    _scalar(global_scale, "global_scale")
    tokens, hidden = _tail_shapes(x, residual, gamma, norm)
    q, sf = _nvfp4_outs(q, sf, x.shape[:-1], tokens, hidden, dev)
    if norm_out and norm is None:
        norm = torch.empty_like(x)
    st = _call("add_rmsnorm_quant_nvfp4", _ptr(x), _ptr(residual), _ptr(gamma), _ptr(global_scale),
                                       eps, tokens, hidden, _dtype_code(x), _ptr(q), _ptr(sf),
                                       _ptr(norm), _stream(dev, stream))
    if st:
        raise AnqError("add_rmsnorm_quant_nvfp4", st)
    return q, sf, norm


def _qk_inputs(qkv, gamma_q, gamma_k, positions, cos_sin, nq, nk, head_dim, rotary_dim, tokens):
    """gamma_q / gamma_k [head_dim] in the dtype of qkv where there are Q / K
    heads, one position per token, and a [max_pos, rotary_dim] cos|sin table."""
    if nq > 0:
        _need(gamma_q, head_dim, qkv.dtype, "gamma_q")
    if nk > 0:
        _need(gamma_k, head_dim, qkv.dtype, "gamma_k")
    _need(positions, tokens, torch.int64, "positions")
    if positions.dtype != torch.int64 or cos_sin.dtype != torch.float32:
        raise ValueError("positions must be int64 and cos_sin float32")
    if cos_sin.dim() != 2 or cos_sin.shape[1] != rotary_dim:
        raise ValueError(f"cos_sin must be [max_pos, rotary_dim={rotary_dim}] float32")


def _qk_tokens(qkv, nq, nk, nv, head_dim) -> int:
    cols = (nq + nk + nv) * head_dim
    if qkv.shape[-1] != cols:
        raise ValueError(f"qkv last dim {qkv.shape[-1]} != (nq+nk+nv)*head_dim = {cols}")
    return qkv.numel() // cols if cols else 0


def qk_norm_rope_fp8(qkv, gamma_q, gamma_k, positions, cos_sin, scale, eps: float, nq: int,
                     nk: int, nv: int, head_dim: int, rotary_dim: int | None = None, out=None,
                     stream=None):
    """Q/K per-head RMSNorm + NeoX RoPE (of the last rotary_dim elements of
    each Q/K head; default all of it) + FP8 E4M3 of o / scale; V heads E4M3 of
    v / scale. cos_sin is [max_pos, rotary_dim]. Returns out (uint8, the shape of qkv)."""
    dev = _check_gpu(qkv, gamma_q, gamma_k, positions, cos_sin, scale, out)
    _scalar(scale, "scale")
    rot = head_dim if rotary_dim is None else rotary_dim
    tokens = _qk_tokens(qkv, nq, nk, nv, head_dim)
    _qk_inputs(qkv, gamma_q, gamma_k, positions, cos_sin, nq, nk, head_dim, rot, tokens)
    _need(out, qkv.numel(), torch.uint8, "out")
    if out is None:
        out = torch.empty(qkv.shape, dtype=torch.uint8, device=dev)
    st = _call("qk_norm_rope_fp8", _ptr(qkv), _ptr(gamma_q), _ptr(gamma_k), _ptr(positions),
                                _ptr(cos_sin), cos_sin.shape[0], _ptr(scale), eps, tokens, nq, nk,
                                nv, head_dim, rot, _dtype_code(qkv), _ptr(out),
                                _stream(dev, stream))
    if st:
        raise AnqError("qk_norm_rope_fp8", st)
    return out


def _qk_store(fn_name, kv_cols, qkv, gamma_q, gamma_k, positions, cos_sin, scale, eps, nq, nk,
              nv, head_dim, rot, slot_mapping, kv_cache, q_out, stream):
    dev = _check_gpu(qkv, gamma_q, gamma_k, positions, cos_sin, scale, slot_mapping, kv_cache,
                     q_out)
    _scalar(scale, "scale")
    if slot_mapping.dtype != torch.int64 or kv_cache.dtype != torch.uint8:
        raise ValueError("slot_mapping must be int64 and kv_cache uint8")
    tokens = _qk_tokens(qkv, nq, nk, nv, head_dim)
    if kv_cache.dim() < 1 or (kv_cols and kv_cache.numel() % kv_cols):
        raise ValueError(f"kv_cache must hold whole rows of {kv_cols} bytes")
    num_slots = kv_cache.numel() // kv_cols if kv_cols else 0
    if slot_mapping.numel() != tokens:
        raise ValueError("slot_mapping must hold one slot per token")
    _qk_inputs(qkv, gamma_q, gamma_k, positions, cos_sin, nq, nk, head_dim, rot, tokens)
    _need(q_out, tokens * nq * head_dim, torch.uint8, "q_out")
    if q_out is None:
        q_out = torch.empty(*qkv.shape[:-1], nq * head_dim, dtype=torch.uint8, device=dev)
    st = _call(fn_name, 
        _ptr(qkv), _ptr(gamma_q), _ptr(gamma_k), _ptr(positions), _ptr(cos_sin), cos_sin.shape[0],
        _ptr(scale), eps, tokens, nq, nk, nv, head_dim, rot, _dtype_code(qkv), _ptr(slot_mapping),
        num_slots, _ptr(q_out) if q_out.numel() else None,
        _ptr(kv_cache) if kv_cache.numel() else None, _stream(dev, stream))
    if st:
        raise AnqError(fn_name, st)
    return q_out


def qk_norm_rope_fp8_kv_store(qkv, gamma_q, gamma_k, positions, cos_sin, scale, eps: float,
                              nq: int, nk: int, nv: int, head_dim: int, slot_mapping, kv_cache,
                              rotary_dim: int | None = None, q_out=None, stream=None):
    """qk_norm_rope_fp8 with the KV-cache store epilogue: Q codes to q_out
    [.., nq*head_dim]; token t's K and V codes to kv_cache[slot_mapping[t]]
    (a [num_slots, (nk+nv)*head_dim] uint8 pool, updated in place; slots
    outside [0, num_slots) store nothing). Returns q_out."""
    rot = head_dim if rotary_dim is None else rotary_dim
    return _qk_store("qk_norm_rope_fp8_kv_store", (nk + nv) * head_dim, qkv, gamma_q, gamma_k,
                     positions, cos_sin, scale, eps, nq, nk, nv, head_dim, rot, slot_mapping,
                     kv_cache, q_out, stream)


def mixed_kv_row_bytes(nk: int, nv: int, head_dim: int, rotary_dim: int) -> int:
    """Bytes of one row of the mixed KV pool: nk*(head_dim + rotary_dim) + nv*head_dim."""
    return nk * (head_dim + rotary_dim) + nv * head_dim


def qk_norm_rope_kv_store_mixed(qkv, gamma_q, gamma_k, positions, cos_sin, scale, eps: float,
                                nq: int, nk: int, nv: int, head_dim: int, rotary_dim: int,
                                slot_mapping, kv_cache, q_out=None, stream=None):
    """The Q/K op with the mixed KV pool: Q codes to q_out [.., nq*head_dim];
    token t's row kv_cache[slot_mapping[t]] (rows of mixed_kv_row_bytes) gets,
    per K head, the E4M3 codes of its first head_dim - rotary_dim elements and
    then its last rotary_dim elements as bf16, then the V heads' codes.
    Returns q_out."""
    return _qk_store("qk_norm_rope_kv_store_mixed", mixed_kv_row_bytes(nk, nv, head_dim, rotary_dim),
                     qkv, gamma_q, gamma_k, positions, cos_sin, scale, eps, nq, nk, nv, head_dim,
                     rotary_dim, slot_mapping, kv_cache, q_out, stream)


# ------------------------------------------------------------ separated tail


def add_rmsnorm(x, residual, gamma, eps: float, norm=None, stream=None):
    """residual += x (in place, rounded to T); returns norm_out = RMSNorm(residual) * gamma in T.
    The first kernel of the separated (unfused) tail."""
    dev = _check_gpu(x, residual, gamma, norm)
    tokens, hidden = _tail_shapes(x, residual, gamma, norm)
    if norm is None:
        norm = torch.empty_like(x)
    st = _call("add_rmsnorm", _ptr(x), _ptr(residual), _ptr(gamma), eps, tokens, hidden,
                           _dtype_code(x), _ptr(norm), _stream(dev, stream))
    if st:
        raise AnqError("add_rmsnorm", st)
    return norm


def quant_fp8(t, scale, q=None, stream=None):
    """E4M3 codes of t / scale for an fp16/bf16 tensor t [..., hidden]."""
    dev = _check_gpu(t, scale, q)
    _scalar(scale, "scale")
    tokens, hidden = _rows(t)
    _need(q, t.numel(), torch.uint8, "q")
    if q is None:
        q = torch.empty(t.shape, dtype=torch.uint8, device=dev)
    st = _call("quant_fp8", _ptr(t), _ptr(scale), tokens, hidden, _dtype_code(t), _ptr(q),
                         _stream(dev, stream))
    if st:
        raise AnqError("quant_fp8", st)
    return q


def quant_nvfp4(t, global_scale, q=None, sf=None, stream=None):
    """NVFP4 (packed E2M1 + per-16 E4M3 scales) of an fp16/bf16 tensor t [..., hidden]."""
    dev = _check_gpu(t, global_scale, q, sf)
    _scalar(global_scale, "global_scale")
    tokens, hidden = _rows(t)
    q, sf = _nvfp4_outs(q, sf, t.shape[:-1], tokens, hidden, dev)
    st = _call("quant_nvfp4", _ptr(t), _ptr(global_scale), tokens, hidden, _dtype_code(t), _ptr(q),
                           _ptr(sf), _stream(dev, stream))
    if st:
        raise AnqError("quant_nvfp4", st)
    return q, sf


# ------------------------------------------------------------ swizzled block scales


def add_rmsnorm_quant_nvfp4_swizzled(x, residual, gamma, global_scale, eps: float,
                                     norm_out: bool = False, q=None, sf=None, norm=None,
                                     stream=None):
    """add_rmsnorm_quant_nvfp4 with the block scales in the 128x4-tiled GEMM
    layout: sf [roundup(tokens,128), roundup(hidden/16,4)] uint8, padding zeroed."""
    dev = _check_gpu(x, residual, gamma, global_scale, q, sf, norm)
    _scalar(global_scale, "global_scale")
    tokens, hidden = _tail_shapes(x, residual, gamma, norm)
    q, sf = _nvfp4_outs(q, sf, x.shape[:-1], tokens, hidden, dev, swizzled=True)
    if norm_out and norm is None:
        norm = torch.empty_like(x)
    st = _call("add_rmsnorm_quant_nvfp4_swizzled", 
        _ptr(x), _ptr(residual), _ptr(gamma), _ptr(global_scale), eps, tokens, hidden,
        _dtype_code(x), _ptr(q), _ptr(sf), _ptr(norm), _stream(dev, stream))
    if st:
        raise AnqError("add_rmsnorm_quant_nvfp4_swizzled", st)
    return q, sf, norm


def quant_nvfp4_swizzled(t, global_scale, q=None, sf=None, stream=None):
    """quant_nvfp4 with the swizzled block-scale layout."""
    dev = _check_gpu(t, global_scale, q, sf)
    _scalar(global_scale, "global_scale")
    tokens, hidden = _rows(t)
    q, sf = _nvfp4_outs(q, sf, t.shape[:-1], tokens, hidden, dev, swizzled=True)
    st = _call("quant_nvfp4_swizzled", _ptr(t), _ptr(global_scale), tokens, hidden, _dtype_code(t),
                                    _ptr(q), _ptr(sf), _stream(dev, stream))
    if st:
        raise AnqError("quant_nvfp4_swizzled", st)
    return q, sf


# ------------------------------------------------------------ gated RMSNorm


def gated_rmsnorm_quant_nvfp4(x, z, gamma, global_scale, eps: float, group: int | None = None,
                              q=None, sf=None, stream=None):
    """n = RMSNorm(x * SiLU(z)) * gamma over groups of `group` elements (default:
    the whole row), then NVFP4: returns (q [.., hidden/2], sf [.., hidden/16])."""
    dev = _check_gpu(x, z, gamma, global_scale, q, sf)
    _scalar(global_scale, "global_scale")
    tokens, hidden = _tail_shapes(x, z, gamma, None, other="z")
    q, sf = _nvfp4_outs(q, sf, x.shape[:-1], tokens, hidden, dev)
    group = hidden if group is None else group
    st = _call("gated_rmsnorm_quant_nvfp4", _ptr(x), _ptr(z), _ptr(gamma), _ptr(global_scale), eps,
                                         tokens, hidden, group, _dtype_code(x), _ptr(q), _ptr(sf),
                                         _stream(dev, stream))
    if st:
        raise AnqError("gated_rmsnorm_quant_nvfp4", st)
    return q, sf


def selfcheck_arith(device=None, stream=None) -> list[int]:
    """Mismatch counts of the device arithmetic self-check (anq_selfcheck_arith):
    [reciprocal, block-scale quotient, FP8 quotient codes, E2M1 saturation];
    all zero where the kernels are exact. Waits for the check to finish."""
    dev = torch.cuda.current_device() if device is None else torch.device(device).index
    if dev is None:
        dev = torch.cuda.current_device()
    counts = torch.empty(4, dtype=torch.int64, device=dev)
    st = lib().anq_selfcheck_arith(_ptr(counts), _stream(dev, stream))
    if st:
        raise AnqError("anq_selfcheck_arith", st)
    torch.cuda.synchronize(dev)
    return [int(v) for v in counts.cpu()]


def silu_gate_f32(x, z, u=None, stream=None):
    """u = x * SiLU(z) in binary32 steps (the gate of gated_rmsnorm_quant_nvfp4)."""
    dev = _check_gpu(x, z, u)
    if z.dtype != x.dtype or z.shape != x.shape:
        raise ValueError("x and z must share dtype and shape")
    _need(u, x.numel(), torch.float32, "u")
    if u is None:
        u = torch.empty(x.shape, dtype=torch.float32, device=dev)
    st = _call("silu_gate_f32", _ptr(x), _ptr(z), x.numel(), _dtype_code(x), _ptr(u),
                             _stream(dev, stream))
    if st:
        raise AnqError("silu_gate_f32", st)
    return u


def stream_rw(src, read_bytes: int, dst, write_bytes: int, nontemporal: bool = True,
              stream=None):
    """The calibration stream (anq_stream_rw): one pass reading read_bytes of
    src and writing write_bytes of dst, no arithmetic; src and dst are uint8
    device tensors at least that large."""
    dev = _check_gpu(src, dst)
    if src.dtype != torch.uint8 or dst.dtype != torch.uint8:
        raise ValueError("src and dst must be uint8")
    if src.numel() < read_bytes or dst.numel() < write_bytes:
        raise ValueError("src / dst smaller than the bytes asked for")
    st = _call("anq_stream_rw", _ptr(src), read_bytes, _ptr(dst), write_bytes, int(nontemporal),
                             _stream(dev, stream))
    if st:
        raise AnqError("anq_stream_rw", st)
    return dst

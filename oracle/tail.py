"""Plain CPU oracle of the fused local tail and of the Q/K norm + RoPE + FP8 store.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, step by step, in the order of the pages: an in-place
residual add, then row-wise RMSNorm, then quantisation in the epilogue
(TensorRT-LLM issue #17900 "Fuse local NVFP4 tail after NCCL fallback",
Proposal: residual + RMSNorm + NVFP4 in one launch, with or without a returned
high-precision norm output; TensorRT-LLM PR #17288 "Add NanoJet backend ...",
Description: RMSNorm with FP8 quantisation in the kernel epilogue, FP8
projection fused with an in-place residual add, Q/K RMSNorm and RoPE).

Where the pages are silent the plainest reading is taken (each is listed in
the design notes of the repository):
  * every arithmetic step is one IEEE binary32 operation rounded to nearest
    even (numpy float32 ufuncs, one rounding each, never fused);
  * the residual sum is formed in binary32 and rounded to the activation type;
    the norm reads that rounded sum;
  * the sum of squares is the exact sum rounded once to binary32;
  * r = 1 / sqrt(ss / H + eps), each of the four operations rounded;
  * n = (h * r) * gamma, two roundings; the optional norm output is n rounded
    to the activation type; the quantiser reads the binary32 n;
  * FP8: q = E4M3(n / s) with s the per-tensor scale (a dequantisation scale);
  * NVFP4: per 16 consecutive elements of a row, amax = max |n|,
    sf = E4M3(G * (amax / 6)), S = decode(sf), mult = G / S (0 when S = 0),
    code = E2M1(n * mult); byte j of a row packs element 2j in the low nibble
    and 2j+1 in the high nibble; sf is stored row-major [tokens, hidden/16];
  * Q/K: each Q and K head of head_dim D is RMS-normalised over D with a
    shared gamma_q / gamma_k, rotated NeoX-style by the cos|sin row of its
    token's position (all of the head, or its last rotary_dim elements),
    divided by the scale and encoded E4M3; V heads are only divided and
    encoded. The KV stores scatter those results into a pool: uniform FP8
    codes, or FP8 for the unrotated part and bf16 for the rotated part.
"""
from __future__ import annotations

import math

import numpy as np

from .codecs import e2m1_encode, e4m3_decode, e4m3_encode, t_decode, t_encode

F32 = np.float32
NVFP4_BLOCK = 16
NVFP4_SCALE_NUM = F32(448.0 * 6.0)  # E4M3 max times E2M1 max


# ----------------------------------------------------------------------------
# step functions
# ----------------------------------------------------------------------------


def residual_add(x_bits: np.ndarray, res_bits: np.ndarray, dtype: str) -> np.ndarray:
    """h = RNE_T(fl32(x + residual)); the new residual, written back in place."""
    s = t_decode(x_bits, dtype) + t_decode(res_bits, dtype)  # float32 + float32
    return t_encode(s, dtype)


def exact_sum_to_f32(terms: list[float]) -> np.float32:
    """The exact real sum of float64 terms, rounded once to binary32 (RNE).

    math.fsum returns the exact sum rounded to float64. Rounding that again
    to binary32 can only go wrong when the float64 value lands exactly on the
    midpoint of two binary32 neighbours; then the sign of (exact - midpoint),
    taken from a second exact fsum, picks the side, and an exact tie keeps
    the even neighbour.
    """
    d = math.fsum(terms)
    with np.errstate(over="ignore"):
        f = F32(d)
    if not np.isfinite(f) or float(f) == d:
        return f
    f_lo = f if float(f) < d else np.nextafter(f, F32(-np.inf))
    f_hi = np.nextafter(f_lo, F32(np.inf))
    if (float(f_lo) + float(f_hi)) / 2.0 == d:
        rem = math.fsum(list(terms) + [-d])
        if rem > 0.0:
            return f_hi
        if rem < 0.0:
            return f_lo
    return f


def sum_of_squares(h: np.ndarray) -> np.ndarray:
    """ss per row of float32 h [rows, H]: exact sum of h_i^2, rounded once.
    Squares of binary32 values (fp16/bf16 ones included) are exact in float64:
    a 24-bit significand squared needs 48 bits."""
    h64 = np.asarray(h, dtype=np.float64)
    sq = h64 * h64
    return np.array([exact_sum_to_f32(row.tolist()) for row in sq.reshape(len(sq), -1)],
                    dtype=F32)


def row_scale(ss: np.ndarray, width: int, eps: float) -> np.ndarray:
    """r = 1 / sqrt(fl32(fl32(ss / width) + eps)), each operation in binary32."""
    ss = np.asarray(ss, dtype=F32)
    mean = ss / F32(width)
    var = mean + F32(eps)
    return F32(1.0) / np.sqrt(var)


def normalize(h: np.ndarray, r: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """n_i = fl32(fl32(h_i * r) * gamma_i)."""
    hr = np.asarray(h, dtype=F32) * np.asarray(r, dtype=F32)[..., None]
    return hr * np.asarray(gamma, dtype=F32)


def quant_fp8(n: np.ndarray, scale: float) -> np.ndarray:
    """Per-tensor FP8: q_i = E4M3(fl32(n_i / s))."""
    return e4m3_encode(np.asarray(n, dtype=F32) / F32(scale))


def nvfp4_global_scale(n: np.ndarray) -> np.float32:
    """G = fl32(448 * 6 / amax|n|) over a whole normed tensor: the global
    scale that maps the largest value to the top of E4M3 x E2M1."""
    amax = F32(np.max(np.abs(np.asarray(n, dtype=F32))))
    return F32(NVFP4_SCALE_NUM / amax)


def quant_nvfp4(n: np.ndarray, global_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """NVFP4 of n [rows, H] (H % 16 == 0) under global scale G.

    Returns (packed [rows, H/2] uint8, sf [rows, H/16] uint8 E4M3 codes)."""
    n = np.asarray(n, dtype=F32)
    rows, width = n.shape
    g = F32(global_scale)
    blk = n.reshape(rows, width // NVFP4_BLOCK, NVFP4_BLOCK)
    amax = np.max(np.abs(blk), axis=2)                       # exact
    s_b = g * (amax / F32(6.0))                              # fl32(G * fl32(amax / 6))
    sf = e4m3_encode(s_b)
    S = e4m3_decode(sf)
    with np.errstate(divide="ignore"):
        mult = np.where(S > 0, g / np.where(S > 0, S, F32(1.0)), F32(0.0)).astype(F32)
    v = blk * mult[..., None]                                # fl32(n_i * mult)
    codes = e2m1_encode(v).reshape(rows, width)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, sf.astype(np.uint8)


def rope_neox(n: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """NeoX rotation of vectors n [..., D] by angle rows cos/sin [..., D/2]:
    o_k = n_k c_k - n_{k+D/2} s_k and o_{k+D/2} = n_{k+D/2} c_k + n_k s_k,
    every product and sum rounded to binary32 (no fused multiply-add)."""
    n = np.asarray(n, dtype=F32)
    half = n.shape[-1] // 2
    a, b = n[..., :half], n[..., half:]
    c, s = np.asarray(cos, dtype=F32), np.asarray(sin, dtype=F32)
    out = np.empty_like(n)
    out[..., :half] = (a * c) - (b * s)
    out[..., half:] = (b * c) + (a * s)
    return out


# ----------------------------------------------------------------------------
# the three operations
# ----------------------------------------------------------------------------


def _rmsnorm(h_bits, gamma_bits, dtype, eps):
    h = t_decode(h_bits, dtype)
    ss = sum_of_squares(h)
    r = row_scale(ss, h.shape[1], eps)
    n = normalize(h, r, t_decode(gamma_bits, dtype))
    return n, ss, r


def add_rmsnorm_quant_fp8(x_bits, res_bits, gamma_bits, dtype: str, scale: float, eps: float,
                          norm_out: bool = False) -> dict:
    """Residual add + RMSNorm + per-tensor FP8 of x, residual [tokens, hidden]."""
    h = residual_add(x_bits, res_bits, dtype)
    n, ss, r = _rmsnorm(h, gamma_bits, dtype, eps)
    out = dict(residual=h, q=quant_fp8(n, scale), n=n, ss=ss, r=r)
    if norm_out:
        out["norm_out"] = t_encode(n, dtype)
    return out


def add_rmsnorm_quant_nvfp4(x_bits, res_bits, gamma_bits, dtype: str, global_scale: float,
                            eps: float, norm_out: bool = False) -> dict:
    """Residual add + RMSNorm + NVFP4 of x, residual [tokens, hidden]."""
    h = residual_add(x_bits, res_bits, dtype)
    n, ss, r = _rmsnorm(h, gamma_bits, dtype, eps)
    q, sf = quant_nvfp4(n, global_scale)
    out = dict(residual=h, q=q, sf=sf, n=n, ss=ss, r=r)
    if norm_out:
        out["norm_out"] = t_encode(n, dtype)
    return out


def rmsnorm_f32(x_bits, res_bits, gamma_bits, dtype: str, eps: float) -> np.ndarray:
    """The binary32 normed tensor n alone (used to derive NVFP4 global scales)."""
    h = residual_add(x_bits, res_bits, dtype)
    return _rmsnorm(h, gamma_bits, dtype, eps)[0]


def qk_norm_rope_fp8(qkv_bits, gamma_q_bits, gamma_k_bits, positions, cos_sin, scale: float,
                     eps: float, nq: int, nk: int, nv: int, head_dim: int, dtype: str,
                     rotary_dim: int | None = None) -> dict:
    """Q/K per-head RMSNorm + NeoX RoPE + uniform FP8 store of a fused QKV row.

    qkv [tokens, (nq+nk+nv)*D] holds Q heads, then K heads, then V heads; the
    output has the same layout in E4M3 codes.

    rotary_dim R (default D): the RMSNorm covers all D elements of a Q/K head;
    the rotation covers its last R elements only, as NeoX pairs
    (D-R+k, D-R+k+R/2) for k < R/2 with the angle row cos_sin[pos] of width R
    (cos in columns k < R/2, sin in columns R/2 + k). The first D-R elements
    (the part without position encoding) keep their normed values. With
    R = D this is the whole-head rotation."""
    D = head_dim
    R = D if rotary_dim is None else rotary_dim
    N = D - R
    half = R // 2
    tokens = qkv_bits.shape[0]
    heads = nq + nk + nv
    u = t_decode(qkv_bits, dtype).reshape(tokens, heads, D)
    tab = np.asarray(cos_sin, dtype=F32)[np.asarray(positions, dtype=np.int64)]  # [tokens, R]
    cos, sin = tab[:, None, :half], tab[:, None, half:]
    out = np.empty((tokens, heads, D), dtype=np.uint8)
    o_all = np.empty((tokens, heads, D), dtype=F32)
    for lo, hi, g in ((0, nq, gamma_q_bits), (nq, nq + nk, gamma_k_bits)):
        if hi == lo:
            continue
        blk = u[:, lo:hi, :].reshape(-1, D)
        ss = sum_of_squares(blk)
        r = row_scale(ss, D, eps)
        n = normalize(blk, r, t_decode(g, dtype)).reshape(tokens, hi - lo, D)
        o = n.copy()
        o[..., N:] = rope_neox(n[..., N:], cos, sin)
        o_all[:, lo:hi] = o
        out[:, lo:hi] = e4m3_encode(o / F32(scale))
    if nv:
        v = u[:, nq + nk:, :]
        o_all[:, nq + nk:] = v
        out[:, nq + nk:] = e4m3_encode(v / F32(scale))
    return dict(out=out.reshape(tokens, heads * D), o=o_all.reshape(tokens, heads * D))


def _scatter_rows(kv_cache, slot_mapping, rows) -> np.ndarray:
    """A copy of the pool with row slot_mapping[t] replaced by rows[t]; a slot
    outside [0, num_slots) stores nothing, and rows no token names keep
    their contents."""
    kv = np.array(kv_cache, dtype=np.uint8, copy=True)
    num_slots = kv.shape[0]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if 0 <= slot < num_slots:
            kv[slot] = rows[t]
    return kv


def qk_norm_rope_fp8_kv_store(qkv_bits, gamma_q_bits, gamma_k_bits, positions, cos_sin,
                              scale: float, eps: float, nq: int, nk: int, nv: int, head_dim: int,
                              dtype: str, slot_mapping, kv_cache,
                              rotary_dim: int | None = None) -> dict:
    """The Q/K op with the KV-cache store as its epilogue (SGLang PR #32975:
    norm + RoPE + store into a uniform FP8 pool).

    The codes are those of qk_norm_rope_fp8. Q codes come back dense
    [tokens, nq*D]; token t's K then V codes overwrite row slot_mapping[t] of a
    copy of kv_cache [num_slots, (nk+nv)*D]; a slot outside [0, num_slots)
    stores nothing, and rows no token names keep their contents."""
    D = head_dim
    codes = qk_norm_rope_fp8(qkv_bits, gamma_q_bits, gamma_k_bits, positions, cos_sin, scale, eps,
                             nq, nk, nv, D, dtype, rotary_dim)["out"]
    return dict(q=codes[:, :nq * D].copy(), kv=_scatter_rows(kv_cache, slot_mapping, codes[:, nq * D:]))


def mixed_kv_row_bytes(nk: int, nv: int, head_dim: int, rotary_dim: int) -> int:
    """Bytes of one token's row of the mixed pool: per K head D-R FP8 codes and
    R bf16 values, per V head D FP8 codes."""
    return nk * (head_dim - rotary_dim + 2 * rotary_dim) + nv * head_dim


def qk_norm_rope_kv_store_mixed(qkv_bits, gamma_q_bits, gamma_k_bits, positions, cos_sin,
                                scale: float, eps: float, nq: int, nk: int, nv: int,
                                head_dim: int, rotary_dim: int, dtype: str, slot_mapping,
                                kv_cache) -> dict:
    """The Q/K op storing K into a mixed pool: the part of each K head without
    position encoding as FP8, the rotated part as bf16 (the FP8-nope /
    BF16-rope KV pool of the FlashMLA counterpart named in SGLang PR #32975's
    discussion; the pages give no layout, so the reading is stated here).

    The values are those of qk_norm_rope_fp8 with the same rotary_dim R: each
    Q/K head is RMS-normalised over all D elements and its last R elements are
    rotated. Q codes come back dense [tokens, nq*D] (E4M3 of o / s, as the
    plain op's). Token t's pool row, written to row slot_mapping[t] of a copy
    of kv_cache [num_slots, mixed_kv_row_bytes], holds for each K head j in
    order: D-R bytes E4M3(fl32(o / s)) of its first D-R elements, then its
    last R elements as bf16 RNE_bf16(o), two bytes each, little endian; then
    for each V head D bytes E4M3(fl32(v / s)). Slots outside [0, num_slots)
    store nothing; other rows keep their contents."""
    D, R = head_dim, rotary_dim
    N = D - R
    r = qk_norm_rope_fp8(qkv_bits, gamma_q_bits, gamma_k_bits, positions, cos_sin, scale, eps,
                         nq, nk, nv, D, dtype, R)
    tokens = qkv_bits.shape[0]
    heads = nq + nk + nv
    codes = r["out"].reshape(tokens, heads, D)
    o = r["o"].reshape(tokens, heads, D)
    rows = np.empty((tokens, mixed_kv_row_bytes(nk, nv, D, R)), dtype=np.uint8)
    for j in range(nk):
        base = j * (N + 2 * R)
        rows[:, base:base + N] = codes[:, nq + j, :N]
        rope = t_encode(o[:, nq + j, N:], "bf16").astype("<u2")
        rows[:, base + N:base + N + 2 * R] = rope.view(np.uint8).reshape(tokens, 2 * R)
    rows[:, nk * (N + 2 * R):] = codes[:, nq + nk:, :].reshape(tokens, nv * D)
    return dict(q=r["out"][:, :nq * D].copy(), kv=_scatter_rows(kv_cache, slot_mapping, rows),
                o=r["o"])


def swizzle_block_scales(sf: np.ndarray) -> np.ndarray:
    """Linear block scales [M, nb] -> the 128x4-tiled layout of block-scaled GEMM
    operands, returned as the buffer's bytes shaped [R, C] (R = M rounded up to
    128, C = nb rounded up to 4; padding bytes 0).

    The layout is the consumer's, which the NVFP4 pages only refer to through
    its sf_size packing math (TensorRT-LLM PR #14361, review thread): scales
    are grouped in tiles of 128 rows x 4 columns, each tile 512 contiguous
    bytes, tiles in row-major order; inside a tile the bytes run over column
    (fastest, 4), then row // 32 (4), then row % 32 (32)."""
    sf = np.asarray(sf, dtype=np.uint8)
    m, nb = sf.shape
    R = -(-m // 128) * 128
    C = -(-nb // 4) * 4
    out = np.zeros(R * C, dtype=np.uint8)
    r = np.arange(m, dtype=np.int64)[:, None]
    c = np.arange(nb, dtype=np.int64)[None, :]
    tile = (r // 128) * (C // 4) + c // 4
    inner = (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4
    out[tile * 512 + inner] = sf
    return out.reshape(R, C)


# ----------------------------------------------------------------------------
# gated RMSNorm + NVFP4
# ----------------------------------------------------------------------------

_EXP_NEG_CACHE: dict = {}


def _rn32_of_decimal(d) -> np.float32:
    """Round a positive decimal.Decimal (far more precise than binary64) to
    binary32, nearest even, without double rounding: float(d) is the correctly
    rounded binary64; only when that lands exactly on a binary32 midpoint can
    rounding it again go the wrong way, and then d itself is compared with the
    midpoint."""
    from decimal import Decimal
    f64 = float(d)
    f32 = np.float32(f64)
    if not np.isfinite(f32) or f32 == 0:
        return f32
    lo = np.nextafter(f32, np.float32(0.0)) if f64 < float(f32) else f32
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (float(lo) + float(hi)) / 2.0          # exact in binary64
    if f64 == mid:
        md = Decimal(mid)
        if d < md:
            return lo
        if d > md:
            return hi
    return f32


def exp_neg_rn32(z: np.ndarray) -> np.ndarray:
    """E = exp(-z) correctly rounded to binary32 (overflow to inf, underflow
    through the subnormals to 0), for binary32 inputs z. Evaluated with
    Python's decimal module at 40 significant digits, whose exp is correctly
    rounded at that precision, then rounded once more to binary32."""
    from decimal import Decimal, localcontext
    z = np.asarray(z, dtype=F32)
    uniq, inv = np.unique(z.reshape(-1), return_inverse=True)   # at most 2^16 values from T
    out = np.empty(uniq.shape, dtype=F32)
    with localcontext() as ctx:
        ctx.prec = 40
        for i, v in enumerate(uniq):
            key = float(v)
            e = _EXP_NEG_CACHE.get(key)
            if e is None:
                if key <= -200.0:      # exp(200) > 2^128: rounds to inf
                    e = F32(np.inf)
                elif key >= 200.0:     # exp(-200) < 2^-150: rounds to 0
                    e = F32(0.0)
                else:
                    e = _rn32_of_decimal((-Decimal(key)).exp())
                _EXP_NEG_CACHE[key] = e
            out[i] = e
    return out[inv].reshape(z.shape)


def silu_gate(x: np.ndarray, z: np.ndarray) -> np.ndarray:
    """u = x * SiLU(z) in binary32 steps: E = RN(exp(-z)), d = 1 + E,
    sigma = 1 / d, s = z * sigma, u = x * s, each rounded once."""
    x = np.asarray(x, dtype=F32)
    z = np.asarray(z, dtype=F32)
    e = exp_neg_rn32(z)
    with np.errstate(over="ignore", divide="ignore"):
        d = F32(1.0) + e
        sigma = F32(1.0) / d
        s = z * sigma
        return x * s


def gated_rmsnorm_quant_nvfp4(x_bits, z_bits, gamma_bits, dtype: str, group: int,
                              global_scale: float, eps: float) -> dict:
    """Gated RMSNorm + NVFP4 (the gated variant of the fused NVFP4 norm ops,
    TensorRT-LLM PR #14361, Changes table). The pages name it but do not define
    the gate; the reading taken is the Mamba-2 gated RMSNorm with the norm
    after the gate: over each group of `group` consecutive elements of a row,
    n = RMSNorm(x * SiLU(z)) * gamma, then the NVFP4 epilogue. No residual.

    x, z [tokens, hidden] T; gamma [hidden] T; hidden % group == 0,
    group % 16 == 0. Returns dict(q, sf, n, u, ss, r)."""
    x = t_decode(x_bits, dtype)
    z = t_decode(z_bits, dtype)
    tokens, hidden = x.shape
    u = silu_gate(x, z)
    ug = u.reshape(-1, group)                                  # one row per group
    ss = sum_of_squares(ug)
    r = row_scale(ss, group, eps)
    g = np.tile(t_decode(gamma_bits, dtype).reshape(hidden // group, group), (tokens, 1))
    n = normalize(ug, r, g)
    q, sf = quant_nvfp4(n.reshape(tokens, hidden), global_scale)
    return dict(q=q, sf=sf, n=n.reshape(tokens, hidden), u=u, ss=ss, r=r)

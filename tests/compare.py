"""Comparators for GPU-vs-oracle parity, one per tolerance class:

  * residual (and every integer/byte output the design makes exact): bit-exact;
  * norm output: max |gpu - oracle| <= 4e-3 after rounding to fp16/bf16;
  * FP8 / E2M1 codes and E4M3 block scales: identical on >= 99.9 % of
    elements and never more than one code step apart. A step is the distance
    in the ordered list of signed code values, with +0 and -0 the same rank.
    E2M1 codes are compared on blocks whose scales agree; where scales differ
    the dequantised values must be within one step at the coarser scale.

The design makes every output bit-exact (same binary32 steps, exact sum of
squares); the summaries also count exact matches so that tests can assert it.
"""
from __future__ import annotations

import numpy as np

import oracle as O

NORM_TOL = 4e-3
CODE_IDENTICAL = 0.999


def e4m3_rank(c):
    c = np.asarray(c).astype(np.int64)
    mag = c & 0x7F
    return np.where((c & 0x80) != 0, -mag, mag)


def e2m1_rank(c):
    c = np.asarray(c).astype(np.int64)
    mag = c & 0x7
    return np.where((c & 0x8) != 0, -mag, mag)


def unpack_e2m1(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def code_stats(gpu, ref, rank):
    g, r = np.asarray(gpu).ravel(), np.asarray(ref).ravel()
    step = np.abs(rank(g) - rank(r))
    n = max(g.size, 1)
    return dict(n=int(g.size), identical=float(np.mean(g == r)) if g.size else 1.0,
                bit_exact=bool(np.array_equal(g, r)), max_step=int(step.max()) if g.size else 0,
                n_diff=int(np.count_nonzero(g != r)), frac_same_rank=float(np.count_nonzero(step == 0)) / n)


def check_codes(stats, what):
    assert stats["max_step"] <= 1, f"{what}: codes more than one step apart: {stats}"
    assert stats["frac_same_rank"] >= CODE_IDENTICAL, f"{what}: too many code differences: {stats}"


def check_residual(gpu_bits, ref_bits, what="residual"):
    g, r = np.asarray(gpu_bits), np.asarray(ref_bits)
    assert g.shape == r.shape, (g.shape, r.shape)
    bad = np.nonzero(g.ravel() != r.ravel())[0]
    assert bad.size == 0, f"{what}: {bad.size} elements differ, first at {bad[:5]}"


def norm_stats(gpu_bits, ref_bits, dtype):
    g = O.t_decode(gpu_bits, dtype).astype(np.float64)
    r = O.t_decode(ref_bits, dtype).astype(np.float64)
    same = np.asarray(gpu_bits) == np.asarray(ref_bits)
    with np.errstate(invalid="ignore"):
        err = np.where(same, 0.0, np.abs(g - r))      # equal infinities: no error
    err = np.where(np.isnan(err), np.inf, err)        # differing non-finite values fail
    return dict(max_abs_err=float(err.max()) if err.size else 0.0,
                bit_exact=bool(np.array_equal(np.asarray(gpu_bits), np.asarray(ref_bits))),
                n_diff=int(np.count_nonzero(np.asarray(gpu_bits) != np.asarray(ref_bits))))


def check_norm(stats, what="norm_out"):
    assert stats["max_abs_err"] <= NORM_TOL, f"{what}: {stats}"


def nvfp4_stats(q_gpu, sf_gpu, q_ref, sf_ref, global_scale):
    """Scale and code agreement of an NVFP4 output pair ([rows, H/2], [rows, H/16])."""
    sfs = code_stats(sf_gpu, sf_ref, e4m3_rank)
    cg, cr = unpack_e2m1(q_gpu), unpack_e2m1(q_ref)
    rows, width = cg.shape
    same = (np.asarray(sf_gpu) == np.asarray(sf_ref))
    same_el = np.repeat(same, 16, axis=1)
    codes = code_stats(cg[same_el], cr[same_el], e2m1_rank)
    # blocks whose scales differ: dequantised values within one step at the coarser scale
    worst = 0.0
    if not same.all():
        G = float(global_scale)
        Sg = np.repeat(O.e4m3_decode(sf_gpu).astype(np.float64), 16, axis=1)
        Sr = np.repeat(O.e4m3_decode(sf_ref).astype(np.float64), 16, axis=1)
        dg = O.e2m1_decode(cg).astype(np.float64) * Sg / G
        dr = O.e2m1_decode(cr).astype(np.float64) * Sr / G
        coarse = np.maximum(Sg, Sr) / G * 2.0  # the largest E2M1 step (4 -> 6) at that scale
        m = ~same_el
        worst = float(np.max(np.abs(dg - dr)[m] / coarse[m]))
    return dict(sf=sfs, codes=codes, blocks_scale_differs=int(np.count_nonzero(~same)),
                deq_over_step=worst,
                bit_exact=bool(np.array_equal(q_gpu, q_ref) and np.array_equal(sf_gpu, sf_ref)))


def check_nvfp4(stats, what="nvfp4"):
    check_codes(stats["sf"], what + " block scales")
    check_codes(stats["codes"], what + " E2M1 codes")
    assert stats["deq_over_step"] <= 1.0, f"{what}: {stats}"

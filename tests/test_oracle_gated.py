"""Pins of the oracle's gated RMSNorm + NVFP4 (oracle/tail.py) against things
other than itself: a rigorous Taylor enclosure of exp in exact rationals,
binary64 exp from the C library, exact step-by-step rounding of the gate,
closed-form limits, and composition from the pinned plain steps."""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle as O
from exact import round_rational

F32 = np.float32


def _exp_enclosure(z: Fr, terms: int = 90) -> tuple[Fr, Fr]:
    """[lo, hi] containing exp(-z) for |z| <= 8: the Taylor sum of exp(-z) to
    `terms` terms, widened by a bound on the remainder (the next term's
    magnitude times 2, valid once the terms shrink by at least half)."""
    s, t = Fr(0), Fr(1)
    for k in range(terms):
        s += t
        t = t * (-z) / (k + 1)
    r = 2 * abs(t)
    return s - r, s + r


def test_exp_neg_is_correctly_rounded_on_a_sample():
    """For 600 fp16 / bf16 values in [-8, 8], both ends of a rigorous enclosure
    of exp(-z) round to the oracle's binary32 result: it is the nearest."""
    rng = np.random.default_rng(3)
    zs = np.concatenate([rng.uniform(-8, 8, 300).astype(np.float16).astype(F32),
                         O.t_decode(O.t_encode(rng.uniform(-8, 8, 300).astype(F32), "bf16"), "bf16"),
                         np.array([0.0, -0.0, 1.0, -1.0, 0.5, 2.0 ** -24, -(2.0 ** -14)], F32)])
    got = O.exp_neg_rn32(zs)
    for z, e in zip(zs, got):
        lo, hi = _exp_enclosure(Fr(float(z)))
        assert round_rational(lo, "f32") == round_rational(hi, "f32") == Fr(float(e)), float(z)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exp_neg_agrees_with_binary64_exp_away_from_midpoints(dtype):
    """Every finite fp16 / bf16 value: RN32(math.exp(-z)) (libm, binary64)
    equals the oracle wherever the binary64 value is not within 4 ulps of a
    binary32 rounding midpoint (where a second rounding could differ)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    z = O.t_decode(b, dtype)
    z = z[np.isfinite(z)]
    got = O.exp_neg_rn32(z)
    checked = 0
    for v, e in zip(z, got):
        try:
            f64 = math.exp(-float(v))
        except OverflowError:
            assert np.isinf(e) and e > 0
            continue
        f32 = np.float32(f64)
        if np.isfinite(f32) and f32 != 0:
            a, c = np.nextafter(f32, F32(0)), np.nextafter(f32, F32(np.inf))
            mids = ((float(a) + float(f32)) / 2, (float(f32) + float(c)) / 2)
            if any(abs(f64 - m) <= 4 * math.ulp(f64) for m in mids):
                continue
        assert f32 == e or (np.isinf(f32) and np.isinf(e)), float(v)
        checked += 1
    assert checked > 40000                   # all but the overflowing z < -88.7


def test_exp_neg_limits():
    e = O.exp_neg_rn32(np.array([0.0, -88.0, -89.0, 103.0, 104.0, 120.0, -65504.0], F32))
    assert e[0] == 1.0
    assert np.isfinite(e[1]) and np.isinf(e[2])             # e^89 > FLT_MAX
    assert e[3] == F32(2.0 ** -149)                           # e^-103 = 1.3 x 2^-149
    assert e[4] == 0.0 and e[5] == 0.0                        # below half the least subnormal
    assert np.isinf(e[6])


def test_silu_gate_each_step_rounded_once():
    """u = RN(x * RN(z * RN(1 / RN(1 + E)))) with E = RN(exp(-z)), checked
    in exact rationals for seeded values."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(200).astype(F32)
    z = (3 * rng.standard_normal(200)).astype(F32)
    u = O.silu_gate(x, z)
    E = O.exp_neg_rn32(z)
    for i in range(200):
        d = round_rational(1 + Fr(float(E[i])), "f32")
        sig = round_rational(1 / d, "f32")
        s = round_rational(Fr(float(z[i])) * sig, "f32")
        want = round_rational(Fr(float(x[i])) * s, "f32")
        assert Fr(float(u[i])) == want, i


def test_silu_gate_limits():
    x = np.array([1.5, -2.0, 3.0, 1.0], F32)
    z = np.array([20.0, 0.0, -200.0, -0.0], F32)
    u = O.silu_gate(x, z)
    assert u[0] == F32(30.0)                  # sigma rounds to 1: s = z
    assert u[1] == 0.0                        # SiLU(0) = 0
    assert u[2] == 0.0 and np.signbit(u[2])   # E = inf, sigma = 0, s = -0, u = 3 * -0
    assert u[3] == 0.0


def test_gated_op_is_per_group_composition():
    """Group j of every row is the pinned plain steps applied to that slice:
    exact sum of squares over the group, r over the group width, gamma slice j,
    then NVFP4 of the whole row; groups equal to the row reduce to one group."""
    rng = np.random.default_rng(21)
    tokens, hidden, group = 5, 192, 64
    xb = O.t_encode(rng.standard_normal((tokens, hidden)).astype(F32), "bf16")
    zb = O.t_encode((2 * rng.standard_normal((tokens, hidden))).astype(F32), "bf16")
    gb = O.t_encode((1 + 0.1 * rng.standard_normal(hidden)).astype(F32), "bf16")
    G = 300.0
    out = O.gated_rmsnorm_quant_nvfp4(xb, zb, gb, "bf16", group, G, 1e-5)
    u = O.silu_gate(O.t_decode(xb, "bf16"), O.t_decode(zb, "bf16"))
    gamma = O.t_decode(gb, "bf16")
    n = np.empty((tokens, hidden), F32)
    for j in range(hidden // group):
        sl = slice(j * group, (j + 1) * group)
        r = O.row_scale(O.sum_of_squares(u[:, sl]), group, 1e-5)
        n[:, sl] = O.normalize(u[:, sl], r, gamma[sl][None, :])
    assert np.array_equal(out["n"], n)
    q, sf = O.quant_nvfp4(n, G)
    assert np.array_equal(out["q"], q) and np.array_equal(out["sf"], sf)
    whole = O.gated_rmsnorm_quant_nvfp4(xb, zb, gb, "bf16", hidden, G, 1e-5)
    r = O.row_scale(O.sum_of_squares(u), hidden, 1e-5)
    assert np.array_equal(whole["n"], O.normalize(u, r, gamma[None, :]))


def test_gated_norm_follows_the_gate():
    """With z = 20 the gate is exactly z (sigma rounds to 1), so the op is the
    RMSNorm of x * 20, whose n is RMSNorm(x)'s up to rounding, not 20 times it
    (a norm taken before the gate would give the latter)."""
    rng = np.random.default_rng(5)
    xb = O.t_encode(rng.standard_normal((3, 64)).astype(F32), "f16")
    zb = O.t_encode(np.full((3, 64), 20.0, F32), "f16")
    gb = O.t_encode(np.ones(64, F32), "f16")
    n = O.gated_rmsnorm_quant_nvfp4(xb, zb, gb, "f16", 64, 1.0, 1e-6)["n"]
    x = O.t_decode(xb, "f16").astype(np.float64)
    ref = x / np.sqrt((x * x).mean(axis=1, keepdims=True))
    assert np.max(np.abs(n - ref)) < 1e-5


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gated_zero_gate_rows(dtype):
    """z = 0 gives u = 0: ss = 0, r = 1/sqrt(eps), n = 0, all codes and scales +-0."""
    xb = O.t_encode(np.ones((2, 32), F32), dtype)
    zb = O.t_encode(np.zeros((2, 32), F32), dtype)
    gb = O.t_encode(np.ones(32, F32), dtype)
    out = O.gated_rmsnorm_quant_nvfp4(xb, zb, gb, dtype, 32, 100.0, 1e-6)
    assert not np.any(out["n"]) and not np.any(out["sf"]) and not np.any(out["q"] & 0x77)


def test_gated_pins_catch_planted_mistakes(monkeypatch):
    """A binary32 exp (numpy's, not correctly rounded) in place of the oracle's
    fails the binary64 comparison; a norm taken before the gate fails the
    gate-order pin."""
    import oracle.tail as T
    with monkeypatch.context() as m:
        def exp32(z):
            with np.errstate(over="ignore"):
                return np.exp(-np.asarray(z, F32)).astype(F32)
        m.setattr(T, "exp_neg_rn32", exp32)
        m.setattr(O, "exp_neg_rn32", exp32)
        with pytest.raises(AssertionError):
            test_exp_neg_agrees_with_binary64_exp_away_from_midpoints("f16")
    with monkeypatch.context() as m:
        real = T.silu_gate
        m.setattr(T, "silu_gate", lambda x, z: np.asarray(x, F32))      # gate dropped before the norm
        orig_norm = T.normalize
        m.setattr(T, "normalize",
                  lambda h, r, g: orig_norm(h, r, g) * real(np.ones_like(h), np.full_like(h, 20.0)))
        with pytest.raises(AssertionError):
            test_gated_norm_follows_the_gate()


def test_library_gate_table_is_the_oracle_gate():
    """The constant bf16 gate table compiled into the library
    (csrc/anq_gate_table.h) holds, for every bf16 z with 2^-25 <= |z| < 128,
    the bit pattern of the oracle's gate s(z) = silu_gate(1, z); its layout is
    positive z in entries 0..4095, negative z in 4096..8191, exponent field
    102 upward."""
    import os
    import re
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "nvfp4_quantization_place_amd", "csrc", "anq_gate_table.h")
    src = open(path).read()
    body = src[src.index("kGateTabBits[8192] = {"):].split("}", 1)[0]
    vals = np.array([int(v, 16) for v in re.findall(r"0x([0-9a-f]{8})u", body)], np.uint32)
    assert len(vals) == 8192
    j = np.arange(8192, dtype=np.uint32)
    b = (((j & 4095) + (102 << 7)) | ((j >> 12) << 15)).astype(np.uint16)
    z = O.t_decode(b, "bf16")
    assert np.all((np.abs(z) >= 2.0 ** -25) & (np.abs(z) < 128))
    with np.errstate(over="ignore"):
        ref = O.silu_gate(np.ones(8192, F32), z)
    np.testing.assert_array_equal(vals, ref.view(np.uint32))

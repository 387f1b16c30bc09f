"""Pins of the oracle's fused tail and Q/K path (oracle/tail.py) against things
other than itself: hand-worked rows, exact rational arithmetic, brute-force
enumeration on tiny inputs, closed forms and invariants."""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle as O
from exact import round_rational, round_sqrt

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32
RNG = np.random.default_rng(2024)


def _bits(vals, dtype):
    """Exact fp16/bf16 bit patterns of values that are representable."""
    f = np.asarray(vals, dtype=np.float32)
    b = O.t_encode(f, dtype)
    assert np.array_equal(O.t_decode(b, dtype), f), "value not representable"
    return b


def _rand_t(shape, dtype, scale=1.0, rng=RNG):
    return O.t_encode((scale * rng.standard_normal(shape)).astype(np.float32), dtype)


def _ulp32(x):
    x = abs(float(x))
    return float(np.spacing(np.float32(x))) if x > 0 else 2.0 ** -149


# ------------------------------------------------------------ worked rows ---

def _worked():
    with open(os.path.join(HERE, "golden", "worked_rows.json")) as fh:
        return json.load(fh)


def test_worked_row_w1():
    w = _worked()["W1"]
    d = w["dtype"]
    o = O.add_rmsnorm_quant_fp8(_bits([w["x"]], d), _bits([w["residual"]], d), _bits(w["gamma"], d),
                                d, w["scale"], w["eps"], norm_out=True)
    assert o["r"].view(np.uint32)[0] == int(w["expect"]["r_bits"], 16)
    assert np.all(o["norm_out"] == int(w["expect"]["norm_out_bits_all"], 16))
    assert np.all(o["q"] == int(w["expect"]["q_all"], 16))


def test_worked_row_w5():
    w = _worked()["W5"]
    d = w["dtype"]
    e = w["expect"]
    o = O.add_rmsnorm_quant_fp8(_bits([w["x"]], d), _bits([w["residual"]], d), _bits(w["gamma"], d),
                                d, w["scale"], w["eps"], norm_out=True)
    assert o["r"][0] == F32(e["r_f32"])
    assert o["n"][0, :2].tolist() == [float(F32(v)) for v in e["n01_f32"]]
    assert o["norm_out"][0, :2].tolist() == [int(v, 16) for v in e["norm_out01_bits"]]
    assert o["q"][0, :2].tolist() == [int(v, 16) for v in e["q01"]]


@pytest.mark.parametrize("key", ["W2", "W3", "W4"])
def test_worked_nvfp4_blocks(key):
    w = _worked()[key]
    q, sf = O.quant_nvfp4(np.array([w["block"]], dtype=np.float32), w["global_scale"])
    assert int(sf[0, 0]) == int(w["expect"]["sf"], 16)
    assert " ".join("%02X" % b for b in q[0]) == w["expect"]["bytes"]


# ------------------------------------------------------ residual (I1) -------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_residual_is_exact_sum_rounded_once(dtype):
    x = _rand_t(3000, dtype, 3.0)
    r = _rand_t(3000, dtype, 0.01)
    h = O.residual_add(x, r, dtype)
    xs, rs, hs = O.t_decode(x, dtype), O.t_decode(r, dtype), O.t_decode(h, dtype)
    for a, b, c in zip(xs, rs, hs):
        assert Fr(float(c)) == round_rational(Fr(float(a)) + Fr(float(b)), dtype)


def test_residual_fp16_matches_native_half_add():
    x = _rand_t(5000, "f16", 5.0)
    r = _rand_t(5000, "f16", 5.0)
    native = (x.view(np.float16) + r.view(np.float16)).view(np.uint16)
    assert np.array_equal(O.residual_add(x, r, "f16"), native)


# ------------------------------------------------------- sum of squares -----

@pytest.mark.parametrize("dtype,spread", [("f16", 1.0), ("f16", 6.0), ("bf16", 1.0), ("bf16", 20.0)])
def test_sum_of_squares_is_exact_sum_rounded_once(dtype, spread):
    rows = []
    for _ in range(40):
        w = 16 * int(RNG.integers(1, 40))
        mag = np.exp(spread * RNG.standard_normal(w)) * RNG.choice([-1, 1], w)
        mag = np.clip(mag, -60000.0, 60000.0) if dtype == "f16" else np.clip(mag, -1e15, 1e15)
        rows.append(O.t_decode(O.t_encode(mag.astype(np.float32), dtype), dtype))
    for h in rows:
        ss = O.sum_of_squares(h[None, :])[0]
        exact = sum(Fr(float(v)) ** 2 for v in h)
        assert Fr(float(ss)) == round_rational(exact, "f32")


def test_sum_of_squares_resolves_float64_midpoints():
    # 2^30 + 2^6 is the midpoint of binary32 2^30 and 2^30 + 2^7; a tiny square
    # (2^-48 from fp16 2^-24, 2^-80 from bf16 2^-40) pushes the exact sum above
    # it, but float64 cannot hold it.
    for dtype, tiny in (("f16", 2.0 ** -24), ("bf16", 2.0 ** -40)):
        h = O.t_decode(_bits([[32768.0, 8.0, tiny] + [0.0] * 13], dtype), dtype)
        naive = F32(float(np.sum(h.astype(np.float64) ** 2)))
        assert naive == F32(2.0 ** 30)  # the trap is real
        assert O.sum_of_squares(h)[0] == F32(2.0 ** 30 + 2.0 ** 7)
        tie = O.t_decode(_bits([[32768.0, 8.0] + [0.0] * 14], dtype), dtype)
        assert O.sum_of_squares(tie)[0] == F32(2.0 ** 30)  # exact tie: even neighbour


def test_sum_of_squares_constant_row_and_permutation():
    for c in (1.0, 3.0, 0.5, 7.0):
        for w in (16, 128, 1024):
            h = np.full((1, w), c, dtype=np.float32)
            assert O.sum_of_squares(h)[0] == F32(w * c * c)  # I5: exact small integers
    h = O.t_decode(_rand_t((1, 7168), "bf16", 4.0), "bf16")
    base = O.sum_of_squares(h)[0]
    for _ in range(5):  # I4: order-free
        assert O.sum_of_squares(h[:, RNG.permutation(7168)])[0] == base


# ------------------------------------------------------------- row scale ----

def test_row_scale_each_operation_rounded_once():
    for _ in range(300):
        ss = F32(np.exp(RNG.uniform(-20, 25)))
        width = int(16 * RNG.integers(1, 600))
        eps = float(F32(10.0 ** RNG.uniform(-8, 0)))
        got = O.row_scale(np.array([ss]), width, eps)[0]
        mean = round_rational(Fr(float(ss)) / width, "f32")
        var = round_rational(mean + Fr(float(F32(eps))), "f32")
        root = round_sqrt(var, "f32")
        want = round_rational(1 / root, "f32")
        assert Fr(float(got)) == want, (ss, width, eps)


def test_normalize_two_roundings():
    h = O.t_decode(_rand_t(2000, "bf16", 2.0), "bf16")
    g = O.t_decode(_rand_t(2000, "bf16", 1.0), "bf16")
    r = F32(0.73123456)
    n = O.normalize(h[None, :], np.array([r]), g)[0]
    for a, b, c in zip(h, g, n):
        t = round_rational(Fr(float(a)) * Fr(float(r)), "f32")
        assert Fr(float(c)) == round_rational(t * Fr(float(b)), "f32")


@pytest.mark.parametrize("dtype,eps", [("f16", 1e-6), ("bf16", 1e-5), ("f16", 0.5), ("bf16", 3.0)])
def test_norm_close_to_real_number_formula(dtype, eps):
    """n = h * gamma / sqrt(mean(h^2) + eps) evaluated with 40 significant
    digits; the binary32 oracle is within 3 ulps (a dropped eps, a mean over
    H-1, a 1+gamma or a missing gamma all fail this by far)."""
    getcontext().prec = 40
    width = 64
    x = _rand_t((3, width), dtype, 1.0)
    res = _rand_t((3, width), dtype, 0.5)
    g = O.t_encode((1 + 0.1 * RNG.standard_normal(width)).astype(np.float32), dtype)
    o = O.add_rmsnorm_quant_fp8(x, res, g, dtype, 0.02, eps, norm_out=True)
    h = O.t_decode(o["residual"], dtype)
    gg = O.t_decode(g, dtype)
    for i in range(3):
        ms = sum(Decimal(float(v)) ** 2 for v in h[i]) / width
        inv = 1 / (ms + Decimal(float(F32(eps)))).sqrt()
        for j in range(width):
            real = float(Decimal(float(h[i, j])) * inv * Decimal(float(gg[j])))
            assert abs(float(o["n"][i, j]) - real) <= 3 * _ulp32(real), (i, j)


# ----------------------------------------------------------------- FP8 ------

def test_fp8_brute_force_and_half_step_bound():
    """Each code is the nearest of all 254 finite E4M3 values to fl32(n/s)
    (ties even), and |decode(q)*s - n| stays within half an E4M3 step of
    n/s (times s, plus the one binary32 rounding of the quotient) or q is
    +-448 (I2)."""
    table = O.e4m3_decode(np.arange(256)).astype(np.float64)
    x = _rand_t((4, 32), "bf16", 1.0)
    res = _rand_t((4, 32), "bf16", 2.0)
    g = _rand_t(32, "bf16", 1.0)
    s = 0.01
    o = O.add_rmsnorm_quant_fp8(x, res, g, "bf16", s, 1e-6)
    n = o["n"].ravel()
    for v, q in zip(n, o["q"].ravel()):
        quo = float(F32(v) / F32(s))
        fin = ~np.isnan(table)
        cand = np.nonzero(fin & ((np.arange(256) >= 128) == bool(np.signbit(np.float32(quo)))))[0]
        if abs(quo) >= 448:
            assert table[q] == math.copysign(448.0, quo)
            continue
        d = np.abs(table[cand] - quo)
        best = cand[d == d.min()]
        if len(best) > 1:
            best = best[best % 2 == 0]
        assert q == best[0]
        pos = np.sort(np.abs(table[fin]))
        k = np.searchsorted(pos, abs(quo))
        step = pos[min(k, len(pos) - 1)] - pos[max(k - 1, 0)]
        assert abs(table[q] * float(F32(s)) - float(v)) <= 0.5 * step * float(F32(s)) + 2 * _ulp32(v)


# --------------------------------------------------------------- NVFP4 ------

def test_nvfp4_block_scale_and_codes_brute_force():
    e4 = O.e4m3_decode(np.arange(0x7F)).astype(np.float64)  # 127 non-negative values
    n = (RNG.standard_normal((6, 64)) * np.exp(RNG.uniform(-3, 3, (6, 1)))).astype(np.float32)
    n[0, :16] = 0.0            # an all-zero block
    n[1, 16:32] = -0.0         # negative zeros
    G = float(O.nvfp4_global_scale(n))
    q, sf = O.quant_nvfp4(n, G)
    e2 = O.E2M1_VALUES
    for i in range(n.shape[0]):
        for b in range(n.shape[1] // 16):
            blk = n[i, 16 * b:16 * b + 16]
            amax = float(np.max(np.abs(blk)))
            s_b = float(F32(G) * (F32(amax) / F32(6.0)))
            d = np.abs(e4 - s_b)
            best = np.nonzero(d == d.min())[0]
            if len(best) > 1:
                best = best[best % 2 == 0]
            want_sf = 0x7E if s_b >= 448 else int(best[0])
            assert sf[i, b] == want_sf
            S = float(e4[want_sf])
            mult = F32(G) / F32(S) if S > 0 else F32(0.0)
            for j in range(16):
                v = float(F32(blk[j]) * mult)
                c = int(q[i, (16 * b + j) // 2] >> (4 * ((16 * b + j) % 2))) & 0xF
                assert (c >> 3) == int(np.signbit(np.float32(v)))
                if abs(v) >= 6:
                    assert c & 7 == 7
                    continue
                dd = np.abs(e2 - abs(v))
                bb = np.nonzero(dd == dd.min())[0]
                if len(bb) > 1:
                    bb = bb[bb % 2 == 0]
                assert c & 7 == bb[0]
                # I3: dequantised value within half an E2M1 step of v, scaled back
                k = np.searchsorted(e2, abs(v))
                step = e2[min(k, 7)] - e2[max(k - 1, 0)]
                deq = float(O.e2m1_decode(c)) * S / G
                assert abs(deq - float(blk[j])) <= (0.5 * step + 1e-6) * S / G + 2 * _ulp32(blk[j])
    assert sf[0, 0] == 0 and np.all(q[0, :8] == 0)
    assert np.all(q[1, 8:16] == 0x88)


def test_nvfp4_packing_low_nibble_first():
    n = np.zeros((1, 16), dtype=np.float32)
    n[0, 0], n[0, 1] = 6.0, -0.5
    q, sf = O.quant_nvfp4(n, 1.0)  # amax 6 -> S = 1, mult = 1
    assert sf[0, 0] == 0x38
    assert q[0, 0] == (0x7 | (0x9 << 4))


def test_nvfp4_grid_values_encode_exactly():
    # I7: with S = 1 (G = 1, amax = 6) every grid value comes back as itself
    vals = np.array([[0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6, 6]], dtype=np.float32)
    q, sf = O.quant_nvfp4(vals, 1.0)
    codes = np.stack([q[0] & 0xF, q[0] >> 4], axis=1).ravel()
    assert np.array_equal(O.e2m1_decode(codes), vals[0])


def test_global_scale_definition():
    n = np.array([[0.5, -7.25, 3.0, 1.0]], dtype=np.float32)
    assert O.nvfp4_global_scale(n) == F32(2688.0) / F32(7.25)


# ------------------------------------------------------------------ RoPE ----

def test_rope_identity_swap_and_norm():
    n = RNG.standard_normal((5, 128)).astype(np.float32)
    half = 64
    ones, zeros = np.ones((5, half), np.float32), np.zeros((5, half), np.float32)
    assert np.array_equal(O.rope_neox(n, ones, zeros), n)                  # pos 0
    o = O.rope_neox(n, zeros, ones)                                        # (cos, sin) = (0, 1)
    assert np.array_equal(o[:, :half], -n[:, half:])
    assert np.array_equal(o[:, half:], n[:, :half])
    ang = RNG.uniform(0, 2 * np.pi, (5, half))
    o = O.rope_neox(n, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32))
    before = n[:, :half].astype(np.float64) ** 2 + n[:, half:].astype(np.float64) ** 2
    after = o[:, :half].astype(np.float64) ** 2 + o[:, half:].astype(np.float64) ** 2
    assert np.allclose(after, before, rtol=1e-6, atol=1e-12)


def test_rope_each_product_and_sum_rounded():
    n = RNG.standard_normal((1, 32)).astype(np.float32)
    ang = RNG.uniform(0, 2 * np.pi, (1, 16))
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    o = O.rope_neox(n, c, s)
    for k in range(16):
        a, b, cc, ss = (Fr(float(v)) for v in (n[0, k], n[0, k + 16], c[0, k], s[0, k]))
        lo = round_rational(round_rational(a * cc, "f32") - round_rational(b * ss, "f32"), "f32")
        hi = round_rational(round_rational(b * cc, "f32") + round_rational(a * ss, "f32"), "f32")
        assert Fr(float(o[0, k])) == lo and Fr(float(o[0, k + 16])) == hi


def test_qk_heads_match_per_head_composition():
    """The Q/K op equals, head by head, the pinned steps applied to one head:
    norm over D with the Q or K gamma, NeoX rotation by the token's row, E4M3
    of o/s; V heads are E4M3 of v/s. Position 0 leaves Q/K unrotated."""
    import workloads as W
    inp = W.make_qk(7, "bf16", tokens=5, nq=2, nk=1, nv=1, head_dim=32,
                    positions=np.array([0, 3, 1, 4, 2]), max_pos=8)
    qkv = W.bits(inp.qkv)
    out = O.qk_norm_rope_fp8(qkv, W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
                             inp.cos_sin, inp.scale, inp.eps, 2, 1, 1, 32, "bf16")["out"]
    D = 32
    for t in range(5):
        pos = int(inp.positions[t])
        for hd in range(4):
            u = O.t_decode(qkv[t, hd * D:(hd + 1) * D], "bf16")[None, :]
            if hd < 3:
                g = W.bits(inp.gamma_q if hd < 2 else inp.gamma_k)
                r = O.row_scale(O.sum_of_squares(u), D, inp.eps)
                nn = O.normalize(u, r, O.t_decode(g, "bf16"))
                o = O.rope_neox(nn, inp.cos_sin[pos, :16][None], inp.cos_sin[pos, 16:][None])
                if pos == 0:
                    assert np.array_equal(o, nn)
            else:
                o = u
            want = O.e4m3_encode(o / F32(inp.scale))[0]
            assert np.array_equal(out[t, hd * D:(hd + 1) * D], want), (t, hd)


def test_qk_kv_store_is_a_scatter_of_the_plain_op():
    """The store epilogue moves the plain op's codes and nothing else: with the
    identity mapping the pool is the K|V columns of the plain output; with a
    permutation row perm[t] holds token t's K|V codes; a padding slot (-1) or
    one past the pool stores nothing, and rows no token names keep their bytes."""
    import workloads as W
    inp = W.make_qk(8, "f16", tokens=6, nq=2, nk=1, nv=2, head_dim=32)
    D, nq, kvw = 32, 2, 3 * 32
    args = (W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
            inp.cos_sin, inp.scale, inp.eps, nq, 1, 2, D, "f16")
    plain = O.qk_norm_rope_fp8(*args)["out"]
    r = O.qk_norm_rope_fp8_kv_store(*args, np.arange(6), np.zeros((6, kvw), np.uint8))
    assert np.array_equal(r["q"], plain[:, :nq * D]) and np.array_equal(r["kv"], plain[:, nq * D:])
    perm = np.array([4, 0, 5, 2, 1, 3])
    r = O.qk_norm_rope_fp8_kv_store(*args, perm, np.zeros((6, kvw), np.uint8))
    for t in range(6):
        assert np.array_equal(r["kv"][perm[t]], plain[t, nq * D:])
    pool = np.full((9, kvw), 0xAB, np.uint8)
    slots = np.array([7, -1, 0, 9, 3, -5])
    r = O.qk_norm_rope_fp8_kv_store(*args, slots, pool)
    written = {7: 0, 0: 2, 3: 4}
    for row in range(9):
        want = plain[written[row], nq * D:] if row in written else pool[row]
        assert np.array_equal(r["kv"][row], want), row
    assert np.all(pool == 0xAB)                      # the input pool is not modified


def test_swizzled_scale_layout():
    """Offsets worked by hand from the tile description (128x4 tiles of 512
    bytes, row-major tiles; inside a tile column fastest, then row // 32, then
    row % 32), and the structure that follows: a bijection onto the padded
    buffer, 16-byte groups holding rows k, k+32, k+64, k+96, zero padding."""
    m, nb = 300, 10                                  # R = 384, C = 12: 3 x 3 tiles
    sf = (np.arange(m * nb, dtype=np.int64) % 251 + 1).astype(np.uint8).reshape(m, nb)
    out = O.swizzle_block_scales(sf)
    assert out.shape == (384, 12)
    flat = out.reshape(-1)
    # (row, col) -> byte, by hand: tile (r//128)*3 + c//4; inner (r%32)*16 + ((r%128)//32)*4 + c%4
    hand = {(0, 0): 0, (0, 3): 3, (1, 0): 16, (31, 2): 498, (32, 0): 4, (33, 1): 21, (64, 0): 8,
            (127, 3): 511, (0, 4): 512, (5, 9): 1024 + 80 + 1, (128, 0): 1536,
            (299, 9): (2 * 3 + 2) * 512 + (299 % 32) * 16 + ((299 % 128) // 32) * 4 + 1}
    assert hand[(299, 9)] == 4096 + 11 * 16 + 1 * 4 + 1
    for (r, c), off in hand.items():
        assert flat[off] == sf[r, c], (r, c, off)
    # every real scale lands exactly once (two byte planes carry the flat index + 1)
    idx = np.arange(1, m * nb + 1, dtype=np.int64).reshape(m, nb)
    lo = O.swizzle_block_scales((idx % 256).astype(np.uint8)).reshape(-1).astype(np.int64)
    hi = O.swizzle_block_scales((idx // 256).astype(np.uint8)).reshape(-1).astype(np.int64)
    got = hi * 256 + lo
    assert np.array_equal(np.sort(got[got > 0]), np.arange(1, m * nb + 1))
    assert np.count_nonzero(got) == m * nb        # everything else is padding (0)
    # the 4 bytes at 16k + 4j of tile (0, 0) are row k + 32j, columns 0..3
    for k in (0, 7, 31):
        for j in range(4):
            assert np.array_equal(flat[16 * k + 4 * j: 16 * k + 4 * j + 4], sf[k + 32 * j, :4])
    # column padding (cols 10, 11) and row padding (rows 300..383) are zero
    assert not flat[[2 * 512 + 16 * 3 + 2, 2 * 512 + 16 * 3 + 3]].any()
    assert not flat[8 * 512 + (300 % 32) * 16 + ((300 % 128) // 32) * 4:][:4].any()


# ------------------------------------------------- planted mistakes fail ---

def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible slips in the oracle (on the CPU) and check a pin above
    fails for each: a mean over H-1, eps outside the sqrt, a 1+gamma weight,
    the E2M1 tie rule flipped, and the float64-midpoint guard removed."""
    import oracle.tail as T

    def run(pin):
        try:
            pin()
        except AssertionError:
            return True
        return False

    good_rs = T.row_scale
    monkeypatch.setattr(O, "row_scale", lambda ss, w, e: good_rs(ss, w - 1, e))
    assert run(test_row_scale_each_operation_rounded_once)
    monkeypatch.setattr(O, "row_scale", lambda ss, w, e: F32(1.0) / np.sqrt(np.asarray(ss, F32) / F32(w)) + F32(0) * F32(e))
    assert run(lambda: test_row_scale_each_operation_rounded_once())
    monkeypatch.setattr(O, "row_scale", good_rs)

    good_norm = T.normalize
    monkeypatch.setattr(T, "normalize", lambda h, r, g: good_norm(h, r, np.asarray(g, F32) + F32(1)))
    assert run(test_worked_row_w5)
    monkeypatch.setattr(T, "normalize", good_norm)

    good_e2 = O.e2m1_encode
    monkeypatch.setattr(T, "e2m1_encode", lambda v: np.where(
        np.abs(np.asarray(v, F32)) == F32(0.25), np.uint8(1), good_e2(v)).astype(np.uint8))
    assert run(lambda: test_worked_nvfp4_blocks("W2"))
    monkeypatch.setattr(T, "e2m1_encode", good_e2)

    monkeypatch.setattr(O, "sum_of_squares", lambda h: np.array(
        [F32(float(np.sum(np.asarray(r, np.float64) ** 2))) for r in np.asarray(h)], F32))
    assert run(test_sum_of_squares_resolves_float64_midpoints)

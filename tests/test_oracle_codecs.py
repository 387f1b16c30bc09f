"""Pins of the oracle's number formats (oracle/codecs.py) against things other
than itself: torch's own float8_e4m3fn / float16 / bfloat16 conversions, the
closed-form value tables, and brute-force nearest-value search."""
import numpy as np
import pytest
import torch

import oracle as O


def _sweep_f32(max_abs: float) -> np.ndarray:
    """Structured binary32 sweep: every pattern of the top 20 bits below
    max_abs (covers every E4M3/E2M1/fp16/bf16 rounding interval), each with
    low-12-bit tails 0, 1, 0x7FF, 0x800, 0x801, 0xFFF (exact ties, one ulp off
    either side, interior points)."""
    hi = np.arange(0, 1 << 19, dtype=np.uint32) << np.uint32(12)  # sign bit 0
    tails = np.array([0, 1, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    u = (hi[:, None] | tails[None, :]).ravel()
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (f <= max_abs)]
    return np.concatenate([f, -f])


# ---------------------------------------------------------------- E4M3 ------

def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))  # incl. -0


def test_e4m3_decode_closed_form_spots():
    spots = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x64: 48.0, 0x6F: 120.0, 0x72: 160.0, 0x7E: 448.0, 0xFE: -448.0, 0x35: 0.8125}
    for c, v in spots.items():
        assert float(O.e4m3_decode(c)) == v, hex(c)


def test_e4m3_encode_matches_torch_below_max():
    # torch rounds to nearest even and is only compared where it cannot overflow
    f = _sweep_f32(448.0)
    ours = O.e4m3_encode(f)
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(f[i]), hex(ours[i]), hex(ref[i])) for i in bad[:5]]


def test_e4m3_encode_brute_force_nearest():
    rng = np.random.default_rng(11)
    table = O.e4m3_decode(np.arange(256)).astype(np.float64)
    finite = ~np.isnan(table)
    codes = np.arange(256)[finite]
    vals = table[finite]
    # random magnitudes across the whole range, plus every exact midpoint
    a = np.exp2(rng.uniform(-12, 9.5, 4000)) * rng.choice([-1, 1], 4000)
    pos = np.sort(np.unique(vals[vals >= 0]))
    mids = (pos[:-1] + pos[1:]) / 2
    f = np.concatenate([a, mids, -mids, pos, -pos]).astype(np.float32)
    got = O.e4m3_encode(f)
    for v, g in zip(f.astype(np.float64), got):
        if abs(v) >= 448:
            assert g == (0xFE if v < 0 else 0x7E)
            continue
        same_sign = codes[(codes >= 128) == bool(np.signbit(v))]
        d = np.abs(table[same_sign] - v)
        best = same_sign[d == d.min()]
        if len(best) > 1:  # exact tie: the even code (even mantissa)
            best = best[best % 2 == 0]
        assert g == best[0], (v, hex(g), [hex(b) for b in best])


def test_e4m3_saturation_signed_zero_subnormal_ties():
    # (a list, not a dict: 0.0 and -0.0 are equal keys)
    cases = [(448.0, 0x7E), (448.5, 0x7E), (464.0, 0x7E), (480.0, 0x7E), (1e30, 0x7E),
             (-1e30, 0xFE), (0.0, 0x00), (-0.0, 0x80), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (5 * 2.0 ** -10, 0x02), (2.0 ** -9, 0x01), (15 * 2.0 ** -10, 0x08),
             (50.0, 0x64), (49.999996, 0x64), (50.000004, 0x65)]
    for v, c in cases:
        assert int(O.e4m3_encode(np.float32(v))) == c, (v, hex(int(O.e4m3_encode(np.float32(v)))))


def test_e4m3_grid_values_encode_exactly():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    assert np.array_equal(O.e4m3_encode(O.e4m3_decode(codes)), codes)


# ---------------------------------------------------------------- E2M1 ------

def test_e2m1_ties_go_to_even_code():
    # every midpoint of the value set, and the saturation point
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for v, c in ties.items():
        assert int(O.e2m1_encode(np.float32(v))) == c, v
        assert int(O.e2m1_encode(np.float32(-v))) == c | 8, -v
    assert int(O.e2m1_encode(np.float32(6.0))) == 7
    assert int(O.e2m1_encode(np.float32(100.0))) == 7
    assert int(O.e2m1_encode(np.float32(-0.0))) == 8
    assert int(O.e2m1_encode(np.float32(0.0))) == 0


def test_e2m1_brute_force_nearest():
    table = O.e2m1_decode(np.arange(16)).astype(np.float64)
    f = _sweep_f32(8.0)[::7]
    got = O.e2m1_encode(f)
    neg = np.signbit(f)
    for v, g, s in zip(f.astype(np.float64)[:200000], got[:200000], neg[:200000]):
        cand = np.arange(8, 16) if s else np.arange(0, 8)
        if abs(v) >= 6:
            assert g == cand[7]
            continue
        d = np.abs(table[cand] - v)
        best = cand[d == d.min()]
        if len(best) > 1:
            best = best[best % 2 == 0]
        assert g == best[0], (v, g)


def test_e2m1_decode_value_set():
    assert O.e2m1_decode(np.arange(8)).tolist() == [0, .5, 1, 1.5, 2, 3, 4, 6]
    assert O.e2m1_decode(np.arange(9, 16)).tolist() == [-.5, -1, -1.5, -2, -3, -4, -6]


# ------------------------------------------------------------ fp16 / bf16 ---

@pytest.mark.parametrize("dtype,tdt,limit", [("f16", torch.float16, 65504.0),
                                             ("bf16", torch.bfloat16, 3.0e38)])
def test_activation_rounding_matches_torch(dtype, tdt, limit):
    f = _sweep_f32(limit)
    ours = O.t_encode(f, dtype)
    ref = torch.from_numpy(f).to(tdt).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(f[i]), hex(ours[i]), hex(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("dtype,tdt", [("f16", torch.float16), ("bf16", torch.bfloat16)])
def test_activation_decode_matches_torch(dtype, tdt):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.t_decode(b, dtype)
    ref = torch.from_numpy(b.view(np.int16)).view(tdt).to(torch.float32).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin].view(np.uint32), ref[fin].view(np.uint32))

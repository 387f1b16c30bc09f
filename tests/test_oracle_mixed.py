"""Pins of the oracle's partial-width rotation and of its mixed KV-cache store
(FP8 for the part of a K head without position encoding, bf16 for the rotated
part), against things other than the oracle itself:

  * a hand-worked head (tests/golden/worked_rows.json, W6) whose every value
    is exact, so the bytes follow from the definitions by hand;
  * composition from the separately pinned steps (sum of squares, row scale,
    normalize, NeoX rotation, E4M3 and bf16 encoders), head by head;
  * the full-width case equals the whole-head op;
  * the scatter rules of the pool (padding, out-of-range slots, untouched rows);
  * the error bounds of the two stored formats;
  * planted mistakes (rotating the first R elements, pairing across half the
    head, a little-endian slip, an fp16 rope part) each fail a pin.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import oracle.tail as T
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
F32 = np.float32


def _w6():
    with open(os.path.join(HERE, "golden", "worked_rows.json")) as fh:
        return json.load(fh)["W6"]


def _w6_run(w):
    D = w["head_dim"]
    qkv = np.array([w["q_head"] + w["k_head"] + w["v_head"]], np.float32)
    qb = O.t_encode(qkv, "bf16")
    gq = O.t_encode(np.array(w["gamma_q"], np.float32), "bf16")
    gk = O.t_encode(np.array(w["gamma_k"], np.float32), "bf16")
    cs = np.array(w["cos_sin"], np.float32)
    pool = np.full((3, O.mixed_kv_row_bytes(1, 1, D, w["rotary_dim"])), 0xEE, np.uint8)
    return O.qk_norm_rope_kv_store_mixed(qb, gq, gk, np.array([w["position"]]), cs, w["scale"],
                                         w["eps"], 1, 1, 1, D, w["rotary_dim"], "bf16",
                                         np.array([2]), pool)


def test_worked_head_w6():
    w = _w6()
    r = _w6_run(w)
    assert [f"0x{c:02X}" for c in r["q"][0]] == w["expect"]["q_codes"]
    assert r["kv"][2].tobytes().hex() == w["expect"]["pool_row_hex"]
    assert np.all(r["kv"][:2] == 0xEE)                        # rows no token names are untouched


def _composed(inp, R, s):
    """The mixed pool row and Q codes of each token, from the pinned steps."""
    D, nq, nk, nv = inp.head_dim, inp.nq, inp.nk, inp.nv
    N = D - R
    qkv = W.bits(inp.qkv)
    rows, qs = [], []
    for t in range(inp.tokens):
        pos = int(inp.positions[t])
        cos, sin = inp.cos_sin[pos, :R // 2][None], inp.cos_sin[pos, R // 2:][None]
        row, qrow = b"", b""
        for hd in range(nq + nk + nv):
            u = O.t_decode(qkv[t, hd * D:(hd + 1) * D], inp.dtype)[None, :]
            if hd < nq + nk:
                g = W.bits(inp.gamma_q if hd < nq else inp.gamma_k)
                r = O.row_scale(O.sum_of_squares(u), D, inp.eps)
                n = O.normalize(u, r, O.t_decode(g, inp.dtype))
                rot = O.rope_neox(n[:, N:], cos, sin)
                o = np.concatenate([n[:, :N], rot], axis=1)
                if hd < nq:
                    qrow += O.e4m3_encode(o / F32(s))[0].tobytes()
                else:
                    row += O.e4m3_encode(n[:, :N] / F32(s))[0].tobytes()
                    row += O.t_encode(rot, "bf16")[0].astype("<u2").tobytes()
            else:
                row += O.e4m3_encode(u / F32(s))[0].tobytes()
        rows.append(row)
        qs.append(qrow)
    return qs, rows


@pytest.mark.parametrize("D,R", [(32, 16), (64, 32), (128, 64), (128, 16), (256, 64), (64, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_mixed_store_is_the_composition_of_the_pinned_steps(D, R, dtype):
    pos = np.array([0, 5, 2, 9, 1])
    inp = W.make_qk(40 + D + R, dtype, 5, 2, 2, 1, D, positions=pos, max_pos=12, rotary_dim=R,
                    scale=0.04)
    slots = np.array([3, 0, 6, 1, 4])
    rb = O.mixed_kv_row_bytes(2, 1, D, R)
    r = O.qk_norm_rope_kv_store_mixed(W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k),
                                      pos, inp.cos_sin, inp.scale, inp.eps, 2, 2, 1, D, R, dtype,
                                      slots, np.zeros((7, rb), np.uint8))
    qs, rows = _composed(inp, R, inp.scale)
    for t in range(5):
        assert r["q"][t].tobytes() == qs[t], t
        assert r["kv"][slots[t]].tobytes() == rows[t], t
    assert np.all(r["kv"][[2, 5]] == 0)


@pytest.mark.parametrize("D", [32, 128])
def test_partial_rotation_at_full_width_is_the_whole_head_op(D):
    inp = W.make_qk(9, "bf16", 4, 2, 1, 1, D, positions=np.array([3, 0, 7, 1]), max_pos=8)
    args = (W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
            inp.cos_sin, inp.scale, inp.eps, 2, 1, 1, D, "bf16")
    a, b = O.qk_norm_rope_fp8(*args), O.qk_norm_rope_fp8(*args, rotary_dim=D)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["o"], b["o"])


def test_partial_rotation_leaves_the_leading_part_unrotated():
    """With R < D the first D-R elements of a Q/K head are its normed values at
    every position, and the last R are the R-wide rotation of theirs."""
    D, R = 64, 16
    inp = W.make_qk(11, "bf16", 6, 1, 1, 0, D, positions=np.arange(6), max_pos=6, rotary_dim=R)
    args = (W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
            inp.cos_sin, inp.scale, inp.eps, 1, 1, 0, D, "bf16")
    o = O.qk_norm_rope_fp8(*args, rotary_dim=R)["o"].reshape(6, 2, D)
    o0 = O.qk_norm_rope_fp8(*args[:4], np.tile(np.r_[np.ones(R // 2), np.zeros(R // 2)],
                                                (6, 1)).astype(np.float32),
                            *args[5:], rotary_dim=R)["o"].reshape(6, 2, D)   # angle 0 everywhere
    assert np.array_equal(o[..., :D - R], o0[..., :D - R])
    assert not np.array_equal(o[1:, :, D - R:], o0[1:, :, D - R:])
    for t in range(6):
        rot = O.rope_neox(o0[t, :, D - R:], inp.cos_sin[t, :R // 2][None], inp.cos_sin[t, R // 2:][None])
        assert np.array_equal(o[t, :, D - R:], rot)


def test_mixed_store_error_bounds():
    """Decoded FP8 codes are within half an E4M3 step of o / s (the unrotated
    part, where |o/s| <= 448) and decoded bf16 values within half a bf16 ulp of o."""
    D, R, s = 128, 64, 0.05
    inp = W.make_qk(12, "bf16", 16, 0, 3, 0, D, positions=np.arange(16), max_pos=16, rotary_dim=R,
                    scale=s)
    rb = O.mixed_kv_row_bytes(3, 0, D, R)
    r = O.qk_norm_rope_kv_store_mixed(W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k),
                                      inp.positions.numpy(), inp.cos_sin, s, inp.eps, 0, 3, 0, D, R,
                                      "bf16", np.arange(16), np.zeros((16, rb), np.uint8))
    o = r["o"].reshape(16, 3, D).astype(np.float64)
    kv = r["kv"].reshape(16, 3, D - R + 2 * R)
    nope = O.e4m3_decode(kv[..., :D - R]).astype(np.float64)
    v = o[..., :D - R] / s
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) - 3)   # E4M3 step at |v|
    assert np.all(np.abs(nope - v) <= step / 2)
    rope = O.t_decode(kv[..., D - R:].copy().view("<u2"), "bf16").astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(o[..., D - R:]), 2.0 ** -126))) - 7)
    assert np.all(np.abs(rope - o[..., D - R:]) <= ulp / 2)


def test_mixed_store_scatter_rules():
    D, R = 32, 16
    inp = W.make_qk(13, "f16", 5, 1, 1, 1, D, rotary_dim=R)
    rb = O.mixed_kv_row_bytes(1, 1, D, R)
    args = (W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
            inp.cos_sin, inp.scale, inp.eps, 1, 1, 1, D, R, "f16")
    ident = O.qk_norm_rope_kv_store_mixed(*args, np.arange(5), np.zeros((5, rb), np.uint8))["kv"]
    pool = np.full((8, rb), 0xAB, np.uint8)
    slots = np.array([6, -1, 0, 8, 3])
    r = O.qk_norm_rope_kv_store_mixed(*args, slots, pool)
    written = {6: 0, 0: 2, 3: 4}
    for row in range(8):
        want = ident[written[row]] if row in written else pool[row]
        assert np.array_equal(r["kv"][row], want), row
    assert np.all(pool == 0xAB)                                  # the input pool is not modified


def _planted_qk(where: str):
    """The Q/K op with one slip in the rotation: where = "first" rotates the
    first R elements of a head instead of the last R; "half_head" pairs
    element k with k + D/2 of the whole head (the full-width pairing)."""
    def f(qkv_bits, gq, gk, positions, cos_sin, scale, eps, nq, nk, nv, D, dtype, rotary_dim=None):
        R = D if rotary_dim is None else rotary_dim
        tokens = qkv_bits.shape[0]
        u = O.t_decode(qkv_bits, dtype).reshape(tokens, nq + nk + nv, D)
        tab = np.asarray(cos_sin, np.float32)[np.asarray(positions)]
        o = u.copy()
        for lo, hi, g in ((0, nq, gq), (nq, nq + nk, gk)):
            for h in range(lo, hi):
                n = O.normalize(u[:, h], O.row_scale(O.sum_of_squares(u[:, h]), D, eps),
                                O.t_decode(g, dtype))
                o[:, h] = n
                if where == "first":
                    o[:, h, :R] = O.rope_neox(n[:, :R], tab[:, :R // 2], tab[:, R // 2:])
                else:
                    c = np.tile(tab[:, :R // 2], (1, D // R))
                    s_ = np.tile(tab[:, R // 2:], (1, D // R))
                    o[:, h] = O.rope_neox(n, c, s_)
        o = o.reshape(tokens, -1)
        return dict(out=O.e4m3_encode(o / F32(scale)), o=o)
    return f


def test_pins_catch_planted_mistakes(monkeypatch):
    """Each plausible slip in the mixed store's definition fails the W6 pin."""
    def w6_fails():
        try:
            test_worked_head_w6()
        except AssertionError:
            return True
        return False

    assert not w6_fails()
    good_qk, good_enc = T.qk_norm_rope_fp8, T.t_encode
    for where in ("first", "half_head"):
        monkeypatch.setattr(T, "qk_norm_rope_fp8", _planted_qk(where))
        assert w6_fails(), where
    monkeypatch.setattr(T, "qk_norm_rope_fp8", good_qk)
    # bf16 bytes stored big endian; the rotated part stored as fp16
    monkeypatch.setattr(T, "t_encode",
                        lambda f, d: good_enc(f, d).byteswap() if d == "bf16" else good_enc(f, d))
    assert w6_fails()
    monkeypatch.setattr(T, "t_encode", lambda f, d: good_enc(f, "f16") if d == "bf16" else good_enc(f, d))
    assert w6_fails()
    monkeypatch.setattr(T, "t_encode", good_enc)
    assert not w6_fails()

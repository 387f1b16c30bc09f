"""Seeded random shapes for every op, against the oracle, bit for bit.

Hidden sizes are drawn from all multiples of 16 up to 65536, so lane mappings,
vector counts that are not multiples of a wavefront and ragged last vectors
appear that a hand-picked grid can miss. Token counts are small (1-9, and up
to 300 where the swizzled scale padding matters), and both input types and
both epilogues occur. The Q/K op gets random head layouts and head sizes (and
random rotary widths through the mixed KV pool), and the gated op random group
widths, with the bf16 gate table forced on for half
of its cases. The seed is fixed, so every case is reproducible and named by
its id.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np, gpu_qk, gpu_tail, oracle_global_scale, oracle_qk, oracle_tail

pytestmark = pytest.mark.gpu

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _A():
    import nvfp4_quantization_place_amd as A
    return A


def _hidden(rng, small: bool) -> int:
    return 16 * int(rng.integers(1, 65) if small else rng.integers(65, 4097))


def _tail_cases(n=48):
    rng = np.random.default_rng(20261202)
    out = []
    for i in range(n):
        op = ("fp8", "nvfp4")[i % 2]
        dtype = ("f16", "bf16")[(i // 2) % 2]
        out.append((i, op, dtype, int(rng.integers(1, 10)), _hidden(rng, i % 3 != 2),
                    bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _tail_cases(),
                         ids=lambda c: f"{c[1]}-{c[2]}-{c[3]}x{c[4]}{'-norm' if c[5] else ''}")
def test_random_tail_shapes(case):
    i, op, dtype, tokens, hidden, norm = case
    inp = W.make_tail(7000 + i, op, dtype, tokens, hidden, norm_out=norm,
                      scale=0.03 if op == "fp8" else None, outliers=0.002)
    scale = float(inp.scale) if op == "fp8" else float(oracle_global_scale(inp))
    got = gpu_tail(inp, scale)
    ref = oracle_tail(inp, scale)
    np.testing.assert_array_equal(got["residual"], ref["residual"])
    np.testing.assert_array_equal(got["q"], ref["q"])
    if op == "nvfp4":
        np.testing.assert_array_equal(got["sf"], ref["sf"])
    if norm:
        np.testing.assert_array_equal(got["norm_out"], ref["norm_out"])


def _qk_cases(n=24):
    rng = np.random.default_rng(31337)
    out = []
    for i in range(n):
        head_dim = int(rng.choice([32, 64, 128, 256, 512]))
        nq, nk, nv = (int(v) for v in rng.integers(0, (7, 4, 4)))
        if nq + nk + nv == 0:
            nq = 1
        out.append((i, ("f16", "bf16")[i % 2], int(rng.integers(1, 10)), nq, nk, nv, head_dim))
    return out


@pytest.mark.parametrize("case", _qk_cases(),
                         ids=lambda c: f"{c[1]}-t{c[2]}-q{c[3]}k{c[4]}v{c[5]}-d{c[6]}")
def test_random_qk_shapes(case):
    i, dtype, tokens, nq, nk, nv, head_dim = case
    rng = np.random.default_rng(100 + i)
    inp = W.make_qk(8000 + i, dtype, tokens, nq, nk, nv, head_dim,
                    positions=rng.integers(0, 97, tokens), max_pos=97, scale=0.04)
    np.testing.assert_array_equal(gpu_qk(inp), oracle_qk(inp))


def _mixed_cases(n=24):
    rng = np.random.default_rng(5151)
    out = []
    for i in range(n):
        D = int(rng.choice([32, 64, 128, 256, 512]))
        R = int(rng.choice([r for r in (16, 32, 64, 128, 256, 512) if r <= D]))
        nq, nk, nv = int(rng.integers(0, 6)), int(rng.integers(0, 4)), int(rng.integers(0, 4))
        if nk + nv == 0:
            nk = 1
        out.append((i, ("f16", "bf16")[i % 2], int(rng.integers(1, 40)), nq, nk, nv, D, R))
    return out


@pytest.mark.parametrize("case", _mixed_cases(),
                         ids=lambda c: f"{c[1]}-{c[2]}tok-{c[3]}.{c[4]}.{c[5]}x{c[6]}-rot{c[7]}")
def test_random_qk_mixed_pool(case):
    """Random head sizes, rotary widths and head layouts through the mixed
    pool store, with padding and past-the-pool slots."""
    i, dtype, tokens, nq, nk, nv, D, R = case
    rng = np.random.default_rng(300 + i)
    inp = W.make_qk(8500 + i, dtype, tokens, nq, nk, nv, D, positions=rng.integers(0, 97, tokens),
                    max_pos=97, rotary_dim=R, scale=0.04)
    num_slots = tokens + int(rng.integers(0, 8))
    slots = rng.permutation(num_slots)[:tokens].astype(np.int64)
    slots[rng.random(tokens) < 0.15] = -1
    slots[rng.random(tokens) < 0.05] = num_slots + 3
    A = _A()
    width = A.mixed_kv_row_bytes(nk, nv, D, R)
    pool = torch.full((num_slots, width), 0x5A, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_kv_store_mixed(inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(),
                                      inp.positions.cuda(), torch.from_numpy(inp.cos_sin).cuda(),
                                      torch.tensor([inp.scale], device="cuda"), inp.eps, nq, nk,
                                      nv, D, R, torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope_kv_store_mixed(W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k),
                                        inp.positions.numpy(), inp.cos_sin, inp.scale, inp.eps, nq,
                                        nk, nv, D, R, dtype, slots,
                                        np.full((num_slots, width), 0x5A, np.uint8))
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(pool), ref["kv"])


def _gated_cases(n=24):
    rng = np.random.default_rng(4242)
    out = []
    for i in range(n):
        group = 16 * int(rng.integers(1, 65)) if i % 4 else int(rng.choice([2048, 4096]))
        ngroups = int(rng.integers(1, 5))
        dtype = ("f16", "bf16")[i % 2]
        table = dtype == "bf16" and group <= 1024 and (i // 2) % 2 == 1
        out.append((i, dtype, int(rng.integers(1, 10)), group * ngroups, group, table))
    return out


@pytest.mark.parametrize("case", _gated_cases(),
                         ids=lambda c: f"{c[1]}-{c[2]}x{c[3]}-g{c[4]}{'-table' if c[5] else ''}")
def test_random_gated_shapes(case, monkeypatch):
    i, dtype, tokens, hidden, group, table = case
    monkeypatch.setenv("ANQ_GATE_LUT", "1" if table else "")
    inp = W.make_gated(9000 + i, dtype, tokens, hidden, group, z=("normal", 3.0), eps=1e-5)
    xb, zb, gb = W.bits(inp.x), W.bits(inp.residual), W.bits(inp.gamma)
    G = float(O.nvfp4_global_scale(
        O.gated_rmsnorm_quant_nvfp4(xb, zb, gb, dtype, group, 1.0, inp.eps)["n"]))
    q, sf = _A().gated_rmsnorm_quant_nvfp4(inp.x.cuda(), inp.residual.cuda(), inp.gamma.cuda(),
                                           torch.tensor([G], device="cuda"), inp.eps, group=group)
    torch.cuda.synchronize()
    ref = O.gated_rmsnorm_quant_nvfp4(xb, zb, gb, dtype, group, G, inp.eps)
    np.testing.assert_array_equal(_np(sf), ref["sf"])
    np.testing.assert_array_equal(_np(q), ref["q"])


def _swizzled_cases(n=12):
    rng = np.random.default_rng(777)
    return [(i, ("f16", "bf16")[i % 2], int(rng.integers(1, 301)), _hidden(rng, i % 2 == 0))
            for i in range(n)]


@pytest.mark.parametrize("case", _swizzled_cases(), ids=lambda c: f"{c[1]}-{c[2]}x{c[3]}")
def test_random_swizzled_shapes(case):
    i, dtype, tokens, hidden = case
    inp = W.make_tail(9500 + i, "nvfp4", dtype, tokens, hidden, scale=None)
    G = float(oracle_global_scale(inp))
    A = _A()
    r, c = A.nvfp4_swizzled_sf_shape(tokens, hidden)
    sf = torch.full((r, c), 0xFF, dtype=torch.uint8, device="cuda")
    res = inp.residual.cuda()
    q, sf, _ = A.add_rmsnorm_quant_nvfp4_swizzled(inp.x.cuda(), res, inp.gamma.cuda(),
                                                  torch.tensor([G], device="cuda"), inp.eps, sf=sf)
    torch.cuda.synchronize()
    ref = oracle_tail(inp, G)
    np.testing.assert_array_equal(_np(res), ref["residual"])
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(sf), O.swizzle_block_scales(ref["sf"]))


def _qk_many_token_cases(n=4):
    rng = np.random.default_rng(909)
    out = []
    for i in range(n):
        head_dim = int(rng.choice([64, 128, 256]))
        nq, nk, nv = int(rng.integers(1, 40)), int(rng.integers(0, 9)), int(rng.integers(0, 9))
        out.append((i, ("bf16", "f16")[i % 2], int(rng.integers(2048, 4097)), nq, nk, nv, head_dim))
    return out


@pytest.mark.parametrize("case", _qk_many_token_cases(),
                         ids=lambda c: f"{c[1]}-t{c[2]}-q{c[3]}k{c[4]}v{c[5]}-d{c[6]}")
def test_random_qk_many_tokens(case):
    """Enough tokens for one wavefront per token, so each wavefront loads
    several head groups at once (the launcher's default path at scale), with
    random head layouts and positions across an 8192-entry table."""
    i, dtype, tokens, nq, nk, nv, head_dim = case
    rng = np.random.default_rng(300 + i)
    inp = W.make_qk(700 + i, dtype, tokens, nq, nk, nv, head_dim,
                    positions=rng.integers(0, 8192, tokens), max_pos=8192, scale=0.05)
    np.testing.assert_array_equal(gpu_qk(inp), oracle_qk(inp))

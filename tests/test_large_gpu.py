"""Calls whose tensors pass 4 GiB, so every row, token and code offset past
2^32 bytes must be computed in 64 bits. The inputs are a seeded block of
1000 rows (or tokens) repeated down the tensor; 1000 does not divide 2^18
or 2^19, so a row address truncated to 32 bits would read or write a row
whose data differs. Outputs start poisoned and are checked on rows around
the 2^32-byte boundaries, the last rows and a seeded sample, against the
oracle run on the block rows they repeat."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np

pytestmark = pytest.mark.gpu

BLOCK = 1000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _A():
    import nvfp4_quantization_place_amd as A
    return A


def _tile(t, rows):
    """rows x t.shape[1] on the GPU: t (on the host) repeated, then cut."""
    reps = -(-rows // t.shape[0])
    return t.cuda().repeat(reps, 1)[:rows].contiguous()


def _rows(n, row_bytes, seed):
    """Rows on both sides of each 2^32-byte boundary of an n-row tensor, the
    last rows and a seeded sample."""
    picks = [0, 1, n - 2, n - 1]
    for k in range(1, 4):
        b = (k << 32) // row_bytes
        picks += [b - 1, b, b + 1]
    picks += list(np.random.default_rng(seed).choice(n, 24))
    return np.unique(np.array([p for p in picks if 0 <= p < n], np.int64))


@pytest.mark.parametrize("op", ["fp8", "nvfp4"])
def test_tail_past_4gib(op):
    H, M = 8192, 270_000                      # x and residual 4.4 GB each
    blk = W.make_tail(910, op, "bf16", BLOCK, H, scale=0.02 if op == "fp8" else None,
                      outliers=0.002)
    scale = 0.02 if op == "fp8" else float(O.nvfp4_global_scale(
        O.rmsnorm_f32(W.bits(blk.x), W.bits(blk.residual), W.bits(blk.gamma), "bf16", blk.eps)))
    A = _A()
    x, res = _tile(blk.x, M), _tile(blk.residual, M)
    s = torch.tensor([scale], device="cuda")
    if op == "fp8":
        q = torch.full((M, H), 0xEE, dtype=torch.uint8, device="cuda")
        A.add_rmsnorm_quant_fp8(x, res, blk.gamma.cuda(), s, blk.eps, q=q)
        sf = None
    else:
        q = torch.full((M, H // 2), 0xEE, dtype=torch.uint8, device="cuda")
        sf = torch.full((M, H // 16), 0xEE, dtype=torch.uint8, device="cuda")
        A.add_rmsnorm_quant_nvfp4(x, res, blk.gamma.cuda(), s, blk.eps, q=q, sf=sf)
    torch.cuda.synchronize()
    rows = _rows(M, H * 2, 7)
    src = rows % BLOCK
    ref = (O.add_rmsnorm_quant_fp8 if op == "fp8" else O.add_rmsnorm_quant_nvfp4)(
        W.bits(blk.x)[src], W.bits(blk.residual)[src], W.bits(blk.gamma), "bf16", scale,
        blk.eps, False)
    idx = torch.from_numpy(rows).cuda()
    np.testing.assert_array_equal(_np(res.index_select(0, idx)), ref["residual"])
    np.testing.assert_array_equal(_np(q.index_select(0, idx)), ref["q"])
    if sf is not None:
        np.testing.assert_array_equal(_np(sf.index_select(0, idx)), ref["sf"])


def test_gated_past_4gib():
    H, group, M = 8192, 1024, 270_000         # x and z 4.4 GB each, the gate-table tiling
    blk = W.make_gated(911, "bf16", BLOCK, H, group)
    G = 100.0
    A = _A()
    x, z = _tile(blk.x, M), _tile(blk.residual, M)
    q = torch.full((M, H // 2), 0xEE, dtype=torch.uint8, device="cuda")
    sf = torch.full((M, H // 16), 0xEE, dtype=torch.uint8, device="cuda")
    A.gated_rmsnorm_quant_nvfp4(x, z, blk.gamma.cuda(), torch.tensor([G], device="cuda"),
                                blk.eps, group=group, q=q, sf=sf)
    torch.cuda.synchronize()
    rows = _rows(M, H * 2, 8)
    src = rows % BLOCK
    ref = O.gated_rmsnorm_quant_nvfp4(W.bits(blk.x)[src], W.bits(blk.residual)[src],
                                      W.bits(blk.gamma), "bf16", group, G, blk.eps)
    idx = torch.from_numpy(rows).cuda()
    np.testing.assert_array_equal(_np(q.index_select(0, idx)), ref["q"])
    np.testing.assert_array_equal(_np(sf.index_select(0, idx)), ref["sf"])


def test_qk_past_4gib():
    nq, nk, nv, D, T = 16, 8, 8, 128, 540_000  # qkv 4.4 GB, codes 2.2 GB
    blk = W.make_qk(912, "bf16", BLOCK, nq, nk, nv, D, scale=0.05)
    A = _A()
    qkv = _tile(blk.qkv, T)
    pos = torch.from_numpy(np.arange(T, dtype=np.int64) % BLOCK).cuda()
    out = torch.full((T, (nq + nk + nv) * D), 0xEE, dtype=torch.uint8, device="cuda")
    A.qk_norm_rope_fp8(qkv, blk.gamma_q.cuda(), blk.gamma_k.cuda(), pos,
                       torch.from_numpy(blk.cos_sin).cuda(), torch.tensor([blk.scale], device="cuda"),
                       blk.eps, nq, nk, nv, D, out=out)
    torch.cuda.synchronize()
    rows = _rows(T, (nq + nk + nv) * D * 2, 9)
    src = rows % BLOCK
    ref = O.qk_norm_rope_fp8(W.bits(blk.qkv)[src], W.bits(blk.gamma_q), W.bits(blk.gamma_k),
                             blk.positions.numpy()[src], blk.cos_sin, blk.scale, blk.eps, nq, nk, nv,
                             D, "bf16")
    np.testing.assert_array_equal(_np(out.index_select(0, torch.from_numpy(rows).cuda())),
                                  ref["out"])

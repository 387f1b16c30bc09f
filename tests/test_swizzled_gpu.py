"""GPU parity of the NVFP4 ops with the swizzled (128x4-tiled) block-scale
layout: the scales are the oracle's, placed by the oracle's swizzle, and every
padding byte is zero (the output buffers start filled with 0xFF). Codes,
residual and norm output equal the linear-layout op's."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np, oracle_global_scale, oracle_tail

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _A():
    import nvfp4_quantization_place_amd as A
    return A


def _poisoned_sf(tokens, hidden):
    r, c = _A().nvfp4_swizzled_sf_shape(tokens, hidden)
    return torch.full((r, c), 0xFF, dtype=torch.uint8, device="cuda")


SHAPES = [(1, 16), (5, 48), (7, 400), (9, 512), (37, 1040), (128, 7168), (129, 1024), (300, 2048),
          (64, 8192), (3, 16400), (2, 40976), (3, 65520),
          (1030, 7168)]  # 14 wavefronts padded to 16: lanes past the row gather zero codes


@pytest.mark.parametrize("tokens,hidden", SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fused_swizzled(tokens, hidden, dtype):
    inp = W.make_tail(hidden + tokens, "nvfp4", dtype, tokens, hidden, norm_out=True, scale=None)
    G = float(oracle_global_scale(inp))
    A = _A()
    res = inp.residual.cuda()
    sf = _poisoned_sf(tokens, hidden)
    q, sf, norm = A.add_rmsnorm_quant_nvfp4_swizzled(inp.x.cuda(), res, inp.gamma.cuda(),
                                                     torch.tensor([G], device="cuda"), inp.eps,
                                                     norm_out=True, sf=sf)
    torch.cuda.synchronize()
    ref = oracle_tail(inp, G)
    np.testing.assert_array_equal(_np(res), ref["residual"])
    np.testing.assert_array_equal(_np(norm), ref["norm_out"])
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(sf), O.swizzle_block_scales(ref["sf"]))


@pytest.mark.parametrize("hidden,tiling,rows", [
    (112, "16:1", "1"), (256, "32:1", "3"), (400, "64:1", "2"), (512, "64:1", "1"),
    (1008, "64:2", "2"), (1040, "0:1", "1"), (1040, "0:2", "5"), (1040, "0:4", "64"),
    (400, "0:1", "3")])
@pytest.mark.parametrize("order", ["0", "1"])
def test_fused_swizzled_every_tiling(hidden, tiling, rows, order, monkeypatch):
    """Padded rows are shared among however many lane groups the tiling
    launches; every lane-group width gathers the four codes of a scale word.
    Each override names a tiling that exists for its row width (others are
    refused with ANQ_ERR_CONFIG, never replaced)."""
    monkeypatch.setenv("ANQ_TAIL_TILING", tiling)
    monkeypatch.setenv("ANQ_ROWS_PER_GROUP", rows)
    monkeypatch.setenv("ANQ_ROW_ORDER", order)
    inp = W.make_tail(77, "nvfp4", "bf16", 45, hidden, norm_out=False, scale=None)
    G = float(oracle_global_scale(inp))
    sf = _poisoned_sf(45, hidden)
    q, sf, _ = _A().add_rmsnorm_quant_nvfp4_swizzled(inp.x.cuda(), inp.residual.cuda(),
                                                     inp.gamma.cuda(),
                                                     torch.tensor([G], device="cuda"), inp.eps,
                                                     sf=sf)
    torch.cuda.synchronize()
    ref = oracle_tail(inp, G)
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(sf), O.swizzle_block_scales(ref["sf"]))


@pytest.mark.parametrize("tokens,hidden", SHAPES + [(0, 64), (1000, 112)])
@pytest.mark.parametrize("stream_hint", ["0", "1"])
def test_quant_swizzled(tokens, hidden, stream_hint, monkeypatch):
    monkeypatch.setenv("ANQ_STREAM", stream_hint)
    t = W.to_dtype(2.0 * W.normal(5, tokens + hidden, tokens * hidden), "f16").reshape(tokens, hidden)
    sf = _poisoned_sf(tokens, hidden)
    q, sf = _A().quant_nvfp4_swizzled(t.cuda(), torch.tensor([150.0], device="cuda"), sf=sf)
    torch.cuda.synchronize()
    rq, rsf = O.quant_nvfp4(O.t_decode(W.bits(t), "f16").reshape(tokens, hidden), 150.0)
    np.testing.assert_array_equal(_np(q), rq)
    np.testing.assert_array_equal(_np(sf), O.swizzle_block_scales(rsf))


def test_swizzled_at_the_nvfp4_workload_size():
    """bf16 [8192, 7168] with norm out: the swizzled scales are the linear op's
    scales placed by the swizzle; codes identical (GPU against GPU), and the
    oracle checks a sample of rows."""
    inp = W.make_config(4)
    print(f"workload {inp.name} swizzled", flush=True)
    G = float(oracle_global_scale(inp))
    A = _A()
    g = torch.tensor([G], device="cuda")
    q1, sf1, n1 = A.add_rmsnorm_quant_nvfp4(inp.x.cuda(), inp.residual.cuda(), inp.gamma.cuda(), g,
                                            inp.eps, norm_out=True)
    q2, sf2, n2 = A.add_rmsnorm_quant_nvfp4_swizzled(inp.x.cuda(), inp.residual.cuda(),
                                                     inp.gamma.cuda(), g, inp.eps, norm_out=True,
                                                     sf=_poisoned_sf(inp.tokens, inp.hidden))
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(n1, n2)
    lin = _np(sf1)
    np.testing.assert_array_equal(_np(sf2), O.swizzle_block_scales(lin))
    rows = np.random.default_rng(4).choice(inp.tokens, 24, replace=False)
    ref = oracle_tail(inp, G, rows)
    np.testing.assert_array_equal(lin[rows], ref["sf"])

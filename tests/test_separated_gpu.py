"""GPU parity of the separated local tail (add_rmsnorm, then quant_fp8 or
quant_nvfp4) and of the standalone quantisers, against the CPU oracle.

The separated path quantises the norm output after it has been rounded to T
(TensorRT-LLM issue #17900, Proposal: a residual/RMSNorm kernel writes the
normalised activations, a second kernel quantises them), so its reference is
the oracle's quantiser applied to the oracle's T-rounded norm output. Every
output is compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np, oracle_global_scale

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


def _dev_scalar(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def _from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(TORCH_DT[dtype])


def _finite_patterns(dtype: str) -> np.ndarray:
    """Every finite 16-bit pattern of T (NaN and infinities excluded: the
    quantisers are specified for finite activations)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[np.isfinite(O.t_decode(b, dtype))]


# ------------------------------------------------------------ add_rmsnorm


@pytest.mark.parametrize("hidden", [16, 128, 1040, 7168, 8192, 16400, 65536])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_add_rmsnorm_matches_oracle(hidden, dtype):
    tokens = max(3, min(300, (1 << 20) // hidden)) | 1     # several tiles and a ragged tail
    inp = W.make_tail(71, "fp8", dtype, tokens, hidden, norm_out=True)
    A = _A()
    x, res, g = inp.x.cuda(), inp.residual.cuda(), inp.gamma.cuda()
    norm = A.add_rmsnorm(x, res, g, inp.eps)
    torch.cuda.synchronize()
    ref = O.add_rmsnorm_quant_fp8(W.bits(inp.x), W.bits(inp.residual), W.bits(inp.gamma), dtype,
                                  1.0, inp.eps, True)
    np.testing.assert_array_equal(_np(res), ref["residual"])
    np.testing.assert_array_equal(_np(norm), ref["norm_out"])


def test_add_rmsnorm_equals_fused_norm_out():
    """The unfused first kernel and the fused kernels agree on residual and norm output."""
    A = _A()
    inp = W.make_tail(72, "nvfp4", "bf16", 257, 7168, norm_out=True)
    r1 = inp.residual.cuda()
    norm1 = A.add_rmsnorm(inp.x.cuda(), r1, inp.gamma.cuda(), inp.eps)
    r2 = inp.residual.cuda()
    _, _, norm2 = A.add_rmsnorm_quant_nvfp4(inp.x.cuda(), r2, inp.gamma.cuda(), _dev_scalar(400.0),
                                            inp.eps, norm_out=True)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2) and torch.equal(norm1, norm2)


# ------------------------------------------------------------ standalone quantisers


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.02, 3.0e-3, 7.5])
def test_quant_fp8_every_finite_input(dtype, scale):
    b = _finite_patterns(dtype)
    hidden = 64
    b = np.concatenate([b, np.zeros((-len(b)) % hidden, np.uint16)]).reshape(-1, hidden)
    q = _A().quant_fp8(_from_bits(b, dtype).cuda(), _dev_scalar(scale))
    ref = O.quant_fp8(O.t_decode(b, dtype), scale)
    np.testing.assert_array_equal(_np(q), ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("gscale", [1.0, 499.2738, 2.5e-2, 3.0e4])
def test_quant_nvfp4_every_finite_input(dtype, gscale):
    """Each finite pattern appears in a block with 15 seeded neighbours, so every
    value meets many block scales; rows of zeros cover the S = 0 block."""
    b = _finite_patterns(dtype)
    rng = np.random.default_rng(5)
    rng.shuffle(b)
    hidden = 256
    pad = (-len(b)) % hidden
    b = np.concatenate([b, np.zeros(pad + 2 * hidden, np.uint16)]).reshape(-1, hidden)
    q, sf = _A().quant_nvfp4(_from_bits(b, dtype).cuda(), _dev_scalar(gscale))
    rq, rsf = O.quant_nvfp4(O.t_decode(b, dtype), gscale)
    np.testing.assert_array_equal(_np(sf), rsf)
    np.testing.assert_array_equal(_np(q), rq)


@pytest.mark.parametrize("gscale", [2.0 ** 118, 1.5 * 2.0 ** 118, 1.1875 * 2.0 ** 118,
                                    float.fromhex("0x1.fffffep118")])
def test_quant_nvfp4_tiny_blocks_huge_global_scale(gscale):
    """Blocks whose every |value| is below 2^-125 (bf16 subnormals and the
    lowest normal binade), under global scales large enough that the last ulp
    of amax / 6, a subnormal binary32, decides the block-scale code (G stays
    below 2^119, so every multiplier G / value(sf) is finite). Each such
    value is the amax of one block of zeros and of one block of smaller tiny
    values, so every subnormal quotient the input can give is met."""
    b = _finite_patterns("bf16")
    mag = np.abs(O.t_decode(b, "bf16"))
    tiny = b[(mag > 0) & (mag < 2.0 ** -125)]
    tmag = np.abs(O.t_decode(tiny, "bf16"))
    rng = np.random.default_rng(29)
    blocks = []
    for lead, m in zip(tiny, tmag):
        blocks.append(np.concatenate([[lead], np.zeros(15, np.uint16)]))
        pool = tiny[tmag <= m]
        blk = rng.choice(pool, 16)
        blk[rng.integers(16)] = lead
        blocks.append(blk)
    hidden = 256
    flat = np.concatenate(blocks).astype(np.uint16)
    flat = np.concatenate([flat, np.zeros((-len(flat)) % hidden, np.uint16)]).reshape(-1, hidden)
    q, sf = _A().quant_nvfp4(_from_bits(flat, "bf16").cuda(), _dev_scalar(gscale))
    rq, rsf = O.quant_nvfp4(O.t_decode(flat, "bf16"), gscale)
    np.testing.assert_array_equal(_np(sf), rsf)
    np.testing.assert_array_equal(_np(q), rq)
    assert np.any(rsf != 0)                       # the scale codes are not all zero


def test_fused_nvfp4_tiny_norm_huge_global_scale():
    """The fused op with gamma in bf16's subnormal range: every n is below
    2^-125, and the largest allowed G (just below 2^119) makes the subnormal
    amax / 6 decide the scale code."""
    A = _A()
    rng = np.random.default_rng(31)
    H = 1024
    x = W.to_dtype(rng.standard_normal((9, H)), "bf16")
    res = W.to_dtype(rng.standard_normal((9, H)), "bf16")
    g = W.to_dtype(rng.uniform(2.0 ** -133, 2.0 ** -127, H), "bf16")
    G = float.fromhex("0x1.fffffep118")
    rc = res.cuda()
    q, sf, _ = A.add_rmsnorm_quant_nvfp4(x.cuda(), rc, g.cuda(), _dev_scalar(G), 1e-6)
    torch.cuda.synchronize()
    ref = O.add_rmsnorm_quant_nvfp4(W.bits(x), W.bits(res), W.bits(g), "bf16", G, 1e-6, False)
    assert np.all(np.abs(ref["n"]) < 2.0 ** -125) and np.any(ref["sf"] != 0)
    np.testing.assert_array_equal(_np(rc), ref["residual"])
    np.testing.assert_array_equal(_np(sf), ref["sf"])
    np.testing.assert_array_equal(_np(q), ref["q"])


@pytest.mark.parametrize("op", ["fp8", "nvfp4"])
@pytest.mark.parametrize("tokens,hidden", [(0, 128), (1, 16), (3, 48), (37, 1040), (513, 7168)])
@pytest.mark.parametrize("stream_hint", ["0", "1"])
def test_quant_shapes_and_stream_hint(op, tokens, hidden, stream_hint, monkeypatch):
    """Ragged vector counts (not a multiple of the 256-thread block), a row of one
    block, no rows, both load forms."""
    monkeypatch.setenv("ANQ_STREAM", stream_hint)
    n64 = W.normal(91, tokens * 7 + hidden, tokens * hidden).reshape(tokens, hidden) * 3.0
    t = W.to_dtype(n64, "bf16")
    b = W.bits(t)
    A = _A()
    if op == "fp8":
        q = A.quant_fp8(t.cuda(), _dev_scalar(0.05))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_np(q), O.quant_fp8(O.t_decode(b, "bf16"), 0.05))
    else:
        q, sf = A.quant_nvfp4(t.cuda(), _dev_scalar(60.0))
        torch.cuda.synchronize()
        rq, rsf = O.quant_nvfp4(O.t_decode(b, "bf16").reshape(tokens, hidden), 60.0)
        np.testing.assert_array_equal(_np(sf), rsf)
        np.testing.assert_array_equal(_np(q), rq)


# ------------------------------------------------------------ the separated path


def _separated(inp, gscale=None):
    A = _A()
    res = inp.residual.cuda()
    norm = A.add_rmsnorm(inp.x.cuda(), res, inp.gamma.cuda(), inp.eps)
    if inp.op == "fp8":
        out = dict(q=A.quant_fp8(norm, _dev_scalar(inp.scale)))
    else:
        q, sf = A.quant_nvfp4(norm, _dev_scalar(gscale))
        out = dict(q=q, sf=sf)
    torch.cuda.synchronize()
    out.update(residual=res, norm_out=norm)
    return {k: _np(v) for k, v in out.items()}


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_separated_path_on_the_workloads(k):
    """Both kernels at every tail workload's full size; rows sampled at the large
    ones (first, last, a seeded draw)."""
    inp = W.make_config(k)
    print(f"workload {inp.name}: tokens={inp.tokens} hidden={inp.hidden}", flush=True)
    gscale = float(oracle_global_scale(inp)) if inp.op == "nvfp4" else None
    got = _separated(inp, gscale)
    if inp.tokens <= 64:
        rows = np.arange(inp.tokens)
    else:
        rows = np.unique(np.concatenate([[0, inp.tokens - 1],
                                         np.random.default_rng(k).choice(inp.tokens, 48)]))
    ref = O.add_rmsnorm_quant_fp8(W.bits(inp.x)[rows], W.bits(inp.residual)[rows],
                                  W.bits(inp.gamma), inp.dtype, 1.0, inp.eps, True)
    np.testing.assert_array_equal(got["residual"][rows], ref["residual"])
    np.testing.assert_array_equal(got["norm_out"][rows], ref["norm_out"])
    nt = O.t_decode(ref["norm_out"], inp.dtype)       # the separated path quantises RNE_T(n)
    if inp.op == "fp8":
        np.testing.assert_array_equal(got["q"][rows], O.quant_fp8(nt, inp.scale))
    else:
        rq, rsf = O.quant_nvfp4(nt, gscale)
        np.testing.assert_array_equal(got["sf"][rows], rsf)
        np.testing.assert_array_equal(got["q"][rows], rq)

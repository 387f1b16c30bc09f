"""GPU parity of the gated RMSNorm + NVFP4 (n = RMSNorm(x * SiLU(z)) * gamma per
group, then NVFP4) and of its gate alone, against the oracle, bit for bit.

The gate is checked on every finite fp16 and bf16 z: its exp(-z) is evaluated
in binary64 on the GPU and rounded once, and the oracle's is correctly rounded
by construction, so agreement over all 2^16 patterns is the whole proof that
the GPU gate is exact for every input.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
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


def _from_bits(b, dtype):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(TORCH_DT[dtype])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("xval", ["one", "seeded"])
def test_gate_every_finite_input(dtype, xval):
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    b = b[np.isfinite(O.t_decode(b, dtype))]
    b = np.concatenate([b, np.zeros((-len(b)) % 8, np.uint16)])
    if xval == "one":
        xb = O.t_encode(np.ones(len(b), np.float32), dtype)
    else:
        xb = O.t_encode((3 * np.random.default_rng(8).standard_normal(len(b))).astype(np.float32),
                        dtype)
    u = _A().silu_gate_f32(_from_bits(xb, dtype).cuda(), _from_bits(b, dtype).cuda())
    torch.cuda.synchronize()
    ref = O.silu_gate(O.t_decode(xb, dtype), O.t_decode(b, dtype))
    np.testing.assert_array_equal(_np(u).view(np.uint32), ref.view(np.uint32))


def _run(inp, G, stream=None):
    A = _A()
    q, sf = A.gated_rmsnorm_quant_nvfp4(inp.x.cuda(), inp.residual.cuda(), inp.gamma.cuda(),
                                        torch.tensor([G], device="cuda"), inp.eps,
                                        group=inp.meta["group"], stream=stream)
    torch.cuda.synchronize()
    return _np(q), _np(sf)


def _oracle(inp, G, rows=None):
    sel = slice(None) if rows is None else rows
    return O.gated_rmsnorm_quant_nvfp4(W.bits(inp.x)[sel], W.bits(inp.residual)[sel],
                                       W.bits(inp.gamma), inp.dtype, inp.meta["group"], G, inp.eps)


GRID = [(5, 64, 16), (37, 1024, 1024), (37, 1024, 128), (64, 8192, 1024), (16, 8192, 8192),
        (9, 2048, 64), (3, 16384, 16384), (130, 4096, 512), (1, 16, 16),
        # groups past 16384: four and eight vectors per lane (the computed gate
        # for both dtypes; 40976: the last vectors of a lane past the group end)
        (5, 65536, 32768), (3, 32768, 32768), (2, 65536, 65536), (3, 40976, 40976)]


@pytest.mark.parametrize("tokens,hidden,group", GRID)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gated_matches_oracle(tokens, hidden, group, dtype):
    inp = W.make_gated(hidden + group + tokens, dtype, tokens, hidden, group,
                       z=("normal", 3.0), eps=1e-5)
    G = float(O.nvfp4_global_scale(_oracle(inp, 1.0)["n"]))
    q, sf = _run(inp, G)
    ref = _oracle(inp, G)
    np.testing.assert_array_equal(sf, ref["sf"])
    np.testing.assert_array_equal(q, ref["q"])


@pytest.mark.parametrize("group,tiling,rows,stream", [
    (128, "16:1", "1", "0"), (256, "32:1", "2", "1"), (256, "64:1", "3", "0"),
    (256, "64:2", "2", "1"), (256, "0:1", "1", "1"), (256, "0:2", "4", "0"),
    (128, "32:1", "5", "1"), (256, "0:4", "3", "1"), (512, "0:8", "2", "0")])
@pytest.mark.parametrize("order", ["0", "1"])
def test_gated_every_tiling(group, tiling, rows, stream, order, monkeypatch):
    """Groups over rows of 1024: the per-group gamma slice (also when a lane
    group's rows are interleaved, a whole grid of groups apart), the lane
    mapping and the streaming hints change no bit (each override names a
    tiling that exists for the group width)."""
    monkeypatch.setenv("ANQ_TAIL_TILING", tiling)
    monkeypatch.setenv("ANQ_ROWS_PER_GROUP", rows)
    monkeypatch.setenv("ANQ_ROW_ORDER", order)
    monkeypatch.setenv("ANQ_STREAM", stream)
    inp = W.make_gated(61, "bf16", 23, 1024, group)
    G = 200.0
    q, sf = _run(inp, G)
    ref = _oracle(inp, G)
    np.testing.assert_array_equal(sf, ref["sf"])
    np.testing.assert_array_equal(q, ref["q"])


def test_gated_edge_rows():
    """A zero gate (u = 0: zero codes and scales), gates at the ends of the
    exp range (E = inf gives u = -0 for z < -88.7; E = 0 gives s = z), x = z
    (overlapping inputs are allowed), and a row whose gated values sit on a
    binary32 midpoint of the sum of squares (the double-double fallback)."""
    H = 64
    rows_x, rows_z = [], []
    rows_x.append(np.ones(H)); rows_z.append(np.zeros(H))
    rows_x.append(np.linspace(-3, 3, H)); rows_z.append(np.linspace(-300, 300, H))
    rows_x.append(np.full(H, 0.5)); rows_z.append(np.full(H, 120.0))
    # z = 32: E < 2^-24, so 1 + E rounds to 1 and the gate is exactly 32 x. The
    # first group's u = (4096, 1, 2^-15): ss = 2^24 + 1 + 2^-30, just past a
    # binary32 midpoint that float64 cannot hold; without the last term, a tie.
    mid_x = np.zeros(H); mid_x[0], mid_x[1], mid_x[2] = 128.0, 2.0 ** -5, 2.0 ** -20
    rows_x.append(mid_x); rows_z.append(np.full(H, 32.0))
    tie_x = mid_x.copy(); tie_x[2] = 0.0
    rows_x.append(tie_x); rows_z.append(np.full(H, 32.0))
    x = np.stack(rows_x).astype(np.float32)
    z = np.stack(rows_z).astype(np.float32)
    for dtype in ("f16", "bf16"):
        tdt = TORCH_DT[dtype]
        zz = np.clip(z, -6e4, 6e4)
        inp = W.TailInputs(name="edge", op="gated", dtype=dtype, tokens=len(x), hidden=H,
                           x=torch.from_numpy(x).to(tdt), residual=torch.from_numpy(zz).to(tdt),
                           gamma=torch.ones(H, dtype=tdt), eps=1e-6, scale=None, norm_out=False,
                           meta={"group": 16})
        q, sf = _run(inp, 50.0)
        ref = _oracle(inp, 50.0)
        np.testing.assert_array_equal(sf, ref["sf"])
        np.testing.assert_array_equal(q, ref["q"])
        assert not sf[0].any()
    A = _A()
    t = W.to_dtype(W.normal(9, 0, 16 * 256), "bf16").reshape(16, 256).cuda()
    q1, sf1 = A.gated_rmsnorm_quant_nvfp4(t, t, torch.ones(256, dtype=torch.bfloat16, device="cuda"),
                                          torch.tensor([100.0], device="cuda"), 1e-6, group=64)
    torch.cuda.synchronize()
    tb = W.bits(t.cpu())
    ref = O.gated_rmsnorm_quant_nvfp4(tb, tb, W.bits(torch.ones(256, dtype=torch.bfloat16)),
                                      "bf16", 64, 100.0, 1e-6)
    np.testing.assert_array_equal(_np(sf1), ref["sf"])
    np.testing.assert_array_equal(_np(q1), ref["q"])


def test_gated_workload_size():
    """The gated workload (bf16 [8192, 8192], groups of 1024) with its stored
    global scale: 64 sampled rows against the oracle; no NaN scale anywhere."""
    inp = W.make_config(6)
    print(f"workload {inp.name}", flush=True)
    with open(os.path.join(HERE, "golden", "workload_scalars.json")) as fh:
        G = json.load(fh)["6"]["global_scale"]
    q, sf = _run(inp, G)
    rows = np.unique(np.concatenate([[0, inp.tokens - 1],
                                     np.random.default_rng(6).choice(inp.tokens, 62)]))
    ref = _oracle(inp, G, rows)
    np.testing.assert_array_equal(sf[rows], ref["sf"])
    np.testing.assert_array_equal(q[rows], ref["q"])
    assert not np.any((sf & 0x7F) == 0x7F) and not np.any(sf & 0x80)


@pytest.mark.parametrize("tokens,hidden,group", [(5, 64, 16), (37, 1024, 1024), (37, 1024, 128),
                                                 (64, 8192, 1024), (9, 2048, 64), (130, 4096, 512),
                                                 (5, 2048, 2048), (7, 8192, 8192), (9, 5120, 5120),
                                                 (4, 3072, 1536), (5, 16384, 16384),
                                                 (3, 12288, 12288), (5, 65536, 32768),
                                                 (3, 40976, 40976), (2, 65536, 65536)])
@pytest.mark.parametrize("rows", ["", "1", "3"])
@pytest.mark.parametrize("block", ["", "256"])
@pytest.mark.parametrize("order", ["", "0"])
def test_gated_table_path_matches_oracle(tokens, hidden, group, rows, block, order, monkeypatch):
    """The bf16 gate read from the workgroup's LDS table (forced on small
    calls), with several rows per lane group, interleaved (the default) or
    consecutive, and both workgroup sizes of the lane-group tiling (groups of
    1040 and more take a workgroup per row whatever the size asked; past
    16384, four or eight vectors per lane), gives the oracle's codes."""
    monkeypatch.setenv("ANQ_GATE_LUT", "1")
    monkeypatch.setenv("ANQ_ROWS_PER_GROUP", rows)
    monkeypatch.setenv("ANQ_ROW_ORDER", order)
    monkeypatch.setenv("ANQ_GATE_BLOCK", block)
    inp = W.make_gated(hidden + 7 * group + tokens, "bf16", tokens, hidden, group,
                       z=("normal", 3.0), eps=1e-5)
    G = float(O.nvfp4_global_scale(_oracle(inp, 1.0)["n"]))
    q, sf = _run(inp, G)
    ref = _oracle(inp, G)
    np.testing.assert_array_equal(sf, ref["sf"])
    np.testing.assert_array_equal(q, ref["q"])


@pytest.mark.parametrize("tokens,hidden,group", [(37, 1024, 128), (9, 2048, 64), (7, 8192, 8192),
                                                 (9, 5120, 5120)])
@pytest.mark.parametrize("stream,codes", [("1", "1"), ("1", "0"), ("0", "1")])
def test_gated_table_path_streaming_hints(tokens, hidden, group, stream, codes, monkeypatch):
    """The streaming hints on the rows and on the code and scale stores of
    the gate-table kernel (forced on small calls, both tilings) change no
    bit."""
    monkeypatch.setenv("ANQ_GATE_LUT", "1")
    monkeypatch.setenv("ANQ_STREAM", stream)
    monkeypatch.setenv("ANQ_STREAM_CODES", codes)
    inp = W.make_gated(hidden + group + 3 * tokens, "bf16", tokens, hidden, group,
                       z=("normal", 3.0), eps=1e-5)
    G = float(O.nvfp4_global_scale(_oracle(inp, 1.0)["n"]))
    q, sf = _run(inp, G)
    ref = _oracle(inp, G)
    np.testing.assert_array_equal(sf, ref["sf"])
    np.testing.assert_array_equal(q, ref["q"])


@pytest.mark.parametrize("tokens,hidden,group", [(2048, 8192, 1024), (4096, 4096, 128),
                                                 (1500, 3072, 256), (8192, 2048, 64),
                                                 (512, 8192, 8192), (2048, 8192, 4096),
                                                 (4096, 5120, 5120), (1501, 4096, 2048),
                                                 (2048, 16384, 16384), (512, 32768, 32768),
                                                 (130, 65536, 65536)])
def test_gated_table_interleaved_large(tokens, hidden, group):
    """Calls large enough that the gate-table tiling gives each lane group
    several interleaved rows (2 to 8; at [8192, 2048] in groups of 64 the
    grid doubles to 1024 workgroups, and [1500, 3072] ends in a ragged last
    sweep), and wide groups with a workgroup per row (one to eight rows each,
    640-lane workgroups at 5120): whole tokens sampled against the oracle."""
    inp = W.make_gated(tokens + hidden + group, "bf16", tokens, hidden, group,
                       z=("normal", 2.0), eps=1e-5)
    rows = np.unique(np.concatenate([[0, tokens - 1],
                                     np.random.default_rng(tokens).choice(tokens, 40)]))
    G = float(O.nvfp4_global_scale(_oracle(inp, 1.0, rows)["n"]))
    q, sf = _run(inp, G)
    ref = _oracle(inp, G, rows)
    np.testing.assert_array_equal(sf[rows], ref["sf"])
    np.testing.assert_array_equal(q[rows], ref["q"])


def test_gated_table_path_edge_rows(monkeypatch):
    """Gates outside the table (|z| < 2^-25, |z| >= 128, z = 0) next to table
    entries in one vector, and every bf16 z in the table's range once."""
    monkeypatch.setenv("ANQ_GATE_LUT", "1")
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    z = O.t_decode(b, "bf16")
    b = b[np.isfinite(z) & (np.abs(z) < 1e4)]
    rng = np.random.default_rng(12)
    rng.shuffle(b)
    H = 256
    b = np.concatenate([b, np.zeros((-len(b)) % H, np.uint16)]).reshape(-1, H)
    x = O.t_encode((1 + 0.5 * rng.standard_normal(b.shape)).astype(np.float32), "bf16")
    tdt = torch.bfloat16
    inp = W.TailInputs(name="edge", op="gated", dtype="bf16", tokens=b.shape[0], hidden=H,
                       x=_from_bits(x, "bf16"), residual=_from_bits(b, "bf16"),
                       gamma=torch.ones(H, dtype=tdt), eps=1e-6, scale=None, norm_out=False,
                       meta={"group": 64})
    q, sf = _run(inp, 300.0)
    ref = _oracle(inp, 300.0)
    np.testing.assert_array_equal(sf, ref["sf"])
    np.testing.assert_array_equal(q, ref["q"])

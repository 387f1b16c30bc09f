"""Parity at the extremes of the input types, bit for bit against the oracle.

Activations are drawn uniformly over all finite fp16 / bf16 bit patterns, so
magnitudes run from the subnormals to the top of the type: sums of squares
that overflow binary32 (r = 0), rows dominated by one element, subnormal
norms, quotients past the top code (saturation) and below the smallest code,
and the midpoint fallback all occur. Gamma is a random bit pattern in a third
of the cases; scales are drawn log-uniformly over the allowed domain (positive
normal; FP8 s <= 2^119, NVFP4 G < 2^119). The residual is zero, so the add
cannot overflow T (the inputs stay within the header's finite-input domain).
The Q/K op gets the same activations with moderate gamma: a huge gamma can make
RoPE's n_k c - n_{k+D/2} s an infinity minus an infinity, which the header
leaves unspecified.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import gpu_qk, gpu_tail, oracle_qk, oracle_tail

pytestmark = pytest.mark.gpu

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _finite_bits(rng, dtype, shape):
    b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    while True:
        bad = ~np.isfinite(O.t_decode(b, dtype))
        if not bad.any():
            return b
        b[bad] = rng.integers(0, 1 << 16, size=int(bad.sum()), dtype=np.uint32).astype(np.uint16)


def _tensor(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype])


def _tail_cases(n=48):
    rng = np.random.default_rng(4096)
    out = []
    for i in range(n):
        op = ("fp8", "nvfp4")[i % 2]
        dtype = ("f16", "bf16")[(i // 2) % 2]
        top = 119.0 if op == "fp8" else 118.9
        out.append((i, op, dtype, int(rng.integers(1, 8)), 16 * int(rng.integers(1, 513)),
                    i % 3 == 0, i % 5 == 0, float(rng.choice([1e-6, 1e-30, 3.0])),
                    float(np.float32(2.0 ** rng.uniform(-126, top)))))
    return out


@pytest.mark.parametrize("case", _tail_cases(),
                         ids=lambda c: f"{c[1]}-{c[2]}-{c[3]}x{c[4]}{'-wildgamma' if c[5] else ''}")
def test_extreme_tail(case):
    i, op, dtype, tokens, hidden, wild_gamma, norm, eps, scale = case
    rng = np.random.default_rng(10_000 + i)
    xb = _finite_bits(rng, dtype, (tokens, hidden))
    gb = (_finite_bits(rng, dtype, (hidden,)) if wild_gamma else
          O.t_encode((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), dtype))
    inp = W.TailInputs(name="extreme", op=op, dtype=dtype, tokens=tokens, hidden=hidden,
                       x=_tensor(xb, dtype), residual=_tensor(np.zeros_like(xb), dtype),
                       gamma=_tensor(gb, dtype), eps=eps, scale=scale if op == "fp8" else None,
                       norm_out=norm, meta={})
    got, ref = gpu_tail(inp, scale), oracle_tail(inp, scale)
    for k in ["residual", "q"] + (["sf"] if op == "nvfp4" else []) + (["norm_out"] if norm else []):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


@pytest.mark.parametrize("i", range(16))
def test_extreme_qk(i):
    rng = np.random.default_rng(20_000 + i)
    dtype = ("f16", "bf16")[i % 2]
    head_dim = int(rng.choice([32, 64, 128, 256]))
    nq, nk, nv = int(rng.integers(0, 4)), int(rng.integers(0, 3)), int(rng.integers(0, 3))
    if nq + nk + nv == 0:
        nv = 1
    tokens = int(rng.integers(1, 6))
    inp = W.make_qk(30_000 + i, dtype, tokens, nq, nk, nv, head_dim,
                    positions=rng.integers(0, 64, tokens), max_pos=64,
                    scale=float(np.float32(2.0 ** rng.uniform(-20, 20))))
    inp.qkv = _tensor(_finite_bits(rng, dtype, tuple(inp.qkv.shape)), dtype)
    np.testing.assert_array_equal(gpu_qk(inp), oracle_qk(inp))


@pytest.mark.parametrize("stream", ["", "1"])
@pytest.mark.parametrize("op", ["fp8", "nvfp4"])
def test_wide_span_midpoint_rows(op, stream, monkeypatch):
    """bf16 rows whose large squares sum exactly to a binary32 midpoint
    (2^120 + 2^96) next to tiny ones (2^-10, 2^-30, 2^-60) far below float64's reach
    of the large part: the exact sum is just above the midpoint and rounds up,
    and the double-double fallback keeps the tiny part in its low word. A row
    without the tiny element is the exact tie (to even, down). With streaming
    hints forced on, the fallback re-reads residual elements the same lanes
    have just written with non-temporal stores."""
    monkeypatch.setenv("ANQ_STREAM", stream)
    H = 64
    rows = []
    for tiny in (2.0 ** -10, 2.0 ** -30, 2.0 ** -60, 0.0):
        r = np.zeros(H, np.float32)
        r[0], r[1], r[2] = 2.0 ** 60, 2.0 ** 48, tiny
        rows.append(r)
    xb = O.t_encode(np.stack(rows), "bf16")
    gb = O.t_encode(np.ones(H, np.float32), "bf16")
    scale = 0.01 if op == "fp8" else 300.0
    inp = W.TailInputs(name="span", op=op, dtype="bf16", tokens=len(rows), hidden=H,
                       x=_tensor(xb, "bf16"), residual=_tensor(np.zeros_like(xb), "bf16"),
                       gamma=_tensor(gb, "bf16"), eps=1e-30, scale=scale if op == "fp8" else None,
                       norm_out=True, meta={})
    got, ref = gpu_tail(inp, scale), oracle_tail(inp, scale)
    assert [float(v) for v in ref["ss"]] == [2.0 ** 120 * (1 + 2.0 ** -23)] * 3 + [2.0 ** 120]
    for k in ["residual", "norm_out", "q"] + (["sf"] if op == "nvfp4" else []):
        np.testing.assert_array_equal(got[k], ref[k], err_msg=k)


@pytest.mark.parametrize("cap", ["1", "2", "3", "4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("head_dim", [64, 128])
def test_qk_midpoint_heads(head_dim, dtype, cap, monkeypatch):
    """Q and K heads whose squares sum exactly to a binary32 midpoint
    (2^30 + 64, from 32768 and 8), with or without a tiny element whose square
    float64 cannot hold beside 2^30: the tie rounds to even (down), the rest up
    through the double-double path. The planted elements sit in both halves of
    a head, in heads of every pass (17 heads: a ragged last pass), and the op
    runs with one wavefront per token where the cap on the head groups a
    wavefront loads at once allows it (so 1-3 groups per wavefront)."""
    monkeypatch.setenv("ANQ_QK_WAVES", "1")
    monkeypatch.setenv("ANQ_QK_GROUPS", cap)
    nq, nk, nv, D = 9, 5, 3, head_dim
    tokens = 6
    rng = np.random.default_rng(4711 + D)
    inp = W.make_qk(40_000 + D, dtype, tokens, nq, nk, nv, D,
                    positions=rng.integers(0, 32, tokens), max_pos=32, scale=0.05)
    q = inp.qkv.float().numpy().reshape(tokens, nq + nk + nv, D).copy()
    tiny = 2.0 ** -24 if dtype == "f16" else 2.0 ** -40
    for t in range(tokens):
        for h in (t, nq + (t % nk), (3 * t + 7) % (nq + nk)):
            q[t, h] = 0.0
            q[t, h, D // 2 + 3] = 32768.0
            q[t, h, 1 + t] = 8.0
            if (t + h) % 3:
                q[t, h, D - 1 - t] = tiny
    inp.qkv = _tensor(O.t_encode(q.reshape(tokens, -1).astype(np.float32), dtype), dtype)
    np.testing.assert_array_equal(gpu_qk(inp), oracle_qk(inp))

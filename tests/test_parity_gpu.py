"""GPU parity: the HIP kernels (through the C ABI and its Python binding)
against the CPU oracle on the same seeded inputs.

Bars (see tests/compare.py): residual bit-exact; norm output within 4e-3 after
rounding; FP8/E2M1 codes and E4M3 block scales identical on >= 99.9 % and never
more than one step apart. The design makes every output bit-exact, and the
tests assert that as well.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from compare import (check_codes, check_norm, check_nvfp4, check_residual, code_stats, e4m3_rank,
                     norm_stats, nvfp4_stats)
from runners import gpu_qk, gpu_tail, oracle_global_scale, oracle_qk, oracle_tail

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()  # fail loudly when the library is missing


def _scale(inp):
    return float(inp.scale) if inp.op == "fp8" else float(oracle_global_scale(inp))


def compare_tail(inp, scale, got, ref, rows=None, exact=True):
    sel = slice(None) if rows is None else rows
    check_residual(got["residual"][sel], ref["residual"])
    if inp.norm_out:
        ns = norm_stats(got["norm_out"][sel], ref["norm_out"], inp.dtype)
        check_norm(ns)
        if exact:
            assert ns["bit_exact"], ns
    if inp.op == "fp8":
        cs = code_stats(got["q"][sel], ref["q"], e4m3_rank)
        check_codes(cs, "fp8")
        if exact:
            assert cs["bit_exact"], cs
    else:
        st = nvfp4_stats(got["q"][sel], got["sf"][sel], ref["q"], ref["sf"], scale)
        check_nvfp4(st)
        if exact:
            assert st["bit_exact"], st


def run_and_compare(inp, rows=None):
    scale = _scale(inp)
    got = gpu_tail(inp, scale)
    ref = oracle_tail(inp, scale, rows)
    compare_tail(inp, scale, got, ref, rows)
    return got


# ------------------------------------------------------------- workloads ---

@pytest.mark.parametrize("k", [1, 2])
def test_workload_small_full_compare(k):
    run_and_compare(W.make_config(k))


@pytest.mark.parametrize("k", [3, 4])
def test_workload_full_size_sampled_rows(k):
    """Full-size launch (the configuration the benchmark times); the oracle
    checks the whole residual and 320 sampled rows of every other output."""
    inp = W.make_config(k)
    print(f"workload {inp.name}: tokens={inp.tokens} hidden={inp.hidden}", flush=True)
    scale = _scale(inp)
    got = gpu_tail(inp, scale)
    full_h = O.residual_add(W.bits(inp.x), W.bits(inp.residual), inp.dtype)
    check_residual(got["residual"], full_h)
    rng = np.random.default_rng(k)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(inp.tokens - 32, inp.tokens),
                                     rng.choice(inp.tokens, 256, replace=False)]))
    ref = oracle_tail(inp, scale, rows)
    compare_tail(inp, scale, got, ref, rows)
    if inp.op == "fp8":  # properties over the whole tensor: no NaN code is ever produced
        assert not np.any((got["q"] & 0x7F) == 0x7F)
    else:
        assert not np.any((got["sf"] & 0x7F) == 0x7F) and not np.any(got["sf"] & 0x80)


def test_workload_qk_full_compare():
    inp = W.make_config(5)
    got = gpu_qk(inp)
    ref = oracle_qk(inp)
    cs = code_stats(got, ref, e4m3_rank)
    check_codes(cs, "qk")
    assert cs["bit_exact"], cs


# ------------------------------------------------------------ shape grid ---

GRID_H = [16, 48, 128, 256, 400, 512, 1024, 1040, 2048, 4112, 7168, 8192, 16400, 32768, 40976,
          65520, 65536]  # 40976 and 65520: 8 vectors per lane, the last ones past the row end


@pytest.mark.parametrize("hidden", GRID_H)
@pytest.mark.parametrize("op,dtype,norm", [("fp8", "f16", False), ("fp8", "bf16", True),
                                           ("nvfp4", "f16", True), ("nvfp4", "bf16", False)])
def test_tail_shape_grid(hidden, op, dtype, norm):
    tokens = 37 if hidden <= 8192 else 3
    inp = W.make_tail(100 + hidden, op, dtype, tokens, hidden, eps=1e-5,
                      scale=0.02 if op == "fp8" else None, norm_out=norm, outliers=0.002)
    run_and_compare(inp)


@pytest.mark.parametrize("hidden,tokens", [(128, 16), (128, 256), (7168, 16), (7168, 256)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tail_published_grid_nvfp4_with_norm(hidden, tokens, dtype):
    """hidden 128/7168 x sequence 16/256 (TensorRT-LLM issue #17900,
    Correctness; the 8192-token rows are the full-size workload test)."""
    inp = W.make_tail(7 + tokens, "nvfp4", dtype, tokens, hidden, norm_out=True)
    run_and_compare(inp)


@pytest.mark.parametrize("tokens,hidden,op", [(4099, 4000, "fp8"), (4099, 4000, "nvfp4"),
                                               (4100, 8192, "nvfp4")])
def test_tail_default_interleaved_rows(tokens, hidden, op):
    """Calls whose default tiling gives each workgroup two rows (one vector
    per lane, 512 or more lanes, 4096 or more tokens), taken interleaved
    across the grid; an odd token count leaves the last sweep ragged. Sampled
    rows against the oracle, every output."""
    inp = W.make_tail(tokens + hidden, op, "bf16", tokens, hidden, norm_out=True,
                      scale=0.02 if op == "fp8" else None, outliers=0.002)
    rows = np.unique(np.concatenate([[0, 1, tokens // 2, tokens - 2, tokens - 1],
                                     np.random.default_rng(hidden).choice(tokens, 200)]))
    run_and_compare(inp, rows)


@pytest.mark.parametrize("tokens,hidden,op,dtype", [(1031, 7168, "nvfp4", "bf16"),
                                                     (1100, 6656, "fp8", "f16"),
                                                     (1024, 7680, "nvfp4", "f16")])
def test_tail_padded_workgroups(tokens, hidden, op, dtype):
    """One vector per lane in 13 to 15 wavefronts, which the default tiling
    pads to 16 at 1024 rows or more: the padding lanes own no vector, add
    nothing to the sum and store nothing. Sampled rows, every output."""
    inp = W.make_tail(tokens + hidden, op, dtype, tokens, hidden, norm_out=True,
                      scale=0.02 if op == "fp8" else None, outliers=0.002)
    rows = np.unique(np.concatenate([[0, tokens - 1],
                                     np.random.default_rng(hidden).choice(tokens, 150)]))
    run_and_compare(inp, rows)


# ------------------------------------------------------------ edge rows ----

def _tail_from_arrays(op, dtype, x, res, gamma, eps=1e-6, scale=0.02, norm=True):
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    return W.TailInputs(name="edge", op=op, dtype=dtype, tokens=x.shape[0], hidden=x.shape[1],
                        x=torch.from_numpy(x).to(tdt), residual=torch.from_numpy(res).to(tdt),
                        gamma=torch.from_numpy(gamma).to(tdt), eps=eps,
                        scale=scale if op == "fp8" else None, norm_out=norm)


@pytest.mark.parametrize("stream", ["", "1"])
@pytest.mark.parametrize("op", ["fp8", "nvfp4"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("hidden", [64, 1024, 7168, 16384, 32768, 40976, 65536])
def test_edge_rows(op, dtype, hidden, stream, monkeypatch):
    """All-zero rows (with a negative gamma: signed zeros), a one-hot row,
    x = -residual (exact cancellation), x50 and x1000 outliers (E4M3 and E2M1
    saturation), tiny values (E4M3 subnormals), and rows whose exact sum of
    squares sits on or just past a binary32 rounding midpoint that float64
    cannot resolve (the double-double path, which re-reads the residual the
    lanes just stored: with and without streaming hints)."""
    monkeypatch.setenv("ANQ_STREAM", stream)
    rng = np.random.default_rng(hidden)
    H = hidden
    rows = []
    rows.append(np.zeros(H))
    oh = np.zeros(H); oh[H // 3] = 3.0; rows.append(oh)
    rows.append(rng.standard_normal(H))                       # cancels below
    out = rng.standard_normal(H); out[::97] *= 50.0; out[5] = 1000.0; rows.append(out)
    rows.append(rng.standard_normal(H) * 1e-3)
    big, tiny = 32768.0, (2.0 ** -24 if dtype == "f16" else 2.0 ** -40)
    mid = np.zeros(H); mid[0], mid[1], mid[2] = big, 8.0, tiny; rows.append(mid)
    tie = np.zeros(H); tie[0], tie[1] = big, 8.0; rows.append(tie)
    x = np.stack(rows).astype(np.float32)
    res = np.zeros_like(x)
    res[2] = -x[2]
    gamma = (1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    gamma[::7] *= -1.0
    inp = _tail_from_arrays(op, dtype, x, res, gamma, eps=1e-6, scale=0.05)
    got = run_and_compare(inp)
    if op == "fp8":
        assert np.any(got["q"][0] == 0x80) and np.any(got["q"][0] == 0x00)  # signed zeros


@pytest.mark.parametrize("op,scale", [("fp8", 1e-36), ("fp8", 0.05), ("nvfp4", 1e30),
                                      ("nvfp4", 1.0)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_overflow_saturates(op, scale, dtype):
    """gamma entries at the top of T's range drive n (binary32), n / s, G * amax / 6
    and n * mult past the largest finite value: every code saturates (E4M3 to
    448, E2M1 to 6) as the definitions say, never a NaN code."""
    rng = np.random.default_rng(17)
    H = 1024
    x = rng.standard_normal((6, H)).astype(np.float32)
    x[1, 3] = 200.0                                        # |h r| near sqrt(H)
    top = 65504.0 if dtype == "f16" else 3.3895313892515355e38
    gamma = (1.0 + 0.1 * rng.standard_normal(H)).astype(np.float32)
    gamma[::5] = top
    gamma[3::10] = -top
    inp = _tail_from_arrays(op, dtype, x, np.zeros_like(x), gamma, scale=scale)
    got = gpu_tail(inp, scale)
    ref = oracle_tail(inp, scale)
    compare_tail(inp, scale, got, ref)
    if op == "fp8":
        assert np.any((got["q"] & 0x7F) == 0x7E) and not np.any((got["q"] & 0x7F) == 0x7F)
    else:
        assert np.any(got["sf"] == 0x7E) and not np.any((got["sf"] & 0x7F) == 0x7F)


def test_zero_tokens_is_a_noop_and_errors_raise():
    import nvfp4_quantization_place_amd as A
    x = torch.zeros(0, 128, dtype=torch.bfloat16, device="cuda")
    res = torch.zeros_like(x)
    g = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    s = torch.ones(1, dtype=torch.float32, device="cuda")
    q, norm = A.add_rmsnorm_quant_fp8(x, res, g, s, 1e-6, norm_out=True)
    assert q.shape == (0, 128)
    x = torch.randn(4, 128, device="cuda").to(torch.bfloat16)
    res = torch.randn(4, 128, device="cuda").to(torch.bfloat16)
    with pytest.raises(A.AnqError) as e:
        A.add_rmsnorm_quant_fp8(x, res, g, s, 1e-6, q=res.view(torch.uint8).view(-1)[:512].view(4, 128))
    assert e.value.code == 5
    with pytest.raises(A.AnqError) as e:
        A.add_rmsnorm_quant_nvfp4(x[:, :120].contiguous(), res[:, :120].contiguous(), g[:120], s, 1e-6)
    assert e.value.code == 2


def test_non_default_stream_and_repeatability():
    inp = W.make_tail(55, "nvfp4", "bf16", 300, 7168, norm_out=True)
    scale = _scale(inp)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        a = gpu_tail(inp, scale, stream=st)
    b = gpu_tail(inp, scale)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    compare_tail(inp, scale, a, oracle_tail(inp, scale))


# ------------------------------------------------------------------ Q/K ----

@pytest.mark.parametrize("stream", ["", "1"])
@pytest.mark.parametrize("head_dim", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("heads", [(4, 2, 2), (3, 1, 0), (0, 2, 1), (1, 0, 0)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_qk_grid(head_dim, heads, dtype, stream, monkeypatch):
    monkeypatch.setenv("ANQ_STREAM", stream)
    nq, nk, nv = heads
    tokens = 29
    rng = np.random.default_rng(head_dim + 10 * nq + nk)
    pos = rng.integers(0, 300, tokens)
    inp = W.make_qk(head_dim + nq, dtype, tokens, nq, nk, nv, head_dim, positions=pos,
                    max_pos=300, scale=0.03)
    got = gpu_qk(inp)
    ref = oracle_qk(inp)
    cs = code_stats(got, ref, e4m3_rank)
    check_codes(cs, "qk")
    assert cs["bit_exact"], cs


# ----------------------------------------------------- every tiling agrees --

@pytest.mark.parametrize("hidden,tilings", [
    (128, ["16:1", "32:1", "64:1", "0:1", "0:2"]),
    (1024, ["64:2", "0:1", "0:2", "0:4", "0:8"]),
    (512, ["64:1", "0:1", "0:2"]),
    (1040, ["0:1", "0:2", "0:4"]),
    (7168, ["0:1", "0:2", "0:4", "0:8"]),
])
@pytest.mark.parametrize("op", ["fp8", "nvfp4"])
def test_every_tiling_matches_the_oracle(hidden, tilings, op, monkeypatch):
    """The lane mapping (lanes per row, vectors per lane, rows per lane group,
    consecutive or interleaved rows) and the streaming hints (none, on the row
    streams, on the row streams and the code stores) change only the order of
    float64 partial sums and cache behaviour, never a result bit."""
    inp = W.make_tail(900 + hidden, op, "bf16", 67, hidden, norm_out=True,
                      scale=0.03 if op == "fp8" else None, outliers=0.002)
    scale = _scale(inp)
    ref = oracle_tail(inp, scale)
    for t in tilings:
        for rows, order, stream, codes in (("", "", "", ""), ("1", "1", "1", ""),
                                           ("1", "0", "1", "0"), ("3", "1", "0", ""),
                                           ("64", "0", "1", "1"), ("5", "1", "1", "1")):
            monkeypatch.setenv("ANQ_TAIL_TILING", t)
            monkeypatch.setenv("ANQ_ROWS_PER_GROUP", rows)
            monkeypatch.setenv("ANQ_ROW_ORDER", order)
            monkeypatch.setenv("ANQ_STREAM", stream)
            monkeypatch.setenv("ANQ_STREAM_CODES", codes)
            got = gpu_tail(inp, scale)
            compare_tail(inp, scale, got, ref)


@pytest.mark.parametrize("groups", ["", "2", "3"])
@pytest.mark.parametrize("waves", ["1", "2", "3", "5"])
@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("block", ["", "64", "1024"])
def test_qk_waves_per_token_agree(head_dim, waves, block, groups, monkeypatch):
    """Splitting a token's heads over several wavefronts (also unevenly: the
    cap on head groups per wavefront raises the count), and packing wavefronts
    into workgroups of other sizes, changes nothing."""
    monkeypatch.setenv("ANQ_QK_WAVES", waves)
    monkeypatch.setenv("ANQ_QK_BLOCK", block)
    monkeypatch.setenv("ANQ_QK_GROUPS", groups)
    pos = np.random.default_rng(3).integers(0, 64, 23)
    inp = W.make_qk(31, "bf16", 23, 9, 5, 3, head_dim, positions=pos, max_pos=64, scale=0.04)
    got = gpu_qk(inp)
    cs = code_stats(got, oracle_qk(inp), e4m3_rank)
    assert cs["bit_exact"], cs


@pytest.mark.parametrize("groups", ["", "1", "4"])
def test_qk_wide_heads_small_workgroups(groups, monkeypatch):
    """Heads of 512 with 64-lane workgroups asked for: the launcher widens the
    workgroup to 128 lanes, one gamma vector per lane, and the op still
    matches (9 groups of 2 heads per token, one wavefront per token)."""
    monkeypatch.setenv("ANQ_QK_BLOCK", "64")
    monkeypatch.setenv("ANQ_QK_WAVES", "1")
    monkeypatch.setenv("ANQ_QK_GROUPS", groups)
    pos = np.random.default_rng(5).integers(0, 16, 5)
    inp = W.make_qk(37, "f16", 5, 9, 5, 3, 512, positions=pos, max_pos=16, scale=0.04)
    np.testing.assert_array_equal(gpu_qk(inp), oracle_qk(inp))

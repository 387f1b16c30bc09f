"""bench.py's host logic, on the CPU: the algorithmic bytes it divides by
(against the per-workload byte table the byte formulas give, worked out by
hand below), the store bytes of the KV pools, the rotation that keeps every
timed call streaming from HBM, the split-row shapes, and the refusal to
report anything but one GPU."""
import math
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# bytes per call, by hand: x and residual read (2 B each), residual written
# (2 B), codes (FP8 1 B, NVFP4 0.5 + 1/16 B), norm output 2 B, gamma 2H, the
# 4-byte scale; Q/K: qkv read 2 B, codes 1 B per element, the cos|sin row
# (4D) and the position (8) per token, gamma_q and gamma_k (2D each), scale
HAND = {
    1: 16 * 128 * (2 + 2 + 2 + 1) + 2 * 128 + 4,                          # 14 596
    2: 64 * 8192 * 6 + 64 * 8192 // 2 + 64 * 8192 // 16 + 2 * 8192 + 4,  # 3 457 028
    3: 65536 * 1024 * (2 + 2 + 2 + 1 + 2) + 2 * 1024 + 4,                 # 603 981 828
    4: 8192 * 7168 * 8 + 8192 * 7168 // 2 + 8192 * 7168 // 16 + 2 * 7168 + 4,
    5: 4096 * 4096 * 3 + 4096 * (4 * 128 + 8) + 4 * 128 + 4,             # 52 462 084
}


@pytest.mark.parametrize("k", sorted(HAND))
def test_algorithmic_bytes(k):
    rd, wr = bench.rw_bytes(W.make_config(k))
    assert rd + wr == HAND[k]
    assert {1: 14596, 2: 3457028, 3: 603981828, 4: 502806532, 5: 52462084}[k] == HAND[k]


def test_gated_bytes():
    rd, wr = bench.rw_bytes(W.make_config(6))
    n = 8192 * 8192
    assert (rd, wr) == (4 * n + 2 * 8192 + 4, n // 2 + n // 16)


def test_separated_bytes_count_the_norm_round_trip():
    inp = W.make_config(4)
    rd, wr = bench.rw_bytes(inp, "separated")
    n = 8192 * 7168
    # add_rmsnorm reads x, residual, gamma and writes residual and norm; the
    # quantiser reads the norm and writes codes and scales
    assert rd == 4 * n + 2 * 7168 + 2 * n + 4
    assert wr == 4 * n + n // 2 + n // 16


@pytest.mark.parametrize("kind", ["kv_store", "kv_mixed"])
def test_pool_bytes_count_only_stored_tokens(kind):
    inp = W.make_config(7 if kind == "kv_mixed" else 5)
    T, D, R = inp.tokens, inp.head_dim, inp.rotary_dim
    slots = W.kv_slots(7 if kind == "kv_mixed" else 5, T, T * 5 // 4)
    stored = int((slots >= 0).sum())
    assert stored == T - T // 16                      # every 16th token is padding
    rd, wr = bench.rw_bytes(inp, kind, stored)
    C = (inp.nq + inp.nk + inp.nv) * D
    assert rd == T * C * 2 + T * (4 * R + 8) + 4 * D + 4 + 8 * T
    row = inp.nk * (D + R) + inp.nv * D if kind == "kv_mixed" else (inp.nk + inp.nv) * D
    assert wr == T * inp.nq * D + stored * row
    if kind == "kv_mixed":
        import nvfp4_quantization_place_amd as A
        assert row == A.mixed_kv_row_bytes(inp.nk, inp.nv, D, R) == 2560


@pytest.mark.parametrize("bytes_per_call", [14596, 3457028, 52462084, 306200580, 603981828])
@pytest.mark.parametrize("steps", [1, 5, 20, 200])
def test_rotation_streams_from_hbm(bytes_per_call, steps):
    """At least 1 GiB of buffers rotate (so nothing is left in the 256 MB
    last-level cache when a graph comes round again), the graphs partition the
    sets, or, for calls so small that this would take more than MAX_GRAPHS
    graphs, one graph with a cache flush before its timed replay."""
    s = bench.rotating_sets(bytes_per_call, steps)
    assert s >= 2
    graphs = math.ceil(s / steps)
    if s * bytes_per_call < bench.ROTATE_BYTES:
        assert s == max(2, steps) and bench.FLUSH_BYTES >= bench.ROTATE_BYTES
    else:
        assert graphs <= bench.MAX_GRAPHS
        assert s <= steps or s % steps == 0
    assert bench.ROTATE_BYTES >= 1 << 30


def test_headline_rotation_at_20_steps():
    assert bench.rotating_sets(bench.rw_bytes(W.make_config(2))[0] +
                               bench.rw_bytes(W.make_config(2))[1], 20) == 320


def test_split_rows_move_the_headline_bytes():
    head = sum(bench.rw_bytes(W.make_config(2)))
    for M, H in bench.SPLIT_SHAPES:
        assert M * H == 64 * 8192
        inp = W.make_tail(2, "nvfp4", "f16", M, H, scale=None)
        got = sum(bench.rw_bytes(inp))
        assert got - 2 * H - 4 == head - 2 * 8192 - 4   # only gamma's size differs


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", gpus,
                        "--no-cpu"], capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_bytes_per_row_are_the_workloads():
    """The CPU baseline converts rows per second with the same algorithmic
    bytes per row as the GPU figure (the mixed workload's sample stores every
    row, so all of its rows count a pool row)."""
    inp = W.make_config(7)
    rd, wr = bench.rw_bytes(inp, "kv_mixed")
    rd_s, wr_s = bench.rw_bytes(inp, "kv_mixed", inp.tokens)
    assert (rd, wr) == (rd_s, wr_s)
    # per token: qkv read (2 B x 4096), cos|sin row (4 x 64), position and
    # slot (8 + 8); Q codes (16 x 128) and the pool row (2560); per call:
    # gamma_q, gamma_k and the scale
    assert np.isclose((rd + wr) / inp.tokens,
                      (2 * 4096 + 4 * 64 + 8 + 8) + (16 * 128 + 2560) + (4 * 128 + 4) / 4096)

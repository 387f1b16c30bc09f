"""The front end's launch choices, on the CPU: the C-ABI front end and the
tiling choice built for the host with stand-in launchers
(tests/hostcheck/stub_launch.cpp) that check each launch's geometry against
the work it must cover and record it instead of running a kernel. Calls here
have tokens > 0 and fake device addresses that nothing dereferences.

Covered: the tiling each workload shape gets; that every ANQ_* override is
taken exactly as given (the launch shows it); that an override naming a
tiling without a kernel, or a malformed one, fails with ANQ_ERR_CONFIG before
anything is launched; and that the grid covers every row for a sweep of
shapes and overrides.
"""
import ctypes
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "hostcheck"))

import nvfp4_quantization_place_amd as A  # noqa: E402

OK, CONFIG, LAUNCH = 0, 9, 7
BASE = 1 << 40
MB = 1 << 20
ENV = ("ANQ_TAIL_TILING", "ANQ_ROWS_PER_GROUP", "ANQ_ROW_ORDER", "ANQ_STREAM", "ANQ_STREAM_CODES",
       "ANQ_GATE_LUT",
       "ANQ_GATE_BLOCK", "ANQ_QK_WAVES", "ANQ_QK_GROUPS", "ANQ_QK_BLOCK")


def addr(i):
    return BASE + i * 4096 * MB   # 4 GiB apart: disjoint for every shape used here


@pytest.fixture(scope="module")
def L():
    path = os.environ.get("ANQ_HOSTCHECK_LIB")
    if not path:
        import build_hostcheck
        path = build_hostcheck.build(sanitize=False)
    lib = A.load(path)
    lib.anq_hostcheck_last.restype = ctypes.c_char_p
    lib.anq_hostcheck_calls.restype = ctypes.c_int64
    return lib


@pytest.fixture(autouse=True)
def _clean_env(monkeypatch):
    for k in ENV:
        monkeypatch.delenv(k, raising=False)


def last(L) -> dict:
    return dict(kv.split("=") for kv in L.anq_hostcheck_last().decode().split())


def tail(L, op, tokens, hidden, dtype=1, norm=True):
    if op == "fp8":
        st = L.add_rmsnorm_quant_fp8(addr(0), addr(1), addr(2), addr(3), 1e-6, tokens, hidden,
                                     dtype, addr(4), addr(5) if norm else None, None)
    elif op == "nvfp4":
        st = L.add_rmsnorm_quant_nvfp4(addr(0), addr(1), addr(2), addr(3), 1e-6, tokens, hidden,
                                       dtype, addr(4), addr(6), addr(5) if norm else None, None)
    elif op == "swizzled":
        st = L.add_rmsnorm_quant_nvfp4_swizzled(addr(0), addr(1), addr(2), addr(3), 1e-6, tokens,
                                                hidden, dtype, addr(4), addr(6),
                                                addr(5) if norm else None, None)
    else:
        st = L.add_rmsnorm(addr(0), addr(1), addr(2), 1e-6, tokens, hidden, dtype, addr(5), None)
    return st


@pytest.mark.parametrize("tokens,hidden,want", [
    (16, 128, dict(group="16", vec_per_lane="1", block="256", rows="1", stream="0",
                   stream_codes="0")),
    (64, 8192, dict(group="0", vec_per_lane="1", block="1024", rows="1", stream="1",
                    stream_codes="1")),
    (65536, 1024, dict(group="0", vec_per_lane="1", block="128", rows="1", stream="1",
                       stream_codes="0")),
    (8192, 7168, dict(group="0", vec_per_lane="2", block="448", rows="1", stream="1",
                      stream_codes="0")),
    (1024, 7168, dict(group="0", vec_per_lane="1", block="1024", rows="1", stream="1",
                      stream_codes="1")),     # 14 wavefronts padded to 16
    (512, 7168, dict(group="0", vec_per_lane="1", block="896")),   # too few rows to pad
    (1024, 6144, dict(group="0", vec_per_lane="1", block="768")),  # 12 wavefronts: not padded
    (1024, 7680, dict(group="0", vec_per_lane="1", block="1024")),
    (8192, 8192, dict(group="0", vec_per_lane="1", block="1024", rows="2", interleave="1",
                      stream="1", stream_codes="0")),
    (65536, 1024, dict(interleave="0")),
    (3, 65536, dict(group="0", vec_per_lane="8", block="1024")),
])
def test_workload_tilings(L, tokens, hidden, want):
    assert tail(L, "nvfp4", tokens, hidden) == OK
    got = last(L)
    assert got["kind"] == "tail" and got["ok"] == "1"
    for k, v in want.items():
        assert got[k] == v, (k, got)


@pytest.mark.parametrize("hidden", [16, 48, 128, 256, 400, 512, 1024, 1040, 7168, 8192, 16400,
                                    40976, 65536])
@pytest.mark.parametrize("tokens", [1, 3, 67, 4096, 5000])
def test_every_accepted_tiling_covers_the_rows(L, hidden, tokens, monkeypatch):
    vec = hidden // 8
    for g, k in [(16, 1), (32, 1), (64, 1), (64, 2), (0, 1), (0, 2), (0, 4), (0, 8)]:
        for rows, order in (("", ""), ("1", "0"), ("3", "1")):
            monkeypatch.setenv("ANQ_TAIL_TILING", f"{g}:{k}")
            monkeypatch.setenv("ANQ_ROWS_PER_GROUP", rows)
            monkeypatch.setenv("ANQ_ROW_ORDER", order)
            exists = (g == 0 and (vec + k - 1) // k <= 1024) or (g in (16, 32) and k == 1 and g >= vec) \
                or (g == 64 and g * k >= vec)
            for op in ("fp8", "nvfp4", "swizzled", "none"):
                st = tail(L, op, tokens, hidden)
                if not exists:
                    assert st == CONFIG, (g, k, op)
                    continue
                assert st == OK, (g, k, rows, op, last(L))
                got = last(L)
                assert got["group"] == str(g) and got["vec_per_lane"] == str(k), got
                if rows:
                    assert got["rows"] == rows and got["interleave"] == order, got
                else:   # default: interleaved exactly when a lane group takes several rows
                    assert got["interleave"] == ("1" if int(got["rows"]) > 1 else "0"), got


@pytest.mark.parametrize("value", ["16:2", "32:2", "0:3", "8:1", "64:4", "0:1x", "abc", "0",
                                   "0:1:2", "0:1 "])
def test_bad_tiling_override_is_refused(L, value, monkeypatch):
    """'16:2' and '32:2' name lane groups with two vectors per lane, for which
    no kernel exists: refused, never run as a one-vector kernel that would
    leave half of the row untouched."""
    n = L.anq_hostcheck_calls()
    monkeypatch.setenv("ANQ_TAIL_TILING", value)
    assert tail(L, "nvfp4", 8, 256) == CONFIG
    assert L.anq_hostcheck_calls() == n          # nothing launched


@pytest.mark.parametrize("name,value", [("ANQ_ROWS_PER_GROUP", "0"), ("ANQ_ROWS_PER_GROUP", "-2"),
                                        ("ANQ_ROWS_PER_GROUP", "two"), ("ANQ_STREAM", "2"),
                                        ("ANQ_STREAM", "yes"), ("ANQ_STREAM_CODES", "2"),
                                        ("ANQ_ROW_ORDER", "2"), ("ANQ_ROW_ORDER", "-1"),
                                        ("ANQ_GATE_LUT", "2"),
                                        ("ANQ_GATE_BLOCK", "96"), ("ANQ_GATE_BLOCK", "2048"),
                                        ("ANQ_QK_WAVES", "0"), ("ANQ_QK_GROUPS", "5"),
                                        ("ANQ_QK_BLOCK", "100"), ("ANQ_QK_BLOCK", "2048")])
def test_bad_tuning_values_are_refused(L, name, value, monkeypatch):
    monkeypatch.setenv(name, value)
    if name.startswith("ANQ_QK"):
        st = qk(L, 64, 16, 8, 8, 128)
    elif name.startswith("ANQ_GATE"):
        monkeypatch.setenv("ANQ_GATE_LUT", "1") if name == "ANQ_GATE_BLOCK" else None
        st = L.gated_rmsnorm_quant_nvfp4(addr(0), addr(1), addr(2), addr(3), 1e-5, 4096, 8192,
                                         1024, 1, addr(4), addr(6), None)
    else:
        st = tail(L, "nvfp4", 8, 256)
    assert st == CONFIG


def test_stream_override_is_taken(L, monkeypatch):
    assert tail(L, "fp8", 65536, 1024) == OK and last(L)["stream"] == "1"
    monkeypatch.setenv("ANQ_STREAM", "0")
    assert tail(L, "fp8", 65536, 1024) == OK and last(L)["stream"] == "0"
    assert tail(L, "fp8", 16, 128) == OK and last(L)["stream"] == "0"
    monkeypatch.setenv("ANQ_STREAM", "1")
    assert tail(L, "fp8", 16, 128) == OK and last(L)["stream"] == "1"


def test_code_store_hint_policy_and_override(L, monkeypatch):
    """The streaming hint on the code and scale stores: on for hinted calls
    below 32 MiB of x with linear scales, off for larger calls, for the
    swizzled layout and for unhinted calls; ANQ_STREAM_CODES overrides."""
    assert tail(L, "nvfp4", 64, 8192) == OK and last(L)["stream_codes"] == "1"
    assert tail(L, "fp8", 2047, 8192) == OK and last(L)["stream_codes"] == "1"   # 31.98 MiB
    assert tail(L, "fp8", 2048, 8192) == OK and last(L)["stream_codes"] == "0"   # 32 MiB
    assert tail(L, "swizzled", 64, 8192) == OK and last(L)["stream_codes"] == "0"
    assert tail(L, "nvfp4", 16, 8192) == OK and last(L)["stream_codes"] == "0"   # unhinted
    monkeypatch.setenv("ANQ_STREAM", "0")
    assert tail(L, "nvfp4", 64, 8192) == OK and last(L)["stream_codes"] == "0"
    monkeypatch.delenv("ANQ_STREAM")
    monkeypatch.setenv("ANQ_STREAM_CODES", "0")
    assert tail(L, "nvfp4", 64, 8192) == OK and last(L)["stream_codes"] == "0"
    monkeypatch.setenv("ANQ_STREAM_CODES", "1")
    assert tail(L, "fp8", 65536, 1024) == OK and last(L)["stream_codes"] == "1"


def test_gated_table_choice(L, monkeypatch):
    g = lambda tokens, dtype=1: L.gated_rmsnorm_quant_nvfp4(  # noqa: E731
        addr(0), addr(1), addr(2), addr(3), 1e-5, tokens, 8192, 1024, dtype, addr(4), addr(6), None)
    assert g(8192) == OK and last(L)["epi"] == "5" and last(L)["block"] == "512"
    assert g(16) == OK and last(L)["epi"] == "4"                  # few rows: computed gate
    assert g(8192, dtype=0) == OK and last(L)["epi"] == "4"       # fp16 z: no table
    monkeypatch.setenv("ANQ_GATE_LUT", "0")
    assert g(8192) == OK and last(L)["epi"] == "4"
    monkeypatch.setenv("ANQ_GATE_LUT", "1")
    assert g(16) == OK and last(L)["epi"] == "5"
    monkeypatch.setenv("ANQ_GATE_BLOCK", "256")
    assert g(8192) == OK and last(L)["block"] == "256"


@pytest.mark.parametrize("tokens,hidden,group,rows,grid", [
    (8192, 8192, 1024, 8, 1024),     # 16 rows per group at 512 workgroups: halved
    (4096, 8192, 1024, 8, 512),
    (2048, 8192, 1024, 4, 512),
    (2048, 1024, 1024, 1, 256),      # fewer rows than lane groups at 512 workgroups
    (8192, 4096, 128, 8, 1024),      # 16-lane groups, 32 per workgroup
    (4096, 4096, 256, 8, 512),       # 32-lane groups
])
def test_gated_table_tiling_interleaves(L, tokens, hidden, group, rows, grid, monkeypatch):
    """The table tiling: 512-lane workgroups, rows interleaved across lane
    groups, about 512 workgroups (1024 once that leaves 8 rows per group);
    ANQ_ROW_ORDER=0 restores consecutive rows with the same grid."""
    monkeypatch.setenv("ANQ_GATE_LUT", "1")
    call = lambda: L.gated_rmsnorm_quant_nvfp4(  # noqa: E731
        addr(0), addr(1), addr(2), addr(3), 1e-5, tokens, hidden, group, 1, addr(4), addr(6), None)
    assert call() == OK
    got = last(L)
    assert got["ok"] == "1" and got["epi"] == "5" and got["block"] == "512"
    assert (got["rows"], got["grid"], got["interleave"]) == (str(rows), str(grid), "1"), got
    monkeypatch.setenv("ANQ_ROW_ORDER", "0")
    assert call() == OK
    assert (last(L)["grid"], last(L)["interleave"]) == (str(grid), "0")


@pytest.mark.parametrize("tokens,hidden,group,block,rows,grid", [
    (8192, 8192, 8192, 1024, 16, 512),   # one workgroup per CU: two waves of 256
    (8192, 8192, 4096, 512, 16, 1024),   # two per CU
    (8192, 8192, 2048, 256, 16, 2048),   # four per CU (four tables of LDS)
    (4096, 5120, 5120, 640, 8, 512),
    (300, 8192, 8192, 1024, 1, 300),     # fewer rows than resident workgroups
    (2048, 16384, 16384, 1024, 4, 512),  # two vectors per lane
    (4096, 12288, 12288, 768, 8, 512),
    (512, 32768, 32768, 1024, 1, 512),   # four vectors per lane
    (4096, 65536, 65536, 1024, 8, 512),  # eight
    (300, 40976, 40976, 704, 1, 300),    # eight, the last ones past the group end
])
def test_gated_table_wide_groups(L, tokens, hidden, group, block, rows, grid):
    """Groups of 1040 to 65536 elements use the gate table with one workgroup
    per row (one vector per lane, two past 8192 elements, four past 16384,
    eight past 32768), interleaved rows, about two waves of the workgroups the
    GPU holds at once."""
    assert L.gated_rmsnorm_quant_nvfp4(addr(0), addr(1), addr(2), addr(3), 1e-5, tokens, hidden,
                                       group, 1, addr(4), addr(6), None) == OK
    got = last(L)
    assert got["ok"] == "1" and got["epi"] == "5" and got["group"] == "0", got
    assert (got["vec_per_lane"], got["block"], got["rows"], got["grid"], got["interleave"]) == \
        (str(1 if group <= 8192 else 2 if group <= 16384 else 4 if group <= 32768 else 8),
         str(block), str(rows), str(grid), "1"), got


def test_gated_table_choice_by_size(L, monkeypatch):
    """The table is used for bf16 z in groups of 8192 or more, and in
    narrower groups once a call has 2048 group rows or 2^21 elements."""
    g = lambda tokens, hidden, group: L.gated_rmsnorm_quant_nvfp4(  # noqa: E731
        addr(0), addr(1), addr(2), addr(3), 1e-5, tokens, hidden, group, 1, addr(4), addr(6), None)
    assert g(256, 4096, 4096) == OK and last(L)["epi"] == "4"
    assert g(512, 4096, 4096) == OK and last(L)["epi"] == "5"    # 2^21 elements
    assert g(1, 8192, 8192) == OK and last(L)["epi"] == "5"      # groups of 8192 and more
    assert g(1, 16384, 8192) == OK and last(L)["epi"] == "5"
    assert g(1024, 2048, 2048) == OK and last(L)["epi"] == "5"
    assert g(512, 3072, 1536) == OK and last(L)["epi"] == "4"    # 1.5 M elements
    assert g(4096, 16384, 16384) == OK and last(L)["epi"] == "5"
    assert g(4096, 32768, 32768) == OK and last(L)["epi"] == "5"
    assert g(1, 65536, 65536) == OK and last(L)["epi"] == "5"
    monkeypatch.setenv("ANQ_GATE_LUT", "1")
    assert g(2, 16384, 16384) == OK and last(L)["epi"] == "5"
    assert g(2, 65536, 65536) == OK and last(L)["epi"] == "5"
    monkeypatch.setenv("ANQ_GATE_LUT", "0")
    assert g(8192, 8192, 8192) == OK and last(L)["epi"] == "4"


def qk(L, tokens, nq, nk, nv, D, rot=None, store=False):
    rot = D if rot is None else rot
    if store:
        return L.qk_norm_rope_fp8_kv_store(addr(0), addr(1), addr(2), addr(3), addr(4), 4096,
                                           addr(5), 1e-6, tokens, nq, nk, nv, D, rot, 1, addr(8),
                                           tokens, addr(6), addr(9), None)
    return L.qk_norm_rope_fp8(addr(0), addr(1), addr(2), addr(3), addr(4), 4096, addr(5), 1e-6,
                              tokens, nq, nk, nv, D, rot, 1, addr(6), None)


def test_qk_tilings(L, monkeypatch):
    assert qk(L, 4096, 16, 8, 8, 128) == OK
    got = last(L)
    assert got["waves"] == "1" and got["groups"] == "4" and got["block"] == "256" and got["ok"] == "1"
    assert qk(L, 64, 16, 8, 8, 128) == OK and last(L)["waves"] == "4"   # few tokens: spread heads
    assert qk(L, 4096, 64, 8, 8, 128) == OK and last(L)["groups"] == "4" and last(L)["waves"] == "3"
    monkeypatch.setenv("ANQ_QK_WAVES", "2")
    monkeypatch.setenv("ANQ_QK_BLOCK", "64")
    assert qk(L, 4096, 16, 8, 8, 512) == OK
    got = last(L)
    # 16 passes of 2 heads: 2 wavefronts would take 8 groups each, past the cap of 4
    assert got["waves"] == "4" and got["groups"] == "4"
    assert got["block"] == "128"                                        # one gamma vector per lane
    for D in (32, 64, 128, 256, 512):
        for heads in ((1, 0, 0), (4, 2, 2), (9, 5, 3), (64, 8, 8)):
            for waves in ("", "1", "2", "5"):
                monkeypatch.setenv("ANQ_QK_WAVES", waves)
                for store in (False, True):
                    assert qk(L, 23, *heads, D, store=store) == OK, (D, heads, waves)
                    assert last(L)["ok"] == "1"


def test_quant_and_stream_grids(L):
    for tokens, hidden in ((1, 16), (3, 1040), (8192, 7168), (65536, 1024)):
        for epi, fn in ((0, "quant_fp8"), (1, "quant_nvfp4"), (3, "quant_nvfp4_swizzled")):
            if epi == 0:
                st = L.quant_fp8(addr(0), addr(3), tokens, hidden, 1, addr(4), None)
            elif epi == 1:
                st = L.quant_nvfp4(addr(0), addr(3), tokens, hidden, 1, addr(4), addr(6), None)
            else:
                st = L.quant_nvfp4_swizzled(addr(0), addr(3), tokens, hidden, 1, addr(4), addr(6),
                                            None)
            assert st == OK and last(L)["ok"] == "1", (fn, tokens, hidden)
    assert L.anq_stream_rw(addr(0), 1 << 20, addr(1), 3 << 19, 1, None) == OK
    assert last(L)["kind"] == "stream" and last(L)["ok"] == "1"

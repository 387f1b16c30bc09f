"""The C-ABI library on a machine without a GPU: it loads, exports every entry
point that include/addnormq.h declares, and its host-side validation rejects
bad arguments with the documented status before any HIP call (tokens == 0 is
a no-op). No compute call is made here.

With ANQ_HOSTCHECK_LIB set (tests/test_hostcheck.py does this), the same tests
run against the host-only build of the front end under AddressSanitizer and
UndefinedBehaviorSanitizer instead of the product library."""
import ctypes
import os
import re

import pytest

import nvfp4_quantization_place_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "addnormq.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, UNSUP, LAUNCH, VALUE, CONFIG = range(10)
HOSTCHECK = os.environ.get("ANQ_HOSTCHECK_LIB")

# fake, well-aligned, disjoint device addresses: validation never dereferences them
BASE = 1 << 40
MB = 1 << 20


def addr(i, off=0):
    return BASE + i * 64 * MB + off


@pytest.fixture(scope="module")
def L():
    if HOSTCHECK:
        saved = A._lib
        A._lib = A.load(HOSTCHECK)
        yield A._lib
        A._lib = saved
        return
    if not os.path.exists(A.LIB_PATH):
        from nvfp4_quantization_place_amd import build
        build.build()
    yield A.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["add_rmsnorm_quant_fp8", "add_rmsnorm_quant_nvfp4",
                                           "qk_norm_rope_fp8", "qk_norm_rope_fp8_kv_store",
                                           "add_rmsnorm", "quant_fp8",
                                           "quant_nvfp4", "add_rmsnorm_quant_nvfp4_swizzled",
                                           "quant_nvfp4_swizzled", "anq_nvfp4_swizzled_sf_shape",
                                           "gated_rmsnorm_quant_nvfp4", "silu_gate_f32",
                                           "anq_nvfp4_shape", "anq_selfcheck_arith",
                                           "anq_status_string", "anq_stream_rw",
                                           "qk_norm_rope_kv_store_mixed"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    # exported as plain C symbols (no C++ mangling)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", HOSTCHECK or A.LIB_PATH],
                         capture_output=True, text=True).stdout
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


def test_status_strings(L):
    for code in range(10):
        s = A.status_string(code)
        assert s and s != "unknown status"
    assert A.status_string(99) == "unknown status"


def test_nvfp4_shape_helper(L):
    assert A.nvfp4_shape(64, 8192) == (4096, 512)
    assert A.nvfp4_shape(8192, 7168) == (3584, 448)
    assert A.nvfp4_shape(0, 16) == (8, 1)
    q, s = ctypes.c_int64(), ctypes.c_int64()
    assert L.anq_nvfp4_shape(4, 24, ctypes.byref(q), ctypes.byref(s)) == SHAPE
    assert L.anq_nvfp4_shape(4, 0, ctypes.byref(q), ctypes.byref(s)) == SHAPE
    assert L.anq_nvfp4_shape(-1, 16, ctypes.byref(q), ctypes.byref(s)) == SHAPE
    assert L.anq_nvfp4_shape(4, 16, None, ctypes.byref(s)) == NULL


def test_swizzled_sf_shape_helper(L):
    assert A.nvfp4_swizzled_sf_shape(64, 8192) == (128, 512)
    assert A.nvfp4_swizzled_sf_shape(8192, 7168) == (8192, 448)
    assert A.nvfp4_swizzled_sf_shape(300, 1040) == (384, 68)     # 65 blocks -> 68
    assert A.nvfp4_swizzled_sf_shape(0, 16) == (0, 4)
    assert A.nvfp4_swizzled_sf_shape(1, 16) == (128, 4)
    r, c = ctypes.c_int64(), ctypes.c_int64()
    assert L.anq_nvfp4_swizzled_sf_shape(4, 24, ctypes.byref(r), ctypes.byref(c)) == SHAPE
    assert L.anq_nvfp4_swizzled_sf_shape(-1, 16, ctypes.byref(r), ctypes.byref(c)) == SHAPE
    assert L.anq_nvfp4_swizzled_sf_shape(4, 16, ctypes.byref(r), None) == NULL


def test_swizzled_nvfp4_validation(L):
    def sw(**kw):
        a = dict(x=addr(0), res=addr(1), gamma=addr(2), scale=addr(3), eps=1e-6, tokens=0,
                 hidden=128, dtype=1, q=addr(4), sf=addr(6), norm=addr(5), stream=None)
        a.update(kw)
        return L.add_rmsnorm_quant_nvfp4_swizzled(a["x"], a["res"], a["gamma"], a["scale"],
                                                  a["eps"], a["tokens"], a["hidden"], a["dtype"],
                                                  a["q"], a["sf"], a["norm"], a["stream"])

    def qs(**kw):
        a = dict(t=addr(0), scale=addr(3), tokens=0, hidden=128, dtype=1, q=addr(4), sf=addr(6))
        a.update(kw)
        return L.quant_nvfp4_swizzled(a["t"], a["scale"], a["tokens"], a["hidden"], a["dtype"],
                                      a["q"], a["sf"], None)

    for op in (sw, qs):
        assert op() == OK
        assert op(sf=addr(6, 2)) == ALIGN                 # swizzled scales: 4-byte words
        assert op(sf=addr(6, 4)) == OK
        assert op(tokens=4, sf=None) == NULL
        assert op(hidden=40) == SHAPE
        # the padded scale buffer (128 rows x 8 cols = 1 KiB for 1 token) may not reach q,
        # although the 8 linear scale bytes of that token would end 992 bytes before it
        assert op(tokens=1, sf=addr(4) - 1000) == ALIAS
    assert sw(hidden=65536 + 16) == UNSUP
    assert nvfp4(L, sf=addr(6, 2)) == OK                  # the linear layout has no alignment rule


def test_gated_validation(L):
    def g(**kw):
        a = dict(x=addr(0), z=addr(1), gamma=addr(2), scale=addr(3), eps=1e-6, tokens=0,
                 hidden=1024, group=256, dtype=1, q=addr(4), sf=addr(6))
        a.update(kw)
        return L.gated_rmsnorm_quant_nvfp4(a["x"], a["z"], a["gamma"], a["scale"], a["eps"],
                                           a["tokens"], a["hidden"], a["group"], a["dtype"],
                                           a["q"], a["sf"], None)

    assert g() == OK
    for k in ("x", "z", "q", "sf"):
        assert g(tokens=4, **{k: None}) == NULL, k
        assert g(tokens=0, **{k: None}) == OK, k
    assert g(gamma=None) == NULL and g(scale=None) == NULL
    for grp in (0, -16, 24, 384, 2048):       # not a multiple of 16, or not dividing hidden
        assert g(group=grp) == SHAPE, grp
    assert g(hidden=1 << 17, group=1 << 17) == UNSUP        # one group wider than a row kernel takes
    assert g(hidden=1 << 17, group=1024) == OK              # wide rows of narrow groups are fine
    assert g(dtype=4) == DTYPE
    assert g(eps=float("nan")) == VALUE
    assert g(z=addr(1, 8)) == ALIGN
    assert g(tokens=4, q=addr(1)) == ALIAS                   # codes over z
    gate = L.silu_gate_f32
    assert gate(addr(0), addr(1), 0, 1, addr(2), None) == OK
    assert gate(None, addr(1), 8, 1, addr(2), None) == NULL
    assert gate(addr(0), addr(1), 12, 1, addr(2), None) == SHAPE
    assert gate(addr(0), addr(1), 8, 2, addr(2), None) == DTYPE
    assert gate(addr(0), addr(1), 8, 1, addr(2, 4), None) == ALIGN
    assert gate(addr(0), addr(1), 8, 1, addr(1), None) == ALIAS
    assert g(tokens=4, sf=addr(4, 16)) == ALIAS              # scales over the codes


def test_stream_validation(L):
    """The calibration stream: sizes in 16-byte units, something to write,
    aligned and disjoint buffers."""
    s = L.anq_stream_rw
    assert s(addr(0), 0, addr(1), 0, 1, None) == OK
    assert s(None, 16, addr(1), 16, 1, None) == NULL
    assert s(addr(0), 16, None, 16, 1, None) == NULL
    assert s(None, 0, addr(1), 0, 1, None) == OK
    assert s(addr(0), 24, addr(1), 16, 1, None) == SHAPE
    assert s(addr(0), 16, addr(1), 8, 1, None) == SHAPE
    assert s(addr(0), 32, addr(1), 0, 1, None) == SHAPE      # reads with nothing to write
    assert s(addr(0), -16, addr(1), 16, 1, None) == SHAPE
    assert s(addr(0), 16, addr(1), 16, 2, None) == VALUE
    assert s(addr(0, 8), 16, addr(1), 16, 1, None) == ALIGN
    assert s(addr(0), 64, addr(0, 32), 64, 1, None) == ALIAS


def test_selfcheck_validation(L):
    """The arithmetic self-check rejects a missing or misaligned count array
    before any device work."""
    assert L.anq_selfcheck_arith(None, None) == NULL
    assert L.anq_selfcheck_arith(addr(0, 4), None) == ALIGN


def fp8(L, **kw):
    a = dict(x=addr(0), res=addr(1), gamma=addr(2), scale=addr(3), eps=1e-6, tokens=0,
             hidden=128, dtype=0, q=addr(4), norm=addr(5), stream=None)
    a.update(kw)
    return L.add_rmsnorm_quant_fp8(a["x"], a["res"], a["gamma"], a["scale"], a["eps"], a["tokens"],
                                   a["hidden"], a["dtype"], a["q"], a["norm"], a["stream"])


def nvfp4(L, **kw):
    a = dict(x=addr(0), res=addr(1), gamma=addr(2), scale=addr(3), eps=1e-6, tokens=0,
             hidden=128, dtype=1, q=addr(4), sf=addr(6), norm=addr(5), stream=None)
    a.update(kw)
    return L.add_rmsnorm_quant_nvfp4(a["x"], a["res"], a["gamma"], a["scale"], a["eps"],
                                     a["tokens"], a["hidden"], a["dtype"], a["q"], a["sf"],
                                     a["norm"], a["stream"])


def qk(L, **kw):
    a = dict(qkv=addr(0), gq=addr(1), gk=addr(2), pos=addr(3), cs=addr(4), max_pos=4096,
             scale=addr(5), eps=1e-6, tokens=0, nq=16, nk=8, nv=8, D=128, rot=128, dtype=1,
             out=addr(6), stream=None)
    a.update(kw)
    return L.qk_norm_rope_fp8(a["qkv"], a["gq"], a["gk"], a["pos"], a["cs"], a["max_pos"],
                              a["scale"], a["eps"], a["tokens"], a["nq"], a["nk"], a["nv"], a["D"],
                              a["rot"], a["dtype"], a["out"], a["stream"])


@pytest.mark.parametrize("op", [fp8, nvfp4])
def test_row_ops_validation(L, op):
    assert op(L) == OK                                   # tokens == 0: no-op, no HIP call
    assert op(L, norm=None) == OK                        # norm_out is optional
    for k in ("x", "res", "gamma", "scale", "q"):
        assert op(L, tokens=4, **{k: None}) == NULL, k
    for k in ("x", "res", "q", "norm"):                  # empty tensors carry NULL pointers
        assert op(L, tokens=0, **{k: None}) == OK, k
    for k in ("gamma", "scale"):
        assert op(L, tokens=0, **{k: None}) == NULL, k
    assert op(L, dtype=2) == DTYPE
    assert op(L, dtype=-1) == DTYPE
    for h in (0, -16, 24, 100, 8):
        assert op(L, hidden=h) == SHAPE, h
    assert op(L, tokens=-1) == SHAPE
    assert op(L, hidden=65536 + 16) == UNSUP
    assert op(L, tokens=1 << 60, hidden=1024) == SHAPE   # size overflow
    for eps in (-1e-6, float("nan"), float("inf")):
        assert op(L, eps=eps) == VALUE
    for k in ("x", "res", "gamma", "q", "norm"):
        assert op(L, **{k: addr(7, 8)}) == ALIGN, k
    assert op(L, scale=addr(3, 2)) == ALIGN
    assert op(L, scale=addr(3, 4)) == OK                 # 4-byte aligned scalar is fine


def test_row_ops_alias_rules(L):
    t, h = 16, 128
    act = t * h * 2
    # every case below with tokens > 0 is rejected before any HIP call
    assert fp8(L, tokens=t, hidden=h, res=addr(0)) == ALIAS   # x is read while residual is written
    assert fp8(L, tokens=0, hidden=h, res=addr(0)) == OK      # empty buffers overlap nothing
    assert fp8(L, tokens=t, hidden=h, q=addr(1, act - 16)) == ALIAS  # q overlaps residual's tail
    assert fp8(L, tokens=t, hidden=h, norm=addr(4, 16)) == ALIAS     # norm_out overlaps q
    assert fp8(L, tokens=t, hidden=h, scale=addr(4, 4)) == ALIAS     # scale inside q
    assert fp8(L, tokens=0, hidden=h, gamma=addr(0)) == OK           # read-only inputs may overlap
    assert nvfp4(L, tokens=t, hidden=h, sf=addr(4, 16)) == ALIAS     # sf inside q
    assert nvfp4(L, tokens=4, sf=None) == NULL
    assert nvfp4(L, tokens=0, sf=None) == OK


def test_qk_validation(L):
    assert qk(L) == OK
    for k in ("qkv", "pos", "cs", "scale", "out"):
        assert qk(L, tokens=4, **{k: None}) == NULL, k
    for k in ("qkv", "pos", "out"):
        assert qk(L, tokens=0, **{k: None}) == OK, k
    assert qk(L, gq=None) == NULL
    assert qk(L, gq=None, nq=0) == OK                   # gamma_q unused without Q heads
    assert qk(L, gk=None, nk=0) == OK
    assert qk(L, dtype=5) == DTYPE
    for rot in (16, 32, 64):                             # the last rot elements rotate
        assert qk(L, rot=rot) == OK, rot
    for rot in (0, 8, 48, 96, 256, -128):                # below 16, not a power of two, past D
        assert qk(L, rot=rot) == UNSUP, rot
    for d in (48, 96, 1024, 16):
        assert qk(L, D=d, rot=d) == UNSUP, d
    assert qk(L, nq=-1) == VALUE
    assert qk(L, max_pos=0) == VALUE
    assert qk(L, nq=0, nk=0, nv=0) == SHAPE
    big = 2 ** 31 - 1                                    # head counts summed in 64 bits
    assert qk(L, tokens=4, nq=big, nk=big, nv=big) == SHAPE
    assert qk(L, tokens=4, nq=(1 << 20) + 1, nk=0, nv=0) == SHAPE
    assert qks(L, tokens=4, nq=0, nk=big, nv=big) == SHAPE
    assert qk(L, tokens=-2) == SHAPE
    assert qk(L, eps=-1.0) == VALUE
    assert qk(L, qkv=addr(0, 8)) == ALIGN
    assert qk(L, pos=addr(3, 4)) == ALIGN
    assert qk(L, tokens=4, out=addr(0)) == ALIAS        # rejected before any HIP call
    assert qk(L, tokens=4, cs=addr(6)) == ALIAS
    assert qk(L, tokens=4, pos=addr(6, 8)) == ALIAS


def qks(L, **kw):
    a = dict(qkv=addr(0), gq=addr(1), gk=addr(2), pos=addr(3), cs=addr(4), max_pos=4096,
             scale=addr(5), eps=1e-6, tokens=0, nq=16, nk=8, nv=8, D=128, rot=128, dtype=1,
             slots=addr(8), num_slots=1024, q=addr(6), kv=addr(9), stream=None)
    a.update(kw)
    return L.qk_norm_rope_fp8_kv_store(a["qkv"], a["gq"], a["gk"], a["pos"], a["cs"], a["max_pos"],
                                       a["scale"], a["eps"], a["tokens"], a["nq"], a["nk"], a["nv"],
                                       a["D"], a["rot"], a["dtype"], a["slots"], a["num_slots"],
                                       a["q"], a["kv"], a["stream"])


def test_qk_kv_store_validation(L):
    assert qks(L) == OK
    for k in ("qkv", "pos", "q", "slots", "kv"):
        assert qks(L, tokens=4, **{k: None}) == NULL, k
        assert qks(L, tokens=0, **{k: None}) == OK, k
    assert qks(L, nq=0, q=None, gq=None) == OK           # no Q heads: q_out unused
    assert qks(L, nk=0, nv=0, slots=None, kv=None) == OK  # no K/V heads: no pool
    assert qks(L, num_slots=-1) == VALUE
    assert qks(L, rot=64) == OK
    assert qks(L, rot=24) == UNSUP
    assert qks(L, kv=addr(9, 8)) == ALIGN
    assert qks(L, slots=addr(8, 4)) == ALIGN
    assert qks(L, tokens=4, kv=addr(0)) == ALIAS         # pool over qkv
    assert qks(L, tokens=4, kv=addr(6)) == ALIAS         # pool over q_out
    assert qks(L, tokens=4, slots=addr(9)) == ALIAS      # slots inside the pool
    assert qks(L, tokens=4, num_slots=1 << 62) == SHAPE  # pool size overflow


def qkm(L, **kw):
    a = dict(qkv=addr(0), gq=addr(1), gk=addr(2), pos=addr(3), cs=addr(4), max_pos=4096,
             scale=addr(5), eps=1e-6, tokens=0, nq=16, nk=8, nv=8, D=128, rot=64, dtype=1,
             slots=addr(8), num_slots=1024, q=addr(6), kv=addr(9), stream=None)
    a.update(kw)
    return L.qk_norm_rope_kv_store_mixed(a["qkv"], a["gq"], a["gk"], a["pos"], a["cs"],
                                         a["max_pos"], a["scale"], a["eps"], a["tokens"], a["nq"],
                                         a["nk"], a["nv"], a["D"], a["rot"], a["dtype"], a["slots"],
                                         a["num_slots"], a["q"], a["kv"], a["stream"])


def test_qk_mixed_store_validation(L):
    """The mixed pool's rows are nk*(D+R) + nv*D bytes: the alias check uses
    that size, and a pool whose rows are that wide may end right before
    another buffer."""
    assert qkm(L) == OK
    for k in ("qkv", "pos", "q", "slots", "kv"):
        assert qkm(L, tokens=4, **{k: None}) == NULL, k
        assert qkm(L, tokens=0, **{k: None}) == OK, k
    assert qkm(L, nk=0, nv=0, slots=None, kv=None) == OK
    assert qkm(L, rot=128) == OK                         # the whole head in bf16
    for rot in (8, 24, 256):
        assert qkm(L, rot=rot) == UNSUP, rot
    assert qkm(L, num_slots=-1) == VALUE
    assert qkm(L, kv=addr(9, 8)) == ALIGN
    row = 8 * (128 + 64) + 8 * 128                       # 2560 bytes per slot
    # a pool ending where q_out starts passes validation (then the launch: no GPU here, so
    # ANQ_ERR_LAUNCH from the product library, ANQ_OK from the host-check build)
    assert qkm(L, tokens=4, num_slots=4, kv=addr(6) - 4 * row) in (OK, LAUNCH)
    assert qkm(L, tokens=4, num_slots=4, kv=addr(6) - 4 * row + 16) == ALIAS
    assert qkm(L, tokens=4, cs=addr(9) + 1024 * row - 16) == ALIAS        # table inside the pool
    assert qkm(L, tokens=4, num_slots=1 << 62) == SHAPE


def addnorm(L, **kw):
    a = dict(x=addr(0), res=addr(1), gamma=addr(2), eps=1e-6, tokens=0, hidden=128, dtype=1,
             norm=addr(5), stream=None)
    a.update(kw)
    return L.add_rmsnorm(a["x"], a["res"], a["gamma"], a["eps"], a["tokens"], a["hidden"],
                         a["dtype"], a["norm"], a["stream"])


def qfp8(L, **kw):
    a = dict(t=addr(0), scale=addr(3), tokens=0, hidden=128, dtype=0, q=addr(4), stream=None)
    a.update(kw)
    return L.quant_fp8(a["t"], a["scale"], a["tokens"], a["hidden"], a["dtype"], a["q"], a["stream"])


def qnv(L, **kw):
    a = dict(t=addr(0), scale=addr(3), tokens=0, hidden=128, dtype=1, q=addr(4), sf=addr(6),
             stream=None)
    a.update(kw)
    return L.quant_nvfp4(a["t"], a["scale"], a["tokens"], a["hidden"], a["dtype"], a["q"], a["sf"],
                         a["stream"])


def test_separated_tail_validation(L):
    assert addnorm(L) == OK
    for k in ("x", "res", "norm"):
        assert addnorm(L, tokens=4, **{k: None}) == NULL, k
        assert addnorm(L, tokens=0, **{k: None}) == OK, k
    assert addnorm(L, gamma=None) == NULL
    assert addnorm(L, hidden=24) == SHAPE
    assert addnorm(L, hidden=65536 + 16) == UNSUP
    assert addnorm(L, dtype=7) == DTYPE
    assert addnorm(L, eps=-1.0) == VALUE
    assert addnorm(L, norm=addr(5, 8)) == ALIGN
    assert addnorm(L, tokens=4, norm=addr(1)) == ALIAS      # norm over residual
    assert addnorm(L, tokens=4, res=addr(0)) == ALIAS       # residual over x
    for op in (qfp8, qnv):
        assert op(L) == OK
        assert op(L, tokens=4, t=None) == NULL
        assert op(L, tokens=0, t=None, q=None) == OK
        assert op(L, scale=None) == NULL
        assert op(L, hidden=40) == SHAPE
        assert op(L, hidden=1 << 20) == OK                  # no row-width limit below 2^34
        assert op(L, hidden=1 << 35) == SHAPE               # 16-byte vectors per row beyond int32
        assert op(L, dtype=9) == DTYPE
        assert op(L, t=addr(0, 8)) == ALIGN
        assert op(L, scale=addr(3, 2)) == ALIGN
        assert op(L, tokens=4, q=addr(0, 16)) == ALIAS       # codes over the input
        assert op(L, tokens=4, scale=addr(4, 4)) == ALIAS
    assert qnv(L, tokens=4, sf=None) == NULL
    assert qnv(L, tokens=4, sf=addr(4, 32)) == ALIAS         # scales over the codes


def test_gate_exp2_table_is_correctly_rounded():
    """The binary64 literals of the gate's exp table are 2^(j/64), j < 64, each
    the nearest binary64 (checked with 60-digit decimal arithmetic)."""
    from decimal import Decimal, localcontext
    src = open(os.path.join(ROOT, "nvfp4_quantization_place_amd", "csrc", "anq_device.h")).read()
    body = src[src.index("kExp2Tab[64] = {"):].split("}", 1)[0]
    vals = [float.fromhex(t) for t in re.findall(r"0x[0-9a-f.]+p[+-]\d+", body)]
    assert len(vals) == 64
    with localcontext() as ctx:
        ctx.prec = 60
        for j, v in enumerate(vals):
            exact = Decimal(2) ** (Decimal(j) / 64)
            assert float(exact) == v, j                      # float(Decimal) rounds to nearest


def test_product_fails_loudly_without_library_or_gpu(monkeypatch):
    """There is no CPU path: a missing library raises, and CPU tensors are
    refused before any library call."""
    import torch
    monkeypatch.setattr(A, "_lib", None)
    monkeypatch.setattr(A, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libaddnormq.so"))
    with pytest.raises(RuntimeError, match="missing"):
        A.lib()
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        A.add_rmsnorm_quant_nvfp4(x, x.clone(), torch.ones(64, dtype=torch.bfloat16),
                                  torch.ones(1), 1e-6)
    with pytest.raises(ValueError, match="GPU"):
        A.quant_fp8(x, torch.ones(1))
    # prepare() runs the same checks and leaves no recording behind
    with pytest.raises(ValueError, match="GPU"):
        A.prepare(A.add_rmsnorm_quant_nvfp4, x, x.clone(), torch.ones(64, dtype=torch.bfloat16),
                  torch.ones(1), 1e-6)
    assert A._record is None

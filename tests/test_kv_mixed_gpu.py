"""GPU parity of the Q/K op with a partial rotary width and of its mixed KV
pool (E4M3 for the unrotated part of each K head, bf16 for the rotated part),
against the oracle, byte for byte: the plain op's codes, the uniform pool and
the mixed pool over head_dim x rotary_dim x head layouts x dtype, with and
without streaming hints and with several wavefronts per token; every pool
row no token names keeps its sentinel bytes, and nothing is written past the
outputs."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5
DIMS = [(D, R) for D in (32, 64, 128, 256, 512) for R in (16, 32, 64, 128, 256, 512) if R <= D]
HEADS = [(4, 2, 2), (3, 1, 0), (0, 2, 1), (1, 0, 3), (0, 3, 0), (9, 5, 3)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _A():
    import nvfp4_quantization_place_amd as A
    return A


def _slots(rng, tokens, num_slots):
    s = rng.permutation(num_slots)[:tokens].astype(np.int64)
    s[rng.random(tokens) < 0.1] = -1
    if tokens > 3:
        s[3] = num_slots + 5          # past the pool: stores nothing
    return s


def _dev_args(inp):
    return (inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(), inp.positions.cuda(),
            torch.from_numpy(inp.cos_sin).cuda(),
            torch.tensor([inp.scale], dtype=torch.float32, device="cuda"), inp.eps, inp.nq, inp.nk,
            inp.nv, inp.head_dim)


def _ora_args(inp):
    return (W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
            inp.cos_sin, inp.scale, inp.eps, inp.nq, inp.nk, inp.nv, inp.head_dim)


def _inp(D, R, heads, dtype, tokens=21, seed=0):
    rng = np.random.default_rng(D * 7 + R + seed)
    pos = rng.integers(0, 200, tokens)
    return W.make_qk(D + R + 3 * heads[0] + heads[1] + seed, dtype, tokens, *heads, D,
                     positions=pos, max_pos=200, rotary_dim=R, scale=0.03)


@pytest.mark.parametrize("stream", ["", "0"])
@pytest.mark.parametrize("heads", HEADS)
@pytest.mark.parametrize("D,R", DIMS)
def test_mixed_pool_grid(D, R, heads, stream, monkeypatch):
    monkeypatch.setenv("ANQ_STREAM", stream)
    dtype = "bf16" if (D + R + heads[0]) % 2 else "f16"
    inp = _inp(D, R, heads, dtype)
    A = _A()
    nq, nk, nv = heads
    rng = np.random.default_rng(D + R)
    num_slots = 40
    slots = _slots(rng, inp.tokens, num_slots)
    width = A.mixed_kv_row_bytes(nk, nv, D, R)
    pool = torch.full((num_slots, width), SENTINEL, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_kv_store_mixed(*_dev_args(inp), R, torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope_kv_store_mixed(*_ora_args(inp), R, dtype, slots,
                                        np.full((num_slots, width), SENTINEL, np.uint8))
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(pool), ref["kv"])


@pytest.mark.parametrize("heads", [(4, 2, 2), (1, 0, 3), (9, 5, 3)])
@pytest.mark.parametrize("D,R", [(64, 16), (128, 32), (128, 64), (256, 128), (512, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_partial_rotary_plain_and_uniform_pool(D, R, heads, dtype):
    """The plain op and the uniform FP8 pool with a partial rotary width."""
    inp = _inp(D, R, heads, dtype, seed=1)
    A = _A()
    out = A.qk_norm_rope_fp8(*_dev_args(inp), rotary_dim=R)
    num_slots = 30
    slots = _slots(np.random.default_rng(R), inp.tokens, num_slots)
    nq, nk, nv = heads
    pool = torch.full((num_slots, (nk + nv) * D), SENTINEL, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_fp8_kv_store(*_dev_args(inp), torch.from_numpy(slots).cuda(), pool,
                                    rotary_dim=R)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope_fp8(*_ora_args(inp), dtype, rotary_dim=R)
    np.testing.assert_array_equal(_np(out), ref["out"])
    refs = O.qk_norm_rope_fp8_kv_store(*_ora_args(inp), dtype, slots,
                                       np.full((num_slots, (nk + nv) * D), SENTINEL, np.uint8),
                                       rotary_dim=R)
    np.testing.assert_array_equal(_np(q), refs["q"])
    np.testing.assert_array_equal(_np(pool), refs["kv"])


@pytest.mark.parametrize("waves", ["1", "2", "3", "5"])
@pytest.mark.parametrize("block", ["", "64", "1024"])
def test_mixed_pool_waves_and_blocks(waves, block, monkeypatch):
    """Splitting a token's heads over several wavefronts and packing them into
    workgroups of other sizes changes no byte of the mixed pool."""
    monkeypatch.setenv("ANQ_QK_WAVES", waves)
    monkeypatch.setenv("ANQ_QK_BLOCK", block)
    inp = _inp(128, 64, (9, 5, 3), "bf16", tokens=23, seed=2)
    A = _A()
    num_slots = 30
    slots = _slots(np.random.default_rng(9), inp.tokens, num_slots)
    width = A.mixed_kv_row_bytes(5, 3, 128, 64)
    pool = torch.full((num_slots, width), SENTINEL, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_kv_store_mixed(*_dev_args(inp), 64, torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope_kv_store_mixed(*_ora_args(inp), 64, "bf16", slots,
                                        np.full((num_slots, width), SENTINEL, np.uint8))
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(pool), ref["kv"])


@pytest.mark.parametrize("groups", ["4", "3", "2"])
@pytest.mark.parametrize("D,R,heads", [(128, 128, (16, 8, 8)), (128, 64, (16, 8, 8)),
                                       (64, 64, (32, 16, 16)), (256, 256, (7, 5, 4)),
                                       (256, 64, (8, 4, 4))])
@pytest.mark.parametrize("stream", ["", "0"])
def test_mixed_pool_several_groups_per_wavefront(D, R, heads, groups, stream, monkeypatch):
    """One wavefront per token taking up to four head groups, all computed
    before any is stored (the layout of large calls): every group's codes and
    bf16 halves reach their own heads, with the whole head rotated too."""
    monkeypatch.setenv("ANQ_QK_WAVES", "1")
    monkeypatch.setenv("ANQ_QK_GROUPS", groups)
    monkeypatch.setenv("ANQ_STREAM", stream)
    inp = _inp(D, R, heads, "bf16", tokens=19, seed=4)
    A = _A()
    nq, nk, nv = heads
    num_slots = 32
    slots = _slots(np.random.default_rng(D + R + 4), inp.tokens, num_slots)
    width = A.mixed_kv_row_bytes(nk, nv, D, R)
    pool = torch.full((num_slots, width), SENTINEL, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_kv_store_mixed(*_dev_args(inp), R, torch.from_numpy(slots).cuda(), pool)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope_kv_store_mixed(*_ora_args(inp), R, "bf16", slots,
                                        np.full((num_slots, width), SENTINEL, np.uint8))
    np.testing.assert_array_equal(_np(q), ref["q"])
    np.testing.assert_array_equal(_np(pool), ref["kv"])


def test_mixed_pool_writes_nothing_outside_its_outputs():
    """q_out and the pool sit inside larger buffers filled with a canary; every
    byte outside them keeps it."""
    A = _A()
    inp = _inp(256, 64, (4, 2, 2), "bf16", tokens=17, seed=3)
    width = A.mixed_kv_row_bytes(2, 2, 256, 64)
    num_slots = 20
    slots = np.arange(17, dtype=np.int64)[::-1].copy()
    qbig = torch.full((17 * 4 * 256 + 4096,), 0x3C, dtype=torch.uint8, device="cuda")
    pbig = torch.full((num_slots * width + 4096,), 0x3C, dtype=torch.uint8, device="cuda")
    q = qbig[2048:2048 + 17 * 4 * 256].view(17, 4 * 256)
    pool = pbig[2048:2048 + num_slots * width].view(num_slots, width)
    pool.fill_(SENTINEL)
    A.qk_norm_rope_kv_store_mixed(*_dev_args(inp), 64, torch.from_numpy(slots).cuda(), pool,
                                  q_out=q)
    torch.cuda.synchronize()
    for big, lo, hi in ((qbig, 2048, 2048 + q.numel()), (pbig, 2048, 2048 + pool.numel())):
        b = big.cpu().numpy()
        assert np.all(b[:lo] == 0x3C) and np.all(b[hi:] == 0x3C)
    ref = O.qk_norm_rope_kv_store_mixed(*_ora_args(inp), 64, "bf16", slots,
                                        np.full((num_slots, width), SENTINEL, np.uint8))
    np.testing.assert_array_equal(_np(pool), ref["kv"])
    np.testing.assert_array_equal(_np(q), ref["q"])


def test_mixed_pool_equals_the_plain_op_rounded():
    """GPU against GPU: the mixed pool's FP8 bytes are the plain op's codes of
    the unrotated part of each K head and of the V heads, and its Q codes are
    the plain op's."""
    A = _A()
    D, R = 128, 64
    inp = _inp(D, R, (4, 2, 2), "bf16", tokens=64, seed=4)
    plain = _np(A.qk_norm_rope_fp8(*_dev_args(inp), rotary_dim=R)).reshape(64, 8, D)
    width = A.mixed_kv_row_bytes(2, 2, D, R)
    pool = torch.zeros((64, width), dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_kv_store_mixed(*_dev_args(inp), R,
                                      torch.arange(64, dtype=torch.int64, device="cuda"), pool)
    torch.cuda.synchronize()
    p = _np(pool)
    assert np.array_equal(_np(q), plain[:, :4].reshape(64, -1))
    for j in range(2):
        kh = p[:, j * (D + R):(j + 1) * (D + R)]
        assert np.array_equal(kh[:, :D - R], plain[:, 4 + j, :D - R])
    assert np.array_equal(p[:, 2 * (D + R):], plain[:, 6:].reshape(64, -1))


def test_mixed_pool_empty_and_errors():
    A = _A()
    inp = _inp(64, 32, (2, 1, 1), "f16", tokens=4, seed=5)
    width = A.mixed_kv_row_bytes(1, 1, 64, 32)
    empty = W.make_qk(1, "f16", 0, 2, 1, 1, 64, rotary_dim=32)
    pool = torch.zeros(4, width, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_kv_store_mixed(*_dev_args(empty), 32,
                                      torch.zeros(0, dtype=torch.int64, device="cuda"), pool)
    assert q.shape == (0, 128) and not pool.any()
    for bad_r in (8, 48, 128):   # below 16, not a power of two, past head_dim: unsupported
        bad = W.make_qk(1, "f16", 4, 2, 1, 1, 64, rotary_dim=bad_r)
        with pytest.raises(A.AnqError) as e:
            A.qk_norm_rope_kv_store_mixed(*_dev_args(bad), bad_r,
                                          torch.zeros(4, dtype=torch.int64, device="cuda"),
                                          torch.zeros(4, A.mixed_kv_row_bytes(1, 1, 64, bad_r),
                                                      dtype=torch.uint8, device="cuda"))
        assert e.value.code == 6
        with pytest.raises(A.AnqError) as e:
            A.qk_norm_rope_fp8(*_dev_args(bad), rotary_dim=bad_r)
        assert e.value.code == 6
    with pytest.raises(ValueError):                # a table narrower than the rotary width
        A.qk_norm_rope_fp8(*_dev_args(inp), rotary_dim=64)
    assert not pool.any()

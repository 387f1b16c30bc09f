"""GPU parity of the Q/K norm + RoPE + FP8 op with the KV-cache store
epilogue (SGLang PR #32975: norm + RoPE + store into a uniform FP8 pool)
against the oracle's scatter of the plain op's codes. Every byte is compared,
pool rows that no token names included.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from runners import _np

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _slots(rng, tokens, num_slots, pad_frac=0.1):
    """Distinct slots drawn from the pool, some tokens padded (-1) and one
    pointing past the pool (stores nothing)."""
    s = rng.permutation(num_slots)[:tokens].astype(np.int64)
    s[rng.random(tokens) < pad_frac] = -1
    if tokens > 3:
        s[3] = num_slots + 7
    return s


def _run(inp, slots, num_slots, stream=None):
    import nvfp4_quantization_place_amd as A
    kvw = (inp.nk + inp.nv) * inp.head_dim
    pool = torch.full((num_slots, kvw), SENTINEL, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_fp8_kv_store(
        inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(), inp.positions.cuda(),
        torch.from_numpy(inp.cos_sin).cuda(),
        torch.tensor([inp.scale], dtype=torch.float32, device="cuda"), inp.eps,
        inp.nq, inp.nk, inp.nv, inp.head_dim, torch.from_numpy(slots).cuda(), pool, stream=stream)
    torch.cuda.synchronize()
    return _np(q), _np(pool)


def _oracle(inp, slots, num_slots):
    kvw = (inp.nk + inp.nv) * inp.head_dim
    return O.qk_norm_rope_fp8_kv_store(
        W.bits(inp.qkv), W.bits(inp.gamma_q), W.bits(inp.gamma_k), inp.positions.numpy(),
        inp.cos_sin, inp.scale, inp.eps, inp.nq, inp.nk, inp.nv, inp.head_dim, inp.dtype, slots,
        np.full((num_slots, kvw), SENTINEL, np.uint8))


@pytest.mark.parametrize("stream", ["", "1"])
@pytest.mark.parametrize("head_dim", [32, 64, 128, 256, 512])
@pytest.mark.parametrize("heads", [(4, 2, 2), (3, 1, 0), (0, 2, 1), (2, 0, 0), (0, 0, 3)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_kv_store_grid(head_dim, heads, dtype, stream, monkeypatch):
    monkeypatch.setenv("ANQ_STREAM", stream)
    nq, nk, nv = heads
    tokens, num_slots = 37, 64
    rng = np.random.default_rng(head_dim * 7 + nq * 3 + nk + nv)
    inp = W.make_qk(head_dim + 31 * nq + nv, dtype, tokens, nq, nk, nv, head_dim,
                    positions=rng.integers(0, 200, tokens), max_pos=200, scale=0.04)
    slots = _slots(rng, tokens, num_slots)
    q, kv = _run(inp, slots, num_slots)
    ref = _oracle(inp, slots, num_slots)
    np.testing.assert_array_equal(q, ref["q"])
    np.testing.assert_array_equal(kv, ref["kv"])


def test_kv_store_workload_size():
    """The Q/K workload (4096 tokens, 16 Q + 8 K + 8 V heads of 128, bf16) into
    a paged pool of 512 blocks x 16 slots, slots shuffled, a tenth padded."""
    inp = W.make_config(5)
    print(f"workload {inp.name} with a KV store", flush=True)
    rng = np.random.default_rng(55)
    num_slots = 512 * 16
    slots = _slots(rng, inp.tokens, num_slots)
    q, kv = _run(inp, slots, num_slots)
    ref = _oracle(inp, slots, num_slots)
    np.testing.assert_array_equal(q, ref["q"])
    np.testing.assert_array_equal(kv, ref["kv"])


def test_kv_store_matches_the_plain_op_and_streams():
    """Same codes as qk_norm_rope_fp8 (GPU against GPU), on a side stream too."""
    import nvfp4_quantization_place_amd as A
    inp = W.make_qk(66, "bf16", 300, 8, 2, 2, 128, scale=0.05)
    plain = A.qk_norm_rope_fp8(inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(),
                               inp.positions.cuda(), torch.from_numpy(inp.cos_sin).cuda(),
                               torch.tensor([0.05], device="cuda"), inp.eps, 8, 2, 2, 128)
    slots = np.arange(300, dtype=np.int64)[::-1].copy()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        q, kv = _run(inp, slots, 300, stream=st)
    p = _np(plain)
    np.testing.assert_array_equal(q, p[:, :8 * 128])
    np.testing.assert_array_equal(kv[slots], p[:, 8 * 128:])


def test_kv_store_empty_and_errors():
    import nvfp4_quantization_place_amd as A
    inp = W.make_qk(67, "f16", 0, 2, 1, 1, 64)
    pool = torch.zeros(4, 128, dtype=torch.uint8, device="cuda")
    q = A.qk_norm_rope_fp8_kv_store(inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(),
                                    inp.positions.cuda(), torch.from_numpy(inp.cos_sin).cuda(),
                                    torch.tensor([1.0], device="cuda"), 1e-6, 2, 1, 1, 64,
                                    torch.zeros(0, dtype=torch.int64, device="cuda"), pool)
    assert q.shape == (0, 128) and not pool.any()
    inp = W.make_qk(68, "f16", 4, 2, 1, 1, 64)
    qkv = inp.qkv.cuda()
    with pytest.raises(A.AnqError) as e:                # pool over the input
        A.qk_norm_rope_fp8_kv_store(qkv, inp.gamma_q.cuda(), inp.gamma_k.cuda(),
                                    inp.positions.cuda(), torch.from_numpy(inp.cos_sin).cuda(),
                                    torch.tensor([1.0], device="cuda"), 1e-6, 2, 1, 1, 64,
                                    torch.zeros(4, dtype=torch.int64, device="cuda"),
                                    qkv.view(torch.uint8).view(-1)[:1024].view(8, 128))
    assert e.value.code == 5

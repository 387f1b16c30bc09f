"""The prepared-call API: a call prepared once (the binding's checks run at
prepare time) and replayed gives exactly the outputs of the plain call, on
the inputs' contents at each replay, on the current stream; bad arguments
fail at prepare time."""
import numpy as np
import pytest
import torch

import workloads as W
from runners import _np

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


def _tail_pair(seed, dtype, tokens, hidden):
    inp = W.make_tail(seed, "nvfp4", dtype, tokens, hidden, norm_out=True, scale=None)
    a = [t.cuda() for t in (inp.x, inp.residual, inp.gamma)]
    b = [t.clone() for t in a]
    return a, b


@pytest.mark.parametrize("op", ["nvfp4", "fp8"])
def test_prepared_tail_equals_the_plain_call(op):
    A = _A()
    (x, r, g), (x2, r2, g2) = _tail_pair(31, "f16", 64, 8192)
    s = torch.tensor([0.02 if op == "fp8" else 400.0], device="cuda")
    fn = A.add_rmsnorm_quant_fp8 if op == "fp8" else A.add_rmsnorm_quant_nvfp4
    r0 = _np(r).copy()
    plain = fn(x, r, g, s, 1e-6, norm_out=True)
    call = A.prepare(fn, x2, r2, g2, s, 1e-6, norm_out=True)
    assert isinstance(call, A.Prepared) and call.name == fn.__name__
    torch.cuda.synchronize()
    assert np.array_equal(_np(r2), r0)                          # nothing ran at prepare time
    out = call()
    torch.cuda.synchronize()
    assert out is call.outputs
    assert np.array_equal(_np(r), _np(r2))                      # residual updated in place
    for p, q in zip(plain, out):
        assert np.array_equal(_np(p), _np(q))


def test_replays_read_the_inputs_at_call_time():
    A = _A()
    (x, r, g), (x2, r2, g2) = _tail_pair(32, "bf16", 16, 1024)
    s = torch.tensor([300.0], device="cuda")
    call = A.prepare(A.add_rmsnorm_quant_nvfp4, x2, r2, g2, s, 1e-6)
    for k in range(3):
        new = torch.randn_like(x)
        x.copy_(new)
        x2.copy_(new)
        q, sf, _ = A.add_rmsnorm_quant_nvfp4(x, r, g, s, 1e-6)
        q2, sf2, _ = call()
        torch.cuda.synchronize()
        assert np.array_equal(_np(q), _np(q2)) and np.array_equal(_np(sf), _np(sf2)), k
        assert np.array_equal(_np(r), _np(r2)), k


def test_prepared_qk_and_mixed_pool_on_another_stream():
    A = _A()
    inp = W.make_qk(33, "bf16", 37, 4, 2, 2, 128, rotary_dim=64, scale=0.05)
    args = (inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(), inp.positions.cuda(),
            torch.from_numpy(inp.cos_sin).cuda(), torch.tensor([inp.scale], device="cuda"),
            inp.eps, 4, 2, 2, 128)
    slots = torch.arange(37, dtype=torch.int64, device="cuda")
    width = A.mixed_kv_row_bytes(2, 2, 128, 64)
    p1 = torch.zeros(40, width, dtype=torch.uint8, device="cuda")
    p2 = torch.zeros_like(p1)
    q1 = A.qk_norm_rope_kv_store_mixed(*args, 64, slots, p1)
    call = A.prepare(A.qk_norm_rope_kv_store_mixed, *args, 64, slots, p2)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q2 = call()                      # enqueued on the side stream, the current one here
    side.synchronize()
    torch.cuda.synchronize()
    assert np.array_equal(_np(q1), _np(q2)) and np.array_equal(_np(p1), _np(p2))
    out = torch.empty(args[0].shape, dtype=torch.uint8, device="cuda")
    plain = A.qk_norm_rope_fp8(*args, rotary_dim=64)
    again = A.prepare(A.qk_norm_rope_fp8, *args, rotary_dim=64, out=out)
    assert again() is out
    torch.cuda.synchronize()
    assert np.array_equal(_np(plain), _np(out))


def test_bad_arguments_fail_at_prepare_time():
    A = _A()
    (x, r, g), _ = _tail_pair(34, "f16", 4, 256)
    s = torch.tensor([300.0], device="cuda")
    with pytest.raises(ValueError):
        A.prepare(A.add_rmsnorm_quant_nvfp4, x, r, g[:128], s, 1e-6)     # short gamma
    assert A._record is None
    # what only the library checks (here a negative eps) fails at the call,
    # with nothing enqueued
    call = A.prepare(A.add_rmsnorm_quant_nvfp4, x, r, g, s, -1.0)
    before = _np(r).copy()
    with pytest.raises(A.AnqError) as e:
        call()
    assert e.value.code == 8
    torch.cuda.synchronize()
    assert np.array_equal(_np(r), before)


def test_prepared_with_an_explicit_stream_keeps_it():
    A = _A()
    (x, r, g), (x2, r2, g2) = _tail_pair(35, "f16", 8, 2048)
    s = torch.tensor([300.0], device="cuda")
    side = torch.cuda.Stream()
    call = A.prepare(A.add_rmsnorm_quant_nvfp4, x2, r2, g2, s, 1e-6, stream=side)
    assert not call._current
    side.wait_stream(torch.cuda.current_stream())
    q2, sf2, _ = call()                  # on `side`, whatever the current stream is
    side.synchronize()
    q, sf, _ = A.add_rmsnorm_quant_nvfp4(x, r, g, s, 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(_np(q), _np(q2)) and np.array_equal(_np(sf), _np(sf2))
    assert np.array_equal(_np(r), _np(r2))

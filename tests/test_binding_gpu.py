"""The Python binding rejects tensors whose sizes or dtypes disagree with the
call, before anything is launched.

The C library takes device pointers and sizes and trusts the sizes, so a short
gamma or a small caller-supplied output would be read or written past its end.
Every case here builds a valid call, breaks one argument, and expects
ValueError; a final valid call checks that nothing was left half done.
"""
import numpy as np
import pytest
import torch

import workloads as W
from runners import gpu_qk, oracle_qk

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


def _tail(T=4, H=256, dt=torch.bfloat16):
    x = torch.randn(T, H, device="cuda").to(dt)
    res = torch.randn(T, H, device="cuda").to(dt)
    g = torch.ones(H, device="cuda").to(dt)
    s = torch.tensor([0.05], device="cuda")
    return x, res, g, s


def _u8(n):
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("op", ["fp8", "nvfp4", "nvfp4_swizzled", "add_rmsnorm", "gated"])
def test_gamma_must_hold_hidden(op):
    A = _A()
    x, res, g, s = _tail()
    short = g[:128].contiguous()
    call = {
        "fp8": lambda: A.add_rmsnorm_quant_fp8(x, res, short, s, 1e-6),
        "nvfp4": lambda: A.add_rmsnorm_quant_nvfp4(x, res, short, s, 1e-6),
        "nvfp4_swizzled": lambda: A.add_rmsnorm_quant_nvfp4_swizzled(x, res, short, s, 1e-6),
        "add_rmsnorm": lambda: A.add_rmsnorm(x, res, short, 1e-6),
        "gated": lambda: A.gated_rmsnorm_quant_nvfp4(x, res, short, s, 1e-6, group=128),
    }[op]
    before = res.clone()
    with pytest.raises(ValueError, match="gamma"):
        call()
    torch.cuda.synchronize()
    assert torch.equal(res, before)  # nothing ran: the residual is untouched


def test_outputs_must_have_the_call_size():
    A = _A()
    x, res, g, s = _tail()
    T, H = x.shape
    with pytest.raises(ValueError, match="q"):
        A.add_rmsnorm_quant_fp8(x, res, g, s, 1e-6, q=_u8(T * H - 16))
    with pytest.raises(ValueError, match="norm"):
        A.add_rmsnorm_quant_fp8(x, res, g, s, 1e-6, norm_out=True,
                                norm=torch.empty(T, H, dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError, match="q"):
        A.add_rmsnorm_quant_nvfp4(x, res, g, s, 1e-6, q=_u8(T * H // 2 - 1))
    with pytest.raises(ValueError, match="sf"):
        A.add_rmsnorm_quant_nvfp4(x, res, g, s, 1e-6, sf=_u8(T * H // 16 - 1))
    with pytest.raises(ValueError, match="q"):
        A.quant_fp8(x, s, q=_u8(T * H // 2))
    with pytest.raises(ValueError, match="sf"):
        A.quant_nvfp4(x, s, sf=torch.zeros(T * H // 16, dtype=torch.int8, device="cuda"))
    r, c = A.nvfp4_swizzled_sf_shape(T, H)
    with pytest.raises(ValueError, match="swizzled"):
        A.add_rmsnorm_quant_nvfp4_swizzled(x, res, g, s, 1e-6, sf=_u8(T * H // 16))
    with pytest.raises(ValueError, match="swizzled"):
        A.quant_nvfp4_swizzled(x, s, sf=_u8(r * c - 4))
    with pytest.raises(ValueError, match="q"):
        A.gated_rmsnorm_quant_nvfp4(x, res, g, s, 1e-6, group=128, q=_u8(T * H))
    with pytest.raises(ValueError, match="u"):
        A.silu_gate_f32(x, res, u=torch.empty(T * H, dtype=torch.float16, device="cuda"))


def test_inputs_must_be_contiguous():
    A = _A()
    x, res, g, s = _tail(T=8, H=256)
    with pytest.raises(ValueError, match="contiguous"):
        A.add_rmsnorm_quant_nvfp4(x.t(), res.t(), g, s, 1e-6)


def test_qk_sizes_are_checked():
    A = _A()
    inp = W.make_qk(3, "bf16", 5, 2, 1, 1, 128)
    qkv, gq, gk = inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda()
    pos, cs = inp.positions.cuda(), torch.from_numpy(inp.cos_sin).cuda()
    s = torch.tensor([0.05], device="cuda")
    args = dict(nq=2, nk=1, nv=1, head_dim=128)
    with pytest.raises(ValueError, match="gamma_q"):
        A.qk_norm_rope_fp8(qkv, gq[:64].contiguous(), gk, pos, cs, s, 1e-6, **args)
    with pytest.raises(ValueError, match="gamma_k"):
        A.qk_norm_rope_fp8(qkv, gq, gk[:64].contiguous(), pos, cs, s, 1e-6, **args)
    with pytest.raises(ValueError, match="positions"):
        A.qk_norm_rope_fp8(qkv, gq, gk, pos[:4].contiguous(), cs, s, 1e-6, **args)
    with pytest.raises(ValueError, match="cos_sin"):
        A.qk_norm_rope_fp8(qkv, gq, gk, pos, cs[:, :64].contiguous(), s, 1e-6, **args)
    with pytest.raises(ValueError, match="out"):
        A.qk_norm_rope_fp8(qkv, gq, gk, pos, cs, s, 1e-6, **args, out=_u8(qkv.numel() - 16))
    pool = _u8(9 * 2 * 128).view(9, 256)
    slots = torch.arange(5, dtype=torch.int64, device="cuda")
    with pytest.raises(ValueError, match="q_out"):
        A.qk_norm_rope_fp8_kv_store(qkv, gq, gk, pos, cs, s, 1e-6, 2, 1, 1, 128, slots, pool,
                                    q_out=_u8(5 * 128))
    # the mixed pool: rows of nk*(D+R) + nv*D bytes, a table as wide as the rotary width
    csr = torch.from_numpy(W.rope_table(5, 64, 1e6)).cuda()
    with pytest.raises(ValueError, match="whole rows"):
        A.qk_norm_rope_kv_store_mixed(qkv, gq, gk, pos, csr, s, 1e-6, 2, 1, 1, 128, 64, slots,
                                      _u8(9 * 256).view(9, 256))
    with pytest.raises(ValueError, match="cos_sin"):
        A.qk_norm_rope_kv_store_mixed(qkv, gq, gk, pos, cs, s, 1e-6, 2, 1, 1, 128, 64, slots,
                                      _u8(9 * 320).view(9, 320))
    # a layout without K heads does not look at gamma_k at all
    inp2 = W.make_qk(4, "bf16", 5, 2, 0, 1, 128)
    out = A.qk_norm_rope_fp8(inp2.qkv.cuda(), inp2.gamma_q.cuda(), None, inp2.positions.cuda(),
                             torch.from_numpy(inp2.cos_sin).cuda(), s, 1e-6, 2, 0, 1, 128)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), oracle_qk(inp2))
    # and a valid call after the rejected ones still matches the oracle
    np.testing.assert_array_equal(gpu_qk(inp), oracle_qk(inp))

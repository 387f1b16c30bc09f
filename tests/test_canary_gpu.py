"""Every entry point writes only inside its output buffers: each output is a
view at the start of a larger buffer filled with a sentinel, and after the
call every byte past the view (and the inputs) is unchanged. Shapes are small
and ragged so that stray offsets would land in the guard."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

GUARD = 4096
SENT = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _guarded(shape, dtype=torch.uint8):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((n + GUARD,), SENT, dtype=torch.uint8, device="cuda")
    return buf, buf[:n].view(dtype).view(*shape)


def _guard_intact(buf, n_bytes):
    torch.cuda.synchronize()
    tail = buf[n_bytes:].cpu().numpy()
    return bool(np.all(tail == SENT))


@pytest.mark.parametrize("tokens,hidden", [(1, 16), (5, 64), (3, 1040), (2, 7168), (40, 1024)])
def test_row_ops_write_inside_their_buffers(tokens, hidden):
    import nvfp4_quantization_place_amd as A
    inp = W.make_tail(3, "nvfp4", "bf16", tokens, hidden)
    x, g = inp.x.cuda(), inp.gamma.cuda()
    s = torch.tensor([50.0], device="cuda")
    checks = []
    bq, q = _guarded((tokens, hidden // 2))
    bs, sf = _guarded((tokens, hidden // 16))
    bn, nrm = _guarded((tokens, hidden), torch.bfloat16)
    A.add_rmsnorm_quant_nvfp4(x, inp.residual.cuda(), g, s, 1e-6, q=q, sf=sf, norm=nrm)
    checks += [(bq, q.numel()), (bs, sf.numel()), (bn, nrm.numel() * 2)]
    bq8, q8 = _guarded((tokens, hidden))
    A.add_rmsnorm_quant_fp8(x, inp.residual.cuda(), g, s, 1e-6, q=q8)
    checks.append((bq8, q8.numel()))
    r, c = A.nvfp4_swizzled_sf_shape(tokens, hidden)
    bss, ssf = _guarded((r, c))
    A.add_rmsnorm_quant_nvfp4_swizzled(x, inp.residual.cuda(), g, s, 1e-6, sf=ssf)
    checks.append((bss, ssf.numel()))
    bss2, ssf2 = _guarded((r, c))
    A.quant_nvfp4_swizzled(x, s, sf=ssf2)
    checks.append((bss2, ssf2.numel()))
    for grp in sorted({16, hidden}):
        if hidden % grp:
            continue
        bgq, gq = _guarded((tokens, hidden // 2))
        bgs, gs = _guarded((tokens, hidden // 16))
        A.gated_rmsnorm_quant_nvfp4(x, inp.residual.cuda(), g, s, 1e-6, group=grp, q=gq, sf=gs)
        checks += [(bgq, gq.numel()), (bgs, gs.numel())]
    bu, u = _guarded((tokens, hidden), torch.float32)
    A.silu_gate_f32(x, inp.residual.cuda(), u=u)
    checks.append((bu, u.numel() * 4))
    for i, (buf, n) in enumerate(checks):
        assert _guard_intact(buf, n), i


def test_qk_ops_write_inside_their_buffers():
    import nvfp4_quantization_place_amd as A
    inp = W.make_qk(4, "bf16", 7, 2, 1, 1, 64)
    args = (inp.qkv.cuda(), inp.gamma_q.cuda(), inp.gamma_k.cuda(), inp.positions.cuda(),
            torch.from_numpy(inp.cos_sin).cuda(), torch.tensor([0.05], device="cuda"), 1e-6, 2, 1, 1,
            64)
    bo, out = _guarded((7, 4 * 64))
    A.qk_norm_rope_fp8(*args, out=out)
    bq, q = _guarded((7, 2 * 64))
    bkv, kv = _guarded((5, 2 * 64))
    slots = torch.tensor([4, -1, 0, 9, 2, 3, 1], dtype=torch.int64, device="cuda")
    A.qk_norm_rope_fp8_kv_store(*args, slot_mapping=slots, kv_cache=kv, q_out=q)
    checks = [(bo, out.numel()), (bq, q.numel()), (bkv, kv.numel())]
    for R in (16, 32):       # partial rotation, and the mixed pool (rows of nk*(D+R) + nv*D)
        p = W.make_qk(4, "bf16", 7, 2, 1, 1, 64, rotary_dim=R)
        pargs = (p.qkv.cuda(), p.gamma_q.cuda(), p.gamma_k.cuda(), p.positions.cuda(),
                 torch.from_numpy(p.cos_sin).cuda(), torch.tensor([0.05], device="cuda"), 1e-6, 2,
                 1, 1, 64)
        bo2, out2 = _guarded((7, 4 * 64))
        A.qk_norm_rope_fp8(*pargs, rotary_dim=R, out=out2)
        bqm, qm = _guarded((7, 2 * 64))
        bkm, km = _guarded((5, A.mixed_kv_row_bytes(1, 1, 64, R)))
        A.qk_norm_rope_kv_store_mixed(*pargs, R, slot_mapping=slots, kv_cache=km, q_out=qm)
        checks += [(bo2, out2.numel()), (bqm, qm.numel()), (bkm, km.numel())]
    for i, (buf, n) in enumerate(checks):
        assert _guard_intact(buf, n), i

"""The entry points captured in a HIP graph (how the benchmark times them)
give, replay after replay, exactly what eager calls give. The residual is
updated in place, so the static input buffers are refilled before each
replay; eager work and synchronisation run between the replays."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


def _calls(A, b):
    """Every op once, on the static buffers in b; returns the output tensors."""
    A.add_rmsnorm_quant_nvfp4(b["x"], b["res"], b["g"], b["G"], 1e-5, q=b["q4"], sf=b["sf4"],
                              norm=b["n4"])
    A.add_rmsnorm_quant_fp8(b["x"], b["res2"], b["g"], b["s"], 1e-6, q=b["q8"], norm=b["n8"])
    A.add_rmsnorm_quant_nvfp4_swizzled(b["x"], b["res3"], b["g"], b["G"], 1e-5, q=b["qs"],
                                       sf=b["sfs"])
    A.gated_rmsnorm_quant_nvfp4(b["x"], b["z"], b["g"], b["G"], 1e-5, group=256, q=b["qg"],
                                sf=b["sfg"])
    # groups of 64: 4800 group-rows, the gate-table tiling with interleaved rows
    A.gated_rmsnorm_quant_nvfp4(b["x"], b["z"], b["g"], b["G"], 1e-5, group=64, q=b["qg2"],
                                sf=b["sfg2"])
    A.qk_norm_rope_fp8(b["qkv"], b["gq"], b["gk"], b["pos"], b["cs"], b["s"], 1e-6, 4, 2, 2, 128,
                       out=b["qko"])
    A.qk_norm_rope_fp8_kv_store(b["qkv"], b["gq"], b["gk"], b["pos"], b["cs"], b["s"], 1e-6, 4, 2,
                                2, 128, slot_mapping=b["slots"], kv_cache=b["kv"], q_out=b["qq"])
    A.quant_nvfp4(b["n4"], b["G"], q=b["qq4"], sf=b["qsf4"])
    A.qk_norm_rope_kv_store_mixed(b["qkv"], b["gq"], b["gk"], b["pos"], b["cs64"], b["s"], 1e-6,
                                  4, 2, 2, 128, 64, slot_mapping=b["slots"], kv_cache=b["kvm"],
                                  q_out=b["qqm"])
    return [b[k] for k in ("res", "q4", "sf4", "n4", "res2", "q8", "n8", "res3", "qs", "sfs", "qg",
                           "sfg", "qg2", "sfg2", "qko", "qq", "kv", "qq4", "qsf4", "qqm", "kvm")]


def test_graph_replays_match_eager():
    import nvfp4_quantization_place_amd as A
    M, H = 300, 1024
    inp = W.make_tail(31, "nvfp4", "bf16", M, H)
    qk = W.make_qk(32, "bf16", 77, 4, 2, 2, 128)
    dev = "cuda"
    b = dict(x=inp.x.to(dev), res=torch.empty_like(inp.residual, device=dev),
             res2=torch.empty_like(inp.residual, device=dev),
             res3=torch.empty_like(inp.residual, device=dev),
             z=inp.residual.to(dev), g=inp.gamma.to(dev),
             G=torch.tensor([60.0], device=dev), s=torch.tensor([0.05], device=dev),
             q4=torch.empty(M, H // 2, dtype=torch.uint8, device=dev),
             sf4=torch.empty(M, H // 16, dtype=torch.uint8, device=dev),
             n4=torch.empty(M, H, dtype=torch.bfloat16, device=dev),
             q8=torch.empty(M, H, dtype=torch.uint8, device=dev),
             n8=torch.empty(M, H, dtype=torch.bfloat16, device=dev),
             qs=torch.empty(M, H // 2, dtype=torch.uint8, device=dev),
             sfs=torch.empty(*A.nvfp4_swizzled_sf_shape(M, H), dtype=torch.uint8, device=dev),
             qg=torch.empty(M, H // 2, dtype=torch.uint8, device=dev),
             sfg=torch.empty(M, H // 16, dtype=torch.uint8, device=dev),
             qg2=torch.empty(M, H // 2, dtype=torch.uint8, device=dev),
             sfg2=torch.empty(M, H // 16, dtype=torch.uint8, device=dev),
             qkv=qk.qkv.to(dev), gq=qk.gamma_q.to(dev), gk=qk.gamma_k.to(dev),
             pos=qk.positions.to(dev), cs=torch.from_numpy(qk.cos_sin).to(dev),
             qko=torch.empty(77, 8 * 128, dtype=torch.uint8, device=dev),
             qq=torch.empty(77, 4 * 128, dtype=torch.uint8, device=dev),
             kv=torch.zeros(100, 4 * 128, dtype=torch.uint8, device=dev),
             slots=torch.from_numpy(np.random.default_rng(3).permutation(100)[:77].astype(np.int64)).to(dev),
             qq4=torch.empty(M, H // 2, dtype=torch.uint8, device=dev),
             qsf4=torch.empty(M, H // 16, dtype=torch.uint8, device=dev),
             cs64=torch.from_numpy(W.rope_table(77, 64, 1e6)).to(dev),
             qqm=torch.empty(77, 4 * 128, dtype=torch.uint8, device=dev),
             kvm=torch.zeros(100, A.mixed_kv_row_bytes(2, 2, 128, 64), dtype=torch.uint8, device=dev))
    res0 = inp.residual.to(dev)

    def refill():
        for k in ("res", "res2", "res3"):
            b[k].copy_(res0)
        b["kv"].zero_()
        b["kvm"].zero_()

    refill()
    eager = [t.clone() for t in _calls(A, b)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        refill()
        _calls(A, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _calls(A, b)
    for rep in range(4):
        refill()
        for t in outs:                              # stale results would show
            if any(t is b[k] for k in ("kv", "kvm", "res", "res2", "res3")):
                continue
            t.fill_(0xEE if t.dtype == torch.uint8 else float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        junk = torch.randn(1 << 20, device=dev).sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for i, (got, want) in enumerate(zip(outs, eager)):
            assert torch.equal(got, want), (rep, i)

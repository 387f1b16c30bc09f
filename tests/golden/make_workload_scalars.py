"""Write tests/golden/workload_scalars.json: for each workload the checksums
of its seeded inputs, and for the NVFP4 workloads (gated included) the global scale
G = fl32(448 * 6 / amax|n|) over the oracle's binary32 normed tensor (the
reading of "global fp32 scale = 448*6/amax(normed)"). Calls only the oracle
and the input generator.

    python tests/golden/make_workload_scalars.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_scalars.json")


def main():
    res = {"_about": "Written by make_workload_scalars.py from the oracle; do not edit by hand."}
    for k in sorted(W.CONFIGS):
        inp = W.make_config(k)
        e = {"name": inp.name}
        if isinstance(inp, W.QKInputs):
            e["checksums"] = {"qkv": W.checksum(inp.qkv), "gamma_q": W.checksum(inp.gamma_q),
                              "gamma_k": W.checksum(inp.gamma_k), "cos_sin": W.checksum(inp.cos_sin)}
        else:
            e["checksums"] = {"x": W.checksum(inp.x), "residual": W.checksum(inp.residual),
                              "gamma": W.checksum(inp.gamma)}
            if inp.op in ("nvfp4", "gated"):
                if inp.op == "gated":
                    n = O.gated_rmsnorm_quant_nvfp4(W.bits(inp.x), W.bits(inp.residual),
                                                    W.bits(inp.gamma), inp.dtype,
                                                    inp.meta["group"], 1.0, inp.eps)["n"]
                else:
                    n = O.rmsnorm_f32(W.bits(inp.x), W.bits(inp.residual), W.bits(inp.gamma),
                                      inp.dtype, inp.eps)
                G = O.nvfp4_global_scale(n)
                e["global_scale"] = float(G)
                e["global_scale_bits"] = "0x%08X" % int(G.view("uint32"))
        res[str(k)] = e
        print(k, e, flush=True)
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=1)


if __name__ == "__main__":
    main()

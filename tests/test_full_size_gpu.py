"""Every output byte of every full-size workload against the oracle.

The full outputs are hundreds of MB, so the oracle's are stored as SHA-256
digests, whole and per run of rows (tests/golden/workload_digests.json,
written by tests/golden/make_workload_digests.py, which calls only the oracle
and the input generator). Each test launches one workload at its full size on
fresh inputs, in the launch configuration the benchmark times, and digests
every output the same way. A mismatching chunk is recomputed by the oracle
and its first differing elements are reported.

Covered: the six workloads (residual, codes, block scales and norm output of
the fused tail ops; the Q/K op's codes; the gated op's codes and scales), the
separated two-kernel tail on workloads 2-4, the swizzled block scales on
workloads 2 and 4, and the KV-cache store on the Q/K workload.
"""
import importlib.util
import json
import os

import numpy as np
import pytest
import torch

import workloads as W
from runners import gpu_full_workload

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DIGESTS = os.path.join(HERE, "golden", "workload_digests.json")

CASES = [(1, "fused"), (2, "fused"), (3, "fused"), (4, "fused"), (5, "fused"), (6, "fused"),
         (2, "separated"), (3, "separated"), (4, "separated"),
         (2, "swizzled"), (4, "swizzled"), (5, "kv_store"), (7, "fused"), (7, "kv_mixed")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_quantization_place_amd as A
    A.lib()


@pytest.fixture(scope="module")
def digests():
    with open(DIGESTS) as fh:
        return json.load(fh)


def _oracle_rows(k, r0, r1):
    spec = importlib.util.spec_from_file_location(
        "make_workload_digests", os.path.join(HERE, "golden", "make_workload_digests.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    m._init(k)
    return m._rows(r0, r1)


def _explain(k, name, got, want, bad_chunks):
    """Oracle values of the first mismatching chunk (plain row outputs only)."""
    cr = want["chunk_rows"]
    c = bad_chunks[0]
    msg = f"workload {k} {name}: {len(bad_chunks)} of {len(want['chunks'])} chunks differ " \
          f"(first rows {c * cr}..{(c + 1) * cr - 1})"
    if name in ("kv_store_pool", "sf_swizzled", "kv_store_q", "kv_mixed_pool", "kv_mixed_q"):
        return msg
    ref = _oracle_rows(k, c * cr, min((c + 1) * cr, got.shape[0]))
    if name not in ref:
        return msg
    g = got[c * cr:(c + 1) * cr]
    r = ref[name]
    diff = np.argwhere(g != r)
    msg += f"; {len(diff)} elements differ in that chunk, first at (row, col) " \
           f"{[(int(i) + c * cr, int(j)) for i, j in diff[:5]]}: gpu " \
           f"{[int(g[i, j]) for i, j in diff[:5]]} oracle {[int(r[i, j]) for i, j in diff[:5]]}"
    return msg


@pytest.mark.parametrize("k,variant", CASES)
def test_full_size_every_output_byte(k, variant, digests):
    entry = digests[str(k)]
    print(f"workload {k} {entry['name']} ({variant}): {entry['rows']} rows, full size",
          flush=True)
    got = gpu_full_workload(k, variant)
    assert got, "no outputs"
    for name, a in got.items():
        want = entry["outputs"][name]
        d = W.row_chunk_digests(a, want["chunk_rows"])
        if d["sha256"] != want["sha256"]:
            bad = [i for i, (x, y) in enumerate(zip(d["chunks"], want["chunks"])) if x != y]
            if len(d["chunks"]) != len(want["chunks"]):
                bad = bad or [0]
            pytest.fail(_explain(k, name, a, want, bad))

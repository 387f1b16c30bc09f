"""The stored full-size digests (tests/golden/workload_digests.json) are the
oracle's: recomputed here for the two small workloads, in one process (the
stored file was written with worker processes; rows are independent, so the
digests cannot depend on how rows were split). The large workloads take
minutes of oracle time and are recomputed by running the script itself."""
import json
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_workload_digests as MWD  # noqa: E402


@pytest.fixture(scope="module")
def stored():
    with open(MWD.OUT) as fh:
        return json.load(fh)


@pytest.mark.parametrize("k", [1, 2])
def test_small_workload_digests_are_the_oracles(k, stored):
    assert MWD.workload(k, procs=1) == stored[str(k)]


def test_every_workload_and_variant_is_digested(stored):
    import workloads as W
    for k in W.CONFIGS:
        e = stored[str(k)]
        assert e["name"] == W.CONFIGS[k]["name"]
        for name, d in e["outputs"].items():
            assert len(d["sha256"]) == 64 and all(len(c) == 16 for c in d["chunks"]), (k, name)
            assert len(d["chunks"]) * d["chunk_rows"] >= e["rows"] or name.endswith("swizzled") \
                or name == "kv_store_pool"
    assert {"q_separated", "sf_separated", "sf_swizzled"} <= set(stored["4"]["outputs"])
    assert {"kv_store_q", "kv_store_pool"} <= set(stored["5"]["outputs"])

"""Fixed-token regression pins: the oracle's routing and sort digests for every
seeded workload equal the recorded ones (tests/golden/routing_hashes.json,
written by tests/golden/make_golden.py from the oracle)."""
import json
import os

import pytest

from fp4_routed_mixture_amd import synth as S

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "routing_hashes.json")))


@pytest.mark.parametrize("name", sorted(S.WORKLOADS))
def test_routing_hashes_reproduce(oracle, name):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "make_golden", os.path.join(os.path.dirname(__file__), "golden", "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    assert mg.routing_record(S.WORKLOADS[name]) == GOLD[name]

"""The seeded inputs of the measured workloads, and the oracle's result on the tiny one, are the
bytes recorded in tests/golden/manifest.json (written by tests/golden/make_golden.py): the GPU
runs, the oracle and the benchmark all consume these exact buffers."""
import json
import os

import pytest

from golden import make_golden as mg

MANIFEST = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "manifest.json")))


@pytest.mark.parametrize("name", sorted(MANIFEST["inputs"]))
def test_workload_inputs_match_manifest(name):
    inp = mg.workloads()[name]()
    assert mg.input_hashes(inp) == MANIFEST["inputs"][name]


def test_oracle_tiny_matches_manifest(oracle_lib):
    inp = mg.workloads()["tiny"]()
    assert mg.oracle_hash(inp) == MANIFEST["oracle"]["tiny"]

"""Stored oracle outputs for the tiny workload still reproduce (to 1e-13)."""

import json
import os

import numpy as np

import oracle
from workloads import make_config_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_gqa8_oracle.json")


def _unhex(xs):
    return np.array([float.fromhex(x) for x in xs])


def test_tiny_workload_oracle_matches_stored_values():
    with open(GOLDEN) as f:
        g = json.load(f)
    case = make_config_case("tiny_gqa8")
    assert case.context_lens.tolist() == g["context_lens"]
    assert case.block_table.tolist() == g["block_table"]
    assert float(case.q.double().sum()).hex() == g["q_sum"]
    O, L = oracle.run_case(case)
    _, Lp = oracle.run_case(case, num_splits=3)
    # BLAS may round differently on another host CPU: allow 1e-13.
    assert np.abs(O.ravel() - _unhex(g["out"])).max() <= 1e-13
    assert np.abs(L.ravel() - _unhex(g["lse"])).max() <= 1e-13
    assert np.abs(Lp.ravel() - _unhex(g["lse_split3"])).max() <= 1e-13

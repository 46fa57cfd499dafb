"""Write the stored oracle outputs under tests/golden/ (run from the repo root).

The values come from the CPU oracle only (``oracle.run_case``) on the seeded
tiny workload (batch 2, 8 q heads / 1 kv head, D128, bs16, context {37, 100},
16-page pool, scale 1/sqrt(128)). They guard the oracle and the input
generator against silent drift: the golden test regenerates them and demands
agreement to 1e-13 (BLAS rounding may differ between host CPUs). Floats are stored with ``float.hex`` so they round-trip
exactly.

    python tests/golden/make_golden.py
"""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import make_config_case  # noqa: E402


def build():
    case = make_config_case("tiny_gqa8")
    O, L = oracle.run_case(case)
    Op, Lp = oracle.run_case(case, num_splits=3)
    return {
        "workload": "tiny_gqa8 (batch 2, Hq 8, Hkv 1, D 128, bs 16, ctx 37/100, seed 101)",
        "source": "oracle.run_case on workloads.make_config_case('tiny_gqa8')",
        "context_lens": case.context_lens.tolist(),
        "block_table": case.block_table.tolist(),
        "q_sum": float(case.q.double().sum()).hex(),
        "out": [float(x).hex() for x in O.ravel()],
        "lse": [float(x).hex() for x in L.ravel()],
        "lse_split3": [float(x).hex() for x in Lp.ravel()],
    }


if __name__ == "__main__":
    path = os.path.join(HERE, "tiny_gqa8_oracle.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=0)
    print("wrote", path)

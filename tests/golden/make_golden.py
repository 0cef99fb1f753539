"""Write tests/golden/oracle_regression.json from the CPU oracle alone.

This is a regression fixture, not a pin: it freezes what the (separately pinned)
oracle returns on small seeded inputs so that an unintended change to the
oracle's arithmetic shows up as a diff. Run from the repository root:
    python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import workloads  # noqa: E402

CASES = [
    ("cfg1", lambda: workloads.config1(), 15),
    ("cfg2_small", lambda: workloads.config2(96, 160), 6),
    ("cfg3_small", lambda: workloads.config3("up", 80, 192), 6),
    ("cfg4_small", lambda: workloads.config4(64, 96), 6),
    ("cfg5_small", lambda: workloads.config5_layer(0, scale_down=32)[6], 6),
]


def digest(arr) -> str:
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()


def run_case(make, T):
    w = make()
    out = oracle.solve(w.W, w.dtype, w.fmt, w.group, T)
    return {
        "workload": w.name, "input_sha256": w.sha256(), "fmt": w.fmt, "group": w.group, "T": T,
        "codes_sha256": digest(out["codes"]), "scales_sha256": digest(out["scales"]),
        "a_sha256": digest(out["a"]), "b_sha256": digest(out["b"]),
        "g": out["g"], "mse": [float(v).hex() for v in out["mse"]],
    }


def main():
    oracle.set_threads(1)
    res = {name: run_case(make, T) for name, make, T in CASES}
    with open(os.path.join(HERE, "oracle_regression.json"), "w") as f:
        json.dump(res, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()

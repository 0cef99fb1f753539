"""Golden fixtures: format facts the pages state, and the oracle regression file.

format_facts.json holds what the DualQuant pages fix about the formats (each entry
cites its page and section); the oracle must honour each. oracle_regression.json
is written by tests/golden/make_golden.py, which calls only the oracle, and freezes
its outputs on small seeded inputs.
"""
import json
import os
import sys

import numpy as np

import fmt_brute as fb

HERE = os.path.dirname(os.path.abspath(__file__))
GOLD = os.path.join(HERE, "golden")


def test_format_facts_hold_in_the_oracle(oracle_lib):
    facts = json.load(open(os.path.join(GOLD, "format_facts.json")))
    lo, hi = facts["e8m0_exponent_range"]["min"], facts["e8m0_exponent_range"]["max"]
    assert oracle_lib.project("mxint4", 1e-300) == 2.0 ** lo
    assert oracle_lib.project("mxint4", 1e300) == 2.0 ** hi
    # INT4 codes stay inside [-8, 7] for any input (here: extreme columns)
    rng = np.random.default_rng(0)
    W = (rng.normal(0, 1, (8, 64)) * np.exp(rng.normal(0, 3, 64))).astype(np.float32)
    out = oracle_lib.quantize(W, "f32", "int4_bf16", 32)
    q = fb.unpack_codes(out["codes"], "int4_bf16")
    assert q.min() >= facts["int4_codebook"]["min"] and q.max() <= facts["int4_codebook"]["max"]
    # block sizes of the MX / NV formats are accepted as group sizes
    for fmt, key in (("mxfp4", "mxfp4_block"), ("nvfp4", "nvfp4_block")):
        G = facts[key]["elements"]
        out = oracle_lib.quantize(W, "f32", fmt, G)
        assert out["scales"].shape == (8, 64 // G)


def test_oracle_regression_fixture(oracle_lib):
    sys.path.insert(0, GOLD)
    import make_golden

    want = json.load(open(os.path.join(GOLD, "oracle_regression.json")))
    for name, make, T in make_golden.CASES:
        got = make_golden.run_case(make, T)
        assert got == want[name], name

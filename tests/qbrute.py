"""Brute-force check of one Q pass: given the scaled values X the pass quantized, the scale
rule of every group and the code of sampled elements are recomputed by enumeration (exact
rational distances to every codebook value) and compared with the output."""
from fractions import Fraction

import numpy as np

import fmt_brute as fb


def check_q_output(out, X, fmt, group, g_in, samples=3000, seed=0):
    """out: a Q pass's codes, scales and g; X: the fp32 values it quantized (rows x cols)."""
    rows, cols = X.shape
    ng = cols // group
    m = np.abs(X).reshape(rows, ng, group).max(-1)
    g = out["g"]
    if fmt == "nvfp4" and g_in <= 0:
        amax = np.float32(np.abs(X).max())
        want_g = np.float32(1.0) if amax == 0 else max(np.float32(amax / np.float32(2688.0)),
                                                       np.float32(2.0 ** -126))
        assert np.float32(g) == want_g
    s_got = fb.decode_scales(out["scales"], fmt)
    # scale rule per group
    for i in range(rows):
        for k in range(ng):
            mm = m[i, k]
            if mm == 0:
                assert s_got[i, k] == 1.0
                continue
            if fmt == "int4_bf16":
                s = fb.torch_bf16(np.array([np.float32(mm) / np.float32(7.0)], np.float32))[0]
                assert s_got[i, k] == max(s, 2.0 ** -133)
            elif fmt in ("mxint4", "mxfp4"):
                d = s_got[i, k]
                clamped = d in (2.0 ** -126, 2.0 ** 126)
                assert clamped or 4.0 <= mm / d < 8.0
                if d == 2.0 ** -126:
                    assert mm < 2.0 ** -123
            else:
                u = np.float32(mm) / (np.float32(6.0) * np.float32(g))
                s = max(fb.e4m3_nearest_sat(float(u)), 2.0 ** -9)
                assert s_got[i, k] == s
    # codes: nearest codebook value to the exact quotient x/d (ties to even)
    q = fb.unpack_codes(out["codes"], fmt)
    d = np.repeat(fb.divisors(out["scales"], fmt, g), group, axis=1)
    rng = np.random.default_rng(seed)
    idx = rng.choice(rows * cols, size=min(samples, rows * cols), replace=False)
    # also every element of the first group of each row (where the ties were planted)
    extra = [i * cols + j for i in range(rows) for j in range(group)]
    for flat in np.unique(np.concatenate([idx, extra])):
        i, j = divmod(int(flat), cols)
        x, dd = Fraction(float(X[i, j])), Fraction(float(d[i, j]))
        if fmt in ("int4_bf16", "mxint4"):
            lo = -8 if fmt == "int4_bf16" else -7
            cands = [(abs(x - k * dd), k % 2, k) for k in range(lo, 8)]
        else:
            cands = [(abs(x - Fraction(float(v)) * dd), c & 1, float(v))
                     for c, v in enumerate(fb.E2M1_TABLE) if c != 8]
        want = min(cands)[2]
        assert q[i, j] == want, (fmt, i, j, float(X[i, j]), float(d[i, j]), q[i, j], want)

"""Seeded small test matrices shared by the oracle pins and the GPU parity tests:
random weights with outlier columns, and adversarial rows whose scaled values sit exactly
on rounding ties, plus zero groups, subnormals and outliers."""
import numpy as np


def rand_w(rows, cols, seed, dtype="f32", outliers=3):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, (rows, cols))
    cols_o = rng.choice(cols, size=outliers, replace=False)
    W[:, cols_o] *= rng.uniform(5, 30, size=outliers)
    W32 = W.astype(np.float32)
    if dtype == "bf16":
        h = (W32.view(np.uint32) + 0x7FFF + ((W32.view(np.uint32) >> 16) & 1)) >> 16
        return h.astype(np.uint16)
    return W32


def adversarial_w(fmt, group, rows, seed):
    """Rows whose scaled values sit exactly on rounding ties, plus zero groups,
    subnormals and outliers (a = b = 1)."""
    rng = np.random.default_rng(seed)
    cols = 4 * group
    W = rng.normal(0, 0.05, (rows, cols)).astype(np.float32)
    for i in range(rows):
        kind = i % 5
        if kind == 0:  # exact ties against a known scale
            d = np.float32(2.0 ** rng.integers(-8, 2))
            if fmt == "int4_bf16":
                ks = rng.integers(-7, 7, group) + 0.5
                ks[0] = 7.0  # makes bf16(m/7) = d exactly
                W[i, :group] = (ks * d).astype(np.float32)
            elif fmt == "mxint4":
                ks = rng.integers(-6, 6, group) + 0.5
                ks[0] = 4.0  # m/d in [4, 8) -> scale d
                W[i, :group] = (ks * d).astype(np.float32)
            else:
                mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
                ks = rng.choice(mids, group) * rng.choice([-1, 1], group)
                ks[0] = 6.0 if fmt == "mxfp4" else 6.0
                W[i, :group] = (ks * d).astype(np.float32)
        elif kind == 1:
            W[i, group:2 * group] = 0.0  # zero group
        elif kind == 2:
            W[i, :group] = (rng.normal(0, 1, group) * 1e-39).astype(np.float32)  # subnormals
        elif kind == 3:
            W[i, 3] = 40.0  # outlier
    return W

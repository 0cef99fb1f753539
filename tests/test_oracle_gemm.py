"""Pins of the oracle's W4A4 product (dq_ref_gemm_mx): Y[t][i] = a_i * sum_k x^[t][k] Qhat[i][k]
with MXFP4 codes and E8M0 block scales on both sides (daiwk notes, "核心公式" eq. 1: the
factorized product X W^T ~= (X D_b) Qhat^T D_a; the flowchart ends in the matmul of the
quantized activations with the weight codes and the row output scale).

Against independent computation: on-grid operands are decoded here (fmt_brute's E2M1 and
E8M0 tables) and multiplied with numpy's float64 matmul; the exponent range is kept small
enough that every partial sum is exact in double, so the comparison is exact whatever the
summation order. A pure-Python loop checks a tiny case; invariants (operand swap transposes,
power-of-two scale shifts, zero codes, a = None) and the composition with both quantizers
(the product approximates X W^T) catch transposed or misapplied scales."""
import numpy as np
import pytest

import fmt_brute as fb
import workloads
from cases import rand_w


def _operands(rows, K, seed, lo=120, hi=135):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales


def _dequant(codes, scales):
    return fb.dequant(codes, scales, "mxfp4", 32, 0.0)


@pytest.mark.parametrize("tokens,out,K", [(7, 5, 96), (33, 40, 256), (3, 70, 32)])
def test_on_grid_product_is_exact(oracle_lib, tokens, out, K):
    xc, xs = _operands(tokens, K, seed=tokens)
    wc, ws = _operands(out, K, seed=out + 1000)
    a = np.random.default_rng(K).uniform(0.01, 3.0, out).astype(np.float32)
    Y = oracle_lib.gemm_mx(xc, xs, wc, ws, a)
    # products are multiples of 2^-2 * 2^(ex + ew - 254) with |ex + ew - 254| <= 28, and K
    # of them sum below 2^(6 + 28 + 9): every partial sum is exact in float64
    want = (_dequant(xc, xs) @ _dequant(wc, ws).T) * a.astype(np.float64)[None, :]
    assert Y.shape == (tokens, out)
    assert np.array_equal(Y, want)


def test_pure_python_brute_force(oracle_lib):
    xc, xs = _operands(3, 64, seed=5, lo=100, hi=160)
    wc, ws = _operands(2, 64, seed=6, lo=100, hi=160)
    a = np.array([0.75, 1.5], np.float32)
    Y = oracle_lib.gemm_mx(xc, xs, wc, ws, a)

    def val(codes, scales, r, k):
        byte = int(codes[r, k // 2])
        nib = byte >> 4 if k % 2 else byte & 0xF
        return fb.e2m1_decode(nib) * 2.0 ** (int(scales[r, k // 32]) - 127)

    for t in range(3):
        for i in range(2):
            acc = 0.0
            for k in range(64):
                acc += val(xc, xs, t, k) * val(wc, ws, i, k)
            assert Y[t, i] == acc * float(a[i]), (t, i)


def test_operand_swap_transposes_and_a_scales_columns(oracle_lib):
    xc, xs = _operands(9, 128, seed=11)
    wc, ws = _operands(6, 128, seed=12)
    Y = oracle_lib.gemm_mx(xc, xs, wc, ws)
    assert np.array_equal(oracle_lib.gemm_mx(wc, ws, xc, xs), Y.T)
    assert np.array_equal(oracle_lib.gemm_mx(xc, xs, wc, ws, np.ones(6, np.float32)), Y)
    a = np.array([2.0, 0.5, 1.0, 4.0, 0.25, 8.0], np.float32)  # powers of two: exact
    assert np.array_equal(oracle_lib.gemm_mx(xc, xs, wc, ws, a), Y * a[None, :])


def test_power_of_two_scale_shifts(oracle_lib):
    xc, xs = _operands(8, 192, seed=21)
    wc, ws = _operands(10, 192, seed=22)
    Y = oracle_lib.gemm_mx(xc, xs, wc, ws)
    assert np.array_equal(oracle_lib.gemm_mx(xc, xs + 3, wc, ws), Y * 8.0)
    assert np.array_equal(oracle_lib.gemm_mx(xc, xs, wc, ws - 2), Y / 4.0)
    # shifting one k block of one token scales only that block's contribution
    xs2 = xs.copy()
    xs2[2, 1] += 1
    Y2 = oracle_lib.gemm_mx(xc, xs2, wc, ws)
    blk = _dequant(xc[2:3, 16:32], xs[2:3, 1:2]) @ _dequant(wc[:, 16:32], ws[:, 1:2]).T
    assert np.array_equal(np.delete(Y2, 2, 0), np.delete(Y, 2, 0))
    assert np.allclose(Y2[2], Y[2] + blk[0], rtol=1e-15, atol=0)


def test_zero_codes_and_nan_scales(oracle_lib):
    xc, xs = _operands(5, 64, seed=31)
    wc, ws = _operands(4, 64, seed=32)
    zero = np.zeros_like(xc)
    assert np.all(oracle_lib.gemm_mx(zero, xs, wc, ws) == 0.0)
    neg0 = np.full_like(xc, 0x88)  # -0 codes
    assert np.all(oracle_lib.gemm_mx(neg0, xs, wc, ws) == 0.0)
    xs2 = xs.copy()
    xs2[1, 0] = 0xFF  # the E8M0 NaN
    Y = oracle_lib.gemm_mx(xc, xs2, wc, ws)
    assert np.all(np.isnan(Y[1])) and not np.any(np.isnan(np.delete(Y, 1, 0)))


def test_quantized_product_approximates_the_float_product(oracle_lib):
    # the solver's (codes, scales, a, b) with the activation quantizer's x^ = Q(X b) give
    # Y ~= X W^T: the product's error is the weight-side and the activation-side errors
    # combined (independent, so about in quadrature); a transposed operand, a or b applied on
    # the wrong side, or a scale misread by one block would break this by far more
    K, out, tokens = 256, 48, 40
    W = rand_w(out, K, seed=51, outliers=2)
    X = workloads.activations(tokens, K, seed=52, dtype="f32")
    sol = oracle_lib.solve(W, "f32", "mxfp4", 32, 6)
    act = oracle_lib.quantize_act(X, "f32", "mxfp4", 32, sol["b"])
    Y = oracle_lib.gemm_mx(act["codes"], act["scales"], sol["codes"], sol["scales"], sol["a"])
    X64, W64 = X.astype(np.float64), W.astype(np.float64)
    ref = X64 @ W64.T
    Xq = _dequant(act["codes"], act["scales"])  # Q(X b)
    Wq = _dequant(sol["codes"], sol["scales"])  # Qhat
    # exact composition: x^ and Qhat decoded here, the sum exact in double up to rounding
    want = (Xq @ Wq.T) * sol["a"].astype(np.float64)[None, :]
    assert np.allclose(Y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())

    def rel(A):
        return np.linalg.norm(A - ref) / np.linalg.norm(ref)

    What = sol["a"][:, None] * Wq * sol["b"][None, :]  # D_a Qhat D_b
    Xhat = Xq / sol["b"][None, :]  # Q(X D_b) D_b^-1
    e_w, e_x = rel(X64 @ What.T), rel(Xhat @ W64.T)
    assert max(e_w, e_x) < rel(Y) < 1.25 * np.hypot(e_w, e_x), (rel(Y), e_w, e_x)
    assert rel(Y) < 0.6


def test_status_codes(oracle_lib):
    xc, xs = _operands(4, 64, seed=41)
    wc, ws = _operands(4, 64, seed=42)
    with pytest.raises(oracle_lib.OracleError) as e:  # K = 48 is not a whole number of blocks
        oracle_lib.gemm_mx(xc[:, :24], xs, wc[:, :24], ws)
    assert e.value.status == 1
    with pytest.raises(oracle_lib.OracleError) as e:
        oracle_lib.gemm_mx(xc, xs, wc, ws, np.array([1, 0, 1, 1], np.float32))
    assert e.value.status == 1

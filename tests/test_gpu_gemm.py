"""GPU parity of the W4A4 product (dq_gemm_mx) against the oracle (dq_ref_gemm_mx, float64).

Tolerance, from the arithmetic: every product x^ * Qhat is exact (E2M1 times E2M1 times two
powers of two); the matrix cores add them into fp32 accumulators, one 64-k step per
instruction, so the accumulated sum is within (K / 64 + 1) * 2 * 2^-24 * S of the exact one,
S = sum_k |x^_tk Qhat_ik| (computed by the oracle on sign-cleared codes); the a_i product adds
one fp32 rounding, and a bf16 output at most 2^-8 relative more. Where every partial sum fits
fp32's 24 bits the product is exact, whatever the order, and the test asks for bit equality.

Cases: ragged token / channel counts and K not a multiple of the 256-k stage (the slow
path), the fast path at tile multiples, both output types, a = None, the exact case, NaN
block scales, the quantizers' own outputs, the Llama-3.1-8B MLP shapes at full size on
sampled outputs, and a K large enough that a call is split into several launches; the same
for the product with packed weights, whose packing is checked byte for byte against the
documented layout restated here with numpy."""
import numpy as np
import pytest

import workloads
from parity import host, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dq():
    import torch

    assert torch.cuda.is_available()
    import dual_scale_w4a4_amd

    dual_scale_w4a4_amd.lib()
    return dual_scale_w4a4_amd


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bound(oracle, xc, xs, wc, ws, a, K):
    S = np.abs(oracle.gemm_mx(xc & 0x77, xs, wc & 0x77, ws, a))
    return (K / 64 + 2) * 2.0 * 2.0 ** -24 * S


def _gemm(dq, xc, xs, wc, ws, a, out_dtype, packed):
    ad = None if a is None else _dev(a)
    if packed:
        pk = dq.gemm_pack_weights(_dev(wc), _dev(ws))
        return dq.gemm_mx_packed(_dev(xc), _dev(xs), pk, ad, out_dtype=out_dtype)
    return dq.gemm_mx(_dev(xc), _dev(xs), _dev(wc), _dev(ws), ad, out_dtype=out_dtype)


def _check(dq, oracle, xc, xs, wc, ws, a, out_dtype, name="", packed=False):
    K = xc.shape[1] * 2
    print(f"[gemm] {name} tokens={xc.shape[0]} out={wc.shape[0]} K={K} {out_dtype} "
          f"a={'yes' if a is not None else 'no'} packed={packed}", flush=True)
    y = _gemm(dq, xc, xs, wc, ws, a, out_dtype, packed)
    got = host(y).astype(np.float64) if out_dtype == "f32" else _bf16_host(y)
    ref = oracle.gemm_mx(xc, xs, wc, ws, a)
    tol = _bound(oracle, xc, xs, wc, ws, a, K)
    if out_dtype == "bf16":
        tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    err = np.abs(got - ref)
    bad = np.argwhere(~(err <= tol))
    assert bad.size == 0, (name, bad[:5], got[tuple(bad[0])], ref[tuple(bad[0])])
    return got, ref


def _bf16_host(y):
    import torch

    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("tokens,out,K", [
    (256, 256, 512),     # one tile, fast path
    (300, 520, 1024),    # ragged tokens and channels, full stages
    (33, 70, 96),        # everything ragged: K is not a multiple of the stage, out % 4 != 0
    (520, 260, 800),     # several tiles with a partial last stage
    (1, 4, 32),          # the smallest call
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_gemm_matches_oracle(dq, oracle_lib, tokens, out, K, out_dtype):
    xc, xs = workloads.mx_operands(tokens, K, seed=1)
    wc, ws = workloads.mx_operands(out, K, seed=2)
    a = np.random.default_rng(out).uniform(0.02, 2.0, out).astype(np.float32)
    _check(dq, oracle_lib, xc, xs, wc, ws, a, out_dtype, name="random")
    if out_dtype == "f32":
        _check(dq, oracle_lib, xc, xs, wc, ws, None, out_dtype, name="a=None")


def _pack_reference(codes, scales, K):
    """The packed layout as dq.h states it: per 32-row block rb, stage s and k step i, 64 lanes
    x 16 bytes (lane L: row 32 rb + L % 32, chunk 4 (L / 32) + i of the stage); per rb and s,
    64 lanes x 4 scale bytes (k blocks 8 s + 4 (L / 32) .. + 3); padding rows zero / 127."""
    out, nst = codes.shape[0], K // 256
    nrb = -(-out // 32)
    c = np.zeros((nrb * 32, K // 2), np.uint8)
    c[:out] = codes
    sc = np.full((nrb * 32, K // 32), 127, np.uint8)
    sc[:out] = scales
    pc = np.empty((nrb, nst, 4, 64, 16), np.uint8)
    ps = np.empty((nrb, nst, 64, 4), np.uint8)
    for L in range(64):
        rl, h = L % 32, L // 32
        rows_c = c[rl::32].reshape(nrb, nst, 8, 16)
        for i in range(4):
            pc[:, :, i, L, :] = rows_c[:, :, 4 * h + i, :]
        ps[:, :, L, :] = sc[rl::32].reshape(nrb, nst, 8)[:, :, 4 * h:4 * h + 4]
    return pc.reshape(-1), ps.reshape(-1)


@pytest.mark.parametrize("out,K", [(70, 1024), (256, 512), (33, 2048)])
def test_pack_weights_layout(dq, out, K):
    wc, ws = workloads.mx_operands(out, K, seed=out)
    print(f"[gemm] pack out={out} K={K}", flush=True)
    pk = dq.gemm_pack_weights(_dev(wc), _dev(ws))
    want_c, want_s = _pack_reference(wc, ws, K)
    assert np.array_equal(host(pk["codes"]), want_c)
    assert np.array_equal(host(pk["scales"]), want_s)


@pytest.mark.parametrize("tokens,out,K", [
    (256, 256, 512),     # one tile
    (300, 520, 1024),    # ragged tokens and channels
    (97, 70, 512),       # channels neither a multiple of 32 nor of 4
    (33, 1000, 1536),    # several channel tiles, an odd number of stage pairs
    (1, 4, 512),         # the smallest call
    (300, 300, 3072),    # K % 1024 == 0: the four-stage ring, three trips of its loop
    (520, 260, 2048),    # the four-stage ring over several token tiles
])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_packed_gemm_matches_oracle(dq, oracle_lib, tokens, out, K, out_dtype):
    xc, xs = workloads.mx_operands(tokens, K, seed=5)
    wc, ws = workloads.mx_operands(out, K, seed=6)
    a = np.random.default_rng(out + 1).uniform(0.02, 2.0, out).astype(np.float32)
    _check(dq, oracle_lib, xc, xs, wc, ws, a, out_dtype, name="random", packed=True)
    if out_dtype == "f32":
        _check(dq, oracle_lib, xc, xs, wc, ws, None, out_dtype, name="a=None", packed=True)


# Whole 256 x 256 tiles with bf16 output (the shapes of the 8B MLP products): the 16-byte
# aligned output path, with and without a, against the oracle.
@pytest.mark.parametrize("tokens,out,K", [(512, 768, 1024), (256, 512, 2048), (768, 256, 3072)])
def test_packed_gemm_whole_tiles_match_oracle(dq, oracle_lib, tokens, out, K):
    xc, xs = workloads.mx_operands(tokens, K, seed=15)
    wc, ws = workloads.mx_operands(out, K, seed=16)
    a = np.random.default_rng(out + 3).uniform(0.02, 2.0, out).astype(np.float32)
    _check(dq, oracle_lib, xc, xs, wc, ws, a, "bf16", name="whole tiles", packed=True)
    _check(dq, oracle_lib, xc, xs, wc, ws, None, "bf16", name="whole tiles, a=None", packed=True)


def _bf16_rne(x):
    """float64 values that are exact in fp32, rounded to bf16 (nearest, ties to even)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def test_packed_gemm_whole_tiles_bf16_exact(dq, oracle_lib):
    # sums that fit fp32 exactly and power-of-two a: the bf16 output is the exact product
    # rounded once, the same bits as the oracle's value rounded to bf16
    tokens, out, K = 512, 512, 2048
    xc, xs = workloads.mx_operands(tokens, K, seed=17, lo=126, hi=129)
    wc, ws = workloads.mx_operands(out, K, seed=18, lo=126, hi=129)
    a = (2.0 ** np.random.default_rng(19).integers(-3, 4, out)).astype(np.float32)
    print(f"[gemm] whole tiles bf16 exact tokens={tokens} out={out} K={K}", flush=True)
    y = _bf16_host(_gemm(dq, xc, xs, wc, ws, a, "bf16", True))
    ref = oracle_lib.gemm_mx(xc, xs, wc, ws, a)
    assert np.array_equal(y, _bf16_rne(ref))


def test_packed_gemm_whole_tiles_more_than_one_per_cu(dq, oracle_lib):
    # 16 x 17 = 272 tiles, more than one per CU; sampled rows and channels, every tile's first
    # and last ones included
    tokens, out, K = 4096, 4352, 1024
    xc, xs = workloads.mx_operands(tokens, K, seed=25)
    wc, ws = workloads.mx_operands(out, K, seed=26)
    a = np.random.default_rng(27).uniform(0.5, 2.0, out).astype(np.float32)
    rng = np.random.default_rng(28)
    ts = np.unique(np.concatenate([np.arange(0, tokens, 256), np.arange(255, tokens, 256),
                                   rng.choice(tokens, 16, replace=False)]))
    cs = np.unique(np.concatenate([np.arange(0, out, 256), np.arange(255, out, 256),
                                   rng.choice(out, 16, replace=False)]))
    for aa in (a, None):
        print(f"[gemm] whole tiles x272 a={'yes' if aa is not None else 'no'}", flush=True)
        got = _bf16_host(_gemm(dq, xc, xs, wc, ws, aa, "bf16", True))[np.ix_(ts, cs)]
        asub = None if aa is None else aa[cs]
        ref = oracle_lib.gemm_mx(xc[ts], xs[ts], wc[cs], ws[cs], asub)
        tol = _bound(oracle_lib, xc[ts], xs[ts], wc[cs], ws[cs], asub, K)
        tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
        assert np.all(np.abs(got - ref) <= tol)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("tokens,out,K", [(256, 512, 2048), (97, 131, 224)])
def test_gemm_exact_when_the_sums_fit_fp32(dq, oracle_lib, tokens, out, K, packed):
    if packed and K % 512:
        pytest.skip("the packed form needs K % 512 == 0")
    # scales 2^-1 .. 2^1: products are multiples of 2^-4 below 2^7.2, sums of K of them stay
    # within 24 significant bits, so fp32 accumulation in any order is exact
    xc, xs = workloads.mx_operands(tokens, K, seed=3, lo=126, hi=129)
    wc, ws = workloads.mx_operands(out, K, seed=4, lo=126, hi=129)
    a = (2.0 ** np.random.default_rng(5).integers(-3, 4, out)).astype(np.float32)
    print(f"[gemm] exact tokens={tokens} out={out} K={K} packed={packed}", flush=True)
    y = host(_gemm(dq, xc, xs, wc, ws, a, "f32", packed))
    ref = oracle_lib.gemm_mx(xc, xs, wc, ws, a)
    assert np.array_equal(y.astype(np.float64), ref)


def test_gemm_nan_scale_and_zero_codes(dq, oracle_lib):
    xc, xs = workloads.mx_operands(64, 512, seed=6)
    wc, ws = workloads.mx_operands(96, 512, seed=7)
    xs = xs.copy()
    xs[5, 3] = 0xFF  # the E8M0 NaN: every output of token 5
    xc[9] = 0x88     # token 9 is all -0 codes
    print("[gemm] nan scale / zero codes", flush=True)
    y = host(dq.gemm_mx(_dev(xc), _dev(xs), _dev(wc), _dev(ws), out_dtype="f32"))
    ref = oracle_lib.gemm_mx(xc, xs, wc, ws)
    assert np.all(np.isnan(y[5])) and np.all(np.isnan(ref[5]))
    assert np.all(y[9] == 0.0)
    rest = np.delete(np.arange(64), [5])
    assert np.all(np.isfinite(y[rest]))


def test_gemm_on_the_quantizers_outputs(dq, oracle_lib):
    # the chain the product serves: W solved (MXFP4 G32), X quantized with the solver's b;
    # the GPU product of the GPU codes agrees with the oracle's product of the same codes
    import torch

    W = workloads.activations(192, 512, seed=11, dtype="f32")  # any well-scaled matrix
    X = workloads.activations(130, 512, seed=12, dtype="f32")
    print("[gemm] quantizer chain", flush=True)
    sol = dq.solve(torch.from_numpy(W).cuda(), "mxfp4", 32, 8)
    act = dq.quantize_act(torch.from_numpy(X).cuda(), "mxfp4", 32, sol["b"])
    y = host(dq.gemm_mx(act["codes"], act["scales"], sol["codes"], sol["scales"], sol["a"],
                        out_dtype="f32"))
    xc, xs = host(act["codes"]), host(act["scales"])
    wc, ws, a = host(sol["codes"]), host(sol["scales"]), host(sol["a"])
    ref = oracle_lib.gemm_mx(xc, xs, wc, ws, a)
    tol = _bound(oracle_lib, xc, xs, wc, ws, a, 512)
    assert np.all(np.abs(y - ref) <= tol)
    full = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.linalg.norm(y - full) / np.linalg.norm(full) < 0.6


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("which", ["up", "down"])
def test_gemm_full_size_llama8b_mlp_sampled(dq, oracle_lib, which, packed):
    # up / gate: 8192 tokens x 4096 -> 14336 channels; down: 8192 x 14336 -> 4096; bf16 out,
    # checked on sampled token rows x channel columns
    tokens = 8192
    K, out = {"up": (4096, 14336), "down": (14336, 4096)}[which]
    xc, xs = workloads.mx_operands(tokens, K, seed=21)
    wc, ws = workloads.mx_operands(out, K, seed=22)
    a = np.random.default_rng(23).uniform(0.5, 2.0, out).astype(np.float32)
    print(f"[gemm] full size {which} packed={packed}", flush=True)
    y = _gemm(dq, xc, xs, wc, ws, a, "bf16", packed)
    rng = np.random.default_rng(24)
    ts = np.sort(rng.choice(tokens, 24, replace=False))
    ts[0], ts[-1] = 0, tokens - 1
    cs = np.sort(rng.choice(out, 40, replace=False))
    cs[0], cs[-1] = 0, out - 1
    got = _bf16_host(y)[np.ix_(ts, cs)]
    ref = oracle_lib.gemm_mx(xc[ts], xs[ts], wc[cs], ws[cs], a[cs])
    tol = _bound(oracle_lib, xc[ts], xs[ts], wc[cs], ws[cs], a[cs], K)
    tol = tol + 2.0 ** -8 * (np.abs(ref) + tol)
    assert np.all(np.abs(got - ref) <= tol)


@pytest.mark.parametrize("packed", [False, True])
def test_gemm_split_into_launches_at_the_largest_k(dq, oracle_lib, packed):
    # K = 2^22: 2 MiB of codes per row; a launch keeps every offset below 2^31, so the 1100
    # tokens run as launches over chunks of 512 tokens
    import torch

    K, tokens, out = 2 ** 22, 1100, 8
    g = torch.Generator(device="cuda").manual_seed(31)
    xc = torch.randint(0, 256, (tokens, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    xs = torch.randint(124, 131, (tokens, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    wc = torch.randint(0, 256, (out, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    ws = torch.randint(124, 131, (out, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    print(f"[gemm] K=2^22 tokens={tokens} out={out} packed={packed}", flush=True)
    if packed:
        y = host(dq.gemm_mx_packed(xc, xs, dq.gemm_pack_weights(wc, ws), out_dtype="f32"))
    else:
        y = host(dq.gemm_mx(xc, xs, wc, ws, out_dtype="f32"))
    ts = np.array([0, 511, 512, 767, 768, 1023, 1024, 1099])  # around every chunk edge
    xch, xsh = host(xc[ts]), host(xs[ts])
    wch, wsh = host(wc), host(ws)
    ref = oracle_lib.gemm_mx(xch, xsh, wch, wsh)
    tol = _bound(oracle_lib, xch, xsh, wch, wsh, None, K)
    assert np.all(np.abs(y[ts] - ref) <= tol)
    del xc, wc


def test_gemm_random_shapes(dq, oracle_lib):
    # seeded random shapes through both forms and both output types: tokens and channels
    # anywhere in 1..600, K any multiple of 32 (of 512 for the packed form)
    rng = np.random.default_rng(2024)
    for case in range(16):
        tokens, out = int(rng.integers(1, 600)), int(rng.integers(1, 600))
        packed = bool(case % 2)
        K = int(rng.integers(1, 5)) * 512 if packed else int(rng.integers(1, 48)) * 32
        out_dtype = "bf16" if case % 3 == 0 else "f32"
        xc, xs = workloads.mx_operands(tokens, K, seed=100 + case)
        wc, ws = workloads.mx_operands(out, K, seed=200 + case)
        a = rng.uniform(0.05, 3.0, out).astype(np.float32) if case % 4 else None
        _check(dq, oracle_lib, xc, xs, wc, ws, a, out_dtype, name=f"random case {case}",
               packed=packed)


def test_matrix_core_rate_hook(dq):
    # dq_bench_fp4_mfma_rate: a positive dense-equivalent rate below the published 10.1 PFLOP/s
    # peak (a stream at a settled clock reaches 8.6-8.9 on MI355X; a short, cold one less)
    print("[gemm] matrix-core rate hook", flush=True)
    rates = [dq.bench_fp4_mfma_rate(2000) for _ in range(3)]
    assert all(0.0 < r < 10100.0 for r in rates), rates
    assert max(rates) > 2000.0, rates

"""The seeded generators are deterministic and follow their stated recipe."""
import numpy as np

import workloads


def test_generators_are_deterministic():
    a = workloads.config2(64, 128)
    b = workloads.config2(64, 128)
    assert a.sha256() == b.sha256()
    c = workloads.config3("up", 40, 256)
    assert c.W.dtype == np.uint16 and c.W.shape == (40, 256)


def test_chunked_draws_match_one_shot():
    # rows beyond one chunk continue the same PCG64 stream
    w = workloads.config4(2100, 32)
    rng = workloads.rng_for(4)
    mult = np.exp(rng.normal(0.0, 0.7, size=32))
    z = rng.standard_normal((2100, 32))
    want = workloads.fp32_to_bf16_bits((z * 0.01 * mult[None, :]).astype(np.float32))
    assert np.array_equal(w.W, want)


def test_outlier_columns_present():
    w = workloads.config3("up", 64, 1000)
    x = workloads.bf16_bits_to_fp32(w.W)
    norms = np.sqrt((x.astype(np.float64) ** 2).sum(0))
    big = norms > 5 * np.median(norms)
    assert big.sum() == 10  # 1% of 1000 input columns
    layer = workloads.config5_layer(0, scale_down=16)
    assert [m.name.split("_")[2] for m in layer] == ["q", "k", "v", "o", "gate", "up", "down"]


def test_bf16_rounding_of_generator_matches_torch():
    import torch

    rng = np.random.default_rng(1)
    x = (rng.normal(0, 1, 10000) * np.exp(rng.normal(0, 5, 10000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.fp32_to_bf16_bits(x), want)

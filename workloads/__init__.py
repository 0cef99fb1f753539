"""Seeded synthetic weight matrices for the dual-scale solver workloads.

This module only draws inputs. It holds none of the solver's arithmetic (no
quantizer, no scale rule, no projection), and both the HIP path and the CPU
oracle consume the buffers it returns.

The shapes stand in for the Llama-3.1-8B / 70B checkpoints and the
SmolLM2-135M layers that the DualQuant pages evaluate on (daiwk reproduction
notes, "论文离线与线上效果" Table 1 and "本地复现"); no checkpoint is used. Value
distributions mimic what the pages attribute to real weights: a few input
columns with much larger norms, which line up with activation-outlier
channels (trove summary, "How it works").

Recipe (identical on every machine):
  * generator: ``numpy.random.default_rng(SeedSequence([20261009, cfg, layer, matrix]))``
    (PCG64); a layer-wide outlier set uses ``matrix = 99``;
  * draws are float64, scaled in float64, rounded to fp32 with RNE, then to
    bf16 with RNE where the workload is bf16;
  * bf16 arrays are returned as ``uint16`` bit patterns (numpy has no bf16).

Workloads (rows = output channels, cols = input channels, groups run along cols):
  1. 128x256 fp32, N(0, 0.02^2), 4 random columns x20.  INT4/BF16, G=32, T=15.
  2. 2048x2048 bf16, Student-t(nu=4) * 0.02/sqrt(2) (std 0.02), per-column
     multipliers exp(N(0, 0.5^2)).  MXINT4, G=32, T=15.
  3. MLP up 14336x4096 and down 4096x14336 bf16, N(0, 0.015^2), 1% of input
     columns (41 / 143) scaled by U(10, 50).  MXFP4, G=32, T=20.
  4. 28672x8192 bf16, N(0, 0.01^2) * exp(N(0, 0.7^2)) per column.  NVFP4, G=16, T=20.
  5. 32 decoder layers x {q, o 4096x4096; k, v 1024x4096; gate, up 14336x4096;
     down 4096x14336} bf16, N(0, 0.02^2); per layer one outlier set per input
     space (20 of 4096 shared by q/k/v/gate/up, 20 of 4096 for o, 72 of 14336
     for down) scaled x20.  INT4/BF16, G=64, T=15.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Iterator, List, Optional, Tuple

import numpy as np

SEED_ROOT = 20261009
_CHUNK_ROWS = 2048  # rows drawn per chunk; the PCG64 stream is consumed in order


@dataclasses.dataclass
class Workload:
    """One weight matrix together with the solver settings it is solved with."""

    name: str
    W: np.ndarray  # float32 (dtype 'f32') or uint16 bf16 bit patterns (dtype 'bf16')
    dtype: str  # 'f32' or 'bf16'
    fmt: str  # 'int4_bf16' | 'mxint4' | 'mxfp4' | 'nvfp4'
    group: int
    T: int

    @property
    def rows(self) -> int:
        return int(self.W.shape[0])

    @property
    def cols(self) -> int:
        return int(self.W.shape[1])

    def sha256(self) -> str:
        return hashlib.sha256(np.ascontiguousarray(self.W).tobytes()).hexdigest()

    def as_fp32(self) -> np.ndarray:
        return self.W if self.dtype == "f32" else bf16_bits_to_fp32(self.W)


def rng_for(cfg: int, layer: int = 0, matrix: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED_ROOT, cfg, layer, matrix]))


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round to nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_fp32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _finish(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else fp32_to_bf16_bits(x32)


def _gaussian_matrix(rng: np.random.Generator, rows: int, cols: int, std: float,
                     col_mult: np.ndarray, dtype: str) -> np.ndarray:
    """rows x cols of N(0, std^2) * col_mult[col], drawn row-chunk by row-chunk."""
    out = np.empty((rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        z = rng.standard_normal((r1 - r0, cols))
        out[r0:r1] = _finish(z * std * col_mult[None, :], dtype)
    return out


def outlier_multipliers(rng: np.random.Generator, cols: int, count: int,
                        lo: float, hi: Optional[float]) -> np.ndarray:
    """Per-column multipliers: 1 everywhere, and on ``count`` distinct random
    columns either a fixed factor ``lo`` (hi is None) or U(lo, hi)."""
    mult = np.ones(cols, dtype=np.float64)
    idx = rng.choice(cols, size=count, replace=False)
    mult[idx] = lo if hi is None else rng.uniform(lo, hi, size=count)
    return mult


# --------------------------------------------------------------------------- configs
def config1(rows: int = 128, cols: int = 256) -> Workload:
    rng = rng_for(1)
    mult = outlier_multipliers(rng, cols, 4, 20.0, None)
    W = _gaussian_matrix(rng, rows, cols, 0.02, mult, "f32")
    return Workload(f"cfg1_tile_{rows}x{cols}", W, "f32", "int4_bf16", 32, 15)


def config2(rows: int = 2048, cols: int = 2048) -> Workload:
    rng = rng_for(2)
    mult = np.exp(rng.normal(0.0, 0.5, size=cols))
    out = np.empty((rows, cols), dtype=np.uint16)
    scale = 0.02 / np.sqrt(2.0)  # Student-t(4) has variance 2
    for r0 in range(0, rows, _CHUNK_ROWS):
        r1 = min(rows, r0 + _CHUNK_ROWS)
        z = rng.standard_t(4.0, size=(r1 - r0, cols))
        out[r0:r1] = _finish(z * scale * mult[None, :], "bf16")
    return Workload(f"cfg2_student_t_{rows}x{cols}", out, "bf16", "mxint4", 32, 15)


def config3(which: str, rows: Optional[int] = None, cols: Optional[int] = None) -> Workload:
    """``which`` is 'up' (14336x4096) or 'down' (4096x14336); 1% outlier input columns."""
    full = {"up": (14336, 4096), "down": (4096, 14336)}[which]
    rows = full[0] if rows is None else rows
    cols = full[1] if cols is None else cols
    rng = rng_for(3, 0, 0 if which == "up" else 1)
    count = max(1, int(round(0.01 * cols)))
    mult = outlier_multipliers(rng, cols, count, 10.0, 50.0)
    W = _gaussian_matrix(rng, rows, cols, 0.015, mult, "bf16")
    return Workload(f"cfg3_{which}_{rows}x{cols}", W, "bf16", "mxfp4", 32, 20)


def config4(rows: int = 28672, cols: int = 8192) -> Workload:
    rng = rng_for(4)
    mult = np.exp(rng.normal(0.0, 0.7, size=cols))
    W = _gaussian_matrix(rng, rows, cols, 0.01, mult, "bf16")
    return Workload(f"cfg4_70b_mlp_{rows}x{cols}", W, "bf16", "nvfp4", 16, 20)


CONFIG5_MATRICES: Tuple[Tuple[str, int, int, str], ...] = (
    # name, rows, cols, input space (which outlier set the columns use)
    ("q", 4096, 4096, "hidden"),
    ("k", 1024, 4096, "hidden"),
    ("v", 1024, 4096, "hidden"),
    ("o", 4096, 4096, "attn_out"),
    ("gate", 14336, 4096, "hidden"),
    ("up", 14336, 4096, "hidden"),
    ("down", 4096, 14336, "mlp_inner"),
)


def config5_layer(layer: int, scale_down: int = 1,
                  only: Optional[Tuple[str, ...]] = None) -> List[Workload]:
    """The seven matrices of decoder layer ``layer`` (or those named in ``only``; each
    matrix has its own stream, so a subset draws the same values). ``scale_down`` > 1
    divides every dimension (for oracle-sized test cases); outlier counts stay 0.5%."""
    orng = rng_for(5, layer, 99)
    spaces = {}
    for space, width in (("hidden", 4096), ("attn_out", 4096), ("mlp_inner", 14336)):
        w = width // scale_down
        count = max(1, int(round(0.005 * w)))
        spaces[space] = outlier_multipliers(orng, w, count, 20.0, None)
    out = []
    for mi, (name, r, c, space) in enumerate(CONFIG5_MATRICES):
        if only is not None and name not in only:
            continue
        r //= scale_down
        c //= scale_down
        rng = rng_for(5, layer, mi)
        W = _gaussian_matrix(rng, r, c, 0.02, spaces[space], "bf16")
        out.append(Workload(f"cfg5_L{layer}_{name}_{r}x{c}", W, "bf16", "int4_bf16", 64, 15))
    return out


def config5(layers: int = 32, scale_down: int = 1) -> Iterator[Workload]:
    for layer in range(layers):
        yield from config5_layer(layer, scale_down)


def reduced(cfg: int) -> List[Workload]:
    """Oracle-sized versions of each workload: same recipe, smaller shapes that
    still span several 512-column tiles and leave ragged row and column tails."""
    if cfg == 1:
        return [config1()]
    if cfg == 2:
        return [config2(384, 1056)]
    if cfg == 3:
        return [config3("up", 700, 1568), config3("down", 300, 2720)]
    if cfg == 4:
        return [config4(520, 1104)]
    if cfg == 5:
        return config5_layer(0, scale_down=8)
    raise ValueError(cfg)


def full(cfg: int) -> List[Workload]:
    if cfg == 1:
        return [config1()]
    if cfg == 2:
        return [config2()]
    if cfg == 3:
        return [config3("up"), config3("down")]
    if cfg == 4:
        return [config4()]
    raise ValueError("config 5 is a stream of 224 matrices: use config5()")


# ------------------------------------------------------------------- activations (next row)
ACT_CFG = 6  # seed-stream id of the activation inputs


def activations(tokens: int, cols: int, seed: int = 0, dtype: str = "bf16") -> np.ndarray:
    """Activation-like rows for the activation quantizer: N(0, 1) per entry times a
    per-channel lognormal(0, 0.5) level, and 1% of the channels a further x U(10, 50) (the
    outlier channels that the DualQuant pages tie to large-norm weight columns)."""
    rng = rng_for(ACT_CFG, 0, seed)
    level = np.exp(rng.normal(0.0, 0.5, size=cols))
    level *= outlier_multipliers(rng, cols, max(1, cols // 100), 10.0, 50.0)
    return _gaussian_matrix(rng, tokens, cols, 1.0, level, dtype)


def act_column_scales(cols: int, seed: int = 0) -> np.ndarray:
    """Column inverse scales for the activation inputs: powers of two 2^k, k uniform in
    [-3, 3], which are exact values of every outer scale set (BF16, E8M0 and E4M3)."""
    rng = rng_for(ACT_CFG, 1, seed)
    return np.ldexp(np.ones(cols, np.float32), rng.integers(-3, 4, size=cols)).astype(np.float32)


def act_inputs(name: str) -> Tuple[np.ndarray, np.ndarray]:
    """The activation quantizer's measured inputs: the Llama-3.1-8B MLP inputs of a batch of
    8192 tokens, 'up' (8192 x 4096, the input of the up / gate projections) or 'down'
    (8192 x 14336), bf16, with their column inverse scales."""
    cols = {"up": 4096, "down": 14336}[name]
    seed = {"up": 1, "down": 2}[name]
    return activations(8192, cols, seed), act_column_scales(cols, seed)


MX_CFG = 7  # seed-stream id of the packed MXFP4 operands


def mx_operands(rows: int, K: int, seed: int = 0, lo: int = 120, hi: int = 135,
                ) -> Tuple[np.ndarray, np.ndarray]:
    """Packed MXFP4 operands for the W4A4 product: rows x K/2 code bytes with every nibble
    uniform over the 16 E2M1 codes (both zeros included), and rows x K/32 E8M0 block-scale
    bytes uniform in [lo, hi) (the band a unit-scale tensor's blocks fall in)."""
    rng = rng_for(MX_CFG, rows, seed)
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales

"""Seeded synthetic inputs for the any4 dequantize-GEMM.

This module draws random numbers and rounds them to bf16; it holds none of
the method's arithmetic (no packing, dequantisation, GEMM or quantiser).  Both
the CPU oracle's tests and the HIP path's tests and benchmark take their
inputs from here, so the two sides always see identical bit patterns.

Rounding of draws to bf16 goes fp64 -> fp32 (numpy, nearest even) -> bf16
(torch's CPU conversion, nearest even).

The five workloads are decode-sized linear layers with Llama-like shapes (the
pages measure on Llama 2/3, Mistral and Mixtral weights, which are not
available here; these synthetic layers stand in for them):

  0  N=K=512, g=128, M=1 (small parity case)
  1  N=K=4096, g=128, M=1, x with 1% outlier channels scaled x20
  2  N=14336, K=4096, g=128, M in {1,2,4,8,16} (MLP up/gate)
  3  N=4096, K=14336, g=1024, M in {1,16} (MLP down), Student-t(4) tables
  4  70B decoder-layer shapes, g=128, M in {1,4,16}: raw W ~ N(0, 0.02) with
     0.1% of elements x10 and E|x| ~ LogNormal(0, 1); the any4 indices, table,
     alpha and beta come from the CPU oracle's weighted k-means (10 rounds),
     which the caller runs.

Draw order for configs 0-3: idx, LUT, alpha, beta, x.  x is drawn for the
largest M of the config; smaller M use its first rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def to_bf16_bits(a) -> np.ndarray:
    """fp64/fp32 values -> bf16 bit patterns (uint16), nearest even."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    t = torch.from_numpy(f).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    N: int
    K: int
    g: int
    Ms: tuple
    seed: int
    lut_dist: str = "normal"          # "normal" | "t4"
    alpha_range: tuple = (0.005, 0.02)
    beta_std: float = 0.002
    outlier_frac: float = 0.0         # fraction of x channels scaled
    outlier_scale: float = 20.0
    kmeans: bool = False              # config 4: weights come from k-means
    extra: dict = field(default_factory=dict)

    @property
    def max_m(self) -> int:
        return max(self.Ms)


CONFIGS = {
    0: Config(0, "any4 linear 512x512 g128", 512, 512, 128, (1,), seed=0),
    1: Config(1, "attention projection 4096x4096 g128, 1% outlier x channels", 4096, 4096,
              128, (1,), seed=1, outlier_frac=0.01),
    2: Config(2, "MLP up/gate 14336x4096 g128", 14336, 4096, 128, (1, 2, 4, 8, 16), seed=2),
    3: Config(3, "MLP down 4096x14336 g1024 Student-t LUT", 4096, 14336, 1024, (1, 16), seed=3,
              lut_dist="t4", alpha_range=(0.01, 0.05), beta_std=0.005),
}

# Config 4: one generated layer per distinct 70B decoder-layer shape.
CONFIG4_LAYERS = {
    "qkvo": dict(N=8192, K=8192, seed=40),
    "up_gate": dict(N=28672, K=8192, seed=41),
    "down": dict(N=8192, K=28672, seed=42),
}
CONFIG4_G = 128
CONFIG4_MS = (1, 4, 16)
CONFIG4_ITERS = 10


@dataclass
class Any4Inputs:
    """bf16 bit arrays for one any4 layer plus the x batch."""
    N: int
    K: int
    g: int
    idx: np.ndarray      # u8 [N, K], values 0..15
    lut: np.ndarray      # u16 [N, 16]
    alpha: np.ndarray    # u16 [N, K/g]
    beta: np.ndarray     # u16 [N, K/g]
    x: np.ndarray        # u16 [Mmax, K]


def _draw_lut(rng, N: int, dist: str) -> np.ndarray:
    if dist == "normal":
        v = rng.standard_normal((N, 16))
    elif dist == "t4":
        v = rng.standard_t(4, size=(N, 16))
    else:
        raise ValueError(dist)
    return to_bf16_bits(np.sort(v, axis=1))


def _draw_x(rng, M: int, K: int, outlier_frac: float, outlier_scale: float) -> np.ndarray:
    x = rng.standard_normal((M, K))
    if outlier_frac > 0:
        nout = int(round(outlier_frac * K))
        ch = rng.choice(K, size=nout, replace=False)
        x[:, ch] *= outlier_scale
    return to_bf16_bits(x)


def generate(cfg: int | Config, M: int | None = None, N: int | None = None,
             K: int | None = None) -> Any4Inputs:
    """Inputs for configs 0-3 (optionally resized: N, K override, same recipe)."""
    c = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    if c.kmeans:
        raise ValueError("config 4 comes from raw_layer() + the oracle quantiser")
    N = c.N if N is None else N
    K = c.K if K is None else K
    Mx = c.max_m if M is None else max(M, 1)
    rng = np.random.default_rng(c.seed)
    idx = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    lut = _draw_lut(rng, N, c.lut_dist)
    G = K // c.g
    alpha = to_bf16_bits(rng.uniform(c.alpha_range[0], c.alpha_range[1], size=(N, G)))
    beta = to_bf16_bits(rng.normal(0.0, c.beta_std, size=(N, G)))
    x = _draw_x(rng, Mx, K, c.outlier_frac, c.outlier_scale)
    return Any4Inputs(N, K, c.g, idx, lut, alpha, beta, x)


def generic(seed: int, M: int, N: int, K: int, g: int, lut_dist: str = "normal",
            alpha_range=(0.005, 0.02), beta_std: float = 0.002) -> Any4Inputs:
    """Any shape with the config-0 recipe (for ragged and edge-case tests)."""
    c = Config(-1, "generic", N, K, g, (M,), seed=seed, lut_dist=lut_dist,
               alpha_range=alpha_range, beta_std=beta_std)
    return generate(c, M=M)


@dataclass
class RawLayer:
    """Unquantised config-4 layer: W fp64 [N, K], E|x| fp64 [K], x bf16 bits."""
    name: str
    N: int
    K: int
    g: int
    W: np.ndarray
    Ex: np.ndarray
    x: np.ndarray


def raw_layer(name: str, rows: int | None = None) -> RawLayer:
    """Config-4 raw layer.  `rows` keeps only the first rows of W (the draw
    itself is unchanged, so row n is the same whatever `rows` is)."""
    spec = CONFIG4_LAYERS[name]
    N, K, seed = spec["N"], spec["K"], spec["seed"]
    rng = np.random.default_rng(seed)
    W = rng.normal(0.0, 0.02, size=(N, K))
    mask = rng.random((N, K)) < 0.001
    W[mask] *= 10.0
    Ex = rng.lognormal(0.0, 1.0, size=K)
    x = to_bf16_bits(rng.standard_normal((max(CONFIG4_MS), K)))
    if rows is not None:
        W = np.ascontiguousarray(W[:rows])
        N = rows
    return RawLayer(name, N, K, CONFIG4_G, W, Ex, x)


def fixed_table(name: str) -> np.ndarray:
    """The 16 values of a fixed 4-bit format as bf16 bits, for running the
    baseline formats the pages compare any4 with through the same table path:

      "int4"  0, 1, ..., 15 (uniform integer grid; scale and offset do the rest)
      "fp4"   E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit): code
              s<<3 | e<<1 | m is (-1)^s * (m/2) for e = 0, else
              (-1)^s * 2^(e-1) * (1 + m/2); 0..7 positive, 8..15 negative
      "nf4"   normal-float grid: quantiles of N(0, 1), eight on the positive
              side and seven on the negative side, each side scaled to reach
              1 in magnitude, plus an exact 0 (this module's reading of the
              published construction: the outermost quantile is taken at
              probability 1 - 1/32 on each side)
    """
    if name == "int4":
        v = np.arange(16, dtype=np.float64)
    elif name == "fp4":
        v = np.empty(16)
        for code in range(16):
            s, e, m = code >> 3, (code >> 1) & 3, code & 1
            mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
            v[code] = -mag if s else mag
    elif name == "nf4":
        from scipy.stats import norm
        top = 1.0 - 1.0 / 32.0
        pos = norm.ppf(0.5 + np.arange(1, 9) * (top - 0.5) / 8)
        neg = -norm.ppf(0.5 + np.arange(1, 8) * (top - 0.5) / 7)
        v = np.concatenate([np.sort(neg / neg.min() * -1.0), [0.0], pos / pos.max()])
    else:
        raise ValueError(name)
    return to_bf16_bits(v)

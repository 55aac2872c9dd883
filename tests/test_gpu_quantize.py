"""GPU parity of the any4 quantiser (any4_quantize, also at 3 and 2 bits) against the CPU oracle's
weighted k-means: the indices, tables, scales and offsets must be bit-identical
(both sides work in binary64 in the same order), on small layers, on the
degenerate cases (constant groups, a single round, no round), and on the first
rows of the 70B-shaped synthetic layers; and the quantised layer run through
pack and gemm gives the oracle's product."""
import numpy as np
import pytest
import torch

import gemm_any4_amd as any4
import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    gu.require_gpu()
    any4.lib()


def _quantize_both(W32, ex32, g, iters, bits=4):
    Wd = torch.from_numpy(W32).to(gu.DEV)
    exd = torch.from_numpy(ex32).to(gu.DEV)
    idx, lut, a, b = any4.quantize(Wd, exd, g, iters, bits=bits)
    torch.cuda.synchronize()
    ref = oracle.kmeans_quantize(W32.astype(np.float64), ex32.astype(np.float64), g, iters,
                                 bits=bits)
    got = (idx.cpu().numpy(), gu.host_b16(lut), gu.host_b16(a), gu.host_b16(b))
    return got, ref


def _check(got, ref, what):
    for name, x, y in zip(("idx", "lut", "alpha", "beta"), got, ref):
        if not np.array_equal(x, y):
            bad = np.argwhere(x != y)
            raise AssertionError(f"{what}: {name} differs at {len(bad)} places, first {tuple(bad[0])}:"
                                 f" {x[tuple(bad[0])]} vs {y[tuple(bad[0])]}")


@pytest.mark.parametrize("N,K,g,iters", [(100, 512, 128, 10), (65, 1024, 256, 3), (7, 384, 128, 1),
                                         (33, 256, 128, 0), (130, 2048, 1024, 10)])
def test_quantize_matches_oracle(N, K, g, iters):
    rng = np.random.default_rng(N * 7 + K + iters)
    W = rng.normal(0.0, 0.02, size=(N, K))
    W[rng.random((N, K)) < 0.001] *= 10.0
    ex = rng.lognormal(0.0, 1.0, size=K)
    got, ref = _quantize_both(W.astype(np.float32), ex.astype(np.float32), g, iters)
    _check(got, ref, f"{N}x{K} g{g} iters{iters}")


@pytest.mark.parametrize("N,K,g,iters", [(9, 96, 32, 4), (6, 200, 8, 3), (4, 330, 11, 3),
                                         (5, 2048, 1, 2)])
def test_quantize_odd_shapes(N, K, g, iters):
    """K not a multiple of 64 (a ragged last chunk of the wave-per-row
    kernel), groups shorter than a chunk or not dividing 64, and K/g above the
    wave kernel's LDS share (2048 groups: the thread-per-row kernel)."""
    rng = np.random.default_rng(N * 31 + K + g)
    W = rng.normal(0.0, 0.02, size=(N, K))
    ex = rng.lognormal(0.0, 1.0, size=K)
    got, ref = _quantize_both(W.astype(np.float32), ex.astype(np.float32), g, iters)
    _check(got, ref, f"{N}x{K} g{g} iters{iters}")


def test_quantize_degenerate_groups():
    """Constant groups (alpha = 0: every normalised weight is 0), a zero row,
    and zero importance on some channels."""
    rng = np.random.default_rng(3)
    N, K, g = 20, 512, 128
    W = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)
    W[0, :] = 0.0
    W[1, 128:256] = 0.5
    W[2, :] = -3.0
    ex = rng.lognormal(0.0, 1.0, size=K).astype(np.float32)
    ex[:64] = 0.0
    got, ref = _quantize_both(W, ex, g, 10)
    _check(got, ref, "degenerate")


@pytest.mark.parametrize("name", ["qkvo", "down"])
def test_quantize_70b_rows(name):
    """The first 64 rows of the 70B-shaped synthetic layers (K = 8192, 28672)."""
    raw = workloads.raw_layer(name, rows=64)
    got, ref = _quantize_both(raw.W.astype(np.float32), raw.Ex.astype(np.float32), raw.g,
                              workloads.CONFIG4_ITERS)
    _check(got, ref, name)


def test_quantize_then_gemm():
    """GPU quantise -> pack -> gemm against the oracle's dequantised product."""
    rng = np.random.default_rng(11)
    N, K, g, M = 200, 1024, 128, 4
    W = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)
    ex = rng.lognormal(0.0, 1.0, size=K).astype(np.float32)
    idx, lut, a, b = any4.quantize(torch.from_numpy(W).to(gu.DEV), torch.from_numpy(ex).to(gu.DEV),
                                   g, 10)
    packed = any4.pack(idx)
    x = workloads.to_bf16_bits(rng.standard_normal((M, K)))
    y = any4.gemm(gu.dev_b16(x), packed, lut, a, b, g)
    torch.cuda.synchronize()
    ridx, rlut, ra, rb = oracle.kmeans_quantize(W.astype(np.float64), ex.astype(np.float64), g, 10)
    w_ref = oracle.dequant(oracle.pack(ridx), rlut, ra, rb, g)
    y_ref, ad = oracle.gemm(x, w_ref)
    gu.assert_within_bound(y, y_ref, ad, "quantise then gemm")


@pytest.mark.parametrize("bits,N,K,g,iters", [(3, 100, 512, 128, 10), (2, 65, 1024, 256, 10),
                                              (3, 33, 256, 128, 0), (2, 64, 8192, 128, 10)])
def test_quantize_any3_any2_matches_oracle(bits, N, K, g, iters):
    rng = np.random.default_rng(bits * 100 + N)
    W = rng.normal(0.0, 0.02, size=(N, K))
    W[rng.random((N, K)) < 0.001] *= 10.0
    ex = rng.lognormal(0.0, 1.0, size=K)
    got, ref = _quantize_both(W.astype(np.float32), ex.astype(np.float32), g, iters, bits)
    _check(got, ref, f"any{bits} {N}x{K} g{g} iters{iters}")
    assert got[0].max() < (1 << bits)


@pytest.mark.parametrize("bits", [3, 2])
def test_any3_any2_layer_through_gemm(bits):
    """An any3 / any2 layer (indices below 8 / 4, table zero past them) runs
    through pack, dequant and gemm: dequant bit-exact, gemm within the bound."""
    rng = np.random.default_rng(50 + bits)
    N, K, g = 300, 2048, 128
    W = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)
    ex = rng.lognormal(0.0, 1.0, size=K).astype(np.float32)
    idx, lut, a, b = any4.quantize(torch.from_numpy(W).to(gu.DEV), torch.from_numpy(ex).to(gu.DEV),
                                   g, 10, bits=bits)
    packed = any4.pack(idx)
    ridx, rlut, ra, rb = oracle.kmeans_quantize(W.astype(np.float64), ex.astype(np.float64), g, 10,
                                                bits=bits)
    w_ref = oracle.dequant(oracle.pack(ridx), rlut, ra, rb, g)
    w = any4.dequant(packed, lut, a, b, g)
    x = workloads.to_bf16_bits(rng.standard_normal((16, K)))
    for M in (1, 16):
        y = any4.gemm(gu.dev_b16(x[:M]), packed, lut, a, b, g)
        torch.cuda.synchronize()
        y_ref, ad = oracle.gemm(x[:M], w_ref)
        gu.assert_within_bound(y, y_ref, ad, f"any{bits} M={M}")
    assert np.array_equal(gu.host_b16(w), w_ref)

"""Pins for the oracle's fp64 GEMM reference y = x * W^T (CPU only).

  * exact rational brute force on tiny non-square shapes (catches a
    transposed operand or a wrong index);
  * agreement with numpy's float64 matmul (a library routine) within the
    fp64 error bound;
  * one-hot x returns a column of W exactly; a constant table gives the
    rank-1 closed form w_n * sum_k x_k; table/index permutation leaves y
    bit-identical; x = 0 gives 0; doubling x doubles y exactly; each row of an
    M = 16 batch equals the M = 1 result on that row.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests import exact


def _layer(seed, M, N, K, g):
    inp = workloads.generic(seed, M, N, K, g)
    w = oracle.dequant(oracle.pack(inp.idx), inp.lut, inp.alpha, inp.beta, g)
    return inp, w


@pytest.mark.parametrize("M,N,K,g", [(1, 8, 128, 128), (2, 5, 256, 128), (2, 3, 256, 256)])
def test_gemm_exact_rational(M, N, K, g):
    inp, w = _layer(10 + M + N, M, N, K, g)
    y, ad = oracle.gemm(inp.x[:M], w)
    for m in range(M):
        for n in range(N):
            s = sum((exact.bf16_bits_to_fraction(int(inp.x[m, k])) *
                     exact.bf16_bits_to_fraction(int(w[n, k])) for k in range(K)), Fraction(0))
            a = sum((abs(exact.bf16_bits_to_fraction(int(inp.x[m, k])) *
                         exact.bf16_bits_to_fraction(int(w[n, k]))) for k in range(K)), Fraction(0))
            assert abs(Fraction(y[m, n]) - s) <= K * Fraction(1, 2 ** 52) * a
            assert abs(Fraction(ad[m, n]) - a) <= K * Fraction(1, 2 ** 52) * a


def test_gemm_vs_numpy_matmul():
    inp, w = _layer(20, 16, 96, 1024, 128)
    y, ad = oracle.gemm(inp.x, w)
    X = workloads.bf16_bits_to_f64(inp.x)
    Wf = workloads.bf16_bits_to_f64(w)
    ref = X @ Wf.T
    assert np.all(np.abs(y - ref) <= 2 * 1024 * 2.0 ** -53 * ad)
    assert np.allclose(ad, np.abs(X) @ np.abs(Wf).T, rtol=1e-12, atol=0)


def test_gemm_threads_do_not_change_results():
    inp, w = _layer(21, 4, 77, 512, 128)
    y1, a1 = oracle.gemm(inp.x, w, nthreads=1)
    y8, a8 = oracle.gemm(inp.x, w, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(a1, a8)


def test_one_hot_x_returns_column():
    inp, w = _layer(22, 1, 40, 256, 128)
    one = workloads.to_bf16_bits(np.array([1.0]))[0]
    for k in [0, 1, 127, 128, 255]:
        x = np.zeros((1, 256), np.uint16)
        x[0, k] = one
        y, _ = oracle.gemm(x, w)
        assert np.array_equal(y[0], workloads.bf16_bits_to_f64(w[:, k]))


def test_constant_lut_rank1():
    N, K, g = 12, 512, 128
    inp = workloads.generic(23, 4, N, K, g)
    c = workloads.to_bf16_bits(np.linspace(-1, 1, N))
    lut = np.repeat(c[:, None], 16, axis=1)
    a = np.repeat(inp.alpha[:, :1], K // g, axis=1)       # alpha, beta constant per row
    b = np.repeat(inp.beta[:, :1], K // g, axis=1)
    w = oracle.dequant(oracle.pack(inp.idx), lut, a, b, g)
    wn = workloads.bf16_bits_to_f64(w[:, 0])
    assert np.all(w == w[:, :1])
    y, ad = oracle.gemm(inp.x, w)
    X = workloads.bf16_bits_to_f64(inp.x)
    closed = np.outer(X.sum(axis=1), wn)
    assert np.all(np.abs(y - closed) <= 4 * K * 2.0 ** -53 * ad + 1e-300)
    assert np.linalg.matrix_rank(y) == 1


def test_permutation_gives_identical_y():
    inp = workloads.generic(24, 3, 18, 384, 128)
    rng = np.random.default_rng(24)
    lut2, idx2 = inp.lut.copy(), inp.idx.copy()
    for n in range(18):
        pi = rng.permutation(16)
        lut2[n, pi] = inp.lut[n]
        idx2[n] = pi[inp.idx[n]]
    w1 = oracle.dequant(oracle.pack(inp.idx), inp.lut, inp.alpha, inp.beta, 128)
    w2 = oracle.dequant(oracle.pack(idx2), lut2, inp.alpha, inp.beta, 128)
    assert np.array_equal(oracle.gemm(inp.x, w1)[0], oracle.gemm(inp.x, w2)[0])


def test_zero_x_and_doubling():
    inp, w = _layer(25, 2, 30, 256, 128)
    y0, _ = oracle.gemm(np.zeros_like(inp.x), w)
    assert np.all(y0 == 0)
    y1, _ = oracle.gemm(inp.x, w)
    x2 = workloads.to_bf16_bits(workloads.bf16_bits_to_f64(inp.x) * 2)
    y2, _ = oracle.gemm(x2, w)
    assert np.array_equal(y2, 2 * y1)


def test_batch_rows_equal_single_rows():
    inp, w = _layer(26, 16, 33, 512, 128)
    y16, a16 = oracle.gemm(inp.x, w)
    for m in [0, 5, 15]:
        y1, a1 = oracle.gemm(inp.x[m:m + 1], w)
        assert np.array_equal(y16[m], y1[0]) and np.array_equal(a16[m], a1[0])


def test_tolerance_formula():
    ad = np.array([0.0, 1.0, 100.0])
    assert np.allclose(oracle.tolerance(ad), [1e-3, 3e-3, 0.201])

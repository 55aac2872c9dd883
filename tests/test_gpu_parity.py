"""GPU parity: the HIP path through the C ABI against the CPU oracle.

  * pack and dequant: bit-exact on every config at full size and on ragged
    shapes;
  * gemm: every output within |y - y_ref| <= 2e-3 * sum|x w| + 1e-3 of the
    oracle's fp64 product, for configs 0-3 at every batch size (all outputs)
    and config 4 (70B decoder-layer shapes from the oracle's k-means) on
    sampled rows;
  * M > 16 (16-row slices, the tiled kernel): within the bound on ragged shapes, sampled rows
    of the 14336x4096 layer, and one-hot rows giving dequantised columns;
  * fixed formats (int4, fp4 E2M1, nf4) as tables: dequant bit-exact, gemm
    within the bound;
  * plain int4 (no table): bitwise equal to the table path with every row
    0..15 and within the bound of the oracle;
  * invariants on the device: identity table returns the indices, one-hot x
    returns a column of the dequantised W bit-exactly (also for table rows
    spanning more than 2^31, where the stated exactness condition holds), an
    inf in one x row leaves the other rows finite, permuting the table
    with its indices leaves y bit-identical, x = 0 gives 0, runs are
    deterministic, nothing is written outside y, the call honours a
    non-default stream, empty shapes are no-ops and K = 0 gives zeros.
"""
import functools

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


# --------------------------------------------------------------------------
# pack
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_pack_bitexact_configs(cfg):
    L = gu.config_layer(cfg)
    idx = gu.dev_u8(L.inp.idx)
    packed = any4.pack(idx)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), oracle.tile(L.packed_host))


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (7, 384), (17, 1024), (64, 4096),
                                 (33, 128), (1000, 640)])
def test_pack_ragged(N, K):
    rng = np.random.default_rng(N * 1000 + K)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)   # high bits must be ignored
    # the padding rows of the last block must come out zero, whatever was there
    packed = torch.full((any4.packed_bytes(N, K),), 0xA5, dtype=torch.uint8, device=gu.DEV)
    any4.pack(gu.dev_u8(idx), out=packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), oracle.tile(oracle.pack(idx)))


# --------------------------------------------------------------------------
# dequant
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_dequant_bitexact_configs(cfg):
    L = gu.config_layer(cfg)
    w = any4.dequant(L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref())


@pytest.mark.parametrize("N,K,g", [(1, 128, 128), (3, 384, 128), (33, 640, 128), (7, 2048, 1024),
                                   (5, 1536, 512), (129, 128, 128)])
def test_dequant_ragged(N, K, g):
    inp = workloads.generic(N + K + g, 1, N, K, g)
    L = gu.Layer(inp)
    w = any4.dequant(L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref())


def test_identity_table_returns_indices():
    """pack + in-kernel decode: LUT[i] = i, alpha = 1, beta = 0 gives idx exactly."""
    N, K, g = 40, 512, 128
    rng = np.random.default_rng(77)
    idx = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    lut = np.tile(workloads.to_bf16_bits(np.arange(16.0)), (N, 1))
    one = workloads.to_bf16_bits(np.ones((N, K // g)))
    zero = np.zeros((N, K // g), np.uint16)
    packed = any4.pack(gu.dev_u8(idx))
    w = any4.dequant(packed, gu.dev_b16(lut), gu.dev_b16(one), gu.dev_b16(zero), g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_f64(w), idx.astype(np.float64))


def test_dequant_rounding_ties_on_device():
    """alpha*L exactly half way between two bf16 values (beta = 0): nearest even."""
    N, K, g = 16, 256, 128
    rng = np.random.default_rng(5)
    a = rng.integers(0x3F80, 0x3FFF, size=(N, K // g)).astype(np.uint16)
    lut = rng.integers(0x3F80, 0x3FFF, size=(N, 16)).astype(np.uint16)
    idx = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    zero = np.zeros((N, K // g), np.uint16)
    inp = workloads.Any4Inputs(N, K, g, idx, lut, a, zero, np.zeros((1, K), np.uint16))
    L = gu.Layer(inp)
    w = any4.dequant(L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref())


# --------------------------------------------------------------------------
# gemm against the oracle
# --------------------------------------------------------------------------
CONFIG_MS = [(0, 1), (1, 1), (2, 1), (2, 2), (2, 4), (2, 8), (2, 16), (3, 1), (3, 16)]


@pytest.mark.parametrize("cfg,M", CONFIG_MS)
def test_gemm_configs(cfg, M):
    L = gu.config_layer(cfg)
    y = any4.gemm(L.x[:M], L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    y_ref, ad = gu.config_ref(cfg, M)
    r = gu.assert_within_bound(y, y_ref, ad, f"config {cfg} M={M}")
    print(f"config {cfg} M={M}: max err/tol = {r:.3e}", flush=True)


@functools.lru_cache(maxsize=1)
def _config4(name):
    raw = workloads.raw_layer(name)
    idx, lut, a, b = oracle.kmeans_quantize(raw.W, raw.Ex, raw.g, workloads.CONFIG4_ITERS)
    del raw.W
    inp = workloads.Any4Inputs(raw.N, raw.K, raw.g, idx, lut, a, b, raw.x)
    return gu.Layer(inp)


@pytest.mark.parametrize("name", ["qkvo", "up_gate", "down"])
def test_gemm_config4_all_outputs(name):
    """Every output of each 70B decoder-layer projection (weights from the
    oracle's weighted k-means) at M = 1, 4 and 16 against the oracle's fp64
    product over the whole dequantised matrix.  The oracle's y[m][n] depends
    on x row m only, so one product with 16 rows serves every M."""
    L = _config4(name)
    Mmax = max(workloads.CONFIG4_MS)
    y_ref, ad = oracle.gemm(L.inp.x[:Mmax], L.w_ref(), nthreads=oracle.default_threads())
    for M in workloads.CONFIG4_MS:
        y = any4.gemm(L.x[:M], L.packed, L.lut, L.alpha, L.beta, L.g)
        torch.cuda.synchronize()
        r = gu.assert_within_bound(y, y_ref[:M], ad[:M], f"config 4 {name} M={M}")
        print(f"config 4 {name} M={M}: all {M * L.N} outputs, max err/tol = {r:.3e}", flush=True)


@pytest.mark.parametrize("M,N,K,g", [(7, 16 * 700 + 5, 256, 128), (1, 16 * 1300, 512, 256),
                                     (1, 17, 128, 128), (3, 50, 384, 128), (5, 1, 256, 256),
                                     (7, 33, 1024, 512), (16, 15, 128, 128), (9, 100, 2048, 1024),
                                     (12, 272, 640, 128), (2, 4097, 256, 128),
                                     # row blocks per workgroup 5..8: two groups of decoded
                                     # blocks (3+2, 4+3, 4+4), and more than 256 workgroups
                                     (4, 16 * 1100, 256, 128), (16, 16 * 1700 + 9, 128, 128),
                                     (1, 16 * 2000 + 3, 128, 128), (3, 16 * 2100, 128, 128)])
def test_gemm_ragged(M, N, K, g):
    inp = workloads.generic(M * 7 + N + K, M, N, K, g)
    L = gu.Layer(inp)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref())
    gu.assert_within_bound(y, y_ref, ad, f"ragged {M}x{N}x{K} g{g}")


# The streaming kernel's two prologue orders: with a build item per thread
# (NBG * 256 threads or more) each wave stages its own blocks' table rows
# (one block, or the two blocks of a table region); K of 33 chunks makes the
# plan take fewer waves, so the first 32 * NBG threads stage every block and
# the workgroup meets at a barrier before the build.  Both against the
# oracle, at one, two and four blocks per group, M = 1 (x in LDS) and 16.
@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("N,K", [(16 * 200 + 3, 4096), (16 * 500, 4096), (16 * 900 + 9, 4096),
                                 (16 * 200 + 3, 33 * 128), (16 * 500, 33 * 128),
                                 (16 * 900 + 9, 33 * 128)])
def test_gemm_streaming_prologues(M, N, K):
    inp = workloads.generic(M * 13 + N + K, M, N, K, 128)
    L = gu.Layer(inp)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, 128)
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    gu.assert_within_bound(y, y_ref, ad, f"prologue {M}x{N}x{K}")


# Large K (> 4096): x staged in LDS (M <= 2, x <= 56 KB) or carried with the
# tiles; one or two row blocks decoded together, one or two groups of them.
@pytest.mark.parametrize("M,N,K,g", [(1, 64, 16384, 128), (16, 100, 8192, 1024),
                                     (4, 300, 14336, 1024), (2, 17, 28672, 128),
                                     (16, 33, 65536, 128), (3, 16, 4224, 384),
                                     (2, 16 * 300 + 7, 8192, 128), (1, 16 * 1000, 20480, 128),
                                     (5, 16 * 900, 6144, 256)])
def test_gemm_large_k(M, N, K, g):
    inp = workloads.generic(M * 3 + N + K, M, N, K, g)
    L = gu.Layer(inp)
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    gu.assert_within_bound(y, y_ref, ad, f"large K {M}x{N}x{K} g{g}")


# --------------------------------------------------------------------------
# M > 16: M <= 48 in one pass of the streaming kernel where it runs (two or
# three 16-row slices of x against each decoded weight tile), else 16-row
# slices through the decode kernels; above 48 the LDS-tiled MFMA kernel (64
# or 128 x rows per workgroup)
# --------------------------------------------------------------------------
# one pass: two to four row blocks per CU, or one with K > 4096 (including
# a workgroup with one block beside others with two, and ragged N and M)
@pytest.mark.parametrize("M,N,K,g", [(20, 16 * 600, 512, 128), (32, 16 * 600 + 5, 1024, 128),
                                     (33, 16 * 300, 256, 128), (48, 16 * 600, 640, 128),
                                     (24, 100, 8192, 1024), (47, 16 * 257, 384, 128),
                                     (17, 16 * 900, 4096, 128)])
def test_gemm_wide_batch_one_pass(M, N, K, g):
    inp = workloads.generic(M * 9 + N + K, M, N, K, g)
    L = gu.Layer(inp)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    r = gu.assert_within_bound(y, y_ref, ad, f"wide batch {M}x{N}x{K} g{g}")
    print(f"wide batch {M}x{N}x{K} g{g}: max err/tol = {r:.3e}", flush=True)


def test_gemm_wide_batch_one_hot_x_returns_dequantised_columns():
    """One-hot x rows, M = 48 on three row blocks per CU: every x row of each
    16-row slice lands in its own output row, bit-exactly the dequantised
    column (the slices share the decoded weights)."""
    inp = workloads.generic(93, 48, 16 * 600, 512, 128)
    L = gu.Layer(inp)
    w_ref = L.w_ref()
    one = workloads.to_bf16_bits(np.array([1.0]))[0]
    x = np.zeros((48, 512), np.uint16)
    ks = np.arange(48) * 10 + 7
    x[np.arange(48), ks] = one
    y = any4.gemm(gu.dev_b16(x), L.packed, L.lut, L.alpha, L.beta, 128)
    torch.cuda.synchronize()
    yb = gu.host_b16(y)
    for m, k in enumerate(ks):
        assert np.array_equal(yb[m], w_ref[:, k]), (m, k)


# 17..48 elsewhere: 16-row slices through the decode kernels; above: the tiled kernel
@pytest.mark.parametrize("M,N,K,g", [(17, 40, 256, 128), (48, 70, 256, 128), (49, 33, 256, 128),
                                     (64, 64, 128, 128), (65, 100, 512, 128),
                                     (100, 300, 1024, 256), (128, 17, 384, 128),
                                     (129, 65, 2048, 1024), (300, 130, 640, 128),
                                     (33, 16 * 50 + 3, 14336, 1024)])
def test_gemm_large_m(M, N, K, g):
    inp = workloads.generic(M * 5 + N + K, M, N, K, g)
    L = gu.Layer(inp)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    gu.assert_within_bound(y, y_ref, ad, f"large M {M}x{N}x{K} g{g}")


@pytest.mark.parametrize("M", [32, 256])
def test_gemm_large_m_config2_sampled_rows(M):
    """The 14336x4096 layer at prefill batches: sampled rows against the oracle."""
    L = gu.config_layer(2)
    rng = np.random.default_rng(M)
    x_host = workloads.to_bf16_bits(rng.standard_normal((M, L.K)))
    y = any4.gemm(gu.dev_b16(x_host), L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, L.N - 1], rng.choice(L.N, 200, replace=False)]))
    y_ref, ad = oracle.gemm(x_host, L.w_ref()[rows], nthreads=oracle.default_threads())
    gu.assert_within_bound(y[:, torch.from_numpy(rows).to(gu.DEV)], y_ref, ad,
                           f"config 2 M={M}")


def test_gemm_large_m_one_hot_x_returns_dequantised_columns():
    """One-hot x rows (M = 40) give the dequantised columns exactly: the tiled
    kernel multiplies the any4_dequant values."""
    inp = workloads.generic(91, 40, 48, 512, 128)
    L = gu.Layer(inp)
    w_ref = L.w_ref()
    one = workloads.to_bf16_bits(np.array([1.0]))[0]
    x = np.zeros((40, 512), np.uint16)
    ks = np.arange(40) * 12 + 3
    x[np.arange(40), ks] = one
    y = any4.gemm(gu.dev_b16(x), L.packed, L.lut, L.alpha, L.beta, 128)
    torch.cuda.synchronize()
    yb = gu.host_b16(y)
    for m, k in enumerate(ks):
        assert np.array_equal(yb[m], w_ref[:, k]), k


# --------------------------------------------------------------------------
# plain int4 (no table): w = alpha * q + beta
# --------------------------------------------------------------------------
def _identity_table(N):
    return np.tile(workloads.to_bf16_bits(np.arange(16.0)), (N, 1))


# Full-size layers (14336x4096 and 4096x14336, the k-major kernels for K <= 4096
# and for larger K), ragged shapes and large K.
@pytest.mark.parametrize("M,N,K,g,cfg", [(1, 0, 0, 0, 2), (16, 0, 0, 0, 2), (1, 0, 0, 0, 3),
                                         (16, 0, 0, 0, 3), (3, 16 * 700 + 5, 256, 128, None),
                                         (1, 17, 128, 128, None), (16, 15, 128, 128, None),
                                         (1, 16 * 2000 + 3, 128, 128, None),
                                         (2, 16 * 300 + 7, 8192, 128, None),
                                         (5, 100, 14336, 1024, None), (16, 33, 65536, 128, None),
                                         (40, 70, 512, 128, None), (200, 33, 1024, 256, None),
                                         (32, 16 * 600, 512, 128, None)])
def test_gemm_int4(M, N, K, g, cfg):
    """any4_gemm_int4 is bitwise any4_gemm with every table row 0..15 and the
    same workspace (none, or one that lets K split), and both are within the
    bound of the oracle's product with the int4 weights."""
    if cfg is not None:
        inp = gu.config_layer(cfg).inp
        x = gu.config_layer(cfg).x[:M]
        x_host = inp.x[:M]
    else:
        inp = workloads.generic(M * 11 + N + K, M, N, K, g)
        x, x_host = gu.dev_b16(inp.x), inp.x
    lut = _identity_table(inp.N)
    L = gu.Layer(workloads.Any4Inputs(inp.N, inp.K, inp.g, inp.idx, lut, inp.alpha, inp.beta,
                                      x_host))
    y4 = any4.gemm_int4(x, L.packed, L.alpha, L.beta, inp.g, workspace=gu.no_workspace())
    y = any4.gemm(x, L.packed, L.lut, L.alpha, L.beta, inp.g, workspace=gu.no_workspace())
    y4s = any4.gemm_int4(x, L.packed, L.alpha, L.beta, inp.g)             # K may be split
    ys = any4.gemm(x, L.packed, L.lut, L.alpha, L.beta, inp.g)            # ... the same way
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(y4), gu.host_b16(y))
    assert np.array_equal(gu.host_b16(y4s), gu.host_b16(ys))
    w_int4 = L.w_ref()     # the oracle's dequant with the identity table is int4
    rows = np.arange(inp.N)
    if inp.N * inp.K > 1 << 24:   # full-size layers: sampled rows
        rng = np.random.default_rng(M)
        rows = np.unique(np.concatenate([[0, inp.N - 1], rng.choice(inp.N, 300, replace=False)]))
    y_ref, ad = oracle.gemm(x_host, w_int4[rows], nthreads=oracle.default_threads())
    sel = torch.from_numpy(rows).to(gu.DEV)
    gu.assert_within_bound(y4[:, sel], y_ref, ad, f"int4 {M}x{inp.N}x{inp.K} g{inp.g}")
    gu.assert_within_bound(ys[:, sel], y_ref, ad, f"table 0..15 {M}x{inp.N}x{inp.K} g{inp.g}")
    gu.assert_within_bound(y4s[:, sel], y_ref, ad, f"int4, split {M}x{inp.N}x{inp.K} g{inp.g}")


def test_gemm_int4_empty_and_k0():
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device=gu.DEV)
    e = torch.zeros((40, 0), dtype=torch.bfloat16, device=gu.DEV)
    y = torch.full((3, 40), 7.0, dtype=torch.bfloat16, device=gu.DEV)
    any4.gemm_int4(x, torch.zeros((0,), dtype=torch.uint8, device=gu.DEV), e, e, 128, out=y)
    torch.cuda.synchronize()
    assert (y == 0).all()


# --------------------------------------------------------------------------
# fixed 4-bit formats (int4, fp4, nf4) as tables through the same kernels
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["int4", "fp4", "nf4"])
@pytest.mark.parametrize("N,K,g", [(1000, 2048, 128), (300, 8192, 1024)])
def test_fixed_formats(fmt, N, K, g):
    inp = workloads.generic(17 + N + K, 16, N, K, g)
    lut = np.tile(workloads.fixed_table(fmt), (N, 1))
    L = gu.Layer(workloads.Any4Inputs(N, K, g, inp.idx, lut, inp.alpha, inp.beta, inp.x))
    w = any4.dequant(L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref())
    for M in (1, 16):
        y = any4.gemm(L.x[:M], L.packed, L.lut, L.alpha, L.beta, g)
        torch.cuda.synchronize()
        y_ref, ad = oracle.gemm(inp.x[:M], L.w_ref(), nthreads=oracle.default_threads())
        gu.assert_within_bound(y, y_ref, ad, f"{fmt} M={M} {N}x{K} g{g}")


# --------------------------------------------------------------------------
# invariants on the device
# --------------------------------------------------------------------------
def test_one_hot_x_returns_dequantised_columns():
    inp = workloads.generic(31, 16, 64, 1024, 256)
    L = gu.Layer(inp)
    w_ref = L.w_ref()
    one = workloads.to_bf16_bits(np.array([1.0]))[0]
    ks = [0, 1, 2, 31, 32, 127, 128, 255, 256, 511, 777, 1023]
    x = np.zeros((len(ks), 1024), np.uint16)
    for m, k in enumerate(ks):
        x[m, k] = one
    y = any4.gemm(gu.dev_b16(x), L.packed, L.lut, L.alpha, L.beta, 256)
    torch.cuda.synchronize()
    yb = gu.host_b16(y)
    for m, k in enumerate(ks):
        assert np.array_equal(yb[m], w_ref[:, k]), k


def test_permutation_gives_bitwise_identical_y():
    inp = workloads.generic(32, 16, 96, 1024, 128)
    rng = np.random.default_rng(32)
    lut2, idx2 = inp.lut.copy(), inp.idx.copy()
    for n in range(inp.N):
        pi = rng.permutation(16)
        lut2[n, pi] = inp.lut[n]
        idx2[n] = pi[inp.idx[n]]
    L1 = gu.Layer(inp)
    L2 = gu.Layer(workloads.Any4Inputs(inp.N, inp.K, inp.g, idx2, lut2, inp.alpha, inp.beta,
                                       inp.x))
    for M in (1, 4, 16):
        y1 = any4.gemm(L1.x[:M], L1.packed, L1.lut, L1.alpha, L1.beta, 128)
        y2 = any4.gemm(L2.x[:M], L2.packed, L2.lut, L2.alpha, L2.beta, 128)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_constant_table_rank1():
    N, K, g = 64, 1024, 128
    inp = workloads.generic(33, 16, N, K, g)
    c = workloads.to_bf16_bits(np.linspace(-2, 2, N))
    lut = np.repeat(c[:, None], 16, axis=1)
    a = np.repeat(inp.alpha[:, :1], K // g, axis=1)
    b = np.repeat(inp.beta[:, :1], K // g, axis=1)
    L = gu.Layer(workloads.Any4Inputs(N, K, g, inp.idx, lut, a, b, inp.x))
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    w_ref = L.w_ref()
    wn = workloads.bf16_bits_to_f64(w_ref[:, 0])
    X = workloads.bf16_bits_to_f64(inp.x)
    closed = np.outer(X.sum(axis=1), wn)
    _, ad = oracle.gemm(inp.x, w_ref)
    gu.assert_within_bound(y, closed, ad, "rank-1")


@pytest.mark.parametrize("M,N,K,g", [(1, 40, 512, 128), (16, 33, 1536, 128), (2, 20, 128 * 113, 128),
                                     (5, 17, 128 * 41, 128)])
def test_unused_non_finite_table_entry(M, N, K, g):
    """A table entry no weight uses may be inf or NaN: the product is still the
    finite oracle product (shapes with chunks past K in some waves)."""
    inp = workloads.generic(M + N + K, M, N, K, g)
    idx = np.maximum(inp.idx, 1)                      # entry 0 is never used
    lut = inp.lut.copy()
    lut[:, 0] = 0x7F80                                 # +inf
    lut[1::2, 0] = 0x7FC0                              # NaN on odd rows
    L = gu.Layer(workloads.Any4Inputs(N, K, g, idx, lut, inp.alpha, inp.beta, inp.x))
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref())
    gu.assert_within_bound(y, y_ref, ad, f"non-finite unused entry {M}x{N}x{K}")


def test_zero_x_gives_exact_zero():
    L = gu.config_layer(0)
    x = torch.zeros((16, L.K), dtype=torch.bfloat16, device=gu.DEV)
    y = any4.gemm(x, L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()) == 0


def test_deterministic():
    L = gu.config_layer(1)
    y1 = any4.gemm(L.x[:1], L.packed, L.lut, L.alpha, L.beta, L.g)
    y2 = any4.gemm(L.x[:1], L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_no_writes_outside_y():
    inp = workloads.generic(34, 5, 37, 512, 128)
    L = gu.Layer(inp)
    pad = 4096
    buf = torch.full((pad + 5 * 37 + pad,), -12345, dtype=torch.int16, device=gu.DEV)
    y = buf[pad:pad + 5 * 37].view(5, 37)
    any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, 128, out=y.view(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == -12345) and torch.all(buf[pad + 5 * 37:] == -12345)
    y_ref, ad = oracle.gemm(inp.x, L.w_ref())
    gu.assert_within_bound(y.view(torch.bfloat16), y_ref, ad, "guarded")


def test_non_default_stream():
    L = gu.config_layer(2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = any4.gemm(L.x[:4], L.packed, L.lut, L.alpha, L.beta, L.g)
        w = any4.dequant(L.packed, L.lut, L.alpha, L.beta, L.g)
    s.synchronize()
    y_ref, ad = gu.config_ref(2, 4)
    gu.assert_within_bound(y, y_ref, ad, "stream")
    assert np.array_equal(gu.host_b16(w), L.w_ref())


def test_empty_and_k0():
    L = gu.config_layer(0)
    y = torch.empty((0, L.N), dtype=torch.bfloat16, device=gu.DEV)
    any4.gemm(L.x[:0], L.packed, L.lut, L.alpha, L.beta, L.g, out=y)
    # K = 0: an empty sum
    x0 = torch.empty((3, 0), dtype=torch.bfloat16, device=gu.DEV)
    p0 = torch.empty((0,), dtype=torch.uint8, device=gu.DEV)
    ab0 = torch.empty((L.N, 0), dtype=torch.bfloat16, device=gu.DEV)
    y0 = torch.full((3, L.N), 7.0, dtype=torch.bfloat16, device=gu.DEV)
    any4.gemm(x0, p0, L.lut, ab0, ab0, 128, out=y0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y0.float()) == 0


def test_misaligned_pointer_is_rejected():
    L = gu.config_layer(0)
    xs = torch.zeros(L.K + 8, dtype=torch.bfloat16, device=gu.DEV)
    y = torch.zeros((1, L.N), dtype=torch.bfloat16, device=gu.DEV)
    s = any4.gemm_raw(xs.data_ptr() + 2, L.packed.data_ptr(), L.lut.data_ptr(),
                      L.alpha.data_ptr(), L.beta.data_ptr(), y.data_ptr(), 1, L.N, L.K, L.g)
    assert s == 3
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()) == 0


# --------------------------------------------------------------------------
# the table's range: the kernels hold a row's values as f16 scaled by a power
# of two (the row's largest finite magnitude lands in [2^14, 2^15)); a value
# is used exactly when it is 0 or its biased exponent is at least
# max(e_max - 31, 50), e_max that of the row's largest finite magnitude
# --------------------------------------------------------------------------
def _exact_in_kernel(lut_row: np.ndarray) -> np.ndarray:
    e = (lut_row.astype(np.int64) >> 7) & 0xFF
    finite = e != 0xFF
    emax = int(e[finite].max()) if finite.any() else 0
    mag = lut_row & 0x7FFF
    return (mag == 0) | (e >= max(emax - 31, 50))


def _row_scale(lut_row: np.ndarray) -> int:
    """The kernels' row scale exponent: 2^-s brings the row's largest finite
    magnitude into [2^14, 2^15), and s is at least -60."""
    e = (lut_row.astype(np.int64) >> 7) & 0xFF
    finite = e != 0xFF
    emax = int(e[finite].max()) if finite.any() else 0
    return max(emax - 141, -60)


@pytest.mark.parametrize("N", [48, 16 * 600])   # one row block per workgroup / three
def test_table_rows_spanning_more_than_2_31(N):
    """Table rows spanning far more than 2^31: 1.0 beside 2^-40 and a bf16
    subnormal; rows of only tiny or only subnormal values; 2^100 beside values
    near 1.  One-hot x (alpha = 1, beta = 0) returns each table value exactly
    where the exactness condition holds; any other value v comes back rounded
    to the f16 grid of the scaled row, within 2^(s-24) + 2^-8 |v| (a value
    below 2^(s-25) becomes 0).  Random x over the rows whose small values are
    negligible (all but the 2^100 rows): every output within the bound."""
    K, g, M = 512, 128, 16
    rng = np.random.default_rng(N)
    f = workloads.to_bf16_bits
    lut = f(rng.standard_normal((N, 16)))
    lut[0::5, :9] = f(np.array([1.0, 2.0 ** -40, 0.0, -0.5, 2.0 ** -20, 2.0 ** -31,
                                2.0 ** -32, -(2.0 ** -31), 3.0]))
    lut[0::5, 2] = 0x0001                                   # smallest bf16 subnormal
    lut[1::5] = f(rng.standard_normal((len(lut[1::5]), 16)) * 2.0 ** -100)   # all tiny
    lut[2::5] = rng.integers(1, 0x80, size=lut[2::5].shape).astype(np.uint16)  # subnormals
    lut[3::5, 0] = f(np.array([2.0 ** 100]))[0]
    idx = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    idx[:, :16] = np.arange(16, dtype=np.uint8)             # k < 16 uses entry k
    one = f(np.ones((N, K // g)))
    zero = np.zeros((N, K // g), np.uint16)
    x1 = np.zeros((M, K), np.uint16)
    x1[np.arange(M), np.arange(M)] = f(np.array([1.0]))[0]  # one-hot rows: column m
    L = gu.Layer(workloads.Any4Inputs(N, K, g, idx, lut, one, zero, x1))
    y = gu.host_b16(any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g))
    torch.cuda.synchronize()
    w = L.w_ref()
    exact = np.stack([_exact_in_kernel(lut[n]) for n in range(N)])     # [N][16]
    assert exact.any() and not exact.all()
    yv = workloads.bf16_bits_to_f64(y)
    wv = workloads.bf16_bits_to_f64(w[:, :M])
    scale = np.array([2.0 ** (_row_scale(lut[n]) - 24) for n in range(N)])
    for m in range(M):
        sel = exact[:, m]
        assert np.array_equal(y[m][sel], w[sel, m]), m
        err = np.abs(yv[m] - wv[:, m])
        assert np.all(err <= scale + np.abs(wv[:, m]) / 256), m
    # random x, random alpha and beta, rows without the 2^100 entry: within the bound
    keep = np.ones(N, bool)
    keep[3::5] = False
    inp = workloads.generic(N + 5, M, N, K, g)
    L2 = gu.Layer(workloads.Any4Inputs(N, K, g, idx, lut, inp.alpha, inp.beta, inp.x))
    y2 = any4.gemm(L2.x, L2.packed, L2.lut, L2.alpha, L2.beta, g)
    torch.cuda.synchronize()
    y_ref2, ad2 = oracle.gemm(inp.x, L2.w_ref()[keep])
    gu.assert_within_bound(y2[:, torch.from_numpy(np.flatnonzero(keep)).to(gu.DEV)], y_ref2,
                           ad2, "wide-range rows")


@pytest.mark.parametrize("N,K", [(40, 512), (16 * 600, 512), (16 * 600, 3840), (40, 384)])
def test_inf_in_one_x_row_stays_in_that_row(N, K):
    """M = 2 with x[1] holding +inf: y[0] is finite and matches the oracle
    (chunks past K in some waves must not read x row 1 for row 0)."""
    g = 128
    inp = workloads.generic(N * 3 + K, 2, N, K, g)
    x = inp.x.copy()
    x[1, 7] = 0x7F80
    L = gu.Layer(workloads.Any4Inputs(N, K, g, inp.idx, inp.lut, inp.alpha, inp.beta, x))
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert torch.isfinite(y[0].float()).all()
    y_ref, ad = oracle.gemm(x[:1], L.w_ref())
    gu.assert_within_bound(y[:1], y_ref, ad, f"row 0 beside an inf row, {N}x{K}")


# --------------------------------------------------------------------------
# K split over workgroups (with a workspace): long K, one or two row blocks
# per CU, more x rows than 4 per row block of a CU (M > 4 with one block,
# M > 8 with two); partial sums added in split order by a second kernel
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,M", [(3, 5), (3, 8), (3, 16)])
def test_split_k_config3(cfg, M):
    L = gu.config_layer(cfg)
    need = any4.workspace_size(M, L.N, L.K, L.g)
    assert need == 4 * M * L.N * 4          # four splits of fp32 partial sums
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=gu.DEV)   # never zeroed
    y1 = any4.gemm(L.x[:M], L.packed, L.lut, L.alpha, L.beta, L.g, workspace=ws)
    y2 = any4.gemm(L.x[:M], L.packed, L.lut, L.alpha, L.beta, L.g, workspace=ws)
    y0 = any4.gemm(L.x[:M], L.packed, L.lut, L.alpha, L.beta, L.g, workspace=gu.no_workspace())
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))   # deterministic
    y_ref, ad = gu.config_ref(cfg, M)
    r1 = gu.assert_within_bound(y1, y_ref, ad, f"split K, config {cfg} M={M}")
    r0 = gu.assert_within_bound(y0, y_ref, ad, f"unsplit, config {cfg} M={M}")
    print(f"config {cfg} M={M}: split max err/tol {r1:.3e}, unsplit {r0:.3e}", flush=True)


@pytest.mark.parametrize("M,N,K,g", [(5, 16 * 256, 12288, 128), (16, 16 * 512, 28672, 128),
                                     (11, 16 * 300, 16384 + 128, 128), (9, 16 * 256 + 3, 12800, 256)])
def test_split_k_ragged(M, N, K, g):
    inp = workloads.generic(M * 19 + N + K, M, N, K, g)
    L = gu.Layer(inp)
    assert any4.workspace_size(M, N, K, g) > 0
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    gu.assert_within_bound(y, y_ref, ad, f"split K {M}x{N}x{K} g{g}")


def test_split_k_workspace_errors():
    L = gu.config_layer(3)
    M = 16
    need = any4.workspace_size(M, L.N, L.K, L.g)
    small = torch.zeros(need - 16, dtype=torch.uint8, device=gu.DEV)
    y = torch.zeros((M, L.N), dtype=torch.bfloat16, device=gu.DEV)
    s = any4.gemm_raw(L.x.data_ptr(), L.packed.data_ptr(), L.lut.data_ptr(), L.alpha.data_ptr(),
                      L.beta.data_ptr(), y.data_ptr(), M, L.N, L.K, L.g, small.data_ptr(),
                      small.numel())
    assert s == 4          # ANY4_E_WORKSPACE, nothing launched
    torch.cuda.synchronize()
    assert torch.count_nonzero(y.float()) == 0
    assert any4.workspace_size(1, L.N, L.K, L.g) == 0       # M <= 2: never split
    assert any4.workspace_size(4, L.N, L.K, L.g) == 0       # 4 x rows, one block per CU
    assert any4.workspace_size(8, 8192, 28672, 128) == 0    # 8 x rows, two blocks per CU
    assert any4.workspace_size(9, 8192, 28672, 128) == 2 * 9 * 8192 * 4
    assert any4.workspace_size(16, 14336, 4096, 128) == 0   # short K: never split
    assert any4.workspace_size(16, 8192, 8192, 128) == 0


# --------------------------------------------------------------------------
# the M = 1 product on the vector ALUs (v_dot2), kept for comparison
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_gemv_dot_configs(cfg):
    L = gu.config_layer(cfg)
    y = any4.gemv_dot(L.x[:1], L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    y_ref, ad = gu.config_ref(cfg, 1)
    r = gu.assert_within_bound(y, y_ref, ad, f"gemv_dot config {cfg}")
    print(f"gemv_dot config {cfg}: max err/tol = {r:.3e}", flush=True)


@pytest.mark.parametrize("N,K,g", [(17, 128, 128), (16 * 700 + 5, 256, 128), (100, 14336, 1024),
                                   (16 * 300 + 9, 4096, 128), (40, 8192 + 128, 128)])
def test_gemv_dot_ragged(N, K, g):
    inp = workloads.generic(N * 7 + K, 1, N, K, g)
    L = gu.Layer(inp)
    y = any4.gemv_dot(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(inp.x, L.w_ref())
    gu.assert_within_bound(y, y_ref, ad, f"gemv_dot {N}x{K} g{g}")


def test_gemv_dot_one_hot_returns_dequantised_columns():
    inp = workloads.generic(35, 1, 16 * 300, 1024, 256)
    L = gu.Layer(inp)
    w_ref = L.w_ref()
    one = workloads.to_bf16_bits(np.array([1.0]))[0]
    for k in (0, 33, 511, 1023):
        x = np.zeros((1, 1024), np.uint16)
        x[0, k] = one
        y = any4.gemv_dot(gu.dev_b16(x), L.packed, L.lut, L.alpha, L.beta, 256)
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_b16(y)[0], w_ref[:, k]), k

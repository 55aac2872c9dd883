"""GPU parity of the any2 path (2-bit codes, four per byte) against the CPU
oracle: pack bit-exact against the oracle's restatement of the tile layout,
dequant bit-exact, gemm within the bound at every batch size (both GEMM
kernels, the 16-row slices and the tiled kernel for larger M) and bitwise equal
to any4_gemm on the same weights stored at 4 bits (same decode, same
summation order); and a layer from the GPU quantiser at 2 bits end to end."""
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


class Layer2:
    def __init__(self, seed, M, N, K, g):
        inp = workloads.generic(seed, M, N, K, g)
        self.N, self.K, self.g = N, K, g
        self.codes = (inp.idx & 3).astype(np.uint8)
        self.inp = inp
        self.packed = gu.dev_u8(oracle.tile2(oracle.pack2(self.codes)))
        self.packed4 = gu.dev_u8(oracle.tile(oracle.pack(self.codes)))
        self.lut, self.alpha, self.beta = (gu.dev_b16(inp.lut), gu.dev_b16(inp.alpha),
                                           gu.dev_b16(inp.beta))
        self.x = gu.dev_b16(inp.x)
        self.w_ref = oracle.dequant(oracle.pack(self.codes), inp.lut, inp.alpha, inp.beta, g)


@pytest.mark.parametrize("N,K", [(1, 128), (16, 256), (17, 384), (100, 1024), (1000, 4096)])
def test_any2_pack_bitexact(N, K):
    rng = np.random.default_rng(N + K)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)   # bits above 1 ignored
    packed = torch.full((any4.any2_packed_bytes(N, K),), 0x5A, dtype=torch.uint8, device=gu.DEV)
    any4.any2_pack(gu.dev_u8(idx), out=packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), oracle.tile2(oracle.pack2(idx)))


@pytest.mark.parametrize("N,K,g", [(33, 640, 128), (300, 2048, 1024), (16 * 900, 4096, 128)])
def test_any2_dequant_bitexact(N, K, g):
    L = Layer2(N + K, 1, N, K, g)
    w = any4.any2_dequant(L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref)


@pytest.mark.parametrize("M,N,K,g", [(1, 16 * 900, 4096, 128), (16, 16 * 900, 4096, 128),
                                     (2, 40, 512, 128), (4, 16 * 300 + 5, 1024, 256),
                                     (8, 33, 384, 128), (1, 4096 // 4, 14336, 1024),
                                     (16, 300, 14336, 1024), (3, 17, 8192 + 128, 128),
                                     (32, 70, 512, 128), (100, 65, 1024, 128),
                                     (1, 17, 128, 128), (16, 300, 128, 128)])
def test_any2_gemm(M, N, K, g):
    L = Layer2(M * 13 + N + K, M, N, K, g)
    y = any4.any2_gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    y4 = any4.gemm(L.x, L.packed4, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(y), gu.host_b16(y4))
    rows = np.arange(N)
    if N * K > 1 << 24:
        rng = np.random.default_rng(M)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 200, replace=False)]))
    y_ref, ad = oracle.gemm(L.inp.x, L.w_ref[rows], nthreads=oracle.default_threads())
    gu.assert_within_bound(y[:, torch.from_numpy(rows).to(gu.DEV)], y_ref, ad,
                           f"any2 {M}x{N}x{K} g{g}")


def test_any2_unused_table_entries_are_never_read():
    """Entries 4..15 of the table may hold anything (inf, NaN)."""
    L = Layer2(5, 4, 50, 1536, 128)
    lut = L.inp.lut.copy()
    lut[:, 4:] = 0x7FC0
    lut[::3, 4:] = 0x7F80
    y = any4.any2_gemm(L.x, L.packed, gu.dev_b16(lut), L.alpha, L.beta, 128)
    w = any4.any2_dequant(L.packed, gu.dev_b16(lut), L.alpha, L.beta, 128)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref)
    y_ref, ad = oracle.gemm(L.inp.x, L.w_ref)
    gu.assert_within_bound(y, y_ref, ad, "any2 non-finite unused entries")


def test_any2_quantised_layer_end_to_end():
    rng = np.random.default_rng(77)
    N, K, g = 400, 2048, 128
    W = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)
    ex = rng.lognormal(0.0, 1.0, size=K).astype(np.float32)
    idx, lut, a, b = any4.quantize(torch.from_numpy(W).to(gu.DEV), torch.from_numpy(ex).to(gu.DEV),
                                   g, 10, bits=2)
    packed = any4.any2_pack(idx)
    x = workloads.to_bf16_bits(rng.standard_normal((16, K)))
    ridx, rlut, ra, rb = oracle.kmeans_quantize(W.astype(np.float64), ex.astype(np.float64), g, 10,
                                                bits=2)
    w_ref = oracle.dequant(oracle.pack(ridx), rlut, ra, rb, g)
    for M in (1, 16):
        y = any4.any2_gemm(gu.dev_b16(x[:M]), packed, lut, a, b, g)
        torch.cuda.synchronize()
        y_ref, ad = oracle.gemm(x[:M], w_ref)
        gu.assert_within_bound(y, y_ref, ad, f"any2 quantised M={M}")

"""GPU parity of the any3 path (3-bit codes, 12 bytes per 32 weights) against
the CPU oracle: pack bit-exact against the oracle's restatement of the tile
layout, dequant bit-exact, gemm within the bound at every batch size (both
streaming kernels, the 16-row slices and the tiled kernel for larger M) and
bitwise equal to any4_gemm on the same weights stored at 4 bits (same table
values, same summation order); and a layer from the GPU quantiser at 3 bits
end to end."""
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


class Layer3:
    def __init__(self, seed, M, N, K, g):
        inp = workloads.generic(seed, M, N, K, g)
        self.N, self.K, self.g = N, K, g
        self.codes = (inp.idx & 7).astype(np.uint8)
        self.inp = inp
        self.packed = gu.dev_u8(oracle.tile3(self.codes))
        self.packed4 = gu.dev_u8(oracle.tile(oracle.pack(self.codes)))
        self.lut, self.alpha, self.beta = (gu.dev_b16(inp.lut), gu.dev_b16(inp.alpha),
                                           gu.dev_b16(inp.beta))
        self.x = gu.dev_b16(inp.x)
        self.w_ref = oracle.dequant(oracle.pack(self.codes), inp.lut, inp.alpha, inp.beta, g)


@pytest.mark.parametrize("N,K", [(1, 128), (16, 256), (17, 384), (100, 1024), (1000, 4096)])
def test_any3_pack_bitexact(N, K):
    rng = np.random.default_rng(N + K + 3)
    idx = rng.integers(0, 256, size=(N, K), dtype=np.uint8)   # bits above 2 ignored
    packed = torch.full((any4.any3_packed_bytes(N, K),), 0x5A, dtype=torch.uint8, device=gu.DEV)
    any4.any3_pack(gu.dev_u8(idx), out=packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), oracle.tile3(idx))


@pytest.mark.parametrize("N,K,g", [(33, 640, 128), (300, 2048, 1024), (16 * 900, 4096, 128)])
def test_any3_dequant_bitexact(N, K, g):
    L = Layer3(N + K + 1, 1, N, K, g)
    w = any4.any3_dequant(L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref)


@pytest.mark.parametrize("M,N,K,g", [(1, 16 * 900, 4096, 128), (16, 16 * 900, 4096, 128),
                                     (2, 40, 512, 128), (4, 16 * 300 + 5, 1024, 256),
                                     (8, 33, 384, 128), (1, 4096 // 4, 14336, 1024),
                                     (16, 300, 14336, 1024), (3, 17, 8192 + 128, 128),
                                     (32, 70, 512, 128), (100, 65, 1024, 128),
                                     (1, 17, 128, 128), (16, 300, 128, 128),
                                     # one pass of the streaming kernel for 17..48 rows
                                     (24, 16 * 600, 512, 128), (40, 16 * 300 + 5, 1024, 256),
                                     # K split over workgroups (with the default workspace)
                                     (16, 16 * 256, 12288, 128)])
def test_any3_gemm(M, N, K, g):
    L = Layer3(M * 17 + N + K, M, N, K, g)
    y = any4.any3_gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g, workspace=gu.no_workspace())
    y4 = any4.gemm(L.x, L.packed4, L.lut, L.alpha, L.beta, g, workspace=gu.no_workspace())
    ys = any4.any3_gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)      # K may be split
    y4s = any4.gemm(L.x, L.packed4, L.lut, L.alpha, L.beta, g)           # ... the same way
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(y), gu.host_b16(y4))
    assert np.array_equal(gu.host_b16(ys), gu.host_b16(y4s))
    rows = np.arange(N)
    if N * K > 1 << 24:
        rng = np.random.default_rng(M)
        rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 200, replace=False)]))
    y_ref, ad = oracle.gemm(L.inp.x, L.w_ref[rows], nthreads=oracle.default_threads())
    gu.assert_within_bound(y[:, torch.from_numpy(rows).to(gu.DEV)], y_ref, ad,
                           f"any3 {M}x{N}x{K} g{g}")


def test_any3_one_hot_x_gives_the_columns():
    """x = e_k gives column k of the dequantised W exactly, for every k of
    the first chunk and of a later one: each pair position of a lane slot
    (the three dwords and the top-bit pairs) reaches the right column."""
    L = Layer3(9, 1, 40, 512, 128)
    ks = list(range(128)) + list(range(384, 512))
    x = np.zeros((len(ks), 512), np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80                   # bf16 1.0
    xd = gu.dev_b16(x)
    for m0 in range(0, len(ks), 16):
        y = any4.any3_gemm(xd[m0:m0 + 16], L.packed, L.lut, L.alpha, L.beta, 128)
        torch.cuda.synchronize()
        yb = gu.host_b16(y)
        for m in range(yb.shape[0]):
            assert np.array_equal(yb[m], L.w_ref[:, ks[m0 + m]]), ks[m0 + m]


def test_any3_unused_table_entries_are_never_read():
    """Entries 8..15 of the table may hold anything (inf, NaN)."""
    L = Layer3(6, 4, 50, 1536, 128)
    lut = L.inp.lut.copy()
    lut[:, 8:] = 0x7FC0
    lut[::3, 8:] = 0x7F80
    y = any4.any3_gemm(L.x, L.packed, gu.dev_b16(lut), L.alpha, L.beta, 128)
    w = any4.any3_dequant(L.packed, gu.dev_b16(lut), L.alpha, L.beta, 128)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), L.w_ref)
    y_ref, ad = oracle.gemm(L.inp.x, L.w_ref)
    gu.assert_within_bound(y, y_ref, ad, "any3 non-finite unused entries")


def test_any3_quantised_layer_end_to_end():
    rng = np.random.default_rng(78)
    N, K, g = 400, 2048, 128
    W = rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)
    ex = rng.lognormal(0.0, 1.0, size=K).astype(np.float32)
    idx, lut, a, b = any4.quantize(torch.from_numpy(W).to(gu.DEV), torch.from_numpy(ex).to(gu.DEV),
                                   g, 10, bits=3)
    packed = any4.any3_pack(idx)
    x = workloads.to_bf16_bits(rng.standard_normal((16, K)))
    ridx, rlut, ra, rb = oracle.kmeans_quantize(W.astype(np.float64), ex.astype(np.float64), g, 10,
                                                bits=3)
    w_ref = oracle.dequant(oracle.pack(ridx), rlut, ra, rb, g)
    w = any4.any3_dequant(packed, lut, a, b, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(w), w_ref)
    for M in (1, 16):
        y = any4.any3_gemm(gu.dev_b16(x[:M]), packed, lut, a, b, g)
        torch.cuda.synchronize()
        y_ref, ad = oracle.gemm(x[:M], w_ref)
        gu.assert_within_bound(y, y_ref, ad, f"any3 quantised M={M}")

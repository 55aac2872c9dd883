"""GPU parity of the prefill path (M >= 128 with a workspace of N*K bf16): the
layer is dequantised into the workspace by the format's dequant kernel, then
multiplied by a library bf16 GEMM with fp32 accumulation.  Checked against
the CPU oracle (every output), against the tiled kernel that runs without a
workspace, with one-hot x (the dequantised columns exactly), through the
workspace contents (the exact any4_dequant values), for every weight format,
and through the allocation-free entry point (which runs the tiled kernel)."""
import numpy as np
import pytest
import torch

import gemm_any4_amd as any4
import oracle
import workloads
from tests import gpu_util as gu
from tests.test_gpu_any2 import Layer2
from tests.test_gpu_any3 import Layer3

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    gu.require_gpu()
    any4.lib()


SHAPES = [(128, 200, 512, 128), (256, 300, 1024, 128), (257, 17, 128, 128), (300, 16 * 40 + 3, 768, 256),
          (512, 1000, 2048, 1024), (1024, 64, 384, 128)]


@pytest.mark.parametrize("M,N,K,g", SHAPES)
def test_prefill_within_bound_and_beside_tiled(M, N, K, g):
    inp = workloads.generic(M * 3 + N + K, M, N, K, g)
    L = gu.Layer(inp)
    assert any4.workspace_size(M, N, K, g) == N * K * 2
    ws = torch.zeros(N * K * 2, dtype=torch.uint8, device=gu.DEV)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g, workspace=ws)
    yt = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g, workspace=gu.no_workspace())
    torch.cuda.synchronize()
    w_ref = L.w_ref()
    # the workspace holds the dequantised layer, bit for bit
    assert np.array_equal(ws.view(torch.int16).cpu().numpy().view(np.uint16).reshape(N, K), w_ref)
    y_ref, ad = oracle.gemm(inp.x, w_ref, nthreads=oracle.default_threads())
    gu.assert_within_bound(y, y_ref, ad, f"prefill {M}x{N}x{K} g{g}")
    gu.assert_within_bound(yt, y_ref, ad, f"tiled {M}x{N}x{K} g{g}")


def test_prefill_repeats_bit_for_bit():
    """The library GEMM's algorithm is picked on the first call of a shape (by
    timing the candidates on that call's operands, y overwritten meanwhile);
    that first result and every later one are the same bits."""
    M, N, K, g = 192, 16 * 20 + 5, 640, 128
    inp = workloads.generic(4242, M, N, K, g)
    L = gu.Layer(inp)
    ys = [any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    gu.assert_within_bound(ys[0], y_ref, ad, f"prefill first call {M}x{N}x{K} g{g}")


def test_prefill_one_hot_x_returns_dequantised_columns():
    M, N, K, g = 256, 48, 512, 128
    inp = workloads.generic(95, M, N, K, g)
    L = gu.Layer(inp)
    w_ref = L.w_ref()
    one = workloads.to_bf16_bits(np.array([1.0]))[0]
    x = np.zeros((M, K), np.uint16)
    ks = (np.arange(M) * 7 + 1) % K
    x[np.arange(M), ks] = one
    y = any4.gemm(gu.dev_b16(x), L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    yb = gu.host_b16(y)
    for m, k in enumerate(ks):
        assert np.array_equal(yb[m], w_ref[:, k]), (m, k)


def test_prefill_config2_sampled_rows():
    """The 14336x4096 layer at M = 1024 (the bench's largest prefill batch)."""
    L = gu.config_layer(2)
    M = 1024
    rng = np.random.default_rng(7)
    x_host = workloads.to_bf16_bits(rng.standard_normal((M, L.K)))
    y = any4.gemm(gu.dev_b16(x_host), L.packed, L.lut, L.alpha, L.beta, L.g)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, L.N - 1], rng.choice(L.N, 100, replace=False)]))
    y_ref, ad = oracle.gemm(x_host, L.w_ref()[rows], nthreads=oracle.default_threads())
    gu.assert_within_bound(y[:, torch.from_numpy(rows).to(gu.DEV)], y_ref, ad, "config 2 M=1024")


def test_prefill_int4_equals_identity_table():
    M, N, K, g = 256, 100, 1024, 128
    inp = workloads.generic(97, M, N, K, g)
    lut = np.tile(workloads.to_bf16_bits(np.arange(16.0)), (N, 1))
    L = gu.Layer(workloads.Any4Inputs(N, K, g, inp.idx, lut, inp.alpha, inp.beta, inp.x))
    y4 = any4.gemm_int4(L.x, L.packed, L.alpha, L.beta, g)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(y4), gu.host_b16(y))
    y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
    gu.assert_within_bound(y4, y_ref, ad, "prefill int4")


@pytest.mark.parametrize("bits", [2, 3])
def test_prefill_lowbit(bits):
    M, N, K, g = 256, 16 * 20 + 5, 1024, 256
    L = (Layer2 if bits == 2 else Layer3)(bits * 11, M, N, K, g)
    fn = any4.any2_gemm if bits == 2 else any4.any3_gemm
    y = fn(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    yt = fn(L.x, L.packed, L.lut, L.alpha, L.beta, g, workspace=gu.no_workspace())
    torch.cuda.synchronize()
    y_ref, ad = oracle.gemm(L.inp.x, L.w_ref, nthreads=oracle.default_threads())
    gu.assert_within_bound(y, y_ref, ad, f"prefill any{bits}")
    gu.assert_within_bound(yt, y_ref, ad, f"tiled any{bits}")


def test_prefill_noalloc_runs_the_tiled_kernel():
    M, N, K, g = 256, 40, 512, 128
    inp = workloads.generic(99, M, N, K, g)
    L = gu.Layer(inp)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=gu.DEV)
    rc = any4.gemm_noalloc_raw(L.x.data_ptr(), L.packed.data_ptr(), L.lut.data_ptr(),
                               L.alpha.data_ptr(), L.beta.data_ptr(), y.data_ptr(), M, N, K, g)
    assert rc == 0
    yt = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g, workspace=gu.no_workspace())
    torch.cuda.synchronize()
    assert np.array_equal(gu.host_b16(y), gu.host_b16(yt))

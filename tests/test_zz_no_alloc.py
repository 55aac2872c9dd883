"""GPU test of any4_gemm_noalloc, the entry point for callers that cannot
allocate: through the C ABI, two calls in a row (the second on a smaller
input), each bit-identical to any4_gemm given a workspace of
any4_gemm_workspace_size bytes and within the bound of the CPU oracle; and a
shape that needs no scratch."""
import numpy as np
import pytest
import torch

import gemm_any4_amd as any4
import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# both split K (the partial sums go to the library's scratch array); the
# second call is smaller in every dimension but N's block count
CASES = [(16, 4096, 14336, 1024), (5, 4096, 12288, 256)]


def _noalloc(L, M, N, K, g):
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=gu.DEV)
    s = any4.gemm_noalloc_raw(L.x.data_ptr(), L.packed.data_ptr(), L.lut.data_ptr(),
                              L.alpha.data_ptr(), L.beta.data_ptr(), y.data_ptr(), M, N, K, g)
    any4.check(s)
    return y


def test_noalloc_matches_the_workspace_entry_point_twice():
    gu.require_gpu()
    for M, N, K, g in CASES:
        need = any4.workspace_size(M, N, K, g)
        assert need > 0
        inp = workloads.generic(M * 31 + N + K, M, N, K, g)
        L = gu.Layer(inp)
        y_na = _noalloc(L, M, N, K, g)
        ws = torch.empty(need, dtype=torch.uint8, device=gu.DEV)
        y_ws = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), (M, N, K, g)
        y_ref, ad = oracle.gemm(inp.x, L.w_ref(), nthreads=oracle.default_threads())
        gu.assert_within_bound(y_na, y_ref, ad, f"noalloc {M}x{N}x{K} g{g}")


def test_noalloc_without_scratch():
    """A shape that does not split K uses no scratch and equals any4_gemm."""
    gu.require_gpu()
    M, N, K, g = 16, 1000, 2048, 128
    assert any4.workspace_size(M, N, K, g) == 0
    inp = workloads.generic(77, M, N, K, g)
    L = gu.Layer(inp)
    y_na = _noalloc(L, M, N, K, g)
    y = any4.gemm(L.x, L.packed, L.lut, L.alpha, L.beta, g)
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int16), y.view(torch.int16))

"""The GEMM calls inside a captured HIP graph: every replay, with eager work
and synchronisations between the replays and the output poisoned before
each one, gives bitwise the eager result.  Covers each format (any4, plain
int4, any2, any3), both streaming kernels, the 16-row slices, the tiled
kernel and the K = 0 fill (a kernel, not a memset, so that it can be
captured)."""
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


def _layer(M, N, K, g, seed):
    inp = workloads.generic(seed, M, N, K, g)
    codes3 = (inp.idx & 7).astype(np.uint8)
    codes2 = (inp.idx & 3).astype(np.uint8)
    return {
        "x": gu.dev_b16(inp.x), "lut": gu.dev_b16(inp.lut), "alpha": gu.dev_b16(inp.alpha),
        "beta": gu.dev_b16(inp.beta), "g": g, "N": N,
        "p4": gu.dev_u8(oracle.tile(oracle.pack(inp.idx))),
        "p2": gu.dev_u8(oracle.tile2(oracle.pack2(codes2))),
        "p3": gu.dev_u8(oracle.tile3(codes3)),
    }


def _call(fmt, L, M, out):
    x, lut, a, b, g = L["x"][:M], L["lut"], L["alpha"], L["beta"], L["g"]
    if fmt == "any4":
        any4.gemm(x, L["p4"], lut, a, b, g, out=out)
    elif fmt == "int4":
        any4.gemm_int4(x, L["p4"], a, b, g, out=out)
    elif fmt == "any2":
        any4.any2_gemm(x, L["p2"], lut, a, b, g, out=out)
    else:
        any4.any3_gemm(x, L["p3"], lut, a, b, g, out=out)


@pytest.mark.parametrize("fmt", ["any4", "int4", "any2", "any3"])
@pytest.mark.parametrize("M,N,K,g", [(1, 16 * 300 + 5, 1024, 128), (16, 33, 512, 128),
                                     (2, 70, 4096 + 1024, 256), (20, 40, 512, 128),
                                     (64, 70, 256, 128)])
def test_graph_replays_match_eager(fmt, M, N, K, g):
    L = _layer(M, N, K, g, M * 31 + N + K)
    eager = torch.empty((M, N), dtype=torch.bfloat16, device=gu.DEV)
    _call(fmt, L, M, eager)
    torch.cuda.synchronize()
    ref = gu.host_b16(eager)

    y = torch.empty((M, N), dtype=torch.bfloat16, device=gu.DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            _call(fmt, L, M, y)
    torch.cuda.synchronize()
    other = torch.empty_like(eager)
    for rep in range(3):
        y.fill_(float("nan"))                       # every output must be rewritten
        _call("any4", L, M, other)                  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gu.host_b16(y), ref), (fmt, rep)


def test_graph_k0_fill():
    """K = 0: y = 0 from a fill kernel inside the graph."""
    x = torch.empty((3, 0), dtype=torch.bfloat16, device=gu.DEV)
    lut = torch.zeros((10, 16), dtype=torch.bfloat16, device=gu.DEV)
    ab = torch.empty((10, 0), dtype=torch.bfloat16, device=gu.DEV)
    packed = torch.empty((0,), dtype=torch.uint8, device=gu.DEV)
    y = torch.empty((3, 10), dtype=torch.bfloat16, device=gu.DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            any4.gemm(x, packed, lut, ab, ab, 128, out=y)
    torch.cuda.synchronize()
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.count_nonzero(y.float()) == 0

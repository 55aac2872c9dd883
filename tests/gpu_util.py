"""Helpers shared by the GPU tests: host <-> device copies of bit arrays and
cached oracle results (the oracle runs on the CPU; nothing here computes the
method)."""
import functools

import numpy as np
import torch

import oracle
import workloads

DEV = torch.device("cuda:0")


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")


def no_workspace() -> torch.Tensor:
    """An empty workspace: any4_gemm then uses the kernels that need none (K
    is not split), the same summation order as the entry points without a
    workspace argument."""
    return torch.empty(0, dtype=torch.uint8, device=DEV)


def dev_u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_b16(a) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a torch.bfloat16 device tensor."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)


def host_b16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class Layer:
    """Device copies of one any4 layer plus its oracle dequant."""

    def __init__(self, inp: workloads.Any4Inputs, packed_host=None):
        self.inp = inp
        self.N, self.K, self.g = inp.N, inp.K, inp.g
        # row-major packing for the oracle; the device gets the same bytes in
        # the library's tile layout, both produced by the oracle
        self.packed_host = oracle.pack(inp.idx) if packed_host is None else packed_host
        self.packed = dev_u8(oracle.tile(self.packed_host))
        self.lut = dev_b16(inp.lut)
        self.alpha = dev_b16(inp.alpha)
        self.beta = dev_b16(inp.beta)
        self.x = dev_b16(inp.x)
        self._w = None

    def w_ref(self):
        if self._w is None:
            self._w = oracle.dequant(self.packed_host, self.inp.lut, self.inp.alpha,
                                     self.inp.beta, self.g)
        return self._w


@functools.lru_cache(maxsize=4)
def config_layer(cfg: int) -> Layer:
    return Layer(workloads.generate(cfg))


@functools.lru_cache(maxsize=16)
def config_ref(cfg: int, M: int):
    L = config_layer(cfg)
    return oracle.gemm(L.inp.x[:M], L.w_ref(), nthreads=oracle.default_threads())


def assert_within_bound(y_dev: torch.Tensor, y_ref: np.ndarray, absdot: np.ndarray, what=""):
    y = host_f64(y_dev)
    err = np.abs(y - y_ref)
    tol = oracle.tolerance(absdot)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs outside the bound; first at {tuple(i)}:"
                             f" y={y[tuple(i)]!r} ref={y_ref[tuple(i)]!r} tol={tol[tuple(i)]!r}")
    return float((err / tol).max()) if err.size else 0.0

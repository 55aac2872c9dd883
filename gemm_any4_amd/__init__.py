"""Python binding of libany4.so, the MI355X any4 dequantize-GEMM.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
in ``include/any4.h``.  PyTorch provides device memory and the current HIP
stream.  There is no CPU fallback: if the library is missing or a call fails,
a ``RuntimeError`` is raised.

Tensors
  idx     uint8  [N, K]     values 0..15, K a multiple of 128
  packed  uint8  [packed_bytes(N, K)]  the indices in the library's tile layout
                            (16 rows x 128 k per 1 KB tile; include/any4.h)
  lut     bf16   [N, 16]    per-row table
  alpha   bf16   [N, K/g]   per-group scale
  beta    bf16   [N, K/g]   per-group offset
  x       bf16   [M, K]     M = 1..16 (decode); larger M also accepted
  y       bf16   [M, N]
  w       bf16   [N, K]
(bf16 tensors may also be given as int16/uint16 bit patterns.)

Calls: pack, dequant, gemm (any4); gemm_int4 (plain int4, no table);
any2_pack / any2_dequant / any2_gemm and any3_pack / any3_dequant / any3_gemm
(2- and 3-bit codes in their own tile layouts); quantize (the weighted
k-means quantiser at 4, 3 or 2 bits); each also as a ``*_raw`` function on
device pointers that returns the C status.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libany4.so")

ANY4_OK = 0
_STATUS_NAMES = {0: "ANY4_OK", 1: "ANY4_E_NULL", 2: "ANY4_E_SHAPE", 3: "ANY4_E_ALIGN",
                 4: "ANY4_E_WORKSPACE", 5: "ANY4_E_HIP"}

# every symbol include/any4.h declares
EXPORTS = ("any4_packed_bytes", "any4_pack", "any4_dequant", "any4_gemm_workspace_size",
           "any4_gemm", "any4_gemm_noalloc", "any4_gemv_dot", "any4_gemm_int4", "any4_quantize", "any4_status_string",
           "any2_packed_bytes", "any2_pack", "any2_dequant", "any2_gemm",
           "any3_packed_bytes", "any3_pack", "any3_dequant", "any3_gemm", "any4_read_probe")

_lib = None


class Any4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libany4.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m gemm_any4_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.any4_packed_bytes.restype = SZ
        L.any4_packed_bytes.argtypes = [I64, I64]
        L.any4_pack.restype = ctypes.c_int
        L.any4_pack.argtypes = [P, P, I64, I64, P]
        L.any4_dequant.restype = ctypes.c_int
        L.any4_dequant.argtypes = [P, P, P, P, P, I64, I64, I64, P]
        L.any4_gemm_workspace_size.restype = SZ
        L.any4_gemm_workspace_size.argtypes = [I64, I64, I64, I64]
        L.any4_gemm.restype = ctypes.c_int
        L.any4_gemm.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, SZ, P]
        L.any4_gemm_noalloc.restype = ctypes.c_int
        L.any4_gemm_noalloc.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P]
        L.any4_gemv_dot.restype = ctypes.c_int
        L.any4_gemv_dot.argtypes = [P, P, P, P, P, P, I64, I64, I64, P]
        L.any4_gemm_int4.restype = ctypes.c_int
        L.any4_gemm_int4.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, SZ, P]
        L.any4_quantize.restype = ctypes.c_int
        L.any4_quantize.argtypes = [P, P, P, P, P, P, I64, I64, I64, ctypes.c_int, ctypes.c_int, P]
        for v in ("any2", "any3"):
            getattr(L, v + "_packed_bytes").restype = SZ
            getattr(L, v + "_packed_bytes").argtypes = [I64, I64]
            getattr(L, v + "_pack").restype = ctypes.c_int
            getattr(L, v + "_pack").argtypes = [P, P, I64, I64, P]
            getattr(L, v + "_dequant").restype = ctypes.c_int
            getattr(L, v + "_dequant").argtypes = [P, P, P, P, P, I64, I64, I64, P]
            getattr(L, v + "_gemm").restype = ctypes.c_int
            getattr(L, v + "_gemm").argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, P, SZ, P]
        L.any4_read_probe.restype = ctypes.c_int
        L.any4_read_probe.argtypes = [P, SZ, P, P]
        L.any4_status_string.restype = ctypes.c_char_p
        L.any4_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().any4_status_string(s).decode()


def check(s: int) -> None:
    if s != ANY4_OK:
        raise Any4Error(s, status_string(s))


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None or t.numel() == 0:
        return None
    return t.data_ptr()


def _u8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be uint8, got {t.dtype}")
    return _dev(t, name)


def _b16(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16 (or 16-bit bit patterns), got {t.dtype}")
    return _dev(t, name)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# --------------------------------------------------------------------------
# raw C-ABI calls (device pointers as ints)
# --------------------------------------------------------------------------
def pack_raw(idx_ptr, packed_ptr, N, K, stream=None) -> int:
    return lib().any4_pack(idx_ptr, packed_ptr, N, K, _stream(stream))


def dequant_raw(packed_ptr, lut_ptr, alpha_ptr, beta_ptr, w_ptr, N, K, g, stream=None) -> int:
    return lib().any4_dequant(packed_ptr, lut_ptr, alpha_ptr, beta_ptr, w_ptr, N, K, g,
                              _stream(stream))


def workspace_size(M: int, N: int, K: int, g: int) -> int:
    return int(lib().any4_gemm_workspace_size(M, N, K, g))


def packed_bytes(N: int, K: int) -> int:
    return int(lib().any4_packed_bytes(N, K))


def gemm_raw(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
             ws_ptr=None, ws_bytes=0, stream=None) -> int:
    return lib().any4_gemm(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                           ws_ptr, ws_bytes, _stream(stream))


def gemm_noalloc_raw(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                     stream=None) -> int:
    return lib().any4_gemm_noalloc(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M,
                                   N, K, g, _stream(stream))


def gemv_dot_raw(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, N, K, g,
                 stream=None) -> int:
    return lib().any4_gemv_dot(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, N, K, g,
                               _stream(stream))


def gemv_dot(x: torch.Tensor, packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor,
             beta: torch.Tensor, g: int, out: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
    """y [1, N] = x [1, K] * W^T on the vector ALUs (v_dot2) instead of the
    matrix cores: the same product as gemm at M = 1, for comparison."""
    _b16(x, "x"), _b16(lut, "lut"), _b16(alpha, "alpha"), _b16(beta, "beta")
    if x.dim() != 2 or x.shape[0] != 1:
        raise ValueError("x must be [1, K]")
    K = x.shape[1]
    N = lut.shape[0]
    if g <= 0 or K % g or alpha.shape != (N, K // g) or beta.shape != (N, K // g):
        raise ValueError("alpha/beta must be [N, K/g]")
    _check_packed(packed, N, K)
    if out is None:
        out = torch.empty((1, N), dtype=torch.bfloat16, device=x.device)
    _b16(out, "y")
    check(gemv_dot_raw(_ptr(x), _ptr(packed), _ptr(lut), _ptr(alpha), _ptr(beta), _ptr(out),
                       N, K, g, stream))
    return out


def gemm_int4_raw(x_ptr, packed_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                  ws_ptr=None, ws_bytes=0, stream=None) -> int:
    return lib().any4_gemm_int4(x_ptr, packed_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                                ws_ptr, ws_bytes, _stream(stream))


def quantize_raw(w_ptr, ex_ptr, idx_ptr, lut_ptr, alpha_ptr, beta_ptr, N, K, g, iters,
                 bits=4, stream=None) -> int:
    return lib().any4_quantize(w_ptr, ex_ptr, idx_ptr, lut_ptr, alpha_ptr, beta_ptr, N, K, g,
                               iters, bits, _stream(stream))


# --------------------------------------------------------------------------
# tensor API
# --------------------------------------------------------------------------
def pack(idx: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """idx uint8 [N, K] -> packed uint8 [packed_bytes(N, K)] (tile layout)."""
    _u8(idx, "idx")
    N, K = idx.shape
    nbytes = packed_bytes(N, K)
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=idx.device)
    _u8(out, "packed")
    if out.numel() != nbytes:
        raise ValueError(f"packed must hold {nbytes} bytes")
    check(pack_raw(_ptr(idx), _ptr(out), N, K, stream))
    return out


def _check_packed(packed: torch.Tensor, N: int, K: int) -> None:
    _u8(packed, "packed")
    if packed.numel() != packed_bytes(N, K):
        raise ValueError(f"packed must hold packed_bytes({N}, {K}) = {packed_bytes(N, K)} bytes")


def dequant(packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
            g: int, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Materialise the bf16 weights w [N, K] (N from lut, K = alpha.shape[1] * g)."""
    _b16(lut, "lut"), _b16(alpha, "alpha"), _b16(beta, "beta")
    if lut.dim() != 2 or lut.shape[1] != 16:
        raise ValueError("lut must be [N, 16]")
    N = lut.shape[0]
    if g <= 0 or alpha.dim() != 2 or alpha.shape[0] != N or beta.shape != alpha.shape:
        raise ValueError("alpha/beta must be [N, K/g]")
    K = alpha.shape[1] * g
    _check_packed(packed, N, K)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=lut.device)
    _b16(out, "w")
    if out.shape != (N, K):
        raise ValueError("w must be [N, K]")
    check(dequant_raw(_ptr(packed), _ptr(lut), _ptr(alpha), _ptr(beta), _ptr(out), N, K, g,
                      stream))
    return out


# One workspace per (device, stream), grown on demand: calls on one stream run
# one after another, so they can share it.  The kernels write every partial
# sum before they read it, so it needs no initialisation.
_workspaces: dict = {}


def _workspace(need: int, device: torch.device, stream_handle: int) -> torch.Tensor:
    key = (device.index, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def gemm(x: torch.Tensor, packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor,
         beta: torch.Tensor, g: int, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [M, N] = x [M, K] * W^T with W the any4 weights (N from lut).

    workspace: optional uint8 device tensor of at least workspace_size(M, N, K, g)
    bytes (contents need not be initialised); with it, K may be split over
    workgroups, their fp32 partial sums kept there, or (M >= 128) the layer is
    dequantised into it for one library bf16 GEMM.  An empty tensor runs the
    kernels that need no workspace.  By default a workspace kept per device
    and stream is used."""
    _b16(x, "x"), _b16(lut, "lut"), _b16(alpha, "alpha"), _b16(beta, "beta")
    M, K = x.shape
    if lut.dim() != 2 or lut.shape[1] != 16:
        raise ValueError("lut must be [N, 16]")
    N = lut.shape[0]
    if g <= 0 or K % g or alpha.shape != (N, K // g) or beta.shape != (N, K // g):
        raise ValueError("alpha/beta must be [N, K/g]")
    _check_packed(packed, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _b16(out, "y")
    if out.shape != (M, N):
        raise ValueError("y must be [M, N]")
    sh = _stream(stream)
    ws_ptr, ws_bytes = _workspace_args(workspace, M, N, K, g, x.device, sh)
    check(gemm_raw(_ptr(x), _ptr(packed), _ptr(lut), _ptr(alpha), _ptr(beta), _ptr(out), M, N, K,
                   g, ws_ptr, ws_bytes, sh))
    return out


def _workspace_args(workspace, M: int, N: int, K: int, g: int, device, sh):
    """(pointer, bytes) of the workspace for a GEMM call (split-K partial sums,
    or the dequantised layer for prefill batches): the caller's
    tensor (an empty one: none), else the cached one of this device and
    stream, or (None, 0) where the shape needs none."""
    need = workspace_size(M, N, K, g)
    if not need:
        return None, 0
    if workspace is None:
        workspace = _workspace(need, device, sh)
    if not workspace.numel():
        return None, 0
    _dev(workspace, "workspace")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def gemm_int4(x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
              g: int, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """y [M, N] = x [M, K] * W^T with plain int4 weights w = alpha * q + beta
    (q the 4-bit code, 0..15; N from alpha).  workspace as for gemm()."""
    _b16(x, "x"), _b16(alpha, "alpha"), _b16(beta, "beta")
    M, K = x.shape
    if g <= 0 or K % g or alpha.dim() != 2 or alpha.shape[1] != K // g or beta.shape != alpha.shape:
        raise ValueError("alpha/beta must be [N, K/g]")
    N = alpha.shape[0]
    _check_packed(packed, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _b16(out, "y")
    if out.shape != (M, N):
        raise ValueError("y must be [M, N]")
    sh = _stream(stream)
    ws_ptr, ws_bytes = _workspace_args(workspace, M, N, K, g, x.device, sh)
    check(gemm_int4_raw(_ptr(x), _ptr(packed), _ptr(alpha), _ptr(beta), _ptr(out), M, N, K, g,
                        ws_ptr, ws_bytes, sh))
    return out


def quantize(W: torch.Tensor, ex: torch.Tensor, g: int, iters: int = 10, bits: int = 4,
             stream=None):
    """any4-quantise W fp32 [N, K] with channel importance ex fp32 [K] (E|x|);
    bits = 3 or 2 for any3 / any2 (8 or 4 table values, indices below them).

    Returns (idx uint8 [N, K], lut bf16 [N, 16], alpha bf16 [N, K/g],
    beta bf16 [N, K/g]); pack idx with pack() before gemm()."""
    for t, name in ((W, "W"), (ex, "ex")):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {t.dtype}")
        _dev(t, name)
    N, K = W.shape
    if ex.shape != (K,):
        raise ValueError("ex must be [K]")
    if g <= 0 or K % g:
        raise ValueError("g must divide K")
    dev = W.device
    idx = torch.empty((N, K), dtype=torch.uint8, device=dev)
    lut = torch.empty((N, 16), dtype=torch.bfloat16, device=dev)
    alpha = torch.empty((N, K // g), dtype=torch.bfloat16, device=dev)
    beta = torch.empty((N, K // g), dtype=torch.bfloat16, device=dev)
    check(quantize_raw(_ptr(W), _ptr(ex), _ptr(idx), _ptr(lut), _ptr(alpha), _ptr(beta), N, K, g,
                       iters, bits, stream))
    return idx, lut, alpha, beta


# --------------------------------------------------------------------------
# any2 (2-bit codes, four per byte) and any3 (3-bit codes, 12 bytes per 32):
# tile layouts in include/any4.h
# --------------------------------------------------------------------------
def any2_packed_bytes(N: int, K: int) -> int:
    return int(lib().any2_packed_bytes(N, K))


def any3_packed_bytes(N: int, K: int) -> int:
    return int(lib().any3_packed_bytes(N, K))


def any2_pack_raw(idx_ptr, packed_ptr, N, K, stream=None) -> int:
    return lib().any2_pack(idx_ptr, packed_ptr, N, K, _stream(stream))


def any3_pack_raw(idx_ptr, packed_ptr, N, K, stream=None) -> int:
    return lib().any3_pack(idx_ptr, packed_ptr, N, K, _stream(stream))


def any2_dequant_raw(packed_ptr, lut_ptr, alpha_ptr, beta_ptr, w_ptr, N, K, g,
                     stream=None) -> int:
    return lib().any2_dequant(packed_ptr, lut_ptr, alpha_ptr, beta_ptr, w_ptr, N, K, g,
                              _stream(stream))


def any3_dequant_raw(packed_ptr, lut_ptr, alpha_ptr, beta_ptr, w_ptr, N, K, g,
                     stream=None) -> int:
    return lib().any3_dequant(packed_ptr, lut_ptr, alpha_ptr, beta_ptr, w_ptr, N, K, g,
                              _stream(stream))


def any2_gemm_raw(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                  ws_ptr=None, ws_bytes=0, stream=None) -> int:
    return lib().any2_gemm(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                           ws_ptr, ws_bytes, _stream(stream))


def any3_gemm_raw(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                  ws_ptr=None, ws_bytes=0, stream=None) -> int:
    return lib().any3_gemm(x_ptr, packed_ptr, lut_ptr, alpha_ptr, beta_ptr, y_ptr, M, N, K, g,
                           ws_ptr, ws_bytes, _stream(stream))


_LOWBIT = {2: (any2_packed_bytes, any2_pack_raw, any2_dequant_raw, any2_gemm_raw),
           3: (any3_packed_bytes, any3_pack_raw, any3_dequant_raw, any3_gemm_raw)}


def _lowbit_pack(bits: int, idx: torch.Tensor, out, stream) -> torch.Tensor:
    nbytes_of, pack_raw_, _, _ = _LOWBIT[bits]
    _u8(idx, "idx")
    N, K = idx.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    nbytes = nbytes_of(N, K)
    if out is None:
        out = torch.empty((nbytes,), dtype=torch.uint8, device=idx.device)
    _u8(out, "packed")
    if out.numel() != nbytes:
        raise ValueError(f"packed must hold {nbytes} bytes")
    check(pack_raw_(_ptr(idx), _ptr(out), N, K, stream))
    return out


def _check_lowbit_packed(bits: int, packed: torch.Tensor, N: int, K: int) -> None:
    _u8(packed, "packed")
    if packed.numel() != _LOWBIT[bits][0](N, K):
        raise ValueError(f"packed must hold any{bits}_packed_bytes({N}, {K}) bytes")


def _lowbit_dequant(bits: int, packed, lut, alpha, beta, g: int, out, stream) -> torch.Tensor:
    _b16(lut, "lut"), _b16(alpha, "alpha"), _b16(beta, "beta")
    if lut.dim() != 2 or lut.shape[1] != 16:
        raise ValueError("lut must be [N, 16]")
    N = lut.shape[0]
    if g <= 0 or alpha.dim() != 2 or alpha.shape[0] != N or beta.shape != alpha.shape:
        raise ValueError("alpha/beta must be [N, K/g]")
    K = alpha.shape[1] * g
    _check_lowbit_packed(bits, packed, N, K)
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=lut.device)
    _b16(out, "w")
    if out.shape != (N, K):
        raise ValueError("w must be [N, K]")
    check(_LOWBIT[bits][2](_ptr(packed), _ptr(lut), _ptr(alpha), _ptr(beta), _ptr(out), N, K, g,
                           stream))
    return out


def _lowbit_gemm(bits: int, x, packed, lut, alpha, beta, g: int, out, workspace,
                 stream) -> torch.Tensor:
    _b16(x, "x"), _b16(lut, "lut"), _b16(alpha, "alpha"), _b16(beta, "beta")
    M, K = x.shape
    if lut.dim() != 2 or lut.shape[1] != 16:
        raise ValueError("lut must be [N, 16]")
    N = lut.shape[0]
    if g <= 0 or K % g or alpha.shape != (N, K // g) or beta.shape != (N, K // g):
        raise ValueError("alpha/beta must be [N, K/g]")
    _check_lowbit_packed(bits, packed, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _b16(out, "y")
    if out.shape != (M, N):
        raise ValueError("y must be [M, N]")
    sh = _stream(stream)
    ws_ptr, ws_bytes = _workspace_args(workspace, M, N, K, g, x.device, sh)
    check(_LOWBIT[bits][3](_ptr(x), _ptr(packed), _ptr(lut), _ptr(alpha), _ptr(beta), _ptr(out),
                           M, N, K, g, ws_ptr, ws_bytes, sh))
    return out


def any2_pack(idx: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """idx uint8 [N, K] (codes 0..3) -> packed uint8 [any2_packed_bytes(N, K)]."""
    return _lowbit_pack(2, idx, out, stream)


def any3_pack(idx: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """idx uint8 [N, K] (codes 0..7) -> packed uint8 [any3_packed_bytes(N, K)]."""
    return _lowbit_pack(3, idx, out, stream)


def any2_dequant(packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor,
                 beta: torch.Tensor, g: int, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """bf16 weights [N, K] of an any2 layer (N from lut, K = alpha.shape[1] * g)."""
    return _lowbit_dequant(2, packed, lut, alpha, beta, g, out, stream)


def any3_dequant(packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor,
                 beta: torch.Tensor, g: int, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """bf16 weights [N, K] of an any3 layer (N from lut, K = alpha.shape[1] * g)."""
    return _lowbit_dequant(3, packed, lut, alpha, beta, g, out, stream)


def any2_gemm(x: torch.Tensor, packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor,
              beta: torch.Tensor, g: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [M, N] = x [M, K] * W^T with W an any2 layer (N from lut); workspace
    as for gemm()."""
    return _lowbit_gemm(2, x, packed, lut, alpha, beta, g, out, workspace, stream)


def any3_gemm(x: torch.Tensor, packed: torch.Tensor, lut: torch.Tensor, alpha: torch.Tensor,
              beta: torch.Tensor, g: int, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y [M, N] = x [M, K] * W^T with W an any3 layer (N from lut); workspace
    as for gemm()."""
    return _lowbit_gemm(3, x, packed, lut, alpha, beta, g, out, workspace, stream)


def read_probe_raw(buf_ptr, nbytes: int, out_ptr, stream=None) -> int:
    """The streaming-read probe (a measurement aid; see include/any4.h)."""
    return lib().any4_read_probe(buf_ptr, nbytes, out_ptr, _stream(stream))

"""any4 CPU oracle -- TEST INFRASTRUCTURE ONLY.

numpy-level wrappers around ``liboracle.so`` (plain C, see ``any4_oracle.c``).
Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's CPU
baseline leg may import this package; the product path (``gemm_any4_amd``)
never does.

All bf16 data is passed as ``uint16`` bit patterns.  Layouts are dense
row-major: idx ``[N, K]`` u8, packed ``[N, K/2]`` u8 (byte j holds index 2j in
bits 0..3 and 2j+1 in bits 4..7), lut ``[N, 16]``, alpha/beta ``[N, K/g]``,
x ``[M, K]``, w ``[N, K]``.  ``tile``/``untile`` convert the row-major
packing to and from the GPU library's tile layout, written here from the
layout's written specification (include/any4.h), not from the kernels.

What each function follows (the pages, by title and section):
  * the 10100.com any4 explainer, section 二: a row is 4-bit indices plus a
    16-entry bf16 table; step 1 "分组缩放": contiguous groups of g with a scale
    alpha and an offset beta; step 2 "E-Step"/"M-Step": weighted k-means with
    L_q = sum(alpha*w_s*E|x|) / sum(alpha*E|x|);
  * "any4: Learned 4-bit Numeric Representation for LLMs", abstract: the
    lookup-table matmul.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_bf16_to_f32.restype = ctypes.c_float
        lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_f32_to_bf16.restype = ctypes.c_uint16
        lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.orc_f64_to_bf16.restype = ctypes.c_uint16
        lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.orc_f32_to_bf16_array.restype = None
        lib.orc_f32_to_bf16_array.argtypes = [P, P, I64]
        lib.orc_pack.restype = None
        lib.orc_pack.argtypes = [P, P, I64, I64]
        lib.orc_unpack.restype = None
        lib.orc_unpack.argtypes = [P, P, I64, I64]
        lib.orc_dequant_one.restype = ctypes.c_uint16
        lib.orc_dequant_one.argtypes = [ctypes.c_uint16] * 3
        lib.orc_dequant.restype = None
        lib.orc_dequant.argtypes = [P, P, P, P, P, I64, I64, I64]
        lib.orc_gemm.restype = None
        lib.orc_gemm.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int]
        lib.orc_group_scale.restype = None
        lib.orc_group_scale.argtypes = [P, I64, I64, I64, P, P]
        lib.orc_kmeans_row.restype = None
        lib.orc_kmeans_row.argtypes = [P, P, I64, ctypes.c_int, P, P, P]
        lib.orc_kmeans_quantize_q.restype = ctypes.c_int
        lib.orc_kmeans_quantize_q.argtypes = [P, P, I64, I64, I64, ctypes.c_int, ctypes.c_int,
                                              P, P, P, P, ctypes.c_int]
        lib.orc_kmeans_row_q.restype = None
        lib.orc_kmeans_row_q.argtypes = [P, P, I64, ctypes.c_int, ctypes.c_int, P, P, P]
        lib.orc_group_scale_q.restype = None
        lib.orc_group_scale_q.argtypes = [P, I64, I64, I64, ctypes.c_int, P, P]
        lib.orc_kmeans_quantize.restype = ctypes.c_int
        lib.orc_kmeans_quantize.argtypes = [P, P, I64, I64, I64, ctypes.c_int, P, P, P, P,
                                            ctypes.c_int]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


# --------------------------------------------------------------------------
# bf16 helpers
# --------------------------------------------------------------------------
def bf16_to_f32(h) -> np.ndarray:
    """Exact widening: bf16 bits are the upper half of the binary32 bits."""
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f) -> np.ndarray:
    """binary32 -> bf16 bits, round to nearest even (oracle's own C routine)."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().orc_f32_to_bf16_array(_ptr(f), _ptr(out), f.size)
    return out


def f64_to_bf16_scalar(d: float) -> int:
    """binary64 -> bf16 bits with one rounding to nearest even."""
    return int(_load().orc_f64_to_bf16(float(d)))


# --------------------------------------------------------------------------
# pack / dequant / gemm
# --------------------------------------------------------------------------
def pack(idx) -> np.ndarray:
    idx = _c(idx, np.uint8)
    N, K = idx.shape
    assert K % 2 == 0
    out = np.empty((N, K // 2), np.uint8)
    _load().orc_pack(_ptr(idx), _ptr(out), N, K)
    return out


def unpack(packed, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K), np.uint8)
    _load().orc_unpack(_ptr(packed), _ptr(out), N, K)
    return out


# --------------------------------------------------------------------------
# the GPU library's tile layout (16 rows x 128 k per 1 KB tile)
# --------------------------------------------------------------------------
TILE_ROWS = 16
TILE_K = 128


def tiled_bytes(N: int, K: int) -> int:
    """Bytes of the tile layout: rows padded to a multiple of 16, K/2 bytes each."""
    return -(-N // TILE_ROWS) * TILE_ROWS * (K // 2)


def tile(packed) -> np.ndarray:
    """Row-major packed [N, K/2] -> tile layout (flat uint8).

    Pad the rows with zero rows to a multiple of 16, view the bytes as
    [N/16 blocks][16 rows][K/128 chunks][4 quarters][16 bytes] and store them
    in the order [blocks][chunks][quarters][rows][bytes]."""
    packed = _c(packed, np.uint8)
    N, K2 = packed.shape
    K = 2 * K2
    assert K % TILE_K == 0
    NB = -(-N // TILE_ROWS)
    P = np.zeros((NB * TILE_ROWS, K2), np.uint8)
    P[:N] = packed
    t = P.reshape(NB, TILE_ROWS, K // TILE_K, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def untile(t, N: int, K: int) -> np.ndarray:
    """Inverse of tile: tile layout -> row-major packed [N, K/2] (padding dropped)."""
    t = _c(t, np.uint8)
    NB = -(-N // TILE_ROWS)
    assert t.size == NB * TILE_ROWS * (K // 2)
    P = t.reshape(NB, K // TILE_K, 4, TILE_ROWS, 16).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(P).reshape(NB * TILE_ROWS, K // 2)[:N].copy()


# --------------------------------------------------------------------------
# any2: 2-bit codes, four per byte (the any4 paper's abstract names any2)
# --------------------------------------------------------------------------
def pack2(idx) -> np.ndarray:
    """idx u8 [N, K] (codes 0..3; higher bits ignored) -> [N, K/4] bytes:
    byte j of a row holds codes 4j .. 4j+3 in bits 0-1, 2-3, 4-5, 6-7."""
    idx = _c(idx, np.uint8)
    N, K = idx.shape
    assert K % 4 == 0
    q = (idx & 3).reshape(N, K // 4, 4).astype(np.uint8)
    return (q[:, :, 0] | (q[:, :, 1] << 2) | (q[:, :, 2] << 4) | (q[:, :, 3] << 6)).astype(np.uint8)


def unpack2(packed, K: int) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    out = np.empty((N, K // 4, 4), np.uint8)
    for s in range(4):
        out[:, :, s] = (packed >> (2 * s)) & 3
    return out.reshape(N, K)


def tiled2_bytes(N: int, K: int) -> int:
    """Bytes of the any2 tile layout: rows padded to a multiple of 16, K/4 bytes each."""
    return -(-N // TILE_ROWS) * TILE_ROWS * (K // 4)


def tile2(packed2) -> np.ndarray:
    """Row-major any2 bytes [N, K/4] -> the any2 tile layout (flat uint8):
    512-byte tiles of 16 rows x 128 k.  Pad the rows to a multiple of 16, view
    the bytes as [N/16][16 rows][K/128][4 quarters][8 bytes] and store them in
    the order [blocks][chunks][quarters][rows][bytes]."""
    packed2 = _c(packed2, np.uint8)
    N, K4 = packed2.shape
    K = 4 * K4
    assert K % TILE_K == 0
    NB = -(-N // TILE_ROWS)
    P = np.zeros((NB * TILE_ROWS, K4), np.uint8)
    P[:N] = packed2
    t = P.reshape(NB, TILE_ROWS, K // TILE_K, 4, 8).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def untile2(t, N: int, K: int) -> np.ndarray:
    """Inverse of tile2 (padding rows dropped)."""
    NB = -(-N // TILE_ROWS)
    t = _c(t, np.uint8).reshape(NB, K // TILE_K, 4, TILE_ROWS, 8).transpose(0, 3, 1, 2, 4)
    return np.ascontiguousarray(t).reshape(NB * TILE_ROWS, K // 4)[:N]


# --------------------------------------------------------------------------
# any3: 3-bit codes in the GPU library's 768-byte tiles (the any4 paper's
# abstract names any3; the storage is this library's own, specified in
# include/any4.h)
# --------------------------------------------------------------------------
def tiled3_bytes(N: int, K: int) -> int:
    """Bytes of the any3 tile layout: rows padded to a multiple of 16, 3K/8 bytes each."""
    return -(-N // TILE_ROWS) * TILE_ROWS * (K // 8 * 3)


def tile3(idx) -> np.ndarray:
    """Codes [N, K] (0..7; higher bits ignored) -> the any3 tile layout (flat
    uint8).  Per lane slot (row n, 32 consecutive k): pair indices
    P_i = c[2i] | c[2i+1] << 3 for i = 0..15; byte j < 12 is P_j plus, in bits
    6-7, bits 2(j//4) and 2(j//4)+1 of P_{12 + j%4}.  Slots are ordered
    [row blocks][K/128 chunks][4 quarters of 32 k][16 rows]."""
    idx = _c(idx, np.uint8)
    N, K = idx.shape
    assert K % TILE_K == 0
    NB = -(-N // TILE_ROWS)
    codes = np.zeros((NB * TILE_ROWS, K), np.uint8)
    codes[:N] = idx & 7
    q = codes.reshape(NB, TILE_ROWS, K // TILE_K, 4, 16, 2)
    P = q[..., 0] | (q[..., 1] << 3)                      # [NB][16][Kc][4][16 pairs]
    j = np.arange(12)
    top = (P[..., 12 + j % 4] >> (2 * (j // 4))) & 3      # the top-bit parts, byte by byte
    B = (P[..., :12] | (top << 6)).astype(np.uint8)       # [NB][16][Kc][4][12]
    return np.ascontiguousarray(B.transpose(0, 2, 3, 1, 4)).reshape(-1)


def untile3(t, N: int, K: int) -> np.ndarray:
    """Inverse of tile3: the codes [N, K] (padding rows dropped)."""
    NB = -(-N // TILE_ROWS)
    B = _c(t, np.uint8).reshape(NB, K // TILE_K, 4, TILE_ROWS, 12).transpose(0, 3, 1, 2, 4)
    P = np.empty(B.shape[:-1] + (16,), np.uint8)
    P[..., :12] = B & 63
    for t4 in range(4):
        P[..., 12 + t4] = ((B[..., t4] >> 6) | ((B[..., 4 + t4] >> 6) << 2) |
                           ((B[..., 8 + t4] >> 6) << 4))
    codes = np.stack([P & 7, P >> 3], axis=-1)            # [NB][16][Kc][4][16][2]
    return np.ascontiguousarray(codes).reshape(NB * TILE_ROWS, K)[:N]


def dequant_one(alpha: int, lut_value: int, beta: int) -> int:
    return int(_load().orc_dequant_one(alpha, lut_value, beta))


def dequant(packed, lut, alpha, beta, g: int) -> np.ndarray:
    """w[n][k] = bf16(fp32(alpha*LUT[n][idx] + beta)) as bf16 bits [N, K]."""
    packed = _c(packed, np.uint8)
    lut = _c(lut, np.uint16)
    alpha = _c(alpha, np.uint16)
    beta = _c(beta, np.uint16)
    N = packed.shape[0]
    K = packed.shape[1] * 2
    assert lut.shape == (N, 16)
    assert K % g == 0 and alpha.shape == (N, K // g) and beta.shape == (N, K // g)
    w = np.empty((N, K), np.uint16)
    _load().orc_dequant(_ptr(packed), _ptr(lut), _ptr(alpha), _ptr(beta), _ptr(w), N, K, g)
    return w


def gemm(x, w, nthreads: int = 1):
    """fp64 reference y[m][n] = sum_k x[m][k]*w[n][k] and sum_k |x*w|.

    x: bf16 bits [M, K]; w: bf16 bits [N, K] (the dequantised weights).
    Returns (y_ref, absdot), both float64 [M, N]."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    M, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    _load().orc_gemm(_ptr(x), _ptr(w), _ptr(y), _ptr(a), M, N, K, nthreads)
    return y, a


def tolerance(absdot: np.ndarray) -> np.ndarray:
    """Per-element GEMM bound |y - y_ref| <= 2e-3 * sum_k |x_k w_k| + 1e-3."""
    return 2e-3 * absdot + 1e-3


# --------------------------------------------------------------------------
# quantiser
# --------------------------------------------------------------------------
def group_scale(W, g: int, levels: int = 16):
    """Min-max group scale onto [0, levels - 1] (bf16 alpha, beta)."""
    W = _c(W, np.float64)
    N, K = W.shape
    a = np.empty((N, K // g), np.uint16)
    b = np.empty((N, K // g), np.uint16)
    _load().orc_group_scale_q(_ptr(W), N, K, g, levels, _ptr(a), _ptr(b))
    return a, b


def kmeans_row(ws, wt, iters: int, init=None, trace: bool = False, levels: int = 16):
    """Weighted k-means of one row in the normalised domain (fp64), with
    `levels` table values (16; 8 or 4 for any3 / any2).

    Returns (L[levels] fp64, idx[K] u8) or (L, idx, trace[2*iters])."""
    ws = _c(ws, np.float64)
    wt = _c(wt, np.float64)
    K = ws.size
    L = _c(np.arange(levels) if init is None else init, np.float64).copy()
    assert L.shape == (levels,)
    idx = np.empty(K, np.uint8)
    tr = np.empty(max(1, 2 * iters), np.float64)
    _load().orc_kmeans_row_q(_ptr(ws), _ptr(wt), K, iters, levels, _ptr(L), _ptr(idx),
                             _ptr(tr) if trace else None)
    if trace:
        return L, idx, tr[: 2 * iters]
    return L, idx


def kmeans_quantize(W, Ex, g: int, iters: int = 10, nthreads: int | None = None,
                    bits: int = 4):
    """any4-quantise W[N, K] (fp64) with channel importance Ex[K] = E|x|
    (bits = 3 or 2: any3 / any2, 8 or 4 table values, the rest of the 16-entry
    row zero).

    Returns (idx u8 [N, K], lut bf16 bits [N, 16], alpha, beta bf16 bits [N, K/g])."""
    W = _c(W, np.float64)
    Ex = _c(Ex, np.float64)
    N, K = W.shape
    assert Ex.shape == (K,) and K % g == 0 and bits in (2, 3, 4)
    idx = np.empty((N, K), np.uint8)
    lut = np.empty((N, 16), np.uint16)
    a = np.empty((N, K // g), np.uint16)
    b = np.empty((N, K // g), np.uint16)
    rc = _load().orc_kmeans_quantize_q(_ptr(W), _ptr(Ex), N, K, g, iters, 1 << bits, _ptr(idx),
                                       _ptr(lut), _ptr(a), _ptr(b),
                                       nthreads or default_threads())
    if rc != 0:
        raise MemoryError("oracle quantiser could not allocate its row buffers")
    return idx, lut, a, b

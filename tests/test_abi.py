"""The C-ABI library loads, exports what include/any4.h declares, and rejects bad
arguments before touching the GPU (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

import gemm_any4_amd as any4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "any4.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(any[234]_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared_functions() == sorted(any4.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(any4.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s, name in any4._STATUS_NAMES.items():
        assert any4.status_string(s).startswith(name)
    assert "unknown" in any4.status_string(99)


# Every call below fails validation, so nothing reaches the HIP runtime.
A = 1 << 20          # a 16-byte aligned fake address (never dereferenced)


@pytest.mark.parametrize("M,N,K,g", [(65535 * 64 + 1, 16, 128, 128), (-1, 16, 128, 128),
                                     (1, -1, 128, 128),
                                     (1, 16, 128, 64), (1, 16, 256, 96), (1, 16, 384, 256),
                                     (1, 16, -128, 128), (1, 16, 128, 0)])
def test_gemm_shape_errors(M, N, K, g):
    assert any4.gemm_raw(A, A, A, A, A, A, M, N, K, g, stream=0) == 2


def test_gemm_null_errors():
    assert any4.gemm_raw(None, A, A, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_raw(A, None, A, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_raw(A, A, None, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_raw(A, A, A, A, A, None, 1, 16, 128, 128, stream=0) == 1


def test_gemm_alignment_errors():
    assert any4.gemm_raw(A + 2, A, A, A, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_raw(A, A + 8, A, A, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_raw(A, A, A + 4, A, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_raw(A, A, A, A + 1, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_raw(A, A, A, A, A, A + 1, 1, 16, 128, 128, stream=0) == 3


def test_empty_calls_are_no_ops():
    # nothing to do: success without touching pointers or the runtime
    assert any4.gemm_raw(None, None, None, None, None, None, 0, 16, 128, 128, stream=0) == 0
    assert any4.gemm_raw(None, None, None, None, None, None, 4, 0, 128, 128, stream=0) == 0
    assert any4.dequant_raw(None, None, None, None, None, 0, 128, 128, stream=0) == 0
    assert any4.pack_raw(None, None, 0, 128, stream=0) == 0
    assert any4.pack_raw(None, None, 8, 0, stream=0) == 0


def test_pack_and_dequant_errors():
    assert any4.pack_raw(A, A, 4, 7, stream=0) == 2
    assert any4.pack_raw(A, A, 4, 64, stream=0) == 2      # K must be a multiple of 128
    assert any4.pack_raw(None, A, 4, 128, stream=0) == 1
    assert any4.pack_raw(A + 1, A, 4, 128, stream=0) == 3
    assert any4.dequant_raw(A, A, A, A, A, 4, 256, 192, stream=0) == 2
    assert any4.dequant_raw(A, A, None, A, A, 4, 256, 128, stream=0) == 1
    assert any4.dequant_raw(A, A, A, A, A + 2, 4, 256, 128, stream=0) == 3


def test_packed_bytes():
    assert any4.packed_bytes(16, 128) == 1024
    assert any4.packed_bytes(17, 128) == 2048        # rows padded to a multiple of 16
    assert any4.packed_bytes(14336, 4096) == 14336 * 2048
    assert any4.packed_bytes(5, 100) == 0            # K not a multiple of 128
    assert any4.packed_bytes(-1, 128) == 0


def test_gemm_limits():
    # K/g at most 512 (the alpha/beta staging of one row block)
    assert any4.gemm_raw(A, A, A, A, A, A, 1, 16, 128 * 513, 128, stream=0) == 2
    # alpha and beta are read with 16-byte loads
    assert any4.gemm_raw(A, A, A, A + 2, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_raw(A, A, A, A, A + 8, A, 1, 16, 128, 128, stream=0) == 3


def test_workspace_size_is_defined_for_all_shapes():
    for M in (1, 2, 4, 8, 16):
        assert any4.workspace_size(M, 14336, 4096, 128) >= 0
    assert any4.workspace_size(17, 16, 128, 128) == 0
    # prefill (M >= 128): the layer dequantised into the workspace, N*K bf16
    assert any4.workspace_size(127, 14336, 4096, 128) == 0
    assert any4.workspace_size(128, 14336, 4096, 128) == 14336 * 4096 * 2
    assert any4.workspace_size(1024, 17, 384, 128) == 17 * 384 * 2
    assert any4.workspace_size(256, 17, 384, 96) == 0   # g not a multiple of 128


def test_prefill_workspace_errors():
    M, N, K, g = 256, 16, 128, 128
    need = N * K * 2
    assert any4.gemm_raw(A, A, A, A, A, A, M, N, K, g, A, need - 1, stream=0) == 4
    assert any4.gemm_raw(A, A, A, A, A, A, M, N, K, g, A + 8, need, stream=0) == 3
    assert any4.any2_gemm_raw(A, A, A, A, A, A, M, N, K, g, A, need - 1, stream=0) == 4


def test_gemm_int4_errors():
    # same checks as any4_gemm, without the table
    assert any4.gemm_int4_raw(A, A, A, A, A, 65535 * 64 + 1, 16, 128, 128, stream=0) == 2
    assert any4.gemm_int4_raw(A, A, A, A, A, 1, 16, 384, 256, stream=0) == 2
    assert any4.gemm_int4_raw(A, A, A, A, A, 1, 16, 128 * 513, 128, stream=0) == 2
    assert any4.gemm_int4_raw(None, A, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_int4_raw(A, None, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_int4_raw(A, A, None, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_int4_raw(A, A, A, A, None, 1, 16, 128, 128, stream=0) == 1
    assert any4.gemm_int4_raw(A + 2, A, A, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_int4_raw(A, A, A + 2, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.gemm_int4_raw(None, None, None, None, None, 0, 16, 128, 128, stream=0) == 0


def test_workspace_errors_of_every_format():
    """A shape that splits K (M = 16, 256 row blocks, K = 12288) needs a
    workspace of any4_gemm_workspace_size bytes; every GEMM entry point that
    takes one rejects a smaller one (ANY4_E_WORKSPACE) or a misaligned one
    (ANY4_E_ALIGN) before any launch."""
    M, N, K, g = 16, 16 * 256, 12288, 128
    need = any4.workspace_size(M, N, K, g)
    assert need == 4 * M * N * 4
    calls = [lambda w, b: any4.gemm_raw(A, A, A, A, A, A, M, N, K, g, w, b, stream=0),
             lambda w, b: any4.gemm_int4_raw(A, A, A, A, A, M, N, K, g, w, b, stream=0),
             lambda w, b: any4.any2_gemm_raw(A, A, A, A, A, A, M, N, K, g, w, b, stream=0),
             lambda w, b: any4.any3_gemm_raw(A, A, A, A, A, A, M, N, K, g, w, b, stream=0)]
    for call in calls:
        assert call(A, need - 1) == 4
        assert call(A + 8, need) == 3


def test_quantize_errors():
    assert any4.quantize_raw(A, A, A, A, A, A, 4, 256, 96, 10, stream=0) == 2     # K % g
    assert any4.quantize_raw(A, A, A, A, A, A, 4, 256, 128, -1, stream=0) == 2    # iters
    assert any4.quantize_raw(A, A, A, A, A, A, 4, 256, 128, 1, bits=1, stream=0) == 2
    assert any4.quantize_raw(A, A, A, A, A, A, 4, 256, 128, 1, bits=5, stream=0) == 2
    assert any4.quantize_raw(A, A, A, A, A, A, -1, 256, 128, 1, stream=0) == 2
    assert any4.quantize_raw(A, None, A, A, A, A, 4, 256, 128, 1, stream=0) == 1
    assert any4.quantize_raw(A + 2, A, A, A, A, A, 4, 256, 128, 1, stream=0) == 3
    assert any4.quantize_raw(None, None, None, None, None, None, 0, 256, 128, 1, stream=0) == 0


def test_any2_errors_and_sizes():
    assert any4.any2_packed_bytes(16, 128) == 512
    assert any4.any2_packed_bytes(17, 256) == 32 * 64
    assert any4.any2_packed_bytes(5, 100) == 0
    assert any4.any2_pack_raw(A, A, 4, 64, stream=0) == 2
    assert any4.any2_pack_raw(None, A, 4, 128, stream=0) == 1
    assert any4.any2_pack_raw(A + 1, A, 4, 128, stream=0) == 3
    assert any4.any2_dequant_raw(A, A, A, A, A, 4, 256, 192, stream=0) == 2
    assert any4.any2_dequant_raw(A, None, A, A, A, 4, 256, 128, stream=0) == 1
    assert any4.any2_gemm_raw(A, A, A, A, A, A, 1, 16, 384, 256, stream=0) == 2
    assert any4.any2_gemm_raw(A, A, None, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.any2_gemm_raw(A, A, A, A + 2, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.any2_gemm_raw(None, None, None, None, None, None, 0, 16, 128, 128, stream=0) == 0


def test_any3_errors_and_sizes():
    assert any4.any3_packed_bytes(16, 128) == 768
    assert any4.any3_packed_bytes(17, 256) == 32 * 96
    assert any4.any3_packed_bytes(5, 100) == 0
    assert any4.any3_packed_bytes(-1, 128) == 0
    assert any4.any3_pack_raw(A, A, 4, 64, stream=0) == 2
    assert any4.any3_pack_raw(None, A, 4, 128, stream=0) == 1
    assert any4.any3_pack_raw(A + 1, A, 4, 128, stream=0) == 3
    assert any4.any3_pack_raw(None, None, 0, 128, stream=0) == 0
    assert any4.any3_dequant_raw(A, A, A, A, A, 4, 256, 192, stream=0) == 2
    assert any4.any3_dequant_raw(A, None, A, A, A, 4, 256, 128, stream=0) == 1
    assert any4.any3_dequant_raw(A, A, A, A, A + 8, 4, 256, 128, stream=0) == 3
    assert any4.any3_gemm_raw(A, A, A, A, A, A, 1, 16, 384, 256, stream=0) == 2
    assert any4.any3_gemm_raw(A, A, A, A, A, A, 17 + 65535 * 64, 16, 128, 128, stream=0) == 2
    assert any4.any3_gemm_raw(A, A, None, A, A, A, 1, 16, 128, 128, stream=0) == 1
    assert any4.any3_gemm_raw(A, A, A, A + 2, A, A, 1, 16, 128, 128, stream=0) == 3
    assert any4.any3_gemm_raw(None, None, None, None, None, None, 0, 16, 128, 128, stream=0) == 0


def test_read_probe_errors():
    assert any4.read_probe_raw(A, 1000, A, stream=0) == 2
    assert any4.read_probe_raw(None, 1024, A, stream=0) == 1
    assert any4.read_probe_raw(A + 8, 1024, A, stream=0) == 3
    assert any4.read_probe_raw(None, 0, None, stream=0) == 0

"""The C ABI used from plain C: tests/c/abi_demo (built by
__graft_entry__.build(), no Python or torch in the process) packs,
dequantises and multiplies a layer through libany4.so; its outputs are
checked here against the CPU oracle (dequant bit-exact, gemm within the
bound)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_demo")


@pytest.mark.parametrize("M,N,K,g", [(1, 70, 512, 128), (16, 16 * 40 + 3, 4096, 256),
                                     (5, 33, 8192, 1024)])
def test_c_caller(tmp_path, M, N, K, g):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with __graft_entry__.build()")
    inp = workloads.generic(M * 5 + N + K, M, N, K, g)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([M, N, K, g], np.int64).tobytes())
        for a, dt in ((inp.idx, np.uint8), (inp.lut, np.uint16), (inp.alpha, np.uint16),
                      (inp.beta, np.uint16), (inp.x[:M], np.uint16)):
            f.write(np.ascontiguousarray(a, dtype=dt).tobytes())
    print(f"abi_demo M={M} N={N} K={K} g={g}", flush=True)
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr + r.stdout
    out = np.fromfile(dst, dtype=np.uint16)
    w, y = out[:N * K].reshape(N, K), out[N * K:].reshape(M, N)
    w_ref = oracle.dequant(oracle.pack(inp.idx), inp.lut, inp.alpha, inp.beta, g)
    assert np.array_equal(w, w_ref)
    y_ref, ad = oracle.gemm(inp.x[:M], w_ref)
    yf = workloads.bf16_bits_to_f64(y)
    assert np.all(np.abs(yf - y_ref) <= oracle.tolerance(ad))

"""Build tests/c/abi_demo (a plain C caller of libany4.so, test
infrastructure) with gcc against the HIP runtime and the in-tree library."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_demo.c")
EXE = os.path.join(HERE, "abi_demo")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    libdir = os.path.join(ROOT, "gemm_any4_amd")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-o", EXE, SRC, "-L", libdir, "-lany4", "-Wl,-rpath,$ORIGIN/../../gemm_any4_amd",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    build(verbose=True)

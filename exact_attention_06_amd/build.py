"""Ahead-of-time build of libfa.so (the HIP library behind include/fa_fwd.h) for gfx950.

Run as `python -m exact_attention_06_amd.build`. The shared library is written next to
this file, inside the package, so it travels with the source tree.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa_fwd.hip")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # keep packed fp32 VALU ops (v_pk_{add,mul,fma}_f32) out of every code object. The host
    # pass warns that it does not know this feature (it is an amdgcn feature); the device
    # pass applies it: the gfx950 code object holds none of these instructions with it and
    # about 14,600 without it (tests/test_build.py disassembles the built library).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs (the online-softmax rescale touches them with VALU ops)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-I", os.path.join(PKG, "csrc"),
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Host-side AddressSanitizer build (the device code is the same gfx950 code object, built
# without sanitizers): the C ABI's argument checks run under ASan in the contract tests.
ASAN_LIB = os.path.join(ROOT, "_build", "libfa_asan_host.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that an ASan-built library needs preloaded."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    import glob

    hits = glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang", "*", "lib",
                                  "linux", "libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return hits[0]


def build_asan_host(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(ASAN_LIB), exist_ok=True)
    return build(verbose, extra=ASAN_FLAGS, out=ASAN_LIB)


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {SRC}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

"""The built library's gfx950 code object (our own build, disassembled on the CPU)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "exact_attention_06_amd", "libfa.so")
LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")


def _disassemble(tmp_path, lib=LIB):
    if not os.path.exists(lib):
        pytest.skip(f"{os.path.basename(lib)} is not built")
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools not found")
    objcopy, bundler, objdump = tools
    fat, co = str(tmp_path / "fatbin.bin"), str(tmp_path / "gfx950.o")
    shutil.copy(lib, tmp_path / "lib.so")
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", str(tmp_path / "lib.so"),
                    str(tmp_path / "lib2.so")], check=True)
    subprocess.run([bundler, "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={fat}",
                    f"--output={co}", "--unbundle"], check=True)
    return subprocess.run([objdump, "-d", "--mcpu=gfx950", co], check=True, capture_output=True,
                          text=True).stdout


def test_code_object_is_gfx950_and_has_no_packed_fp32(tmp_path):
    dis = _disassemble(tmp_path)
    assert "v_mfma_f32_32x32x16_bf16" in dis  # the forward kernels' matrix-core instruction
    for op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"):
        assert op not in dis, f"{op} in the code object: the -packed-fp32-ops feature was not applied"


def test_microbenchmark_builds_with_the_library_flags(tmp_path):
    # the measurement kernel (not part of libfa.so) compiles for gfx950 with the same flags,
    # exports its entry points, and carries no packed fp32 VALU ops either
    import ctypes

    from exact_attention_06_amd import microbench

    lib = microbench.build()
    so = ctypes.CDLL(lib)
    assert so.ub_mfmas_per_iter(0) == 2 and so.ub_mfmas_per_iter(4) == 4
    dis = _disassemble(tmp_path, lib)
    assert "ds_read_b64_tr_b16" in dis and "v_mfma_f32_32x32x16_bf16" in dis
    for op in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"):
        assert op not in dis

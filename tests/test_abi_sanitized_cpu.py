"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/abi_host_check.c drives every validation path, the size queries, the
timing calls and (without a GPU) a well-formed call up to its first HIP
call.  Here the library's host source is rebuilt with both sanitizers on the
host side only (the kernels' objects are the ordinary ones, their device
code untouched), linked with the host test program, and run: any heap, stack or
undefined-behaviour error in the host runtime fails the test.  CPU only.
"""

import glob
import os
import subprocess

import pytest

from sparse_weight_memory_amd import build as B

ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")


def _asan_runtime_dir():
    hits = glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                  "libclang_rt.asan-x86_64.so"))
    return os.path.dirname(hits[0]) if hits else None


def test_abi_host_code_is_clean_under_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("checks the no-GPU paths")
    rt = _asan_runtime_dir()
    if not (os.path.exists(CLANG) and rt):
        pytest.skip("ROCm clang with the sanitizer runtimes is not available")
    objs = sorted(glob.glob(os.path.join(B.BUILD, "k*.o")))
    if len(objs) < 6:
        B.build()
        objs = sorted(glob.glob(os.path.join(B.BUILD, "k*.o")))
    api = tmp_path / "fwpkm_api_san.o"
    lib = tmp_path / "libfwpkm_san.so"
    exe = tmp_path / "abi_host_check"
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
    run = lambda cmd: subprocess.run(cmd, capture_output=True, text=True)
    r = run([B.hipcc(), "-x", "hip", *B.common_flags(debug=True), *host_san, "-c",
             os.path.join(B.CSRC, "fwpkm_api.cpp"), "-o", str(api)])
    assert r.returncode == 0, r.stderr
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libsan"]
    r = run([CLANG + "++", "-shared", "-fPIC", *san, str(api), *objs, "-L", os.path.join(ROCM, "lib"),
             "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", str(lib)])
    assert r.returncode == 0, r.stderr
    r = run([CLANG, "-g", *san, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
             "-I", B.INCLUDE, os.path.join(os.path.dirname(__file__), "abi_host_check.c"), str(lib),
             "-Wl,-rpath," + str(tmp_path), "-lm", "-o", str(exe)])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_LIBRARY_PATH=rt + ":" + os.environ.get("LD_LIBRARY_PATH", ""),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi host checks ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr

"""The C ABI's host code (argument validation, workspace sizing, error text in
fa_api.cpp) built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer, then run through every case of test_abi_cpu.py.

The kernel launchers are replaced by stand-ins that abort
(tests/abi_host/stub_launchers.cpp): those cases must be rejected before any
launch.  UBSan is built non-recovering, so undefined behaviour fails the run;
ASan reports any out-of-bounds or use-after-free access.  A planted
out-of-bounds read, built and loaded the same way, shows that the sanitizer is
live in this setup.  CPU only.
"""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_forward_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

if torch.cuda.device_count() > 0:
    pytest.skip("runs the fake-pointer validation tests; CPU only", allow_module_level=True)
if not os.path.exists(CLANG):
    pytest.skip("ROCm's clang++ is not installed", allow_module_level=True)


def asan_runtime() -> str:
    return subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True, check=True).stdout.strip()


def sanitized_env(lib: str) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_runtime(), FA_ABI_TEST_LIB=lib,
               # the interpreter's own allocations are not this library's leaks
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return env


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("abi_asan") / "libfa_abi_sanitized.so")
    cmd = [CLANG, *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(ROOT, "tests", "abi_host",
                                                          "stub_launchers.cpp"),
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def test_validation_suite_is_clean_under_asan_and_ubsan(sanitized_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests",
                        "test_abi_cpu.py"), "-q", "-p", "no:cacheprovider"],
                       capture_output=True, text=True, cwd=ROOT, env=sanitized_env(sanitized_lib),
                       timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out and " failed" not in out


def test_the_sanitizer_is_live(tmp_path):
    src = tmp_path / "oob.cpp"
    src.write_text('#include <cstdlib>\nextern "C" int oob(int i) {\n'
                   '  int* p = (int*)std::malloc(4 * sizeof(int));\n'
                   '  int v = p[i];\n  std::free(p);\n  return v;\n}\n')
    lib = str(tmp_path / "liboob.so")
    subprocess.run([CLANG, *FLAGS, str(src), "-o", lib], check=True, capture_output=True)
    code = f"import ctypes; print(ctypes.CDLL({lib!r}).oob(4))"
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       env=sanitized_env(lib), timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

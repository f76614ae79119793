"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer: a C driver (tests/host/abi_host_check.c) calls
every host-only path of the C ABI against a sanitized build of libtra.  No
GPU is needed; the device code is built as usual and never launched."""
import os
import subprocess

import pytest

from sparse_self_attention_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_host_library_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "libtra_san.so"
    B.build_sanitized(str(lib), verbose=False)
    exe = tmp_path / "abi_host_check"
    # The driver is host C: built with clang (no device code) and linked with
    # the sanitizer runtimes the library's host code needs.
    cmd = [CLANG, "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host", "abi_host_check.c"),
           "-o", str(exe), str(lib), f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib",
           "-L/opt/rocm/lib", "-lamdhip64", "-lstdc++"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    supp = tmp_path / "lsan.supp"
    # Leaks inside the HIP runtime's own initialisation are not the library's.
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:librocprofiler\n")
    env = dict(os.environ)
    env.pop("TRA_FAULT", None)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=23"
    env["LSAN_OPTIONS"] = f"suppressions={supp}"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "abi host checks passed" in out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out

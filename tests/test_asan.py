"""The library's host code under AddressSanitizer, on the CPU: the HIP sources are built with the host
half instrumented (the device code is unchanged), and tests/abi_asan_driver.c calls every entry point
down its argument-checking paths (errors, zero-size work, the operand check without a device).  Any
out-of-bounds access, use after free or similar in the host validation ends the driver with a
sanitizer report."""
import os
import shutil
import subprocess
import tempfile

import pytest

from paged_kv_cache_msa_amd import _build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_validation_under_address_sanitizer():
    inc = os.path.join(ROOT, "include")
    tmp = tempfile.mkdtemp(prefix="msa_asan_")
    try:
        lib = os.path.join(tmp, "libmsa_asan.so")
        # Host half instrumented only: every sanitizer flag goes to the host compilation.
        flags = [f for f in _build.HIP_FLAGS if f not in ("-O3",)] + [
            "-O1", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
        r = subprocess.run([HIPCC, *flags, "-I", inc, *_build.SRCS, "-o", lib], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in nm, "host code was not instrumented"
        exe = os.path.join(tmp, "abi_asan_driver")
        clang = os.path.join(os.path.dirname(HIPCC), "..", "lib", "llvm", "bin", "clang")
        clang = clang if os.path.exists(clang) else shutil.which("clang") or "clang"
        r = subprocess.run([clang, "-O1", "-g", "-fsanitize=address", "-I", inc,
                            os.path.join(HERE, "abi_asan_driver.c"), lib, "-Wl,-rpath," + tmp,
                            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", HIP_VISIBLE_DEVICES="")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = r.stdout + r.stderr
        assert "AddressSanitizer" not in out, out
        assert r.returncode == 0, out
        assert "all host checks passed under the sanitizer" in r.stdout, out
    finally:
        shutil.rmtree(tmp, ignore_errors=True)

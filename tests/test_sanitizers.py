"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two host-only builds, each run as its own process with every sanitizer
finding fatal:
  * the fp64 oracle (oracle/oracle.c) with a driver that runs the forward and
    backward on small and degenerate shapes (tests/sanitize/oracle_driver.c);
  * libfa's entry points (io_aware_exact_amd/csrc/api.cpp, argument checks
    and parameter blocks) with the kernel launches replaced by counting stubs
    generated from the launch declarations in fa_internal.h, driven with
    random extreme sizes, strides and pointers and with valid argument sets
    (tests/sanitize/api_fuzz.cpp).
No GPU code is built: the device kernels are not part of either program.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout + r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c99", "-Wall", *SAN, os.path.join(HERE, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe], check=True)
    out = run(exe)
    assert "0 failures" in out


def launch_stubs():
    """Counting stubs for every launch function fa_internal.h declares."""
    text = open(os.path.join(ROOT, "io_aware_exact_amd", "csrc", "fa_internal.h")).read()
    decls = re.findall(r"^hipError_t\s+(launch_\w+|noalloc_scratch)\s*\(([^;]*?)\)\s*;", text,
                       flags=re.M | re.S)
    assert len(decls) >= 10
    body = ['#include "fa_internal.h"', "long g_launches = 0;"]
    for name, params in decls:
        if name == "noalloc_scratch":   # a fixed stand-in address, never dereferenced
            body.append(f"hipError_t {name}({params}) {{ *ptr = (void*)0x200000000000ull; return hipSuccess; }}")
        else:
            body.append(f"hipError_t {name}({params}) {{ ++g_launches; return hipSuccess; }}")
    # the FA_DEBUG check's runtime calls: the harness passes host arrays there
    body += ["#include <string.h>",
             'extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }',
             'extern "C" hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) '
             '{ memcpy(dst, src, n); return hipSuccess; }']
    return "\n".join(body) + "\n"


def test_api_host_checks_under_sanitizers(tmp_path):
    if not os.path.exists(CLANG):
        pytest.skip("clang++ not available")
    stubs = tmp_path / "stubs.cpp"
    stubs.write_text(launch_stubs())
    exe = str(tmp_path / "api_san")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "io_aware_exact_amd", "csrc"),
           "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    subprocess.run([CLANG, "-x", "c++", "-std=c++17", *SAN, *inc,
                    os.path.join(ROOT, "io_aware_exact_amd", "csrc", "api.cpp"), str(stubs),
                    os.path.join(HERE, "api_fuzz.cpp"), "-o", exe], check=True)
    out = run(exe)
    assert "api fuzz:" in out

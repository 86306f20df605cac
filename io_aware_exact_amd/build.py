"""Builds libfa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and
libfa_probe.so, a measurement probe the bench uses (not part of the path)."""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfa.so")
PROBE_LIB = os.path.join(HERE, "libfa_probe.so")
PROBE_SOURCES = ["probe_dq_accum.hip", "probe_hbm_read.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "fwd.hip", "fwd_pp.hip", "fwd_f32.hip", "bwd.hip", "decode.hip", "fp8.hip",
           "kvcache.hip", "merge.hip", "noalloc.hip", "bwd_fp8.hip"]

# Packed fp32 VALU forms are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    return obj


def build(verbose=False):
    """Compile every source for gfx950 and link libfa.so (always rebuilds)."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES + PROBE_SOURCES))
    for lib, o in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + o
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

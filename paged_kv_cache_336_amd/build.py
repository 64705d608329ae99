"""Build libpagedkv.so (HIP for gfx950) in-tree with hipcc.

    python -m paged_kv_cache_336_amd.build [--verbose]

Every HIP source under csrc/ is compiled into one shared library next to this
file.  Packed-fp32 instruction selection is disabled for the device code
(``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpagedkv.so")
SOURCES = ["pagedkv_api.hip", "attn_decode.hip", "attn_multi.hip",
           "cache_ops.hip", "block_manager.cpp"]
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libpagedkv.so")
    if verbose and res.stderr.strip():
        sys.stderr.write(res.stderr)


def build_library(verbose=False, extra_flags=()):
    """Compile every source to an object (in parallel), then link."""
    from concurrent.futures import ThreadPoolExecutor
    tmp = LIB + ".tmp"
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Wall", "-Wno-unused-result",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(HERE, "..", "include"), *extra_flags]
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o")
            for s in SOURCES]
    jobs = [[hipcc(), *flags, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs,
          "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="--verbose" in sys.argv))

"""Build the HIP library (gfx950) in-tree: dropless_moe_dispatch_amd/lib/libmoe_dispatch.so.

Every translation unit is compiled with hipcc for gfx950 only.  Packed fp32
instructions are disabled for the device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "lib")
LIB = os.path.join(OUT_DIR, "libmoe_dispatch.so")
SOURCES = ["api.hip", "route.hip", "index.hip", "index_dense.hip", "experts.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def compile_flags(debug: bool = False):
    return ["-std=c++17", "-fPIC", "-O3" if not debug else "-O1", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", "-ffp-contract=fast"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(os.path.join(OUT_DIR, "obj"), exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OUT_DIR, "obj", src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len([p for p in procs if p[1].poll() is None]) >= jobs:
            procs[-jobs][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out.decode(errors="replace")))
        elif verbose and out:
            print(out.decode(errors="replace"))
    if failed:
        for src, msg in failed:
            sys.stderr.write(f"--- {src} ---\n{msg}\n")
        raise RuntimeError("HIP compilation failed: " + ", ".join(s for s, _ in failed))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_pack_check(verbose)
    return LIB


PACK_CHECK_SRC = os.path.join(os.path.dirname(HERE), "tests", "bf16_pack_check.hip")
PACK_CHECK = os.path.join(OUT_DIR, "bf16_pack_check")


def build_pack_check(verbose: bool = False) -> str:
    """The GPU test program that checks the library's bf16 packing rounds to
    nearest even (tests/test_gpu_bf16_pack.py runs it)."""
    cmd = [hipcc(), *[f for f in compile_flags() if f != "-fPIC"], PACK_CHECK_SRC, "-o", PACK_CHECK + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(PACK_CHECK + ".tmp", PACK_CHECK)
    return PACK_CHECK


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

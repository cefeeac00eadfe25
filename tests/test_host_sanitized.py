"""The C ABI's host validation and workspace carving under AddressSanitizer
and UndefinedBehaviorSanitizer (no GPU): tests/abi_host_check.cpp is linked
with the ABI translation unit (csrc/api.hip) and stand-in kernel launchers,
both built with the sanitizers on their host code, and run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_check")


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.timeout(600)
def test_abi_host_checks_under_sanitizers():
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_host_check")
    # sanitizers on host code only: each -fsanitize= right after -Xarch_host
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    srcs = [os.path.join(ROOT, "tests", "abi_host_check.cpp"),
            os.path.join(ROOT, "dropless_moe_dispatch_amd", "csrc", "api.hip")]
    objs = []
    for src in srcs:
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", *san, *lang, "-c", src, "-o", obj]
        p = subprocess.run(cmd, capture_output=True, text=True)
        assert p.returncode == 0, p.stderr[-4000:]
        objs.append(obj)
    p = subprocess.run([cc, "--offload-arch=gfx950", *san, *objs, "-o", exe], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=500)
    assert p.returncode == 0 and "abi host checks ok" in p.stdout, (p.returncode, p.stdout[-2000:],
                                                                    p.stderr[-6000:])

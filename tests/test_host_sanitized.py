"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

`tests/host_checks/host_checks.cpp` drives every entry point along the paths
that its argument checks and size arithmetic answer alone (invalid and
extreme sizes, null pointers, small workspaces, the no-alloc scratch limit,
an update that appends nothing, the timing window): none of them reaches the
GPU, so the test runs on the CPU.  The library's sources are compiled as for
the shipped library, with the sanitizers on the host side only; the build
is cached under tests/host_checks/_build and redone when a source changes.
"""

import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lsh_sampled_sparse_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_checks")
OUT = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["lsh_api.hip", "build_kernels.hip", "decode_kernels.hip", "attend_bf16.hip"]
# sanitizers on the host side only: each -fsanitize= follows -Xarch_host
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _digest():
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    files += [os.path.join(ROOT, "include", "lsh_attn.h"), os.path.join(HERE, "host_checks.cpp")]
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(FLAGS + SAN).encode())
    return h.hexdigest()[:16]


def _build():
    exe = os.path.join(OUT, "host_checks")
    stamp = os.path.join(OUT, "digest")
    dig = _digest()
    if os.path.exists(exe) and os.path.exists(stamp) and open(stamp).read() == dig:
        return exe
    os.makedirs(OUT, exist_ok=True)

    def cc(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        lang = ["-x", "c++"] if src.endswith(".cpp") else []
        r = subprocess.run([HIPCC, *FLAGS, *SAN, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
        return obj

    srcs = [os.path.join(CSRC, f) for f in SOURCES] + [os.path.join(HERE, "host_checks.cpp")]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(cc, srcs))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, "-o", exe, *objs], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    with open(stamp, "w") as fh:
        fh.write(dig)
    return exe


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_code_under_sanitizers():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr[-4000:]
    assert "host checks passed" in r.stdout

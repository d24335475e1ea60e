"""Ahead-of-time build of liblsh_attn.so for gfx950 with hipcc.

Usage: python -m lsh_sampled_sparse_amd.build   (or build() from Python)
The library is written next to this file so that it travels with the tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblsh_attn.so")
SOURCES = ["lsh_api.hip", "build_kernels.hip", "decode_kernels.hip", "attend_bf16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# per-source extra flags: the projection reads every MFMA result with VALU
# instructions, so its accumulators are kept in VGPRs (no AGPR copies)
EXTRA = {"build_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


# the checked build (kernels test their index arithmetic, see LSH_CHECKED in
# csrc/lsh_kernels.h): a debugging library beside the shipped one
CHECKED_LIB = os.path.join(HERE, "liblsh_attn_checked.so")
CHECKED_OBJ = os.path.join(HERE, "_build_checked")


def _compile(src: str, checked: bool = False) -> str:
    obj = os.path.join(CHECKED_OBJ if checked else OBJ, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *(["-DLSH_CHECKED"] if checked else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, lib)
    if verbose:
        print(f"built {lib}")


def build(verbose: bool = True, checked: bool = True) -> str:
    """Compile every HIP source and link the shared library (and, with
    `checked`, the checked debugging library); returns the library's path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = [(src, False) for src in SOURCES]
    if checked:
        os.makedirs(CHECKED_OBJ, exist_ok=True)
        jobs += [(src, True) for src in SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    if checked:
        _link(objs[len(SOURCES):], CHECKED_LIB, verbose)
    build_c_consumer(verbose)
    return LIB


ROOT = os.path.dirname(HERE)
C_CONSUMER_SRC = os.path.join(ROOT, "tests", "c_consumer", "abi_smoke.c")
C_CONSUMER = os.path.join(ROOT, "tests", "c_consumer", "abi_smoke")


def build_c_consumer(verbose: bool = True) -> str | None:
    """The plain-C test program that drives the library through its header
    alone (gcc, HIP runtime API for device memory); None when absent."""
    if not os.path.exists(C_CONSUMER_SRC):
        return None
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm}/include", f"-I{os.path.join(ROOT, 'include')}", C_CONSUMER_SRC, f"-L{HERE}", "-llsh_attn",
           f"-L{rocm}/lib", "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../lsh_sampled_sparse_amd",
           f"-Wl,-rpath,{rocm}/lib", "-o", C_CONSUMER]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"C consumer build failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {C_CONSUMER}")
    return C_CONSUMER


if __name__ == "__main__":
    build()

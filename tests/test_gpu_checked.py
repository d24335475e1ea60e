"""The checked library (built with LSH_CHECKED: the kernels test their index
arithmetic against the bounds the arguments promise and OR a bit into a
device word on a violation) over parity cases that cover the build, the
growing-cache update, the plain, hybrid and cached decodes, fp32 and bf16,
K = 15 at stride 256, ragged lengths, a per-head W and more count workgroups
than one round: every case must match the oracle and leave the word zero.
One more case hands the decode tables that hold more keys than it is told:
its accesses stay clamped into the chunk, and the word must report it.

The cases run in a child process that loads liblsh_attn_checked.so in place
of the shipped library (a process loads one of them)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

CHILD = r"""
import ctypes, os, sys
sys.path[:0] = [{root!r}, {tests!r}]
import torch
import lsh_sampled_sparse_amd as lsh
lsh.LIB_PATH = os.path.join(os.path.dirname(lsh.__file__), "liblsh_attn_checked.so")
L = lsh.lib()
L.lsh_check_set.argtypes = [ctypes.c_void_p]
L.lsh_check_set.restype = None
word = torch.zeros(1, dtype=torch.int32, device="cuda:0")
L.lsh_check_set(ctypes.c_void_p(word.data_ptr()))
import workloads
import test_gpu_parity as P
import test_gpu_cache as C

def say(*a):
    print(*a, flush=True)

cases = [
    ("small ragged-gqa3", lambda: P.check_case(P.SMALL[1], workloads.generate(P.SMALL[1]))),
    ("small fp32-multi", lambda: P.check_case(P.SMALL[4], workloads.generate(P.SMALL[4]))),
    ("K15 stride 256", lambda: P.check_case(P.SMALL[9], workloads.generate(P.SMALL[9]), stride=256)),
    ("hybrid across chunks", lambda: P.check_case(P.SMALL[1], workloads.generate(P.SMALL[1]), stride=1024,
                                                  n_sink=16, n_window=1500)),
    ("many count rounds", lambda: P.check_case(P.MANY_ROUNDS[0][0], workloads.generate(P.MANY_ROUNDS[0][0]),
                                               stride=256, n_sink=4, n_window=300)),
]
for name, run in cases:
    say("case checked", name)
    run()
    torch.cuda.synchronize()
    say("  violation bits", int(word.item()))
    assert int(word.item()) == 0, (name, int(word.item()))
cfg = workloads.Config("checked-ragged", B=3, Hq=8, Hkv=2, N=5000, d=128, K=8, L=20, T=2, dtype="bf16",
                       planted=4, a=0.8, offset="per_head", seed=36)
say("case checked ragged growth with per-head W")
C.grow(cfg, [[1000, 0, 300], [1001, 0, 301], [3000, 2500, 1025], [3001, 2756, 1025], [5000, 5000, 4097]],
       stride=1024, n_sink=2, n_window=100,
       W_heads=workloads.per_head_projections(cfg, seed=1036))
torch.cuda.synchronize()
say("  violation bits", int(word.item()))
assert int(word.item()) == 0
# tables that hold more keys than the decode is told (3000 built, 2500
# attended): the count clamps every probed bucket into the chunk's 2500 - 2048
# keys and masks entries into the chunk, so every access stays in bounds, and
# the checked build reports the inconsistency (segment and entry bits)
say("case checked tables longer than the decode")
cfg = workloads.Config("checked-short", B=1, Hq=2, Hkv=1, N=3000, d=128, K=6, L=8, T=2, dtype="bf16",
                       planted=2, a=0.8, offset="none", seed=37)
data = workloads.generate(cfg)
dev = torch.device("cuda:0")
keys, vals, W = (data[k].to(dev) for k in ("keys", "values", "W"))
q = data["q"][0].to(dev).contiguous()
tb = lsh.build_tables(keys, W, cfg.K, cfg.L, stride=1024)
torch.cuda.synchronize()
assert int(word.item()) == 0
out = torch.empty(1, 2, 128, device=dev)
lsh.lsh_decode_attention_cached(q, keys, vals, W, tb["indices"], tb["offsets"], 2500, cfg.K, cfg.L, cfg.T,
                                tb["stride"], cfg.scale, 0, 0, out)
torch.cuda.synchronize()
bits = int(word.item())
say("  violation bits", bits)
assert bits & (2 | 4), bits      # segment bounds past the chunk, entries past its length
L.lsh_check_set(None)
print("checked cases passed", flush=True)
"""


def test_checked_build_finds_no_violation():
    lib = os.path.join(ROOT, "lsh_sampled_sparse_amd", "liblsh_attn_checked.so")
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is missing: build it with python -m lsh_sampled_sparse_amd.build")
    print("case checked library", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", CHILD.format(root=ROOT, tests=TESTS)], capture_output=True,
                       text=True, timeout=600)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "checked cases passed" in r.stdout

"""LSH_DEBUG_LAUNCH: with the variable set, every launch prints its kernel,
grid, block and LDS bytes to stderr; without it, nothing is printed.  Each
case runs one small build and decode in a child process (the variable is
read once, at the library's first launch)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, torch
sys.path.insert(0, {root!r})
import lsh_sampled_sparse_amd as lsh
dev = torch.device("cuda:0")
g = torch.Generator(device="cpu").manual_seed(5)
keys = torch.randn(1, 1, 3000, 128, generator=g).to(torch.bfloat16).to(dev)
vals = torch.randn(1, 1, 3000, 128, generator=g).to(torch.bfloat16).to(dev)
W = torch.randn(128, 8 * 12, generator=g).to(torch.bfloat16).to(dev)
q = torch.randn(1, 2, 128, generator=g).to(torch.bfloat16).to(dev)
tb = lsh.build_tables(keys, W, 8, 12)
r = lsh.decode_attention(q, keys, vals, W, tb, 8, 12, 2)
torch.cuda.synchronize()
assert torch.isfinite(r["out"]).all()
print("child done", flush=True)
"""


def run_child(flag):
    env = dict(os.environ)
    env.pop("LSH_DEBUG_LAUNCH", None)
    if flag is not None:
        env["LSH_DEBUG_LAUNCH"] = flag
    print(f"case debug launch flag={flag!r}", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True, text=True,
                       env=env, timeout=180)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "child done" in r.stdout
    return [ln for ln in r.stderr.splitlines() if ln.startswith("[lsh] launch")]


def test_debug_launch_prints_every_launch():
    lines = run_child("1")
    names = [ln.split()[2] for ln in lines]
    # the build (W transpose, projection, sort) and the decode (query hash, decode)
    assert names == ["transpose_w", "project_codes", "chunk_sort", "qhash", "decode"], lines
    assert all("grid (" in ln and "block (" in ln for ln in lines)


@pytest.mark.parametrize("flag", [None, "0"])
def test_debug_launch_off(flag):
    assert run_child(flag) == []

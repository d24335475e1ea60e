"""The C ABI loads and validates arguments on the host (no GPU work).

Every call here returns before anything is enqueued: invalid arguments,
unsupported shapes and short workspaces are rejected by the host checks.
"""

import ctypes
import os
import re

import pytest

import lsh_sampled_sparse_amd as lsh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsh_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(lsh.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lsh_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "lsh_build_tables" in names and "lsh_decode_attention" in names
    L = ctypes.CDLL(lsh.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert sorted(lsh.EXPORTS) == names


def test_library_resolves_its_own_symbols():
    """Every kernel the library launches has its host-side stub in the
    library: no symbol of its own namespace is left undefined (a kernel
    template whose host pass fails substitution quietly loses its stub, and
    a lazily bound library would only fail at that kernel's launch)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", "-C", lsh.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    own = [ln for ln in out.splitlines() if "lsh::" in ln]
    assert not own, "undefined library symbols:\n" + "\n".join(own[:10])


def test_status_strings():
    for s in range(5):
        assert lsh.lsh_status_string(s).startswith("LSH_")
    assert lsh.lsh_status_string(99) == "unknown lsh_status"


def test_num_chunks_and_default_stride():
    assert lsh.lsh_num_chunks(131072, 16384) == 8
    assert lsh.lsh_num_chunks(5000, 256) == 20
    assert lsh.lsh_num_chunks(0, 256) == 0
    for N, K in [(131072, 10), (16384, 10), (32768, 9), (32768, 10), (4096, 8), (1, 0), (10**6, 15)]:
        s = lsh.lsh_default_stride(N, K)
        assert 256 <= s <= 8192 and (s & (s - 1)) == 0
        assert s >= min(N, 8192)
    assert lsh.lsh_default_stride(300, 8) == 512
    assert lsh.lsh_default_stride(0, 3) == 0 and lsh.lsh_default_stride(10, 16) == 0


def test_workspace_queries():
    good = lsh.lsh_build_workspace_size(1, 4, 131072, 128, 10, 150, 8192, lsh.LSH_BF16)
    # at least the uint16 codes of every (unit, table, key)
    assert good >= 4 * 150 * 131072 * 2
    assert lsh.lsh_build_workspace_size(1, 4, 131072, 64, 10, 150, 8192, 1) == 0      # d != 128
    assert lsh.lsh_build_workspace_size(1, 4, 131072, 128, 16, 150, 8192, 1) == 0     # K > 15
    assert lsh.lsh_build_workspace_size(1, 4, 131072, 128, 10, 150, 1000, 1) == 0     # stride not 2^k
    assert lsh.lsh_build_workspace_size(1, 4, 131072, 128, 10, 150, 16384, 1) == 0    # stride > 8192
    dec = lsh.lsh_decode_workspace_size(1, 32, 4, 131072, 128, 10, 150, 8192)
    assert dec >= 32 * 131072 // 8            # the selection bitmask
    assert lsh.lsh_decode_workspace_size(1, 30, 4, 131072, 128, 10, 150, 8192) == 0   # Hq % Hkv
    assert lsh.lsh_decode_workspace_size(1, 68, 4, 131072, 128, 10, 150, 8192) == 0   # G > 16


def _build(**kw):
    a = dict(keys=1, W=1, B=1, Hkv=1, N=4096, d=128, K=8, L=32, stride=4096, dtype=1,
             offsets=1, indices=1, codes=None, ws=1, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lsh.lib().lsh_build_tables(p(a["keys"]), p(a["W"]), a["B"], a["Hkv"], a["N"], a["d"], a["K"],
                                      a["L"], a["stride"], a["dtype"], p(a["offsets"]), p(a["indices"]),
                                      p(a["codes"]), p(a["ws"]), a["ws_bytes"], a["stream"])


def _decode(**kw):
    a = dict(q=1, keys=1, values=1, W=1, indices=1, offsets=1, B=1, Hq=4, Hkv=1, N=4096, d=128, K=8,
             L=32, T=2, stride=4096, scale=0.088, dtype=1, out=1, ws=1, ws_bytes=1 << 40)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lsh.lib().lsh_decode_attention(
        p(a["q"]), p(a["keys"]), p(a["values"]), p(a["W"]), p(a["indices"]), p(a["offsets"]),
        a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["K"], a["L"], a["T"], a["stride"],
        ctypes.c_float(a["scale"]), a["dtype"], p(a["out"]), None, None, None, None, p(a["ws"]),
        a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(keys=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(W=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(offsets=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(indices=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(ws=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(B=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(N=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(K=-1), lsh.LSH_ERR_INVALID_ARG),
    (dict(K=16), lsh.LSH_ERR_INVALID_ARG),
    (dict(L=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(L=256), lsh.LSH_ERR_INVALID_ARG),
    (dict(dtype=7), lsh.LSH_ERR_INVALID_ARG),
    (dict(stride=3000), lsh.LSH_ERR_INVALID_ARG),
    (dict(d=64), lsh.LSH_ERR_UNSUPPORTED),
    (dict(stride=128), lsh.LSH_ERR_UNSUPPORTED),
    (dict(stride=16384), lsh.LSH_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), lsh.LSH_ERR_WORKSPACE),
    (dict(N=(1 << 30) + 1), lsh.LSH_ERR_UNSUPPORTED),
])
def test_build_rejects(kw, status):
    assert _build(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(values=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(out=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(offsets=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), lsh.LSH_ERR_INVALID_ARG),
    (dict(T=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(T=33), lsh.LSH_ERR_INVALID_ARG),
    (dict(scale=float("nan")), lsh.LSH_ERR_INVALID_ARG),
    (dict(scale=float("inf")), lsh.LSH_ERR_INVALID_ARG),
    (dict(Hq=17, Hkv=1), lsh.LSH_ERR_UNSUPPORTED),
    (dict(d=96), lsh.LSH_ERR_UNSUPPORTED),
    (dict(ws_bytes=100), lsh.LSH_ERR_WORKSPACE),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


def _hybrid(n_sink, n_window, **kw):
    a = dict(q=1, keys=1, values=1, W=1, indices=1, offsets=1, B=1, Hq=4, Hkv=1, N=4096, d=128, K=8,
             L=32, T=2, stride=4096, scale=0.088, dtype=1, out=1, ws=1, ws_bytes=1 << 40)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lsh.lib().lsh_decode_attention_hybrid(
        p(a["q"]), p(a["keys"]), p(a["values"]), p(a["W"]), p(a["indices"]), p(a["offsets"]),
        a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["K"], a["L"], a["T"], a["stride"],
        ctypes.c_float(a["scale"]), a["dtype"], n_sink, n_window, p(a["out"]), None, None, None, None,
        p(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("n_sink,n_window,kw,status", [
    (-1, 0, {}, lsh.LSH_ERR_INVALID_ARG),
    (0, -5, {}, lsh.LSH_ERR_INVALID_ARG),
    (4, 64, dict(q=None), lsh.LSH_ERR_INVALID_ARG),
    (4, 64, dict(T=0), lsh.LSH_ERR_INVALID_ARG),
    (4, 64, dict(ws_bytes=100), lsh.LSH_ERR_WORKSPACE),
])
def test_hybrid_rejects(n_sink, n_window, kw, status):
    assert _hybrid(n_sink, n_window, **kw) == status


def _noalloc(**kw):
    a = dict(q=1, keys=1, values=1, W=1, indices=1, offsets=1, B=1, Hq=4, Hkv=1, N=4096, d=128, K=8,
             L=32, T=2, stride=4096, scale=0.088, dtype=1, out=1)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lsh.lib().lsh_decode_attention_noalloc(
        p(a["q"]), p(a["keys"]), p(a["values"]), p(a["W"]), p(a["indices"]), p(a["offsets"]),
        a["B"], a["Hq"], a["Hkv"], a["N"], a["N"], None, a["d"], a["K"], a["L"], a["T"], a["stride"],
        ctypes.c_float(a["scale"]), a["dtype"], 0, 0, 0, p(a["out"]), None, None, None, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(out=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(T=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(Hq=17, Hkv=1), lsh.LSH_ERR_UNSUPPORTED),
    # 256 x 32 heads of 128K keys need far more than the 64 MiB scratch
    (dict(B=256, Hq=32, Hkv=8, N=131072, stride=8192, K=10, L=150), lsh.LSH_ERR_WORKSPACE),
])
def test_noalloc_rejects(kw, status):
    """Argument checks and the scratch-size limit come before any HIP call."""
    assert _noalloc(**kw) == status
    size = lsh.lsh_decode_workspace_size(kw.get("B", 1), kw.get("Hq", 4), kw.get("Hkv", 1), kw.get("N", 4096),
                                         128, kw.get("K", 8), kw.get("L", 32), kw.get("stride", 4096))
    assert (size > lsh.NOALLOC_SCRATCH_BYTES) == (status == lsh.LSH_ERR_WORKSPACE)


def _update(**kw):
    a = dict(keys=1, W=1, B=1, Hkv=1, n_old=100, n_new=200, n_cap=4096, d=128, K=8, L=32, stride=1024, dtype=1,
             w_per_head=0, offsets=1, indices=1, codes=None, ws=1, ws_bytes=1 << 40)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lsh.lib().lsh_update_tables(p(a["keys"]), p(a["W"]), a["B"], a["Hkv"], a["n_old"], a["n_new"],
                                       a["n_cap"], None, None, a["d"], a["K"], a["L"], a["stride"], a["dtype"],
                                       a["w_per_head"], p(a["offsets"]), p(a["indices"]), p(a["codes"]),
                                       p(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_old=-1), lsh.LSH_ERR_INVALID_ARG),
    (dict(n_old=300), lsh.LSH_ERR_INVALID_ARG),          # n_old > n_new
    (dict(n_new=5000), lsh.LSH_ERR_INVALID_ARG),         # n_new > n_cap
    (dict(n_cap=0, n_old=0, n_new=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(keys=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(stride=100), lsh.LSH_ERR_INVALID_ARG),
    (dict(d=64), lsh.LSH_ERR_UNSUPPORTED),
    (dict(ws_bytes=16), lsh.LSH_ERR_WORKSPACE),
    (dict(w_per_head=2), lsh.LSH_ERR_INVALID_ARG),
    (dict(n_old=200), lsh.LSH_OK),                       # nothing new: launches nothing
])
def test_update_rejects(kw, status):
    assert _update(**kw) == status


def _cached(**kw):
    a = dict(q=1, keys=1, values=1, W=1, indices=1, offsets=1, B=1, Hq=4, Hkv=1, N=3000, n_cap=4096, d=128, K=8,
             L=32, T=2, stride=1024, scale=0.088, dtype=1, w_per_head=0, n_sink=0, n_window=0, out=1, ws=1,
             ws_bytes=1 << 40)
    a.update(kw)
    p = lambda v: None if v is None else ctypes.c_void_p(v)
    return lsh.lib().lsh_decode_attention_cached(
        p(a["q"]), p(a["keys"]), p(a["values"]), p(a["W"]), p(a["indices"]), p(a["offsets"]),
        a["B"], a["Hq"], a["Hkv"], a["N"], a["n_cap"], None, a["d"], a["K"], a["L"], a["T"], a["stride"],
        ctypes.c_float(a["scale"]), a["dtype"], a["w_per_head"], a["n_sink"], a["n_window"], p(a["out"]), None,
        None, None, None, p(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_cap=2999), lsh.LSH_ERR_INVALID_ARG),         # N > n_cap
    (dict(N=0), lsh.LSH_ERR_INVALID_ARG),
    (dict(n_sink=-2), lsh.LSH_ERR_INVALID_ARG),
    (dict(values=None), lsh.LSH_ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=4), lsh.LSH_ERR_INVALID_ARG),
    (dict(w_per_head=-1), lsh.LSH_ERR_INVALID_ARG),
    (dict(ws_bytes=100), lsh.LSH_ERR_WORKSPACE),
])
def test_cached_decode_rejects(kw, status):
    assert _cached(**kw) == status


@pytest.mark.parametrize("B,Hq,Hkv,L,stride", [(1, 32, 4, 150, 8192), (1, 32, 8, 150, 1024), (64, 32, 8, 150, 8192),
                                                (2, 6, 2, 20, 256)])
def test_decode_workspace_grows_with_n(B, Hq, Hkv, L, stride):
    # the size at a cache's capacity covers every shorter prefix
    prev = 0
    for N in list(range(1, 3000, 97)) + list(range(3000, 300000, 4093)):
        w = lsh.lsh_decode_workspace_size(B, Hq, Hkv, N, 128, 10, L, stride)
        assert w >= prev, (N, w, prev)
        prev = w


def test_binding_raises_without_gpu_work():
    with pytest.raises(lsh.LshError) as e:
        lsh.lib()  # loads fine
        raise lsh.LshError(lsh.LSH_ERR_WORKSPACE)
    assert "WORKSPACE" in str(e.value)


def test_header_is_plain_c():
    # the boundary header compiles as C99 and as C++ (no torch or HIP types)
    import shutil
    import subprocess
    for cc, args in (("gcc", ["-std=c99", "-x", "c"]), ("g++", ["-std=c++11", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        r = subprocess.run([cc, "-fsyntax-only", "-Wall", "-Wextra", "-Werror", *args, HEADER],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr

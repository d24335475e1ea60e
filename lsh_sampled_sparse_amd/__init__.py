"""Python binding of liblsh_attn.so (LSH-sampled decode attention, gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels; this module checks tensor shapes and dtypes, allocates outputs and
workspaces with PyTorch, and passes raw device pointers and the current HIP
stream across the C ABI declared in ``include/lsh_attn.h``.  If the shared
library is missing, every call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblsh_attn.so")

LSH_OK, LSH_ERR_INVALID_ARG, LSH_ERR_UNSUPPORTED, LSH_ERR_WORKSPACE, LSH_ERR_HIP = range(5)
LSH_F32, LSH_BF16 = 0, 1

EXPORTS = (
    "lsh_status_string",
    "lsh_num_chunks",
    "lsh_default_stride",
    "lsh_build_workspace_size",
    "lsh_build_tables",
    "lsh_update_tables",
    "lsh_decode_workspace_size",
    "lsh_decode_attention",
    "lsh_decode_attention_hybrid",
    "lsh_decode_attention_cached",
    "lsh_decode_attention_noalloc",
    "lsh_kernel_count",
    "lsh_kernel_name",
    "lsh_timing_begin",
    "lsh_timing_end",
)

_lib = None
_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


def lib():
    """Load the shared library once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m lsh_sampled_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.lsh_status_string.restype = ctypes.c_char_p
        L.lsh_status_string.argtypes = [_i]
        L.lsh_num_chunks.restype = _i
        L.lsh_num_chunks.argtypes = [_i, _i]
        L.lsh_default_stride.restype = _i
        L.lsh_default_stride.argtypes = [_i, _i]
        L.lsh_build_workspace_size.restype = _sz
        L.lsh_build_workspace_size.argtypes = [_i] * 8
        L.lsh_build_tables.restype = _i
        L.lsh_build_tables.argtypes = [_p, _p] + [_i] * 8 + [_p, _p, _p, _p, _sz, _p]
        L.lsh_update_tables.restype = _i
        L.lsh_update_tables.argtypes = ([_p, _p] + [_i] * 5 + [_p, _p] + [_i] * 6
                                        + [_p, _p, _p, _p, _sz, _p])
        L.lsh_decode_workspace_size.restype = _sz
        L.lsh_decode_workspace_size.argtypes = [_i] * 8
        L.lsh_decode_attention.restype = _i
        L.lsh_decode_attention.argtypes = ([_p] * 6 + [_i] * 9 + [ctypes.c_float, _i]
                                           + [_p] * 6 + [_sz, _p])
        L.lsh_decode_attention_hybrid.restype = _i
        L.lsh_decode_attention_hybrid.argtypes = ([_p] * 6 + [_i] * 9 + [ctypes.c_float, _i, _i, _i]
                                                  + [_p] * 6 + [_sz, _p])
        L.lsh_decode_attention_cached.restype = _i
        L.lsh_decode_attention_cached.argtypes = ([_p] * 6 + [_i] * 5 + [_p] + [_i] * 5
                                                  + [ctypes.c_float] + [_i] * 4 + [_p] * 6 + [_sz, _p])
        L.lsh_decode_attention_noalloc.restype = _i
        L.lsh_decode_attention_noalloc.argtypes = ([_p] * 6 + [_i] * 5 + [_p] + [_i] * 5
                                                   + [ctypes.c_float] + [_i] * 4 + [_p] * 5 + [_p])
        L.lsh_kernel_count.restype = _i
        L.lsh_kernel_count.argtypes = []
        L.lsh_kernel_name.restype = ctypes.c_char_p
        L.lsh_kernel_name.argtypes = [_i]
        L.lsh_timing_begin.restype = _i
        L.lsh_timing_begin.argtypes = []
        L.lsh_timing_end.restype = _i
        L.lsh_timing_end.argtypes = [_p, _p]
        _lib = L
    return _lib


class LshError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(lsh_status_string(status))


def _check(status):
    if status != LSH_OK:
        raise LshError(status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return LSH_BF16
    if dt == torch.float32:
        return LSH_F32
    raise TypeError(f"unsupported dtype {dt}; use bfloat16 or float32")


def _require(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _check_decode_tensors(q, keys, values, W, indices, offsets, K, L, stride, n_cap, w_per_head_ok):
    """Host-side checks of a decode call's tensors before any pointer crosses
    the C ABI: every array on the GPU and contiguous, q / keys / values / W of
    one dtype, W [d, L*K] (or [Hkv, d, L*K] where one W per kv head is
    accepted), and tables of the shapes the kernels index with K, L, stride and
    the cache capacity n_cap: offsets [B, Hkv, L, nchunks(n_cap), 2^K],
    indices [B, Hkv, L, n_cap] (int16 holding uint16)."""
    for name, t in (("q", q), ("keys", keys), ("values", values)):
        _require(t, name, keys.dtype)
    _require(W, "W", keys.dtype)
    _require(indices, "indices", torch.int16)
    _require(offsets, "offsets", torch.int16)
    if q.dim() != 3 or keys.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and keys / values [B, Hkv, n_cap, d]")
    B, Hq, d = q.shape
    _, Hkv, cap, _ = keys.shape
    if tuple(values.shape) != tuple(keys.shape) or keys.shape[0] != B or keys.shape[3] != d:
        raise ValueError("q [B,Hq,d] and keys/values [B,Hkv,n_cap,d] disagree")
    if cap != n_cap:
        raise ValueError(f"keys hold {cap} positions per (sequence, kv head), the tables {n_cap}")
    shapes = [(d, L * K)] + ([(Hkv, d, L * K)] if w_per_head_ok else [])
    if tuple(W.shape) not in shapes:
        raise ValueError(f"W must be {' or '.join(str(list(x)) for x in shapes)}, got {list(W.shape)}")
    nch = lsh_num_chunks(n_cap, stride)
    if nch < 1:
        raise ValueError(f"invalid stride {stride} for {n_cap} keys")
    if tuple(offsets.shape) != (B, Hkv, L, nch, 1 << K):
        raise ValueError(f"offsets must be {[B, Hkv, L, nch, 1 << K]} for K={K}, L={L}, stride={stride}, "
                         f"got {list(offsets.shape)}")
    if tuple(indices.shape) != (B, Hkv, L, n_cap):
        raise ValueError(f"indices must be {[B, Hkv, L, n_cap]}, got {list(indices.shape)}")


# ------------------------------------------------------------------ C-ABI names

def lsh_status_string(status: int) -> str:
    return lib().lsh_status_string(int(status)).decode()


def lsh_num_chunks(N: int, stride: int) -> int:
    return lib().lsh_num_chunks(int(N), int(stride))


def lsh_default_stride(N: int, K: int) -> int:
    return lib().lsh_default_stride(int(N), int(K))


def lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, dtype) -> int:
    return lib().lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, dtype)


def lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride) -> int:
    return lib().lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride)


def lsh_build_tables(keys, W, K, L, stride, offsets, indices, key_codes=None, workspace=None):
    """Marshal tensors to ``lsh_build_tables``; outputs are filled in place.

    keys [B, Hkv, N, d], W [d, L*K] (bf16 or fp32, contiguous, on the GPU).
    """
    B, Hkv, N, d = keys.shape
    dt = _dtype_code(keys.dtype)
    if workspace is None:
        workspace = torch.empty(max(1, lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, dt)),
                                dtype=torch.uint8, device=keys.device)
    _check(lib().lsh_build_tables(
        _ptr(keys), _ptr(W), B, Hkv, N, d, K, L, stride, dt,
        _ptr(offsets), _ptr(indices), _ptr(key_codes),
        _ptr(workspace), workspace.numel(), _stream(keys.device)))


def lsh_update_tables(keys, W, K, L, stride, n_old, n_new, offsets, indices, key_codes=None, workspace=None,
                      old_lens=None, new_lens=None):
    """Marshal tensors to ``lsh_update_tables``; keys [B, Hkv, n_cap, d] is the
    cache, offsets / indices are updated in place.  W [d, L*K] is shared,
    W [Hkv, d, L*K] is one per kv head; old_lens / new_lens are optional int32
    device tensors [B] of per-sequence lengths."""
    B, Hkv, n_cap, d = keys.shape
    dt = _dtype_code(keys.dtype)
    if workspace is None:
        workspace = torch.empty(max(1, lsh_build_workspace_size(B, Hkv, n_cap, d, K, L, stride, dt)),
                                dtype=torch.uint8, device=keys.device)
    _check(lib().lsh_update_tables(
        _ptr(keys), _ptr(W), B, Hkv, int(n_old), int(n_new), n_cap, _ptr(old_lens), _ptr(new_lens),
        d, K, L, stride, dt, 1 if W.dim() == 3 else 0,
        _ptr(offsets), _ptr(indices), _ptr(key_codes),
        _ptr(workspace), workspace.numel(), _stream(keys.device)))


def lsh_decode_attention_cached(q, keys, values, W, indices, offsets, N, K, L, T, stride, sm_scale, n_sink,
                                n_window, out, lse=None, nsel=None, q_codes=None, counts=None, workspace=None,
                                seq_lens=None):
    """Marshal tensors to ``lsh_decode_attention_cached``: keys / values
    [B, Hkv, n_cap, d], of which the first N (or seq_lens[b], an int32 device
    tensor [B]) are attended; W as in ``lsh_update_tables``."""
    _check_decode_tensors(q, keys, values, W, indices, offsets, K, L, stride, keys.shape[2], True)
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = keys.shape
    dt = _dtype_code(keys.dtype)
    if workspace is None:
        workspace = torch.empty(max(1, lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride)),
                                dtype=torch.uint8, device=keys.device)
    _check(lib().lsh_decode_attention_cached(
        _ptr(q), _ptr(keys), _ptr(values), _ptr(W), _ptr(indices), _ptr(offsets),
        B, Hq, Hkv, int(N), n_cap, _ptr(seq_lens), d, K, L, T, stride, ctypes.c_float(sm_scale), dt,
        1 if W.dim() == 3 else 0, int(n_sink), int(n_window),
        _ptr(out), _ptr(lse), _ptr(nsel), _ptr(q_codes), _ptr(counts),
        _ptr(workspace), workspace.numel(), _stream(keys.device)))


NOALLOC_SCRATCH_BYTES = 64 << 20


def lsh_decode_attention_noalloc(q, keys, values, W, indices, offsets, N, K, L, T, stride, sm_scale, n_sink,
                                 n_window, out, lse=None, nsel=None, q_codes=None, counts=None, seq_lens=None):
    """Marshal tensors to ``lsh_decode_attention_noalloc``: the cached decode
    with the library's static scratch as its workspace (nothing allocated);
    arguments as ``lsh_decode_attention_cached`` without ``workspace``."""
    _check_decode_tensors(q, keys, values, W, indices, offsets, K, L, stride, keys.shape[2], True)
    B, Hq, d = q.shape
    _, Hkv, n_cap, _ = keys.shape
    dt = _dtype_code(keys.dtype)
    _check(lib().lsh_decode_attention_noalloc(
        _ptr(q), _ptr(keys), _ptr(values), _ptr(W), _ptr(indices), _ptr(offsets),
        B, Hq, Hkv, int(N), n_cap, _ptr(seq_lens), d, K, L, T, stride, ctypes.c_float(sm_scale), dt,
        1 if W.dim() == 3 else 0, int(n_sink), int(n_window),
        _ptr(out), _ptr(lse), _ptr(nsel), _ptr(q_codes), _ptr(counts), _stream(keys.device)))


def lsh_decode_attention(q, keys, values, W, indices, offsets, K, L, T, stride, sm_scale, out,
                         lse=None, nsel=None, q_codes=None, counts=None, workspace=None):
    """Marshal tensors to ``lsh_decode_attention``; outputs are filled in place."""
    _check_decode_tensors(q, keys, values, W, indices, offsets, K, L, stride, keys.shape[2], False)
    B, Hq, d = q.shape
    _, Hkv, N, _ = keys.shape
    dt = _dtype_code(keys.dtype)
    if workspace is None:
        workspace = torch.empty(max(1, lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride)),
                                dtype=torch.uint8, device=keys.device)
    _check(lib().lsh_decode_attention(
        _ptr(q), _ptr(keys), _ptr(values), _ptr(W), _ptr(indices), _ptr(offsets),
        B, Hq, Hkv, N, d, K, L, T, stride, ctypes.c_float(sm_scale), dt,
        _ptr(out), _ptr(lse), _ptr(nsel), _ptr(q_codes), _ptr(counts),
        _ptr(workspace), workspace.numel(), _stream(keys.device)))


def lsh_decode_attention_hybrid(q, keys, values, W, indices, offsets, K, L, T, stride, sm_scale, n_sink,
                                n_window, out, lse=None, nsel=None, q_codes=None, counts=None, workspace=None):
    """Marshal tensors to ``lsh_decode_attention_hybrid``; outputs are filled in place."""
    _check_decode_tensors(q, keys, values, W, indices, offsets, K, L, stride, keys.shape[2], False)
    B, Hq, d = q.shape
    _, Hkv, N, _ = keys.shape
    dt = _dtype_code(keys.dtype)
    if workspace is None:
        workspace = torch.empty(max(1, lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride)),
                                dtype=torch.uint8, device=keys.device)
    _check(lib().lsh_decode_attention_hybrid(
        _ptr(q), _ptr(keys), _ptr(values), _ptr(W), _ptr(indices), _ptr(offsets),
        B, Hq, Hkv, N, d, K, L, T, stride, ctypes.c_float(sm_scale), dt, int(n_sink), int(n_window),
        _ptr(out), _ptr(lse), _ptr(nsel), _ptr(q_codes), _ptr(counts),
        _ptr(workspace), workspace.numel(), _stream(keys.device)))


def lsh_kernel_count() -> int:
    return lib().lsh_kernel_count()


def lsh_kernel_name(kid: int):
    n = lib().lsh_kernel_name(int(kid))
    return None if n is None else n.decode()


def lsh_timing_begin() -> None:
    _check(lib().lsh_timing_begin())


def lsh_timing_end():
    """Close the timing window; returns {kernel name: (total ms, launches)}."""
    n = lsh_kernel_count()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int32 * n)()
    _check(lib().lsh_timing_end(ms, cnt))
    return {lsh_kernel_name(k): (ms[k], cnt[k]) for k in range(n)}


# ------------------------------------------------------------------ convenience


def build_tables(keys, W, K, L, stride=None, return_codes=False):
    """Build the bucket tables of every (sequence, kv head).

    Returns dict: offsets [B,Hkv,L,nchunks,2^K] (int16 holding the uint16
    start of each bucket inside each chunk's region), indices [B,Hkv,L,N]
    (int16 holding the uint16 chunk-relative key index, chunk-major), stride,
    and codes [B,Hkv,L,N] (int16 holding uint16) when ``return_codes``.
    """
    _require(keys, "keys")
    _require(W, "W", keys.dtype)
    B, Hkv, N, d = keys.shape
    if tuple(W.shape) != (d, L * K):
        raise ValueError(f"W must be [{d}, {L * K}], got {tuple(W.shape)}")
    if stride is None:
        stride = lsh_default_stride(N, K)
    nch = lsh_num_chunks(N, stride)
    dev = keys.device
    offsets = torch.empty(B, Hkv, L, nch, 1 << K, dtype=torch.int16, device=dev)
    indices = torch.empty(B, Hkv, L, N, dtype=torch.int16, device=dev)
    codes = torch.empty(B, Hkv, L, N, dtype=torch.int16, device=dev) if return_codes else None
    lsh_build_tables(keys, W, K, L, stride, offsets, indices, codes)
    res = {"offsets": offsets, "indices": indices, "stride": stride}
    if return_codes:
        res["codes"] = codes
    return res


def alloc_tables(keys, K, L, stride=None, return_codes=False):
    """Empty tables for a key cache keys [B, Hkv, n_cap, d] that will grow to
    n_cap keys; fill them with ``update_tables``.  Returns the dict of
    ``build_tables`` with the pitch n_cap, "lens" (keys held per sequence,
    all 0) and "n" (the longest)."""
    B, Hkv, n_cap, d = keys.shape
    if stride is None:
        stride = lsh_default_stride(n_cap, K)
    nch = lsh_num_chunks(n_cap, stride)
    dev = keys.device
    res = {"offsets": torch.empty(B, Hkv, L, nch, 1 << K, dtype=torch.int16, device=dev),
           "indices": torch.empty(B, Hkv, L, n_cap, dtype=torch.int16, device=dev),
           "stride": stride, "n": 0, "n_cap": n_cap, "lens": [0] * B, "lens_dev": None}
    if return_codes:
        res["codes"] = torch.empty(B, Hkv, L, n_cap, dtype=torch.int16, device=dev)
    return res


def _lens_tensor(lens, device):
    return torch.tensor(lens, dtype=torch.int32, device=device)


def update_tables(keys, W, tables, n_new, K, L, workspace=None):
    """Extend ``tables`` (from ``alloc_tables``) to hold keys 0 .. n_new - 1
    of the cache ``keys``: n_new is one length for every sequence or a list
    of B lengths.  Afterwards each sequence's tables equal a build over its
    keys.  W [d, L*K] is shared by all heads, W [Hkv, d, L*K] one per kv head."""
    _require(keys, "keys")
    _require(W, "W", keys.dtype)
    B, Hkv, n_cap, d = keys.shape
    if n_cap != tables["n_cap"]:
        raise ValueError("keys and tables disagree on the capacity")
    if tuple(W.shape) not in ((d, L * K), (Hkv, d, L * K)):
        raise ValueError(f"W must be [{d}, {L * K}] or [{Hkv}, {d}, {L * K}], got {tuple(W.shape)}")
    old = list(tables["lens"])
    new = [int(n_new)] * B if isinstance(n_new, int) else [int(x) for x in n_new]
    if len(new) != B or any(nw < od or nw > n_cap for nw, od in zip(new, old)):
        raise ValueError(f"new lengths {new} must lie between the held lengths {old} and {n_cap}")
    uniform = len(set(old)) == 1 and len(set(new)) == 1
    old_t = None if uniform else _lens_tensor(old, keys.device)
    new_t = None if uniform else _lens_tensor(new, keys.device)
    lsh_update_tables(keys, W, K, L, tables["stride"], min(old), max(new), tables["offsets"], tables["indices"],
                      tables.get("codes"), workspace, old_t, new_t)
    tables["lens"] = new
    tables["n"] = max(new)
    tables["lens_dev"] = None if len(set(new)) == 1 else (new_t if new_t is not None
                                                          else _lens_tensor(new, keys.device))
    return tables


def decode_attention(q, keys, values, W, tables, K, L, T, sm_scale=None, return_codes=False,
                     return_counts=False, workspace=None, n_sink=0, n_window=0):
    """One decode step.  Returns dict: out [B,Hq,d] fp32, lse [B,Hq], nsel [B,Hq],
    and q_codes [B,Hq,L] / counts [B,Hq,N] (uint8) when requested.  With
    n_sink / n_window > 0 it is the hybrid decode: the first n_sink and the
    last n_window keys are attended exactly and merged with the estimate.
    Tables from ``alloc_tables`` / ``update_tables`` attend the first
    tables["n"] keys of the cache."""
    for name, t in (("q", q), ("keys", keys), ("values", values)):
        _require(t, name, keys.dtype)
    B, Hq, d = q.shape
    _, Hkv, N, _ = keys.shape
    cached = "n_cap" in tables
    if cached and tables["n_cap"] != N:
        raise ValueError("keys and tables disagree on the capacity")
    # one W per kv head only goes with cache tables (the cached entry point
    # takes the flag; the plain one would read a 3-D W as a shared one)
    _check_decode_tensors(q, keys, values, W, tables["indices"], tables["offsets"], K, L, tables["stride"], N,
                          cached)
    if cached:
        N = tables["n"]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    dev = keys.device
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    nsel = torch.empty(B, Hq, dtype=torch.int32, device=dev)
    qc = torch.empty(B, Hq, L, dtype=torch.int16, device=dev) if return_codes else None
    cnt = torch.empty(B, Hq, N, dtype=torch.uint8, device=dev) if return_counts else None
    if cached:
        lsh_decode_attention_cached(q, keys, values, W, tables["indices"], tables["offsets"], N, K, L, T,
                                    tables["stride"], sm_scale, n_sink, n_window, out, lse, nsel, qc, cnt,
                                    workspace, seq_lens=tables.get("lens_dev"))
    elif n_sink or n_window:
        lsh_decode_attention_hybrid(q, keys, values, W, tables["indices"], tables["offsets"], K, L, T,
                                    tables["stride"], sm_scale, n_sink, n_window, out, lse, nsel, qc, cnt,
                                    workspace)
    else:
        lsh_decode_attention(q, keys, values, W, tables["indices"], tables["offsets"], K, L, T,
                             tables["stride"], sm_scale, out, lse, nsel, qc, cnt, workspace)
    res = {"out": out, "lse": lse, "nsel": nsel}
    if return_codes:
        res["q_codes"] = qc
    if return_counts:
        res["counts"] = cnt
    return res

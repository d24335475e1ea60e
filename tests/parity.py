"""Comparison of the HIP path with the fp64 oracle (test helper).

The oracle only ever receives the seeded inputs from ``workloads``; nothing it
computes is fed by the GPU.  A SimHash bit whose projection lies inside the
band |proj| < 1e-4 * ||x|| * ||w_c|| may legitimately differ between fp32 and
fp64 arithmetic, so:
  * codes must match the oracle bit for bit outside that band, and flips
    inside it must stay below 1e-5 of all bits;
  * every table whose codes agree must give bit-identical chunk offsets and
    indices (the oracle's buckets, split by key chunk through its chunk
    bounds and laid out chunk-major); a table with a flipped bit must still be
    a valid stable bucketing of the GPU's own codes;
  * collision counts and selections must agree exactly for every key whose
    codes (and the probing query's codes) agree; others may differ by at most
    the number of disagreeing tables;
  * outputs must be within 2e-3 relative L2 of the oracle.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import lsh_oracle as O

BAND = 1e-4
FLIP_FRACTION_MAX = 1e-5
OUT_RTOL = 2e-3
LSE_ATOL = 2e-3


def u16(t):
    return (np.asarray(t).astype(np.int64)) & 0xFFFF


def band_mask(x, W):
    """[n, L*K] bool: projection of row i on column c is inside the flip band."""
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    proj = x @ W
    scale = np.linalg.norm(x, axis=1)[:, None] * np.linalg.norm(W, axis=0)[None, :]
    return np.abs(proj) < BAND * scale


def compare_codes(gpu, ref, band, K, L):
    """gpu/ref int [L, n]; band [n, L*K].  Returns the number of flipped bits."""
    gpu = u16(gpu)
    ref = np.asarray(ref, np.int64)
    diff = gpu ^ ref
    flips = 0
    for l, n in zip(*np.nonzero(diff)):
        for b in range(K):
            if (diff[l, n] >> b) & 1:
                assert band[n, l * K + b], f"code bit outside the flip band differs: table {l} key {n} bit {b}"
                flips += 1
    return flips


def indices_to_global(idx, stride):
    """Chunk-major uint16 entries [L, N] -> key indices (int64): position p
    lies in chunk p // stride and holds (key - chunk * stride)."""
    idx = u16(idx)
    N = idx.shape[-1]
    return idx + (np.arange(N, dtype=np.int64) // stride) * stride


def expected_chunk_layout(ref, stride):
    """The chunk-major layout of the oracle's tables.

    Bucket c of chunk j is ref indices[l, bounds[l, c, j]:bounds[l, c, j + 1]];
    chunk j lists its buckets in code order.  Returns (offsets [L, nJ, nb],
    global key order [L, N])."""
    bnd = np.asarray(ref["bounds"], np.int64)
    idx = np.asarray(ref["indices"], np.int64)
    L, nb, nJ1 = bnd.shape
    lens = np.diff(bnd, axis=2).transpose(0, 2, 1)              # [L, nJ, nb]
    off = np.cumsum(lens, axis=2) - lens
    order = np.empty_like(idx)
    for l in range(L):
        # runs (bucket c, chunk j) in chunk-major order: j outer, c inner
        starts = bnd[l, :, :-1].T.ravel()
        ln = lens[l].ravel()
        pos = np.repeat(starts - np.concatenate(([0], np.cumsum(ln)[:-1])), ln) + np.arange(ln.sum())
        order[l] = idx[l][pos]
    return off, order


def check_tables(gpu_off, gpu_idx, gpu_codes, ref, K, stride):
    """Compare one unit's tables.  ``ref`` from ``O.build_tables`` on the same
    keys; ``gpu_off`` [L, nJ, 2^K] and ``gpu_idx`` [L, N] are the library's
    chunk-major outputs.  Returns the number of tables with a flipped bit."""
    gpu_idx = indices_to_global(gpu_idx, stride)
    gpu_off = u16(gpu_off)
    gpu_codes = u16(gpu_codes)
    L, N = gpu_codes.shape
    nb = 1 << K
    nJ = gpu_off.shape[1]
    assert nJ == O.num_chunks(N, stride)
    exp_off, exp_idx = expected_chunk_layout(ref, stride)
    same = np.all(gpu_codes == ref["codes"], axis=1)
    chunk = np.arange(N, dtype=np.int64) // stride
    for l in range(L):
        if same[l]:
            np.testing.assert_array_equal(gpu_off[l], exp_off[l])
            np.testing.assert_array_equal(gpu_idx[l], exp_idx[l])
        else:
            # valid stable bucketing of the GPU's own codes, chunk by chunk
            hist = np.bincount(chunk * nb + gpu_codes[l], minlength=nJ * nb).reshape(nJ, nb)
            np.testing.assert_array_equal(gpu_off[l], np.cumsum(hist, axis=1) - hist)
            keys = np.arange(N, dtype=np.int64)
            np.testing.assert_array_equal(gpu_idx[l], keys[np.lexsort((keys, gpu_codes[l], chunk))])
    return int((~same).sum())


def check_head(gpu, ref, q_band, key_codes_gpu, key_codes_ref, K, L, T, exact=None):
    """Compare one query head.  gpu: dict of numpy (q_codes [L], counts [N] or
    None, out [d], lse, nsel).  ref: dict from ``O.decode_head``, or from
    ``O.hybrid_decode_head`` with ``exact`` its exact set (bool [N]): those
    keys keep their collision counts but are never part of the selection."""
    N = len(ref["counts"])
    excl = np.zeros(N, bool) if exact is None else np.asarray(exact, bool)
    qflips = compare_codes(gpu["q_codes"][:, None], ref["qcodes"][:, None], q_band, K, L)
    bad_q = u16(gpu["q_codes"]) != ref["qcodes"]                        # tables whose probe differs
    key_bad = (u16(key_codes_gpu) != key_codes_ref)                     # [L, N]
    affected = key_bad.copy()
    affected[bad_q, :] = True
    n_aff = affected.sum(axis=0)                                        # per key
    exact_keys = n_aff == 0
    if gpu.get("counts") is not None:
        c = np.asarray(gpu["counts"]).astype(np.int64)
        np.testing.assert_array_equal(c[exact_keys], ref["counts"][exact_keys])
        assert np.all(np.abs(c - ref["counts"]) <= n_aff)
        np.testing.assert_array_equal(((c >= T) & ~excl)[exact_keys], ref["mask"][exact_keys])
    if exact_keys.all():
        assert int(gpu["nsel"]) == ref["nsel"]
    else:
        assert abs(int(gpu["nsel"]) - ref["nsel"]) <= int((~exact_keys).sum())
    out = np.asarray(gpu["out"], np.float64)
    if ref["nsel"] == 0 and not excl.any():
        assert int(gpu["nsel"]) == 0 or not exact_keys.all()
        if int(gpu["nsel"]) == 0:
            assert np.all(out == 0) and gpu["lse"] == -np.inf
        return {"qflips": qflips, "rel": 0.0}
    rel = np.linalg.norm(out - ref["out"]) / max(np.linalg.norm(ref["out"]), 1e-30)
    assert rel <= OUT_RTOL, f"relative L2 error {rel:.3e} > {OUT_RTOL}"
    assert abs(float(gpu["lse"]) - ref["lse"]) <= LSE_ATOL * max(1.0, abs(ref["lse"]))
    return {"qflips": qflips, "rel": rel}


def estimate_error(out, exact):
    return float(np.linalg.norm(np.asarray(out, np.float64) - exact[0]) / max(np.linalg.norm(exact[0]), 1e-30))

"""Plain, slow, fp64 CPU oracle for LSH-sampled decode attention (MagicPIG).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or constant with the HIP library; both sides receive the same seeded
inputs from ``workloads.py`` and nothing else.

What is computed, and where it comes from
-----------------------------------------
MagicPIG estimates the attention output of a decode query by *sampling* keys
with locality-sensitive hashing instead of taking the top-k ("MagicPIG: LSH
Sampling for Efficient LLM Generation", GrooveSquid summary, medium-difficulty
summary; MagicPIG project summary on sourcepulse, "How It Works").  The
pages name an LSH kernel and an LSH interface ("How infini-ai-lab/magicpig
works", Components: "LSH Sampling") and an optimised hash-table construction
(sourcepulse summary, "Highlighted Details"), but print no formula.  The
steps below are therefore the plainest concrete reading of the method, each
one stated in its own docstring:

  1. SimHash: K sign bits per table, L tables, from one Gaussian projection
     matrix W of shape [d, L*K]; column l*K + b is bit b of table l, bit 0 is
     the least significant bit, and a bit is 1 iff the projection is > 0.
  2. Per-table buckets: a stable counting sort of key indices by code
     (CSR: offsets[2^K + 1] and indices[N], ascending inside each bucket),
     plus the chunk bounds used to split a bucket by key range.
  3. Query hashing with the same W, probing of the L buckets, per-key
     collision counts, and selection of keys with count >= T.
  4. Importance weights 1/u, where u is the probability that the key is
     selected: u = P[Binomial(L, P) >= T] with P = (1 - theta/pi)^K the
     single-table SimHash collision probability (Charikar 2002) and theta the
     query-key angle.  Weighting selected terms by 1/u is the
     Horvitz-Thompson correction, so the weighted sums are unbiased.
  5. A self-normalised softmax over the selected keys of
     l_n = s * q.k_n - ln u_n, returned with its log-sum-exp.  The
     log-sum-exp merge of split partial states is the same one MAC-Attention
     uses ("MAC-Attention" README, "How It Works").

Everything is float64 numpy.  Ties (projection exactly 0) give bit 0; a zero
norm gives cos = 0; u is clamped below at 1e-30; an empty selection gives
out = 0 and lse = -inf.
"""

from __future__ import annotations

import math

import numpy as np

U_FLOOR = 1e-30


# --------------------------------------------------------------------------
# 1. SimHash codes
# --------------------------------------------------------------------------

def simhash_projections(x, W):
    """Projections x @ W in float64: x [n, d], W [d, L*K] -> [n, L*K]."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    return x @ W


def simhash_codes(x, W, K, L):
    """SimHash codes of the rows of x: returns int64 [L, n].

    code_l(x) = sum_b [ (x @ W)[l*K + b] > 0 ] * 2^b  (bit 0 = LSB).
    With K = 0 every code is 0 (one bucket per table).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    codes = np.zeros((L, n), dtype=np.int64)
    if K == 0:
        return codes
    proj = simhash_projections(x, W)
    if proj.shape[1] != L * K:
        raise ValueError("W must have L*K columns")
    bits = (proj > 0.0).astype(np.int64)
    for l in range(L):
        for b in range(K):
            codes[l] += bits[:, l * K + b] << b
    return codes


# --------------------------------------------------------------------------
# 2. Per-table buckets (CSR) and chunk bounds
# --------------------------------------------------------------------------

def bucket_tables(codes, K):
    """Stable counting sort of key indices by code, one table at a time.

    codes int [L, N] -> offsets int64 [L, 2^K + 1], indices int64 [L, N].
    offsets[l, c] is the number of keys whose code in table l is < c, so
    bucket c of table l is indices[l, offsets[l, c]:offsets[l, c + 1]], and
    the indices inside a bucket are in ascending order.
    """
    codes = np.asarray(codes, dtype=np.int64)
    L, N = codes.shape
    nb = 1 << K
    offsets = np.zeros((L, nb + 1), dtype=np.int64)
    indices = np.zeros((L, N), dtype=np.int64)
    for l in range(L):
        counts = np.bincount(codes[l], minlength=nb)
        offsets[l, 1:] = np.cumsum(counts)
        indices[l] = np.argsort(codes[l], kind="stable")
    return offsets, indices


def num_chunks(N, stride):
    return (N + stride - 1) // stride


def bucket_chunk_bounds(offsets, indices, K, stride):
    """Positions that split every bucket by key range.

    bounds[l, c, j] = position of the first entry of bucket c in table l whose
    key index is >= j * stride (the bucket's end if there is none), for
    j = 0 .. ceil(N / stride).  So bounds[l, c, 0] = offsets[l, c] and
    bounds[l, c, last] = offsets[l, c + 1], and the keys of chunk j that sit in
    bucket c are indices[l, bounds[l, c, j]:bounds[l, c, j + 1]].
    Returns int64 [L, 2^K, nchunks + 1].
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    indices = np.asarray(indices, dtype=np.int64)
    L, N = indices.shape
    nb = 1 << K
    nch = num_chunks(N, stride)
    bounds = np.zeros((L, nb, nch + 1), dtype=np.int64)
    targets = np.minimum(np.arange(nch + 1, dtype=np.int64) * stride, N)
    for l in range(L):
        for c in range(nb):
            lo, hi = offsets[l, c], offsets[l, c + 1]
            seg = indices[l, lo:hi]
            bounds[l, c, :] = lo + np.searchsorted(seg, targets, side="left")
    return bounds


# --------------------------------------------------------------------------
# 3. Probe, count, select
# --------------------------------------------------------------------------

def collision_counts(qcodes, offsets, indices, N):
    """c(n) = number of tables l whose bucket qcodes[l] holds key n.

    Computed by walking the probed buckets of the CSR.
    """
    L = len(qcodes)
    counts = np.zeros(N, dtype=np.int64)
    for l in range(L):
        c = int(qcodes[l])
        seg = indices[l, offsets[l, c]:offsets[l, c + 1]]
        counts[seg] += 1  # a key occurs at most once per table
    return counts


def select(counts, T):
    """Boolean mask of the keys that collide in at least T tables."""
    return np.asarray(counts) >= T


# --------------------------------------------------------------------------
# 4. Importance weights
# --------------------------------------------------------------------------

def cosines(q, keys):
    """cos of the angle between q [d] and each row of keys [N, d]; 0 if a norm is 0."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    dots = keys @ q
    norms = np.linalg.norm(keys, axis=1) * np.linalg.norm(q)
    out = np.zeros_like(dots)
    nz = norms > 0
    out[nz] = dots[nz] / norms[nz]
    return np.clip(out, -1.0, 1.0)


def collision_prob(cos, K):
    """Single-table SimHash collision probability P = (1 - theta/pi)^K.

    A random hyperplane separates two vectors at angle theta with probability
    theta/pi (Goemans-Williamson 1995, Charikar 2002); K independent bits all
    agree with probability (1 - theta/pi)^K.  K = 0 gives 1.
    """
    theta = np.arccos(np.clip(np.asarray(cos, dtype=np.float64), -1.0, 1.0))
    p = 1.0 - theta / math.pi
    if K == 0:
        return np.ones_like(p)
    return p ** K


def _log_binom(L, i):
    return math.lgamma(L + 1) - math.lgamma(i + 1) - math.lgamma(L - i + 1)


def inclusion_prob(P, L, T):
    """u = P[Binomial(L, P) >= T] = sum_{i=T}^{L} C(L,i) P^i (1-P)^(L-i).

    The L tables use disjoint columns of a Gaussian W, so given (q, k) they
    collide independently, each with probability P; the key is selected when
    at least T of them do.  Summed as positive terms in log space; clamped
    below at 1e-30 so that ln u stays finite.
    """
    P = np.asarray(P, dtype=np.float64)
    flat = P.reshape(-1)
    out = np.empty_like(flat)
    out[flat >= 1.0] = 1.0   # only the i = L term survives, and it is 1
    out[flat <= 0.0] = 0.0
    inner = (flat > 0.0) & (flat < 1.0)
    if inner.any():
        p = flat[inner]
        i = np.arange(T, L + 1, dtype=np.float64)
        log_c = np.array([_log_binom(L, int(k)) for k in range(T, L + 1)])
        terms = (log_c[None, :] + i[None, :] * np.log(p)[:, None]
                 + (L - i)[None, :] * np.log1p(-p)[:, None])      # [n, L-T+1]
        m = terms.max(axis=1)
        out[inner] = np.exp(m) * np.exp(terms - m[:, None]).sum(axis=1)
    return np.maximum(out, U_FLOOR).reshape(P.shape)


# --------------------------------------------------------------------------
# 5. Weighted softmax and the log-sum-exp merge
# --------------------------------------------------------------------------

def weighted_softmax_attention(q, keys, values, mask, u, scale):
    """Self-normalised estimate over the selected keys.

    l_n = scale * q.k_n - ln u_n for selected n; out = sum softmax(l)_n v_n,
    lse = ln sum_n exp(l_n).  Empty selection -> (zeros, -inf).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    sel = np.nonzero(np.asarray(mask))[0]
    d = values.shape[1]
    if sel.size == 0:
        return np.zeros(d), -np.inf
    logits = scale * (keys[sel] @ q) - np.log(np.asarray(u, dtype=np.float64)[sel])
    m = logits.max()
    w = np.exp(logits - m)
    z = w.sum()
    out = (w @ values[sel]) / z
    return out, m + math.log(z)


def exact_attention(q, keys, values, scale):
    """Dense softmax attention of one query head (the K = 0 limit)."""
    N = np.asarray(keys).shape[0]
    return weighted_softmax_attention(q, keys, values, np.ones(N, bool), np.ones(N), scale)


def lse_merge(parts):
    """Merge partial softmax states [(out_s, lse_s)] into one (out, lse).

    Each partial is a normalised output with its log-sum-exp; empty parts
    (lse = -inf) contribute nothing.
    """
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    d = len(parts[0][0])
    if np.all(np.isneginf(lses)):
        return np.zeros(d), -np.inf
    M = lses.max()
    wts = np.exp(lses - M)
    out = sum(w * np.asarray(o, np.float64) for w, (o, _) in zip(wts, parts)) / wts.sum()
    return out, M + math.log(wts.sum())


# --------------------------------------------------------------------------
# Whole path
# --------------------------------------------------------------------------

def build_tables(keys, W, K, L, stride):
    """Table build for one (sequence, kv head) unit: keys [N, d].

    Returns dict with codes [L, N], offsets [L, 2^K+1], indices [L, N],
    bounds [L, 2^K, nchunks+1].
    """
    codes = simhash_codes(keys, W, K, L)
    offsets, indices = bucket_tables(codes, K)
    bounds = bucket_chunk_bounds(offsets, indices, K, stride)
    return {"codes": codes, "offsets": offsets, "indices": indices, "bounds": bounds}


def decode_head(q, keys, values, W, offsets, indices, K, L, T, scale, qcodes=None):
    """One query head against its unit's tables.

    Returns dict: qcodes [L], counts [N], mask [N], nsel, u [N] (1 where not
    selected), out [d], lse.  ``qcodes`` may be given to run on codes fixed
    elsewhere.
    """
    N = np.asarray(keys).shape[0]
    if qcodes is None:
        qcodes = simhash_codes(np.asarray(q)[None, :], W, K, L)[:, 0]
    counts = collision_counts(qcodes, offsets, indices, N)
    mask = select(counts, T)
    u = np.ones(N)
    if mask.any():
        cs = cosines(q, np.asarray(keys)[mask])
        u[mask] = inclusion_prob(collision_prob(cs, K), L, T)
    out, lse = weighted_softmax_attention(q, keys, values, mask, u, scale)
    return {"qcodes": np.asarray(qcodes), "counts": counts, "mask": mask,
            "nsel": int(mask.sum()), "u": u, "out": out, "lse": lse}


def exact_set(N, n_sink, n_window):
    """The keys a hybrid decode attends exactly: the first n_sink keys
    (attention sinks) and the last n_window keys (the recent window).

    MagicPIG pairs dense attention with sampled sparse attention ("How
    infini-ai-lab/magicpig works", overview: CPU sparse attention complementing
    GPU attention; sourcepulse summary, "How It Works"); the pages do not say
    which keys the dense part takes.  The reading here is a static set of
    sinks plus a recent window, the set MAC-Attention recomputes exactly and
    merges by log-sum-exp ("MAC-Attention" README, "How It Works", front
    sinks).  Returns bool [N]."""
    E = np.zeros(N, dtype=bool)
    E[:max(0, min(N, n_sink))] = True
    if n_window > 0:
        E[max(0, N - n_window):] = True
    return E


def hybrid_decode_head(q, keys, values, W, offsets, indices, K, L, T, scale, n_sink, n_window, qcodes=None):
    """Hybrid decode of one query head: exact softmax attention over the
    static set E = exact_set(N, n_sink, n_window), the 1/u-weighted estimate
    over the selected keys outside E, and the log-sum-exp merge of the two.

    Returns dict: as decode_head, with mask = selected keys outside E,
    nsel = |mask|, exact = E, and out / lse of the merge.
    """
    r = decode_head(q, keys, values, W, offsets, indices, K, L, T, scale, qcodes=qcodes)
    N = np.asarray(keys).shape[0]
    E = exact_set(N, n_sink, n_window)
    sampled = r["mask"] & ~E
    part_s = weighted_softmax_attention(q, keys, values, sampled, r["u"], scale)
    part_e = weighted_softmax_attention(q, keys, values, E, np.ones(N), scale)
    out, lse = lse_merge([part_s, part_e])
    r.update({"mask": sampled, "nsel": int(sampled.sum()), "exact": E, "out": out, "lse": lse})
    return r


def decode(q, keys, values, W, tables, K, L, T, scale, heads=None):
    """Decode over a batch: q [B, Hq, d], keys/values [B, Hkv, N, d].

    ``tables[(b, g)]`` is the dict from ``build_tables`` for that unit.  Query
    head h uses kv head h // (Hq // Hkv).  ``heads`` optionally restricts the
    work to a list of (b, h) pairs.  Returns dict keyed by (b, h).
    """
    q = np.asarray(q)
    B, Hq, _ = q.shape
    Hkv = np.asarray(keys).shape[1]
    G = Hq // Hkv
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hq)]
    res = {}
    for b, h in heads:
        g = h // G
        t = tables[(b, g)]
        res[(b, h)] = decode_head(q[b, h], keys[b, g], values[b, g], W,
                                  t["offsets"], t["indices"], K, L, T, scale)
    return res

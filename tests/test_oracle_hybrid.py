"""Pins of the oracle's hybrid decode (exact attention over sinks + a recent
window, LSH-sampled estimate over the rest, merged by log-sum-exp), CPU only.

Each pin checks the oracle against something other than itself: torch's
softmax attention in float64, the plain sampled decode, or a brute-force sum
built from direct code comparison and scipy's binomial tail.
"""

import math

import numpy as np
import pytest
import scipy.stats
import torch

from oracle import lsh_oracle as O


def torch_attention(q, keys, values, scale):
    qt = torch.tensor(q, dtype=torch.float64)
    kt = torch.tensor(keys, dtype=torch.float64)
    vt = torch.tensor(values, dtype=torch.float64)
    s = scale * (kt @ qt)
    return (torch.softmax(s, 0) @ vt).numpy(), float(torch.logsumexp(s, 0))


def tiny_case(seed, N=40, d=16, K=3, L=6):
    rng = np.random.default_rng(seed)
    keys = rng.standard_normal((N, d))
    values = rng.standard_normal((N, d))
    W = rng.standard_normal((d, L * K))
    q = 0.8 * keys[5] + 0.6 * rng.standard_normal(d)
    tb = O.build_tables(keys, W, K, L, 16)
    return q, keys, values, W, tb


def test_exact_set_geometry():
    assert O.exact_set(10, 3, 4).tolist() == [1, 1, 1, 0, 0, 0, 1, 1, 1, 1]
    assert O.exact_set(10, 0, 0).sum() == 0
    assert O.exact_set(10, 7, 6).all()                 # sink and window overlap
    assert O.exact_set(10, 20, 0).all() and O.exact_set(10, 0, 20).all()
    assert O.exact_set(5, 2, 0).tolist() == [1, 1, 0, 0, 0]


@pytest.mark.parametrize("sink,window", [(40, 0), (0, 40), (25, 30)])
def test_everything_exact_is_exact_attention(sink, window):
    q, keys, values, W, tb = tiny_case(1)
    r = O.hybrid_decode_head(q, keys, values, W, tb["offsets"], tb["indices"], 3, 6, 2, 0.25, sink, window)
    ref, lse = torch_attention(q, keys, values, 0.25)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    assert abs(r["lse"] - lse) < 1e-12
    assert r["nsel"] == 0


def test_empty_exact_set_is_the_sampled_decode():
    q, keys, values, W, tb = tiny_case(2)
    a = O.hybrid_decode_head(q, keys, values, W, tb["offsets"], tb["indices"], 3, 6, 2, 0.25, 0, 0)
    b = O.decode_head(q, keys, values, W, tb["offsets"], tb["indices"], 3, 6, 2, 0.25)
    np.testing.assert_array_equal(a["out"], b["out"])
    assert a["lse"] == b["lse"] and a["nsel"] == b["nsel"]


@pytest.mark.parametrize("sink,window", [(0, 0), (3, 7), (0, 12)])
def test_k0_is_exact_attention_for_any_exact_set(sink, window):
    rng = np.random.default_rng(3)
    N, d, L = 30, 8, 4
    keys, values = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    q = rng.standard_normal(d)
    W = np.zeros((d, 0))
    tb = O.build_tables(keys, W, 0, L, 16)
    r = O.hybrid_decode_head(q, keys, values, W, tb["offsets"], tb["indices"], 0, L, 2, 0.3, sink, window)
    ref, lse = torch_attention(q, keys, values, 0.3)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    assert abs(r["lse"] - lse) < 1e-12


def brute_hybrid(q, keys, values, W, K, L, T, scale, sink, window):
    """One normaliser over both parts, written out with Python loops."""
    N, d = keys.shape
    def code(x, l):
        c = 0
        for b in range(K):
            p = sum(x[i] * W[i, l * K + b] for i in range(len(x)))
            c |= (1 if p > 0 else 0) << b
        return c
    qc = [code(q, l) for l in range(L)]
    Z, acc = 0.0, np.zeros(d)
    nsel = 0
    for n in range(N):
        s = scale * float(np.dot(q, keys[n]))
        if n < sink or n >= N - window:
            w = math.exp(s)
        else:
            cnt = sum(1 for l in range(L) if code(keys[n], l) == qc[l])
            if cnt < T:
                continue
            nsel += 1
            c = float(np.dot(q, keys[n]) / (np.linalg.norm(q) * np.linalg.norm(keys[n])))
            P = (1.0 - math.acos(max(-1.0, min(1.0, c))) / math.pi) ** K
            u = max(float(scipy.stats.binom.sf(T - 1, L, P)), 1e-30)
            w = math.exp(s) / u
        Z += w
        acc += w * values[n]
    return acc / Z, math.log(Z), nsel


@pytest.mark.parametrize("seed,sink,window", [(4, 2, 5), (5, 0, 9), (6, 6, 0)])
def test_brute_force_hybrid(seed, sink, window):
    q, keys, values, W, tb = tiny_case(seed)
    r = O.hybrid_decode_head(q, keys, values, W, tb["offsets"], tb["indices"], 3, 6, 2, 0.25, sink, window)
    out, lse, nsel = brute_hybrid(q, keys, values, W, 3, 6, 2, 0.25, sink, window)
    np.testing.assert_allclose(r["out"], out, rtol=1e-9, atol=1e-12)
    assert abs(r["lse"] - lse) < 1e-9
    assert r["nsel"] == nsel


def test_brute_force_catches_double_counting(monkeypatch):
    # planted mistake: the sampled part keeps the keys of the exact set too
    def wrong(q, keys, values, W, offsets, indices, K, L, T, scale, n_sink, n_window, qcodes=None):
        r = O.decode_head(q, keys, values, W, offsets, indices, K, L, T, scale, qcodes=qcodes)
        N = np.asarray(keys).shape[0]
        E = O.exact_set(N, n_sink, n_window)
        part_s = O.weighted_softmax_attention(q, keys, values, r["mask"], r["u"], scale)
        part_e = O.weighted_softmax_attention(q, keys, values, E, np.ones(N), scale)
        out, lse = O.lse_merge([part_s, part_e])
        return {"out": out, "lse": lse, "nsel": int(r["mask"].sum())}
    q, keys, values, W, tb = tiny_case(4)
    sel = O.decode_head(q, keys, values, W, tb["offsets"], tb["indices"], 3, 6, 2, 0.25)["mask"]
    sink, window = 2, 5
    assert (sel & O.exact_set(40, sink, window)).any()   # the case overlaps, so the mistake shows
    monkeypatch.setattr(O, "hybrid_decode_head", wrong)
    with pytest.raises(AssertionError):
        test_brute_force_hybrid(4, sink, window)

"""Pins of the estimator-quality harness (oracle/quality.py), CPU only.

TopK and oracle sampling are checked against what fixes them independently
of the code: limits (budget N is exact attention, budget 1 is the argmax
key's value), a point mass, the deterministic count bound of stratified
inverse-CDF sampling, and unbiasedness by Monte Carlo.  A constructed
non-sparse case shows the bias of TopK that the pages argue from, and a
planted mistake (sampling from the wrong distribution) must be caught.
"""

import math

import numpy as np
import pytest

from oracle import lsh_oracle as O
from oracle import quality as Q


def _case(N=64, d=16, seed=0, scale=0.5):
    g = np.random.default_rng(seed)
    return g.standard_normal(d), g.standard_normal((N, d)), g.standard_normal((N, d)), scale


def _softmax_direct(q, keys, values, scale, idx):
    # softmax over the listed keys, written out term by term
    z = [scale * float(np.dot(q, keys[i])) for i in idx]
    m = max(z)
    w = [math.exp(x - m) for x in z]
    s = sum(w)
    return sum(wi / s * values[i] for wi, i in zip(w, idx))


def test_topk_limits():
    q, k, v, s = _case()
    exact, _ = O.exact_attention(q, k, v, s)
    np.testing.assert_allclose(Q.topk_attention(q, k, v, s, len(k)), exact, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Q.topk_attention(q, k, v, s, 10 ** 6), exact, rtol=1e-12, atol=1e-12)
    top = int(np.argmax(k @ q))
    np.testing.assert_allclose(Q.topk_attention(q, k, v, s, 1), v[top], rtol=1e-12)
    assert np.all(Q.topk_attention(q, k, v, s, 0) == 0)


def test_topk_is_softmax_over_the_largest_logits():
    q, k, v, s = _case(N=40, seed=1)
    z = k @ q
    for b in (2, 5, 17):
        idx = sorted(range(len(z)), key=lambda i: -z[i])[:b]
        np.testing.assert_allclose(Q.topk_attention(q, k, v, s, b), _softmax_direct(q, k, v, s, idx),
                                   rtol=1e-10, atol=1e-12)


def test_topk_ties_take_lower_indices():
    d = 4
    k = np.zeros((6, d))
    k[:, 0] = [1, 2, 2, 2, 0, 2]     # four keys tie for the largest logit
    v = np.eye(6)[:, :6]
    q = np.array([1.0, 0, 0, 0])
    out = Q.topk_attention(q, k, v, 1.0, 2)
    np.testing.assert_allclose(out, 0.5 * (v[1] + v[2]), rtol=1e-12)


def test_oracle_sampling_point_mass():
    q, k, v, s = _case(N=30, seed=2)
    k[7] = 50.0 * q / np.linalg.norm(q)     # logit far above every other
    u = np.random.default_rng(3).random(100)
    np.testing.assert_allclose(Q.oracle_sampling_attention(q, k, v, 4.0, u), v[7], rtol=1e-12)


def test_oracle_sampling_stratified_count_bound():
    # stratified uniforms (i + 1/2) / n give every key n p_k samples up to
    # one, so the estimate is within (N / n) max|v| of exact attention
    q, k, v, s = _case(N=50, seed=4)
    exact, _ = O.exact_attention(q, k, v, s)
    for n in (1000, 100000):
        u = (np.arange(n) + 0.5) / n
        est = Q.oracle_sampling_attention(q, k, v, s, u)
        assert np.max(np.abs(est - exact)) <= len(k) / n * np.max(np.abs(v)) + 1e-12


def test_oracle_sampling_unbiased():
    q, k, v, s = _case(N=20, d=8, seed=5)
    exact, _ = O.exact_attention(q, k, v, s)
    g = np.random.default_rng(6)
    reps, n = 4000, 8
    est = np.array([Q.oracle_sampling_attention(q, k, v, s, g.random(n)) for _ in range(reps)])
    sem = est.std(axis=0, ddof=1) / math.sqrt(reps)
    assert np.all(np.abs(est.mean(axis=0) - exact) <= 5 * sem + 1e-12)


def test_topk_biased_when_attention_is_flat():
    # half the keys sit a hair above the rest and carry value +1, the others
    # -1: exact attention is ~0, TopK at half the keys returns +1, sampling
    # is off by about 1/sqrt(budget)
    N, d = 2000, 8
    q = np.zeros(d)
    q[0] = 1.0
    k = np.zeros((N, d))
    k[: N // 2, 0] = 1e-3
    v = np.zeros((N, 1))
    v[: N // 2] = 1.0
    v[N // 2:] = -1.0
    exact, _ = O.exact_attention(q, k, v, 1.0)
    budget = N // 2
    err_topk = abs(Q.topk_attention(q, k, v, 1.0, budget)[0] - exact[0])
    u = np.random.default_rng(8).random(budget)
    err_os = abs(Q.oracle_sampling_attention(q, k, v, 1.0, u)[0] - exact[0])
    assert err_topk > 0.99
    assert err_os < 5.0 / math.sqrt(budget)


def test_compare_head_k0_is_exact():
    # K = 0 keeps every key with u = 1: the LSH "estimate" is exact attention,
    # and TopK at budget N is exact as well
    q, k, v, s = _case(N=100, seed=9)
    W = np.zeros((k.shape[1], 0))
    tables = O.build_tables(k, W, 0, 3, 256)
    r = Q.compare_head(q, k, v, W, tables, 0, 3, 2, s, np.random.default_rng(1).random(100))
    assert r["budget"] == 100
    assert r["lsh"] < 1e-12 and r["topk"] < 1e-12
    assert 0 < r["oracle_sampling"] < 1.0


def test_harness_runs_on_small_workload():
    rows = Q.run(1, units=1, heads=1)
    assert len(rows) == 1
    r = rows[0]
    assert r["budget"] > 0 and all(np.isfinite([r["lsh"], r["topk"], r["oracle_sampling"]]))


def test_planted_wrong_sampling_distribution_is_caught(monkeypatch):
    # sampling uniformly instead of from p must fail the unbiasedness pin
    q, k, v, s = _case(N=20, d=8, seed=5)
    monkeypatch.setattr(Q, "attention_probs", lambda q, keys, scale: np.full(len(keys), 1.0 / len(keys)))
    with pytest.raises(AssertionError):
        test_oracle_sampling_unbiased()

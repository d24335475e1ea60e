"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against mathematics, a library routine it does
not use, brute force, or a hand-worked fixture, so that a plausible mistake
(a dropped term, a wrong sign or index, a transposed operand, a wrong bit
order) fails at least one of them.  ``test_pins_catch_planted_mistakes``
plants such mistakes in the oracle and checks that a pin fails.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import lsh_oracle as O


# ---------------------------------------------------------------- helpers

def pair_at_angle(d, theta, rng):
    """Two vectors in R^d at exactly angle theta (random orientation)."""
    a = rng.standard_normal(d)
    a /= np.linalg.norm(a)
    b = rng.standard_normal(d)
    b -= (b @ a) * a
    b /= np.linalg.norm(b)
    return a * 3.0, (math.cos(theta) * a + math.sin(theta) * b) * 0.5


def brute_codes(x, W, K, L):
    """Bit-by-bit SimHash in plain Python loops."""
    out = []
    for l in range(L):
        row = []
        for n in range(len(x)):
            code = 0
            for b in range(K):
                s = sum(float(x[n][i]) * float(W[i][l * K + b]) for i in range(len(x[n])))
                if s > 0:
                    code |= 1 << b
            row.append(code)
        out.append(row)
    return np.array(out)


# ---------------------------------------------------------------- golden

@pytest.fixture(scope="module")
def gold(golden_dir):
    with open(os.path.join(golden_dir, "hand_worked_tiny.json")) as f:
        return json.load(f)


def test_golden_codes_tables_bounds(gold):
    K, L = gold["K"], gold["L"]
    t = O.build_tables(np.array(gold["keys"], float), np.array(gold["W"], float), K, L, gold["stride"])
    assert t["codes"].tolist() == gold["codes"]
    assert t["offsets"].tolist() == gold["offsets"]
    assert t["indices"].tolist() == gold["indices"]
    assert t["bounds"].tolist() == gold["bounds"]


def test_golden_probe_counts_select(gold):
    K, L = gold["K"], gold["L"]
    t = O.build_tables(np.array(gold["keys"], float), np.array(gold["W"], float), K, L, gold["stride"])
    qc = O.simhash_codes(np.array([gold["q"]], float), np.array(gold["W"], float), K, L)[:, 0]
    assert qc.tolist() == gold["qcodes"]
    cnt = O.collision_counts(qc, t["offsets"], t["indices"], len(gold["keys"]))
    assert cnt.tolist() == gold["counts"]
    assert np.nonzero(O.select(cnt, 1))[0].tolist() == gold["selected_T1"]
    assert np.nonzero(O.select(cnt, 2))[0].tolist() == gold["selected_T2"]


def test_golden_inclusion_and_collision(gold):
    for e in gold["inclusion"]:
        assert O.inclusion_prob(np.array([e["P"]]), e["L"], e["T"])[0] == pytest.approx(e["u"], rel=1e-13)
    for e in gold["collision"]:
        assert O.collision_prob(np.array([e["cos"]]), e["K"])[0] == pytest.approx(e["P"], rel=1e-13)


def test_golden_weighted_softmax(gold):
    e = gold["weighted_softmax"]
    out, lse = O.weighted_softmax_attention(np.array(e["q"], float), np.array(e["keys"], float),
                                            np.array(e["values"], float), np.ones(2, bool),
                                            np.array(e["u"]), e["scale"])
    np.testing.assert_allclose(out, e["out"], rtol=1e-13)
    assert lse == pytest.approx(e["lse"], rel=1e-13)


# ---------------------------------------------------------------- P1: K = 0 is exact attention

@pytest.mark.parametrize("N,L,T", [(257, 4, 2), (1000, 1, 1), (64, 8, 8)])
def test_k0_equals_exact_attention(N, L, T):
    rng = np.random.default_rng(1)
    d = 32
    keys = rng.standard_normal((N, d))
    vals = rng.standard_normal((N, d))
    q = rng.standard_normal(d) * 2
    W = rng.standard_normal((d, 0))
    scale = 1 / math.sqrt(d)
    t = O.build_tables(keys, W, 0, L, 64)
    r = O.decode_head(q, keys, vals, W, t["offsets"], t["indices"], 0, L, T, scale)
    assert r["nsel"] == N and np.all(r["counts"] == L) and np.all(r["u"] == 1.0)
    # independent library: torch's fused attention in float64 on the CPU
    qt = torch.tensor(q)[None, None, None, :]
    kt = torch.tensor(keys)[None, None]
    vt = torch.tensor(vals)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[0, 0, 0].numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    ref_lse = torch.logsumexp(torch.tensor(keys @ q * scale), 0).item()
    assert r["lse"] == pytest.approx(ref_lse, rel=1e-12)


# ---------------------------------------------------------------- P2: SimHash collision rate

@pytest.mark.parametrize("theta", [0.1, 0.5, 1.0, 1.5, 2.0, 3.0])
@pytest.mark.parametrize("K", [1, 3])
def test_simhash_collision_rate(theta, K):
    rng = np.random.default_rng(int(theta * 1000) + K)
    d, M = 16, 20000
    a, b = pair_at_angle(d, theta, rng)
    W = rng.standard_normal((d, K * M))       # M independent tables
    codes = O.simhash_codes(np.stack([a, b]), W, K, M)
    rate = np.mean(codes[:, 0] == codes[:, 1])
    P = (1 - theta / math.pi) ** K
    sigma = math.sqrt(P * (1 - P) / M) + 1e-12
    assert abs(rate - P) < 5 * sigma
    assert O.collision_prob(np.array([math.cos(theta)]), K)[0] == pytest.approx(P, rel=1e-12)


def test_simhash_matches_bitwise_brute_force():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 5))
    W = rng.standard_normal((5, 3 * 4))
    np.testing.assert_array_equal(O.simhash_codes(x, W, 3, 4), brute_codes(x, W, 3, 4))


# ---------------------------------------------------------------- P3: inclusion probability

@pytest.mark.parametrize("L,T", [(1, 1), (8, 2), (32, 2), (150, 2), (120, 2), (150, 1), (150, 150), (20, 7)])
def test_inclusion_prob_vs_scipy(L, T):
    P = np.concatenate([np.logspace(-9, -0.0001, 40), [0.3, 0.5, 0.9, 0.999]])
    u = O.inclusion_prob(P, L, T)
    ref = np.maximum(scipy.stats.binom.sf(T - 1, L, P), O.U_FLOOR)
    np.testing.assert_allclose(u, ref, rtol=1e-10)


def test_inclusion_rate_monte_carlo_through_tables():
    """Empirical P[count >= T] over fresh W draws equals u for a fixed pair."""
    rng = np.random.default_rng(11)
    d, K, L, T, M = 12, 2, 6, 2, 6000
    theta = 1.1
    qv, kv = pair_at_angle(d, theta, rng)
    keys = np.stack([kv, -kv, rng.standard_normal(d)])
    hits = 0
    for _ in range(M):
        W = rng.standard_normal((d, K * L))
        t = O.build_tables(keys, W, K, L, 4)
        qc = O.simhash_codes(qv[None], W, K, L)[:, 0]
        hits += int(O.select(O.collision_counts(qc, t["offsets"], t["indices"], 3), T)[0])
    u = O.inclusion_prob(O.collision_prob(np.array([math.cos(theta)]), K), L, T)[0]
    sigma = math.sqrt(u * (1 - u) / M)
    assert abs(hits / M - u) < 5 * sigma


# ---------------------------------------------------------------- P4: Horvitz-Thompson unbiasedness

def _ht_terms(rng, keys, vals, q, K, L, T, scale, M):
    num = np.zeros((M, vals.shape[1]))
    den = np.zeros(M)
    d = keys.shape[1]
    for m in range(M):
        W = rng.standard_normal((d, K * L))
        t = O.build_tables(keys, W, K, L, 16)
        r = O.decode_head(q, keys, vals, W, t["offsets"], t["indices"], K, L, T, scale)
        z = math.exp(r["lse"]) if np.isfinite(r["lse"]) else 0.0
        num[m] = r["out"] * z
        den[m] = z
    return num, den


def test_horvitz_thompson_unbiased():
    rng = np.random.default_rng(5)
    N, d, K, L, T, M = 24, 8, 2, 6, 2, 3000
    keys = rng.standard_normal((N, d))
    vals = rng.standard_normal((N, d))
    q = keys[3] * 0.8 + rng.standard_normal(d) * 0.3
    scale = 0.5
    num, den = _ht_terms(rng, keys, vals, q, K, L, T, scale, M)
    e = np.exp(scale * keys @ q)
    for est, truth in [(den, e.sum())] + [(num[:, i], (e @ vals)[i]) for i in range(d)]:
        se = est.std(ddof=1) / math.sqrt(M)
        assert abs(est.mean() - truth) < 5 * se + 1e-12


# ---------------------------------------------------------------- P5: brute force on tiny inputs

@pytest.mark.parametrize("seed", range(6))
def test_tiny_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    N = int(rng.integers(1, 64))
    d = int(rng.integers(2, 7))
    K = int(rng.integers(0, 5))
    L = int(rng.integers(1, 9))
    stride = int(rng.choice([1, 2, 4, 8, 16, 64]))
    keys = rng.standard_normal((N, d))
    if N > 3:
        keys[1] = 0.0                        # a zero key
    W = rng.standard_normal((d, K * L))
    q = rng.standard_normal(d)
    t = O.build_tables(keys, W, K, L, stride)
    codes = brute_codes(keys, W, K, L)
    np.testing.assert_array_equal(t["codes"], codes)
    nb = 1 << K
    for l in range(L):
        buckets = [[n for n in range(N) if codes[l][n] == c] for c in range(nb)]
        flat = [n for bkt in buckets for n in bkt]
        assert t["indices"][l].tolist() == flat
        pos = 0
        for c in range(nb):
            assert t["offsets"][l][c] == pos
            for j in range((N + stride - 1) // stride + 1):
                lim = min(j * stride, N)
                first = pos + sum(1 for n in buckets[c] if n < lim)
                assert t["bounds"][l][c][j] == first
            pos += len(buckets[c])
        assert t["offsets"][l][nb] == N
    qc = brute_codes(q[None], W, K, L)[:, 0]
    cnt = O.collision_counts(qc, t["offsets"], t["indices"], N)
    direct = [sum(1 for l in range(L) if codes[l][n] == qc[l]) for n in range(N)]
    assert cnt.tolist() == direct


# ---------------------------------------------------------------- P6: closed forms

def test_closed_forms():
    P = np.array([1e-6, 0.01, 0.2, 0.5, 0.77, 0.999])
    for L in (1, 5, 150):
        np.testing.assert_allclose(O.inclusion_prob(P, L, 1), 1 - (1 - P) ** L, rtol=1e-10)
        np.testing.assert_allclose(O.inclusion_prob(P, L, L), np.maximum(P ** L, O.U_FLOOR), rtol=1e-10)
    np.testing.assert_allclose(O.inclusion_prob(P, 1, 1), P, rtol=1e-12)
    # T = 2: 1 - (1-P)^L - L P (1-P)^(L-1), checked where it does not cancel
    Pm = np.array([0.05, 0.2, 0.5])
    np.testing.assert_allclose(O.inclusion_prob(Pm, 150, 2),
                               1 - (1 - Pm) ** 150 - 150 * Pm * (1 - Pm) ** 149, rtol=1e-9)
    assert O.inclusion_prob(np.array([1.0]), 150, 2)[0] == 1.0          # theta = 0
    for K in (1, 4, 10):
        assert O.collision_prob(np.array([0.0]), K)[0] == pytest.approx(2.0 ** -K, rel=1e-14)
        assert O.collision_prob(np.array([1.0]), K)[0] == 1.0
        assert O.collision_prob(np.array([-1.0]), K)[0] == 0.0
    assert O.inclusion_prob(np.array([0.0]), 150, 2)[0] == O.U_FLOOR      # clamp


# ---------------------------------------------------------------- P7: invariants

def test_invariants():
    rng = np.random.default_rng(21)
    N, d, K, L = 300, 16, 4, 12
    keys = rng.standard_normal((N, d))
    vals = rng.standard_normal((N, d))
    W = rng.standard_normal((d, K * L))
    q = keys[7] + 0.5 * rng.standard_normal(d)
    t = O.build_tables(keys, W, K, L, 64)
    for l in range(L):
        assert sorted(t["indices"][l].tolist()) == list(range(N))
        assert t["offsets"][l][-1] == N and np.all(np.diff(t["offsets"][l]) >= 0)
    # scaling by powers of two leaves codes bit-identical
    for j in (-3, 5):
        np.testing.assert_array_equal(O.simhash_codes(keys * 2.0 ** j, W, K, L), t["codes"])
    r = {T: O.decode_head(q, keys, vals, W, t["offsets"], t["indices"], K, L, T, 0.25) for T in (1, 2, 3, 5)}
    assert np.all((r[1]["counts"] >= 0) & (r[1]["counts"] <= L))
    for a, b in [(1, 2), (2, 3), (3, 5)]:
        assert np.all(r[b]["mask"] <= r[a]["mask"])                      # S shrinks as T grows
    # permuting keys and values relabels S and leaves out unchanged
    perm = rng.permutation(N)
    t2 = O.build_tables(keys[perm], W, K, L, 64)
    r2 = O.decode_head(q, keys[perm], vals[perm], W, t2["offsets"], t2["indices"], K, L, 2, 0.25)
    np.testing.assert_array_equal(r2["mask"], r[2]["mask"][perm])
    np.testing.assert_allclose(r2["out"], r[2]["out"], rtol=1e-12)
    assert r2["lse"] == pytest.approx(r[2]["lse"], rel=1e-12)


# ---------------------------------------------------------------- P8: convex combination

def test_output_is_convex_combination():
    rng = np.random.default_rng(31)
    N, d, K, L, T = 500, 8, 3, 10, 2
    keys = rng.standard_normal((N, d))
    vals = rng.standard_normal((N, d))
    W = rng.standard_normal((d, K * L))
    q = keys[0] * 2
    t = O.build_tables(keys, W, K, L, 128)
    r = O.decode_head(q, keys, vals, W, t["offsets"], t["indices"], K, L, T, 1.0)
    S = vals[r["mask"]]
    assert r["nsel"] > 0
    assert np.all(r["out"] >= S.min(0) - 1e-12) and np.all(r["out"] <= S.max(0) + 1e-12)


# ---------------------------------------------------------------- P9: empty selection

def test_empty_selection():
    rng = np.random.default_rng(41)
    N, d, K, L = 200, 16, 6, 8
    keys = rng.standard_normal((N, d))
    vals = rng.standard_normal((N, d))
    W = rng.standard_normal((d, K * L))
    t = O.build_tables(keys, W, K, L, 64)
    # T = L with a query no key shares all L codes with
    for s in range(50):
        q = rng.standard_normal(d)
        r = O.decode_head(q, keys, vals, W, t["offsets"], t["indices"], K, L, L, 1.0)
        if r["nsel"] == 0:
            break
    assert r["nsel"] == 0 and np.all(r["out"] == 0) and r["lse"] == -np.inf


# ---------------------------------------------------------------- LSE merge

def test_lse_merge_equals_union():
    rng = np.random.default_rng(51)
    N, d = 400, 8
    keys = rng.standard_normal((N, d))
    vals = rng.standard_normal((N, d))
    q = rng.standard_normal(d)
    u = rng.uniform(0.05, 1.0, N)
    mask = rng.random(N) < 0.4
    whole = O.weighted_softmax_attention(q, keys, vals, mask, u, 0.7)
    parts = []
    for lo in range(0, N, 64):
        m = np.zeros(N, bool)
        m[lo:lo + 64] = mask[lo:lo + 64]
        parts.append(O.weighted_softmax_attention(q, keys, vals, m, u, 0.7))
    parts.append((np.zeros(d), -np.inf))
    out, lse = O.lse_merge(parts)
    np.testing.assert_allclose(out, whole[0], rtol=1e-12)
    assert lse == pytest.approx(whole[1], rel=1e-12)
    # reference via scipy's logsumexp over the selected logits
    sel = np.nonzero(mask)[0]
    assert lse == pytest.approx(scipy.special.logsumexp(0.7 * keys[sel] @ q - np.log(u[sel])), rel=1e-12)


# ---------------------------------------------------------------- the pins catch planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch, gold):
    """Plant plausible mistakes in the oracle (CPU) and check a pin fails."""
    # 1. u = P (single-table probability) instead of the binomial tail
    monkeypatch.setattr(O, "inclusion_prob", lambda P, L, T: np.maximum(np.asarray(P, float), O.U_FLOOR))
    with pytest.raises(AssertionError):
        test_horvitz_thompson_unbiased()
    monkeypatch.undo()

    # 2. wrong sign of ln u in the logits
    real = O.weighted_softmax_attention

    def flipped(q, keys, values, mask, u, scale):
        return real(q, keys, values, mask, 1.0 / np.asarray(u, float), scale)
    monkeypatch.setattr(O, "weighted_softmax_attention", flipped)
    with pytest.raises(AssertionError):
        test_golden_weighted_softmax(gold)
    monkeypatch.undo()

    # 3. reversed bit order in the codes
    real_codes = O.simhash_codes

    def reversed_bits(x, W, K, L):
        c = real_codes(x, W, K, L)
        out = np.zeros_like(c)
        for b in range(K):
            out |= ((c >> b) & 1) << (K - 1 - b)
        return out
    monkeypatch.setattr(O, "simhash_codes", reversed_bits)
    with pytest.raises(AssertionError):
        test_golden_codes_tables_bounds(gold)
    monkeypatch.undo()

    # 4. unstable (descending) order inside buckets
    real_tables = O.bucket_tables

    def descending(codes, K):
        off, idx = real_tables(codes, K)
        for l in range(idx.shape[0]):
            for c in range(off.shape[1] - 1):
                idx[l, off[l, c]:off[l, c + 1]] = idx[l, off[l, c]:off[l, c + 1]][::-1]
        return off, idx
    monkeypatch.setattr(O, "bucket_tables", descending)
    with pytest.raises(AssertionError):
        test_tiny_brute_force(0)
    monkeypatch.undo()

    # 5. sign rule with ties counted as 1 (proj >= 0)
    def ge_codes(x, W, K, L):
        x = np.asarray(x, dtype=np.float64)
        codes = np.zeros((L, x.shape[0]), dtype=np.int64)
        if K == 0:
            return codes
        bits = (x @ np.asarray(W, np.float64) >= 0.0).astype(np.int64)
        for l in range(L):
            for b in range(K):
                codes[l] += bits[:, l * K + b] << b
        return codes
    monkeypatch.setattr(O, "simhash_codes", ge_codes)
    with pytest.raises(AssertionError):
        test_golden_codes_tables_bounds(gold)
    monkeypatch.undo()

    # 6. the K-th power dropped from the collision probability
    real_cp = O.collision_prob
    monkeypatch.setattr(O, "collision_prob", lambda cos, K: real_cp(cos, 1))
    with pytest.raises(AssertionError):
        test_golden_inclusion_and_collision(gold)
    monkeypatch.undo()

    # 7. strict threshold (count > T) in the selection
    monkeypatch.setattr(O, "select", lambda counts, T: np.asarray(counts) > T)
    with pytest.raises(AssertionError):
        test_golden_probe_counts_select(gold)
    monkeypatch.undo()

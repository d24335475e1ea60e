"""Estimator quality of LSH sampling against its baselines (fp64, CPU).

TEST INFRASTRUCTURE ONLY, like ``lsh_oracle``: only ``tests/`` and this
module's own command line use it; nothing in the library calls it.

MagicPIG's case is that attention is not always sparse, so keeping the
top-k keys can be a biased approximation, while sampling keys and weighting
them estimates the output without that bias ("Summary of MagicPIG: LSH
Sampling for Efficient LLM Generation", GrooveSquid, medium-difficulty
summary).  The project evaluates against a TopK baseline and against oracle
sampling, i.e. sampling from the exact attention distribution itself ("How
infini-ai-lab/magicpig works", evaluation components: TopK baseline and
oracle-sampling cache).  This module puts the three estimators side by side
on the same query, keys and values, at the same budget:

  * LSH sampling: ``lsh_oracle.decode_head`` (its budget is |S|, the number
    of keys it selects);
  * TopK: exact softmax attention restricted to the ``budget`` keys with the
    largest logits, renormalised over them;
  * oracle sampling: ``budget`` keys drawn independently from the exact
    attention distribution p (with replacement); the estimate is the mean of
    their values, an unbiased estimate of sum_n p_n v_n.

Random draws are inputs: ``oracle_sampling_attention`` takes the uniforms it
maps through the inverse CDF of p.  Errors are relative L2 distances to exact
attention.  ``python -m oracle.quality`` prints a table over the synthetic
workloads.
"""

from __future__ import annotations

import argparse
import math

import numpy as np

from oracle import lsh_oracle as O


def attention_logits(q, keys, scale):
    """s * q.k_n for every key: q [d], keys [N, d] -> [N] (float64)."""
    return scale * (np.asarray(keys, np.float64) @ np.asarray(q, np.float64))


def attention_probs(q, keys, scale):
    """The exact attention distribution p = softmax(s q.k) over all keys."""
    z = attention_logits(q, keys, scale)
    z = z - z.max()
    p = np.exp(z)
    return p / p.sum()


def topk_attention(q, keys, values, scale, budget):
    """Softmax attention over the ``budget`` keys with the largest logits
    (ties to the lower key index), renormalised over that set."""
    z = attention_logits(q, keys, scale)
    N = z.shape[0]
    b = int(min(max(budget, 0), N))
    if b == 0:
        return np.zeros(np.asarray(values).shape[1])
    # stable order: by logit descending, then by index ascending
    order = np.lexsort((np.arange(N), -z))
    keep = order[:b]
    w = np.exp(z[keep] - z[keep].max())
    w /= w.sum()
    return w @ np.asarray(values, np.float64)[keep]


def oracle_sampling_attention(q, keys, values, scale, uniforms):
    """Mean of the values of keys drawn from p by inverse CDF: sample i is
    the smallest n with cumsum(p)[n] > uniforms[i] (uniforms in [0, 1))."""
    p = attention_probs(q, keys, scale)
    cdf = np.cumsum(p)
    cdf[-1] = 1.0
    u = np.asarray(uniforms, np.float64)
    if u.size == 0:
        return np.zeros(np.asarray(values).shape[1])
    idx = np.searchsorted(cdf, u, side="right")
    idx = np.minimum(idx, len(p) - 1)
    return np.asarray(values, np.float64)[idx].mean(axis=0)


def rel_err(est, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(np.asarray(est, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def compare_head(q, keys, values, W, tables, K, L, T, scale, uniforms):
    """The three estimators on one query head at the LSH selection's budget.

    ``tables`` is ``lsh_oracle.build_tables`` of these keys; ``uniforms`` has
    at least |S| entries (the first |S| are used).  Returns a dict of the
    budget, the sparsity of p (how many keys hold 90% of its mass) and the
    three relative errors."""
    exact, _ = O.exact_attention(q, keys, values, scale)
    r = O.decode_head(q, keys, values, W, tables["offsets"], tables["indices"], K, L, T, scale)
    budget = r["nsel"]
    p = np.sort(attention_probs(q, keys, scale))[::-1]
    k90 = int(np.searchsorted(np.cumsum(p), 0.9) + 1)
    return {
        "budget": budget,
        "keys_for_90pct": k90,
        "lsh": rel_err(r["out"], exact) if budget else float("nan"),
        "topk": rel_err(topk_attention(q, keys, values, scale, budget), exact) if budget else float("nan"),
        "oracle_sampling": (rel_err(oracle_sampling_attention(q, keys, values, scale, uniforms[:budget]), exact)
                            if budget else float("nan")),
    }


def run(cfg_id, units=1, heads=4, seed=7):
    """Compare the estimators on the first ``heads`` query heads of the
    first ``units`` (sequence, kv head) units of a synthetic workload."""
    import workloads

    cfg = workloads.CONFIGS[cfg_id]
    data = workloads.generate(cfg)
    W = data["W"].double().numpy()
    q = data["q"][0].double().numpy()
    g = np.random.default_rng(seed)
    rows = []
    for ui in range(units):
        b, gkv = divmod(ui, cfg.Hkv)
        keys = data["keys"][b, gkv].double().numpy()
        vals = data["values"][b, gkv].double().numpy()
        tables = O.build_tables(keys, W, cfg.K, cfg.L, cfg.N)
        for h in range(gkv * cfg.G, gkv * cfg.G + min(heads, cfg.G)):
            res = compare_head(q[b, h], keys, vals, W, tables, cfg.K, cfg.L, cfg.T, cfg.scale,
                               g.random(cfg.N))
            res.update({"workload": cfg.name, "b": b, "h": h})
            rows.append(res)
    return rows


def main():
    ap = argparse.ArgumentParser(description="LSH sampling vs TopK vs oracle sampling (relative L2 to exact)")
    ap.add_argument("--configs", type=int, nargs="+", default=[1, 2, 3])
    ap.add_argument("--units", type=int, default=1)
    ap.add_argument("--heads", type=int, default=4)
    args = ap.parse_args()
    print("| workload | (b, h) | budget |S| | keys for 90% of p | LSH | TopK | oracle sampling |")
    print("|---|---|---|---|---|---|---|")
    for c in args.configs:
        for r in run(c, args.units, args.heads):
            print(f"| {r['workload']} | ({r['b']}, {r['h']}) | {r['budget']} | {r['keys_for_90pct']} | "
                  f"{r['lsh']:.3f} | {r['topk']:.3f} | {r['oracle_sampling']:.3f} |", flush=True)


if __name__ == "__main__":
    main()

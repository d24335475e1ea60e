"""Parity on a seeded sweep of small random configurations.

Each case draws its shape and parameters from a fixed seed: batch, GQA ratio,
key count (ragged, across chunk boundaries), K, L, T, dtype, chunk stride,
key offset, an optional exact set and optional per-sequence lengths, so the
sweep covers combinations the hand-picked cases do not.  Every case is
compared with the oracle in full (tables, counts, selection, outputs).
"""

import numpy as np
import pytest

import workloads
from test_gpu_cache import grow, say

pytestmark = pytest.mark.gpu

N_CASES = 16


def draw(i):
    r = np.random.default_rng(9000 + i)
    Hkv = int(r.choice([1, 2, 3]))
    G = int(r.choice([1, 2, 4, 8, 16]))
    B = int(r.integers(1, 4))
    N = int(r.integers(40, 5000))
    K = int(r.choice([2, 3, 5, 7, 8, 9, 10, 11, 13]))
    L = int(r.integers(1, 40))
    T = int(r.integers(1, min(L, 4) + 1))
    dtype = "f32" if r.random() < 0.25 else "bf16"
    stride = int(r.choice([256, 512, 1024, 4096, 8192]))
    offset = str(r.choice(["none", "per_head", "per_unit"]))
    cfg = workloads.Config(f"rand{i}", B=B, Hq=Hkv * G, Hkv=Hkv, N=N, d=128, K=K, L=L, T=T, dtype=dtype,
                           planted=int(r.integers(1, 5)), a=float(r.uniform(0.5, 0.95)), offset=offset,
                           seed=7000 + i)
    hybrid = r.random() < 0.5
    n_sink = int(r.integers(0, 9)) if hybrid else 0
    n_window = int(r.integers(0, 300)) if hybrid else 0
    if r.random() < 0.5:
        # ragged: every sequence at its own length, grown in two steps
        first = [int(x) for x in r.integers(0, N + 1, size=B)]
        second = [int(min(N, f + r.integers(0, 700))) for f in first]
        schedule = [first, second]
    else:
        schedule = [N]
    return cfg, stride, n_sink, n_window, schedule


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    cfg, stride, n_sink, n_window, schedule = draw(i)
    say(f"case random {i}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} N={cfg.N} K={cfg.K} L={cfg.L} T={cfg.T} "
        f"{cfg.dtype} stride={stride} offset={cfg.offset} sink={n_sink} window={n_window} schedule={schedule}")
    grow(cfg, schedule, stride=stride, n_sink=n_sink, n_window=n_window)

"""Direct pin of the device's ln u (the 1/u importance weight) on a dense
angle grid, through the real decode kernels.

The weight is u = P[Binomial(L, P) >= T] with P = (1 - theta/pi)^K and theta
the query-key angle, clamped at u >= 1e-30 (the Horvitz-Thompson reading of
the pages' importance-weighted estimate: GrooveSquid summary of MagicPIG,
medium-difficulty summary; sourcepulse "How It Works").  The GPU evaluates it
from an fp32 arccos, a table of interval quadratics of the binomial-tail
correction and the hardware log; the oracle sums the tail in fp64.

How the test isolates ln u:
  * W = 0 makes every projection exactly 0, so every key and query code is 0
    (a zero projection gives bit 0) and every key collides in all L tables:
    the selection no longer depends on chance, whatever the angle;
  * each (sequence, kv head) holds ONE key and sm_scale = 0, so each query
    head's log-sum-exp is the single logit 0 * q.k - ln u: -lse is the
    device's ln u of that (query head, key) pair.
Angles cover [0, pi] densely, with extra points towards theta -> 0 and
theta -> pi, where 1/u is largest and the 1e-30 floor is reached.

Tolerance: the device computes the cosine in fp32 from bf16 (or fp32)
inputs, so its ln u is compared with the oracle's at the exact cosine of the
same inputs, allowing for (a) the function's own error, a few 1e-6 relative
to the magnitudes of its two parts T K ln p and g, plus 2e-5, and (b) the
cosine's fp32 rounding, propagated through the oracle's ln u: the largest
change of the fp64 ln u over [c - dc, c + dc], with dc the rounding bound of
the input layout (a few ulp for keys on a coordinate axis, where the dot
product and the key norm are exact; the worst-case bound of a 128-term fp32
dot product for dense vectors).
"""

import math
import sys

import numpy as np
import pytest
import torch

from oracle import lsh_oracle as O

pytestmark = pytest.mark.gpu

D = 128
HKV = 8
G = 16
HQ = HKV * G


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def angle_grid(rng, n):
    """n angles in [0, pi]: a uniform grid, geometric approach to both ends,
    the exact ends and pi/2, and random fill."""
    parts = [np.linspace(0.0, math.pi, 1025),
             math.pi - np.logspace(-7, 0, 240),
             np.logspace(-7, 0, 120),
             np.array([0.0, math.pi / 2, math.pi])]
    th = np.concatenate(parts)
    th = np.clip(th, 0.0, math.pi)
    if len(th) < n:
        th = np.concatenate([th, rng.uniform(0.0, math.pi, n - len(th))])
    return th[:n]


def make_pairs(layout, thetas, dtype, rng):
    """keys [B, HKV, 1, D] and q [B, HQ, D] (torch, CPU, ``dtype``) such that
    query head h of sequence b meets its unit's key at angle thetas[b * HQ + h]
    (before rounding to ``dtype``)."""
    n = len(thetas)
    B = n // HQ
    U = B * HKV
    keys = np.zeros((U, D))
    q = np.zeros((U, G, D))
    th = thetas.reshape(U, G)
    if layout == "axis":
        # key on axis a (a power-of-two length), query in the plane of axes a, b
        for u in range(U):
            a = u % D
            b = (a + 1 + (u // D) % (D - 1)) % D
            keys[u, a] = 2.0 ** ((u % 5) - 2)
            scale = 2.0 ** ((np.arange(G) % 3) - 1)
            q[u, :, a] = np.cos(th[u]) * scale
            q[u, :, b] = np.sin(th[u]) * scale
    else:
        # dense Gaussian key, query at the angle in a random plane through it
        k = rng.standard_normal((U, D))
        keys[:] = k
        kh = k / np.linalg.norm(k, axis=1, keepdims=True)
        w = rng.standard_normal((U, G, D))
        w -= (w * kh[:, None, :]).sum(-1, keepdims=True) * kh[:, None, :]
        w /= np.linalg.norm(w, axis=-1, keepdims=True)
        q[:] = 3.0 * (np.cos(th)[..., None] * kh[:, None, :] + np.sin(th)[..., None] * w)
    kt = torch.from_numpy(keys).to(dtype).reshape(B, HKV, 1, D)
    qt = torch.from_numpy(q).to(dtype).reshape(B, HQ, D)
    return kt, qt


def oracle_lnu(c, K, L, T):
    return np.log(O.inclusion_prob(O.collision_prob(np.clip(c, -1.0, 1.0), K), L, T))


def exact_cosines(kt, qt):
    """fp64 cosine of every (query head, its unit's key) pair of the rounded inputs."""
    k = kt.double().numpy()[:, :, 0, :]                     # [B, HKV, D]
    q = qt.double().numpy().reshape(k.shape[0], HKV, G, D)  # [B, HKV, G, D]
    dots = np.einsum("bgd,bghd->bgh", k, q)
    nrm = np.linalg.norm(k, axis=-1)[..., None] * np.linalg.norm(q, axis=-1)
    return np.clip(np.where(nrm > 0, dots / np.where(nrm > 0, nrm, 1.0), 0.0), -1.0, 1.0).reshape(-1)


# (K, L, T): the workloads' settings, K = 15, T = L, T = 1, a mid-range T of a
# large L, L = 255, and the single-table case u = p
CASES = [
    (10, 150, 2, "bf16", "axis"),
    (10, 150, 2, "bf16", "dense"),
    (9, 120, 2, "bf16", "axis"),
    (8, 32, 2, "f32", "axis"),
    (8, 32, 2, "f32", "dense"),
    (15, 4, 4, "bf16", "axis"),
    (15, 255, 2, "bf16", "dense"),
    (1, 1, 1, "bf16", "axis"),
    (3, 255, 1, "bf16", "axis"),
    (6, 200, 100, "bf16", "axis"),
    (12, 255, 255, "bf16", "axis"),
    (2, 17, 9, "f32", "axis"),
    (4, 255, 200, "bf16", "dense"),
]


@pytest.mark.parametrize("K,L,T,dt,layout", CASES, ids=[f"K{c[0]}-L{c[1]}-T{c[2]}-{c[3]}-{c[4]}" for c in CASES])
def test_device_lnu_grid(K, L, T, dt, layout):
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    say(f"case lnu K={K} L={L} T={T} {dt} {layout}")
    rng = np.random.default_rng(1000 + 7 * K + L + 3 * T)
    B = 16
    thetas = angle_grid(rng, B * HQ)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    kt, qt = make_pairs(layout, thetas, tdt, rng)
    dev = torch.device("cuda:0")
    keys = kt.to(dev)
    vals = torch.zeros_like(keys)
    vals[..., 0] = 1.0
    q = qt.to(dev)
    W = torch.zeros(D, L * K, dtype=tdt, device=dev)
    tb = lsh.build_tables(keys, W, K, L)
    r = lsh.decode_attention(q, keys, vals, W, tb, K, L, T, sm_scale=0.0, return_counts=True)
    torch.cuda.synchronize()
    counts = r["counts"].cpu().numpy().reshape(-1)
    assert np.all(counts == L), "W = 0 must make every key collide in every table"
    assert np.all(r["nsel"].cpu().numpy() == 1)
    gpu = -r["lse"].cpu().double().numpy().reshape(-1)

    c = exact_cosines(kt, qt)
    ref = oracle_lnu(c, K, L, T)
    # fp32 rounding bound of the device's cosine for this input layout
    dc = (6e-7 * np.abs(c)) if layout == "axis" else np.full_like(c, 1.6e-5)
    cond = np.maximum(np.abs(oracle_lnu(c + dc, K, L, T) - ref), np.abs(oracle_lnu(c - dc, K, L, T) - ref))
    theta = np.arccos(c)
    lnp = np.log(np.maximum(1.0 - theta / math.pi, 1e-300))
    mag = abs(math.lgamma(L + 1) - math.lgamma(T + 1) - math.lgamma(L - T + 1)) + T * K * np.minimum(np.abs(lnp), 1e3)
    tol = 2e-5 + 4e-6 * mag + cond
    err = np.abs(gpu - ref)
    floored = ref <= math.log(O.U_FLOOR) + 1e-12
    well = cond < 1e-6
    worst = int(np.argmax(err - tol))
    say(f"  pairs={len(c)} max|dlnu|={err.max():.3e} max|dlnu| where cond<1e-6: "
        f"{err[well].max() if well.any() else float('nan'):.3e} (pairs {int(well.sum())}) "
        f"floored={int(floored.sum())} worst: theta={theta[worst]:.6g} ref={ref[worst]:.6g} "
        f"gpu={gpu[worst]:.6g} tol={tol[worst]:.3e}")
    assert floored.any(), "the grid must reach the 1e-30 floor"
    assert np.all(np.abs(gpu[floored] - math.log(O.U_FLOOR)) <= 1e-5 + cond[floored])
    assert np.all(err <= tol), (f"ln u off at theta={theta[worst]:.8g}: gpu {gpu[worst]:.8g} "
                                f"oracle {ref[worst]:.8g} tol {tol[worst]:.3e}")

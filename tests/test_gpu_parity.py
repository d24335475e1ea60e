"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Small cases span several projection tiles, several key chunks and a ragged
tail and are checked in full; the workload configurations are run at full
size in the launch configuration the benchmark uses and checked on sampled
(sequence, kv head) units, which the oracle recomputes from the same inputs.
"""

import math
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import lsh_oracle as O
import parity as PAR

pytestmark = pytest.mark.gpu


def _lsh():
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    return lsh


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(cfg, data, stride=None, step=0, n_sink=0, n_window=0):
    """Build + one decode step on the GPU (the hybrid decode when n_sink or
    n_window is set)."""
    lsh = _lsh()
    dev = torch.device("cuda:0")
    keys = data["keys"].to(dev)
    vals = data["values"].to(dev)
    W = data["W"].to(dev)
    q = data["q"][step].to(dev).contiguous()
    if cfg.K == 0:
        W = torch.empty(cfg.d, 0, dtype=keys.dtype, device=dev)
    tb = lsh.build_tables(keys, W, cfg.K, cfg.L, stride=stride, return_codes=True)
    r = lsh.decode_attention(q, keys, vals, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale,
                             return_codes=True, return_counts=True, n_sink=n_sink, n_window=n_window)
    torch.cuda.synchronize()
    return tb, r


def to_np(t):
    return t.detach().cpu().numpy()


def check_case(cfg, data, units=None, heads_per_unit=None, stride=None, step=0, n_sink=0, n_window=0):
    """Full comparison on the listed units (default: all)."""
    hybrid = bool(n_sink or n_window)
    tb, r = run_gpu(cfg, data, stride=stride, step=step, n_sink=n_sink, n_window=n_window)
    stride = tb["stride"]
    W = data["W"].float().cpu().numpy() if cfg.K > 0 else np.zeros((cfg.d, 0))
    q = data["q"][step].float().cpu().numpy()
    if units is None:
        units = [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    total_bits = flips = bad_tables = 0
    rels, est = [], []
    G = cfg.G
    for (b, g) in units:
        ku = data["keys"][b, g].float().cpu().numpy()
        vu = data["values"][b, g].float().cpu().numpy()
        ref = O.build_tables(ku, W, cfg.K, cfg.L, stride)
        band = PAR.band_mask(ku, W) if cfg.K > 0 else np.zeros((cfg.N, 0), bool)
        gcodes = to_np(tb["codes"][b, g])
        flips += PAR.compare_codes(gcodes, ref["codes"], band, cfg.K, cfg.L)
        total_bits += cfg.N * cfg.L * cfg.K
        bad_tables += PAR.check_tables(to_np(tb["offsets"][b, g]), to_np(tb["indices"][b, g]),
                                       gcodes, ref, cfg.K, stride)
        hs = list(range(g * G, (g + 1) * G))
        nh = heads_per_unit.get((b, g)) if isinstance(heads_per_unit, dict) else heads_per_unit
        if nh is not None:
            hs = hs[:nh]
        for h in hs:
            if hybrid:
                rr = O.hybrid_decode_head(q[b, h], ku, vu, W, ref["offsets"], ref["indices"],
                                          cfg.K, cfg.L, cfg.T, cfg.scale, n_sink, n_window)
            else:
                rr = O.decode_head(q[b, h], ku, vu, W, ref["offsets"], ref["indices"],
                                   cfg.K, cfg.L, cfg.T, cfg.scale)
            qb = PAR.band_mask(q[b, h][None], W) if cfg.K > 0 else np.zeros((1, 0), bool)
            gh = {"q_codes": to_np(r["q_codes"][b, h]), "counts": to_np(r["counts"][b, h]),
                  "out": to_np(r["out"][b, h]), "lse": float(r["lse"][b, h]), "nsel": int(r["nsel"][b, h])}
            res = PAR.check_head(gh, rr, qb, gcodes, ref["codes"], cfg.K, cfg.L, cfg.T,
                                 exact=rr.get("exact"))
            flips += res["qflips"]
            total_bits += cfg.L * cfg.K
            rels.append(res["rel"])
            if rr["nsel"] > 0 or hybrid:
                est.append(PAR.estimate_error(gh["out"], O.exact_attention(q[b, h], ku, vu, cfg.scale)))
    if total_bits:
        assert flips <= max(1.0, PAR.FLIP_FRACTION_MAX * total_bits), (flips, total_bits)
    say(f"[{cfg.name}{f' sink={n_sink} window={n_window}' if hybrid else ''}] units={len(units)} flips={flips}/{total_bits} bad_tables={bad_tables} "
        f"max_rel={max(rels) if rels else 0:.2e} est_err_vs_exact={np.mean(est) if est else float('nan'):.3e}")
    return tb, r


SMALL = [
    workloads.CONFIGS[1],
    workloads.Config("ragged-gqa3", B=2, Hq=6, Hkv=2, N=5000, d=128, K=6, L=20, T=2, dtype="bf16",
                     planted=4, a=0.8, offset="per_head", seed=11),
    workloads.Config("gqa8-t3", B=1, Hq=16, Hkv=2, N=3000, d=128, K=8, L=40, T=3, dtype="bf16",
                     planted=8, a=0.7, offset="shared_lowrank", seed=12),
    workloads.Config("gqa16-t1", B=1, Hq=16, Hkv=1, N=2100, d=128, K=5, L=10, T=1, dtype="bf16",
                     planted=2, a=0.8, offset="none", seed=13),
    workloads.Config("fp32-multi", B=2, Hq=4, Hkv=2, N=1500, d=128, K=7, L=24, T=2, dtype="f32",
                     planted=3, a=0.8, offset="per_unit", seed=14),
    workloads.Config("n63", B=1, Hq=2, Hkv=1, N=63, d=128, K=4, L=8, T=1, dtype="bf16",
                     planted=1, a=0.9, offset="none", seed=15),
    workloads.Config("n1", B=1, Hq=2, Hkv=2, N=1, d=128, K=3, L=5, T=1, dtype="bf16",
                     planted=1, a=0.9, offset="none", seed=16),
    workloads.Config("T-eq-L", B=1, Hq=4, Hkv=1, N=700, d=128, K=8, L=8, T=8, dtype="bf16",
                     planted=1, a=0.3, offset="none", seed=17),
    workloads.Config("L1", B=1, Hq=3, Hkv=1, N=900, d=128, K=3, L=1, T=1, dtype="bf16",
                     planted=1, a=0.8, offset="none", seed=18),
    workloads.Config("K15", B=1, Hq=2, Hkv=1, N=2048, d=128, K=15, L=4, T=1, dtype="bf16",
                     planted=1, a=0.95, offset="none", seed=19),
    workloads.Config("K12-odd", B=1, Hq=4, Hkv=1, N=9001, d=128, K=12, L=6, T=1, dtype="bf16",
                     planted=2, a=0.9, offset="none", seed=20),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_full_parity(cfg):
    say(f"case {cfg.name}")
    data = workloads.generate(cfg)
    check_case(cfg, data)


@pytest.mark.parametrize("stride", [256, 1024, 8192])
def test_strides(stride):
    cfg = SMALL[1]
    say(f"case strides {stride}")
    data = workloads.generate(cfg)
    check_case(cfg, data, stride=stride)


def test_zero_keys():
    # all-zero key rows: every projection is exactly zero (no flip band), so
    # their codes must be 0, and their cosine is taken as 0
    cfg = SMALL[2]
    say("case zero keys")
    data = workloads.generate(cfg)
    data["keys"][0, 0, 100:140] = 0
    data["keys"][0, 1, 2990:] = 0
    check_case(cfg, data)


def test_k15_small_stride():
    # 2^15 bucket starts per chunk exceed the sort's own LDS at this stride
    cfg = SMALL[9]
    assert cfg.K == 15
    say("case K15 stride 256")
    data = workloads.generate(cfg)
    check_case(cfg, data, stride=256)


def test_k0_is_exact_attention():
    cfg = workloads.Config("k0", B=1, Hq=8, Hkv=2, N=3000, d=128, K=0, L=3, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=21)
    say("case k0")
    data = workloads.generate(cfg)
    tb, r = check_case(cfg, data)
    keys = data["keys"].float().numpy()
    vals = data["values"].float().numpy()
    q = data["q"][0].float().numpy()
    for h in range(cfg.Hq):
        ex, lse = O.exact_attention(q[0, h], keys[0, h // cfg.G], vals[0, h // cfg.G], cfg.scale)
        out = to_np(r["out"][0, h])
        assert np.linalg.norm(out - ex) / np.linalg.norm(ex) <= PAR.OUT_RTOL
        assert int(r["nsel"][0, h]) == cfg.N


# K = 0 puts every key of a chunk in the one probed bucket, so a count
# workgroup walks L * stride / 8 blocks per head: past 512 rows of 64 blocks
# the walk finds each block's segment by binary search instead of the
# segment map.  One head per count workgroup (128 (head, chunk) pairs), and
# two (640 pairs: more than one round of resident workgroups).
K0_LONG = [
    workloads.Config("k0-long", B=1, Hq=8, Hkv=2, N=9000, d=128, K=0, L=40, T=2, dtype="bf16",
                     planted=4, a=0.8, offset="per_head", seed=22),
    workloads.Config("k0-long-2heads", B=8, Hq=16, Hkv=2, N=40000, d=128, K=0, L=40, T=2, dtype="bf16",
                     planted=4, a=0.8, offset="per_head", seed=23),
]


@pytest.mark.parametrize("cfg", K0_LONG, ids=[c.name for c in K0_LONG])
def test_k0_long_walks(cfg):
    say(f"case {cfg.name}")
    data = workloads.generate(cfg)
    units = [(0, 0), (cfg.B - 1, cfg.Hkv - 1)]
    tb, r = check_case(cfg, data, units=units)
    keys = data["keys"].float().numpy()
    vals = data["values"].float().numpy()
    q = data["q"][0].float().numpy()
    for b, g in units:
        for h in range(g * cfg.G, (g + 1) * cfg.G):
            ex, lse = O.exact_attention(q[b, h], keys[b, g], vals[b, g], cfg.scale)
            out = to_np(r["out"][b, h])
            assert np.linalg.norm(out - ex) / np.linalg.norm(ex) <= PAR.OUT_RTOL
            assert int(r["nsel"][b, h]) == cfg.N


def test_deterministic():
    cfg = SMALL[2]
    say("case determinism")
    data = workloads.generate(cfg)
    tb1, r1 = run_gpu(cfg, data)
    tb2, r2 = run_gpu(cfg, data)
    for k in ("offsets", "indices", "codes"):
        assert torch.equal(tb1[k], tb2[k]), k
    for k in ("out", "lse", "nsel", "q_codes", "counts"):
        assert torch.equal(r1[k], r2[k]), k


# ----------------------------------------------------------------- full sizes

# Sampled units.  Per-key arrays are [units, L, N] (codes, indices) and
# [units, N, d] (keys, values): at 64 x 8 units of 32K keys and L = 150 the
# codes and indices of unit u start at element u * L * N = u * 4.9e6, so the
# units from 437 on lie past 2^31 elements; (63, 7) is unit 511 (2.5e9).
# Heads per unit: an int for every unit, or a dict per unit (None = all).
FULL = {
    2: dict(units=None, heads=None, steps=[0]),
    3: dict(units=[(0, 0), (11, 5)], heads=4, steps=[0]),
    4: dict(units=[(0, 1), (0, 3)], heads={(0, 1): 3, (0, 3): None}, steps=[0]),
    5: dict(units=[(37, 6), (63, 7)], heads=2, steps=[0, 7]),
}


@pytest.mark.parametrize("cfg_id", sorted(FULL))
def test_full_size_sampled(cfg_id):
    cfg = workloads.CONFIGS[cfg_id]
    spec = FULL[cfg_id]
    say(f"case full cfg{cfg_id} {cfg.name}")
    data = workloads.generate(cfg, device="cuda")
    for step in spec["steps"]:
        check_case(cfg, data, units=spec["units"], heads_per_unit=spec["heads"], step=step)
    del data
    torch.cuda.empty_cache()


# ------------------------------------------------------------ hybrid decode
# exact attention over the first n_sink and the last n_window keys, merged by
# log-sum-exp with the estimate over the selected keys outside that set

HYBRID = [
    (SMALL[1], 4, 64, None),          # ragged, several chunks
    (SMALL[1], 16, 1500, 1024),       # window spans chunk boundaries
    (SMALL[2], 3000, 3000, None),     # sink and window overlap: everything exact
    (SMALL[3], 0, 100, None),         # window only
    (SMALL[4], 7, 0, None),           # fp32, sinks only
    (SMALL[6], 1, 1, None),           # N = 1: the key is both sink and window
    (SMALL[7], 8, 32, None),          # T = L: the selection is mostly empty
    (SMALL[10], 5, 2000, None),       # K = 12, N = 9001
]


@pytest.mark.parametrize("cfg,n_sink,n_window,stride", HYBRID,
                         ids=[f"{c.name}-s{a}-w{b}" for c, a, b, _ in HYBRID])
def test_hybrid_parity(cfg, n_sink, n_window, stride):
    say(f"case hybrid {cfg.name} sink={n_sink} window={n_window} stride={stride}")
    data = workloads.generate(cfg)
    check_case(cfg, data, stride=stride, n_sink=n_sink, n_window=n_window)


# more (query head, key chunk) pairs than one round of resident workgroups
# (512): a count workgroup then takes several heads of one unit (2, 3 or 4
# here), or counting takes several rounds
MANY_ROUNDS = [
    (workloads.Config("rounds-bf16", B=3, Hq=12, Hkv=3, N=6000, d=128, K=8, L=16, T=2, dtype="bf16",
                      planted=4, a=0.8, offset="per_unit", seed=41), 4, 300),
    (workloads.Config("rounds-f32", B=2, Hq=16, Hkv=2, N=4200, d=128, K=7, L=12, T=2, dtype="f32",
                      planted=3, a=0.8, offset="per_head", seed=42), 0, 0),
    # 1536 (head, chunk) pairs: each count workgroup takes the 4 heads of a unit
    (workloads.Config("rounds-4heads", B=8, Hq=16, Hkv=4, N=3000, d=128, K=8, L=12, T=2, dtype="bf16",
                      planted=3, a=0.8, offset="per_head", seed=43), 2, 100),
    # GQA 3: each count workgroup takes the 3 heads of a unit
    (workloads.Config("rounds-gqa3", B=4, Hq=12, Hkv=4, N=4000, d=128, K=9, L=10, T=1, dtype="bf16",
                      planted=3, a=0.8, offset="per_unit", seed=44), 0, 0),
]


@pytest.mark.parametrize("cfg,n_sink,n_window", MANY_ROUNDS, ids=[c.name for c, _, _ in MANY_ROUNDS])
def test_many_count_rounds(cfg, n_sink, n_window):
    import lsh_sampled_sparse_amd as lsh
    assert cfg.B * cfg.Hq * lsh.lsh_num_chunks(cfg.N, 256) > 512
    say(f"case many count rounds {cfg.name} sink={n_sink} window={n_window}")
    data = workloads.generate(cfg)
    check_case(cfg, data, stride=256, n_sink=n_sink, n_window=n_window)


def test_hybrid_all_exact_is_attention():
    # an exact set covering every key leaves nothing to sample: exact attention
    cfg = SMALL[1]
    say("case hybrid all exact")
    data = workloads.generate(cfg)
    tb, r = run_gpu(cfg, data, n_sink=10, n_window=cfg.N)
    keys = data["keys"].float().numpy()
    vals = data["values"].float().numpy()
    q = data["q"][0].float().numpy()
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            ex, lse = O.exact_attention(q[b, h], keys[b, h // cfg.G], vals[b, h // cfg.G], cfg.scale)
            out = to_np(r["out"][b, h])
            assert np.linalg.norm(out - ex) / np.linalg.norm(ex) <= PAR.OUT_RTOL
            assert abs(float(r["lse"][b, h]) - lse) <= PAR.LSE_ATOL * max(1.0, abs(lse))
            assert int(r["nsel"][b, h]) == 0


def test_hybrid_zero_set_is_plain_decode():
    # n_sink = n_window = 0 through the hybrid entry point: the plain decode, bit for bit
    lsh = _lsh()
    cfg = SMALL[2]
    say("case hybrid empty set")
    data = workloads.generate(cfg)
    dev = torch.device("cuda:0")
    keys, vals, W = data["keys"].to(dev), data["values"].to(dev), data["W"].to(dev)
    q = data["q"][0].to(dev).contiguous()
    tb = lsh.build_tables(keys, W, cfg.K, cfg.L)
    r0 = lsh.decode_attention(q, keys, vals, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale)
    outs = []
    for _ in range(2):
        out = torch.empty_like(r0["out"])
        lse = torch.empty_like(r0["lse"])
        nsel = torch.empty_like(r0["nsel"])
        lsh.lsh_decode_attention_hybrid(q, keys, vals, W, tb["indices"], tb["offsets"], cfg.K, cfg.L, cfg.T,
                                        tb["stride"], cfg.scale, 0, 0, out, lse, nsel)
        outs.append((out, lse, nsel))
    torch.cuda.synchronize()
    for out, lse, nsel in outs:
        assert torch.equal(out, r0["out"]) and torch.equal(lse, r0["lse"]) and torch.equal(nsel, r0["nsel"])


def test_hybrid_full_size_128k():
    cfg = workloads.CONFIGS[4]
    say(f"case hybrid full {cfg.name}")
    data = workloads.generate(cfg, device="cuda")
    check_case(cfg, data, units=[(0, 2)], heads_per_unit=2, n_sink=4, n_window=1024)
    del data
    torch.cuda.empty_cache()


# ------------------------------------------------------ centred-plant variant
# queries planted on the keys less their shared offset: the selection is then
# sparse (a few percent of the keys per head), the regime the pages argue
# sampling is for

@pytest.mark.parametrize("cfg_id,units,heads", [(4, [(0, 2)], 4), (2, [(0, 0), (0, 5)], None)])
def test_full_size_centred_plant(cfg_id, units, heads):
    cfg = workloads.CONFIGS[cfg_id].with_(plant="centred")
    say(f"case full centred cfg{cfg_id} {cfg.name}")
    data = workloads.generate(cfg, device="cuda")
    tb, r = check_case(cfg, data, units=units, heads_per_unit=heads)
    frac = float(r["nsel"].float().mean()) / cfg.N
    say(f"  centred plant: mean selected fraction per head {frac:.4f}")
    assert frac < 0.2
    del data
    torch.cuda.empty_cache()

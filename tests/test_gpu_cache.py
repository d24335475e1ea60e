"""A growing key cache on the GPU: table updates and decodes over a prefix.

The cache has room for n_cap keys per (sequence, kv head); keys arrive in
batches of various sizes (one key, a few hundred, up to a chunk boundary and
across it).  After every update the tables must be those the oracle builds
from the keys held so far, and a decode over that prefix must match the
oracle's decode over the same keys.  Cache positions past the prefix hold
NaN, so a kernel that read them would spoil its outputs.
"""

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


def to_np(t):
    return t.detach().cpu().numpy()


def check_prefix(cfg, data, tb, r, n, units, heads_per_unit=None, n_sink=0, n_window=0):
    """Compare the tables (first n keys) and one decode over them with the oracle."""
    stride = tb["stride"]
    nj = O.num_chunks(n, stride)
    W = data["W"].float().cpu().numpy()
    q = data["q"][0].float().cpu().numpy()
    flips = bits = 0
    rels = []
    for (b, g) in units:
        ku = data["keys"][b, g, :n].float().cpu().numpy()
        vu = data["values"][b, g, :n].float().cpu().numpy()
        ref = O.build_tables(ku, W, cfg.K, cfg.L, stride)
        band = PAR.band_mask(ku, W) if cfg.K > 0 else np.zeros((n, 0), bool)
        gcodes = to_np(tb["codes"][b, g, :, :n])
        flips += PAR.compare_codes(gcodes, ref["codes"], band, cfg.K, cfg.L)
        bits += n * cfg.L * cfg.K
        PAR.check_tables(to_np(tb["offsets"][b, g, :, :nj]), to_np(tb["indices"][b, g, :, :n]), gcodes, ref,
                         cfg.K, stride)
        hs = list(range(g * cfg.G, (g + 1) * cfg.G))[:heads_per_unit]
        for h in hs:
            if n_sink or n_window:
                rr = O.hybrid_decode_head(q[b, h], ku, vu, W, ref["offsets"], ref["indices"], cfg.K, cfg.L, cfg.T,
                                          cfg.scale, n_sink, n_window)
            else:
                rr = O.decode_head(q[b, h], ku, vu, W, ref["offsets"], ref["indices"], cfg.K, cfg.L, cfg.T,
                                   cfg.scale)
            qb = PAR.band_mask(q[b, h][None], W) if cfg.K > 0 else np.zeros((1, 0), bool)
            gh = {"q_codes": to_np(r["q_codes"][b, h]), "counts": to_np(r["counts"][b, h]),
                  "out": to_np(r["out"][b, h]), "lse": float(r["lse"][b, h]), "nsel": int(r["nsel"][b, h])}
            res = PAR.check_head(gh, rr, qb, gcodes, ref["codes"], cfg.K, cfg.L, cfg.T, exact=rr.get("exact"))
            flips += res["qflips"]
            bits += cfg.L * cfg.K
            rels.append(res["rel"])
    if bits:
        assert flips <= max(1.0, PAR.FLIP_FRACTION_MAX * bits), (flips, bits)
    return max(rels) if rels else 0.0


def grow(cfg, schedule, stride=None, n_sink=0, n_window=0, check_units=None, heads_per_unit=None,
         check_at=None, device="cpu"):
    lsh = _lsh()
    dev = torch.device("cuda:0")
    data = workloads.generate(cfg, device=device)
    n_cap = cfg.N
    keys = data["keys"].to(dev)
    vals = data["values"].to(dev)
    W = data["W"].to(dev)
    q = data["q"][0].to(dev).contiguous()
    # the cache: NaN past the keys it holds
    ck = torch.full_like(keys, float("nan"))
    cv = torch.full_like(vals, float("nan"))
    tb = lsh.alloc_tables(ck, cfg.K, cfg.L, stride=stride, return_codes=True)
    units = check_units or [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    for n in schedule:
        n0 = tb["n"]
        ck[:, :, n0:n] = keys[:, :, n0:n]
        cv[:, :, n0:n] = vals[:, :, n0:n]
        lsh.update_tables(ck, W, tb, n, cfg.K, cfg.L)
        r = lsh.decode_attention(q, ck, cv, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale, return_codes=True,
                                 return_counts=True, n_sink=n_sink, n_window=n_window)
        torch.cuda.synchronize()
        assert torch.isfinite(r["out"]).all()
        if check_at is None or n in check_at:
            rel = check_prefix(cfg, data, tb, r, n, units, heads_per_unit, n_sink, n_window)
            say(f"[{cfg.name}] n={n} (from {n0}) stride={tb['stride']} max_rel={rel:.2e}")
    return lsh, data, keys, vals, W, q, ck, cv, tb


GROWTH = [
    (workloads.Config("cache-gqa4", B=2, Hq=8, Hkv=2, N=6000, d=128, K=8, L=24, T=2, dtype="bf16",
                      planted=4, a=0.8, offset="per_head", seed=31),
     [2500, 2501, 2600, 3072, 3073, 4500, 6000], 1024, 0, 0),
    (workloads.Config("cache-fp32", B=1, Hq=4, Hkv=2, N=3000, d=128, K=7, L=16, T=2, dtype="f32",
                      planted=3, a=0.8, offset="per_unit", seed=32),
     [1, 2, 700, 2999, 3000], None, 0, 0),
    (workloads.Config("cache-k12-s256", B=1, Hq=4, Hkv=1, N=2000, d=128, K=12, L=8, T=1, dtype="bf16",
                      planted=2, a=0.9, offset="none", seed=33),
     [255, 256, 257, 1000, 1999, 2000], 256, 0, 0),
    (workloads.Config("cache-hybrid", B=1, Hq=8, Hkv=2, N=5000, d=128, K=8, L=20, T=2, dtype="bf16",
                      planted=4, a=0.8, offset="per_head", seed=34),
     [3000, 3001, 4096, 4097, 5000], 1024, 4, 300),
    (workloads.Config("cache-k0", B=1, Hq=4, Hkv=1, N=1500, d=128, K=0, L=3, T=2, dtype="bf16",
                      planted=2, a=0.8, offset="none", seed=35),
     [700, 701, 1500], 256, 0, 0),
]


@pytest.mark.parametrize("cfg,schedule,stride,n_sink,n_window", GROWTH, ids=[g[0].name for g in GROWTH])
def test_cache_growth(cfg, schedule, stride, n_sink, n_window):
    say(f"case cache growth {cfg.name} schedule={schedule}")
    if cfg.K == 0:
        # no projection columns: the build takes an empty W
        lsh = _lsh()
        dev = torch.device("cuda:0")
        data = workloads.generate(cfg)
        keys, vals = data["keys"].to(dev), data["values"].to(dev)
        q = data["q"][0].to(dev).contiguous()
        W = torch.empty(cfg.d, 0, dtype=keys.dtype, device=dev)
        ck = torch.full_like(keys, float("nan"))
        cv = torch.full_like(vals, float("nan"))
        tb = lsh.alloc_tables(ck, 0, cfg.L, stride=stride)
        for n in schedule:
            n0 = tb["n"]
            ck[:, :, n0:n] = keys[:, :, n0:n]
            cv[:, :, n0:n] = vals[:, :, n0:n]
            lsh.update_tables(ck, W, tb, n, 0, cfg.L)
            r = lsh.decode_attention(q, ck, cv, W, tb, 0, cfg.L, cfg.T, sm_scale=cfg.scale)
            torch.cuda.synchronize()
            kf, vf, qf = data["keys"].float().numpy(), data["values"].float().numpy(), data["q"][0].float().numpy()
            for h in range(cfg.Hq):
                ex, lse = O.exact_attention(qf[0, h], kf[0, h // cfg.G, :n], vf[0, h // cfg.G, :n], cfg.scale)
                out = to_np(r["out"][0, h])
                assert np.linalg.norm(out - ex) / np.linalg.norm(ex) <= PAR.OUT_RTOL
                assert int(r["nsel"][0, h]) == n
            say(f"[{cfg.name}] n={n} exact attention ok")
        return
    grow(cfg, schedule, stride=stride, n_sink=n_sink, n_window=n_window)


def test_update_equals_fresh_build():
    # tables grown one batch at a time are the tables a build over the same
    # keys writes, bit for bit (row pitch aside)
    cfg = GROWTH[0][0]
    say("case update equals fresh build")
    lsh, data, keys, vals, W, q, ck, cv, tb = grow(cfg, [2500, 2501, 3072, 4500], stride=1024, check_at=())
    n = tb["n"]
    fresh = lsh.build_tables(keys[:, :, :n].contiguous(), W, cfg.K, cfg.L, stride=1024, return_codes=True)
    nj = lsh.lsh_num_chunks(n, 1024)
    assert torch.equal(tb["indices"][..., :n], fresh["indices"])
    assert torch.equal(tb["codes"][..., :n], fresh["codes"])
    assert torch.equal(tb["offsets"][:, :, :, :nj], fresh["offsets"])
    r1 = lsh.decode_attention(q, ck, cv, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale)
    r2 = lsh.decode_attention(q, keys[:, :, :n].contiguous(), vals[:, :, :n].contiguous(), W, fresh, cfg.K, cfg.L,
                              cfg.T, sm_scale=cfg.scale)
    torch.cuda.synchronize()
    for k in ("out", "lse", "nsel"):
        assert torch.equal(r1[k], r2[k]), k


def test_full_size_decode_steps_128k():
    # the 128K GQA-8 workload as a cache: built over all but the last 8 keys,
    # then 8 decode steps that each append one key and decode (hybrid: 4
    # sinks + a 64-key window); one (sequence, kv head) checked at the end
    cfg = workloads.CONFIGS[4]
    say(f"case cache full {cfg.name}")
    N = cfg.N
    schedule = [N - 8 + i for i in range(9)]
    grow(cfg, schedule, n_sink=4, n_window=64, check_units=[(0, 3)], heads_per_unit=2, check_at=(N,),
         device="cuda")
    torch.cuda.empty_cache()

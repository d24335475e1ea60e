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


def check_prefix(cfg, data, tb, r, n, units, heads_per_unit=None, n_sink=0, n_window=0, W_heads=None):
    """Compare the tables and one decode with the oracle: sequence b holds
    n[b] keys (n may be one int for all), unit (b, g) hashes with W, or with
    W_heads[g] when there is one W per kv head."""
    stride = tb["stride"]
    lens = [n] * cfg.B if isinstance(n, int) else list(n)
    q = data["q"][0].float().cpu().numpy()
    flips = bits = 0
    rels = []
    for (b, g) in units:
        nb = lens[b]
        hs = list(range(g * cfg.G, (g + 1) * cfg.G))[:heads_per_unit]
        if nb == 0:
            # nothing held: empty estimate
            for h in hs:
                assert float(r["out"][b, h].abs().max()) == 0.0
                assert float(r["lse"][b, h]) == -np.inf and int(r["nsel"][b, h]) == 0
            continue
        W = (W_heads[g] if W_heads is not None else data["W"]).float().cpu().numpy()
        nj = O.num_chunks(nb, stride)
        ku = data["keys"][b, g, :nb].float().cpu().numpy()
        vu = data["values"][b, g, :nb].float().cpu().numpy()
        ref = O.build_tables(ku, W, cfg.K, cfg.L, stride)
        band = PAR.band_mask(ku, W) if cfg.K > 0 else np.zeros((nb, 0), bool)
        gcodes = to_np(tb["codes"][b, g, :, :nb])
        flips += PAR.compare_codes(gcodes, ref["codes"], band, cfg.K, cfg.L)
        bits += nb * cfg.L * cfg.K
        PAR.check_tables(to_np(tb["offsets"][b, g, :, :nj]), to_np(tb["indices"][b, g, :, :nb]), gcodes, ref,
                         cfg.K, stride)
        for h in hs:
            if n_sink or n_window:
                rr = O.hybrid_decode_head(q[b, h], ku, vu, W, ref["offsets"], ref["indices"], cfg.K, cfg.L, cfg.T,
                                          cfg.scale, n_sink, n_window)
            else:
                rr = O.decode_head(q[b, h], ku, vu, W, ref["offsets"], ref["indices"], cfg.K, cfg.L, cfg.T,
                                   cfg.scale)
            qb = PAR.band_mask(q[b, h][None], W) if cfg.K > 0 else np.zeros((1, 0), bool)
            gh = {"q_codes": to_np(r["q_codes"][b, h]), "counts": to_np(r["counts"][b, h, :nb]),
                  "out": to_np(r["out"][b, h]), "lse": float(r["lse"][b, h]), "nsel": int(r["nsel"][b, h])}
            assert not r["counts"][b, h, nb:].any(), "counts past the sequence's length"
            res = PAR.check_head(gh, rr, qb, gcodes, ref["codes"], cfg.K, cfg.L, cfg.T, exact=rr.get("exact"))
            flips += res["qflips"]
            bits += cfg.L * cfg.K
            rels.append(res["rel"])
    if bits:
        assert flips <= max(1.0, PAR.FLIP_FRACTION_MAX * bits), (flips, bits)
    return max(rels) if rels else 0.0


def grow(cfg, schedule, stride=None, n_sink=0, n_window=0, check_units=None, heads_per_unit=None,
         check_at=None, device="cpu", W_heads=None):
    """Fill a NaN cache step by step; ``schedule`` lists the keys held after
    each step, one int for every sequence or a list of B per-sequence
    lengths.  Checks against the oracle after the steps in ``check_at``
    (default: all)."""
    lsh = _lsh()
    dev = torch.device("cuda:0")
    data = workloads.generate(cfg, device=device)
    keys = data["keys"].to(dev)
    vals = data["values"].to(dev)
    W = (W_heads if W_heads is not None else data["W"]).to(dev).contiguous()
    q = data["q"][0].to(dev).contiguous()
    # the cache: NaN past the keys it holds
    ck = torch.full_like(keys, float("nan"))
    cv = torch.full_like(vals, float("nan"))
    tb = lsh.alloc_tables(ck, cfg.K, cfg.L, stride=stride, return_codes=True)
    units = check_units or [(b, g) for b in range(cfg.B) for g in range(cfg.Hkv)]
    for step, n in enumerate(schedule):
        lens = [n] * cfg.B if isinstance(n, int) else list(n)
        for b in range(cfg.B):
            n0 = tb["lens"][b]
            ck[b, :, n0:lens[b]] = keys[b, :, n0:lens[b]]
            cv[b, :, n0:lens[b]] = vals[b, :, n0:lens[b]]
        lsh.update_tables(ck, W, tb, n, cfg.K, cfg.L)
        r = lsh.decode_attention(q, ck, cv, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale, return_codes=True,
                                 return_counts=True, n_sink=n_sink, n_window=n_window)
        torch.cuda.synchronize()
        assert not torch.isnan(r["out"]).any()
        if check_at is None or step in check_at:
            rel = check_prefix(cfg, data, tb, r, lens, units, heads_per_unit, n_sink, n_window,
                               W_heads=W_heads)
            say(f"[{cfg.name}] lens={lens} stride={tb['stride']} max_rel={rel:.2e}")
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


def test_insert_equals_fresh_build():
    # appends of at most 256 keys onto built tables are inserted into their
    # chunks: one key, 256 keys, up to a chunk boundary, into an empty chunk,
    # across a chunk boundary (with rebuilds in between).  After every step
    # the tables are those a fresh build over the same keys writes, bit for
    # bit, and the decodes agree bit for bit
    cfg = GROWTH[0][0]
    schedule = [2500, 2501, 2757, 3000, 3072, 3073, 3100, 3200, 3400, 4096, 4097, 4353]
    say(f"case insert equals fresh build schedule={schedule}")
    lsh = _lsh()
    dev = torch.device("cuda:0")
    data = workloads.generate(cfg)
    keys, vals = data["keys"].to(dev), data["values"].to(dev)
    W = data["W"].to(dev).contiguous()
    q = data["q"][0].to(dev).contiguous()
    ck = torch.full_like(keys, float("nan"))
    cv = torch.full_like(vals, float("nan"))
    tb = lsh.alloc_tables(ck, cfg.K, cfg.L, stride=1024, return_codes=True)
    for n in schedule:
        n0 = tb["n"]
        ck[:, :, n0:n] = keys[:, :, n0:n]
        cv[:, :, n0:n] = vals[:, :, n0:n]
        lsh.update_tables(ck, W, tb, n, cfg.K, cfg.L)
        fresh = lsh.build_tables(keys[:, :, :n].contiguous(), W, cfg.K, cfg.L, stride=1024, return_codes=True)
        torch.cuda.synchronize()
        nj = lsh.lsh_num_chunks(n, 1024)
        assert torch.equal(tb["indices"][..., :n], fresh["indices"]), n
        assert torch.equal(tb["codes"][..., :n], fresh["codes"]), n
        assert torch.equal(tb["offsets"][:, :, :, :nj], fresh["offsets"]), n
        r1 = lsh.decode_attention(q, ck, cv, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale)
        r2 = lsh.decode_attention(q, keys[:, :, :n].contiguous(), vals[:, :, :n].contiguous(), W, fresh, cfg.K,
                                  cfg.L, cfg.T, sm_scale=cfg.scale)
        torch.cuda.synchronize()
        for k in ("out", "lse", "nsel"):
            assert torch.equal(r1[k], r2[k]), (n, k)
        say(f"[{cfg.name}] n={n} ({n - n0} keys {'inserted' if 0 < n0 and n - n0 <= 256 else 'by rebuild'}) "
            f"tables and decode equal a fresh build")


def test_insert_odd_pitch():
    # a cache whose capacity is odd (3001 keys), so most tables' rows start
    # off a 16-byte boundary and the insertion stages and writes them with
    # 2-byte accesses; appends up to, into and across the 1536 chunk
    # boundary; the tables and decodes equal a fresh build's bit for bit
    cfg = workloads.Config("insert-odd-pitch", B=1, Hq=6, Hkv=2, N=3001, d=128, K=9, L=12, T=2, dtype="bf16",
                           planted=3, a=0.8, offset="per_head", seed=42)
    schedule = [1000, 1001, 1257, 1500, 1536, 1537, 1600, 1601]
    say(f"case insert odd pitch schedule={schedule}")
    lsh = _lsh()
    dev = torch.device("cuda:0")
    data = workloads.generate(cfg)
    keys, vals = data["keys"].to(dev), data["values"].to(dev)
    W = data["W"].to(dev).contiguous()
    q = data["q"][0].to(dev).contiguous()
    ck = torch.full_like(keys, float("nan"))
    cv = torch.full_like(vals, float("nan"))
    tb = lsh.alloc_tables(ck, cfg.K, cfg.L, stride=512, return_codes=True)
    for n in schedule:
        n0 = tb["n"]
        ck[:, :, n0:n] = keys[:, :, n0:n]
        cv[:, :, n0:n] = vals[:, :, n0:n]
        lsh.update_tables(ck, W, tb, n, cfg.K, cfg.L)
        fresh = lsh.build_tables(keys[:, :, :n].contiguous(), W, cfg.K, cfg.L, stride=512, return_codes=True)
        torch.cuda.synchronize()
        nj = lsh.lsh_num_chunks(n, 512)
        assert torch.equal(tb["indices"][..., :n], fresh["indices"]), n
        assert torch.equal(tb["codes"][..., :n], fresh["codes"]), n
        assert torch.equal(tb["offsets"][:, :, :, :nj], fresh["offsets"]), n
        r1 = lsh.decode_attention(q, ck, cv, W, tb, cfg.K, cfg.L, cfg.T, sm_scale=cfg.scale)
        r2 = lsh.decode_attention(q, keys[:, :, :n].contiguous(), vals[:, :, :n].contiguous(), W, fresh, cfg.K,
                                  cfg.L, cfg.T, sm_scale=cfg.scale)
        torch.cuda.synchronize()
        for k in ("out", "lse", "nsel"):
            assert torch.equal(r1[k], r2[k]), (n, k)
        say(f"[{cfg.name}] n={n} tables and decode equal a fresh build")


def test_ragged_insert():
    # per-sequence lengths far apart, so the bounds do not settle the choice
    # and each sequence takes it: in one call some insert (1 and 256 keys),
    # one stays, one is rebuilt; tables and decodes checked against the oracle
    cfg = workloads.Config("cache-ragged-insert", B=3, Hq=8, Hkv=2, N=5000, d=128, K=9, L=16, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=41)
    say("case ragged insert")
    schedule = [[1000, 2500, 300], [1001, 2501, 300], [1257, 2502, 1300], [1300, 2700, 1301], [1301, 3072, 1557]]
    grow(cfg, schedule, stride=1024, n_sink=2, n_window=64)


def test_full_size_decode_steps_128k():
    # the 128K GQA-8 workload as a cache: built over all but the last 8 keys,
    # then 8 decode steps that each append one key and decode (hybrid: 4
    # sinks + a 64-key window); one (sequence, kv head) checked at the end
    cfg = workloads.CONFIGS[4]
    say(f"case cache full {cfg.name}")
    N = cfg.N
    schedule = [N - 8 + i for i in range(9)]
    grow(cfg, schedule, n_sink=4, n_window=64, check_units=[(0, 3)], heads_per_unit=2,
         check_at=(len(schedule) - 1,), device="cuda")
    torch.cuda.empty_cache()


def test_ragged_growth():
    # three sequences growing at different rates, one of them empty at first
    # and one that stops growing; hybrid decode over each sequence's own keys
    cfg = workloads.Config("cache-ragged", B=3, Hq=8, Hkv=2, N=5000, d=128, K=8, L=20, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=36)
    say("case ragged growth")
    schedule = [[1000, 0, 300], [1001, 2500, 1024], [3000, 2500, 1025], [3000, 4999, 4096], [5000, 5000, 4097]]
    grow(cfg, schedule, stride=1024, n_sink=2, n_window=100)


def test_per_head_projection():
    # one SimHash projection per kv head: the tables of unit (b, g) and the
    # query codes of head h use W[g], W[h / G]
    cfg = workloads.Config("per-head-w", B=2, Hq=8, Hkv=2, N=3000, d=128, K=9, L=16, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_unit", seed=37)
    say("case per-head W")
    Wh = workloads.per_head_projections(cfg, seed=1037)
    grow(cfg, [1500, [3000, 2200]], stride=1024, W_heads=Wh)


def test_ragged_growth_fp32():
    # the fp32 attention kernel over ragged lengths, with a per-head W
    cfg = workloads.Config("cache-ragged-f32", B=2, Hq=4, Hkv=2, N=2500, d=128, K=7, L=12, T=2, dtype="f32",
                           planted=3, a=0.8, offset="per_unit", seed=38)
    say("case ragged growth fp32")
    Wh = workloads.per_head_projections(cfg, seed=1038)
    grow(cfg, [[300, 0], [1025, 700], [2500, 1800]], stride=512, n_sink=3, n_window=40, W_heads=Wh)


def test_k15_growth():
    # 2^15 bucket starts per chunk: every rebuilt chunk rewrites 64 KB of offsets
    cfg = workloads.Config("cache-k15", B=1, Hq=2, Hkv=1, N=1200, d=128, K=15, L=3, T=1, dtype="bf16",
                           planted=1, a=0.95, offset="none", seed=39)
    say("case K15 growth")
    grow(cfg, [500, 513, 1200], stride=256)


def test_full_size_ragged_batch64():
    # the batch-64 32K workload as a ragged cache: sequences held at different
    # lengths, two decode steps that each append a key to every sequence
    # (hybrid decode), two (sequence, kv head) units checked at the end: unit
    # 511 = (63, 7) sits past 2^31 elements of the [units, L, n_cap] arrays
    cfg = workloads.CONFIGS[5]
    say(f"case cache full ragged {cfg.name}")
    N = cfg.N
    base = [N - 2 - 1000 * (b % 5) for b in range(cfg.B)]
    schedule = [base, [n + 1 for n in base], [n + 2 for n in base]]
    grow(cfg, schedule, n_sink=4, n_window=64, check_units=[(37, 6), (63, 7)], heads_per_unit=2,
         check_at=(len(schedule) - 1,), device="cuda")
    torch.cuda.empty_cache()


def test_per_head_projection_gqa3_hybrid():
    # per-head W with three query heads per kv head (the query hash then
    # works one (sequence, kv head) group per workgroup) and a hybrid decode
    cfg = workloads.Config("per-head-w-gqa3", B=2, Hq=9, Hkv=3, N=1800, d=128, K=10, L=12, T=2, dtype="bf16",
                           planted=3, a=0.8, offset="per_head", seed=40)
    say("case per-head W gqa3")
    Wh = workloads.per_head_projections(cfg, seed=1040)
    grow(cfg, [[1800, 900]], stride=512, n_sink=2, n_window=50, W_heads=Wh)

"""The decode entry point that allocates nothing (lsh_decode_attention_noalloc)
against the cached decode it shares its kernels with.

The no-alloc entry point takes its workspace from a static device array that
keeps the previous call's contents, so the test makes two calls in a row, the
second with a smaller input (fewer sequences, heads and keys, another dtype
and GQA ratio) over the first call's leftovers, and checks each, through the
C ABI, against lsh_decode_attention_cached on the same inputs with a fresh
workspace.  The two run the same kernels in the same order, so the results
must agree bit for bit: outputs, log-sum-exps, selected counts, query codes
and collision counts.  A call that needs more than the scratch holds must be
refused before anything is launched.
"""

import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(cfg, lens, W_heads, stride, dev):
    import lsh_sampled_sparse_amd as lsh
    data = workloads.generate(cfg, device="cpu")
    keys = data["keys"].to(dev)
    vals = data["values"].to(dev)
    q = data["q"][0].to(dev)
    W = (W_heads if W_heads is not None else data["W"]).to(dev)
    tb = lsh.alloc_tables(keys, cfg.K, cfg.L, stride=stride)
    lsh.update_tables(keys, W, tb, lens, cfg.K, cfg.L)
    return q, keys, vals, W, tb


def _decode(entry, q, keys, vals, W, tb, cfg, n_sink, n_window):
    import lsh_sampled_sparse_amd as lsh
    B, Hq, d = q.shape
    N = tb["n"]
    dev = keys.device
    # outputs start as NaN / -1 so that a slot left unwritten shows
    res = {"out": torch.full((B, Hq, d), float("nan"), device=dev),
           "lse": torch.full((B, Hq), float("nan"), device=dev),
           "nsel": torch.full((B, Hq), -1, dtype=torch.int32, device=dev),
           "q_codes": torch.full((B, Hq, cfg.L), -1, dtype=torch.int16, device=dev),
           "counts": torch.full((B, Hq, N), 255, dtype=torch.uint8, device=dev)}
    args = (q, keys, vals, W, tb["indices"], tb["offsets"], N, cfg.K, cfg.L, cfg.T, tb["stride"], cfg.scale,
            n_sink, n_window, res["out"], res["lse"], res["nsel"], res["q_codes"], res["counts"])
    if entry == "noalloc":
        lsh.lsh_decode_attention_noalloc(*args, seq_lens=tb["lens_dev"])
    else:
        lsh.lsh_decode_attention_cached(*args, seq_lens=tb["lens_dev"])
    torch.cuda.synchronize()
    return res


# call 1: bf16, GQA-4, ragged lengths over several chunks, per-head W, hybrid
# decode; call 2 (smaller in every dimension): fp32, GQA-8, one length
CALLS = [
    (workloads.Config("noalloc-bf16-gqa4", B=3, Hq=16, Hkv=4, N=9000, d=128, K=10, L=40, T=2, dtype="bf16",
                      planted=8, a=0.8, offset="per_unit", seed=71),
     [9000, 6001, 2345], True, 2048, 4, 100),
    (workloads.Config("noalloc-f32-gqa8", B=1, Hq=8, Hkv=1, N=3100, d=128, K=8, L=24, T=2, dtype="f32",
                      planted=4, a=0.8, offset="per_head", seed=72),
     3100, False, 1024, 0, 0),
]


def test_noalloc_matches_cached_twice():
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    dev = torch.device("cuda:0")
    sizes = []
    for i, (cfg, lens, per_head, stride, n_sink, n_window) in enumerate(CALLS):
        say(f"case noalloc call {i}: {cfg.name} lens={lens} sink={n_sink} window={n_window}")
        Wh = workloads.per_head_projections(cfg, seed=900 + i) if per_head else None
        q, keys, vals, W, tb = _inputs(cfg, lens, Wh, stride, dev)
        sizes.append(lsh.lsh_decode_workspace_size(cfg.B, cfg.Hq, cfg.Hkv, tb["n"], cfg.d, cfg.K, cfg.L,
                                                   tb["stride"]))
        ref = _decode("cached", q, keys, vals, W, tb, cfg, n_sink, n_window)
        got = _decode("noalloc", q, keys, vals, W, tb, cfg, n_sink, n_window)
        assert torch.isfinite(ref["out"]).all() and (ref["nsel"] >= 0).all()
        for k in ref:
            assert torch.equal(got[k], ref[k]), (i, k)
        say(f"  call {i} equal; workspace {sizes[-1]} bytes; nsel mean {ref['nsel'].float().mean().item():.1f}")
        del q, keys, vals, W, tb, ref, got
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_oversize():
    # 512 sequences of 16 query heads over 64K keys need more workspace
    # than the 64 MiB scratch (their bitmask words alone are 64 MiB):
    # refused before any launch, outputs untouched (the inputs are never
    # read, so they are left uninitialised)
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    dev = torch.device("cuda:0")
    B, Hq, Hkv, N, K, L, stride = 512, 16, 1, 65536, 8, 32, 8192
    assert lsh.lsh_decode_workspace_size(B, Hq, Hkv, N, 128, K, L, stride) > lsh.NOALLOC_SCRATCH_BYTES
    say("case noalloc oversize")
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device=dev)
    keys = torch.empty(B, Hkv, N, 128, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(128, L * K, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(B, Hkv, L, N, dtype=torch.int16, device=dev)
    offs = torch.empty(B, Hkv, L, N // stride, 1 << K, dtype=torch.int16, device=dev)
    out = torch.full((B, Hq, 128), 7.0, device=dev)
    with pytest.raises(lsh.LshError) as ei:
        lsh.lsh_decode_attention_noalloc(q, keys, keys, W, idx, offs, N, K, L, 2, stride, 0.1, 0, 0, out)
    assert ei.value.status == lsh.LSH_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_decode_in_a_graph():
    # the callers it is for: a decode step captured into a HIP graph without a
    # workspace.  Three replays, each followed by an eager no-alloc call on
    # other inputs (which leaves its own data in the shared scratch); every
    # replay equals the cached decode with its own workspace, bit for bit
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    dev = torch.device("cuda:0")
    say("case noalloc graph")
    cfg = workloads.Config("noalloc-graph", B=2, Hq=8, Hkv=2, N=5000, d=128, K=8, L=24, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=73)
    q, keys, vals, W, tb = _inputs(cfg, 5000, None, 1024, dev)
    ref = _decode("cached", q, keys, vals, W, tb, cfg, 2, 64)
    other_cfg = CALLS[1][0]
    oq, okeys, ovals, oW, otb = _inputs(other_cfg, other_cfg.N, None, 1024, dev)
    oref = _decode("cached", oq, okeys, ovals, oW, otb, other_cfg, 0, 0)

    out = torch.full_like(ref["out"], float("nan"))
    lse = torch.full_like(ref["lse"], float("nan"))
    nsel = torch.full_like(ref["nsel"], -1)
    args = (q, keys, vals, W, tb["indices"], tb["offsets"], tb["n"], cfg.K, cfg.L, cfg.T, tb["stride"], cfg.scale,
            2, 64, out, lse, nsel)
    lsh.lsh_decode_attention_noalloc(*args)   # once eagerly: every kernel's one-time set-up before capture
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            lsh.lsh_decode_attention_noalloc(*args)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        nsel.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref["out"]) and torch.equal(lse, ref["lse"]) and torch.equal(nsel, ref["nsel"]), rep
        got = _decode("noalloc", oq, okeys, ovals, oW, otb, other_cfg, 0, 0)
        for k in oref:
            assert torch.equal(got[k], oref[k]), (rep, k)
        say(f"  replay {rep} equal")

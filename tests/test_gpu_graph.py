"""A table build + decode step captured into a HIP graph and replayed gives
the eager step's results on every replay, with eager work in between."""

import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    print("case graph replay", flush=True)
    sys.stdout.flush()
    dev = torch.device("cuda:0")
    cfg = workloads.Config("graph-gqa4", B=2, Hq=8, Hkv=2, N=5000, d=128, K=8, L=24, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=31)
    data = workloads.generate(cfg, device=dev)
    keys, vals, W = data["keys"], data["values"], data["W"]
    q = data["q"][0].contiguous()
    B, Hq, Hkv, N, d, K, L, T = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.K, cfg.L, cfg.T
    stride = lsh.lsh_default_stride(N, K)
    nch = lsh.lsh_num_chunks(N, stride)
    dt = lsh.LSH_BF16

    def buffers():
        return {
            "offsets": torch.empty(B, Hkv, L, nch, 1 << K, dtype=torch.int16, device=dev),
            "indices": torch.empty(B, Hkv, L, N, dtype=torch.int16, device=dev),
            "out": torch.empty(B, Hq, d, dtype=torch.float32, device=dev),
            "lse": torch.empty(B, Hq, dtype=torch.float32, device=dev),
            "nsel": torch.empty(B, Hq, dtype=torch.int32, device=dev),
            "bws": torch.empty(lsh.lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, dt), dtype=torch.uint8,
                               device=dev),
            "dws": torch.empty(lsh.lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride), dtype=torch.uint8,
                               device=dev),
        }

    def step(bf):
        lsh.lsh_build_tables(keys, W, K, L, stride, bf["offsets"], bf["indices"], None, bf["bws"])
        lsh.lsh_decode_attention(q, keys, vals, W, bf["indices"], bf["offsets"], K, L, T, stride, cfg.scale,
                                 bf["out"], bf["lse"], bf["nsel"], None, None, bf["dws"])

    ref = buffers()
    step(ref)
    torch.cuda.synchronize()

    cap = buffers()
    step(cap)                      # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cap)
    other = buffers()
    for rep in range(3):
        for v in cap.values():
            v.zero_()
        g.replay()
        step(other)                # eager work between replays
        torch.cuda.synchronize()
        for k in ("offsets", "indices", "out", "lse", "nsel"):
            assert torch.equal(cap[k], ref[k]), (rep, k)
            assert torch.equal(other[k], ref[k]), (rep, k)


def test_graph_decode_loop_with_growing_ragged_cache():
    # one decode step of a serving loop captured once: the lengths live on the
    # device, so every replay appends one key per sequence (table update over
    # the chunk holding it) and decodes over the keys held, with the launch
    # bounds at 0 and the capacity.  Each replay must agree with an eager
    # update + decode from scratch at the same lengths.
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    print("case graph decode loop", flush=True)
    sys.stdout.flush()
    dev = torch.device("cuda:0")
    cfg = workloads.Config("graph-loop", B=2, Hq=8, Hkv=2, N=3000, d=128, K=8, L=16, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=41)
    data = workloads.generate(cfg, device=dev)
    keys, vals, W = data["keys"], data["values"], data["W"]
    q = data["q"][0].contiguous()
    B, Hq, Hkv, n_cap, d, K, L, T = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.K, cfg.L, cfg.T
    stride = 1024
    start = [1022, 2047]                     # the first appends cross chunk boundaries
    tb = lsh.alloc_tables(keys, K, L, stride=stride)
    lsh.update_tables(keys, W, tb, start, K, L)
    old = torch.tensor(start, dtype=torch.int32, device=dev)
    new = torch.empty_like(old)
    bws = torch.empty(lsh.lsh_build_workspace_size(B, Hkv, n_cap, d, K, L, stride, lsh.LSH_BF16),
                      dtype=torch.uint8, device=dev)
    dws = torch.empty(lsh.lsh_decode_workspace_size(B, Hq, Hkv, n_cap, d, K, L, stride), dtype=torch.uint8,
                      device=dev)
    out = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    nsel = torch.empty(B, Hq, dtype=torch.int32, device=dev)

    def step():
        torch.add(old, 1, out=new)
        lsh.lsh_update_tables(keys, W, K, L, stride, 0, n_cap, tb["offsets"], tb["indices"], None, bws,
                              old_lens=old, new_lens=new)
        lsh.lsh_decode_attention_cached(q, keys, vals, W, tb["indices"], tb["offsets"], n_cap, K, L, T, stride,
                                        cfg.scale, 4, 64, out, lse, nsel, None, None, dws, seq_lens=new)
        old.copy_(new)

    # an eager decode first (at the current lengths), so every kernel's
    # one-time set-up is done before the capture
    lsh.lsh_decode_attention_cached(q, keys, vals, W, tb["indices"], tb["offsets"], n_cap, K, L, T, stride,
                                    cfg.scale, 4, 64, out, lse, nsel, None, None, dws, seq_lens=old)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    assert torch.equal(old, torch.tensor(start, dtype=torch.int32, device=dev))   # capture ran nothing
    for rep in range(1, 5):
        g.replay()
        torch.cuda.synchronize()
        lens = [n + rep for n in start]
        assert old.tolist() == lens
        ref_tb = lsh.alloc_tables(keys, K, L, stride=stride)
        lsh.update_tables(keys, W, ref_tb, lens, K, L)
        ref = lsh.decode_attention(q, keys, vals, W, ref_tb, K, L, T, sm_scale=cfg.scale, n_sink=4, n_window=64)
        torch.cuda.synchronize()
        for b in range(B):
            n = lens[b]
            assert torch.equal(tb["indices"][b, :, :, :n], ref_tb["indices"][b, :, :, :n]), (rep, b)
            nj = lsh.lsh_num_chunks(n, stride)
            assert torch.equal(tb["offsets"][b, :, :, :nj], ref_tb["offsets"][b, :, :, :nj]), (rep, b)
        assert torch.equal(nsel, ref["nsel"]), rep
        torch.testing.assert_close(out, ref["out"], rtol=1e-4, atol=1e-6)
        torch.testing.assert_close(lse, ref["lse"], rtol=1e-5, atol=1e-5)
        print(f"[graph loop] replay {rep} lens={lens} ok", flush=True)

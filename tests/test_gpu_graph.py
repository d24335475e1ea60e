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

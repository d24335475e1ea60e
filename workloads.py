"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random tensors: it holds none of the method's
arithmetic (no hashing, bucketing, counting or attention).  The shapes follow
the Llama-3.1-8B family that MagicPIG supports (MagicPIG project summary,
"Quick Start & Requirements": Llama models such as Llama-3.1-8B-Instruct)
and the GQA-4 / GQA-8, 32K-128K decode sweep used by the MAC-Attention
benchmark ("MAC-Attention" README, "Reproduce the MAC-vs-FlashInfer hit
curve").  Trained weights and RULER data are not available, so these
Gaussian stand-ins with planted query-key correlations replace them.

Recipe (all draws N(0, 1) unless stated, in this order from one generator
seeded with ``seed``):
  1. W [d, L*K].
  2. keys: z [B, Hkv, N, d] plus the configuration's offset:
       none            k = z
       per_head        k = z + mu_g,  mu_g = 8 * unit(N(0, I)) per kv head
       per_unit        k = z + mu_bg, one mu per (sequence, kv head)
       shared_lowrank  k = mu + U_g c + z, mu = 8 * unit(N(0, I)) shared,
                       U_g an orthonormal [d, 8] basis per kv head,
                       c ~ N(0, 8 I_8) per key
  3. values [B, Hkv, N, d].
  4. per decode step: for every (b, h) a set J of ``planted`` distinct key
     indices of kv head h // G, uniform at random, and
       q = a * sum_{j in J} k_j / sqrt(|J|) + sqrt(1 - a^2) * eps.
     With plant="centred" the planted term uses the keys less their offset
     mean (k_j - mu; the rank-8 part of shared_lowrank stays): the queries
     then no longer point along the offset that every key shares, and the
     selection becomes sparse.  The draws are the same in both modes, so the
     keys, values and W are identical and only q differs.
  5. keys, values, W and q are cast to the configuration's dtype last; q is
     built from the already-cast keys.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    K: int
    L: int
    T: int
    dtype: str          # "f32" or "bf16"
    planted: int
    a: float
    offset: str
    steps: int = 1
    seed: int = 1234
    plant: str = "raw"  # "raw": q planted on k_j; "centred": on k_j - mu

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw):
        return replace(self, **kw)


CONFIGS = {
    # one kv head, fp32, one planted key
    1: Config("tiny-fp32-n4096", B=1, Hq=1, Hkv=1, N=4096, d=128, K=8, L=32, T=2,
              dtype="f32", planted=1, a=0.8, offset="none", seed=1235),
    # Llama-3.1-8B-shaped layer, 16K context, GQA-4
    2: Config("llama8b-gqa4-16k", B=1, Hq=32, Hkv=8, N=16384, d=128, K=10, L=150, T=2,
              dtype="bf16", planted=16, a=0.7, offset="per_head", seed=1236),
    # batched decode, 32K context, GQA-4, no key offset
    3: Config("batch16-gqa4-32k", B=16, Hq=32, Hkv=8, N=32768, d=128, K=9, L=120, T=2,
              dtype="bf16", planted=64, a=0.8, offset="none", seed=1237),
    # long context, 128K, GQA-8, shared offset plus rank-8 component
    4: Config("gqa8-128k", B=1, Hq=32, Hkv=4, N=131072, d=128, K=10, L=150, T=2,
              dtype="bf16", planted=32, a=0.7, offset="shared_lowrank", seed=1238),
    # table build over 64 x 8 x 32K keys then 8 decode steps
    5: Config("batch64-gqa4-32k-build", B=64, Hq=32, Hkv=8, N=32768, d=128, K=10, L=150, T=2,
              dtype="bf16", planted=16, a=0.7, offset="per_unit", steps=8, seed=1239),
}


def _unit(v):
    return v / v.norm(dim=-1, keepdim=True)


def generate(cfg: Config, device="cpu"):
    """Draw one workload.  Returns a dict of tensors on ``device``:

    W [d, L*K], keys [B, Hkv, N, d], values [B, Hkv, N, d],
    q [steps, B, Hq, d], planted [steps, B, Hq, planted] (int64),
    all in the configuration's dtype except ``planted``.
    """
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    f32 = dict(device=device, dtype=torch.float32)
    B, Hq, Hkv, N, d = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d

    W = torch.randn(d, cfg.L * cfg.K, generator=g, **f32)

    keys = torch.randn(B, Hkv, N, d, generator=g, **f32)
    mean = torch.zeros(B, Hkv, d, **f32)   # the offset every key of a unit shares
    if cfg.offset == "per_head":
        mu = 8.0 * _unit(torch.randn(Hkv, d, generator=g, **f32))
        keys += mu[None, :, None, :]
        mean += mu[None]
    elif cfg.offset == "per_unit":
        mu = 8.0 * _unit(torch.randn(B, Hkv, d, generator=g, **f32))
        keys += mu[:, :, None, :]
        mean += mu
    elif cfg.offset == "shared_lowrank":
        mu = 8.0 * _unit(torch.randn(d, generator=g, **f32))
        basis = torch.linalg.qr(torch.randn(Hkv, d, 8, generator=g, **f32))[0]  # [Hkv, d, 8]
        coef = math.sqrt(8.0) * torch.randn(B, Hkv, N, 8, generator=g, **f32)
        keys += mu + torch.einsum("hdr,bhnr->bhnd", basis, coef)
        mean += mu
    elif cfg.offset != "none":
        raise ValueError(cfg.offset)
    if cfg.plant not in ("raw", "centred"):
        raise ValueError(cfg.plant)
    values = torch.randn(B, Hkv, N, d, generator=g, **f32)

    dt = cfg.torch_dtype
    W = W.to(dt)
    keys = keys.to(dt)
    values = values.to(dt)

    qs, planted = [], []
    G = cfg.G
    for _ in range(cfg.steps):
        # distinct uniform indices: the planted-count smallest of N uniforms
        r = torch.rand(B, Hq, N, generator=g, **f32)
        J = torch.topk(r, cfg.planted, dim=-1, largest=False).indices  # [B, Hq, P]
        b_idx = torch.arange(B, device=device)[:, None, None]
        g_idx = (torch.arange(Hq, device=device) // G)[None, :, None]
        picked = keys[b_idx, g_idx, J].float()                          # [B, Hq, P, d]
        if cfg.plant == "centred":
            picked = picked - mean[b_idx[..., 0], g_idx[..., 0]][:, :, None, :]
        eps = torch.randn(B, Hq, d, generator=g, **f32)
        q = cfg.a * picked.sum(2) / math.sqrt(cfg.planted) + math.sqrt(1.0 - cfg.a ** 2) * eps
        qs.append(q.to(dt))
        planted.append(J)
        del picked, r
    return {"W": W, "keys": keys, "values": values,
            "q": torch.stack(qs), "planted": torch.stack(planted)}


def per_head_projections(cfg: Config, seed: int, device="cpu"):
    """One SimHash projection per kv head: W [Hkv, d, L*K], i.i.d. N(0, 1)
    from its own seeded generator, cast to the configuration's dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    W = torch.randn(cfg.Hkv, cfg.d, cfg.L * cfg.K, generator=g, device=device, dtype=torch.float32)
    return W.to(cfg.torch_dtype)

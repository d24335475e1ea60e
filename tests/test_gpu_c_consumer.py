"""The library driven from plain C (tests/c_consumer/abi_smoke.c): a process
with no Python or PyTorch builds tables and decodes through include/lsh_attn.h.
Its tables and outputs must equal those of the Python binding on the same
inputs (same kernels), and its outputs must match the oracle."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import lsh_oracle as O
import parity as PAR

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_consumer", "abi_smoke")


def test_c_consumer_matches_binding_and_oracle(tmp_path):
    if not os.path.exists(EXE):
        pytest.skip("C consumer not built (lsh_sampled_sparse_amd.build builds it)")
    import lsh_sampled_sparse_amd as lsh
    lsh.lib()
    print("case C consumer", flush=True)
    sys.stdout.flush()
    cfg = workloads.Config("c-abi", B=1, Hq=8, Hkv=2, N=3000, d=128, K=8, L=24, T=2, dtype="bf16",
                           planted=4, a=0.8, offset="per_head", seed=51)
    data = workloads.generate(cfg)
    stride = lsh.lsh_default_stride(cfg.N, cfg.K)
    q = data["q"][0].contiguous()
    for name, t in (("keys", data["keys"]), ("values", data["values"]), ("W", data["W"]), ("q", q)):
        t.contiguous().view(torch.int16).numpy().tofile(tmp_path / f"{name}.bin")
    (tmp_path / "meta.txt").write_text(f"{cfg.B} {cfg.Hq} {cfg.Hkv} {cfg.N} {cfg.d} {cfg.K} {cfg.L} {cfg.T} "
                                       f"{stride} {cfg.scale!r}\n")
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    print(r.stdout.strip(), flush=True)

    B, Hq, Hkv, N, d, K, L = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.K, cfg.L
    nch = lsh.lsh_num_chunks(N, stride)
    c_out = np.fromfile(tmp_path / "out.bin", np.float32).reshape(B, Hq, d)
    c_lse = np.fromfile(tmp_path / "lse.bin", np.float32).reshape(B, Hq)
    c_nsel = np.fromfile(tmp_path / "nsel.bin", np.int32).reshape(B, Hq)
    c_off = np.fromfile(tmp_path / "offsets.bin", np.int16).reshape(B, Hkv, L, nch, 1 << K)
    c_idx = np.fromfile(tmp_path / "indices.bin", np.int16).reshape(B, Hkv, L, N)

    # the same step through the Python binding
    dev = torch.device("cuda:0")
    keys, vals, W = data["keys"].to(dev), data["values"].to(dev), data["W"].to(dev)
    tb = lsh.build_tables(keys, W, K, L, stride=stride, return_codes=True)
    res = lsh.decode_attention(q.to(dev), keys, vals, W, tb, K, L, cfg.T, sm_scale=cfg.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(c_off, tb["offsets"].cpu().numpy())
    np.testing.assert_array_equal(c_idx, tb["indices"].cpu().numpy())
    np.testing.assert_array_equal(c_out, res["out"].cpu().numpy())
    np.testing.assert_array_equal(c_lse, res["lse"].cpu().numpy())
    np.testing.assert_array_equal(c_nsel, res["nsel"].cpu().numpy())

    # and against the oracle
    Wn = data["W"].float().numpy()
    qn = q.float().numpy()
    for g in range(Hkv):
        ku = data["keys"][0, g].float().numpy()
        vu = data["values"][0, g].float().numpy()
        ref = O.build_tables(ku, Wn, K, L, stride)
        PAR.check_tables(c_off[0, g], c_idx[0, g], tb["codes"][0, g].cpu().numpy(), ref, K, stride)
        for h in range(g * cfg.G, (g + 1) * cfg.G):
            rr = O.decode_head(qn[0, h], ku, vu, Wn, ref["offsets"], ref["indices"], K, L, cfg.T, cfg.scale)
            if rr["nsel"]:
                rel = np.linalg.norm(c_out[0, h] - rr["out"]) / np.linalg.norm(rr["out"])
                assert rel <= PAR.OUT_RTOL, (h, rel)

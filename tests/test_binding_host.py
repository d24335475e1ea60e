"""Host-side checks of the Python binding (no GPU work is launched)."""

import pytest
import torch

import lsh_sampled_sparse_amd as lsh


def test_build_rejects_cpu_tensors():
    keys = torch.zeros(1, 1, 300, 128, dtype=torch.bfloat16)
    W = torch.zeros(128, 8 * 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        lsh.build_tables(keys, W, 8, 4)


def test_decode_rejects_cpu_tensors():
    q = torch.zeros(1, 2, 128, dtype=torch.bfloat16)
    keys = torch.zeros(1, 1, 300, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        lsh.decode_attention(q, keys, keys, torch.zeros(128, 32, dtype=torch.bfloat16), {}, 8, 4, 2)


def test_dtype_codes():
    assert lsh._dtype_code(torch.bfloat16) == lsh.LSH_BF16
    assert lsh._dtype_code(torch.float32) == lsh.LSH_F32
    with pytest.raises(TypeError):
        lsh._dtype_code(torch.float16)


def test_update_rejects_shrinking_lengths():
    # the length checks run before any device work: stand-in tensors that
    # report themselves as GPU tensors are enough to reach them
    class Fake:
        def __init__(self, shape, dtype=torch.bfloat16):
            self.shape, self.dtype, self.is_cuda = shape, dtype, True

        def is_contiguous(self):
            return True

        def dim(self):
            return len(self.shape)

    keys = Fake((2, 1, 1000, 128))
    W = Fake((128, 32))
    tables = {"n_cap": 1000, "lens": [500, 600], "stride": 256, "n": 600}
    with pytest.raises(ValueError, match="between"):
        lsh.update_tables(keys, W, tables, [400, 700], 8, 4)
    with pytest.raises(ValueError, match="between"):
        lsh.update_tables(keys, W, tables, [600, 1001], 8, 4)
    with pytest.raises(ValueError, match="capacity"):
        lsh.update_tables(keys, W, dict(tables, n_cap=999), [600, 700], 8, 4)
    with pytest.raises(ValueError, match="W must be"):
        lsh.update_tables(keys, Fake((128, 31)), tables, [600, 700], 8, 4)


class _Fake:
    """A stand-in that reports itself as a contiguous GPU tensor: enough to
    reach the binding's shape checks, which run before any device work."""

    def __init__(self, shape, dtype=torch.bfloat16):
        self.shape, self.dtype, self.is_cuda = tuple(shape), dtype, True

    def is_contiguous(self):
        return True

    def dim(self):
        return len(self.shape)


def _decode_args(B=1, Hq=4, Hkv=2, N=1000, K=8, L=4, stride=256, dt=torch.bfloat16):
    nch = -(-N // stride)
    return dict(q=_Fake((B, Hq, 128), dt), keys=_Fake((B, Hkv, N, 128), dt), values=_Fake((B, Hkv, N, 128), dt),
                W=_Fake((128, L * K), dt), indices=_Fake((B, Hkv, L, N), torch.int16),
                offsets=_Fake((B, Hkv, L, nch, 1 << K), torch.int16), K=K, L=L, stride=stride)


def _call_decode(a, **over):
    a = dict(a, **over)
    out = _Fake((1, 4, 128), torch.float32)
    lsh.lsh_decode_attention(a["q"], a["keys"], a["values"], a["W"], a["indices"], a["offsets"], a["K"], a["L"], 2,
                             a["stride"], 0.1, out)


@pytest.mark.skipif(not __import__("os").path.exists(lsh.LIB_PATH), reason="library not built")
def test_decode_checks_w_and_tables():
    a = _decode_args()
    # a CPU W, a W of another dtype, and W of the wrong shape
    with pytest.raises(ValueError, match="W must be a GPU tensor"):
        _call_decode(a, W=torch.zeros(128, 32, dtype=torch.bfloat16))
    with pytest.raises(TypeError, match="W must be"):
        _call_decode(a, W=_Fake((128, 32), torch.float32))
    with pytest.raises(ValueError, match="W must be"):
        _call_decode(a, W=_Fake((128, 31)))
    # one W per kv head is refused by the plain decode (it would be read as a shared W)
    with pytest.raises(ValueError, match="W must be"):
        _call_decode(a, W=_Fake((2, 128, 32)))
    # tables built with another K, L or stride
    with pytest.raises(ValueError, match="offsets must be"):
        _call_decode(a, offsets=_Fake((1, 2, 4, 4, 1 << 9), torch.int16))
    with pytest.raises(ValueError, match="offsets must be"):
        _call_decode(a, offsets=_Fake((1, 2, 5, 4, 1 << 8), torch.int16))
    with pytest.raises(ValueError, match="offsets must be"):
        _call_decode(a, stride=512)
    with pytest.raises(ValueError, match="indices must be"):
        _call_decode(a, indices=_Fake((1, 2, 4, 999), torch.int16))
    with pytest.raises(TypeError, match="indices must be"):
        _call_decode(a, indices=_Fake((1, 2, 4, 1000), torch.int32))
    # values of another shape
    with pytest.raises(ValueError, match="disagree"):
        _call_decode(a, values=_Fake((1, 2, 999, 128)))


def test_convenience_decode_checks_tables():
    a = _decode_args()
    tables = {"indices": a["indices"], "offsets": _Fake((1, 2, 4, 4, 1 << 9), torch.int16), "stride": 256}
    with pytest.raises(ValueError, match="offsets must be"):
        lsh.decode_attention(a["q"], a["keys"], a["values"], a["W"], tables, 8, 4, 2)
    tables = {"indices": a["indices"], "offsets": a["offsets"], "stride": 256}
    with pytest.raises(ValueError, match="W must be"):
        lsh.decode_attention(a["q"], a["keys"], a["values"], _Fake((2, 128, 32)), tables, 8, 4, 2)

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

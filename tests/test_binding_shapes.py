"""The Python binding rejects an `out` of the wrong shape and a `sinks` of the wrong length before
anything reaches the library (CPU only: sizes are checked before devices).

Every extent the kernels use comes from q (or part_o), so a smaller `out` would be written past its
end and a shorter `sinks` read past its end.
"""
import pytest
import torch

import sliding_window_attention_index_amd as sattn


def _win(T=10, H=4, Hkv=2, D=64):
    q = torch.zeros(T, H, D, dtype=torch.bfloat16)
    k = torch.zeros(T, Hkv, D, dtype=torch.bfloat16)
    return q, k, k.clone(), torch.tensor([0, T], dtype=torch.int32)


def test_window_out_shape_rejected():
    q, k, v, cu = _win()
    with pytest.raises(ValueError, match="out must have shape"):
        sattn.window_fwd(q, k, v, cu, 10, out=torch.zeros(9, 4, 64, dtype=torch.bfloat16))


def test_window_sinks_length_rejected():
    q, k, v, cu = _win()
    with pytest.raises(ValueError, match="sinks must hold"):
        sattn.window_fwd(q, k, v, cu, 10, sinks=torch.zeros(3), sink_mode="key0")


def test_indexed_out_shape_rejected():
    q = torch.zeros(1, 3, 32, 128, dtype=torch.bfloat16)
    kv = torch.zeros(1, 50, 128, dtype=torch.bfloat16)
    idx = torch.zeros(1, 3, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        sattn.indexed_fwd(q, kv, idx, out=torch.zeros(1, 2, 32, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="sinks must hold"):
        sattn.indexed_fwd(q, kv, idx, sinks=torch.zeros(16), sink_mode="null")


def test_indexed_fp8_out_shape_rejected():
    q = torch.zeros(1, 3, 32, 128, dtype=torch.bfloat16)
    kv8 = torch.zeros(1, 50, 64, dtype=torch.uint8)
    sc = torch.ones(1, 50)
    rope = torch.zeros(1, 50, 64, dtype=torch.bfloat16)
    idx = torch.zeros(1, 3, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        sattn.indexed_fp8_fwd(q, kv8, sc, rope, idx, out=torch.zeros(1, 3, 16, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="sinks must hold"):
        sattn.indexed_fp8_fwd(q, kv8, sc, rope, idx, sinks=torch.zeros(33), sink_mode="key0")


def test_merge_out_shape_rejected():
    po = torch.zeros(2, 5, 8, 64)
    pl = torch.zeros(2, 5, 8)
    with pytest.raises(ValueError, match="out must have shape"):
        sattn.merge_lse(po, pl, out=torch.zeros(4, 8, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="sinks must hold"):
        sattn.merge_lse(po, pl, sinks=torch.zeros(7), sink_mode="null")


def test_block_mass_sinks_length_rejected():
    q = torch.zeros(1, 3, 32, 128, dtype=torch.bfloat16)
    kv = torch.zeros(1, 50, 128, dtype=torch.bfloat16)
    idx = torch.zeros(1, 3, 64, dtype=torch.int32)
    lse = torch.zeros(1, 3, 32)
    with pytest.raises(ValueError, match="sinks must hold"):
        sattn.block_mass(q, kv, idx, lse, block_keys=32, sinks=torch.zeros(31), sink_mode="key0")

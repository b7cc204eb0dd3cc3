"""sattn_indexed_fwd_noalloc (split-K partials in the library's fixed per-GPU scratch) against
sattn_indexed_fwd (partials in a caller workspace), through the C ABI.

Two calls in a row, the second with a smaller input, so that the second runs over a scratch that
still holds the first call's partials; each output must equal the regular entry point's bit for bit
(same kernels, same slices) and match the oracle at the usual bars.  Also: a call that needs no
scratch (one slice), and a call whose partials would not fit, which must be refused.
"""
import pytest
import torch

import sliding_window_attention_index_amd as sattn
import workloads as W
from parity import SINK_NAMES, compare, oracle_indexed

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()
    return torch.device("cuda:0")


def _both(case, dev, splits):
    q, kv, idx = case.q.to(dev), case.kv.to(dev), case.topk_idxs.to(dev)
    sinks = case.sinks.to(dev) if case.sinks is not None else None
    mode = SINK_NAMES[case.sink_mode]
    o_ref, l_ref = sattn.indexed_fwd(q, kv, idx, softmax_scale=case.scale, sinks=sinks, sink_mode=mode,
                                     num_splits=splits, return_lse=True)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    sattn.indexed_fwd_noalloc(q, kv, idx, out=o, lse=lse, softmax_scale=case.scale, sinks=sinks, sink_mode=mode,
                              num_splits=splits)
    torch.cuda.synchronize(dev)
    return o.cpu(), lse.cpu(), o_ref.cpu(), l_ref.cpu()


def _check(case, dev, splits):
    o, lse, o_ref, l_ref = _both(case, dev, splits)
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"{case.name}: noalloc differs from the workspace call"
    B, M, H, D = case.q.shape
    ro, rl = oracle_indexed(case)
    compare(o.reshape(B * M, H, D), ro, case.q.dtype, f"{case.name} o")
    compare(lse.reshape(B * M, H), rl, case.q.dtype, f"{case.name} lse", lse=True)


@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_NULL, W.SINK_KEY0])
def test_noalloc_two_calls_second_smaller(dev, mode):
    big = W.sparse_decode_case(seed=3, sink_mode=mode, name=f"noalloc_big_m{mode}")  # 64 x 64 heads, 8 slices
    small = W.sparse_decode_case(seed=4, batch=5, total_tokens=16384, n_pick=700, num_splits=3, sink_mode=mode,
                                 name=f"noalloc_small_m{mode}")
    _check(big, dev, big.num_splits)
    _check(small, dev, small.num_splits)


def test_noalloc_single_slice_and_fp32(dev):
    case = W.sparse_prefill_case(q_len=300, total_tokens=4096, n_pick=64, first_pos=0, name="noalloc_prefill")
    _check(case, dev, 1)
    rng = torch.Generator().manual_seed(2)
    idx = torch.stack([torch.randperm(200, generator=rng)[:64] for _ in range(6)]).view(1, 6, 64).to(torch.int32)
    c32 = W.make_indexed_case("noalloc_fp32", 1, 6, 8, 64, 200, idx.numpy(), W.SINK_NULL, dtype=torch.float32,
                              seed=5, num_splits=4)
    _check(c32, dev, 4)


def test_noalloc_refuses_partials_beyond_scratch(dev):
    q = torch.zeros(128, 1, 64, 128, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(128, 40, 128, dtype=torch.bfloat16, device=dev)
    idx = torch.full((128, 1, 32), -1, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    with pytest.raises(sattn.SattnError) as e:
        sattn.indexed_fwd_noalloc(q, kv, idx, out=out, num_splits=16)
    assert e.value.status == 9

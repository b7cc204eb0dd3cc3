"""GPU parity of top-k attention over an fp8 cache (sattn_indexed_fp8_fwd) against the oracle.

Rows are e4m3 codes times a power-of-two scale per row on the first 128 - rope_dims dims and bf16
on the last rope_dims.  Tolerances are those of the bf16 indexed path (the dequantised rows are
exact in bf16): max-abs 1e-2 + 2^-8 |o| on the output (the full-size prefill and decode shapes: 1e-2
on the value before the output's rounding, tests/parity.py), 2e-3 on the lse, for unit-normal rows as
there (the probabilities are rounded to bf16 before the PV product, an error of up to
2^-8 sum_i p_i |v_i|, which that bound covers only when |v| stays near |o|).  Because the kernel turns
every fp8 value into the exact bf16 value before the products, its output must also equal, bit
for bit, the bf16 kernel's over a bf16 cache holding the dequantised rows, when both place the same
entries in the same tile rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sliding_window_attention_index_amd as sattn
import workloads as W
from oracle import fp8_cache as F8
from parity import SINK_NAMES, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()
    return torch.device("cuda:0")


def _case(seed, B, M, H, N, K, rd, pad=0, spread=0):
    kv8, sc, rope = W.fp8_cache(seed, B, N, 128, rd, scale_spread=spread)
    g = torch.Generator().manual_seed(seed + 1)
    q = torch.randn(B, M, H, 128, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(B * M)]).view(B, M, K).to(torch.int32)
    if pad:
        idx[:, :, K - pad:] = -1
    sinks = torch.randn(H, generator=g)
    return q, kv8, sc, (rope if rd else None), idx, sinks


def _run(dev, q, kv8, sc, rope, idx, sinks, mode, splits):
    return sattn.indexed_fp8_fwd(q.to(dev), kv8.to(dev), sc.to(dev), None if rope is None else rope.to(dev),
                                 idx.to(dev), sinks=sinks.to(dev) if mode else None, sink_mode=SINK_NAMES[mode],
                                 num_splits=splits, return_lse=True)


CASES = [
    # seed, B, M, H, N, K, rope_dims, pad, sink mode, splits
    (1, 2, 5, 32, 300, 64, 64, 0, 0, 1),
    (2, 2, 5, 32, 300, 64, 0, 0, 0, 1),
    (3, 1, 7, 64, 500, 100, 64, 9, 1, 1),     # ragged last block, pads, key-0 sink, two head groups
    (4, 1, 7, 32, 500, 100, 0, 3, 2, 1),      # null sink
    (5, 2, 3, 32, 2000, 700, 64, 0, 2, 3),    # split-K: lists longer than a staged chunk
    (6, 3, 2, 32, 700, 129, 0, 1, 1, 4),
    (7, 1, 1, 32, 40, 33, 64, 33, 2, 1),      # every entry -1: o = 0, lse = sink
    (8, 1, 4096, 32, 1500, 70, 0, 5, 1, 1),   # 4096 tasks: the 2-tile-ring launch, no rotary dims
    (9, 1, 2048, 64, 1500, 100, 64, 0, 2, 2), # 8192 tasks with two slices, rotary dims
    (10, 1, 3, 96, 3000, 1500, 64, 7, 1, 1),  # one slice of three 512-entry staging chunks, three head groups
    (11, 1, 4, 32, 3000, 1100, 0, 0, 2, 1),   # ... and of 1100 entries, no rotary dims, null sink
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_indexed_fp8_matches_oracle(dev, case):
    seed, B, M, H, N, K, rd, pad, mode, splits = case
    q, kv8, sc, rope, idx, sinks = _case(seed, B, M, H, N, K, rd, pad)
    o, lse = _run(dev, q, kv8, sc, rope, idx, sinks, mode, splits)
    torch.cuda.synchronize(dev)
    o_ref, l_ref = F8.indexed_fp8(q, kv8, sc, rope, idx, softmax_scale=1.0 / np.sqrt(128), sinks=sinks,
                                  sink_mode=mode)
    e = compare(o, o_ref, torch.bfloat16, f"fp8 case {case} o")
    compare(lse, l_ref, torch.bfloat16, f"fp8 case {case} lse", lse=True)
    print(f"[parity] indexed_fp8 {case}: max_abs {e:.3e}", flush=True)


@pytest.mark.parametrize("rd,mode,splits", [(64, 0, 1), (0, 1, 1), (64, 2, 4), (0, 0, 2)])
def test_indexed_fp8_equals_bf16_kernel_on_dequantised_rows(dev, rd, mode, splits):
    """Rows scaled over 2^-4..2^4 (every scale exponent path).  The bf16 kernel of launches with 4096
    or more (query, slice) pairs (one wave per query, 32 heads and slice) places list entry
    (r % 4) * 8 + r / 4 of a 32-entry block in tile row r, the fp8 kernel entry r; the bf16 kernel is
    given each block's entries in that order so that both see the same tiles and sum in the same
    order.  Lists of 384 entries (12 blocks) with pads; slices are whole blocks."""
    M = 2048  # 4096 queries: the bf16 launch that sums a slice's blocks in order within one wave
    q, kv8, sc, rope, idx, sinks = _case(11 + rd + mode, 2, M, 32, 800, 384, rd, 5, spread=4)
    rows = torch.from_numpy(F8.dequant_rows(kv8, sc, rope)).to(torch.bfloat16)
    assert torch.equal(rows.float(), torch.from_numpy(F8.dequant_rows(kv8, sc, rope)))  # exact in bf16
    r = torch.arange(32)
    entry_of_row = (r % 4) * 8 + r // 4
    idx16 = idx.clone().view(2, M, 12, 32)
    idx16[..., entry_of_row] = idx.view(2, M, 12, 32)
    idx16 = idx16.view(2, M, 384).contiguous()
    o8, l8 = _run(dev, q, kv8, sc, rope, idx, sinks, mode, splits)
    o16, l16 = sattn.indexed_fwd(q.to(dev), rows.to(dev), idx16.to(dev), sinks=sinks.to(dev) if mode else None,
                                 sink_mode=SINK_NAMES[mode], num_splits=splits, return_lse=True)
    torch.cuda.synchronize(dev)
    assert torch.equal(o8.cpu(), o16.cpu()) and torch.equal(l8.cpu(), l16.cpu())


def _full_compare(o, lse, o_ref, l_ref, H, what):
    e = compare(o.reshape(-1, H, 128), o_ref, torch.bfloat16, f"{what} o", literal=True)
    compare(lse.reshape(-1, H), l_ref, torch.bfloat16, f"{what} lse", lse=True)
    return e


def test_indexed_fp8_prefill_shape_full(dev):
    """The prefill shape with an fp8 cache as the bench times it (rd = 64): 8192 queries x 32 heads,
    8320 rows, 640-entry lists; every element of o and lse."""
    c = W.sparse_prefill_case(seed=0)
    kv8, sc, rope = W.fp8_cache(3, 1, c.kv.shape[1], 128, 64, scale_spread=0)
    o, lse = sattn.indexed_fp8_fwd(c.q.to(dev), kv8.to(dev), sc.to(dev), rope.to(dev), c.topk_idxs.to(dev),
                                   softmax_scale=c.scale, return_lse=True)
    torch.cuda.synchronize(dev)
    o, lse = o.cpu(), lse.cpu()
    e = 0.0
    for r0 in range(0, 8192, 2048):
        rows = np.arange(r0, r0 + 2048)
        o_ref, l_ref = F8.indexed_fp8(c.q, kv8, sc, rope, c.topk_idxs, softmax_scale=c.scale, rows=rows)
        e = max(e, _full_compare(o[0, r0:r0 + 2048], lse[0, r0:r0 + 2048], o_ref, l_ref, 32, f"fp8 prefill rows {r0}.."))
    print(f"[parity] indexed_fp8 prefill shape, all rows: max_abs {e:.3e}", flush=True)


@pytest.mark.parametrize("rd", [64, 0])
def test_indexed_fp8_decode_shape_split_full(dev, rd):
    """The decode shape with an fp8 cache: 64 rows x 64 heads, 32896-row caches, 2048 entries, 8 splits
    (rd = 64 is the benched layout); every element of o and lse."""
    c = W.sparse_decode_case(seed=0)
    kv8, sc, rope = W.fp8_cache(4, 64, c.kv.shape[1], 128, rd, scale_spread=0)
    rope_d = rope.to(dev) if rd else None
    o, lse = sattn.indexed_fp8_fwd(c.q.to(dev), kv8.to(dev), sc.to(dev), rope_d, c.topk_idxs.to(dev),
                                   softmax_scale=c.scale, num_splits=8, return_lse=True)
    torch.cuda.synchronize(dev)
    o_ref, l_ref = F8.indexed_fp8(c.q, kv8, sc, rope if rd else None, c.topk_idxs, softmax_scale=c.scale)
    e = _full_compare(o.cpu(), lse.cpu(), o_ref, l_ref, 64, f"fp8 decode rd={rd}")
    print(f"[parity] indexed_fp8 decode shape rd={rd}, 8 splits, all rows: max_abs {e:.3e}", flush=True)

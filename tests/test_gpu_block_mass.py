"""GPU parity of the per-block attention mass (sattn_block_mass) against the oracle.

Both sides are given the same fp32 log-sum-exp, so the comparison isolates the kernel's own
arithmetic: an fp32 logit (bf16 or fp32 products summed in fp32 over head_dim), one exp2 and an
fp32 sum per block.  The logit's rounding error is at most about head_dim * 2^-24 * scale *
sum_d |q_d k_d|, which for the unit-normal inputs here (sum ~ 0.64 head_dim) is below 6e-5 in
natural-log units at head_dim 128; the mass inherits it as a relative error, and exp2 and the
summation add a few ulp.  Tolerance: |got - ref| <= 1e-4 * ref + 1e-6 per element.

Large cases (the bench's prefill and decode shapes) take the lse from the GPU attention itself,
as the three-stage flow does (partial statistics per slice, merged, then normalise and block-sum),
and compare sampled rows; a property check (masses plus the null sink's share sum to 1) covers
every row.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sliding_window_attention_index_amd as sattn
import workloads as W
from oracle import index_lists as IL
from parity import SINK_NAMES, run_indexed, sample_rows

pytestmark = pytest.mark.gpu

RTOL, ATOL = 1e-4, 1e-6


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()
    return torch.device("cuda:0")


def _log(name, err):
    print(f"[parity] block_mass {name}: max_abs {err:.3e}", flush=True)


def _gpu_mass(case, dev, lse, block_keys, idx=None):
    sinks = case.sinks.to(dev) if case.sinks is not None else None
    m = sattn.block_mass(case.q.to(dev), case.kv.to(dev), (case.topk_idxs if idx is None else idx).to(dev),
                         lse.to(dev).contiguous(), block_keys=block_keys, softmax_scale=case.scale, sinks=sinks,
                         sink_mode=SINK_NAMES[case.sink_mode])
    torch.cuda.synchronize(dev)
    B, M, H = case.q.shape[:3]
    return m.cpu().numpy().astype(np.float64).reshape(B * M, H, -1)


def _oracle_mass(case, lse, block_keys, rows=None):
    return IL.block_mass(case.q, case.kv, case.topk_idxs.numpy(), lse.numpy(), scale=case.scale,
                         block_keys=block_keys, sinks=case.sinks, sink_mode=case.sink_mode, rows=rows)


def _compare(got, ref, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(got - ref))
        allowed = np.where(np.isinf(ref), 0.0, RTOL * np.abs(ref) + ATOL)
    bad = ~(err <= allowed)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, np.nan_to_num(err, nan=np.inf), -1)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} out of tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r}")
    return float(err.max()) if err.size else 0.0


def _oracle_lse(case):
    """The oracle's log-sum-exp of each list (null sink included), rounded to fp32 for both sides."""
    import oracle
    _, lse = oracle.indexed(case.q, case.kv, case.topk_idxs, scale=case.scale, sinks=case.sinks,
                            sink_mode=case.sink_mode)
    B, M, H = case.q.shape[:3]
    return torch.from_numpy(np.asarray(lse, dtype=np.float32).reshape(B, M, H))


def _lists(rng, B, M, N, K, pattern):
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            if pattern == "all" or N == 0:
                continue
            n = min(K, N) if pattern == "none" else int(rng.integers(1, min(K, N) + 1))
            idx[b, t, :n] = rng.choice(N, size=n, replace=False)
            if pattern in ("some", "oob"):
                idx[b, t] = idx[b, t, rng.permutation(K)]
            if pattern == "oob":
                idx[b, t, ::7] = N + 3 + t  # outside the cache: not a key
    return idx


CASES = [
    # name, B, M, H, D, N, K, block_keys, list pattern, dtype
    ("mfma_bk32_ragged", 2, 5, 32, 128, 300, 200, 32, "some", torch.bfloat16),
    ("mfma_bk64_d64", 1, 7, 64, 64, 500, 256, 64, "none", torch.bfloat16),
    ("mfma_bk96", 2, 3, 32, 128, 1500, 1100, 96, "some", torch.bfloat16),
    ("mfma_block_spans_chunks", 2, 3, 32, 128, 1500, 1100, 1088, "some", torch.bfloat16),
    ("mfma_one_block", 1, 4, 32, 128, 100, 40, 128, "some", torch.bfloat16),
    ("mfma_all_pad", 1, 3, 32, 128, 50, 40, 32, "all", torch.bfloat16),
    ("mfma_out_of_range", 1, 4, 32, 128, 64, 40, 32, "oob", torch.bfloat16),
    ("mfma_decode_slices", 4, 1, 64, 128, 5000, 2048, 64, "some", torch.bfloat16),
    # 4096 (query, 32 heads) tasks: the launch with a 2-tile ring per wave
    ("mfma_many_d64", 1, 2048, 64, 64, 1000, 256, 64, "some", torch.bfloat16),
    ("mfma_many_d128", 1, 4096, 32, 128, 2000, 160, 32, "oob", torch.bfloat16),
    ("valu_bk7", 2, 3, 32, 128, 200, 70, 7, "some", torch.bfloat16),
    ("valu_h16", 2, 3, 16, 64, 200, 70, 32, "some", torch.bfloat16),
    ("valu_fp32", 1, 6, 8, 64, 200, 64, 16, "some", torch.float32),
]


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_KEY0, W.SINK_NULL])
def test_block_mass_cases(dev, spec, mode):
    name, B, M, H, D, N, K, bk, pattern, dt = spec
    rng = np.random.default_rng(21)
    idx = _lists(rng, B, M, N, K, pattern)
    if mode == W.SINK_KEY0 and pattern != "all":
        for b in range(B):  # make row 0 listed in every query of batch row 0 (the bias must land)
            for t in range(M):
                if 0 not in idx[b, t] and b == 0:
                    idx[b, t, K // 2] = 0
    case = W.make_indexed_case(f"{name}_m{mode}", B, M, H, D, N, idx, mode, dtype=dt, seed=13)
    lse = _oracle_lse(case)
    got = _gpu_mass(case, dev, lse, bk)
    ref = _oracle_mass(case, lse, bk)
    _log(case.name, _compare(got, ref, case.name))


@pytest.mark.parametrize("H,bk", [(32, 64), (16, 5)])
def test_block_mass_lse_minus_inf(dev, H, bk):
    """An lse of -inf with valid entries gives +inf for blocks holding them and 0 for the others."""
    rng = np.random.default_rng(4)
    idx = _lists(rng, 1, 3, 200, 160, "none")
    idx[0, 1, 64:] = -1  # blocks past entry 64 are empty for query 1
    case = W.make_indexed_case("lse_ninf", 1, 3, H, 128, 200, idx, W.SINK_NONE, seed=2)
    lse = torch.full((1, 3, H), -float("inf"))
    got = _gpu_mass(case, dev, lse, bk)
    ref = _oracle_mass(case, lse, bk)
    assert np.array_equal(np.isposinf(got), np.isposinf(ref)) and np.array_equal(got == 0, ref == 0)


def test_block_mass_sums_to_one_with_gpu_lse(dev):
    """Prefill lists at positions 0.. (short lists, -1 padded) with the GPU's own lse: masses plus the
    null sink's share sum to 1 in every row and head."""
    for mode in (W.SINK_NONE, W.SINK_KEY0, W.SINK_NULL):
        case = W.sparse_prefill_case(q_len=300, total_tokens=4096, n_pick=64, first_pos=0, sink_mode=mode,
                                     name=f"mass_sum_m{mode}")
        _, lse = run_indexed(case, dev)
        got = _gpu_mass(case, dev, lse.cpu(), 64)
        total = got.sum(-1)
        if mode == W.SINK_NULL:
            total = total + np.exp(case.sinks.double().numpy()[None, :] - lse.cpu().double().numpy().reshape(300, -1))
        err = float(np.abs(total - 1.0).max())
        assert err < 1e-4, (mode, err)
        _log(case.name + " sum-to-one", err)


def test_block_mass_full_prefill_sampled(dev):
    """The bench's prefill workload: 8192 queries x 32 heads x 640 listed rows, blocks of 64 entries,
    lse from the GPU attention; sampled rows against the oracle, sum-to-one on every row."""
    case = W.sparse_prefill_case()
    _, lse = run_indexed(case, dev)
    lse = lse.cpu()
    got = _gpu_mass(case, dev, lse, 64)
    rows = sample_rows(case.q.shape[1], 48, seed=8, must=[0, 8191])
    _log("sparse_prefill full (sampled)", _compare(got[rows], _oracle_mass(case, lse, 64, rows=rows), "prefill"))
    assert float(np.abs(got.sum(-1) - 1.0).max()) < 1e-4


def test_block_mass_full_decode_three_stages(dev):
    """Decode workload: 64 rows x 64 heads, 2048-entry lists over 32896-row caches.  Stage 1 and 2
    are the split-K attention (8 slices) and its merge; stage 3 is the block mass with that lse."""
    case = W.sparse_decode_case(sink_mode=W.SINK_NULL)
    _, lse = run_indexed(case, dev)  # num_splits = 8, merged
    lse = lse.cpu()
    got = _gpu_mass(case, dev, lse, 64)
    _log("sparse_decode full", _compare(got, _oracle_mass(case, lse, 64), "decode"))
    share = np.exp(case.sinks.double().numpy()[None, :] - lse.double().numpy().reshape(64, -1))
    assert float(np.abs(got.sum(-1) + share - 1.0).max()) < 1e-4

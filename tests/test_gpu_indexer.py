"""GPU parity of the synthetic indexer's top-k lists (sattn_indexer_topk) against the oracle.

The window part of every list is integer work and must equal the oracle's bit for bit.  The
compressed part depends on scores: the kernel sums bf16 products (exact in fp32) in fp32 with
MFMA, the oracle in fp64.  Two kinds of input:

* integer-valued qr and kidx (entries in [-3, 3]): every score is a small integer, exact on both
  sides, and ties are common, so the lists (ties to the lower row included) must be identical;
* N(0, 1) inputs: a score can differ from the fp64 one by at most eps = 2 * rank * 2^-24 *
  sum_i |qr_i kidx_i| (fp32 summation of `rank` exact products).  The kernel's chosen set is
  accepted when it has the right size, every chosen row is visible, no chosen row scores below
  tau - eps and no unchosen visible row above tau + eps (tau: the oracle's k-th largest score),
  and it agrees with the oracle's set on every row whose score lies outside [tau - eps, tau + eps].
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sliding_window_attention_index_amd as sattn
import workloads as W
from oracle import index_lists as IL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()
    return torch.device("cuda:0")


def _run(dev, qr, kidx, start_pos, window, ratio, topk):
    B, M, _ = qr.shape
    n_comp = kidx.shape[1]
    out = sattn.indexer_topk(qr.to(dev), kidx.to(dev), torch.tensor(start_pos, dtype=torch.int32, device=dev), M,
                             window=window, ratio=ratio, n_comp=n_comp, topk=topk)
    torch.cuda.synchronize(dev)
    return out.cpu().numpy()


def _check_valid(got, qr, kidx, start_pos, window, ratio, topk, rows, what):
    """got: [len(rows), window + topk] lists for flat rows b * q_len + t."""
    B, M, r = qr.shape
    n_comp = kidx.shape[1]
    qf = qr.float().numpy().astype(np.float64)
    kf = kidx.float().numpy().astype(np.float64)
    ref = IL.indexer_lists(qr, kidx, start_pos, M, window, ratio, n_comp, topk, rows=rows)
    assert np.array_equal(got[:, :window], ref[:, :window]), f"{what}: window part differs"
    n_band = 0
    for i, row in enumerate(rows):
        b, t = divmod(int(row), M)
        p = int(start_pos[b]) + t
        vis = min(n_comp, (p + 1) // ratio) if ratio > 0 and p >= 0 else 0
        want = min(topk, vis)
        comp = got[i, window:]
        assert (comp[want:] == -1).all(), f"{what}: row {row} has {int((comp >= 0).sum())} entries, want {want}"
        c = comp[:want].astype(np.int64) - window
        assert (c >= 0).all() and (c < vis).all(), f"{what}: row {row} lists an invisible row"
        assert (np.diff(c) > 0).all(), f"{what}: row {row} is not strictly increasing"
        if want == 0:
            continue
        s = kf[b, :vis] @ qf[b, t]
        eps = 2.0 * r * 2.0 ** -24 * (np.abs(kf[b, :vis] * qf[b, t]).sum(1)).max()
        tau = np.sort(s)[::-1][want - 1]
        chosen = np.zeros(vis, bool)
        chosen[c] = True
        assert (s[chosen] >= tau - eps).all(), f"{what}: row {row} chose a row scoring below the threshold"
        assert (s[~chosen] <= tau + eps).all(), f"{what}: row {row} left out a row scoring above the threshold"
        ref_set = np.zeros(vis, bool)
        ref_set[ref[i, window:window + want] - window] = True
        outside = np.abs(s - tau) > eps
        assert np.array_equal(chosen[outside], ref_set[outside]), f"{what}: row {row} differs away from the threshold"
        n_band += int((~outside & (chosen != ref_set)).sum())
    print(f"[parity] indexer {what}: {len(rows)} rows valid, {n_band} entries swapped inside the eps band",
          flush=True)


CASES = [
    # B, q_len, n_comp, rank, window, ratio, topk, start_pos
    (2, 70, 40, 16, 8, 4, 6, [0, 100]),         # ragged query tiles, few visible rows early on
    (1, 33, 200, 32, 16, 1, 64, [150]),         # ratio 1
    (2, 64, 300, 64, 128, 4, 32, [1000, 1]),     # window larger than many positions
    (1, 40, 257, 128, 4, 2, 100, [480]),        # rank 128, ragged candidate tail
    (3, 5, 64, 64, 8, 4, 512, [300, 0, 17]),    # topk beyond every visible count
    (1, 16, 50, 16, 8, 4, 0, [400]),            # topk 0: window part only
    (1, 9, 1100, 64, 32, 4, 700, [4399]),       # many tiles per wave, k in the middle
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_indexer_integer_exact(dev, case):
    B, M, n_comp, r, win, ratio, topk, sp = case
    qr, kidx = W.indexer_inputs(seed=M + n_comp, batch=B, q_len=M, n_comp=n_comp, rank=r, integer=True)
    got = _run(dev, qr, kidx, sp, win, ratio, topk)
    ref = IL.indexer_lists(qr, kidx, sp, M, win, ratio, n_comp, topk)
    assert got.shape == ref.shape
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} entries differ, first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    print(f"[parity] indexer integer case {case}: bit-exact", flush=True)


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_indexer_normal_valid(dev, case):
    B, M, n_comp, r, win, ratio, topk, sp = case
    qr, kidx = W.indexer_inputs(seed=7 * M + n_comp, batch=B, q_len=M, n_comp=n_comp, rank=r)
    got = _run(dev, qr, kidx, sp, win, ratio, topk).reshape(B * M, -1)
    _check_valid(got, qr, kidx, sp, win, ratio, topk, list(range(B * M)), f"normal {case}")


def test_indexer_all_scores_equal(dev):
    """Equal scores everywhere: each list takes the lowest visible rows."""
    B, M, n_comp, r, win, ratio, topk = 1, 64, 600, 64, 16, 4, 100
    qr = torch.ones(B, M, r, dtype=torch.bfloat16)
    kidx = torch.full((B, n_comp, r), 0.5, dtype=torch.bfloat16)
    sp = [300]
    got = _run(dev, qr, kidx, sp, win, ratio, topk)
    for t in range(M):
        vis = min(n_comp, (sp[0] + t + 1) // ratio)
        k = min(topk, vis)
        assert np.array_equal(got[0, t, win:win + k], win + np.arange(k))
        assert (got[0, t, win + k:] == -1).all()
    assert np.array_equal(got, IL.indexer_lists(qr, kidx, sp, M, win, ratio, n_comp, topk))


def test_indexer_no_compressed_rows(dev):
    """n_comp 0: lists hold the window part and -1."""
    qr = torch.randn(2, 10, 32).to(torch.bfloat16)
    kidx = torch.empty(2, 0, 32, dtype=torch.bfloat16)
    got = _run(dev, qr, kidx, [5, 50], 8, 4, 12)
    assert np.array_equal(got, IL.indexer_lists(qr, kidx, [5, 50], 10, 8, 4, 0, 12))


def test_indexer_negative_and_tied_scores(dev):
    """Scores of both signs, zeros (+0 and -0 products) and exact ties across wave boundaries."""
    B, M, n_comp, r, win, ratio, topk = 1, 32, 512, 16, 8, 1, 200
    g = torch.Generator().manual_seed(11)
    qr = torch.zeros(B, M, r)
    qr[..., 0] = torch.randint(-1, 2, (B, M), generator=g).float()
    kidx = torch.zeros(B, n_comp, r)
    kidx[..., 0] = torch.randint(-2, 3, (B, n_comp), generator=g).float()
    kidx[..., 1] = -0.0
    qr, kidx = qr.to(torch.bfloat16), kidx.to(torch.bfloat16)
    sp = [480]
    got = _run(dev, qr, kidx, sp, win, ratio, topk)
    assert np.array_equal(got, IL.indexer_lists(qr, kidx, sp, M, win, ratio, n_comp, topk))


def test_indexer_prefill_shape_sampled(dev):
    """The prefill shape: 8192 queries at positions 24576.. (the last 8192 of 32768 tokens), rank 64,
    8192 compressed rows (ratio 4), window 128, top 512; sampled rows against the oracle and every
    row checked for count, visibility and order."""
    B, M, n_comp, r, win, ratio, topk = 1, 8192, 8192, 64, 128, 4, 512
    sp = [24576]
    qr, kidx = W.indexer_inputs(seed=5, batch=B, q_len=M, n_comp=n_comp, rank=r)
    got = _run(dev, qr, kidx, sp, win, ratio, topk).reshape(M, -1)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, M - 1], rng.choice(M, 40, replace=False)]))
    _check_valid(got[rows], qr, kidx, sp, win, ratio, topk, rows, "prefill 8192 x 8192 sampled")
    comp = got[:, win:]
    assert (comp >= 0).all()  # every query sees at least 6144 rows > 512
    assert (np.diff(comp, axis=1) > 0).all()
    vis = (sp[0] + np.arange(M) + 1) // ratio
    assert (comp[:, -1] - win < vis).all()


# The cases below steer the kernel's selection strategy through its inputs (the result must not
# depend on it): the exact scores of every row decide the lists, whichever way they are found.

def test_indexer_threshold_below_bin_window(dev):
    """Top 70 % of the visible rows: the k-th score lies below the bin window placed from the scores'
    root mean square (negative for these normal scores)."""
    qr, kidx = W.indexer_inputs(seed=21, batch=1, q_len=40, n_comp=600, rank=64)
    got = _run(dev, qr, kidx, [2399], 16, 4, 420).reshape(40, -1)
    _check_valid(got, qr, kidx, [2399], 16, 4, 420, list(range(40)), "threshold below the bin window")


def test_indexer_threshold_above_bin_window(dev):
    """The first 32 rows' index keys are 10^4 times smaller than the rest, so the window placed from
    their scores lies far below the k-th score."""
    qr, kidx = W.indexer_inputs(seed=22, batch=1, q_len=40, n_comp=600, rank=64)
    kidx[:, :32] = (kidx[:, :32].float() * 1e-4).to(torch.bfloat16)
    got = _run(dev, qr, kidx, [2399], 16, 4, 60).reshape(40, -1)
    _check_valid(got, qr, kidx, [2399], 16, 4, 60, list(range(40)), "threshold above the bin window")


def test_indexer_large_tied_threshold_bin(dev):
    """Integer scores in [-16, 16] over 600 rows, top 200: the k-th score's value is shared by 65 to
    128 rows for most queries, which are then ordered by row."""
    g = torch.Generator().manual_seed(25)
    qr = torch.randint(-1, 2, (1, 40, 16), generator=g).to(torch.bfloat16)
    kidx = torch.randint(-1, 2, (1, 600, 16), generator=g).to(torch.bfloat16)
    got = _run(dev, qr, kidx, [2399], 16, 4, 200)
    assert np.array_equal(got, IL.indexer_lists(qr, kidx, [2399], 40, 16, 4, 600, 200))


def test_indexer_more_than_8192_visible_rows(dev):
    """Queries that see 8704 compressed rows (beyond one bitmap's 8192)."""
    qr, kidx = W.indexer_inputs(seed=26, batch=1, q_len=8, n_comp=8704, rank=64)
    sp = [4 * 8704 - 1]
    got = _run(dev, qr, kidx, sp, 32, 4, 300).reshape(8, -1)
    _check_valid(got, qr, kidx, sp, 32, 4, 300, list(range(8)), "8704 visible rows")
    qi, ki = W.indexer_inputs(seed=27, batch=1, q_len=8, n_comp=8704, rank=64, integer=True)
    got = _run(dev, qi, ki, sp, 32, 4, 300)
    assert np.array_equal(got, IL.indexer_lists(qi, ki, sp, 8, 32, 4, 8704, 300))

"""Pins of the top-k list oracle (oracle/index_lists.py) against facts other than itself.

* Simulation: replay the cache writes the DeepSeek-V4 CSA/HCA article describes (§3.3: token p
  written to ring slot p % window; a compressed row emitted each time (pos + 1) % ratio == 0,
  stored after the window region) and read off, after position p, which rows hold the last
  `window` positions and which compressed rows exist.  The oracle's closed form must list exactly
  those rows, in position / emission order, then -1.
* The article's example (§2.2): a window list such as [100, 101, 102, 103].
* Counts: min(p + 1, window) window rows and min(n_comp, (p + 1) // ratio) compressed rows.
* Planted mistakes in a copy of the oracle must fail the simulation pin.

Block mass (per-block attention mass normalised by the global log-sum-exp):
* with the lse of the same key set, the masses plus the null sink's share sum to 1;
* they equal a dense softmax over every cache row (unlisted rows masked, the null sink an
  extra column) summed per block of list positions;
* an lse merged from per-chunk partials normalises exactly as the one-pass lse;
* planted mistakes (binning by cache row, dropped key-0 bias, unscaled logits) fail.
"""
from __future__ import annotations

import inspect
import math
import textwrap

import numpy as np
import pytest
import torch

import oracle
from oracle import index_lists as IL


def simulate(p_max: int, window: int, ratio: int, n_comp: int):
    """Per position p: (rows of the window positions in order, compressed rows in order)."""
    ring = [-1] * window          # ring slot -> position held
    n_emitted = 0
    out = {}
    for pos in range(p_max + 1):
        ring[pos % window] = pos                      # the ring write
        if ratio > 0 and (pos + 1) % ratio == 0 and n_emitted < n_comp:
            n_emitted += 1                            # the lazy compressor fires
        held = sorted((ring[s], s) for s in range(window) if ring[s] >= 0 and ring[s] > pos - window)
        out[pos] = ([s for _, s in held], [window + j for j in range(n_emitted)])
    return out


def check_against_simulation(fn, window, ratio, n_comp, p_max):
    sim = simulate(p_max, window, ratio, n_comp)
    for p in range(p_max + 1):
        got = fn(p, window, ratio, n_comp)
        w_rows, c_rows = sim[p]
        want = w_rows + [-1] * (window - len(w_rows)) + c_rows + [-1] * (n_comp - len(c_rows))
        assert got == want, (window, ratio, n_comp, p, got, want)


CASES = [(8, 4, 6, 40), (5, 3, 10, 33), (16, 0, 0, 40), (4, 1, 3, 12), (1, 4, 2, 12), (7, 8, 16, 70)]


@pytest.mark.parametrize("window,ratio,n_comp,p_max", CASES)
def test_oracle_matches_cache_simulation(window, ratio, n_comp, p_max):
    check_against_simulation(IL.query_list, window, ratio, n_comp, p_max)


def test_page_example_window_indices():
    # a 128-row window at position 103 holds positions 0..103 in slots 0..103: the example's
    # consecutive indices [100, 101, 102, 103] appear in order
    lst = IL.query_list(103, 128, 4, 0)
    assert lst[100:104] == [100, 101, 102, 103]
    assert lst[104:] == [-1] * 24


def test_counts_and_padding():
    window, ratio, n_comp = 128, 4, 64
    for p in (0, 3, 4, 127, 128, 255, 1000, -1):
        lst = np.array(IL.query_list(p, window, ratio, n_comp))
        nw = min(max(p + 1, 0), window)
        nc = min(n_comp, max(p + 1, 0) // ratio)
        assert (lst[:window] >= 0).sum() == nw and (lst[nw:window] == -1).all()
        assert (lst[window:] >= 0).sum() == nc and (lst[window + nc:] == -1).all()
        valid = lst[lst >= 0]
        assert len(set(valid.tolist())) == len(valid)  # distinct rows


def test_topk_lists_shape_and_rows():
    sp = [0, 5, 130]
    full = IL.topk_lists(sp, 3, 8, 4, 10)
    assert full.shape == (3, 3, 18) and full.dtype == np.int32
    some = IL.topk_lists(sp, 3, 8, 4, 10, rows=[8, 0, 4])
    assert (some == full.reshape(9, 18)[[8, 0, 4]]).all()
    assert full[2, 1].tolist() == IL.query_list(131, 8, 4, 10)


MUTANTS = {
    "slot_plus_one": ("win.append(q % window)", "win.append((q + 1) % window)"),
    "window_one_short": ("range(max(0, p - window + 1), p + 1)", "range(max(0, p - window + 2), p + 1)"),
    "compress_trigger_early": ("if (c + 1) * ratio - 1 <= p:", "if c * ratio <= p:"),
    "compress_rows_from_zero": ("comp.append(window + c)", "comp.append(c)"),
    "no_padding_order": ("win += [-1] * (window - len(win))", "win = [-1] * (window - len(win)) + win"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail(name):
    old, new = MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(IL.query_list))
    assert old in src
    ns = {}
    exec(src.replace(old, new), ns)
    with pytest.raises(AssertionError):
        for window, ratio, n_comp, p_max in CASES:
            check_against_simulation(ns["query_list"], window, ratio, n_comp, p_max)


# ---------------------------------------------------------------------------------------------
# block mass (third stage of the chunked estimate: normalise with global statistics, sum per block)
# ---------------------------------------------------------------------------------------------
def _mass_inputs(seed, B=2, M=3, H=4, D=16, N=40, K=48, pad=True):
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q = torch.randn(B, M, H, D, generator=g)
    kv = torch.randn(B, N, D, generator=g)
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            n = K - 9 if pad and t == 1 else min(K, N)
            row = rng.choice(N, size=n, replace=False)
            if t == 0 and 0 not in row:
                row[0] = 0
            idx[b, t, :n] = row
    sinks = torch.randn(H, generator=g)
    return q, kv, idx, sinks


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_block_mass_sums_to_one(mode):
    q, kv, idx, sinks = _mass_inputs(1)
    _, lse = oracle.indexed(q, kv, idx, scale=0.25, sinks=sinks, sink_mode=mode)
    B, M, H = q.shape[:3]
    mass = IL.block_mass(q, kv, idx, lse.reshape(B, M, H), scale=0.25, block_keys=8, sinks=sinks, sink_mode=mode)
    total = mass.sum(-1)
    if mode == 2:
        total = total + np.exp(sinks.double().numpy()[None, :] - lse)
    assert np.allclose(total, 1.0, atol=1e-12)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_block_mass_matches_dense_softmax(mode):
    """Dense softmax over all N cache rows (unlisted rows masked; null sink = extra column), then
    the probability of each list entry's row summed per block of list positions."""
    q, kv, idx, sinks = _mass_inputs(2)
    B, M, H, D = q.shape
    N, K = kv.shape[1], idx.shape[2]
    _, lse = oracle.indexed(q, kv, idx, scale=0.25, sinks=sinks, sink_mode=mode)
    mass = IL.block_mass(q, kv, idx, lse.reshape(B, M, H), scale=0.25, block_keys=16, sinks=sinks, sink_mode=mode)
    for b in range(B):
        for t in range(M):
            logits = 0.25 * (q[b, t].double() @ kv[b].double().T)  # [H, N]
            listed = torch.zeros(N, dtype=torch.bool)
            for x in idx[b, t]:
                if 0 <= x < N:
                    listed[x] = True
            logits = logits.masked_fill(~listed, -math.inf)
            if mode == 1:
                logits[:, 0] += sinks.double()
            if mode == 2:
                logits = torch.cat([logits, sinks.double()[:, None]], 1)
            prob = torch.softmax(logits, -1)[:, :N]
            want = np.zeros((H, (K + 15) // 16))
            for k, x in enumerate(idx[b, t]):
                if 0 <= x < N:
                    want[:, k // 16] += prob[:, x].numpy()
            assert np.allclose(mass[b * M + t], want, atol=1e-12)


def test_block_mass_with_merged_statistics():
    """The page's two stages before it: per-chunk statistics merged into global ones give the same
    normalisation as one pass (stage 3 only needs the merged lse)."""
    q, kv, idx, sinks = _mass_inputs(3)
    B, M, H = q.shape[:3]
    K = idx.shape[2]
    _, lse1 = oracle.indexed(q, kv, idx, scale=0.25, sinks=sinks, sink_mode=2)
    parts_o, parts_l = [], []
    for c0 in range(0, K, 20):
        sub = np.full_like(idx, -1)
        sub[:, :, c0:c0 + 20] = idx[:, :, c0:c0 + 20]
        o, l = oracle.indexed(q, kv, sub, scale=0.25)
        parts_o.append(o)
        parts_l.append(l)
    _, lse2 = oracle.merge(np.stack(parts_o), np.stack(parts_l), sinks=sinks, sink_mode=2)
    m1 = IL.block_mass(q, kv, idx, lse1.reshape(B, M, H), scale=0.25, block_keys=8, sinks=sinks, sink_mode=2)
    m2 = IL.block_mass(q, kv, idx, lse2.reshape(B, M, H), scale=0.25, block_keys=8, sinks=sinks, sink_mode=2)
    assert np.allclose(m1, m2, atol=1e-12)


MASS_MUTANTS = {
    "bins_by_cache_row": ("(slice(None), pos // block_keys)", "(slice(None), np.minimum(x, K - 1) // block_keys)"),
    "key0_bias_dropped": ("logit[:, x == 0] += snk[:, None]", "pass"),
    "unscaled_logit": ("logit = scale * (qf", "logit = (qf"),
    "lse_not_subtracted": ("np.exp(logit - ls[b, t][:, None])", "np.exp(logit)"),
}


@pytest.mark.parametrize("name", sorted(MASS_MUTANTS))
def test_block_mass_planted_mistakes_fail(name):
    old, new = MASS_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(IL.block_mass))
    assert old in src
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    saved = IL.block_mass
    IL.block_mass = ns["block_mass"]
    try:
        with pytest.raises(AssertionError):
            for mode in (1, 2):
                test_block_mass_matches_dense_softmax(mode)
    finally:
        IL.block_mass = saved

"""Pins of the top-k list oracle (oracle/index_lists.py) against facts other than itself.

* Simulation: replay the cache writes the DeepSeek-V4 CSA/HCA article describes (§3.3: token p
  written to ring slot p % window; a compressed row emitted each time (pos + 1) % ratio == 0,
  stored after the window region) and read off, after position p, which rows hold the last
  `window` positions and which compressed rows exist.  The oracle's closed form must list exactly
  those rows, in position / emission order, then -1.
* The article's example (§2.2): a window list such as [100, 101, 102, 103].
* Counts: min(p + 1, window) window rows and min(n_comp, (p + 1) // ratio) compressed rows.
* Planted mistakes in a copy of the oracle must fail the simulation pin.
"""
from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest

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

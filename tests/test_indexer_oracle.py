"""Pins of the synthetic indexer oracle (oracle/index_lists.py::indexer_lists).

* With topk at least the number of visible compressed rows, the lists equal the list builder's
  (every visible row, in order) -- the cache-write simulation pins that one.
* Scores that grow with the row index select the last `topk` visible rows; all-equal scores
  select the first `topk` (ties go to the lower row).
* Relabelling the index keys permutes the selection with them.
* The chosen rows always carry the `topk` largest scores among the visible rows (checked
  against a brute-force ranking by numpy argsort).
* Planted mistakes fail.
"""
from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest

from oracle import index_lists as IL


def _keys_with_scores(scores, r=4):
    """kidx rows whose score against qr = e_0 is `scores`."""
    k = np.zeros((1, len(scores), r))
    k[0, :, 0] = scores
    q = np.zeros((1, 1, r))
    q[0, 0, 0] = 1.0
    return q, k


def test_large_topk_equals_list_builder():
    rng = np.random.default_rng(0)
    sp, M, W, R, C = [5, 130], 7, 8, 4, 40
    qr = rng.standard_normal((2, M, 16))
    kidx = rng.standard_normal((2, C, 16))
    got = IL.indexer_lists(qr, kidx, sp, M, W, R, C, topk=C)
    assert np.array_equal(got, IL.topk_lists(sp, M, W, R, C))


def test_increasing_scores_take_the_last_rows_and_ties_the_first():
    C, W, R, k = 30, 4, 2, 5
    q, kidx = _keys_with_scores(np.arange(C, dtype=float))
    p = 40  # visible: c with 2c + 1 <= 40 -> c <= 19
    got = IL.indexer_lists(q, kidx, [p], 1, W, R, C, topk=k)[0, 0]
    assert got[W:].tolist() == [W + c for c in range(15, 20)]
    q, kidx = _keys_with_scores(np.zeros(C))
    got = IL.indexer_lists(q, kidx, [p], 1, W, R, C, topk=k)[0, 0]
    assert got[W:].tolist() == [W + c for c in range(5)]
    got = IL.indexer_lists(q, kidx, [3], 1, W, R, C, topk=k)[0, 0]  # only c = 0, 1 visible
    assert got[W:].tolist() == [W, W + 1, -1, -1, -1]


def test_relabelled_keys_permute_the_selection():
    rng = np.random.default_rng(1)
    C, W, R, k = 64, 4, 1, 9
    qr = rng.standard_normal((1, 1, 8))
    kidx = rng.standard_normal((1, C, 8))
    perm = rng.permutation(C)
    base = IL.indexer_lists(qr, kidx, [1000], 1, W, R, C, topk=k)[0, 0, W:] - W
    moved = IL.indexer_lists(qr, kidx[:, perm], [1000], 1, W, R, C, topk=k)[0, 0, W:] - W
    inv = np.argsort(perm)
    assert sorted(perm[moved].tolist()) == sorted(base.tolist())
    assert sorted(inv[base].tolist()) == sorted(moved.tolist())


def test_chosen_rows_carry_the_largest_scores():
    rng = np.random.default_rng(2)
    B, M, W, R, C, k = 2, 6, 8, 4, 100, 12
    sp = [50, 400]
    qr = rng.standard_normal((B, M, 16))
    kidx = rng.standard_normal((B, C, 16))
    got = IL.indexer_lists(qr, kidx, sp, M, W, R, C, topk=k)
    for b in range(B):
        for t in range(M):
            vis = np.array([x - W for x in IL.query_list(sp[b] + t, W, R, C)[W:] if x >= 0])
            s = kidx[b, vis] @ qr[b, t]
            want = np.sort(vis[np.argsort(-s, kind="stable")[:k]])
            chosen = got[b, t, W:]
            assert np.array_equal(chosen[chosen >= 0] - W, want)
            assert (chosen[len(want):] == -1).all()


MUTANTS = {
    "lowest_scores": ("key=lambda j: (-scores[j], visible[j])", "key=lambda j: (scores[j], visible[j])"),
    "ties_to_higher_row": ("key=lambda j: (-scores[j], visible[j])", "key=lambda j: (-scores[j], -visible[j])"),
    "invisible_rows_scored": ("visible = [x - window for x in full[window:] if x >= 0]",
                              "visible = list(range(n_comp))"),
    "rows_not_offset": ("[window + c for c in chosen]", "[c for c in chosen]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail(name):
    old, new = MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(IL.indexer_lists))
    assert old in src
    ns = {"np": np, "query_list": IL.query_list}
    exec(src.replace(old, new), ns)
    saved = IL.indexer_lists
    IL.indexer_lists = ns["indexer_lists"]
    try:
        with pytest.raises(AssertionError):
            test_large_topk_equals_list_builder()
            test_increasing_scores_take_the_last_rows_and_ties_the_first()
            test_chosen_rows_carry_the_largest_scores()
    finally:
        IL.indexer_lists = saved

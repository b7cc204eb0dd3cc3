"""Pins of the compressor pooling oracle (oracle/index_lists.py::compress_pool) against facts other
than itself (DeepSeek-V4 CSA/HCA article, §5.1 and its overlap-transform description).

* Equal scores: the softmax weights are uniform, so a compressed row is the plain mean of the
  window's entries (ratio tokens without overlap; with overlap the previous window's tokens with
  the first feature half plus its own with the second half, window 0 its own tokens only).
* A score, or an ape entry, far above the rest selects one entry exactly.
* Adding a constant to every score of a window and feature changes nothing.
* Membership: a kv that is one-hot in (token, feature) shows up only in the windows and output
  features the transform routes it to, with weight 1 / (entries of that window).
* A trailing partial window is not compressed.
* Planted mistakes fail these pins.
"""
from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest

from oracle import index_lists as IL


def _mean_pool(kv, ratio, overlap):
    B, S, F = kv.shape
    d = F // (2 if overlap else 1)
    out = np.zeros((B, S // ratio, d))
    for w in range(S // ratio):
        own = kv[:, w * ratio:(w + 1) * ratio, d:] if overlap else kv[:, w * ratio:(w + 1) * ratio, :]
        parts = [own]
        if overlap and w > 0:
            parts.append(kv[:, (w - 1) * ratio:w * ratio, :d])
        out[:, w] = np.concatenate(parts, 1).mean(1)
    return out


@pytest.mark.parametrize("overlap", [False, True])
@pytest.mark.parametrize("ratio", [1, 4, 8])
def test_equal_scores_give_the_mean(overlap, ratio):
    rng = np.random.default_rng(ratio)
    F = 16 if overlap else 8
    kv = rng.standard_normal((2, 5 * ratio + ratio - 1, F))  # a partial window at the end when ratio > 1
    got = IL.compress_pool(kv, np.zeros_like(kv), np.zeros((ratio, F)), ratio=ratio, overlap=overlap)
    assert got.shape == (2, 5, F // (2 if overlap else 1))
    assert np.allclose(got, _mean_pool(kv, ratio, overlap), atol=1e-12)


@pytest.mark.parametrize("overlap", [False, True])
def test_dominant_score_selects_one_entry(overlap):
    rng = np.random.default_rng(2)
    ratio, d = 4, 6
    F = 2 * d if overlap else d
    kv = rng.standard_normal((1, 4 * ratio, F))
    sc = np.zeros_like(kv)
    # window 2: its own token 2*ratio+1 dominates every feature (own half)
    lo = d if overlap else 0
    sc[0, 2 * ratio + 1, lo:lo + d] = 80.0
    got = IL.compress_pool(kv, sc, np.zeros((ratio, F)), ratio=ratio, overlap=overlap)
    assert np.allclose(got[0, 2], kv[0, 2 * ratio + 1, lo:lo + d], atol=1e-12)
    if overlap:  # the same token's first half dominates window 3 through the previous-window half
        sc2 = np.zeros_like(kv)
        sc2[0, 2 * ratio + 1, :d] = 80.0
        got2 = IL.compress_pool(kv, sc2, np.zeros((ratio, F)), ratio=ratio, overlap=True)
        assert np.allclose(got2[0, 3], kv[0, 2 * ratio + 1, :d], atol=1e-12)


def test_ape_is_a_per_position_score_offset():
    rng = np.random.default_rng(3)
    ratio, d = 4, 5
    kv = rng.standard_normal((1, 3 * ratio, d))
    ape = np.zeros((ratio, d))
    ape[2] = 90.0  # position 2 of every window dominates
    got = IL.compress_pool(kv, np.zeros_like(kv), ape, ratio=ratio, overlap=False)
    for w in range(3):
        assert np.allclose(got[0, w], kv[0, w * ratio + 2], atol=1e-12)


@pytest.mark.parametrize("overlap", [False, True])
def test_shift_of_scores_changes_nothing(overlap):
    rng = np.random.default_rng(4)
    ratio, d = 4, 3
    F = 2 * d if overlap else d
    kv = rng.standard_normal((1, 6 * ratio, F))
    sc = rng.standard_normal(kv.shape)
    ape = rng.standard_normal((ratio, F))
    base = IL.compress_pool(kv, sc, ape, ratio=ratio, overlap=overlap)
    shifted = IL.compress_pool(kv, sc + 7.5, ape - 2.0, ratio=ratio, overlap=overlap)
    assert np.allclose(base, shifted, atol=1e-12)


@pytest.mark.parametrize("overlap", [False, True])
def test_membership_of_each_token_and_feature(overlap):
    ratio, d, S = 4, 3, 18  # 4 complete windows, 2 tail tokens dropped
    F = 2 * d if overlap else d
    n_out = S // ratio
    for t in range(S):
        for f in range(F):
            kv = np.zeros((1, S, F))
            kv[0, t, f] = 1.0
            got = IL.compress_pool(kv, np.zeros_like(kv), np.zeros((ratio, F)), ratio=ratio, overlap=overlap)
            want = np.zeros((n_out, F // (2 if overlap else 1)))
            w = t // ratio
            if not overlap:
                if w < n_out:
                    want[w, f] = 1.0 / ratio
            elif f >= d:  # own half: window t // ratio
                if w < n_out:
                    want[w, f - d] = 1.0 / (ratio if w == 0 else 2 * ratio)
            else:  # first half: the next window, through its previous-window part
                if w + 1 < n_out:
                    want[w + 1, f] = 1.0 / (2 * ratio)
            assert np.allclose(got[0], want, atol=1e-15), (t, f)


MUTANTS = {
    "softmax_over_features": ("e = np.exp(sc - sc.max(axis=0))", "e = np.exp(sc - sc.max(axis=1, keepdims=True))"),
    "halves_swapped": ("rows_kv.append(kvf[b, t, :d])", "rows_kv.append(kvf[b, t, d:2 * d])"),
    "ape_dropped": ("rows_sc.append(scf[b, t, lo:lo + d] + apf[i, lo:lo + d])", "rows_sc.append(scf[b, t, lo:lo + d])"),
    "previous_window_off_by_one": ("t = (w - 1) * ratio + i", "t = max(0, w - 2) * ratio + i"),
    "window0_zero_padded": ("if overlap and w > 0:", "if overlap:"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail(name):
    old, new = MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(IL.compress_pool))
    assert old in src
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    saved = IL.compress_pool
    IL.compress_pool = ns["compress_pool"]
    try:
        with pytest.raises(AssertionError):
            for ov in (False, True):
                test_equal_scores_give_the_mean(ov, 4)
                test_dominant_score_selects_one_entry(ov)
                test_membership_of_each_token_and_feature(ov)
            test_ape_is_a_per_position_score_offset()
    finally:
        IL.compress_pool = saved

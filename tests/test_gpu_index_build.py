"""GPU parity of the device-side top-k list builder (sattn_build_topk_idxs) against the oracle.

Integer work: every compared entry must be bit-identical.  Large cases compare sampled rows
against the oracle and check properties of every row.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_index_amd as sattn
from oracle import index_lists as IL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def _build(dev, start_pos, q_len, window, ratio, n_comp):
    sp = torch.tensor(start_pos, dtype=torch.int32, device=dev)
    out = sattn.build_topk_idxs(sp, q_len, window=window, ratio=ratio, n_comp=n_comp)
    torch.cuda.synchronize(dev)
    return out.cpu().numpy()


SMALL = [
    # start_pos, q_len, window, ratio, n_comp
    ([0], 40, 8, 4, 10),                 # early positions: padded window, few compressed rows
    ([0, 3, 17, 100], 9, 8, 4, 6),       # compressed rows truncated at n_comp
    ([5, 1000], 7, 5, 3, 10),            # K = 15: element stores
    ([0, 50], 33, 16, 0, 0),             # pure window (no compressed region)
    ([-5, -1, 0], 8, 4, 1, 3),           # negative positions see nothing until 0
    ([127, 128, 129], 3, 128, 4, 64),    # around the ring wrap
    ([24576], 64, 128, 4, 8192),         # the prefill configuration's first queries
    ([-3, 0, 300, 5000], 5, 4, 2, 1024), # K = 1028: one wave per 4 KB piece, the last piece one chunk
    ([-3, 10, 600], 4, 4, 2, 252),       # K = 256: one piece, mostly compressed rows
    ([1000, 255], 3, 256, 0, 0),         # K = 256, window only, the ring slot wrapping inside a piece
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_build_small_bit_exact(dev, case):
    start_pos, q_len, window, ratio, n_comp = case
    got = _build(dev, start_pos, q_len, window, ratio, n_comp)
    want = IL.topk_lists(start_pos, q_len, window, ratio, n_comp)
    assert got.shape == want.shape
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_build_decode_full_bit_exact(dev):
    """Decode shape: 64 rows of one query, ring 128, ratio 4, 32768 compressed rows."""
    rng = np.random.default_rng(7)
    start_pos = rng.integers(0, 131072, size=64).tolist()
    start_pos[0], start_pos[1] = 131071, 0
    got = _build(dev, start_pos, 1, 128, 4, 32768)
    want = IL.topk_lists(start_pos, 1, 128, 4, 32768)
    assert np.array_equal(got, want)


def test_build_prefill_full_sampled(dev):
    """Prefill shape: 8192 queries at positions 24576.., ring 128, ratio 4, 8192 compressed rows."""
    B, M, W, R, C = 1, 8192, 128, 4, 8192
    got = _build(dev, [24576], M, W, R, C).reshape(M, W + C)
    rows = np.random.default_rng(3).choice(M, size=96, replace=False)
    rows = np.concatenate([rows, [0, M - 1]])
    assert np.array_equal(got[rows], IL.topk_lists([24576], M, W, R, C, rows=rows))
    # every row: valid counts, ranges and distinctness
    p = 24576 + np.arange(M)
    nw = (got[:, :W] >= 0).sum(1)
    nc = (got[:, W:] >= 0).sum(1)
    assert (nw == np.minimum(p + 1, W)).all() and (nc == np.minimum(C, (p + 1) // R)).all()
    assert ((got[:, :W] >= -1) & (got[:, :W] < W)).all()
    srt = np.sort(got[:, :W], axis=1)
    assert (np.diff(srt, axis=1)[srt[:, 1:] >= 0] > 0).all()


def test_built_lists_drive_indexed_attention(dev):
    """Decode over a ring cache with device-built lists == causal window attention (oracle)."""
    L, W, D, H = 300, 64, 64, 32
    g = torch.Generator().manual_seed(11)
    kv_seq = torch.randn(L, D, generator=g).to(torch.bfloat16)
    q_seq = torch.randn(L, H, D, generator=g).to(torch.bfloat16)
    p = L - 1
    ring = torch.zeros(W, D, dtype=torch.bfloat16)
    for pos in range(p - W + 1, p + 1):
        ring[pos % W] = kv_seq[pos]           # the ring holds the last W positions
    idx = sattn.build_topk_idxs(torch.tensor([p], dtype=torch.int32, device=dev), 1, window=W, ratio=0, n_comp=0)
    o = sattn.indexed_fwd(q_seq[p].reshape(1, 1, H, D).to(dev), ring.reshape(1, W, D).to(dev), idx,
                          softmax_scale=D ** -0.5)
    torch.cuda.synchronize(dev)
    cu = np.array([0, L], np.int32)
    ro, _ = oracle.window(q_seq, kv_seq.reshape(L, 1, D), kv_seq.reshape(L, 1, D), cu, window_left=W - 1,
                          window_right=0, scale=D ** -0.5, rows=[p])
    err = np.abs(o.float().cpu().numpy().reshape(H, D) - ro.reshape(H, D)).max()
    assert err < 1e-2, err

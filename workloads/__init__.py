"""Seeded synthetic inputs shaped like the workloads the pages describe.

This module holds no attention arithmetic.  It only draws random tensors and
builds integer index lists, so that the CPU oracle and the HIP library can be
fed identical inputs.  Everything is generated on the CPU with torch's and
numpy's seeded generators; callers move tensors to the GPU themselves.

Workloads (sizes follow the two pages that define the problem):

* window attention over a varlen batch described by ``cu_seqlens`` (vLLM PR
  #49815 report, "关键源码片段": ``context_attention_fwd`` and the dense test
  reference ``_reference``), with per-head ``sinks``;
* top-k index-gathered attention over a single shared K=V cache row per token
  (DeepSeek-V4 CSA/HCA article, §3.3 cache layout and §4.2 gather): the index
  list of a query is its sliding-window ring slots followed by compressed-region
  rows, padded with -1.

Draw order per case is fixed: lengths -> q -> k -> v (or kv) -> sinks, then the
index lists from a numpy Generator seeded with the same seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

SINK_NONE, SINK_KEY0, SINK_NULL = 0, 1, 2
SINK_MODES = {"none": SINK_NONE, "key0": SINK_KEY0, "null": SINK_NULL}


@dataclass
class WindowCase:
    name: str
    q: torch.Tensor            # [T, H, D]
    k: torch.Tensor            # [T, H_kv, D]
    v: torch.Tensor            # [T, H_kv, D]
    cu_seqlens: torch.Tensor   # int32 [S+1]
    sinks: torch.Tensor | None  # fp32 [H]
    sink_mode: int
    window_left: int
    window_right: int
    scale: float
    max_seqlen: int = 0

    @property
    def dims(self):
        t, h, d = self.q.shape
        return t, h, self.k.shape[1], d

    def pairs(self) -> int:
        """Attended (query token, query head, key) triples: keys that enter the numerator."""
        lens = (self.cu_seqlens[1:] - self.cu_seqlens[:-1]).tolist()
        h = self.q.shape[1]
        return h * sum(window_pairs(L, self.window_left, self.window_right) for L in lens)


@dataclass
class IndexedCase:
    name: str
    q: torch.Tensor            # [B, M, H, D]
    kv: torch.Tensor           # [B, N, D]
    topk_idxs: torch.Tensor    # int32 [B, M, K]; -1 = pad
    sinks: torch.Tensor | None
    sink_mode: int
    scale: float
    num_splits: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def dims(self):
        b, m, h, d = self.q.shape
        return b, m, h, d, self.kv.shape[1], self.topk_idxs.shape[2]

    def pairs(self) -> int:
        n = self.kv.shape[1]
        valid = ((self.topk_idxs >= 0) & (self.topk_idxs < n)).sum().item()
        return int(valid) * self.q.shape[2]


def window_pairs(L: int, wl: int, wr: int) -> int:
    """Number of (query, key) pairs of one sequence of length L under window (wl, wr).

    Key j is attended by query i iff j >= i - wl (wl < 0: unbounded) and
    j <= i + wr (wr < 0: unbounded), with 0 <= j < L.  Pure integer counting.
    """
    total = 0
    for i in range(L):
        lo = 0 if wl < 0 else max(0, i - wl)
        hi = L - 1 if wr < 0 else min(L - 1, i + wr)
        total += max(0, hi - lo + 1)
    return total


def _randn(g: torch.Generator, shape, dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(dtype) if dtype != torch.float32 else x


def make_window_case(name: str, lens, num_heads: int, num_kv_heads: int, head_dim: int,
                     window_left: int, window_right: int, sink_mode: int,
                     dtype=torch.bfloat16, seed: int = 0, scale: float | None = None,
                     sinks_value: float | None = None, generator: torch.Generator | None = None) -> WindowCase:
    g = generator if generator is not None else torch.Generator().manual_seed(seed)
    lens = [int(x) for x in lens]
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    if lens:
        cu[1:] = torch.tensor(np.cumsum(lens), dtype=torch.int32)
    T = int(cu[-1])
    q = _randn(g, (T, num_heads, head_dim), dtype)
    k = _randn(g, (T, num_kv_heads, head_dim), dtype)
    v = _randn(g, (T, num_kv_heads, head_dim), dtype)
    sinks = None
    if sink_mode != SINK_NONE:
        sinks = torch.randn(num_heads, generator=g, dtype=torch.float32)
        if sinks_value is not None:
            sinks.fill_(sinks_value)
    sc = 1.0 / math.sqrt(head_dim) if scale is None else scale
    return WindowCase(name, q, k, v, cu, sinks, sink_mode, window_left, window_right, sc,
                      max(lens) if lens else 0)


def make_window_case_random_lens(name, num_seqs, lo, hi, *args, seed=0, **kw) -> WindowCase:
    """Lengths uniform in [lo, hi] (inclusive), drawn first from the same generator as the tensors."""
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()
    return make_window_case(name, lens, *args, seed=seed, generator=g, **kw)


# ---------------------------------------------------------------------------
# index lists for the shared-KV cache (window ring + compressed region)
# ---------------------------------------------------------------------------

def ring_window_rows(pos: int, win: int) -> np.ndarray:
    """Ring slots holding positions max(0, pos-win+1) .. pos in position order.

    The window region keeps token p in slot p % win (DeepSeek-V4 article §3.3,
    ring write with cutoff = start_pos % win).
    """
    lo = max(0, pos - win + 1)
    return (np.arange(lo, pos + 1, dtype=np.int64) % win).astype(np.int32)


def compressed_candidates(pos: int, ratio: int) -> int:
    """Number of complete compressed rows visible at position pos: rows c with ratio*c + ratio-1 <= pos."""
    return max(0, (pos + 1) // ratio)


def build_topk_lists(rng: np.random.Generator, positions, win: int, ratio: int, n_compressed_rows: int,
                     n_pick: int, topk: int, comp_offset: int) -> np.ndarray:
    """Index lists [len(positions), topk]: window ring rows then n_pick distinct compressed rows.

    Compressed row c lives at cache row comp_offset + c; only rows fully
    below the query's position are candidates.  Lists are padded with -1.
    """
    out = np.full((len(positions), topk), -1, dtype=np.int32)
    for t, p in enumerate(positions):
        w = ring_window_rows(int(p), win)
        ncand = min(compressed_candidates(int(p), ratio), n_compressed_rows)
        take = min(n_pick, ncand)
        c = rng.choice(ncand, size=take, replace=False).astype(np.int64) if take > 0 else np.zeros(0, np.int64)
        row = np.concatenate([w.astype(np.int64), comp_offset + c])
        assert row.size <= topk
        out[t, :row.size] = row
    return out


def make_indexed_case(name: str, batch: int, q_len: int, num_heads: int, head_dim: int,
                      kv_len: int, topk_idxs: np.ndarray, sink_mode: int = SINK_NONE,
                      dtype=torch.bfloat16, seed: int = 0, num_splits: int = 1,
                      scale: float | None = None) -> IndexedCase:
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, (batch, q_len, num_heads, head_dim), dtype)
    kv = _randn(g, (batch, kv_len, head_dim), dtype)
    sinks = torch.randn(num_heads, generator=g, dtype=torch.float32) if sink_mode != SINK_NONE else None
    sc = 1.0 / math.sqrt(head_dim) if scale is None else scale
    idx = torch.from_numpy(np.ascontiguousarray(topk_idxs, dtype=np.int32))
    assert idx.shape[:2] == (batch, q_len)
    return IndexedCase(name, q, kv, idx, sinks, sink_mode, sc, num_splits)


def sparse_prefill_case(seed: int = 0, q_len: int = 8192, num_heads: int = 32, head_dim: int = 128,
                        win: int = 128, ratio: int = 4, total_tokens: int = 32768, n_pick: int = 512,
                        first_pos: int | None = None, sink_mode: int = SINK_NONE,
                        dtype=torch.bfloat16, name: str = "sparse_prefill") -> IndexedCase:
    """Top-k prefill over one shared K=V cache: win ring rows + total_tokens/ratio compressed rows.

    Queries sit at positions first_pos .. first_pos+q_len-1 (default: the last
    q_len tokens).  Each list holds the query's ring rows (<= win) then n_pick
    distinct compressed rows below its position, padded with -1.
    """
    n_comp = -(-total_tokens // ratio)
    kv_len = win + n_comp
    if first_pos is None:
        first_pos = total_tokens - q_len
    positions = np.arange(first_pos, first_pos + q_len)
    rng = np.random.default_rng(seed)
    idx = build_topk_lists(rng, positions, win, ratio, n_comp, n_pick, win + n_pick, comp_offset=win)
    case = make_indexed_case(name, 1, q_len, num_heads, head_dim, kv_len, idx[None], sink_mode,
                             dtype, seed)
    case.extra.update(positions=positions, win=win, ratio=ratio)
    return case


def sparse_decode_case(seed: int = 0, batch: int = 64, num_heads: int = 64, head_dim: int = 128,
                       win: int = 128, ratio: int = 4, total_tokens: int = 131072, n_pick: int = 1920,
                       num_splits: int = 8, sink_mode: int = SINK_NONE, dtype=torch.bfloat16,
                       name: str = "sparse_decode", index_sets: int = 1) -> IndexedCase:
    """Top-k decode: batch sequences with one query each and their own cache [win + total/ratio, D].

    The list is the win ring rows then n_pick distinct compressed rows drawn
    uniformly from every complete compressed row.  With index_sets > 1, extra
    independent list sets are drawn (stored in extra['idx_sets']).
    """
    n_comp = -(-total_tokens // ratio)
    kv_len = win + n_comp
    pos = total_tokens  # the token being decoded; all compressed rows are complete
    rng = np.random.default_rng(seed)
    sets = []
    for _ in range(max(1, index_sets)):
        idx = build_topk_lists(rng, [pos] * batch, win, ratio, n_comp, n_pick, win + n_pick, comp_offset=win)
        sets.append(idx[:, None, :])
    case = make_indexed_case(name, batch, 1, num_heads, head_dim, kv_len, sets[0], sink_mode, dtype, seed,
                             num_splits)
    case.extra["idx_sets"] = [torch.from_numpy(np.ascontiguousarray(s)) for s in sets]
    return case


# ---------------------------------------------------------------------------
# the five workloads (full size) and their reduced parity versions
# ---------------------------------------------------------------------------

def tiny_window_fp32(num_kv_heads: int = 4, seed: int = 0) -> WindowCase:
    """2 sequences of length 5 and 37, 4 query heads, head_dim 64, window |i-j| <= 8, key-0 sinks, fp32."""
    return make_window_case(f"tiny_window_fp32_kv{num_kv_heads}", [5, 37], 4, num_kv_heads, 64, 8, 8,
                            SINK_KEY0, dtype=torch.float32, seed=seed, scale=1.0 / 8.0)


def vision_window(seed: int = 0, num_seqs: int = 16, lo: int = 1024, hi: int = 4096) -> WindowCase:
    """Vision-encoder window attention: 16 seqs, lengths U[1024,4096], 16/8 heads, D=128, window +-128, key-0 sinks."""
    return make_window_case_random_lens("vision_window", num_seqs, lo, hi, 16, 8, 128, 128, 128, SINK_KEY0,
                                        dtype=torch.bfloat16, seed=seed)


def causal_window_null(seed: int = 0, num_seqs: int = 4, seqlen: int = 8192) -> WindowCase:
    """Causal sliding window of 128 keys (self included), 64/8 heads, D=64, null-logit sinks."""
    return make_window_case("causal_window_null", [seqlen] * num_seqs, 64, 8, 64, 127, 0, SINK_NULL,
                            dtype=torch.bfloat16, seed=seed)


def indexer_inputs(seed: int, batch: int, q_len: int, n_comp: int, rank: int, integer: bool = False):
    """Low-rank queries qr [batch, q_len, rank] and index keys kidx [batch, n_comp, rank], bf16.

    N(0, 1) entries, or with integer=True small integers in [-3, 3] (every score is then an
    integer, exact in fp32, and equal scores are common).
    """
    g = torch.Generator().manual_seed(seed)
    if integer:
        qr = torch.randint(-3, 4, (batch, q_len, rank), generator=g).to(torch.bfloat16)
        kidx = torch.randint(-3, 4, (batch, n_comp, rank), generator=g).to(torch.bfloat16)
    else:
        qr = _randn(g, (batch, q_len, rank), torch.bfloat16)
        kidx = _randn(g, (batch, n_comp, rank), torch.bfloat16)
    return qr, kidx


def fp8_cache(seed: int, batch: int, n_rows: int, head_dim: int, rope_dims: int, scale_spread: int = 4):
    """An fp8 KV cache: rows ~ N(0, 1) times a per-row power of two in [2^-spread, 2^spread]; the first
    head_dim - rope_dims dims become e4m3 codes (torch's round-to-nearest float8_e4m3fn conversion)
    against one power-of-two scale per row chosen so that the row's largest magnitude fits 448; the
    last rope_dims dims stay bf16.  Returns (kv8 uint8 [B, N, D - rd], scale fp32 [B, N],
    kv_rope bf16 [B, N, rd])."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(batch, n_rows, head_dim, generator=g)
    x = x * torch.exp2(torch.randint(-scale_spread, scale_spread + 1, (batch, n_rows, 1), generator=g).float())
    d8 = head_dim - rope_dims
    nope = x[..., :d8]
    amax = nope.abs().amax(-1).clamp_min(1e-30)
    scale = torch.exp2(torch.ceil(torch.log2(amax / 448.0)))
    kv8 = (nope / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
    kv_rope = x[..., d8:].to(torch.bfloat16)
    return kv8.contiguous(), scale.float().contiguous(), kv_rope.contiguous()

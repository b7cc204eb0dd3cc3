"""CPU oracle for top-k list construction (window rows, synthetic indexer), per-block attention
mass and the compressor's gated pooling (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module; the product path never does.
Plain Python on purpose: one query at a time, straight from the definitions.

Source: DeepSeek-V4 CSA/HCA article, §2.3 (the list of a query is the
concatenation of its sliding-window indices and its compressed-region
indices) and §3.3 (cache layout ``[b, window + max_len / ratio, d]``: the
window region is a ring in which position ``p`` is written to slot
``p % window``; the compressor emits compressed token ``c`` once position
``(c + 1) * ratio - 1`` has been seen, i.e. when ``(pos + 1) % ratio == 0``,
and its row follows the window region).

Readings (the article shows the pieces, not the builder):
  * query position ``p`` sees the window positions ``max(0, p - window + 1)
    .. p`` (the ring holds the last ``window`` positions, itself included),
    listed by ring slot in increasing position order, then ``-1`` up to
    ``window`` entries;
  * it sees compressed token ``c`` iff ``(c + 1) * ratio - 1 <= p`` and
    ``c < n_comp`` (the cache holds ``n_comp`` compressed rows), listed as row
    ``window + c`` in increasing ``c``, then ``-1`` up to ``n_comp`` entries;
  * ``ratio == 0`` means no compressed region (``n_comp`` must be 0);
  * a negative position sees nothing.
"""
from __future__ import annotations

import numpy as np


def query_list(p: int, window: int, ratio: int, n_comp: int) -> list[int]:
    """The ``window + n_comp`` list entries of one query at absolute position p."""
    win = []
    if p >= 0:
        for q in range(max(0, p - window + 1), p + 1):
            win.append(q % window)
    win += [-1] * (window - len(win))
    comp = []
    if ratio > 0:
        for c in range(n_comp):
            if (c + 1) * ratio - 1 <= p:
                comp.append(window + c)
    comp += [-1] * (n_comp - len(comp))
    return win + comp


def topk_lists(start_pos, q_len: int, window: int, ratio: int, n_comp: int, rows=None) -> np.ndarray:
    """Lists of queries (b, t) at positions start_pos[b] + t.

    Returns int32 [B, q_len, window + n_comp], or [len(rows), window + n_comp] for the flat
    query rows ``b * q_len + t`` named in ``rows``.
    """
    sp = np.asarray(start_pos, dtype=np.int64).reshape(-1)
    B = sp.shape[0]
    K = window + n_comp
    flat = range(B * q_len) if rows is None else [int(r) for r in rows]
    out = np.empty((len(flat), K), dtype=np.int32)
    for i, r in enumerate(flat):
        b, t = divmod(r, q_len)
        out[i] = query_list(int(sp[b]) + t, window, ratio, n_comp)
    return out.reshape(B, q_len, K) if rows is None else out


def block_mass(q, kv, topk_idxs, lse, *, scale: float, block_keys: int, sinks=None, sink_mode: int = 0,
               rows=None) -> np.ndarray:
    """Attention mass per block of list entries, normalised by a given log-sum-exp.

    Source: nano-vllm "XAttention Offload Stream Synchronization Fix", technical details: the
    third stage of the chunked estimate normalises with the global softmax statistics and sums
    per block.  Reading: block c of a query's list is entries [c * block_keys, (c + 1) *
    block_keys); its mass for head h is sum over its valid entries (0 <= idx < N) of
    exp(scale * q[h] . kv[idx] + key-0 bias - lse[h]) with the key-0 sink bias of the
    DeepSeek-V4 article's list convention (cache row 0).  With the lse of the same key set
    (null sink included) the masses plus exp(sink - lse) sum to 1.

    q [B, M, H, D], kv [B, N, D], topk_idxs [B, M, K], lse [B, M, H] (natural log).
    Returns float64 [B*M or len(rows), H, ceil(K / block_keys)].
    """
    # bf16 / fp32 values are exact in fp32; rows are widened to fp64 when used
    qf = np.asarray(q, dtype=np.float32) if not hasattr(q, "float") else q.float().numpy()
    kvf = np.asarray(kv, dtype=np.float32) if not hasattr(kv, "float") else kv.float().numpy()
    idx = np.asarray(topk_idxs)
    ls = np.asarray(lse, dtype=np.float64)
    B, M, H, D = qf.shape
    N, K = kvf.shape[1], idx.shape[2]
    nb = (K + block_keys - 1) // block_keys
    snk = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    flat = range(B * M) if rows is None else [int(r) for r in rows]
    out = np.zeros((len(flat), H, nb), dtype=np.float64)
    for i, r in enumerate(flat):
        b, t = divmod(r, M)
        ks = idx[b, t].astype(np.int64)
        pos = np.nonzero((ks >= 0) & (ks < N))[0]  # list positions of the valid entries
        x = ks[pos]                                # their cache rows
        logit = scale * (qf[b, t].astype(np.float64) @ kvf[b, x].astype(np.float64).T)  # [H, n_valid]
        if sink_mode == 1:
            logit[:, x == 0] += snk[:, None]
        e = np.exp(logit - ls[b, t][:, None])
        np.add.at(out[i], (slice(None), pos // block_keys), e)  # entry k goes to block k // block_keys
    return out


def compress_pool(kv, score, ape, *, ratio: int, overlap: bool) -> np.ndarray:
    """Gated pooling of the compressor: one compressed row per complete window of `ratio` tokens.

    Source: DeepSeek-V4 CSA/HCA article, §5.1 (compressed kv = sum over the window of kv_i times
    softmax(score_i), the softmax taken over the window's tokens; the learned absolute position
    term ape [ratio, coff * d] is added to the scores first; coff = 2 with overlap) and its
    overlap-transform description (window i takes the previous window's tokens with the first d
    features and its own tokens with the last d features).  Readings: the softmax is per feature;
    window w holds tokens [w * ratio, (w + 1) * ratio); a trailing partial window is not
    compressed; with overlap, window 0 has no previous window and its first half contributes
    nothing (weight 0).

    kv, score: [B, S, coff * d]; ape: [ratio, coff * d].  Returns float64 [B, S // ratio, d].
    """
    kvf = np.asarray(kv.float().numpy() if hasattr(kv, "float") else kv, dtype=np.float64)
    scf = np.asarray(score.float().numpy() if hasattr(score, "float") else score, dtype=np.float64)
    apf = np.asarray(ape.float().numpy() if hasattr(ape, "float") else ape, dtype=np.float64)
    B, S, F = kvf.shape
    coff = 2 if overlap else 1
    d = F // coff
    n_out = S // ratio
    out = np.zeros((B, n_out, d), dtype=np.float64)
    for b in range(B):
        for w in range(n_out):
            rows_kv, rows_sc = [], []  # one entry per (token, its feature half) in the window
            if overlap and w > 0:
                for i in range(ratio):
                    t = (w - 1) * ratio + i
                    rows_kv.append(kvf[b, t, :d])
                    rows_sc.append(scf[b, t, :d] + apf[i, :d])
            for i in range(ratio):
                t = w * ratio + i
                lo = d if overlap else 0
                rows_kv.append(kvf[b, t, lo:lo + d])
                rows_sc.append(scf[b, t, lo:lo + d] + apf[i, lo:lo + d])
            sc = np.stack(rows_sc)                # [tokens, d]
            e = np.exp(sc - sc.max(axis=0))
            out[b, w] = (e * np.stack(rows_kv)).sum(axis=0) / e.sum(axis=0)
    return out


def indexer_lists(qr, kidx, start_pos, q_len: int, window: int, ratio: int, n_comp: int, topk: int,
                  rows=None) -> np.ndarray:
    """Top-k lists chosen by a synthetic indexer.

    Source: DeepSeek-V4 CSA/HCA article, §2.3 (the indexer, fed the low-rank query qr, chooses
    the compressed-region indices; window indices come first and the two parts are
    concatenated).  Readings (the article gives neither the scoring nor the weights): compressed
    row c is scored qr[b, t] . kidx[b, c] with a per-row index key kidx; only the rows visible
    at the query's position (those query_list lists) are candidates; the `topk` highest scores
    are kept, ties going to the lower row; the chosen rows are listed as window + c in
    increasing c, then -1 up to `topk` entries.  Scores are taken in fp64.

    qr [B, q_len, r], kidx [B, n_comp, r].  Returns int32 [B, q_len, window + topk], or
    [len(rows), window + topk] for the flat query rows b * q_len + t named in `rows`.
    """
    qf = np.asarray(qr.float().numpy() if hasattr(qr, "float") else qr, dtype=np.float64)
    kf = np.asarray(kidx.float().numpy() if hasattr(kidx, "float") else kidx, dtype=np.float64)
    sp = np.asarray(start_pos, dtype=np.int64).reshape(-1)
    B = sp.shape[0]
    flat = range(B * q_len) if rows is None else [int(r) for r in rows]
    out = np.full((len(flat), window + topk), -1, dtype=np.int32)
    for i, r in enumerate(flat):
        b, t = divmod(r, q_len)
        full = query_list(int(sp[b]) + t, window, ratio, n_comp)
        out[i, :window] = full[:window]
        visible = [x - window for x in full[window:] if x >= 0]  # compressed indices c
        if not visible:
            continue
        scores = kf[b, visible] @ qf[b, t]
        order = sorted(range(len(visible)), key=lambda j: (-scores[j], visible[j]))
        chosen = sorted(visible[j] for j in order[:topk])
        out[i, window:window + len(chosen)] = [window + c for c in chosen]
    return out if rows is not None else out.reshape(B, q_len, window + topk)

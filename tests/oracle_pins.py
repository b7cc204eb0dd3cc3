"""Pins for the CPU oracle: checks against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes an oracle library handle (so the same checks can
run against deliberately broken builds of the oracle) and raises
AssertionError on a mismatch.  None of them re-types the oracle's formula:
they compare it with torch's scaled_dot_product_attention / logsumexp on
special cases, with closed forms, with invariants, and with the example values
the pages print (tests/golden/).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from oracle import SINK_KEY0, SINK_NONE, SINK_NULL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


def _rand(g, *shape):
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(a - b))
    m = float(np.nanmax(err)) if err.size else 0.0
    assert np.isfinite(err).all() and m <= tol, f"{what}: max |diff| {m:.3e} > {tol:.1e}"


def _window_mask(L, wl, wr):
    i = torch.arange(L).view(-1, 1)
    j = torch.arange(L).view(1, -1)
    ok = torch.ones(L, L, dtype=torch.bool)
    if wl >= 0:
        ok &= j >= i - wl
    if wr >= 0:
        ok &= j <= i + wr
    return ok


def _sdpa_window(q, k, v, lens, wl, wr, scale, sinks, mode):
    """Library reference: per sequence, SDPA with an additive float mask.

    Out-of-window keys get -inf; KEY0 adds sinks[h] at column 0; NULL appends
    a zero key/value whose mask entry is sinks[h] (logit = sink, no value).
    Returns (o, lse) with lse from torch.logsumexp of the masked logits.
    """
    H = q.shape[1]
    outs, lses = [], []
    a = 0
    for L in lens:
        qs = q[a:a + L].to(F64).transpose(0, 1)[None]   # [1,H,L,D]
        ks = k[a:a + L].to(F64).transpose(0, 1)[None]
        vs = v[a:a + L].to(F64).transpose(0, 1)[None]
        mask = torch.zeros(H, L, L, dtype=F64)
        mask.masked_fill_(~_window_mask(L, wl, wr), -math.inf)
        if mode == SINK_KEY0:
            mask[:, :, 0] += sinks.to(F64).view(-1, 1)
        if mode == SINK_NULL:
            z = torch.zeros(1, ks.shape[1], 1, ks.shape[3], dtype=F64)
            ks = torch.cat([ks, z], 2)
            vs = torch.cat([vs, z], 2)
            mask = torch.cat([mask, sinks.to(F64).view(-1, 1, 1).expand(H, L, 1)], 2)
        o = F.scaled_dot_product_attention(qs, ks, vs, attn_mask=mask[None], scale=scale, enable_gqa=True)
        G = H // ks.shape[1]
        logits = torch.matmul(qs, ks.repeat_interleave(G, 1).transpose(-1, -2)) * scale + mask[None]
        outs.append(o[0].transpose(0, 1))
        lses.append(torch.logsumexp(logits[0], -1).transpose(0, 1))
        a += L
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def _sdpa_indexed(q, kv, idx, scale, sinks, mode):
    """Library reference for the top-k path: SDPA of each query over its gathered rows."""
    B, M, H, D = q.shape
    N = kv.shape[1]
    o = np.zeros((B * M, H, D))
    lse = np.zeros((B * M, H))
    for b in range(B):
        for t in range(M):
            rows = [int(x) for x in idx[b, t] if 0 <= int(x) < N]
            K = kv[b, rows].to(F64)                     # [n,D]
            qq = q[b, t].to(F64)[:, None, :]            # [H,1,D]
            mask = torch.zeros(H, 1, len(rows), dtype=F64)
            if mode == SINK_KEY0 and 0 in rows:
                mask[:, 0, rows.index(0)] += sinks.to(F64)
            kk, vv = K[None].expand(H, -1, -1), K[None].expand(H, -1, -1)
            if mode == SINK_NULL:
                z = torch.zeros(H, 1, D, dtype=F64)
                kk, vv = torch.cat([kk, z], 1), torch.cat([vv, z], 1)
                mask = torch.cat([mask, sinks.to(F64).view(H, 1, 1)], 2)
            if kk.shape[1] == 0:
                o[b * M + t] = 0.0
                lse[b * M + t] = -math.inf
                continue
            oo = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask, scale=scale)
            logits = torch.matmul(qq, kk.transpose(-1, -2)) * scale + mask
            o[b * M + t] = oo[:, 0].numpy()
            lse[b * M + t] = torch.logsumexp(logits[:, 0], -1).numpy()
    return o, lse


# ---------------------------------------------------------------------------
# window path
# ---------------------------------------------------------------------------

def pin_window_full_matches_sdpa(lib):
    """Window >= L-1 on both sides, no sink: plain non-causal attention (library routine), GQA via enable_gqa."""
    g = torch.Generator().manual_seed(11)
    lens = [3, 9, 1, 14]
    T, H, Hkv, D = sum(lens), 4, 2, 16
    q, k, v = _rand(g, T, H, D), _rand(g, T, Hkv, D), _rand(g, T, Hkv, D)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, lse = oracle.window(q, k, v, cu, window_left=-1, window_right=20, scale=0.37, lib=lib)
    ro, rl = _sdpa_window(q, k, v, lens, -1, -1, 0.37, None, SINK_NONE)
    _close(o, ro, 1e-12, "full-window o")
    _close(lse, rl, 1e-12, "full-window lse")


def pin_window_causal_matches_sdpa(lib):
    """(wl, wr) = (unbounded, 0): causal attention, checked against SDPA(is_causal=True)."""
    g = torch.Generator().manual_seed(12)
    L, H, D = 11, 2, 8
    q, k, v = _rand(g, L, H, D), _rand(g, L, H, D), _rand(g, L, H, D)
    o, _ = oracle.window(q, k, v, np.array([0, L], np.int32), window_left=-1, window_right=0, scale=0.5, lib=lib)
    ref = F.scaled_dot_product_attention(q.to(F64).transpose(0, 1)[None], k.to(F64).transpose(0, 1)[None],
                                         v.to(F64).transpose(0, 1)[None], is_causal=True, scale=0.5)
    _close(o, ref[0].transpose(0, 1).numpy(), 1e-12, "causal o")


def pin_window_key0_matches_masked_sdpa(lib):
    """Window + key-0 sink == SDPA with an additive mask (-inf outside window, +sink at column 0)."""
    g = torch.Generator().manual_seed(13)
    lens = [5, 37]
    T, H, D = sum(lens), 4, 64
    for Hkv in (4, 2):
        q, k, v = _rand(g, T, H, D), _rand(g, T, Hkv, D), _rand(g, T, Hkv, D)
        sinks = _rand(g, H) * 2.0
        cu = np.array([0, 5, 42], np.int32)
        for wl, wr in ((8, 8), (3, 0), (0, 5), (127, 0)):
            o, lse = oracle.window(q, k, v, cu, window_left=wl, window_right=wr, scale=0.125, sinks=sinks,
                                   sink_mode=SINK_KEY0, lib=lib)
            ro, rl = _sdpa_window(q, k, v, lens, wl, wr, 0.125, sinks, SINK_KEY0)
            _close(o, ro, 1e-12, f"key0 o Hkv={Hkv} w=({wl},{wr})")
            _close(lse, rl, 1e-12, f"key0 lse Hkv={Hkv} w=({wl},{wr})")


def pin_window_null_matches_extra_key_sdpa(lib):
    """Null sink == an extra key whose logit is the sink and whose value is zero (denominator only)."""
    g = torch.Generator().manual_seed(14)
    lens = [6, 19, 2]
    T, H, Hkv, D = sum(lens), 8, 2, 16
    q, k, v = _rand(g, T, H, D), _rand(g, T, Hkv, D), _rand(g, T, Hkv, D)
    sinks = _rand(g, H) * 2.0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, lse = oracle.window(q, k, v, cu, window_left=4, window_right=0, scale=0.25, sinks=sinks,
                           sink_mode=SINK_NULL, lib=lib)
    ro, rl = _sdpa_window(q, k, v, lens, 4, 0, 0.25, sinks, SINK_NULL)
    _close(o, ro, 1e-12, "null o")
    _close(lse, rl, 1e-12, "null lse")


def pin_window_null_closed_form(lib):
    """Null sink closed form: o_null = o_none * sigmoid(lse_none - sink), lse_null = logaddexp(lse_none, sink)."""
    g = torch.Generator().manual_seed(15)
    T, H, D = 23, 4, 8
    q, k, v = _rand(g, T, H, D), _rand(g, T, H, D), _rand(g, T, H, D)
    sinks = _rand(g, H) * 3.0
    cu = np.array([0, 10, 23], np.int32)
    kw = dict(window_left=5, window_right=2, scale=0.3, lib=lib)
    o0, l0 = oracle.window(q, k, v, cu, **kw)
    o1, l1 = oracle.window(q, k, v, cu, sinks=sinks, sink_mode=SINK_NULL, **kw)
    s = sinks.numpy().astype(np.float64)[None, :]
    sig = 1.0 / (1.0 + np.exp(-(l0 - s)))
    _close(o1, o0 * sig[..., None], 1e-12, "null closed-form o")
    _close(l1, np.logaddexp(l0, s), 1e-12, "null closed-form lse")


def pin_single_key_closed_forms(lib):
    """L = 1: key-0 mode gives o = v_0 for any sink; null mode gives o = v_0 * sigmoid(s_0 - sink)."""
    g = torch.Generator().manual_seed(16)
    H, D = 3, 8
    q, k, v = _rand(g, 1, H, D), _rand(g, 1, H, D), _rand(g, 1, H, D)
    sinks = _rand(g, H) * 2.0
    cu = np.array([0, 1], np.int32)
    o, lse = oracle.window(q, k, v, cu, window_left=8, window_right=8, scale=0.5, sinks=sinks,
                           sink_mode=SINK_KEY0, lib=lib)
    _close(o[0], v[0].numpy(), 1e-12, "L=1 key0 o")
    s0 = 0.5 * np.einsum("hd,hd->h", q[0].numpy().astype(np.float64), k[0].numpy().astype(np.float64))
    _close(lse[0], s0 + sinks.numpy(), 1e-12, "L=1 key0 lse")
    o, lse = oracle.window(q, k, v, cu, window_left=8, window_right=8, scale=0.5, sinks=sinks,
                           sink_mode=SINK_NULL, lib=lib)
    sig = 1.0 / (1.0 + np.exp(-(s0 - sinks.numpy())))
    _close(o[0], v[0].numpy() * sig[:, None], 1e-12, "L=1 null o")
    _close(lse[0], np.logaddexp(s0, sinks.numpy()), 1e-12, "L=1 null lse")


def pin_window_bit_exact_invariants(lib):
    """Key-0 sink of 0 == no sink; null sink of -inf == no sink (both bit-exact)."""
    g = torch.Generator().manual_seed(17)
    T, H, Hkv, D = 30, 4, 2, 16
    q, k, v = _rand(g, T, H, D), _rand(g, T, Hkv, D), _rand(g, T, Hkv, D)
    cu = np.array([0, 4, 30], np.int32)
    kw = dict(window_left=6, window_right=6, scale=0.25, lib=lib)
    o0, l0 = oracle.window(q, k, v, cu, **kw)
    o1, l1 = oracle.window(q, k, v, cu, sinks=torch.zeros(H), sink_mode=SINK_KEY0, **kw)
    o2, l2 = oracle.window(q, k, v, cu, sinks=torch.full((H,), -math.inf), sink_mode=SINK_NULL, **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1), "key0 sink 0 != none"
    assert np.array_equal(o0, o2) and np.array_equal(l0, l2), "null sink -inf != none"


def pin_gqa_equals_mha_repeat(lib):
    """GQA (head h reads KV head h // (H/Hkv)) == MHA on repeat_interleave'd K/V."""
    g = torch.Generator().manual_seed(18)
    T, H, Hkv, D = 17, 8, 2, 8
    q, k, v = _rand(g, T, H, D), _rand(g, T, Hkv, D), _rand(g, T, Hkv, D)
    sinks = _rand(g, H)
    cu = np.array([0, 17], np.int32)
    kw = dict(window_left=3, window_right=3, scale=0.4, sinks=sinks, sink_mode=SINK_KEY0, lib=lib)
    o0, l0 = oracle.window(q, k, v, cu, **kw)
    o1, l1 = oracle.window(q, k.repeat_interleave(4, 1), v.repeat_interleave(4, 1), cu, **kw)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def pin_page1_sink_changes_output(lib):
    """The page's test setup (lens [5,37], window 8, 4 heads, kv heads 4/2): dropping the key-0 sink
    moves the output by well over the 1e-2 threshold the page's test uses (it measured 1.2e-1 / 2.1e-1)."""
    for Hkv in (4, 2):
        g = torch.Generator().manual_seed(0)
        T, H, D = 42, 4, 64
        q, k, v = _rand(g, T, H, D), _rand(g, T, Hkv, D), _rand(g, T, Hkv, D)
        sinks = _rand(g, H)
        cu = np.array([0, 5, 42], np.int32)
        kw = dict(window_left=8, window_right=8, scale=0.125, lib=lib)
        o1, _ = oracle.window(q, k, v, cu, sinks=sinks, sink_mode=SINK_KEY0, **kw)
        o0, _ = oracle.window(q, k, v, cu, **kw)
        assert np.abs(o1 - o0).max() > 1e-2


# ---------------------------------------------------------------------------
# indexed path
# ---------------------------------------------------------------------------

def _indexed_inputs(seed, B, M, H, D, N, K, pad_frac=0.25, with_row0=True):
    """Distinct random lists; every other query's list contains cache row 0 (the key-0 sink's key)."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    q, kv = _rand(g, B, M, H, D), _rand(g, B, N, D)
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            n = int(rng.integers(0, K + 1)) if rng.random() < pad_frac else K
            row = rng.choice(N, size=n, replace=False)
            if with_row0 and (b * M + t) % 2 == 0 and n > 0 and 0 not in row:
                row[int(rng.integers(0, n))] = 0
            idx[b, t, :n] = row
    return q, kv, idx, _rand(g, H) * 2.0


def pin_indexed_matches_sdpa(lib):
    """Each query == SDPA over its gathered rows (K = V = row), for all three sink modes."""
    B, M, H, D, N, K = 2, 5, 4, 16, 40, 12
    q, kv, idx, sinks = _indexed_inputs(21, B, M, H, D, N, K)
    idx[1, 2, :] = -1                      # one query with no key at all
    for mode in (SINK_NONE, SINK_KEY0, SINK_NULL):
        o, lse = oracle.indexed(q, kv, idx, scale=0.3, sinks=sinks, sink_mode=mode, lib=lib)
        ro, rl = _sdpa_indexed(q, kv, idx, 0.3, sinks, mode)
        _close(o.reshape(-1), ro.reshape(-1), 1e-12, f"indexed o mode={mode}")
        _close(lse, rl, 1e-12, f"indexed lse mode={mode}")


def pin_indexed_empty_set(lib):
    """No valid index: o = 0 and lse = -inf; with a null sink lse = sink."""
    H, D = 2, 8
    g = torch.Generator().manual_seed(22)
    q, kv = _rand(g, 1, 1, H, D), _rand(g, 1, 4, D)
    sinks = torch.tensor([0.5, -1.25])
    idx = np.full((1, 1, 3), -1, np.int32)
    o, lse = oracle.indexed(q, kv, idx, scale=1.0, lib=lib)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = oracle.indexed(q, kv, idx, scale=1.0, sinks=sinks, sink_mode=SINK_NULL, lib=lib)
    assert np.all(o == 0) and np.allclose(lse[0], sinks.numpy().astype(np.float64), rtol=0, atol=0)


def pin_indexed_padding_and_order(lib):
    """Appending -1 pads is bit-exact; permuting the list changes only the summation order."""
    B, M, H, D, N, K = 1, 6, 4, 16, 64, 10
    q, kv, idx, sinks = _indexed_inputs(23, B, M, H, D, N, K, pad_frac=0.0)
    for mode in (SINK_NONE, SINK_KEY0, SINK_NULL):
        idx0 = idx
        o0, l0 = oracle.indexed(q, kv, idx0, scale=0.2, sinks=sinks, sink_mode=mode, lib=lib)
        padded = np.concatenate([idx0, np.full((B, M, 5), -1, np.int32)], 2)
        o1, l1 = oracle.indexed(q, kv, padded, scale=0.2, sinks=sinks, sink_mode=mode, lib=lib)
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1), "padding changed the result"
        rng = np.random.default_rng(5)
        perm = padded[..., rng.permutation(padded.shape[-1])]
        o2, l2 = oracle.indexed(q, kv, perm, scale=0.2, sinks=sinks, sink_mode=mode, lib=lib)
        _close(o2, o0, 1e-13, "permuted o")
        _close(l2, l0, 1e-13, "permuted lse")


def pin_indexed_rejects_duplicates(lib):
    g = torch.Generator().manual_seed(24)
    q, kv = _rand(g, 1, 1, 2, 8), _rand(g, 1, 8, 8)
    try:
        oracle.indexed(q, kv, np.array([[[1, 2, 1]]], np.int32), scale=1.0, lib=lib)
    except ValueError:
        return
    raise AssertionError("duplicate indices were accepted")


def pin_window_equals_indexed_lists(lib):
    """The window path equals the indexed path run on the materialised window lists (Hkv = 1, k == v)."""
    g = torch.Generator().manual_seed(25)
    lens = [7, 13]
    T, H, D = sum(lens), 4, 16
    q, kv = _rand(g, T, H, D), _rand(g, T, 1, D)
    sinks = _rand(g, H)
    wl, wr = 3, 2
    cu = np.array([0, 7, 20], np.int32)
    K = wl + wr + 1
    for mode in (SINK_NONE, SINK_KEY0, SINK_NULL):
        ow, lw = oracle.window(q, kv, kv, cu, window_left=wl, window_right=wr, scale=0.3, sinks=sinks,
                               sink_mode=mode, lib=lib)
        oi_all, li_all = [], []
        a = 0
        for L in lens:
            idx = np.full((1, L, K), -1, np.int32)
            for i in range(L):
                js = [j for j in range(max(0, i - wl), min(L - 1, i + wr) + 1)]
                idx[0, i, :len(js)] = js
            oi, li = oracle.indexed(q[a:a + L][None], kv[a:a + L, 0][None], idx, scale=0.3, sinks=sinks,
                                    sink_mode=mode, lib=lib)
            oi_all.append(oi)
            li_all.append(li)
            a += L
        _close(ow, np.concatenate(oi_all), 1e-13, f"window vs indexed o mode={mode}")
        _close(lw, np.concatenate(li_all), 1e-13, f"window vs indexed lse mode={mode}")


def pin_page2_example_lists(lib):
    """The article's example lists (tests/golden/page2_index_examples.json) against SDPA on the gathered rows."""
    with open(os.path.join(GOLDEN, "page2_index_examples.json")) as f:
        ex = json.load(f)
    for name, lst in ex["lists"].items():
        lst = [int(x) for x in lst]
        N = max(lst) + 1
        g = torch.Generator().manual_seed(26)
        H, D = 4, 16
        q, kv = _rand(g, 1, 1, H, D), _rand(g, 1, N, D)
        sinks = _rand(g, H)
        idx = np.array([[lst + [-1, -1, -1]]], np.int32)
        for mode in (SINK_NONE, SINK_NULL):
            o, lse = oracle.indexed(q, kv, idx, scale=0.25, sinks=sinks, sink_mode=mode, lib=lib)
            ro, rl = _sdpa_indexed(q, kv, idx, 0.25, sinks, mode)
            _close(o.reshape(-1), ro.reshape(-1), 1e-12, f"{name} o")
            _close(lse, rl, 1e-12, f"{name} lse")


# ---------------------------------------------------------------------------
# split-K merge
# ---------------------------------------------------------------------------

def pin_split_merge_equals_single_pass(lib):
    """Chunk partials (no sink) merged, with the null sink added once == single pass over the whole list."""
    B, M, H, D, N, K = 2, 3, 4, 16, 80, 24
    q, kv, idx, sinks = _indexed_inputs(31, B, M, H, D, N, K, pad_frac=0.5)
    idx[0, 0, :] = -1
    idx[0, 0, 20] = 5                      # only the last chunk has a key
    for mode in (SINK_NONE, SINK_NULL):
        full_o, full_l = oracle.indexed(q, kv, idx, scale=0.3, sinks=sinks, sink_mode=mode, lib=lib)
        for S in (1, 2, 3, 5):
            step = -(-K // S)
            parts = [oracle.indexed(q, kv, np.ascontiguousarray(idx[..., c * step:(c + 1) * step]), scale=0.3,
                                    lib=lib) for c in range(S)]
            po = np.stack([p[0] for p in parts]).astype(np.float32)
            pl = np.stack([p[1] for p in parts]).astype(np.float32)
            mo, ml = oracle.merge(po, pl, sinks=sinks, sink_mode=mode, lib=lib)
            _close(mo, full_o, 1e-6, f"merge o S={S} mode={mode}")
            _close(ml, full_l, 1e-5, f"merge lse S={S} mode={mode}")


def pin_merge_matches_library(lib):
    """Merge == softmax over the partial lse's (torch.softmax / logsumexp) weighting the partial outputs."""
    g = torch.Generator().manual_seed(32)
    S, R, H, D = 4, 5, 3, 8
    po = _rand(g, S, R, H, D)
    pl = _rand(g, S, R, H) * 4.0
    pl[1, 2, 1] = -math.inf
    pl[:, 4, 0] = -math.inf               # an all-empty row
    sinks = _rand(g, H)
    for mode in (SINK_NONE, SINK_NULL):
        o, lse = oracle.merge(po, pl, sinks=sinks, sink_mode=mode, lib=lib)
        lse_st = pl.to(F64)
        po_st = po.to(F64)
        if mode == SINK_NULL:
            lse_st = torch.cat([lse_st, sinks.to(F64).view(1, 1, H).expand(1, R, H)], 0)
            po_st = torch.cat([po_st, torch.zeros(1, R, H, D, dtype=F64)], 0)
        ref_l = torch.logsumexp(lse_st, 0)
        w = torch.softmax(lse_st, 0).nan_to_num(0.0)
        ref_o = (w[..., None] * po_st).sum(0)
        _close(o, ref_o.numpy(), 1e-12, f"merge o mode={mode}")
        _close(lse, ref_l.numpy(), 1e-12, f"merge lse mode={mode}")


def pin_rescale_worked_example(lib):
    """The article's worked rescale step (tests/golden/rescale_example.json): a running max moving from
    10 to 12 scales the old sum by exp(-2) ~= 0.135, about 7.4x smaller.  Two one-key chunks with logits
    10 and 12 merge with weights in exactly that ratio."""
    with open(os.path.join(GOLDEN, "rescale_example.json")) as f:
        ex = json.load(f)
    old, new = ex["old_max"], ex["new_max"]
    po = np.zeros((2, 1, 1, 2), np.float32)
    po[0, 0, 0] = [1.0, 0.0]
    po[1, 0, 0] = [0.0, 1.0]
    pl = np.array([[[old]], [[new]]], np.float32)
    o, lse = oracle.merge(po, pl, lib=lib)
    ratio = o[0, 0, 0] / o[0, 0, 1]
    assert abs(ratio - ex["scale_factor"]) < 5e-4, ratio
    assert abs(1.0 / ratio - ex["shrink"]) < 0.05, 1.0 / ratio
    assert abs(lse[0, 0] - (new + math.log1p(math.exp(old - new)))) < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

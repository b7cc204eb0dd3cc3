"""Shared helpers for GPU-vs-oracle parity checks (used by the gpu tests and by smoke()).

Tolerances (max-abs, as the target states): 1e-2 for bf16 inputs, 1e-4 for
fp32 inputs, against the fp64 oracle.

bf16 outputs carry two roundings to 8 significant bits (unit roundoff 2^-8)
that a bare 1e-2 cannot absorb once |o| is a few units: the probabilities are
rounded to bf16 for the PV product (an error of up to 2^-8 sum_i p_i |v_i| / l,
about 2^-8 |o| when one value dominates), and the output itself is rounded to
nearest even (at most half an ulp of the stored value).  Two bars follow:

* ``literal=True`` (the five workloads at full size): the value the kernel
  computed before its output was rounded must be within 1e-2 of the oracle,
  i.e. |got - ref| <= 1e-2 + halfulp(got), halfulp(x) = 2^(floor(log2|x|) - 8);
* otherwise (small adversarial cases: a handful of keys, |o| up to ~4):
  |got - ref| <= 1e-2 + 2^-8 |ref|, which also covers the rounding of P.

The fp32 split-K partials carry neither rounding of the output and are compared
at the bare 1e-2 (tests/test_gpu_parity.py).  The log-sum-exp is fp32 in both
paths: 2e-3 (bf16 inputs: fp32 accumulation of bf16 products over the head
dimension) and 1e-4 (fp32 inputs), absolute.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sliding_window_attention_index_amd as sattn
from workloads import IndexedCase, WindowCase

SINK_NAMES = {0: "none", 1: "key0", 2: "null"}
TOL = {torch.bfloat16: 1e-2, torch.float32: 1e-4}
LSE_TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-4}


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values at |x| (x itself a bf16 value): the most that rounding a
    value to nearest even in bf16 can have moved it when the result is x.  Zero and subnormal
    results use the smallest normal exponent."""
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.where(np.isfinite(a), 2.0 ** (e - 8), np.inf)


def compare(got: torch.Tensor, ref: np.ndarray, dtype, what: str, lse: bool = False, tol: float | None = None,
            literal: bool = False) -> float:
    """Assert got (any device) matches ref (float64 numpy) elementwise; returns the max abs error.

    dtype is the input dtype (it picks the bar); `tol` replaces the bar with a bare max-abs value;
    `literal` takes the bare bar on the value before a bf16 output's rounding (module docstring)."""
    g = got.detach().float().cpu().numpy().astype(np.float64).reshape(ref.shape)
    same_inf = np.isinf(g) & np.isinf(ref) & (np.sign(g) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(g - ref))
    if tol is not None:
        allowed = np.full_like(ref, tol)
    elif lse:
        allowed = np.full_like(ref, LSE_TOL[dtype])
    elif dtype == torch.bfloat16 and got.dtype == torch.bfloat16:
        allowed = TOL[dtype] + (bf16_half_ulp(g) if literal else 2.0 ** -8 * np.abs(ref))
    else:
        allowed = np.full_like(ref, TOL[dtype])
    bad = ~(err <= allowed)  # NaN counts as bad
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, -1)), ref.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {ref.size} elements out of tolerance; worst at {i}: "
                             f"got {g[i]!r} ref {ref[i]!r} (err {err[i]:.3e}, allowed {allowed[i]:.3e})")
    return float(np.nanmax(np.where(same_inf, 0.0, err))) if err.size else 0.0


def run_window(case: WindowCase, device, return_lse=True):
    q, k, v = (t.to(device) for t in (case.q, case.k, case.v))
    cu = case.cu_seqlens.to(device)
    sinks = case.sinks.to(device) if case.sinks is not None else None
    return sattn.window_fwd(q, k, v, cu, case.max_seqlen, window=(case.window_left, case.window_right),
                            softmax_scale=case.scale, sinks=sinks, sink_mode=SINK_NAMES[case.sink_mode],
                            return_lse=return_lse)


def oracle_window(case: WindowCase, rows=None):
    return oracle.window(case.q, case.k, case.v, case.cu_seqlens, window_left=case.window_left,
                         window_right=case.window_right, scale=case.scale, sinks=case.sinks,
                         sink_mode=case.sink_mode, rows=rows)


def check_window(case: WindowCase, device, rows=None) -> dict:
    o, lse = run_window(case, device)
    torch.cuda.synchronize(device)
    ro, rl = oracle_window(case, rows)
    sel = slice(None) if rows is None else torch.as_tensor(np.asarray(rows, dtype=np.int64))
    dt = case.q.dtype
    e_o = compare(o.cpu()[sel], ro, dt, f"{case.name} o")
    e_l = compare(lse.cpu()[sel], rl, dt, f"{case.name} lse", lse=True)
    return {"max_abs_o": e_o, "max_abs_lse": e_l}


def run_indexed(case: IndexedCase, device, idx=None, num_splits=None, return_lse=True):
    q, kv = case.q.to(device), case.kv.to(device)
    idx = (case.topk_idxs if idx is None else idx).to(device)
    sinks = case.sinks.to(device) if case.sinks is not None else None
    return sattn.indexed_fwd(q, kv, idx, softmax_scale=case.scale, sinks=sinks,
                             sink_mode=SINK_NAMES[case.sink_mode],
                             num_splits=case.num_splits if num_splits is None else num_splits,
                             return_lse=return_lse)


def oracle_indexed(case: IndexedCase, rows=None, idx=None):
    return oracle.indexed(case.q, case.kv, case.topk_idxs if idx is None else idx, scale=case.scale,
                          sinks=case.sinks, sink_mode=case.sink_mode, rows=rows)


def check_indexed(case: IndexedCase, device, rows=None, num_splits=None) -> dict:
    o, lse = run_indexed(case, device, num_splits=num_splits)
    torch.cuda.synchronize(device)
    ro, rl = oracle_indexed(case, rows)
    B, M, H, D = case.q.shape
    o = o.cpu().reshape(B * M, H, D)
    lse = lse.cpu().reshape(B * M, H)
    sel = slice(None) if rows is None else torch.as_tensor(np.asarray(rows, dtype=np.int64))
    dt = case.q.dtype
    e_o = compare(o[sel], ro, dt, f"{case.name} o")
    e_l = compare(lse[sel], rl, dt, f"{case.name} lse", lse=True)
    return {"max_abs_o": e_o, "max_abs_lse": e_l}


def sample_rows(total: int, n: int, seed: int, must=()) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = rng.choice(total, size=min(n, total), replace=False)
    return np.unique(np.concatenate([pick, np.asarray([m for m in must if 0 <= m < total], dtype=np.int64)]))


def check_window_full(case: WindowCase, device, chunk: int = 4096) -> dict:
    """Every output element of a (large) window case against the oracle, in chunks of query rows so
    that the fp64 reference stays bounded; the GPU runs once, over the whole batch."""
    o, lse = run_window(case, device)
    torch.cuda.synchronize(device)
    o, lse = o.cpu(), lse.cpu()
    T = o.shape[0]
    dt = case.q.dtype
    e_o = e_l = 0.0
    for r0 in range(0, T, chunk):
        rows = np.arange(r0, min(T, r0 + chunk), dtype=np.int64)
        ro, rl = oracle_window(case, rows)
        e_o = max(e_o, compare(o[r0:r0 + rows.size], ro, dt, f"{case.name} o rows {r0}..", literal=True))
        e_l = max(e_l, compare(lse[r0:r0 + rows.size], rl, dt, f"{case.name} lse rows {r0}..", lse=True))
    return {"max_abs_o": e_o, "max_abs_lse": e_l, "rows": T}


def check_indexed_full(case: IndexedCase, device, chunk: int = 2048, num_splits=None) -> dict:
    """Every output element of a (large) indexed case against the oracle, in chunks of queries."""
    o, lse = run_indexed(case, device, num_splits=num_splits)
    torch.cuda.synchronize(device)
    B, M, H, D = case.q.shape
    o = o.cpu().reshape(B * M, H, D)
    lse = lse.cpu().reshape(B * M, H)
    dt = case.q.dtype
    e_o = e_l = 0.0
    for r0 in range(0, B * M, chunk):
        rows = np.arange(r0, min(B * M, r0 + chunk), dtype=np.int64)
        ro, rl = oracle_indexed(case, rows)
        e_o = max(e_o, compare(o[r0:r0 + rows.size], ro, dt, f"{case.name} o rows {r0}..", literal=True))
        e_l = max(e_l, compare(lse[r0:r0 + rows.size], rl, dt, f"{case.name} lse rows {r0}..", lse=True))
    return {"max_abs_o": e_o, "max_abs_lse": e_l, "rows": B * M}


def split_slices(topk: int, num_splits: int):
    """The contiguous list slices of a split-K call: ceil(topk / S) entries each, slices that would
    hold no entry not created (include/sattn.h, sattn_indexed_args.num_splits)."""
    per = -(-topk // num_splits)
    return [(s, min(topk, s + per)) for s in range(0, topk, per)]


def workspace_partials(workspace: torch.Tensor, num_splits: int, rows: int, heads: int, dim: int, parts: int):
    """The fp32 partials a split-K call leaves in its workspace (include/sattn.h: part_o
    [S, rows, H, D], then part_lse [S, rows, H], each from a 256-byte boundary; S = num_splits sizes
    the layout, the first `parts` slices are written)."""
    n_o = num_splits * rows * heads * dim * 4
    off = -(-n_o // 256) * 256
    po = workspace[:n_o].view(torch.float32).view(num_splits, rows, heads, dim)[:parts]
    pl = workspace[off:off + num_splits * rows * heads * 4].view(torch.float32).view(num_splits, rows, heads)[:parts]
    return po, pl

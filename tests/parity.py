"""Shared helpers for GPU-vs-oracle parity checks (used by the gpu tests and by smoke()).

Tolerances (max-abs, as the target states): 1e-2 for bf16 inputs, 1e-4 for
fp32 inputs.  A bf16 output additionally carries its own round-to-nearest
error of at most 2^-9 |o| (half an ulp), which exceeds 1e-2 once |o| > 5; the
allowance per element is therefore tol + 2^-9 |o_ref| for bf16 outputs.
The log-sum-exp is fp32 in both paths: 2e-3 (bf16 inputs: fp32 accumulation of
bf16 products over the head dimension) and 1e-4 (fp32 inputs), absolute.
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


def compare(got: torch.Tensor, ref: np.ndarray, dtype, what: str, lse: bool = False) -> float:
    """Assert got (any device) matches ref (float64 numpy) elementwise; returns the max abs error."""
    g = got.detach().float().cpu().numpy().astype(np.float64).reshape(ref.shape)
    same_inf = np.isinf(g) & np.isinf(ref) & (np.sign(g) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(g - ref))
    if lse:
        allowed = np.full_like(ref, LSE_TOL[dtype])
    else:
        # a bf16 output adds its own rounding: half an ulp, up to 2^-8 |o| for 8 significant bits
        allowed = TOL[dtype] + (2.0 ** -8 * np.abs(ref) if dtype == torch.bfloat16 else 0.0)
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

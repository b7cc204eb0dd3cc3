"""CPU oracle for index-gathered attention forward (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never does.  The arithmetic lives in
``sattn_oracle.c`` (plain C, double precision); this module only builds it
with gcc, marshals numpy/torch arrays and converts bf16 inputs to fp32
(an exact widening).

Functions follow the pages that define the problem:
  * ``window``  -- vLLM PR #49815 report, the dense window reference and the
    two sink semantics of ``_fwd_kernel``;
  * ``indexed`` -- DeepSeek-V4 CSA/HCA article §4.2-§4.4 (top-k gather over a
    shared K=V cache, -1 padding, null-logit sink);
  * ``merge``   -- nano-vllm XAttention offload note, three-stage chunked
    softmax statistics.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "sattn_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

SINK_NONE, SINK_KEY0, SINK_NULL = 0, 1, 2
_ERRORS = {-1: "bad arguments", -2: "duplicate index in a top-k list", -3: "out of memory"}


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (OpenMP over query rows)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load (building first if needed) the oracle library; a custom path gives a separate handle."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _declare(ctypes.CDLL(LIB))
    return _lib


def _declare(lib):
    P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_window.argtypes = [P, P, P, P, I, I, I, I, I, I, D, P, I, P, L, P, P, I]
    lib.oracle_window.restype = I
    lib.oracle_indexed.argtypes = [P, P, P, I, I, I, I, I, I, D, P, I, P, L, P, P, I]
    lib.oracle_indexed.restype = I
    lib.oracle_merge.argtypes = [P, P, I, L, I, I, P, I, P, P]
    lib.oracle_merge.restype = I
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    return lib


def _f32(x) -> np.ndarray:
    """Any tensor/array -> contiguous fp32 numpy (bf16 -> fp32 is exact)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype != torch.float32:
                x = x.to(torch.float32)
            return np.ascontiguousarray(x.numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().to("cpu").to(torch.int32).numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise ValueError(f"oracle: {_ERRORS.get(rc, rc)}")


def window(q, k, v, cu_seqlens, *, window_left: int, window_right: int, scale: float,
           sinks=None, sink_mode: int = SINK_NONE, rows=None, nthreads: int = 0, lib=None):
    """Window attention over a cu_seqlens batch.  Returns (o [R,H,D], lse [R,H]) float64.

    q [T,H,D], k/v [T,Hkv,D]; rows = token indices to evaluate (None = all).
    """
    lib = lib or load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu = _i32(cu_seqlens)
    T, H, D = q.shape
    Hkv = k.shape[1]
    s = None if sinks is None else _f32(sinks)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = T if r is None else r.size
    o = np.zeros((R, H, D), dtype=np.float64)
    lse = np.zeros((R, H), dtype=np.float64)
    _check(lib.oracle_window(_ptr(q), _ptr(k), _ptr(v), _ptr(cu), cu.size - 1, H, Hkv, D,
                             int(window_left), int(window_right), float(scale), _ptr(s), int(sink_mode),
                             _ptr(r), 0 if r is None else r.size, _ptr(o), _ptr(lse), int(nthreads)))
    return o, lse


def indexed(q, kv, topk_idxs, *, scale: float, sinks=None, sink_mode: int = SINK_NONE, rows=None,
            nthreads: int = 0, lib=None):
    """Top-k gathered attention over a shared K=V cache.  Returns (o [R,H,D], lse [R,H]) float64.

    q [B,M,H,D], kv [B,N,D], topk_idxs [B,M,K]; rows = flat query indices b*M+t (None = all).
    """
    lib = lib or load()
    q, kv, idx = _f32(q), _f32(kv), _i32(topk_idxs)
    B, M, H, D = q.shape
    N = kv.shape[1]
    K = idx.shape[2]
    s = None if sinks is None else _f32(sinks)
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    R = B * M if r is None else r.size
    o = np.zeros((R, H, D), dtype=np.float64)
    lse = np.zeros((R, H), dtype=np.float64)
    _check(lib.oracle_indexed(_ptr(q), _ptr(kv), _ptr(idx), B, M, H, D, N, K, float(scale), _ptr(s),
                              int(sink_mode), _ptr(r), 0 if r is None else r.size, _ptr(o), _ptr(lse),
                              int(nthreads)))
    return o, lse


def merge(part_o, part_lse, *, sinks=None, sink_mode: int = SINK_NONE, lib=None):
    """Merge chunk partials part_o [S,R,H,D], part_lse [S,R,H].  Returns (o [R,H,D], lse [R,H]) float64."""
    lib = lib or load()
    po, pl = _f32(part_o), _f32(part_lse)
    S, R, H, D = po.shape
    s = None if sinks is None else _f32(sinks)
    o = np.zeros((R, H, D), dtype=np.float64)
    lse = np.zeros((R, H), dtype=np.float64)
    _check(lib.oracle_merge(_ptr(po), _ptr(pl), S, R, H, D, _ptr(s), int(sink_mode), _ptr(o), _ptr(lse)))
    return o, lse


def max_threads(lib=None) -> int:
    return (lib or load()).oracle_max_threads()

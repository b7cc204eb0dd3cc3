"""CPU oracle for attention over an fp8 KV cache (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import this module; the product path never does.

Source: DeepSeek-V4 CSA/HCA article, §5.3 (after pooling the compressed kv is quantised: the
dims without rotary embedding to fp8, the rotary dims kept at higher precision) and §4.2 (one
cache row serves as the key and the value of every head).  Readings, since the article fixes no
layout: a row of ``D`` dims holds its first ``D - rope_dims`` dims as fp8 e4m3 codes (the OCP
"fn" variant: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is
NaN) times one power-of-two fp32 scale per row, and its last ``rope_dims`` dims as bf16.  The
attention over the dequantised rows is the indexed oracle's.
"""
from __future__ import annotations

import numpy as np

from . import indexed as _indexed


def e4m3_decode(codes) -> np.ndarray:
    """Values of fp8 e4m3 (OCP fn) codes, float64; NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e - 7.0)
    subnormal = sign * (m / 8.0) * np.exp2(-6.0)
    v = np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (m == 7), np.nan, v)


def dequant_rows(kv8, scale, kv_rope=None) -> np.ndarray:
    """Rows [B, N, D] as float32 (exact): e4m3(kv8) * scale on the first D - rope_dims dims, then
    kv_rope.  kv8 uint8 [B, N, D - rope_dims], scale [B, N] (powers of two), kv_rope [B, N, rd]."""
    k8 = np.asarray(kv8.cpu().numpy() if hasattr(kv8, "cpu") else kv8, dtype=np.uint8)
    sc = np.asarray(scale.float().cpu().numpy() if hasattr(scale, "cpu") else scale, dtype=np.float64)
    rows = e4m3_decode(k8) * sc[..., None]
    if kv_rope is not None and kv_rope.shape[-1] > 0:
        rope = np.asarray(kv_rope.float().cpu().numpy() if hasattr(kv_rope, "cpu") else kv_rope, dtype=np.float64)
        rows = np.concatenate([rows, rope], axis=-1)
    out = rows.astype(np.float32)
    assert np.array_equal(out.astype(np.float64), rows, equal_nan=True), "dequantised rows are not exact in fp32"
    return out


def indexed_fp8(q, kv8, scale, kv_rope, topk_idxs, *, softmax_scale: float, sinks=None, sink_mode: int = 0,
                rows=None, nthreads: int = 0):
    """Top-k attention over the dequantised fp8 cache.  Returns (o [R,H,D], lse [R,H]) float64."""
    return _indexed(q, dequant_rows(kv8, scale, kv_rope), topk_idxs, scale=softmax_scale, sinks=sinks,
                    sink_mode=sink_mode, rows=rows, nthreads=nthreads)

"""GPU parity of the compressor's gated pooling (sattn_compress_pool) against the oracle.

Tolerance: the kernel computes in fp32 (online softmax over at most 2 * ratio entries per
feature, base-2 exponentials), a relative error of a few 1e-7; an fp32 output is allowed
1e-5 * |ref| + 1e-6, a bf16 output its own rounding (up to 2^-9 |ref|, twice that when the fp32
value sits next to a rounding boundary) plus 1e-5.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import sliding_window_attention_index_amd as sattn
from oracle import index_lists as IL

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()
    return torch.device("cuda:0")


def _inputs(B, S, d, ratio, overlap, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    F = (2 if overlap else 1) * d
    kv = torch.randn(B, S, F, generator=g).to(dtype)
    score = (2.0 * torch.randn(B, S, F, generator=g)).to(dtype)
    ape = (0.5 * torch.randn(ratio, F, generator=g)).to(dtype)
    return kv, score, ape


def _check(got, ref, dtype, what):
    g = got.float().cpu().numpy().astype(np.float64)
    if dtype == torch.bfloat16:
        allowed = 2.0 ** -8 * np.abs(ref) + 1e-5
    else:
        allowed = 1e-5 * np.abs(ref) + 1e-6
    err = np.abs(g - ref)
    bad = ~(err <= allowed)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {ref.size} out of tolerance; max err {err.max():.3e}"
    print(f"[parity] compress {what}: max_abs {err.max() if err.size else 0.0:.3e}", flush=True)


CASES = [
    # B, S, d, ratio, overlap, dtype
    (2, 37, 64, 4, True, torch.bfloat16),     # trailing partial window
    (1, 64, 128, 4, False, torch.bfloat16),
    (3, 40, 8, 8, True, torch.float32),
    (1, 16, 128, 1, True, torch.bfloat16),    # ratio 1
    (2, 100, 16, 16, True, torch.float32),
    (1, 4, 128, 4, True, torch.bfloat16),     # one window: no previous half
    (2, 250, 24, 4, False, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_compress_cases(dev, case):
    B, S, d, ratio, overlap, dt = case
    kv, score, ape = _inputs(B, S, d, ratio, overlap, dt, seed=S)
    got = sattn.compress_pool(kv.to(dev), score.to(dev), ape.to(dev), ratio=ratio, overlap=overlap)
    torch.cuda.synchronize(dev)
    ref = IL.compress_pool(kv, score, ape, ratio=ratio, overlap=overlap)
    assert tuple(got.shape) == ref.shape
    _check(got, ref, dt, f"B{B} S{S} d{d} r{ratio} ov{int(overlap)}")


def test_compress_no_complete_window(dev):
    kv, score, ape = _inputs(1, 3, 128, 4, True, torch.bfloat16, seed=1)
    got = sattn.compress_pool(kv.to(dev), score.to(dev), ape.to(dev), ratio=4, overlap=True)
    assert tuple(got.shape) == (1, 0, 128)


def test_compress_full_prefill_into_cache(dev):
    """The prefill sequence: 32768 tokens, ratio 4 with overlap, D 128 -> the 8192 compressed rows of
    a [1, 128 + 8192, 128] cache, written in place after its 128-row window region."""
    B, S, d, ratio = 1, 32768, 128, 4
    kv, score, ape = _inputs(B, S, d, ratio, True, torch.bfloat16, seed=7)
    cache = torch.full((B, 128 + S // ratio, d), 3.0, dtype=torch.bfloat16, device=dev)
    sattn.compress_pool(kv.to(dev), score.to(dev), ape.to(dev), ratio=ratio, overlap=True, out=cache[:, 128:, :])
    torch.cuda.synchronize(dev)
    c = cache.cpu()
    assert bool((c[:, :128] == 3.0).all())  # the window region is untouched
    ref = IL.compress_pool(kv, score, ape, ratio=ratio, overlap=True)
    _check(c[:, 128:], ref, torch.bfloat16, "prefill 32768 tokens into the cache")


def test_compress_batch_stride(dev):
    """Two batch rows written into a strided view: rows past S // ratio of each batch stay untouched."""
    B, S, d, ratio = 2, 48, 32, 4
    kv, score, ape = _inputs(B, S, d, ratio, False, torch.float32, seed=3)
    buf = torch.full((B, 20, d), -7.0, dtype=torch.float32, device=dev)
    sattn.compress_pool(kv.to(dev), score.to(dev), ape.to(dev), ratio=ratio, overlap=False, out=buf)
    torch.cuda.synchronize(dev)
    b = buf.cpu()
    assert bool((b[:, 12:] == -7.0).all())
    _check(b[:, :12], IL.compress_pool(kv, score, ape, ratio=ratio, overlap=False), torch.float32, "batch stride")

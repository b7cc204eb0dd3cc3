"""Seeded random shapes across the dispatch boundaries, every output element against the oracle.

The other parity tests pin chosen cases (the five configurations, edge cases, adversarial bands).
This sweep draws shapes at random, with a fixed seed, over everything the two attention entry
points accept: MFMA and VALU head dims, head counts on and off the 32-head MFMA tile, GQA group
sizes, windows that are one-sided, unbounded or empty, -1 pads and out-of-range list entries,
every sink mode, split-K from 1 to 8 slices, and indexed launches on both sides of the
4096 (query, slice) boundary where the decode-shape kernel hands over to the one-wave-per-task
kernel.  Sizes stay small enough for the fp64 oracle to take well under a second per case.
"""
import numpy as np
import pytest
import torch

import workloads as W
from parity import SINK_NAMES, check_indexed, check_window

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import sliding_window_attention_index_amd as sattn
    sattn.load_library()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def _lists(rng, B, M, N, K):
    """Distinct rows per list (the oracle's precondition), a random number of them, at random
    positions among -1 pads; now and then entries at or past N (skipped like -1)."""
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            n = int(rng.integers(0, min(K, N) + 1)) if N > 0 else 0
            if n:
                idx[b, t, :n] = rng.choice(N, size=n, replace=False)
            idx[b, t] = idx[b, t, rng.permutation(K)]
            if rng.random() < 0.2:
                pads = np.flatnonzero(idx[b, t] < 0)
                if pads.size:
                    idx[b, t, pads[0]] = N + int(rng.integers(0, 50))
    return idx


def _indexed_specs(n_cases, seed):
    rng = np.random.default_rng(seed)
    specs = []
    for i in range(n_cases):
        H = int(rng.choice([8, 16, 32, 32, 64, 64, 96]))
        D = int(rng.choice([64, 64, 128, 128, 128, 96, 32]))
        dt = torch.float32 if rng.random() < 0.15 else torch.bfloat16
        big = i % 6 == 5  # enough (query, slice) pairs for the one-wave-per-task kernel
        B = 2 if big else int(rng.integers(1, 3))
        M = int(rng.integers(2100, 2600)) if big else int(rng.choice([1, 2, 5, 17, 33, 130]))
        N = int(rng.integers(1, 3000))
        K = int(rng.integers(1, 48)) if big else int(rng.integers(1, 600))
        splits = int(rng.choice([1, 1, 2, 3, 8]))
        mode = int(rng.integers(0, 3))
        specs.append((f"idx{i}_b{B}m{M}h{H}d{D}n{N}k{K}s{splits}_{SINK_NAMES[mode]}_{str(dt)[6:]}",
                      B, M, H, D, N, K, splits, mode, dt, int(rng.integers(0, 2**31))))
    return specs


INDEXED = _indexed_specs(60, 2024)


@pytest.mark.parametrize("spec", INDEXED, ids=[s[0] for s in INDEXED])
def test_indexed_random_shapes(dev, spec):
    name, B, M, H, D, N, K, splits, mode, dt, seed = spec
    rng = np.random.default_rng(seed)
    idx = _lists(rng, B, M, N, K)
    if mode == W.SINK_KEY0 and N > 0:
        # put cache row 0 into some lists (the key-0 bias only shows where row 0 is listed)
        for b in range(B):
            for t in range(0, M, 3):
                if 0 not in idx[b, t] and (idx[b, t] < 0).any():
                    idx[b, t, int(np.flatnonzero(idx[b, t] < 0)[0])] = 0
    case = W.make_indexed_case(name, B, M, H, D, N, idx, mode, dtype=dt, seed=seed % 1000, num_splits=splits)
    r = check_indexed(case, dev)
    print(f"[parity] {name}: {r}", flush=True)


def _window_specs(n_cases, seed):
    rng = np.random.default_rng(seed)
    specs = []
    for i in range(n_cases):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8, 16, 32, 3, 6]))
        H = Hkv * G
        if H > 64:
            G = max(1, 64 // Hkv)
            H = Hkv * G
        D = int(rng.choice([64, 64, 128, 128, 96, 32]))
        dt = torch.float32 if rng.random() < 0.15 else torch.bfloat16
        S = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(0, 400, size=S)]
        if sum(lens) == 0:
            lens[0] = 1
        kind = rng.integers(0, 5)
        if kind == 0:
            wl = wr = int(rng.integers(0, 160))            # symmetric
        elif kind == 1:
            wl, wr = int(rng.integers(0, 200)), 0           # causal
        elif kind == 2:
            wl, wr = int(rng.integers(0, 100)), int(rng.integers(0, 100))
        elif kind == 3:
            wl, wr = -1, int(rng.integers(0, 50))          # unbounded on the left
        else:
            wl, wr = -1, -1                                 # full attention
        mode = int(rng.integers(0, 3))
        specs.append((f"win{i}_s{S}h{H}g{G}d{D}_w{wl}_{wr}_{SINK_NAMES[mode]}_{str(dt)[6:]}",
                      lens, H, Hkv, D, wl, wr, mode, dt, int(rng.integers(0, 2**31))))
    return specs


WINDOW = _window_specs(60, 7)


@pytest.mark.parametrize("spec", WINDOW, ids=[s[0] for s in WINDOW])
def test_window_random_shapes(dev, spec):
    name, lens, H, Hkv, D, wl, wr, mode, dt, seed = spec
    case = W.make_window_case(name, lens, H, Hkv, D, wl, wr, mode, dtype=dt, seed=seed % 1000)
    r = check_window(case, dev)
    print(f"[parity] {name}: {r}", flush=True)


def _fp8_specs(n_cases, seed):
    rng = np.random.default_rng(seed)
    specs = []
    for i in range(n_cases):
        H = int(rng.choice([32, 64, 96]))
        rd = int(rng.choice([0, 64]))
        big = i % 5 == 4  # 4096 or more (query, head group, slice) tasks: the 2-slot ring
        B = 2 if big else int(rng.integers(1, 3))
        M = int(rng.integers(1100, 1400)) if big else int(rng.choice([1, 3, 17, 130]))
        N = int(rng.integers(1, 2000))
        K = int(rng.integers(1, 40)) if big else int(rng.integers(1, 600))
        splits = int(rng.choice([1, 1, 2, 3, 8]))
        mode = int(rng.integers(0, 3))
        specs.append((f"fp8_{i}_b{B}m{M}h{H}rd{rd}n{N}k{K}s{splits}_{SINK_NAMES[mode]}",
                      B, M, H, rd, N, K, splits, mode, int(rng.integers(0, 2**31))))
    return specs


FP8 = _fp8_specs(20, 99)


@pytest.mark.parametrize("spec", FP8, ids=[s[0] for s in FP8])
def test_indexed_fp8_random_shapes(dev, spec):
    """The fp8 cache entry point on the same kind of lists, unit-scale rows (the bf16 bar's
    reading: the probabilities' rounding stays within it while |v| is near |o|)."""
    import sliding_window_attention_index_amd as sattn
    from oracle import fp8_cache as F8
    from parity import compare
    name, B, M, H, rd, N, K, splits, mode, seed = spec
    rng = np.random.default_rng(seed)
    kv8, sc, rope = W.fp8_cache(seed % 1000, B, N, 128, rd, scale_spread=0)
    g = torch.Generator().manual_seed(seed % 1000 + 1)
    q = torch.randn(B, M, H, 128, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    idx = torch.from_numpy(_lists(rng, B, M, N, K))
    o, lse = sattn.indexed_fp8_fwd(q.to(dev), kv8.to(dev), sc.to(dev), rope.to(dev) if rd else None, idx.to(dev),
                                   sinks=sinks.to(dev) if mode else None, sink_mode=SINK_NAMES[mode],
                                   num_splits=splits, return_lse=True)
    torch.cuda.synchronize(dev)
    o_ref, l_ref = F8.indexed_fp8(q, kv8, sc, rope if rd else None, idx, softmax_scale=128 ** -0.5,
                                  sinks=sinks, sink_mode=mode)
    e = compare(o, o_ref, torch.bfloat16, f"{name} o")
    compare(lse, l_ref, torch.bfloat16, f"{name} lse", lse=True)
    print(f"[parity] {name}: max_abs {e:.3e}", flush=True)

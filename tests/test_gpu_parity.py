"""GPU parity: libsattn (through its C ABI) against the CPU oracle, element by element.

Reduced versions of the five workloads and the full-size workloads, launched
exactly as bench.py times them, are compared on every output element (the
full-size ones in chunks of query rows, so the fp64 reference stays bounded).
The fp32 split-K partials, which carry no output rounding, are compared with
the oracle run on each slice alone at the bare max-abs 1e-2.  Edge cases cover
what the pages flag as risks: windows narrower than a key block, tiles that
start at a sequence boundary (key-0 placement), bands clipped at key 0 so that
rows of one tile reach their first key in different blocks, length-1 and empty
sequences, all-padding index lists, split counts that leave empty slices, and a
non-default stream fed through an event.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_index_amd as sattn
import workloads as W
from parity import (check_indexed, check_indexed_full, check_window, check_window_full, compare, oracle_indexed,
                    oracle_window, run_indexed, run_window, sample_rows, split_slices, workspace_partials)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def _log(name, res):
    print(f"[parity] {name}: {res}", flush=True)


# ---------------------------------------------------------------------------
# window path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kv_heads", [4, 2])
def test_tiny_window_fp32(dev, kv_heads):
    """The page's own test shape: lengths 5 and 37, window 8, 4 heads, key-0 sinks, fp32."""
    case = W.tiny_window_fp32(kv_heads)
    _log(case.name, check_window(case, dev))


WINDOW_CASES = [
    # name, lens, H, Hkv, D, (wl, wr), sink mode, dtype
    ("vision_reduced", [300, 1, 517, 64, 129], 16, 8, 128, (128, 128), W.SINK_KEY0, torch.bfloat16),
    ("causal_null_reduced", [700, 333], 64, 8, 64, (127, 0), W.SINK_NULL, torch.bfloat16),
    ("narrow_window", [70, 3, 45], 8, 2, 128, (3, 2), W.SINK_KEY0, torch.bfloat16),
    ("full_noncausal", [90, 17], 4, 4, 64, (-1, -1), W.SINK_NONE, torch.bfloat16),
    ("full_causal", [150], 8, 1, 64, (-1, 0), W.SINK_NULL, torch.bfloat16),
    ("left_only_unbounded", [100], 32, 1, 128, (-1, 5), W.SINK_KEY0, torch.bfloat16),
    ("gqa16", [80, 40], 16, 1, 128, (20, 20), W.SINK_NONE, torch.bfloat16),
    ("gqa32", [50], 32, 1, 64, (10, 0), W.SINK_NULL, torch.bfloat16),
    ("gqa4_d64", [200, 33], 16, 4, 64, (64, 64), W.SINK_KEY0, torch.bfloat16),
    ("mha_d128", [130, 65], 4, 4, 128, (40, 40), W.SINK_NULL, torch.bfloat16),
    ("gqa8_d128", [300, 7], 16, 2, 128, (127, 0), W.SINK_KEY0, torch.bfloat16),
    ("gqa16_d64", [90, 31], 16, 1, 64, (15, 15), W.SINK_NULL, torch.bfloat16),
    ("gqa2_d64", [260, 3], 8, 4, 64, (32, 64), W.SINK_KEY0, torch.bfloat16),
    # D = 64 runs eight-wave workgroups: 8 * 32 / G queries a tile (256 at G = 1, 128 at G = 2, 32 at
    # G = 8); sequences one query past, one short of and several tiles long.
    ("mha_d64_tiles", [700, 257, 255], 4, 4, 64, (100, 60), W.SINK_KEY0, torch.bfloat16),
    ("gqa2_d64_long_causal", [600, 129], 8, 4, 64, (-1, 0), W.SINK_NULL, torch.bfloat16),
    ("gqa8_d64_window", [520, 33, 32], 32, 4, 64, (127, 0), W.SINK_NULL, torch.bfloat16),
    ("empty_seqs", [0, 40, 0, 1, 0], 4, 2, 64, (8, 8), W.SINK_KEY0, torch.bfloat16),
    ("valu_gqa3", [60, 9], 6, 2, 64, (7, 7), W.SINK_KEY0, torch.bfloat16),
    ("valu_d96", [45], 4, 2, 96, (5, 5), W.SINK_NULL, torch.bfloat16),
    ("valu_d256", [33], 2, 1, 256, (4, 4), W.SINK_KEY0, torch.bfloat16),
    ("fp32_vision", [129, 64], 16, 8, 128, (128, 128), W.SINK_KEY0, torch.float32),
    ("fp32_causal_null", [100], 16, 2, 64, (31, 0), W.SINK_NULL, torch.float32),
    ("fp32_none", [70, 1], 4, 4, 32, (-1, -1), W.SINK_NONE, torch.float32),
]


@pytest.mark.parametrize("spec", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_window_cases(dev, spec):
    name, lens, H, Hkv, D, (wl, wr), mode, dt = spec
    case = W.make_window_case(name, lens, H, Hkv, D, wl, wr, mode, dtype=dt, seed=7)
    _log(name, check_window(case, dev))


def test_window_sink_bit_exact_invariants(dev):
    """Key-0 sink 0 == no sink and null sink -inf == no sink, bit for bit on the GPU as well."""
    base = W.make_window_case("inv", [200, 77], 16, 8, 128, 128, 128, W.SINK_NONE, seed=3)
    o0 = run_window(base, dev, return_lse=False)
    for mode, val in ((W.SINK_KEY0, 0.0), (W.SINK_NULL, -math.inf)):
        c = W.make_window_case("inv", [200, 77], 16, 8, 128, 128, 128, mode, seed=3, sinks_value=val)
        assert torch.equal(c.q, base.q)
        o1 = run_window(c, dev, return_lse=False)
        assert torch.equal(o0, o1), f"sink mode {mode} with neutral value changed the output"


def test_window_max_seqlen_bounds_work(dev):
    """Tokens beyond max_seqlen are not computed (the grid is sized by it, as the page's max_input_len)."""
    case = W.make_window_case("bound", [64, 40], 8, 2, 128, 8, 8, W.SINK_NONE, seed=4)
    q, k, v = (t.to(dev) for t in (case.q, case.k, case.v))
    out = torch.full_like(q, 7.0)
    sattn.window_fwd(q, k, v, case.cu_seqlens.to(dev), 40, window=(8, 8), out=out)
    torch.cuda.synchronize()
    ro, _ = oracle_window(case)
    o = out.cpu()
    compare(o[:40], ro[:40], torch.bfloat16, "first 40 of seq 0")
    compare(o[64:], ro[64:], torch.bfloat16, "seq 1")
    assert torch.all(o[40:64] == 7.0)


def test_vision_window_full_size(dev):
    """16 sequences, lengths U[1024,4096], 16/8 heads, D=128, window +-128, key-0 sinks (bench workload):
    every element of o and lse."""
    _log("vision_window full", check_window_full(W.vision_window(), dev))


def test_causal_window_full_size(dev):
    """4 x 8192 tokens, 64/8 heads, D=64, causal 128-key window, null sinks: every element of o and lse."""
    _log("causal_window_null full", check_window_full(W.causal_window_null(), dev))


# Bands clipped at key 0 inside a tile: rows of one wave see their first key in different key blocks,
# so a block can be empty for some rows while the running max of others grows.
CLIPPED = [
    # name, lens, H, Hkv, D, (wl, wr)
    ("clip_g1_w40", [130, 65], 4, 4, 128, (40, 40)),
    ("clip_g2_w20", [64, 300], 4, 2, 128, (20, 20)),
    ("clip_g1_d64_w40", [200, 33], 4, 4, 64, (40, 40)),
    ("clip_g4_d64_w9", [150, 70], 8, 2, 64, (9, 3)),
]


CLIPPED_MODES = [(W.SINK_NONE, False), (W.SINK_KEY0, False), (W.SINK_NULL, False), (W.SINK_KEY0, True),
                 (W.SINK_NULL, True)]


@pytest.mark.parametrize("spec", CLIPPED, ids=[c[0] for c in CLIPPED])
@pytest.mark.parametrize("mode,neg_inf_sinks", CLIPPED_MODES, ids=["none", "key0", "null", "key0_neginf", "null_neginf"])
def test_window_clipped_band(dev, spec, mode, neg_inf_sinks):
    name, lens, H, Hkv, D, (wl, wr) = spec
    case = W.make_window_case(f"{name}_m{mode}", lens, H, Hkv, D, wl, wr, mode, seed=21)
    if neg_inf_sinks:
        case.sinks[::2] = -math.inf  # every other head: a key-0 logit of -inf, or a null sink that adds nothing
    _log(case.name + ("_neginf" if neg_inf_sinks else ""), check_window(case, dev))


# ---------------------------------------------------------------------------
# indexed path
# ---------------------------------------------------------------------------

def test_sparse_prefill_reduced_with_padding(dev):
    """Top-k prefill, queries at positions 0.. (short lists padded with -1), 32 heads, D=128."""
    case = W.sparse_prefill_case(q_len=300, total_tokens=4096, n_pick=64, first_pos=0, name="prefill_pad")
    _log(case.name, check_indexed(case, dev))


def test_sparse_prefill_reduced_tail(dev):
    case = W.sparse_prefill_case(q_len=256, total_tokens=4096, n_pick=96, name="prefill_tail")
    _log(case.name, check_indexed(case, dev))


@pytest.mark.parametrize("mode", [W.SINK_KEY0, W.SINK_NULL])
def test_sparse_prefill_sinks(dev, mode):
    """Window ring slot 0 is cache row 0, so the key-0 bias is exercised by many lists."""
    case = W.sparse_prefill_case(q_len=200, total_tokens=2048, n_pick=40, first_pos=100, sink_mode=mode,
                                 name=f"prefill_sink{mode}")
    _log(case.name, check_indexed(case, dev))


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 19])
@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_NULL, W.SINK_KEY0])
def test_sparse_decode_reduced_splits(dev, splits, mode):
    """Decode: 4 sequences x 1 query, 64 heads sharing one cache row per token, split-K + merge."""
    case = W.sparse_decode_case(batch=4, total_tokens=8192, n_pick=480, num_splits=splits, sink_mode=mode,
                                name=f"decode_s{splits}_m{mode}")
    _log(case.name, check_indexed(case, dev))


INDEXED_EDGE = [
    # name, B, M, H, D, N, K, pad pattern, dtype, splits
    ("all_pad", 1, 3, 32, 128, 50, 40, "all", torch.bfloat16, 1),
    ("all_pad_split", 1, 3, 64, 128, 50, 40, "all", torch.bfloat16, 4),
    ("ragged_k", 2, 5, 32, 64, 300, 45, "some", torch.bfloat16, 1),
    ("k1", 1, 4, 32, 128, 10, 1, "none", torch.bfloat16, 1),
    ("out_of_range", 1, 4, 32, 128, 64, 40, "oob", torch.bfloat16, 1),
    ("empty_cache", 1, 2, 32, 128, 0, 8, "all", torch.bfloat16, 1),
    ("valu_h16", 2, 3, 16, 128, 200, 70, "some", torch.bfloat16, 1),
    ("valu_h16_split", 2, 3, 16, 64, 200, 70, "some", torch.bfloat16, 3),
    ("fp32", 1, 6, 32, 128, 200, 64, "some", torch.float32, 1),
    ("fp32_split", 1, 6, 8, 64, 200, 64, "some", torch.float32, 4),
]


def _edge_lists(rng, B, M, N, K, pattern):
    idx = np.full((B, M, K), -1, np.int32)
    for b in range(B):
        for t in range(M):
            if pattern == "all" or N == 0:
                continue
            n = K if pattern == "none" else int(rng.integers(0, min(K, N) + 1))
            n = min(n, N)
            idx[b, t, :n] = rng.choice(N, size=n, replace=False)
            if pattern == "some":
                idx[b, t] = idx[b, t, rng.permutation(K)]
            if pattern == "oob":
                idx[b, t, ::7] = N + 3 + t  # outside the cache: must be ignored
    return idx


@pytest.mark.parametrize("spec", INDEXED_EDGE, ids=[c[0] for c in INDEXED_EDGE])
@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_KEY0, W.SINK_NULL])
def test_indexed_edge_cases(dev, spec, mode):
    name, B, M, H, D, N, K, pattern, dt, splits = spec
    rng = np.random.default_rng(5)
    idx = _edge_lists(rng, B, M, N, K, pattern)
    if mode == W.SINK_KEY0 and N > 0 and pattern != "all":
        idx[0, 0, 0] = 0 if 0 not in idx[0, 0] else idx[0, 0, 0]
    case = W.make_indexed_case(f"{name}_m{mode}", B, M, H, D, N, idx, mode, dtype=dt, seed=9, num_splits=splits)
    _log(case.name, check_indexed(case, dev))


MANY_TASKS = [
    # name, B, M, H, D, N, K, pad pattern, splits: 4096 or more (query, 32 heads, slice) tasks take
    # the launch with a 2-tile ring per wave; fewer take the 4-tile one.
    ("many_some", 2, 2048, 32, 128, 3000, 70, "some", 1),
    ("many_oob_split", 1, 2048, 64, 128, 3000, 100, "oob", 3),
    ("many_pad_k33", 1, 4100, 32, 128, 500, 33, "some", 1),
    ("many_d64", 1, 2048, 64, 64, 1000, 90, "some", 1),
    ("many_d64_split", 1, 1024, 32, 64, 800, 200, "oob", 4),
]


@pytest.mark.parametrize("spec", MANY_TASKS, ids=[c[0] for c in MANY_TASKS])
@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_KEY0, W.SINK_NULL])
def test_indexed_many_tasks(dev, spec, mode):
    name, B, M, H, D, N, K, pattern, splits = spec
    rng = np.random.default_rng(13)
    idx = _edge_lists(rng, B, M, N, K, pattern)
    if mode == W.SINK_KEY0:
        sub = idx[:, ::5]
        sub[~(sub == 0).any(-1), 1] = 0  # row 0 in every fifth list, never twice
        idx[:, ::5] = sub
    case = W.make_indexed_case(f"{name}_m{mode}", B, M, H, D, N, idx, mode, seed=10, num_splits=splits)
    _log(case.name, check_indexed(case, dev))


LONG_LISTS = [
    # name, B, M, H, D, N, K, pad pattern, splits, sampled rows (None: all): lists longer than one
    # staging chunk (1024 entries in the one-wave-per-task kernel, 256-entry passes in the decode-shape
    # kernel), so that a slice is staged and streamed in several rounds.
    ("long_h96", 1, 4, 96, 128, 3000, 2500, "some", 1, None),        # wave-per-task, 4-tile ring, 3 chunks
    ("long_slice_h64", 1, 3, 64, 128, 3000, 2500, "some", 1, None),  # decode-shape kernel, 10 passes
    ("long_slice_split", 1, 4, 32, 128, 3000, 2500, "oob", 2, None), # two 1250-entry slices + merge
    ("long_many_d64", 2, 2048, 32, 64, 3000, 1100, "some", 1, 48),   # 2-tile ring, 2 chunks, sampled rows
]


@pytest.mark.parametrize("spec", LONG_LISTS, ids=[c[0] for c in LONG_LISTS])
@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_KEY0, W.SINK_NULL])
def test_indexed_long_lists(dev, spec, mode):
    name, B, M, H, D, N, K, pattern, splits, n_rows = spec
    rng = np.random.default_rng(17)
    idx = _edge_lists(rng, B, M, N, K, pattern)
    if mode == W.SINK_KEY0:
        for b in range(B):
            for t in range(0, M, 3):
                if not (idx[b, t] == 0).any():
                    free = np.flatnonzero(idx[b, t] < 0)
                    idx[b, t, free[-1] if free.size else K - 1] = 0  # row 0 late in the list
    case = W.make_indexed_case(f"{name}_m{mode}", B, M, H, D, N, idx, mode, seed=12, num_splits=splits)
    rows = None if n_rows is None else sample_rows(B * M, n_rows, 5, must=(0, B * M - 1))
    _log(case.name, check_indexed(case, dev, rows=rows))


def test_indexed_padding_bit_exact(dev):
    """Appending -1 padding leaves the single-pass result bit-identical."""
    case = W.sparse_prefill_case(q_len=64, total_tokens=2048, n_pick=32, name="pad_inv")
    o0 = run_indexed(case, dev, return_lse=False)
    padded = torch.cat([case.topk_idxs, torch.full((1, 64, 40), -1, dtype=torch.int32)], 2).contiguous()
    o1 = run_indexed(case, dev, idx=padded, return_lse=False)
    assert torch.equal(o0, o1)


def test_sparse_prefill_full_size(dev):
    """8192 queries x 32 heads x 640 listed rows of a 8320-row shared cache (as timed by the bench):
    every element of o and lse."""
    _log("sparse_prefill full", check_indexed_full(W.sparse_prefill_case(), dev))


def test_sparse_decode_full_size(dev):
    """64 decode queries x 64 heads, 2048-entry lists over 32896-row caches, 8 splits + merge (as timed
    by the bench): every element of o and lse."""
    _log("sparse_decode full", check_indexed_full(W.sparse_decode_case(), dev))


def _check_partials(case, dev, num_splits):
    """Each slice's fp32 partial (o_c, lse_c), read from the workspace after the call, against the oracle
    over that slice of the lists alone (no null sink: it enters in the merge), at the bare max-abs 1e-2
    on o_c (no output rounding) and 2e-3 on lse_c."""
    B, M, H, D, N, K = case.dims
    ws = torch.empty(sattn.indexed_workspace_size(B, M, H, D, num_splits), dtype=torch.uint8, device=dev)
    q, kv, idx = case.q.to(dev), case.kv.to(dev), case.topk_idxs.to(dev)
    sinks = case.sinks.to(dev) if case.sinks is not None else None
    o = sattn.indexed_fwd(q, kv, idx, softmax_scale=case.scale, sinks=sinks,
                          sink_mode=("none", "key0", "null")[case.sink_mode], num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize(dev)
    slices = split_slices(K, num_splits)
    po, pl = (t.cpu() for t in workspace_partials(ws, num_splits, B * M, H, D, len(slices)))
    worst = 0.0
    for c, (a, b) in enumerate(slices):
        ro, rl = oracle.indexed(case.q, case.kv, case.topk_idxs[:, :, a:b].contiguous(), scale=case.scale,
                                sinks=case.sinks, sink_mode=W.SINK_KEY0 if case.sink_mode == W.SINK_KEY0 else W.SINK_NONE)
        worst = max(worst, compare(po[c], ro, case.q.dtype, f"{case.name} part_o[{c}]", tol=1e-2))
        compare(pl[c], rl, case.q.dtype, f"{case.name} part_lse[{c}]", lse=True)
    return {"max_abs_part_o": worst, "parts": len(slices), "o": o}


def test_sparse_prefill_split_partials_literal_bar(dev):
    """The prefill workload cut into 4 slices of 160 entries (ragged 32-entry blocks)."""
    r = _check_partials(W.sparse_prefill_case(), dev, 4)
    _log("sparse_prefill partials", {k: v for k, v in r.items() if k != "o"})


def test_sparse_decode_split_partials_literal_bar(dev):
    """The decode workload's own 8 slices of 256 entries."""
    case = W.sparse_decode_case()
    r = _check_partials(case, dev, case.num_splits)
    _log("sparse_decode partials", {k: v for k, v in r.items() if k != "o"})


@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_KEY0, W.SINK_NULL])
@pytest.mark.parametrize("splits", [3, 8])
def test_split_partials_reduced(dev, mode, splits):
    case = W.sparse_decode_case(batch=4, total_tokens=8192, n_pick=480, num_splits=splits, sink_mode=mode,
                                name=f"partials_s{splits}_m{mode}")
    # the decoded position is a multiple of the ring size, so ring slot 0 (cache row 0) is in every list
    assert bool((case.topk_idxs == 0).any(-1).all())
    r = _check_partials(case, dev, splits)
    _log(case.name, {k: v for k, v in r.items() if k != "o"})


# ---------------------------------------------------------------------------
# merge and streams
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_NULL])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_merge_lse_parity(dev, mode, out_dtype):
    g = torch.Generator().manual_seed(12)
    S, R, H, D = 5, 37, 8, 128
    po = torch.randn(S, R, H, D, generator=g)
    pl = torch.randn(S, R, H, generator=g) * 3
    pl[2, :5] = -math.inf
    pl[:, 7, 3] = -math.inf
    sinks = torch.randn(H, generator=g)
    o, lse = sattn.merge_lse(po.to(dev), pl.to(dev), sinks=sinks.to(dev), sink_mode=("none", "key0", "null")[mode],
                             out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.merge(po, pl, sinks=sinks, sink_mode=mode)
    compare(o.cpu(), ro, out_dtype, "merge o")
    compare(lse.cpu(), rl, torch.float32, "merge lse", lse=True)
    if out_dtype == torch.float32:  # no output rounding: the literal bar of bf16-input work as well
        compare(o.cpu(), ro, torch.float32, "merge o (fp32 out)", tol=1e-2)


def test_non_default_stream_with_event(dev):
    """Inputs produced on one stream, the call made on another that waits on an event (no default stream)."""
    case = W.make_window_case("stream", [900, 300], 16, 8, 128, 128, 128, W.SINK_KEY0, seed=8)
    q_host, k_host, v_host = (t.pin_memory() for t in (case.q, case.k, case.v))
    producer, consumer = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(producer):
        q = q_host.to(dev, non_blocking=True)
        k = k_host.to(dev, non_blocking=True)
        v = v_host.to(dev, non_blocking=True)
        cu = case.cu_seqlens.to(dev, non_blocking=True)
        sinks = case.sinks.to(dev, non_blocking=True)
        ready = torch.cuda.Event()
        ready.record(producer)
    consumer.wait_event(ready)
    with torch.cuda.stream(consumer):
        o = sattn.window_fwd(q, k, v, cu, case.max_seqlen, window=(128, 128), sinks=sinks, sink_mode="key0")
    consumer.synchronize()
    ro, _ = oracle_window(case)
    compare(o.cpu(), ro, torch.bfloat16, "stream o")

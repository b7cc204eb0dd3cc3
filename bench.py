"""Benchmark: attended query-key pairs per second of libsattn on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-extra]

One step is one call of the hot path on one batch of synthetic input that is
already resident in HBM.  The headline workload is the vision-encoder window
attention (16 sequences, lengths U[1024, 4096], 16 query / 8 KV heads,
head_dim 128, symmetric window 128, key-0 sinks, bf16).  The other workloads
(causal window with null sinks, top-k prefill over a shared K=V cache, top-k
decode with split-K and merge, the device-side top-k list builder, the
per-block attention mass at the prefill shape, the compressor pooling of the
prefill sequence, the synthetic indexer's top-k selection at the prefill
shape, and the prefill and decode attention over an fp8 cache) are timed the
same way and reported inside the same JSON line under "workloads".

To keep the 256 MB last-level cache (MALL) from serving a step's inputs from
the previous step, every workload rotates between input sets whose union is
larger than the MALL (the indexer's 2 MB of inputs are the exception: its
21 MB of output lists dominate its traffic).

Roofline: algorithmic bytes (each q/k/v/o element once for the window path;
each listed cache row once per query, plus q/o/index lists, for the top-k
path) or algorithmic flops (4 * head_dim per attended pair) per launch,
divided by the kernel time measured with events on the launch stream.
The CPU baseline times the oracle (plain C, fp64, OpenMP) on a bounded sample
of query tokens of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


# The kernel sources each workload's timed launches are built from (the host dispatch in
# sattn_api.cpp and every csrc/ header these include are added; the public header, declarations and
# their documentation, is not): counters taken of a workload stay valid while these files are
# unchanged.
KERNEL_SOURCES = {
    "vision_window": ["window_mfma.hip"],
    "causal_window_null": ["window_mfma.hip"],
    "sparse_prefill": ["indexed_mfma.hip"],
    "sparse_prefill_block_mass": ["indexed_mfma.hip"],
    "sparse_decode": ["indexed_slice.hip", "valu_fwd.hip"],
    "sparse_prefill_fp8": ["indexed_fp8.hip"],
    "sparse_decode_fp8": ["indexed_fp8.hip", "valu_fwd.hip"],
    "topk_idx_build": ["index_build.hip"],
    "compress_pool": ["compress.hip"],
    "indexer_topk": ["indexer.hip"],
}
_CSRC = os.path.join(ROOT, "sliding_window_attention_index_amd", "csrc")


def _with_includes(names):
    """The csrc/ files and, transitively, the csrc/ headers they include."""
    seen, todo = [], list(names)
    while todo:
        n = todo.pop()
        if n in seen:
            continue
        path = os.path.join(_CSRC, n)
        if not os.path.exists(path):
            continue
        seen.append(n)
        with open(path) as f:
            todo += re.findall(r'^\s*#include\s+"([^"]+)"', f.read(), flags=re.M)
    return sorted(seen)


def _code_only(text: str) -> str:
    """The source without its comments and blank space (// and /* */ comments; the kernel sources
    hold no string literal with either marker), so that a comment edit keeps counters valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def _src_hash(workload: str | None = None) -> str:
    """Hash of the kernel sources' code: of every csrc/ file, or of those a workload's launches use."""
    names = sorted(os.listdir(_CSRC)) if workload is None else _with_includes(KERNEL_SOURCES[workload] + ["sattn_api.cpp"])
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(_CSRC, name), encoding="utf-8") as f:
            h.update((name + "\n" + _code_only(f.read())).encode())
    return h.hexdigest()[:16]


def _counters(workload: str):
    """rocprofv3 counter summary of a workload (profiles/counters_<workload>.json), if it was taken of
    the current kernel sources: HBM bytes per launch (FETCH_SIZE and WRITE_SIZE scaled by a plain
    device copy's readings) and the dominant kernel's MfmaUtil, VALUBusy and LdsUtil."""
    path = os.path.join(PROFILES, f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != _src_hash(workload):
        return None
    return rec


class Workload:
    name: str
    bound: str
    unit = "pairs/s"  # attended (query, head, key) pairs; the list builder counts list entries

    def __init__(self, device):
        self.device = device

    def launch(self, i: int):
        raise NotImplementedError


def _window_sets(make, n_sets, device):
    import torch
    sets = []
    for s in range(n_sets):
        c = make(s)
        sets.append(dict(case=c, q=c.q.to(device), k=c.k.to(device), v=c.v.to(device),
                         cu=c.cu_seqlens.to(device), sinks=None if c.sinks is None else c.sinks.to(device),
                         o=torch.empty_like(c.q, device=device)))
    return sets


class WindowWorkload(Workload):
    def __init__(self, device, name, make, n_sets=2):
        super().__init__(device)
        self.name = name
        self.bound = "hbm"
        self.sets = _window_sets(make, n_sets, device)
        c0 = self.sets[0]["case"]
        T, H, Hkv, D = c0.dims
        # identical lengths across sets (same seed for lengths), so pairs and bytes are per-set constants
        self.pairs = c0.pairs()
        self.bytes = T * (2 * H * D + 2 * Hkv * D) * 2
        self.flops = 4 * D * self.pairs
        self.config = dict(workload=name, tokens=T, num_seqs=int(c0.cu_seqlens.numel() - 1), num_heads=H,
                           num_kv_heads=Hkv, head_dim=D, window=[c0.window_left, c0.window_right],
                           sink_mode=["none", "key0", "null"][c0.sink_mode])
        self.case0 = c0

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        s = self.sets[i % len(self.sets)]
        c = s["case"]
        sattn.window_fwd(s["q"], s["k"], s["v"], s["cu"], c.max_seqlen, window=(c.window_left, c.window_right),
                         softmax_scale=c.scale, sinks=s["sinks"], sink_mode=["none", "key0", "null"][c.sink_mode],
                         out=s["o"])


class IndexedWorkload(Workload):
    def __init__(self, device, name, case, idx_sets, q_sets=1, bound="hbm"):
        import torch
        super().__init__(device)
        self.name = name
        self.bound = bound
        self.case0 = case
        self.kv = case.kv.to(device)
        g = torch.Generator().manual_seed(1234)
        self.qs = [case.q.to(device)] + [torch.randn(case.q.shape, generator=g).to(case.q.dtype).to(device)
                                         for _ in range(q_sets - 1)]
        self.idx = [t.to(device) for t in idx_sets]
        self.o = [torch.empty_like(q) for q in self.qs]
        self.sinks = None if case.sinks is None else case.sinks.to(device)
        B, M, H, D, N, K = case.dims
        self.workspace = None
        import sliding_window_attention_index_amd as sattn
        wsb = sattn.indexed_workspace_size(B, M, H, D, case.num_splits)
        if wsb:
            self.workspace = torch.empty(wsb, dtype=torch.uint8, device=device)
        valid = [int(((t >= 0) & (t < N)).sum()) for t in idx_sets]
        self.pairs = valid[0] * H
        self.bytes = valid[0] * D * 2 + 2 * B * M * H * D * 2 + B * M * K * 4
        self.flops = 4 * D * self.pairs
        self.config = dict(workload=name, batch=B, q_len=M, num_heads=H, head_dim=D, kv_len=N, topk=K,
                           num_splits=case.num_splits, sink_mode=["none", "key0", "null"][case.sink_mode],
                           index_sets=len(self.idx))

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        c = self.case0
        j = i % len(self.qs)
        sattn.indexed_fwd(self.qs[j], self.kv, self.idx[i % len(self.idx)], softmax_scale=c.scale, sinks=self.sinks,
                          sink_mode=["none", "key0", "null"][c.sink_mode], num_splits=c.num_splits, out=self.o[j],
                          workspace=self.workspace)


class IndexedFp8Workload(IndexedWorkload):
    """The indexed workloads over an fp8 cache: each row's first 64 dims as e4m3 codes times a
    power-of-two scale, its last 64 (rotary) dims bf16 (196 bytes a row instead of 256)."""

    RD = 64

    def __init__(self, device, name, case, idx_sets, q_sets=1, bound="hbm"):
        import workloads as W
        super().__init__(device, name, case, idx_sets, q_sets=q_sets, bound=bound)
        B, M, H, D, N, K = case.dims
        kv8, sc, rope = W.fp8_cache(5, B, N, D, self.RD, scale_spread=0)
        self.kv = None
        self.kv8, self.sc, self.rope = kv8.to(device), sc.to(device), rope.to(device)
        valid = [int(((t >= 0) & (t < N)).sum()) for t in idx_sets]
        row_bytes = (D - self.RD) + 2 * self.RD + 4
        self.bytes = valid[0] * row_bytes + 2 * B * M * H * D * 2 + B * M * K * 4
        self.config.update(workload=name, kv_format=f"e4m3 dims 0..{D - self.RD - 1} x pow2 scale, bf16 rotary "
                                                     f"dims {D - self.RD}..{D - 1}")

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        c = self.case0
        j = i % len(self.qs)
        sattn.indexed_fp8_fwd(self.qs[j], self.kv8, self.sc, self.rope, self.idx[i % len(self.idx)],
                              softmax_scale=c.scale, sinks=self.sinks, sink_mode=["none", "key0", "null"][c.sink_mode],
                              num_splits=c.num_splits, out=self.o[j], workspace=self.workspace)


class BuildIdxWorkload(Workload):
    """Device-side top-k lists at the prefill shape: 8192 queries at positions 24576.., ring 128,
    ratio 4, 8192 compressed rows -> [1, 8192, 8320] int32 (a pure store stream)."""

    def __init__(self, device, name, start_pos, q_len, window, ratio, n_comp):
        import torch
        super().__init__(device)
        self.name = name
        self.bound = "hbm"
        self.case0 = None
        self.args = dict(window=window, ratio=ratio, n_comp=n_comp)
        self.q_len = q_len
        self.sp = torch.tensor(start_pos, dtype=torch.int32, device=device)
        K = window + n_comp
        self.out = [torch.empty((len(start_pos), q_len, K), dtype=torch.int32, device=device) for _ in range(2)]
        self.bytes = len(start_pos) * q_len * K * 4 + len(start_pos) * 4
        self.pairs = len(start_pos) * q_len * K  # list entries written
        self.flops = 0
        self.unit = "list entries/s"
        self.config = dict(workload=name, batch=len(start_pos), q_len=q_len, window=window, ratio=ratio,
                           n_comp=n_comp, start_pos=int(start_pos[0]))

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        sattn.build_topk_idxs(self.sp, self.q_len, out=self.out[i % 2], **self.args)


class BlockMassWorkload(IndexedWorkload):
    """Per-block attention mass (normalise with the merged lse, sum per block of list entries) at the
    prefill shape: the lse of each input set comes from the attention run once while preparing."""

    def __init__(self, device, name, case, block_keys, q_sets=3):
        import torch

        import sliding_window_attention_index_amd as sattn
        super().__init__(device, name, case, [case.topk_idxs], q_sets=q_sets, bound="mfma")
        self.block_keys = block_keys
        B, M, H, D, N, K = case.dims
        self.lse = [sattn.indexed_fwd(q, self.kv, self.idx[0], softmax_scale=case.scale, return_lse=True)[1]
                    for q in self.qs]
        nb = -(-K // block_keys)
        self.mass = [torch.empty((B, M, H, nb), dtype=torch.float32, device=device) for _ in self.qs]
        torch.cuda.synchronize()
        # q, the lists, the lse and the masses once, plus each listed row once per query
        valid = int(((case.topk_idxs >= 0) & (case.topk_idxs < N)).sum())
        self.bytes = valid * D * 2 + B * M * H * D * 2 + B * M * K * 4 + B * M * H * 4 + B * M * H * nb * 4
        self.flops = 2 * D * self.pairs  # q . k only
        self.config.update(workload=name, block_keys=block_keys, blocks_per_list=nb)

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        j = i % len(self.qs)
        sattn.block_mass(self.qs[j], self.kv, self.idx[0], self.lse[j], block_keys=self.block_keys,
                         softmax_scale=self.case0.scale, out=self.mass[j])


class CompressWorkload(Workload):
    """Compressor pooling of the prefill sequence: 32768 tokens, ratio 4 with overlap, D 128, bf16
    -> 8192 compressed rows.  Eight input sets (268 MB) rotate so that the MALL does not serve a
    launch's inputs from the previous one."""

    def __init__(self, device, name, batch=1, seq_len=32768, head_dim=128, ratio=4, overlap=True, n_sets=8):
        import torch
        super().__init__(device)
        self.name = name
        self.bound = "hbm"
        self.case0 = None
        F = (2 if overlap else 1) * head_dim
        g = torch.Generator().manual_seed(0)
        self.sets = []
        for _ in range(n_sets):
            kv = torch.randn(batch, seq_len, F, generator=g).to(torch.bfloat16).to(device)
            sc = (2.0 * torch.randn(batch, seq_len, F, generator=g)).to(torch.bfloat16).to(device)
            self.sets.append((kv, sc))
        self.ape = (0.5 * torch.randn(ratio, F, generator=g)).to(torch.bfloat16).to(device)
        n_out = seq_len // ratio
        self.out = torch.empty((batch, n_out, head_dim), dtype=torch.bfloat16, device=device)
        self.ratio, self.overlap = ratio, overlap
        self.bytes = 2 * batch * seq_len * F * 2 + ratio * F * 2 + batch * n_out * head_dim * 2
        self.pairs = batch * n_out  # compressed rows written
        self.flops = 0
        self.unit = "compressed rows/s"
        self.config = dict(workload=name, batch=batch, seq_len=seq_len, head_dim=head_dim, ratio=ratio,
                           overlap=overlap, input_sets=n_sets)

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        kv, sc = self.sets[i % len(self.sets)]
        sattn.compress_pool(kv, sc, self.ape, ratio=self.ratio, overlap=self.overlap, out=self.out)


class IndexerWorkload(Workload):
    """Synthetic indexer at the prefill shape: 8192 queries at positions 24576.. (the last 8192 of
    32768 tokens), low-rank query and index keys of rank 64, 8192 compressed rows (ratio 4), window
    128, the top 512 per query -> [1, 8192, 640] int32 lists.  Two input sets alternate."""

    def __init__(self, device, name, start_pos=24576, q_len=8192, n_comp=8192, rank=64, window=128, ratio=4,
                 topk=512, n_sets=2):
        import torch

        import workloads as W
        super().__init__(device)
        self.name = name
        self.case0 = None
        self.sets = []
        for s in range(n_sets):
            qr, kidx = W.indexer_inputs(seed=s, batch=1, q_len=q_len, n_comp=n_comp, rank=rank)
            self.sets.append((qr.to(device), kidx.to(device)))
        self.sp = torch.tensor([start_pos], dtype=torch.int32, device=device)
        K = window + topk
        self.out = [torch.empty((1, q_len, K), dtype=torch.int32, device=device) for _ in range(n_sets)]
        self.args = dict(window=window, ratio=ratio, n_comp=n_comp, topk=topk)
        self.q_len = q_len
        vis = [min(n_comp, (start_pos + t + 1) // ratio) for t in range(q_len)]
        self.pairs = sum(vis)  # (query, visible compressed row) pairs scored
        self.bytes = q_len * rank * 2 + n_comp * rank * 2 + 4 + q_len * K * 4
        self.flops = 2 * rank * self.pairs
        # Bound: every workgroup (32 queries) must bring the index keys of the rows visible to its last
        # query from L2 into its CU at least once (one score pass); the kernel makes two such passes.
        self.bound = "l2"
        self.l2_bytes = sum(vis[min(q_len, t + 32) - 1] for t in range(0, q_len, 32)) * rank * 2
        self.unit = "scored pairs/s"
        self.config = dict(workload=name, batch=1, q_len=q_len, n_comp=n_comp, rank=rank, window=window,
                           ratio=ratio, topk=topk, start_pos=start_pos, input_sets=n_sets)

    def launch(self, i):
        import sliding_window_attention_index_amd as sattn
        j = i % len(self.sets)
        qr, kidx = self.sets[j]
        sattn.indexer_topk(qr, kidx, self.sp, self.q_len, out=self.out[j], **self.args)


def build_workload(name, device):
    import workloads as W
    if name == "vision_window":
        return WindowWorkload(device, name, lambda s: W.vision_window(seed=0) if s == 0 else _reseed_window(
            W.vision_window(seed=0), s))
    if name == "causal_window_null":
        return WindowWorkload(device, name, lambda s: W.causal_window_null(seed=s))
    if name == "sparse_prefill":
        c = W.sparse_prefill_case(seed=0)
        return IndexedWorkload(device, name, c, [c.topk_idxs], q_sets=3, bound="mfma")
    if name == "sparse_decode":
        c = W.sparse_decode_case(seed=0, index_sets=16)
        return IndexedWorkload(device, name, c, c.extra["idx_sets"], q_sets=1, bound="hbm")
    if name == "sparse_prefill_fp8":
        c = W.sparse_prefill_case(seed=0)
        return IndexedFp8Workload(device, name, c, [c.topk_idxs], q_sets=3, bound="mfma")
    if name == "sparse_decode_fp8":
        c = W.sparse_decode_case(seed=0, index_sets=16)
        return IndexedFp8Workload(device, name, c, c.extra["idx_sets"], q_sets=1, bound="hbm")
    if name == "sparse_prefill_block_mass":
        return BlockMassWorkload(device, name, W.sparse_prefill_case(seed=0), 64)
    if name == "compress_pool":
        return CompressWorkload(device, name)
    if name == "indexer_topk":
        return IndexerWorkload(device, name)
    if name == "topk_idx_build":
        return BuildIdxWorkload(device, name, [24576], 8192, 128, 4, 8192)
    raise ValueError(name)


def _reseed_window(case, s):
    """Same lengths (pair count and bytes unchanged), fresh q/k/v values for input set s."""
    import torch
    g = torch.Generator().manual_seed(1000 + s)
    for attr in ("q", "k", "v"):
        t = getattr(case, attr)
        setattr(case, attr, torch.randn(t.shape, generator=g).to(t.dtype))
    return case


def time_workload(wl, steps, warmup):
    """Wall time of exactly `steps` launches (synchronised on both sides) and the mean per-launch
    event time.

    The launches are captured once into a HIP graph of `group` consecutive launches (the largest
    divisor of `steps` up to 16; the input sets rotate as eager calls would rotate them) and the graph
    is replayed steps / group times: a launch of a few microseconds is shorter than the host's own
    per-call overhead, and eager back-to-back calls would time the host.  Events on the replay
    stream bracket every replay; per-launch time = replay time / group.
    """
    import torch
    group = max(g for g in range(1, 17) if steps % g == 0)
    for i in range(warmup):
        wl.launch(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        for i in range(group):
            wl.launch(i)
    torch.cuda.synchronize()
    replays = steps // group
    for _ in range(2):  # warm replays
        graph.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    for i in range(replays):
        evs[i][0].record(stream)
        graph.replay()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = sorted(a.elapsed_time(b) / group for a, b in evs)
    mean_ev = sum(ev_ms) / len(ev_ms)
    return wall, mean_ev, ev_ms[len(ev_ms) // 2], replays * group


L2_PEAK_GBS = 256 * 64 * 2.4  # L2 -> CU: 256 CUs x 64 bytes per clock x 2.4 GHz (39.3 TB/s)


def roofline(wl, kernel_ms):
    """Algorithmic rate of one launch against its bound's peak, beside the counter-based rates of the
    same launch (HBM bytes per launch / time / HBM peak, and the dominant kernel's MFMA, VALU and LDS
    utilisation) when a counter summary of the current kernels is committed under profiles/."""
    sec = kernel_ms / 1e3
    ctr = _counters(wl.name)
    traffic = ctr.get("hbm_bytes_per_launch") if ctr else None
    counter = None
    if ctr:
        counter = {"hbm_gbs": round(traffic / sec / 1e9, 1), "hbm_frac": round(traffic / sec / 1e9 / HBM_PEAK_GBS, 4),
                   "kernel": ctr.get("dominant_kernel"), "mfma_util_pct": ctr.get("mfma_util_pct"),
                   "valu_busy_pct": ctr.get("valu_busy_pct"), "lds_util_pct": ctr.get("lds_util_pct")}
    if wl.bound == "mfma":
        ach = wl.flops / sec / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic, "counter": counter,
                "algorithmic_flops_per_launch": wl.flops}
    if wl.bound == "l2":
        ach = wl.l2_bytes / sec / 1e9
        return {"bound": "l2", "achieved": round(ach, 1), "peak": round(L2_PEAK_GBS, 1), "unit": "GB/s",
                "frac": round(ach / L2_PEAK_GBS, 4), "traffic": traffic, "counter": counter,
                "algorithmic_l2_bytes_per_launch": wl.l2_bytes, "algorithmic_bytes_per_launch": wl.bytes,
                "hbm_frac": round(wl.bytes / sec / 1e9 / HBM_PEAK_GBS, 4)}
    ach = wl.bytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "counter": counter,
            "algorithmic_bytes_per_launch": wl.bytes,
            "mfma_tflops": round(wl.flops / sec / 1e12, 2)}


def cpu_baseline(wl, budget_s=12.0):
    """Oracle (fp64 C, OpenMP on all host cores) on a seeded sample of query tokens of the same workload."""
    import numpy as np

    import oracle
    import workloads as W
    c = wl.case0
    rng = np.random.default_rng(0)
    if isinstance(c, W.WindowCase):
        T = c.q.shape[0]
        cu = c.cu_seqlens.numpy()
        lens = cu[1:] - cu[:-1]
        seq_of = np.repeat(np.arange(len(lens)), lens)

        def pairs_of(rows):
            tot = 0
            for t in rows:
                s = seq_of[t]
                i = t - cu[s]
                L = lens[s]
                lo = 0 if c.window_left < 0 else max(0, i - c.window_left)
                hi = L - 1 if c.window_right < 0 else min(L - 1, i + c.window_right)
                tot += max(0, hi - lo + 1)
            return tot * c.q.shape[1]

        def run(rows):
            oracle.window(c.q, c.k, c.v, c.cu_seqlens, window_left=c.window_left, window_right=c.window_right,
                          scale=c.scale, sinks=c.sinks, sink_mode=c.sink_mode, rows=rows)
        total = T
    else:
        B, M = c.q.shape[:2]
        N = c.kv.shape[1]
        idx = c.topk_idxs.numpy().reshape(B * M, -1)

        def pairs_of(rows):
            return int(((idx[rows] >= 0) & (idx[rows] < N)).sum()) * c.q.shape[2]

        def run(rows):
            oracle.indexed(c.q, c.kv, c.topk_idxs, scale=c.scale, sinks=c.sinks, sink_mode=c.sink_mode, rows=rows)
        total = B * M
    probe = np.sort(rng.choice(total, size=min(total, 64), replace=False))
    t0 = time.perf_counter()
    run(probe)
    dt = max(time.perf_counter() - t0, 1e-4)
    n = int(min(total, max(64, 64 * budget_s / dt)))
    rows = np.sort(rng.choice(total, size=n, replace=False))
    # repeat the sample until about budget_s of CPU time has been measured
    reps, dt = 0, 0.0
    while dt < budget_s and reps < 100:
        t0 = time.perf_counter()
        run(rows)
        dt += time.perf_counter() - t0
        reps += 1
    p = pairs_of(rows) * reps
    n_desc = f"all {total}" if n == total else f"{n} of {total}"
    return {"value": round(p / dt, 1), "unit": "pairs/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"{n_desc} query tokens (all heads) of {wl.name}, seeded, x{reps} passes; {p} pairs in {dt:.2f} s",
            "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="vision_window",
                    choices=["vision_window", "causal_window_null", "sparse_prefill", "sparse_decode",
                             "topk_idx_build", "sparse_prefill_block_mass", "compress_pool", "indexer_topk",
                             "sparse_prefill_fp8", "sparse_decode_fp8"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); the path shards "
              "without exchange by sequence, query or batch row, so N GPUs run N independent copies.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return
    import sliding_window_attention_index_amd as sattn
    sattn.load_library()

    names = [args.workload]
    if not args.no_extra:
        names += [n for n in ("vision_window", "causal_window_null", "sparse_prefill", "sparse_decode",
                              "topk_idx_build", "sparse_prefill_block_mass", "compress_pool", "indexer_topk",
                             "sparse_prefill_fp8", "sparse_decode_fp8") if n != args.workload]
    results = {}
    main_wl = None
    for name in names:
        print(f"[bench] preparing {name}", file=sys.stderr, flush=True)
        wl = build_workload(name, dev)
        steps = args.steps
        wall, mean_ev, med_ev, launched = time_workload(wl, steps, args.warmup)
        ms = wall / steps * 1e3
        rec = {"value": round(wl.pairs / (ms / 1e3), 1), "unit": wl.unit, "ms_per_step": round(ms, 5),
               "kernel_ms_mean": round(mean_ev, 5), "kernel_ms_median": round(med_ev, 5), "pairs": wl.pairs,
               "config": wl.config, "roofline": roofline(wl, mean_ev)}
        print(f"[bench] {name}: {json.dumps(rec)}", file=sys.stderr, flush=True)
        results[name] = rec
        if name == args.workload:
            main_wl = wl
        else:
            del wl
            torch.cuda.empty_cache()

    head = results[args.workload]
    line = {
        "metric": "attended q-k pairs/sec",
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "cpu_baseline": None if args.no_cpu else cpu_baseline(main_wl),
        "workloads": {k: v for k, v in results.items() if k != args.workload},
        "kernel_source_sha": _src_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

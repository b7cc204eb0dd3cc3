"""SATTN_TRACE=1: the library prints one line per kernel launch (variant, grid, the sizes that chose it).

The CPU test runs in a child process on a machine without a GPU: the arguments pass validation, the
launcher prints its line, and the launch itself then fails (SATTN_ERR_LAUNCH), so no pointer is ever
used.  The GPU test makes real calls in a child process and checks that the decode shape takes the
per-(query, slice) kernel followed by the merge.
"""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CPU_CHILD = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import sliding_window_attention_index_amd as s
from sliding_window_attention_index_amd import _WindowArgs, _IndexedArgs
lib = s.load_library()
F = 0x10000  # never dereferenced: without a GPU every launch fails
w = _WindowArgs(0, F, F, F, F, None, F, 16, 40000, 4096, 16, 8, 128, 128, 128, 0.088, F, 1)
print("window", lib.sattn_window_fwd(ctypes.byref(w), None), flush=True)
i = _IndexedArgs(0, F, F, F, F, None, 1, 8192, 32, 128, 8320, 640, 0.088, None, 0, 1, None, 0)
print("prefill", lib.sattn_indexed_fwd(ctypes.byref(i), None), flush=True)
'''


def _child(code, env_extra, args=()):
    env = dict(os.environ, **env_extra)
    return subprocess.run([sys.executable, "-c", code, ROOT, *args], capture_output=True, text=True, env=env,
                          timeout=120)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake pointers are only safe where no GPU can run them")
def test_trace_lines_without_gpu():
    r = _child(CPU_CHILD, {"SATTN_TRACE": "1"})
    assert "window 7" in r.stdout and "prefill 7" in r.stdout, r.stdout + r.stderr  # SATTN_ERR_LAUNCH
    lines = [l for l in r.stderr.splitlines() if l.startswith("[sattn] ")]
    assert any(l.startswith("[sattn] window_fwd_mfma<D=128, G=2> grid=") and "window=(128, 128) sink_mode=1" in l
               for l in lines), lines
    assert any(l.startswith("[sattn] indexed_fwd_mfma<D=128, NT=2, mass=0> grid=2048 ") and "tasks=8192" in l
               for l in lines), lines


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="fake pointers are only safe where no GPU can run them")
def test_trace_off_by_default():
    r = _child(CPU_CHILD, {"SATTN_TRACE": "0"})
    assert "window 7" in r.stdout, r.stdout + r.stderr
    assert "[sattn]" not in r.stderr


GPU_CHILD = r'''
import sys
sys.path.insert(0, sys.argv[1])
import torch
import sliding_window_attention_index_amd as s
import workloads as W
c = W.sparse_decode_case(batch=4, total_tokens=8192, n_pick=480, num_splits=8)
s.indexed_fwd(c.q.cuda(), c.kv.cuda(), c.topk_idxs.cuda(), num_splits=8)
torch.cuda.synchronize()
print("done", flush=True)
'''


@pytest.mark.gpu
def test_trace_decode_kernels():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    r = _child(GPU_CHILD, {"SATTN_TRACE": "1"})
    assert "done" in r.stdout, r.stdout + r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("[sattn] ")]
    assert len(lines) == 2, lines
    assert lines[0].startswith("[sattn] indexed_slice_mfma<D=128, head groups=2> grid=32 ") and "slices=8" in lines[0]
    assert lines[1].startswith("[sattn] merge4_kernel<bf16> ") and "parts=8" in lines[1]

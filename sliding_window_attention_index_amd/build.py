"""Build libsattn.so (HIP, gfx950) in-tree with hipcc.

    python -m sliding_window_attention_index_amd.build [-v]

Objects go to _build/ at the repository root; the shared library lands next
to this file so that the Python binding (and a copy of the tree sent to a GPU
machine) finds it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["sattn_api.cpp", "sattn_noalloc.hip", "valu_fwd.hip", "indexed_mfma.hip", "indexed_slice.hip", "indexed_fp8.hip", "window_mfma.hip", "index_build.hip",
           "compress.hip", "indexer.hip"]
HEADERS = ["sattn_device.hpp", "sattn_kernels.hpp", "softmax_block.hpp", "lds_tile.hpp"]
# MFMA kernels keep their accumulators in VGPRs: the online-softmax rescale is a VALU
# multiply, which cannot read AGPRs and would otherwise copy the accumulator every block.
EXTRA_FLAGS = {
    "indexed_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "indexed_slice.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "indexed_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "window_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

# Kernels that count their own outstanding LDS-DMA requests (fixed s_waitcnt vmcnt values) must
# not spill: a compiler-inserted scratch access is one more vector-memory operation in flight and
# would make those waits return early.  The build reads the compiler's resource report for these
# sources and fails on any scratch use.
NO_SCRATCH = {"indexed_mfma.hip", "indexed_slice.hip", "indexed_fp8.hip", "window_mfma.hip", "indexer.hip"}
_USAGE = "kernel-resource-usage"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # Packed FP32 instructions (v_pk_{add,mul,fma}_f32) stay off: ordinary float code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def scratch_users(report_lines) -> list[str]:
    """Kernels of a `-Rpass-analysis=kernel-resource-usage` report that use scratch memory or spill
    VGPRs (SGPR spills go to VGPR lanes and are not counted)."""
    fn, bad = "?", []
    for l in report_lines:
        if "Function Name:" in l:
            fn = l.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in l or "VGPRs Spill:" in l:
            if int(l.split(":")[-1].split("[")[0]) != 0:
                bad.append(f"{fn}: {l.split('remark:')[1].split('[-R')[0].strip()}")
    return bad


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += EXTRA_FLAGS.get(src, [])
    if src in NO_SCRATCH:
        cmd += [f"-Rpass-analysis={_USAGE}"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
    err = "\n".join(l for l in lines if _USAGE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if src in NO_SCRATCH:
        bad = scratch_users(lines)
        if bad:
            raise RuntimeError(f"{src}: kernels that count their own memory requests use scratch:\n" + "\n".join(bad))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel source for gfx950 and link libsattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

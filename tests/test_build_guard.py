"""The build's scratch guard: kernels that count their own outstanding DMA requests must not use
scratch memory (a compiler-inserted scratch access would make their fixed vmcnt waits return
early).  Checks the parser of the compiler's resource report on sample remark lines."""
from sliding_window_attention_index_amd.build import scratch_users

_R = "x.hip:56:1: remark: "
_T = " [-Rpass-analysis=kernel-resource-usage]"


def _report(name, scratch, vspill, sspill):
    return [f"{_R}Function Name: {name}{_T}", f"{_R}    VGPRs: 168{_T}", f"{_R}    ScratchSize [bytes/lane]: {scratch}{_T}",
            f"{_R}    SGPRs Spill: {sspill}{_T}", f"{_R}    VGPRs Spill: {vspill}{_T}"]


def test_clean_kernels_pass():
    assert scratch_users(_report("k0", 0, 0, 0) + _report("k1", 0, 0, 12)) == []  # SGPR spills live in VGPR lanes


def test_scratch_and_vgpr_spills_are_reported_per_kernel():
    bad = scratch_users(_report("k0", 0, 0, 0) + _report("k1", 88, 21, 0) + _report("k2", 0, 3, 0))
    assert bad == ["k1: ScratchSize [bytes/lane]: 88", "k1: VGPRs Spill: 21", "k2: VGPRs Spill: 3"]

"""C ABI checks that need no GPU: the library loads, exports what include/sattn.h declares,
and host-side validation rejects bad arguments before anything touches the device.

Every call here fails validation (or is a pure host query), so the HIP runtime
is never asked to launch anything.
"""
import ctypes
import os
import re

import pytest

import sliding_window_attention_index_amd as sattn
from sliding_window_attention_index_amd import (_BlockMassArgs, _BuildIdxArgs, _CompressArgs, _IndexedArgs,
                                                 _IndexedFp8Args, _IndexerArgs, _MergeArgs, _WindowArgs)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sattn.h")

OK, NULL_PTR, SHAPE, DTYPE, UNSUPPORTED, ALIGNMENT, WORKSPACE, LAUNCH, ARG, SCRATCH_LIMIT = range(10)


@pytest.fixture(scope="module")
def lib():
    path = sattn.library_path()
    if not os.path.exists(path):
        from sliding_window_attention_index_amd.build import build
        build()
    return sattn.load_library(path)


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sattn_status|size_t|const char \*|int)\s*(sattn_\w+)\s*\(", text, re.M)))


def test_header_functions_exported(lib):
    names = _declared_functions()
    assert set(names) == {"sattn_window_fwd", "sattn_indexed_fwd", "sattn_indexed_fwd_noalloc", "sattn_merge_lse",
                          "sattn_build_topk_idxs",
                          "sattn_block_mass", "sattn_compress_pool", "sattn_indexer_topk", "sattn_indexed_fp8_fwd",
                          "sattn_indexed_workspace_size", "sattn_status_string", "sattn_abi_version"}
    for name in names:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    m = re.search(r"#define SATTN_ABI_VERSION (\d+)", open(HEADER).read())
    assert lib.sattn_abi_version() == int(m.group(1))
    seen = set()
    for s in range(10):
        txt = lib.sattn_status_string(s).decode()
        assert txt and txt != "unknown status"
        seen.add(txt)
    assert len(seen) == 10
    assert lib.sattn_status_string(99).decode() == "unknown status"


def test_workspace_size(lib):
    ws = lib.sattn_indexed_workspace_size
    assert ws(64, 1, 64, 128, 1) == 0
    # part_o [8,64,64,128] fp32 and part_lse [8,64,64] fp32, each rounded up to 256 bytes
    assert ws(64, 1, 64, 128, 8) == 8 * 64 * 64 * 128 * 4 + 8 * 64 * 64 * 4
    assert ws(3, 5, 7, 8, 3) == ((3 * 15 * 7 * 8 * 4 + 255) // 256 * 256) + ((3 * 15 * 7 * 4 + 255) // 256 * 256)
    assert ws(0, 5, 7, 8, 3) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def _window(**kw):
    base = dict(dtype=0, q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, cu_seqlens=FAKE, num_seqs=2, total_tokens=42,
                max_seqlen=37, num_heads=4, num_kv_heads=2, head_dim=64, window_left=8, window_right=8,
                softmax_scale=0.125, sinks=FAKE, sink_mode=1)
    base.update(kw)
    return _WindowArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), DTYPE),
    (dict(sink_mode=5), ARG),
    (dict(num_heads=4, num_kv_heads=3), SHAPE),
    (dict(num_heads=0), SHAPE),
    (dict(head_dim=12), UNSUPPORTED),
    (dict(head_dim=264), UNSUPPORTED),
    (dict(head_dim=0), SHAPE),
    (dict(softmax_scale=float("nan")), ARG),
    (dict(max_seqlen=0), SHAPE),
    (dict(q=None), NULL_PTR),
    (dict(cu_seqlens=None), NULL_PTR),
    (dict(sinks=None), NULL_PTR),
    (dict(o=FAKE + 8), ALIGNMENT),
    (dict(k=FAKE + 2), ALIGNMENT),
])
def test_window_validation(lib, kw, status):
    assert lib.sattn_window_fwd(ctypes.byref(_window(**kw)), None) == status


def test_window_null_args(lib):
    assert lib.sattn_window_fwd(None, None) == NULL_PTR


def test_window_empty_batch_is_noop(lib):
    # zero tokens: valid and nothing to do, so nothing is launched
    assert lib.sattn_window_fwd(ctypes.byref(_window(total_tokens=0, q=None)), None) == OK


def _indexed(**kw):
    base = dict(dtype=0, q=FAKE, kv=FAKE, topk_idxs=FAKE, o=FAKE, lse=None, batch=1, q_len=4, num_heads=32,
                head_dim=128, kv_len=100, topk=64, softmax_scale=0.1, sinks=None, sink_mode=0, num_splits=1,
                workspace=None, workspace_bytes=0)
    base.update(kw)
    return _IndexedArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), DTYPE),
    (dict(sink_mode=2, sinks=None), NULL_PTR),
    (dict(num_splits=0), ARG),
    (dict(num_splits=65), ARG),
    (dict(topk=-1), SHAPE),
    (dict(kv_len=-5), SHAPE),
    (dict(head_dim=100), UNSUPPORTED),
    (dict(q=None), NULL_PTR),
    (dict(topk_idxs=None), NULL_PTR),
    (dict(kv=FAKE + 4), ALIGNMENT),
    (dict(num_splits=4), WORKSPACE),
    (dict(num_splits=4, workspace=FAKE, workspace_bytes=16), WORKSPACE),
    (dict(num_splits=4, workspace=FAKE + 16, workspace_bytes=1 << 30), WORKSPACE),
])
def test_indexed_validation(lib, kw, status):
    assert lib.sattn_indexed_fwd(ctypes.byref(_indexed(**kw)), None) == status


def test_indexed_empty_is_noop(lib):
    assert lib.sattn_indexed_fwd(ctypes.byref(_indexed(q_len=0, q=None)), None) == OK


def _merge(**kw):
    base = dict(part_o=FAKE, part_lse=FAKE, num_parts=8, rows=64, num_heads=64, head_dim=128, sinks=None,
                sink_mode=0, out_dtype=0, o=FAKE, lse=None)
    base.update(kw)
    return _MergeArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(sink_mode=1, sinks=FAKE), ARG),
    (dict(sink_mode=2, sinks=None), NULL_PTR),
    (dict(out_dtype=3), DTYPE),
    (dict(num_parts=-1), SHAPE),
    (dict(part_o=None), NULL_PTR),
    (dict(o=FAKE + 4), ALIGNMENT),
])
def test_merge_validation(lib, kw, status):
    assert lib.sattn_merge_lse(ctypes.byref(_merge(**kw)), None) == status


def _build(**kw):
    base = dict(out=FAKE, start_pos=FAKE, batch=64, q_len=1, window=128, ratio=4, n_comp=32768)
    base.update(kw)
    return _BuildIdxArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(window=0), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(q_len=-2), SHAPE),
    (dict(n_comp=-1), SHAPE),
    (dict(ratio=-4), ARG),
    (dict(ratio=0), ARG),                      # compressed rows without a ratio
    (dict(window=2**31 - 10, n_comp=100), SHAPE),
    (dict(out=None), NULL_PTR),
    (dict(start_pos=None), NULL_PTR),
    (dict(out=FAKE + 2), ALIGNMENT),
    (dict(start_pos=FAKE + 1), ALIGNMENT),
])
def test_build_topk_idxs_validation(lib, kw, status):
    assert lib.sattn_build_topk_idxs(ctypes.byref(_build(**kw)), None) == status


def test_build_topk_idxs_empty_is_noop(lib):
    assert lib.sattn_build_topk_idxs(ctypes.byref(_build(batch=0, out=None, start_pos=None)), None) == OK
    assert lib.sattn_build_topk_idxs(ctypes.byref(_build(q_len=0, out=None)), None) == OK
    assert lib.sattn_build_topk_idxs(None, None) == NULL_PTR


def _mass(**kw):
    base = dict(dtype=0, q=FAKE, kv=FAKE, topk_idxs=FAKE, lse=FAKE, mass=FAKE, batch=1, q_len=8192, num_heads=32,
                head_dim=128, kv_len=8320, topk=640, block_keys=64, softmax_scale=0.088, sinks=None, sink_mode=0)
    base.update(kw)
    return _BlockMassArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), DTYPE),
    (dict(sink_mode=3), ARG),
    (dict(block_keys=0), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(num_heads=0), SHAPE),
    (dict(head_dim=100), UNSUPPORTED),
    (dict(softmax_scale=float("nan")), ARG),
    (dict(lse=None), NULL_PTR),
    (dict(mass=None), NULL_PTR),
    (dict(topk_idxs=None), NULL_PTR),
    (dict(sink_mode=1, sinks=None), NULL_PTR),
    (dict(q=FAKE + 8), ALIGNMENT),
    (dict(mass=FAKE + 2), ALIGNMENT),
    (dict(lse=FAKE + 1), ALIGNMENT),
])
def test_block_mass_validation(lib, kw, status):
    assert lib.sattn_block_mass(ctypes.byref(_mass(**kw)), None) == status


def test_block_mass_empty_is_noop(lib):
    assert lib.sattn_block_mass(ctypes.byref(_mass(batch=0, q=None, mass=None)), None) == OK
    assert lib.sattn_block_mass(ctypes.byref(_mass(topk=0, mass=None)), None) == OK
    assert lib.sattn_block_mass(None, None) == NULL_PTR


def _comp(**kw):
    base = dict(dtype=0, kv=FAKE, score=FAKE, ape=FAKE, out=FAKE, out_batch_stride=8192, batch=1, seq_len=32768,
                head_dim=128, ratio=4, overlap=1)
    base.update(kw)
    return _CompressArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), DTYPE),
    (dict(overlap=2), ARG),
    (dict(ratio=0), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(seq_len=-4), SHAPE),
    (dict(head_dim=0), SHAPE),
    (dict(head_dim=12), UNSUPPORTED),
    (dict(out_batch_stride=8191), SHAPE),
    (dict(kv=None), NULL_PTR),
    (dict(ape=None), NULL_PTR),
    (dict(out=FAKE + 4), ALIGNMENT),
    (dict(score=FAKE + 8), ALIGNMENT),
])
def test_compress_pool_validation(lib, kw, status):
    assert lib.sattn_compress_pool(ctypes.byref(_comp(**kw)), None) == status


def test_compress_pool_empty_is_noop(lib):
    assert lib.sattn_compress_pool(ctypes.byref(_comp(batch=0, kv=None)), None) == OK
    assert lib.sattn_compress_pool(ctypes.byref(_comp(seq_len=3, out=None, out_batch_stride=0)), None) == OK
    assert lib.sattn_compress_pool(None, None) == NULL_PTR


def _ixr(**kw):
    base = dict(out=FAKE, qr=FAKE, kidx=FAKE, start_pos=FAKE, batch=1, q_len=8192, rank=64, window=128, ratio=4,
                n_comp=8192, topk=512)
    base.update(kw)
    return _IndexerArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(window=0), SHAPE),
    (dict(topk=-1), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(ratio=-1), ARG),
    (dict(ratio=0), ARG),
    (dict(rank=48), UNSUPPORTED),
    (dict(rank=256), UNSUPPORTED),
    (dict(batch=65536), UNSUPPORTED),
    (dict(n_comp=1 << 24, rank=64), UNSUPPORTED),
    (dict(out=None), NULL_PTR),
    (dict(kidx=None), NULL_PTR),
    (dict(start_pos=None), NULL_PTR),
    (dict(qr=FAKE + 4), ALIGNMENT),
    (dict(out=FAKE + 2), ALIGNMENT),
])
def test_indexer_topk_validation(lib, kw, status):
    assert lib.sattn_indexer_topk(ctypes.byref(_ixr(**kw)), None) == status


def test_indexer_topk_empty_is_noop(lib):
    assert lib.sattn_indexer_topk(ctypes.byref(_ixr(batch=0, out=None)), None) == OK
    assert lib.sattn_indexer_topk(ctypes.byref(_ixr(q_len=0, qr=None)), None) == OK
    assert lib.sattn_indexer_topk(None, None) == NULL_PTR


def _f8(**kw):
    base = dict(q=FAKE, kv_fp8=FAKE, kv_scale=FAKE, kv_rope=FAKE, topk_idxs=FAKE, o=FAKE, lse=None, batch=1, q_len=8192,
                num_heads=32, head_dim=128, rope_dims=64, kv_len=8320, topk=640, softmax_scale=0.088, sinks=None,
                sink_mode=0, num_splits=1, workspace=None, workspace_bytes=0)
    base.update(kw)
    return _IndexedFp8Args(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), UNSUPPORTED),
    (dict(rope_dims=32), UNSUPPORTED),
    (dict(num_heads=48), UNSUPPORTED),
    (dict(softmax_scale=-1.0), UNSUPPORTED),
    (dict(rope_dims=129), SHAPE),
    (dict(batch=-1), SHAPE),
    (dict(sink_mode=7), ARG),
    (dict(num_splits=0), ARG),
    (dict(kv_scale=None), NULL_PTR),
    (dict(kv_rope=None), NULL_PTR),
    (dict(sink_mode=2), NULL_PTR),
    (dict(kv_fp8=FAKE + 8), ALIGNMENT),
    (dict(kv_scale=FAKE + 2), ALIGNMENT),
    (dict(num_splits=8), WORKSPACE),
])
def test_indexed_fp8_validation(lib, kw, status):
    assert lib.sattn_indexed_fp8_fwd(ctypes.byref(_f8(**kw)), None) == status


def test_indexed_fp8_empty_is_noop(lib):
    assert lib.sattn_indexed_fp8_fwd(ctypes.byref(_f8(batch=0, q=None)), None) == OK
    assert lib.sattn_indexed_fp8_fwd(None, None) == NULL_PTR


def test_indexed_noalloc_scratch_limit(lib):
    """Split-K partials beyond SATTN_NOALLOC_SCRATCH_BYTES are refused before the device is touched."""
    m = re.search(r"#define SATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    fake = 1 << 20  # never dereferenced: the call returns before any launch
    B, M, H, D, S = 64, 1, 64, 128, 8
    assert lib.sattn_indexed_workspace_size(B, M, H, D, S) <= limit
    big = 2 * B  # twice the rows: twice the partials
    assert lib.sattn_indexed_workspace_size(big, M, H, D, S) > limit
    a = _IndexedArgs(0, fake, fake, fake, fake, None, big, M, H, D, 4096, 2048, 0.088, None, 0, S, None, 0)
    assert lib.sattn_indexed_fwd_noalloc(ctypes.byref(a), None) == SCRATCH_LIMIT
    assert lib.sattn_indexed_fwd_noalloc(None, None) == NULL_PTR

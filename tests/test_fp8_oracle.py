"""Pins of the fp8 cache oracle (oracle/fp8_cache.py) against facts other than itself.

* e4m3 decoding equals torch's float8_e4m3fn conversion for every code, and the format's named
  values (OCP fn variant): largest 448, smallest normal 2^-6, smallest subnormal 2^-9, -0, NaN.
* Rows of bf16 values that are exact e4m3 values, written as codes with scale 1, dequantise to
  the same rows; a power-of-two scale multiplies them exactly.
* Attention over an fp8 cache equals the bf16 attention oracle over a cache holding the same
  values (the fp8 dims first, the rotary dims last), with and without rotary dims and sinks.
* Planted mistakes (exponent bias 8, subnormals as normals, scale left out, scale on the rotary
  dims, rotary dims first) each fail.
"""
from __future__ import annotations

import inspect
import textwrap

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import fp8_cache as F8


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = F8.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def test_named_values():
    d = F8.e4m3_decode([0x7E, 0x08, 0x01, 0x80, 0x7F, 0xFF, 0x38, 0xC0])
    assert d[0] == 448.0 and d[1] == 2.0 ** -6 and d[2] == 2.0 ** -9
    assert d[3] == 0.0 and np.signbit(d[3])
    assert np.isnan(d[4]) and np.isnan(d[5])
    assert d[6] == 1.0 and d[7] == -2.0


def _exact_e4m3_cache(seed, B, N, D, rd):
    """A bf16 cache whose first D - rd dims are exact e4m3 values, and the same cache as fp8."""
    g = torch.Generator().manual_seed(seed)
    codes = torch.randint(0, 256, (B, N, D - rd), generator=g, dtype=torch.int64)
    codes = torch.where((codes & 0x7F) == 0x7F, torch.zeros_like(codes), codes).to(torch.uint8)  # no NaN
    vals = codes.view(torch.float8_e4m3fn).float()
    rope = torch.randn(B, N, rd, generator=g).to(torch.bfloat16)
    kv = torch.cat([vals.to(torch.bfloat16), rope], dim=-1)
    assert torch.equal(kv[..., :D - rd].float(), vals)  # e4m3 values are exact in bf16
    return kv, codes, rope


@pytest.mark.parametrize("rd", [0, 64])
def test_exact_values_dequantise_to_themselves(rd):
    kv, codes, rope = _exact_e4m3_cache(1, 2, 40, 128, rd)
    rows = F8.dequant_rows(codes, torch.ones(2, 40), rope)
    assert np.array_equal(rows, kv.float().numpy())
    sc = torch.exp2(torch.randint(-5, 6, (2, 40)).float())
    rows2 = F8.dequant_rows(codes, sc, rope)
    assert np.array_equal(rows2[..., :128 - rd], (kv[..., :128 - rd].float() * sc[..., None]).numpy())
    assert np.array_equal(rows2[..., 128 - rd:], kv[..., 128 - rd:].float().numpy())


@pytest.mark.parametrize("rd,sink_mode", [(0, oracle.SINK_NONE), (64, oracle.SINK_NONE), (64, oracle.SINK_NULL),
                                          (0, oracle.SINK_KEY0)])
def test_attention_equals_bf16_oracle_on_the_same_values(rd, sink_mode):
    B, M, H, D, N, K = 2, 3, 4, 128, 50, 12
    kv, codes, rope = _exact_e4m3_cache(2, B, N, D, rd)
    sc = torch.exp2(torch.randint(-3, 4, (B, N)).float())
    kv_scaled = torch.cat([(kv[..., :D - rd].float() * sc[..., None]), kv[..., D - rd:].float()], -1)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(B, M, H, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(B * M)]).view(B, M, K).to(torch.int32)
    idx[0, 0, -2:] = -1
    sinks = torch.randn(H, generator=g)
    s = 1.0 / np.sqrt(D)
    o_ref, l_ref = oracle.indexed(q, kv_scaled, idx, scale=s, sinks=sinks, sink_mode=sink_mode)
    o, l = F8.indexed_fp8(q, codes, sc, rope, idx, softmax_scale=s, sinks=sinks, sink_mode=sink_mode)
    assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)


def test_generator_rows_fit_the_format():
    kv8, sc, rope = W.fp8_cache(0, 2, 64, 128, 64)
    assert kv8.dtype == torch.uint8 and kv8.shape == (2, 64, 64) and rope.shape == (2, 64, 64)
    assert not np.isnan(F8.e4m3_decode(kv8.numpy())).any()
    m, e = np.frexp(sc.numpy())
    assert np.all(m == 0.5)  # powers of two


MUTANTS = {
    "bias_8": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "subnormals_as_normals": ("v = np.where(e == 0, subnormal, normal)", "v = normal"),
    "scale_left_out": ("rows = e4m3_decode(k8) * sc[..., None]", "rows = e4m3_decode(k8)"),
    "rope_first": ("rows = np.concatenate([rows, rope], axis=-1)", "rows = np.concatenate([rope, rows], axis=-1)"),
    "scale_on_rope": ("rows = np.concatenate([rows, rope], axis=-1)",
                      "rows = np.concatenate([rows, rope * sc[..., None]], axis=-1)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail(name):
    old, new = MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(F8))
    assert old in src
    ns = {"__name__": "oracle.fp8_mutant", "__package__": "oracle"}
    exec(compile(src.replace(old, new), "fp8_mutant", "exec"), ns)
    saved = (F8.e4m3_decode, F8.dequant_rows, F8.indexed_fp8)
    F8.e4m3_decode, F8.dequant_rows, F8.indexed_fp8 = ns["e4m3_decode"], ns["dequant_rows"], ns["indexed_fp8"]
    try:
        with pytest.raises(AssertionError):
            test_decode_matches_torch_for_every_code()
            test_named_values()
            for rd in (0, 64):
                test_exact_values_dequantise_to_themselves(rd)
            test_attention_equals_bf16_oracle_on_the_same_values(64, oracle.SINK_NULL)
    finally:
        F8.e4m3_decode, F8.dequant_rows, F8.indexed_fp8 = saved

"""Pins of the oracle's number formats, quantiser and fp8 pipeline emulation."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_special_values.json")


def _torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def _torch_e4m3_code(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_decode(codes), _torch_e4m3_value(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_golden_ocp_special_values():
    g = json.load(open(GOLDEN))
    for item in g["values"]:
        code = int(item["code"], 16)
        assert oracle.e4m3_decode(np.array([code]))[0] == item["value"], item
        assert oracle.e4m3_encode(np.array([item["value"]]))[0] == code, item
    for c in g["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(np.array([int(c, 16)]))[0])
    assert oracle.E4M3_MAX == 448.0


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
    assert oracle.e4m3_encode(np.array([np.nan]))[0] == 0x7F
    assert oracle.e4m3_encode(np.array([-np.nan]))[0] == 0xFF


def test_encode_matches_torch_cast_including_ties():
    rng = np.random.default_rng(0)
    vals = oracle.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties, representable in fp32
    rand = rng.uniform(-1, 1, 200000) * np.exp2(rng.integers(-14, 9, 200000))
    x = np.concatenate([vals, mids, -mids, rand]).astype(np.float32)
    x = np.clip(x, -448, 448)
    assert np.array_equal(oracle.e4m3_encode(x.astype(np.float64)), _torch_e4m3_code(x))


def test_encode_saturates():
    got = oracle.e4m3_encode(np.array([448.0, 449.0, 470.0, 1e9, np.inf, -500.0, -np.inf]))
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


def test_bf16_round_matches_torch_cast_including_ties():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, 300000, dtype=np.uint64).astype(np.uint32)
    bits[:100000] = (bits[:100000] & 0xFFFF0000) | 0x8000    # exact ties
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    x = x[np.abs(x) < 3.0e38]                                 # keep clear of overflow to inf
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).double().numpy()
    assert np.array_equal(oracle.bf16_round(x.astype(np.float64)), ref)


# ------------------------------------------------------------------ quantiser
def test_quantizer_maps_absmax_to_448_and_matches_torch():
    rng = np.random.default_rng(2)
    for std in (1.0, 1e-3, 37.0):
        x = torch.from_numpy(rng.standard_normal(50000).astype(np.float32) * std).to(torch.bfloat16)
        codes, descale, s = oracle.quantize_per_tensor(x)
        x32 = x.float().numpy()
        assert s == np.float32(448.0) / np.float32(np.abs(x32).max())
        assert descale == np.float32(1.0) / s
        assert np.max(codes & 0x7F) == 0x7E
        y = np.clip(np.multiply(x32, s, dtype=np.float32), -448, 448)
        assert np.array_equal(codes, _torch_e4m3_code(y))
        back = oracle.e4m3_decode(codes) * np.float64(descale)
        normal = np.abs(y) >= 2.0**-6
        rel = np.abs(back[normal] - x32[normal]) / np.abs(x32[normal])
        assert rel.max() <= 2.0**-4 * (1 + 1e-6)


def test_quantizer_zero_tensor():
    codes, descale, s = oracle.quantize_per_tensor(np.zeros(10, dtype=np.float32))
    assert s == 1.0 and descale == 1.0 and not codes.any()


# ------------------------------------------------------------------ fp8 pipeline
def _fp8_inputs(B, H, N, d, seed):
    g = torch.Generator().manual_seed(seed)
    qkv = [torch.randn((B, H, N, d), generator=g).to(torch.bfloat16) for _ in range(3)]
    return [oracle.quantize_per_tensor(t) for t in qkv]


def test_fp8_pipeline_without_p_rounding_is_plain_attention():
    (q8, dq, _), (k8, dk, _), (v8, dv, _) = _fp8_inputs(1, 2, 96, 32, 5)
    scale = 1 / math.sqrt(32)
    o, lse = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale, round_p=False)
    deq = [oracle.e4m3_decode(c) * np.float64(s) for c, s in ((q8, dq), (k8, dk), (v8, dv))]
    o_ref, lse_ref = oracle.attention(*deq, scale)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12) and np.allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_fp8_pipeline_p_rounding_within_e4m3_bound():
    (q8, dq, _), (k8, dk, _), (v8, dv, _) = _fp8_inputs(1, 2, 200, 64, 6)
    scale = 1 / math.sqrt(64)
    o, _ = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale)
    o0, _ = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale, round_p=False)
    deq = [oracle.e4m3_decode(c) * np.float64(s) for c, s in ((q8, dq), (k8, dk), (v8, dv))]
    _, _, a = oracle.attention(*deq, scale, want_abs=True)
    # normal range: relative error <= 2^-4; subnormal range: absolute <= 2^-10 in units of p*256
    vmax = np.abs(deq[2]).max()
    bound = 2.0**-4 * a + 200 * (2.0**-10 / oracle.P_SCALE) * vmax
    assert (np.abs(o - o0) <= bound).all()
    assert np.abs(o - o0).max() > 0          # the rounding is really applied


def test_fp8_pipeline_rounded_denominator():
    """den_rounded divides by the sum of the rounded P8: a constant V comes back
    exactly (a convex combination), and each row differs from the default
    reading by one factor, the ratio of the two sums, within the e4m3 bound."""
    (q8, dq, _), (k8, dk, _), (v8, dv, _) = _fp8_inputs(1, 2, 150, 32, 8)
    scale = 1 / math.sqrt(32)
    o_r, lse_r = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale, den_rounded=True)
    o_e, lse_e = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale)
    assert np.array_equal(lse_r, lse_e)                  # the log-sum-exp stays the exact one
    big = np.abs(o_e) > 1e-3
    ratio = np.where(big, o_r / np.where(big, o_e, 1.0), np.nan)
    row_ratio = np.nanmedian(ratio, axis=3, keepdims=True)
    assert np.allclose(np.where(big, ratio, row_ratio), row_ratio, rtol=1e-9, atol=0)
    assert np.abs(row_ratio - 1).max() <= 2.0**-4 and np.abs(row_ratio - 1).max() > 0
    c8 = np.full_like(v8, 0x3C)                          # e4m3 1.5
    o_c, _ = oracle.attention_fp8_pipeline(q8, k8, c8, dq, dk, dv, scale, den_rounded=True)
    assert np.allclose(o_c, 1.5 * np.float64(dv), rtol=1e-15, atol=0)
    o_c0, _ = oracle.attention_fp8_pipeline(q8, k8, c8, dq, dk, dv, scale)
    assert np.abs(o_c0 - 1.5 * np.float64(dv)).max() > 1e-6


def test_fp8_pipeline_closed_forms():
    (q8, dq, _), (k8, dk, _), (v8, dv, _) = _fp8_inputs(1, 1, 64, 16, 7)
    k8 = np.broadcast_to(k8[:, :, :1], k8.shape).copy()          # identical keys: p = 1 exactly
    o, _ = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, 0.25)
    v = oracle.e4m3_decode(v8) * np.float64(dv)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=0, atol=1e-15)
    o1, _ = oracle.attention_fp8_pipeline(q8[:, :, :1], k8[:, :, :1], v8[:, :, :1], dq, dk, dv, 0.25)
    assert np.array_equal(o1, v[:, :, :1])

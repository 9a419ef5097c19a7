"""Pins of the block-scaled (MX) e4m3 oracle: the quantiser and the pipeline
emulation, each against things other than themselves. Planted mistakes in
copies of the quantiser must each fail a pin."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import e4m3_decode, e4m3_encode
from workloads import random_qkv


def _x(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _blocks_d(x):
    B, H, N, d = x.shape
    return x.reshape(B, H, N, d // 32, 32)


# ------------------------------------------------------------------ quantiser pins
def pin_torch_cast(q):
    """Each code is torch's float8_e4m3fn cast of the value over its block's power of two."""
    for shape, seed, std in [((1, 2, 37, 64), 1, 1.0), ((2, 1, 65, 128), 2, 1e-3), ((1, 1, 33, 32), 3, 300.0)]:
        x = _x(shape, seed, std)
        codes, scales = q(x, "d")
        e = scales.astype(np.int64) - 127
        y = np.ldexp(x.double().numpy(), -np.repeat(e, 32, axis=-1))
        if np.abs(y).max() > 448:
            return False
        ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if not np.array_equal(codes, ref):
            return False
        codes_t, scales_t = q(x, "tokens")
        N = shape[2]
        nt = -(-N // 32)
        e_t = scales_t.astype(np.int64) - 127                       # (B, H, nt, 32, d/32)
        e_cols = np.swapaxes(e_t, -1, -2).reshape(shape[0], shape[1], nt, shape[3])
        y_t = np.ldexp(x.double().numpy(), -np.repeat(e_cols, 32, axis=2)[:, :, :N])
        if np.abs(y_t).max() > 448:
            return False
        ref_t = torch.from_numpy(y_t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if not np.array_equal(codes_t, ref_t):
            return False
    return True


def pin_block_max_in_range(q):
    """Smallest exponent: each block's largest value lands in (224, 448] (e4m3
    codes 0x6F..0x7E, or at 224 itself when the next exponent would pass 448)."""
    x = _x((1, 2, 200, 128), 4)
    codes, scales = q(x, "d")
    vals = np.abs(e4m3_decode(codes))
    bmax = _blocks_d(torch.from_numpy(vals)).numpy().max(-1)
    return bool(((bmax >= 224) & (bmax <= 448)).all())


def pin_error_bound(q):
    """With y = x / 2^e (e the element's block exponent, read from the returned
    scales in their documented layout): |x - deq| <= 2^e half an e4m3 step at
    y, i.e. 2^e max(2^(floor(log2 |y|) - 4), 2^-10) (2^-10: half the
    subnormal step)."""
    x = _x((1, 2, 100, 128), 5)
    xf = x.double().numpy()
    B, H, N, d = xf.shape
    for along in ("d", "tokens"):
        codes, scales = q(x, along)
        e = scales.astype(np.int64) - 127
        if along == "d":
            e_el = np.repeat(e, 32, axis=-1)
        else:
            nt = -(-N // 32)
            e_el = np.repeat(np.swapaxes(e, -1, -2).reshape(B, H, nt, d), 32, axis=2)[:, :, :N]
        deq = np.ldexp(e4m3_decode(codes), e_el)
        y = np.abs(np.ldexp(xf, -e_el))
        half = np.maximum(np.ldexp(1.0, np.floor(np.log2(np.maximum(y, 1e-300))).astype(np.int64) - 4), 2.0**-10)
        if not (np.abs(xf - deq) <= np.ldexp(half, e_el)).all():
            return False
    return True


def pin_power_of_two_invariance(q):
    """x 2^k: the same codes, every scale byte + k."""
    x = _x((1, 1, 64, 64), 6)
    for along in ("d", "tokens"):
        c0, s0 = q(x, along)
        c1, s1 = q((x.double() * 2.0**5).to(torch.bfloat16), along)
        if not (np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 5)):
            return False
    return True


def pin_exact_blocks(q):
    """Blocks of e4m3 values times 2^s whose maximum is exactly 448 come back exactly, scale 2^s."""
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 0x7E, size=(1, 1, 4, 64)).astype(np.uint8)
    codes[..., 0] = 0x7E                                     # 448 in every block of 32 along d
    codes[..., 32] = 0x7E
    vals = e4m3_decode(codes)
    s = np.array([-3, 0, 2, -10]).reshape(1, 1, 4, 1)
    x = torch.from_numpy(np.ldexp(vals, s))
    c, sc = q(x, "d")
    return np.array_equal(c, codes) and np.array_equal(sc.astype(int) - 127, np.broadcast_to(s, (1, 1, 4, 2)))


def pin_zero_blocks(q):
    x = torch.zeros((1, 1, 40, 64), dtype=torch.bfloat16)
    for along in ("d", "tokens"):
        c, s = q(x, along)
        if c.any() or not (s == 0).all():
            return False
    return True


def pin_token_layout(q):
    """Column c of V holding 300 * 2^(c mod 16 - 8) (and -300 * that at one token):
    its block scale is 2^(c mod 16 - 8) (300 <= 448 < 600); entry (t, i, j)
    belongs to column 32 j + i."""
    N, d = 70, 128
    c = np.arange(d)
    col = 300.0 * np.ldexp(1.0, (c % 16) - 8)
    x = np.broadcast_to(col, (1, 1, N, d)).copy()
    x[0, 0, 5] = -x[0, 0, 5]
    _, s = q(torch.from_numpy(x).to(torch.bfloat16), "tokens")
    want_e = (c % 16) - 8
    for t in range(3):
        for i in range(32):
            for j in range(4):
                if int(s[0, 0, t, i, j]) - 127 != want_e[32 * j + i]:
                    return False
    return True


QPINS = [pin_torch_cast, pin_block_max_in_range, pin_error_bound, pin_power_of_two_invariance, pin_exact_blocks,
         pin_zero_blocks, pin_token_layout]


@pytest.mark.parametrize("pin", QPINS, ids=lambda p: p.__name__)
def test_mx_quantizer_passes_pin(pin):
    assert pin(oracle.mx_quantize)


def _mutant(kind):
    def q(x, along):
        x = x.double().numpy() if hasattr(x, "double") else np.asarray(x, dtype=np.float64)
        B, H, N, d = x.shape
        if kind == "blocks_along_wrong_axis":
            along = "tokens" if along == "d" else "d"
        def quant(xb):
            amax = np.abs(xb).max(-1)
            f, ex = np.frexp(amax)
            if kind == "ocp_floor_saturating":
                e = np.where(amax > 0, ex - 9, -127)
            elif kind == "emax_7":
                e = np.where(amax > 0, ex - 8 + (f > 0.875), -127)
            elif kind == "round_not_floor":
                e = np.where(amax > 0, np.round(np.log2(np.maximum(amax, 1e-300) / 448)), -127).astype(np.int64)
            else:
                e = np.where(amax > 0, ex - 9 + (f > 0.875), -127)
            e = np.maximum(e, -127)
            return e4m3_encode(np.ldexp(xb, -e[..., None])), e
        if along == "d":
            c, e = quant(x.reshape(B, H, N, d // 32, 32))
            return c.reshape(B, H, N, d), (e + 127).astype(np.uint8)
        nt = -(-N // 32)
        xp = np.zeros((B, H, nt * 32, d))
        xp[:, :, :N] = x
        c, e = quant(np.swapaxes(xp.reshape(B, H, nt, 32, d), -1, -2))
        c = np.swapaxes(c, -1, -2).reshape(B, H, nt * 32, d)[:, :, :N]
        if kind == "token_layout_transposed":
            sc = e.reshape(B, H, nt, 32, d // 32) + 127          # (t, c // 4, c % 4): wrong order
        else:
            sc = np.swapaxes(e.reshape(B, H, nt, d // 32, 32), -1, -2) + 127
        return c, sc.astype(np.uint8)
    return q


QMUTANTS = ["blocks_along_wrong_axis", "ocp_floor_saturating", "emax_7", "round_not_floor", "token_layout_transposed"]


def _passes(pin, q):
    """A pin that raises (say, on a scale array of the wrong shape) has caught the mistake."""
    try:
        return bool(pin(q))
    except (ValueError, IndexError):
        return False


@pytest.mark.parametrize("kind", QMUTANTS)
def test_planted_quantizer_mistake_is_caught(kind):
    with np.errstate(all="ignore"):
        failed = [p.__name__ for p in QPINS if not _passes(p, _mutant(kind))]
    assert failed, f"mutant {kind} passed every pin"


def test_unmutated_quantizer_copy_passes():
    assert all(p(_mutant("none")) for p in QPINS)


def test_dequantize_inverts_layouts():
    x = _x((2, 1, 45, 64), 8)
    for along in ("d", "tokens"):
        c, s = oracle.mx_quantize(x, along)
        deq = oracle.mx_dequantize(c, s, along)
        # requantising the dequantised values returns the same values (a block
        # whose maximum rounded down to 224 2^e may come back as 448 2^(e-1))
        c2, s2 = oracle.mx_quantize(torch.from_numpy(deq), along)
        assert np.array_equal(oracle.mx_dequantize(c2, s2, along), deq)


# ------------------------------------------------------------------ pipeline pins
def _mx_inputs(B, H, N, d, seed):
    q, k, v = random_qkv(B, H, N, d, seed=seed)
    (q8, qs), (k8, ks) = oracle.mx_quantize(q, "d"), oracle.mx_quantize(k, "d")
    v8, vs = oracle.mx_quantize(v, "tokens")
    return q8, qs, k8, ks, v8, vs


def test_pipeline_without_p_rounding_is_attention_on_dequantised_inputs():
    q8, qs, k8, ks, v8, vs = _mx_inputs(1, 2, 100, 64, 9)
    o, lse = oracle.attention_mx_pipeline(q8, qs, k8, ks, v8, vs, 0.125, round_p=False)
    qd, kd = oracle.mx_dequantize(q8, qs, "d"), oracle.mx_dequantize(k8, ks, "d")
    vd = oracle.mx_dequantize(v8, vs, "tokens")
    o_ref, lse_ref = oracle.attention(qd, kd, vd, 0.125)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-13) and np.allclose(lse, lse_ref, rtol=0, atol=1e-13)


def test_unit_scales_equal_the_per_tensor_pipeline():
    rng = np.random.default_rng(10)
    q8, k8, v8 = (rng.integers(0, 0x7E, size=(1, 2, 70, 64)).astype(np.uint8) | rng.choice([0, 0x80], (1, 2, 70, 64)).astype(np.uint8)
                  for _ in range(3))
    ones_d = np.full((1, 2, 70, 2), 127, dtype=np.uint8)
    ones_t = np.full((1, 2, 3, 32, 2), 127, dtype=np.uint8)
    for den_rounded in (True, False):
        o, lse = oracle.attention_mx_pipeline(q8, ones_d, k8, ones_d, v8, ones_t, 0.05, den_rounded=den_rounded)
        o2, lse2 = oracle.attention_fp8_pipeline(q8, k8, v8, 1.0, 1.0, 1.0, 0.05, den_rounded=den_rounded)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_v_scales_scale_the_output():
    q8, qs, k8, ks, v8, vs = _mx_inputs(1, 1, 64, 64, 11)
    o, lse = oracle.attention_mx_pipeline(q8, qs, k8, ks, v8, vs, 0.125)
    o2, lse2 = oracle.attention_mx_pipeline(q8, qs, k8, ks, v8, (vs.astype(int) + 1).astype(np.uint8), 0.125)
    assert np.array_equal(o2, 2 * o) and np.array_equal(lse, lse2)


def test_q_scale_trades_with_the_logit_multiplier():
    q8, qs, k8, ks, v8, vs = _mx_inputs(1, 1, 80, 64, 12)
    o, lse = oracle.attention_mx_pipeline(q8, qs, k8, ks, v8, vs, 0.125)
    o2, lse2 = oracle.attention_mx_pipeline(q8, (qs.astype(int) + 3).astype(np.uint8), k8, ks, v8, vs, 0.125 / 8)
    assert np.allclose(o2, o, rtol=0, atol=1e-15) and np.allclose(lse2, lse, rtol=0, atol=1e-13)

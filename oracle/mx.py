"""fp64 oracle of block-scaled e4m3 inputs (OCP MX "MXFP8" style) and of the
attention pipeline on them (TEST INFRASTRUCTURE).

The pages report fp8 attention variants that trade image fidelity for speed
(Japanese summary, third and fourth paragraphs) and do not describe their
scaling. Per-tensor scales are one reading (oracle.formats); this module is
a second, finer one: every 32 consecutive elements along one axis share one
power-of-two scale, the element format is e4m3. It is this library's own
choice, made to cut the fp8 input error, not a method from the pages.

Quantisation of one block of 32 values x_i:
* amax = max |x_i|; the shared exponent e is the smallest integer with
  amax / 2^e <= 448 (e4m3's largest value), at least -127; an all-zero
  block takes e = -127. Reading: the OCP Microscaling specification's MXFP8
  conversion takes e = floor(log2 amax) - 8 and saturates elements above
  448, which clips a block maximum whose significand exceeds 1.75 by up to
  1/8; the exponent here is that one plus 1 exactly for those blocks, so
  nothing saturates;
* the scale is stored as its E8M0 byte e + 127 (value 2^e);
* each element is x_i / 2^e (exact: a power-of-two scaling) rounded to
  e4m3, nearest-even.

Blocks run along d for Q and K (each row has d/32 blocks) and along the
tokens for V (each column has ceil(N/32) blocks, the last one short), so
that every block lies inside one 32-wide slice of the contraction each
product runs over. Scale layouts (uint8):
* along d: [B][H][N][d/32], block j of row n covers d = 32 j .. 32 j + 31;
* along tokens: [B][H][ceil(N/32)][32][d/32]; entry (t, i, j) is the scale
  of column c = 32 j + i over tokens 32 t .. 32 t + 31.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64
from .formats import e4m3_decode, e4m3_encode
from .fp8_attention import P_SCALE, pipeline_on_values

E8M0_BIAS = 127
E4M3_EMAX = 8          # exponent of the largest power of two below e4m3's maximum (2^8 = 256)
BLOCK = 32


def shared_exponent(amax) -> np.ndarray:
    """Smallest e with amax / 2^e <= 448, at least -127; amax = 0 gives -127.

    With amax = f 2^x, f in [0.5, 1): amax / 2^(x - 9) = 512 f lies in
    [256, 512), and it is at most 448 exactly when f <= 7/8."""
    amax = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(amax)
    e = np.where(amax > 0, x - 1 - E4M3_EMAX + (f > 0.875), -E8M0_BIAS)
    return np.maximum(e, -E8M0_BIAS).astype(np.int64)


def _quantize_blocks(xb):
    """xb: (..., nblk, 32) float64 (zero-padded). Returns codes (same shape), exponents (..., nblk)."""
    e = shared_exponent(np.abs(xb).max(axis=-1))
    y = np.ldexp(xb, -e[..., None])             # exact: a power-of-two scaling
    return e4m3_encode(y), e


def mx_quantize(x, along: str):
    """Block-scaled e4m3 codes of a (B, H, N, d) tensor; ``along`` is "d" or "tokens".

    Returns (codes uint8 (B, H, N, d), scales uint8 in the layout above)."""
    x = _f64(x)
    B, H, N, d = x.shape
    assert d % BLOCK == 0
    if along == "d":
        codes, e = _quantize_blocks(x.reshape(B, H, N, d // BLOCK, BLOCK))
        return codes.reshape(B, H, N, d), (e + E8M0_BIAS).astype(np.uint8)
    assert along == "tokens"
    nt = -(-N // BLOCK)
    xp = np.zeros((B, H, nt * BLOCK, d))
    xp[:, :, :N] = x
    # (B, H, nt, 32 tokens, d) -> blocks per column: (B, H, nt, d, 32)
    xb = np.swapaxes(xp.reshape(B, H, nt, BLOCK, d), -1, -2)
    codes, e = _quantize_blocks(xb)                 # e: (B, H, nt, d)
    codes = np.swapaxes(codes, -1, -2).reshape(B, H, nt * BLOCK, d)[:, :, :N]
    # column c = 32 j + i -> entry (i, j)
    scales = np.swapaxes(e.reshape(B, H, nt, d // BLOCK, BLOCK), -1, -2) + E8M0_BIAS
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales).astype(np.uint8)


def mx_dequantize(codes, scales, along: str) -> np.ndarray:
    """float64 values of block-scaled codes (inverse of the layouts of ``mx_quantize``)."""
    codes = np.asarray(codes.cpu() if hasattr(codes, "cpu") else codes).view(np.uint8)
    scales = np.asarray(scales.cpu() if hasattr(scales, "cpu") else scales).view(np.uint8)
    vals = e4m3_decode(codes)
    B, H, N, d = vals.shape
    e = scales.astype(np.int64) - E8M0_BIAS
    if along == "d":
        return np.ldexp(vals, np.repeat(e, BLOCK, axis=-1))
    nt = -(-N // BLOCK)
    e_cols = np.swapaxes(e, -1, -2).reshape(B, H, nt, d)          # (t, c) with c = 32 j + i
    return np.ldexp(vals, np.repeat(e_cols, BLOCK, axis=2)[:, :, :N])


def attention_mx_pipeline(q8, q_scales, k8, k_scales, v8, v_scales, scale, rows=None, block=512,
                          p_scale=P_SCALE, round_p=True, den_rounded=True):
    """(O, lse) of the fp8 pipeline on block-scaled inputs, float64.

    Q and K are scaled along d, V along the tokens. The logits are the exact
    dot products of the dequantised rows; P is rounded to e4m3 after scaling
    by ``p_scale`` relative to the row maximum; O is divided by the sum of
    the rounded P (``den_rounded``, default, as the kernel does) or by the
    exact sum times ``p_scale``. The log-sum-exp is the exact one."""
    q = mx_dequantize(q8, q_scales, "d")
    k = mx_dequantize(k8, k_scales, "d")
    v = mx_dequantize(v8, v_scales, "tokens")
    return pipeline_on_values(q, k, v, 1.0, scale, rows=rows, block=block, p_scale=p_scale, round_p=round_p,
                              den_rounded=den_rounded)

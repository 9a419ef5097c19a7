"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle on the same seeded inputs.

Gates for bf16 output (every compared element, float64 arithmetic):
* spec: max |O_gpu - O| <= 2e-2 and mean |O_gpu - O| <= 2e-3.
* derived bound: |O_gpu - O| <= 2^-8 (A + |O|)(1 + 2^-6) + 2^-12 A + 1e-6,
  with A = sum_j p_ij |V_jc|. bf16 carries 8 significant bits, so rounding
  each probability to bf16 moves the weighted sum by at most 2^-8 A, and
  rounding the output moves it by at most 2^-8 |O|; fp32 accumulation and
  the fp32 exponential add far less than the 2^-12 A slack. The row sum is
  taken from the unrounded probabilities, so it adds no bf16 term.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

SPEC_MAX, SPEC_MEAN = 2e-2, 2e-3
SPEC_MAX_FP8 = 6e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_attention(q, k, v, scale, want_lse=False):
    """q, k, v: CPU tensors (bf16 or float8_e4m3fn). Returns (O float64 numpy, lse or None)."""
    import diffusion_transformer_attention_non_amd as dit
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, H, N, d = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if want_lse else None
    o = dit.attention(qd, kd, vd, scale, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), (lse.cpu().double().numpy() if want_lse else None)


def bf16_bound(o_ref, a_ref):
    return 2.0**-8 * (a_ref + np.abs(o_ref)) * (1 + 2.0**-6) + 2.0**-12 * a_ref + 1e-6


def check_bf16(o_gpu, o_ref, a_ref, label=""):
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    bound = bf16_bound(o_ref, a_ref)
    worst = float((err / bound).max())
    say(f"  {label}: max {mx:.3e} mean {mean:.3e} worst err/bound {worst:.3f}")
    assert np.isfinite(o_gpu).all(), label
    assert mx <= SPEC_MAX and mean <= SPEC_MEAN, (label, mx, mean)
    assert (err <= bound).all(), (label, worst, np.unravel_index(np.argmax(err / bound), err.shape))
    return mx, mean


def rows_of(o, rows):
    return o[:, :, rows, :]

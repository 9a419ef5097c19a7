"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle on the same seeded inputs.

Gates for bf16 output (every compared element, float64 arithmetic):
* spec: max |O_gpu - O| <= 2e-2 and mean |O_gpu - O| <= 2e-3.
* derived bound: |O_gpu - O| <= 2^-8 (A + 2|O|)(1 + 2^-6) + 2^-12 A + 1e-6,
  with A = sum_j p_ij |V_jc| and u = 2^-8 the unit roundoff of bf16 (8
  significant bits). Each probability is rounded to bf16, p~_j = p_j (1 + e_j)
  with |e_j| <= u, and the row is normalised by the sum of the rounded
  values (the weights the MFMAs multiply), so the weights become
  p_j (e_j - e) / (1 + e) away from p_j, e = sum_j p_j e_j: at most
  u (A + |O|) / (1 - u) on the output. Rounding the output adds u |O|. fp32
  accumulation and the fp32 exponential add far less than the 2^-12 A slack.
  (A kernel that normalises by unrounded probabilities meets the tighter
  u (A + |O|) form, which this bound contains.)
* log-sum-exp: the same normalisation moves it by |log(1 + e)| <= -log(1 - u),
  so |lse_gpu - lse| <= 2^-8 (1 + 2^-6) + 2e-5 + 2e-6 |lse|.
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
    return 2.0**-8 * (a_ref + 2 * np.abs(o_ref)) * (1 + 2.0**-6) + 2.0**-12 * a_ref + 1e-6


LSE_ATOL = 2.0**-8 * (1 + 2.0**-6) + 2e-5
LSE_RTOL = 2e-6


def check_lse(l_gpu, l_ref, label=""):
    err = np.abs(l_gpu - l_ref)
    say(f"  {label} lse: max {float(err.max()):.3e}")
    assert np.isfinite(l_gpu).all(), label
    assert (err <= LSE_ATOL + LSE_RTOL * np.abs(l_ref)).all(), (label, float(err.max()))


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

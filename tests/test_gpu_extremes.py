"""GPU parity at the size extremes: a single head far longer than any
workload (N = 99 999, ragged against every tile size), thousands of tiny
heads, and a long fp8 head; sampled rows against the oracle with LSE."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (check_fp8_against_emulation, check_full, fp8_bound, gpu_attention, lse_tolerance, oracle_ref,
                    say)
from workloads import random_qkv, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_very_long_single_head(d):
    B, H, N = 1, 1, 99999
    q, k, v = random_qkv(B, H, N, d, seed=1100 + d)
    say(f"[gpu] long head N={N} d={d}")
    o, l = gpu_attention(q, k, v, 1 / math.sqrt(d), want_lse=True)
    rows = sample_rows(N, seed=3, n_edge=300, stride=400)
    check_full(o[:, :, rows], l[:, :, rows], q, k, 1 / math.sqrt(d),
               oracle_ref(q, k, v, 1 / math.sqrt(d), rows=rows), f"N={N} d={d}", rows=rows)


@pytest.mark.parametrize("B,H,N,d", [(64, 48, 17, 128), (32, 40, 130, 64), (8, 96, 300, 128)])
def test_many_small_heads(B, H, N, d):
    q, k, v = random_qkv(B, H, N, d, seed=1200 + N)
    say(f"[gpu] many heads B={B} H={H} N={N} d={d}")
    o, l = gpu_attention(q, k, v, 1 / math.sqrt(d), want_lse=True)
    check_full(o, l, q, k, 1 / math.sqrt(d), oracle_ref(q, k, v, 1 / math.sqrt(d)),
               f"B={B} H={H} N={N} d={d}")


def test_long_fp8_head_against_emulation():
    import diffusion_transformer_attention_non_amd as dit
    B, H, N, d = 1, 2, 40001, 128
    scale = 1 / math.sqrt(d)
    q, k, v = random_qkv(B, H, N, d, seed=1300)
    say(f"[gpu] long fp8 head N={N}")
    dev = torch.device("cuda:0")
    quant = [dit.quantize_e4m3(t.to(dev)) for t in (q, k, v)]
    descale = torch.cat([ds for _, ds in quant]).contiguous()
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o = dit.attention(*(c for c, _ in quant), scale, descale=descale, lse=lse)
    torch.cuda.synchronize()
    rows = sample_rows(N, seed=4, n_edge=256, stride=500)
    og = o.float().cpu().double().numpy()[:, :, rows]
    codes = [c.view(torch.uint8).cpu().numpy() for c, _ in quant]
    ds = [float(x) for x in descale.cpu()]
    o_emul, lse_emul = oracle.attention_fp8_pipeline(codes[0], codes[1], codes[2], ds[0], ds[1], ds[2], scale,
                                                     rows=rows, den_rounded=True)
    qd, kd, vd = (oracle.e4m3_decode(c) * np.float64(x) for c, x in zip(codes, ds))
    bound, var, det = fp8_bound(qd, kd, vd, scale, o_emul, rows=rows)
    check_fp8_against_emulation(og, o_emul, bound, var, det, f"fp8 N={N}")
    mag = scale * np.linalg.norm(qd[:, :, rows], axis=-1) * np.linalg.norm(kd, axis=-1).max(axis=-1, keepdims=True)
    tol = lse_tolerance(N, lse_emul, mag, logit_rel=2.0**-11)
    d_lse = np.abs(lse.cpu().double().numpy()[:, :, rows] - lse_emul)
    say(f"  fp8 N={N}: lse max |d| {d_lse.max():.3e} (worst d/tol {(d_lse / tol).max():.3f})")
    assert (d_lse <= tol).all()

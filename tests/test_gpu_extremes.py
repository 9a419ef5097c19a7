"""GPU parity at the size extremes: a single head far longer than any
workload (N = 99 999, ragged against every tile size), thousands of tiny
heads, and a long fp8 head; sampled rows against the oracle with LSE."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import check_bf16, check_lse, gpu_attention, say
from workloads import random_qkv, sample_rows

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [64, 128])
def test_very_long_single_head(d):
    B, H, N = 1, 1, 99999
    q, k, v = random_qkv(B, H, N, d, seed=1100 + d)
    say(f"[gpu] long head N={N} d={d}")
    o, l = gpu_attention(q, k, v, 1 / math.sqrt(d), want_lse=True)
    rows = sample_rows(N, seed=3, n_edge=300, stride=400)
    o_ref, l_ref, a_ref = oracle.attention(q, k, v, 1 / math.sqrt(d), rows=rows, want_abs=True)
    check_bf16(o[:, :, rows], o_ref, a_ref, f"N={N} d={d}")
    check_lse(l[:, :, rows], l_ref, f"N={N} d={d}")


@pytest.mark.parametrize("B,H,N,d", [(64, 48, 17, 128), (32, 40, 130, 64), (8, 96, 300, 128)])
def test_many_small_heads(B, H, N, d):
    q, k, v = random_qkv(B, H, N, d, seed=1200 + N)
    say(f"[gpu] many heads B={B} H={H} N={N} d={d}")
    o, l = gpu_attention(q, k, v, 1 / math.sqrt(d), want_lse=True)
    o_ref, l_ref, a_ref = oracle.attention(q, k, v, 1 / math.sqrt(d), want_abs=True)
    check_bf16(o, o_ref, a_ref, f"B={B} H={H} N={N} d={d}")
    check_lse(l, l_ref, f"B={B} H={H} N={N} d={d}")


def test_long_fp8_head_against_emulation():
    import diffusion_transformer_attention_non_amd as dit
    B, H, N, d = 1, 2, 40001, 128
    q, k, v = random_qkv(B, H, N, d, seed=1300)
    say(f"[gpu] long fp8 head N={N}")
    dev = torch.device("cuda:0")
    quant = [dit.quantize_e4m3(t.to(dev)) for t in (q, k, v)]
    descale = torch.cat([ds for _, ds in quant]).contiguous()
    o = dit.attention(*(c for c, _ in quant), 1 / math.sqrt(d), descale=descale)
    torch.cuda.synchronize()
    rows = sample_rows(N, seed=4, n_edge=256, stride=500)
    og = o.float().cpu().double().numpy()[:, :, rows]
    codes = [c.view(torch.uint8).cpu().numpy() for c, _ in quant]
    ds = [float(x) for x in descale.cpu()]
    o_emul, _ = oracle.attention_fp8_pipeline(codes[0], codes[1], codes[2], ds[0], ds[1], ds[2], 1 / math.sqrt(d),
                                              rows=rows, den_rounded=True)
    o_ref, _ = oracle.attention(q, k, v, 1 / math.sqrt(d), rows=rows)
    err, err_e = np.abs(og - o_ref), np.abs(o_emul - o_ref)
    say(f"  fp8 N={N}: gpu max {err.max():.3e} mean {err.mean():.3e} | emulation max {err_e.max():.3e} "
        f"mean {err_e.mean():.3e}")
    assert np.isfinite(og).all()
    assert err.mean() <= 1.25 * err_e.mean() + 1e-5 and err.max() <= 2.0 * err_e.max() + 1e-5

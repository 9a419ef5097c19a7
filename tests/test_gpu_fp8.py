"""GPU parity of the fp8-e4m3 path: the on-device quantiser bit for bit against
the oracle's quantiser, and the fp8 attention against the fp64 oracle.

Gates for the fp8 attention (bf16 output):
* spec: max |O_gpu - O| <= 6e-2 against the exact oracle on the unquantised
  bf16 inputs, at the 16896-token workload it is stated for.
* calibrated: the fp64 emulation of the fp8 pipeline (same e4m3 inputs, P
  rounded to e4m3 after scaling by 2^8, O divided by the sum of the rounded
  P, as the kernel does) has error e_emul against the same exact oracle. The
  kernel rounds P relative to its running maximum rather than the final row
  maximum, so its P rounding noise is statistically alike but not identical;
  the input quantisation, which dominates, is bit-identical.
  Gate: mean error <= 1.25 e_emul(mean) + 1e-5 and max error <= 2 e_emul(max).
* the log-sum-exp is the exact one (sums of the unrounded p), against the
  emulation's to 1e-4 + 1e-5|lse| plus the logit error of the e4m3 MFMA's
  inexact internal sums (see _check_fp8).
* O does not depend on whether the log-sum-exp is requested (two kernel
  forms): bitwise equal at the full workload.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import SPEC_MAX_FP8, gpu_attention, say
from workloads import WORKLOADS, coverage_pattern, make_qkv, random_qkv, sample_rows

pytestmark = pytest.mark.gpu


def _gpu_quantize(x):
    import diffusion_transformer_attention_non_amd as dit
    codes, descale = dit.quantize_e4m3(x.to("cuda"))
    torch.cuda.synchronize()
    return codes, descale


def _check_quantizer(x, label):
    codes, descale = _gpu_quantize(x)
    ref_codes, ref_descale, _ = oracle.quantize_per_tensor(x)
    got = codes.view(torch.uint8).cpu().numpy().reshape(-1)
    assert descale.item() == float(ref_descale), (label, descale.item(), ref_descale)
    ref = ref_codes.reshape(-1)
    assert np.array_equal(got, ref), (label, int((got != ref).sum()))
    return codes, descale


def test_quantizer_bit_exact_small_and_edge_values():
    g = torch.Generator().manual_seed(0)
    for n, std in [(8, 1.0), (64, 1e-3), (4096, 30.0), (100000, 1.0)]:
        x = (torch.randn(n, generator=g) * std).to(torch.bfloat16)
        _check_quantizer(x, f"n={n} std={std}")
    x = torch.zeros(64, dtype=torch.bfloat16)
    codes, descale = _gpu_quantize(x)
    assert descale.item() == 1.0 and not codes.view(torch.uint8).any()
    # values straddling e4m3 rounding ties after scaling
    vals = oracle.e4m3_decode(np.arange(0, 0x7E, dtype=np.uint8))
    mids = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2, [448.0]])
    x = torch.from_numpy(np.concatenate([mids, -mids, np.zeros(8 - (2 * mids.size) % 8)])).to(torch.bfloat16)
    _check_quantizer(x, "ties")


def test_quantizer_bit_exact_full_workload():
    w = WORKLOADS["t2i_2048_fp8"]
    for t, name in zip(make_qkv(w), "qkv"):
        say(f"[gpu] quantise {name} {tuple(t.shape)}")
        _check_quantizer(t.reshape(-1), f"{name} full")


def _fp8_inputs_gpu(q, k, v):
    qs = [_gpu_quantize(t.reshape(-1)) for t in (q, k, v)]
    codes = [c.view(q.shape) for c, _ in qs]
    descale = torch.cat([d for _, d in qs]).contiguous()
    return codes, descale


def _run_fp8(q, k, v, scale, want_lse=True):
    import diffusion_transformer_attention_non_amd as dit
    (q8, k8, v8), descale = _fp8_inputs_gpu(q, k, v)
    B, H, N, d = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda") if want_lse else None
    o = dit.attention(q8, k8, v8, scale, descale=descale, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), (lse.cpu().double().numpy() if want_lse else None)


def _check_fp8(q, k, v, scale, label, rows=None, spec_gate=False):
    say(f"[gpu] fp8 {label}: shape {tuple(q.shape)}")
    o, lse = _run_fp8(q, k, v, scale)
    if rows is None:
        rows = np.arange(q.shape[2])
    o = o[:, :, rows]
    o_ref, _ = oracle.attention(q, k, v, scale, rows=rows)
    (q8, dq, _), (k8, dk, _), (v8, dv, _) = (oracle.quantize_per_tensor(t) for t in (q, k, v))
    o_emul, lse_emul = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale, rows=rows, den_rounded=True)
    err = np.abs(o - o_ref)
    err_e = np.abs(o_emul - o_ref)
    say(f"  {label}: gpu max {err.max():.3e} mean {err.mean():.3e} | emulation max {err_e.max():.3e} "
        f"mean {err_e.mean():.3e}")
    assert np.isfinite(o).all()
    if spec_gate:
        # the 6e-2 figure is stated for the 16896-token shape; at small N (N = 1: O is the
        # quantised V itself) the e4m3 input rounding alone exceeds it for any correct pipeline
        assert err.max() <= SPEC_MAX_FP8
    assert err.mean() <= 1.25 * err_e.mean() + 1e-5
    assert err.max() <= 2.0 * err_e.max() + 1e-5
    # The 32x32x64 e4m3 MFMA does not sum its 64 products exactly: measured,
    # a sum loses up to about 2^-11 of the sum of its terms' magnitudes (small
    # terms beside a large one are truncated). The log-sum-exp moves by at most
    # the largest logit error, so per row
    #   |d lse_i| <= 2^-11 scale max_j sum_k |q_ik k_jk| <= 2^-11 scale |q_i| max_j |k_j|
    # (Cauchy-Schwarz, dequantised values) on top of the fp32 terms.
    qn = np.linalg.norm(oracle.e4m3_decode(q8[:, :, rows]) * np.float64(dq), axis=-1)
    kn = np.linalg.norm(oracle.e4m3_decode(k8) * np.float64(dk), axis=-1).max(axis=-1, keepdims=True)
    tol = 1e-4 + 1e-5 * np.abs(lse_emul) + 2.0**-11 * scale * qn * kn
    d_lse = np.abs(lse[:, :, rows] - lse_emul)
    say(f"  {label}: lse max |d| {d_lse.max():.3e} (largest allowed {tol.max():.3e}, smallest {tol.min():.3e})")
    assert (d_lse <= tol).all(), (d_lse - tol).max()


@pytest.mark.parametrize("N", [1, 65, 300, 1000])
def test_fp8_small(N):
    q, k, v = random_qkv(1, 2, N, 128, seed=100 + N)
    _check_fp8(q, k, v, 1 / math.sqrt(128), f"N={N}")


@pytest.mark.parametrize("name", ["t2i_2048_fp8", "t2i_2048_peaked"])
def test_fp8_workload_sampled_rows(name):
    """The spec gate applies to the workload it is stated for; the peaked rows
    (Q x 4) take the recompute path often and are held to the calibrated gate."""
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    rows = sample_rows(w.N, seed=0, n_edge=128, stride=64)
    _check_fp8(q, k, v, 1 / math.sqrt(128), name, rows=rows, spec_gate=name == "t2i_2048_fp8")


def test_fp8_output_independent_of_lse_request():
    """The kernel form without the log-sum-exp (the one the benchmark times)
    returns the same O, bit for bit, at the full workload and at a split shape."""
    for name, (q, k, v) in [("t2i_2048_fp8", make_qkv(WORKLOADS["t2i_2048_fp8"])),
                            ("B=1 H=3 N=5000", random_qkv(1, 3, 5000, 128, seed=21))]:
        say(f"[gpu] fp8 lse on/off {name}")
        o1, _ = _run_fp8(q, k, v, 1 / math.sqrt(128), want_lse=True)
        o0, _ = _run_fp8(q, k, v, 1 / math.sqrt(128), want_lse=False)
        assert np.array_equal(o0, o1), (name, np.abs(o0 - o1).max())


def test_fp8_growing_logits_rare_path():
    """Logits that grow by about 10 bits per 64-key sub-tile: relative to the
    stale running maximum the probabilities leave the e4m3 range (NaN), and
    every sub-tile takes the recompute path."""
    N, d = 1000, 128
    g = torch.Generator().manual_seed(33)
    q = torch.zeros((1, 2, N, d))
    q[..., 0] = 1.0
    k = 0.01 * torch.randn((1, 2, N, d), generator=g)
    k[..., 0] = 1.25 * torch.arange(N, dtype=torch.float32)
    v = torch.randn((1, 2, N, d), generator=g)
    _check_fp8(q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16), 1 / math.sqrt(d), "ramp")


def test_fp8_tile_coverage_exact():
    """Equal logits and one-hot V (exact in e4m3 after scaling by 448): every
    probability is 1, so O[c] = count_c / N up to the bf16 output rounding."""
    N = 16896
    q, k, v = coverage_pattern(1, 2, N, 128, block=64)
    o, _ = _run_fp8(q, k, v, 1 / math.sqrt(128))
    j = np.arange(N)
    exact = np.broadcast_to(np.bincount((j // 64) % 128, minlength=128) / N, o.shape)
    assert (np.abs(o - exact) <= 2.0**-8 * exact).all(), np.abs(o - exact).max()

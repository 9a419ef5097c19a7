"""GPU parity of the block-scaled (MX) e4m3 path: the on-device quantiser bit
for bit against the oracle's, and dit_attn_fwd_mx against the fp64 emulation
of the pipeline on the same codes and scales, with the gates of the
per-tensor fp8 path (calibrated against the emulation's own error with
respect to the exact attention on the bf16 inputs). Inputs whose blocks carry
different powers of two check that every scale reaches its block; exact
scaling identities check the same bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import SPEC_MAX_FP8, check_fp8_against_emulation, fp8_bound, lse_tolerance, say
from workloads import block_varied_qkv, make_qkv, one_growing_row, random_qkv, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dit():
    import diffusion_transformer_attention_non_amd as dit
    return dit


def _quant(x, along):
    codes, scales = _dit().quantize_mx(x.to(DEV), along)
    torch.cuda.synchronize()
    return codes, scales


def _check_quantizer(x, along, label):
    codes, scales = _quant(x, along)
    ref_c, ref_s = oracle.mx_quantize(x, along)
    got_c = codes.view(torch.uint8).cpu().numpy()
    got_s = scales.cpu().numpy()
    assert np.array_equal(got_s, ref_s), (label, int((got_s != ref_s).sum()))
    assert np.array_equal(got_c, ref_c), (label, int((got_c != ref_c).sum()))
    return codes, scales


@pytest.mark.parametrize("shape,std", [((1, 2, 37, 128), 1.0), ((2, 3, 64, 64), 1e-3), ((1, 1, 100, 32), 300.0),
                                       ((1, 2, 1000, 128), 1.0)])
def test_quantizer_bit_exact(shape, std):
    g = torch.Generator().manual_seed(sum(shape))
    x = (torch.randn(shape, generator=g) * std).to(torch.bfloat16)
    say(f"[gpu] mx quantise {shape} std {std}")
    for along in ("d", "tokens"):
        _check_quantizer(x, along, f"{shape} {along}")


def test_quantizer_edge_values():
    # zeros, powers of two, values at e4m3 rounding ties after scaling, tiny and huge blocks
    vals = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2])
    row = np.zeros(128 * 4)
    row[:mids.size] = mids[:row.size]
    x = np.stack([row, -row, row * 2.0**-100, row * 2.0**100, np.zeros_like(row)]).reshape(1, 1, 5 * 4, 128)
    x = np.concatenate([x, np.full((1, 1, 12, 128), 1.75), np.full((1, 1, 12, 128), 1.7578125)], axis=2)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    say(f"[gpu] mx quantise edge values {tuple(xt.shape)}")
    for along in ("d", "tokens"):
        _check_quantizer(xt, along, f"edges {along}")


def test_quantizer_full_workload():
    q, k, v = make_qkv("t2i_2048")
    say(f"[gpu] mx quantise t2i_2048 {tuple(q.shape)}")
    _check_quantizer(q, "d", "q")
    _check_quantizer(k, "d", "k")
    _check_quantizer(v, "tokens", "v")


def _mx_gpu(q, k, v):
    q8, qs = _check_quantizer(q, "d", "q")
    k8, ks = _check_quantizer(k, "d", "k")
    v8, vs = _check_quantizer(v, "tokens", "v")
    return q8, qs, k8, ks, v8, vs


def _run(inputs, scale, want_lse=True):
    dit = _dit()
    q8 = inputs[0]
    B, H, N, d = q8.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV) if want_lse else None
    o = dit.attention_mx(*inputs, scale, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def _check_mx(q, k, v, scale, label, rows=None, spec_gate=False):
    say(f"[gpu] mx attention {label}: shape {tuple(q.shape)}")
    inputs = _mx_gpu(q, k, v)
    o, lse = _run(inputs, scale)
    if rows is None:
        rows = np.arange(q.shape[2])
    og = o.float().cpu().double().numpy()[:, :, rows]
    lg = lse.cpu().double().numpy()[:, :, rows]
    o_ref, _ = oracle.attention(q, k, v, scale, rows=rows)
    codes = [t.view(torch.uint8).cpu().numpy() if t.dtype == torch.float8_e4m3fn else t.cpu().numpy() for t in inputs]
    o_emul, lse_emul = oracle.attention_mx_pipeline(*codes, scale, rows=rows)
    err = np.abs(og - o_ref)
    say(f"  {label}: gpu vs exact oracle max {err.max():.3e} mean {err.mean():.3e}")
    if spec_gate:
        assert err.max() <= SPEC_MAX_FP8
    qd = oracle.mx_dequantize(codes[0], codes[1], "d")
    kd = oracle.mx_dequantize(codes[2], codes[3], "d")
    vd = oracle.mx_dequantize(codes[4], codes[5], "tokens")
    bound, var, det = fp8_bound(qd, kd, vd, scale, o_emul, rows=rows)
    check_fp8_against_emulation(og, o_emul, bound, var, det, label)
    # exact log-sum-exp against the emulation's, with the e4m3 MFMA's inexact
    # internal sums bounded as in the per-tensor test (dequantised norms)
    mag = scale * np.linalg.norm(qd[:, :, rows], axis=-1) * np.linalg.norm(kd, axis=-1).max(axis=-1, keepdims=True)
    tol = lse_tolerance(q.shape[2], lse_emul, mag, logit_rel=2.0**-11)
    d_lse = np.abs(lg - lse_emul)
    say(f"  {label}: lse max |d| {d_lse.max():.3e} (worst d/tol {(d_lse / tol).max():.3f})")
    assert (d_lse <= tol).all(), (d_lse / tol).max()
    return inputs, o, lse


@pytest.mark.parametrize("N", [64, 65, 300, 1000])
def test_mx_attention_small(N):
    q, k, v = random_qkv(1, 2, N, 128, seed=500 + N)
    _check_mx(q, k, v, 1 / math.sqrt(128), f"iid N={N}")


@pytest.mark.parametrize("N", [128, 777])
def test_mx_attention_block_varied(N):
    q, k, v = block_varied_qkv(1, 2, N, 128, seed=600 + N)
    _check_mx(q, k, v, 1 / math.sqrt(128), f"block-varied N={N}")


def test_mx_one_row_overflow():
    """One row (row 700, lane 12 of its wave) whose logits grow about 40 bits
    per 64-key sub-tile; the block-scaled form's recompute must serve that
    wave alone. Against the MX emulation."""
    q, k, v = one_growing_row(1, 2, 1000, 128)
    _check_mx(q, k, v, 1 / math.sqrt(128), "one growing row")


def test_mx_attention_t2i_2048_sampled_rows():
    q, k, v = make_qkv("t2i_2048")
    rows = sample_rows(q.shape[2], seed=11, n_edge=256, stride=64)
    inputs, o, _ = _check_mx(q, k, v, 1 / math.sqrt(128), "t2i_2048", rows=rows, spec_gate=True)
    # O does not depend on whether the log-sum-exp is requested
    o2, _ = _run(inputs, 1 / math.sqrt(128), want_lse=False)
    assert torch.equal(o, o2)


def test_mx_scale_identities_bitwise():
    """Every V scale + 1 doubles O exactly; every K scale + 1 with half the
    logit multiplier, or every Q scale + 2 with a quarter of it, changes nothing."""
    q, k, v = block_varied_qkv(1, 3, 500, 128, seed=700)
    q8, qs, k8, ks, v8, vs = _mx_gpu(q, k, v)
    say("[gpu] mx scale identities")
    sc = 1 / math.sqrt(128)
    o, l = _run((q8, qs, k8, ks, v8, vs), sc)
    o_v, l_v = _run((q8, qs, k8, ks, v8, vs + 1), sc)
    assert torch.equal(o_v.float(), 2 * o.float()) and torch.equal(l_v, l)
    o_k, l_k = _run((q8, qs, k8, ks + 1, v8, vs), sc / 2)
    assert torch.equal(o_k, o) and torch.equal(l_k, l)
    o_q, l_q = _run((q8, qs + 2, k8, ks, v8, vs), sc / 4)
    assert torch.equal(o_q, o) and torch.equal(l_q, l)


def test_mx_rejects_bad_arguments():
    dit = _dit()
    x = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device=DEV)
    c = torch.empty((1, 1, 64, 128), dtype=torch.uint8, device=DEV)
    s = torch.empty(1024, dtype=torch.uint8, device=DEV)
    assert dit.dit_attn_quantize_mx(x, 1, 1, 64, 128, 2, c, s) == dit.DIT_ATTN_EINVAL
    assert dit.dit_attn_quantize_mx(x, 1, 1, 64, 48, 0, c, s) == dit.DIT_ATTN_EINVAL
    o = torch.empty((1, 1, 64, 64), dtype=torch.bfloat16, device=DEV)
    assert dit.dit_attn_fwd_mx(c, c, c, s, s, s, o, 1, 1, 64, 64, 0.1) == dit.DIT_ATTN_EUNSUPPORTED

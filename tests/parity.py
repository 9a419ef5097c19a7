"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the oracle on the same seeded inputs.

bf16 output, every compared element (float64 arithmetic), u = 2^-8 the unit
roundoff of bf16 (8 significant bits), w_j = p_ij the exact weights of row i,
A = sum_j w_j |V_jc|, M2 = sum_j w_j V_jc^2 (both from the oracle):
* spec: max |O_gpu - O| <= 2e-2 and mean |O_gpu - O| <= 2e-3.
* derived bound (bf16_bound):
      |O_gpu - O| <= (u (1 + 2^-6) + 2^-20 L) D + u |O|
                     + (N/16 + 48) 2^-24 (A + |O|) + 2^-12 A + 1e-6,
      D = min(A + |O|, sqrt(max(M2 - O^2, 0))).
  The kernels round each probability to bf16 (p~_j = p_j (1 + e_j),
  |e_j| <= u) and divide the P V product by the sum of the same rounded p~_j,
  so the weights become w_j (1 + e_j) / (1 + e), e = sum_j w_j e_j, and O
  moves by sum_j w_j e_j (V_j - O) / (1 + e): at most u (1 + 2^-7) D, where
  sum_j w_j |V_j - O| is at most A + |O| and, by Jensen, at most the weighted
  standard deviation sqrt(M2 - O^2). A logit carries at most 2^-21 L of fp32
  error (L = scale |q_i| max_j |k_j|, see logit_scale; 8 roundings of the
  MFMA chain, plus the exponent argument's own rounding and exp2's), which
  moves a weight by at most 2^-20 L relative, again against V_j - O (a common
  shift of every logit cancels). Rounding the output to bf16 adds u |O|. The
  fp32 sums (the PV accumulator over N/16 chained 16-term products, the row
  sum of the rounded P over N/32 sub-tiles of 32-term products, the final
  reciprocal) add at most (N/16 + 48) 2^-24 (A + |O|); 2^-12 A is slack.
* log-sum-exp (see lse_tolerance): the row sum is an fp32 sum of N terms in
  two levels (16 per lane and sub-tile, then N/32 partial sums, then the
  half-wave pair), relative error at most (16 + N/32 + 8) 2^-24; a logit
  carries at most 8 fp32 roundings of its MFMA chain (d/16 = 8 products of
  16 terms), 2^-21 scale sum_k |q_ik k_jk| <= 2^-21 scale |q_i| max_j |k_j|
  (Cauchy-Schwarz); the final log2 and the scaling to natural log add
  2^-22 |lse|.

fp8 (per-tensor or block-scaled) output against the fp64 emulation of the
same pipeline on the same codes (see fp8_bound): both round P to e4m3 (3
fraction bits, relative error <= 2^-4 in the normal range, absolute <= 2^-11
of the row maximum's p below it for the kernel's x2 scale), but relative to
different row maxima (the kernel's running maximum, the emulation's exact
one), so their roundings are independent. Each key j then moves O by
X_j = (eps_j - eps'_j)(V_j - O)/L with |X_j| <= c_j; Hoeffding's inequality
bounds the sum by z sqrt(sum_j c_j^2) except with probability 2 exp(-z^2/2)
(z = 8: 2.5e-14 per element). The e4m3 MFMA's truncated internal sums add a
relative logit error delta_i = 2^-11 scale |q_i| max |k| to the same terms,
and at most 2^-10 (A + |O|) to the products and row sums; the output's bf16
rounding adds u |O|. A second gate per row: the mean over d of the squared
differences must not exceed the mean of the bound's variance terms, whose
expectation it is at most (a coherent error of a fraction of the keys, well
inside the per-element bound, fails it).
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

import oracle

SPEC_MAX, SPEC_MEAN = 2e-2, 2e-3
SPEC_MAX_FP8 = 6e-2
U_BF16 = 2.0**-8
Z_FP8 = 8.0


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_attention(q, k, v, scale, want_lse=False, workspace=None):
    """q, k, v: CPU tensors (bf16 or float8_e4m3fn). Returns (O float64 numpy,
    lse or None). workspace: None (the library's fastest schedule) or a number
    of bytes of device workspace to hand over (0: one workgroup per tile)."""
    import diffusion_transformer_attention_non_amd as dit
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, H, N, d = q.shape
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev) if want_lse else None
    ws = None if workspace is None else torch.empty(workspace, dtype=torch.uint8, device=dev)
    o = dit.attention(qd, kd, vd, scale, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), (lse.cpu().double().numpy() if want_lse else None)


def bf16_bound(o_ref, a_ref, n_keys, m2_ref=None, logit_mag=None):
    """The derived per-element bound of the module docstring. o_ref, a_ref,
    m2_ref: (B, H, R, d); logit_mag: (B, H, R) (logit_scale) or None for
    logits of unit size; n_keys: keys each row attends to."""
    ao = a_ref + np.abs(o_ref)
    dev = ao if m2_ref is None else np.minimum(ao, np.sqrt(np.maximum(m2_ref - o_ref * o_ref, 0.0)))
    lm = 1.0 if logit_mag is None else np.asarray(logit_mag)[..., None]
    return (U_BF16 * (1 + 2.0**-6) + 2.0**-20 * lm) * dev + U_BF16 * np.abs(o_ref) \
        + (n_keys / 16 + 48) * 2.0**-24 * ao + 2.0**-12 * a_ref + 1e-6


def _f64(x):
    return x.detach().cpu().double().numpy() if hasattr(x, "detach") else np.asarray(x, dtype=np.float64)


def logit_scale(q, k, scale, rows=None):
    """scale |q_i| max_j |k_j| per (b, h, row): a bound on scale sum_k |q_ik k_jk|."""
    q, k = _f64(q), _f64(k)
    if rows is not None:
        q = q[:, :, rows]
    return scale * np.linalg.norm(q, axis=-1) * np.linalg.norm(k, axis=-1).max(axis=-1, keepdims=True)


def lse_tolerance(N, lse_ref, logit_mag, logit_rel=2.0**-21):
    """Derived bound on |lse_gpu - lse| (see the module docstring)."""
    return (16 + N / 32 + 8) * 2.0**-24 + logit_rel * logit_mag + 2.0**-22 * np.abs(lse_ref) + 1e-6


def check_lse(l_gpu, l_ref, tol, label=""):
    err = np.abs(l_gpu - l_ref)
    say(f"  {label} lse: max {float(err.max()):.3e} (worst err/tol {float((err / tol).max()):.3f})")
    assert np.isfinite(l_gpu).all(), label
    assert (err <= tol).all(), (label, float(err.max()), float((err / tol).max()))


def check_bf16(o_gpu, o_ref, a_ref, label="", *, n_keys, m2_ref=None, logit_mag=None):
    err = np.abs(o_gpu - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    bound = bf16_bound(o_ref, a_ref, n_keys, m2_ref, logit_mag)
    worst = float((err / bound).max())
    say(f"  {label}: max {mx:.3e} mean {mean:.3e} worst err/bound {worst:.3f}")
    assert np.isfinite(o_gpu).all(), label
    assert mx <= SPEC_MAX and mean <= SPEC_MEAN, (label, mx, mean)
    assert (err <= bound).all(), (label, worst, np.unravel_index(np.argmax(err / bound), err.shape))
    return mx, mean


def check_full(o_gpu, l_gpu, q, k, scale, ref, label, rows=None):
    """bf16 output and LSE against an oracle result ref = (O, lse, A[, M2])."""
    o_ref, l_ref, a_ref = ref[:3]
    m2_ref = ref[3] if len(ref) > 3 else None
    lm = logit_scale(q, k, scale, rows)
    check_bf16(o_gpu, o_ref, a_ref, label, n_keys=q.shape[2], m2_ref=m2_ref, logit_mag=lm)
    if l_gpu is not None:
        tol = lse_tolerance(q.shape[2], l_ref, lm)
        check_lse(l_gpu, l_ref, tol, label)


def oracle_ref(q, k, v, scale, rows=None):
    """(O, lse, A, M2) of the fp64 oracle: what check_full takes."""
    return oracle.attention(q, k, v, scale, rows=rows, want_abs=True, want_sq=True)


@functools.lru_cache(maxsize=2)
def oracle_workload(name: str):
    """The fp64 oracle (O, lse, A, M2) on every row of a named workload, computed
    once per test session (the bf16 and fp8 tests of one shape share it)."""
    from workloads import WORKLOADS, make_qkv
    w = WORKLOADS[name]
    q, k, v = make_qkv(w)
    say(f"  oracle on every row of {name} (B={w.B} H={w.H} N={w.N} d={w.d}) ...")
    return oracle.attention(q, k, v, 1.0 / np.sqrt(w.d), want_abs=True, want_sq=True)


def fp8_bound(q, k, v, scale, o_emul, rows=None, block=512, z=Z_FP8):
    """Per-element bound on |O_kernel - O_emulation| for the e4m3 pipeline,
    and the per-element variance terms of the row gate.

    q, k, v: dequantised float64 values (B, H, N, d) (v including its
    descale); o_emul: the emulation's output on the rows ``rows``. Returns
    (bound, var, det) with bound = z sqrt(var) + det."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    var = np.empty_like(o_emul)
    det = np.empty_like(o_emul)
    beta = 2.0**-11 * (1 + 2.0**-7)        # subnormal floors of the kernel (x2) and the emulation (x256)
    for b in range(B):
        for h in range(H):
            kt = k[b, h].T
            vb = v[b, h]
            v2 = vb * vb
            sv, sv2 = vb.sum(axis=0), v2.sum(axis=0)
            kmax = np.linalg.norm(k[b, h], axis=-1).max()
            for r0 in range(0, idx.size, block):
                sel = idx[r0:r0 + block]
                s = (q[b, h, sel] @ kt) * scale
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                L = p.sum(axis=1, keepdims=True)
                w = p / L
                w2 = w * w
                o = o_emul[b, h, r0:r0 + sel.size]
                t1 = w2 @ v2 - 2 * o * (w2 @ vb) + o * o * w2.sum(axis=1, keepdims=True)   # sum w^2 (v - o)^2
                wv2 = w @ v2
                t2 = wv2 - 2 * o * (w @ vb) + o * o                                      # sum w (v - o)^2
                t3 = sv2 - 2 * o * sv + N * o * o                                        # sum (v - o)^2
                delta = 2.0**-11 * scale * np.linalg.norm(q[b, h, sel], axis=-1, keepdims=True) * kmax
                alpha = 2.0**-3 + delta        # both sides' 2^-4 relative rounding, plus the logit error
                c2 = alpha**2 * t1 + 2 * alpha * beta / L * t2 + (beta / L)**2 * t3
                var[b, h, r0:r0 + sel.size] = np.maximum(c2, 0.0)
                a_ub = np.sqrt(np.maximum(wv2, 0.0))                                      # >= sum w |v|
                det[b, h, r0:r0 + sel.size] = U_BF16 * (1 + 2.0**-6) * np.abs(o) + 2.0**-10 * (a_ub + np.abs(o)) \
                    + 1e-6
    return z * np.sqrt(var) + det, var, det


def check_fp8_against_emulation(o_gpu, o_emul, bound, var, det, label=""):
    diff = np.abs(o_gpu - o_emul)
    worst = float((diff / bound).max())
    row = (diff**2).mean(axis=-1) / (var + det**2).mean(axis=-1)
    say(f"  {label}: gpu vs emulation max {diff.max():.3e} mean {diff.mean():.3e}; worst |diff|/bound {worst:.3f}; "
        f"worst row mean-square ratio {float(row.max()):.3f}")
    assert np.isfinite(o_gpu).all(), label
    assert (diff <= bound).all(), (label, worst, np.unravel_index(np.argmax(diff / bound), diff.shape))
    assert (row <= 1.0).all(), (label, float(row.max()), np.unravel_index(np.argmax(row), row.shape))


def rows_of(o, rows):
    return o[:, :, rows, :]

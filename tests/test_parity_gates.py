"""The parity gates themselves, on the CPU: a numpy model of the kernels'
rounding steps must pass them, and planted mistakes must fail them. The
model is test infrastructure (like the oracle it is compared with); it
follows the steps the kernels take that the oracle does not fix: P relative
to the maximum of the first keys of the row (not the exact row maximum) and,
for fp8, the x2 scale before the e4m3 rounding."""
import math

import numpy as np
import pytest

import oracle
from parity import bf16_bound, check_fp8_against_emulation, fp8_bound, logit_scale
from workloads import random_qkv


def _fp8_model(q8, k8, v8, dq, dk, dv, scale, mistake=None):
    q = oracle.e4m3_decode(q8) * np.float64(dq)
    k = oracle.e4m3_decode(k8) * np.float64(dk)
    v = oracle.e4m3_decode(v8)
    B, H, N, d = q.shape
    out = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            s = q[b, h] @ k[b, h].T * scale
            P = 2 * np.exp(s - s[:, :64].max(axis=1, keepdims=True))
            assert P.max() < 448
            if mistake == "block scaled twice":
                P[:, 64:128] *= 2
            P8 = oracle.e4m3_decode(oracle.e4m3_encode(P))
            if mistake == "one key dropped":
                P8[:, 777] = 0
            out[b, h] = oracle.bf16_round((P8 @ v[b, h]) * np.float64(dv) / P8.sum(axis=1, keepdims=True))
    return out


@pytest.mark.parametrize("N", [300, 2048])
def test_fp8_gate_passes_the_model_and_fails_planted_mistakes(N):
    q, k, v = random_qkv(1, 2, N, 128, seed=5 + N)
    scale = 1 / math.sqrt(128)
    (q8, dq, _), (k8, dk, _), (v8, dv, _) = (oracle.quantize_per_tensor(t) for t in (q, k, v))
    o_emul, _ = oracle.attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale, den_rounded=True)
    qd, kd, vd = (oracle.e4m3_decode(c) * np.float64(x) for c, x in ((q8, dq), (k8, dk), (v8, dv)))
    bound, var, det = fp8_bound(qd, kd, vd, scale, o_emul)
    check_fp8_against_emulation(_fp8_model(q8, k8, v8, dq, dk, dv, scale), o_emul, bound, var, det, "model")
    mistakes = ["block scaled twice"] + (["one key dropped"] if N > 777 else [])
    for m in mistakes:
        with pytest.raises(AssertionError):
            check_fp8_against_emulation(_fp8_model(q8, k8, v8, dq, dk, dv, scale, m), o_emul, bound, var, det, m)


def _bf16_model(q, k, v, scale, mistake=None):
    q, k, v = (t.double().numpy() for t in (q, k, v))
    B, H, N, d = q.shape
    out = np.empty((B, H, N, d))
    for b in range(B):
        for h in range(H):
            s = q[b, h] @ k[b, h].T * scale
            p = np.exp(s - s[:, :32].max(axis=1, keepdims=True))
            pr = oracle.bf16_round(p)
            if mistake == "one key dropped":
                pr[:, N // 2] = 0
            # the kernels' arithmetic: bf16 P, divided by the sum of the same rounded P
            out[b, h] = oracle.bf16_round((pr @ v[b, h]) / pr.sum(axis=1, keepdims=True))
    return out


def test_bf16_bound_passes_the_model_and_fails_a_dropped_key():
    q, k, v = random_qkv(1, 2, 1000, 128, seed=77)
    scale = 1 / math.sqrt(128)
    o_ref, _, a_ref, m2_ref = oracle.attention(q, k, v, scale, want_abs=True, want_sq=True)
    lm = logit_scale(q, k, scale)
    for m2 in (None, m2_ref):
        bound = bf16_bound(o_ref, a_ref, 1000, m2, lm)
        err = np.abs(_bf16_model(q, k, v, scale) - o_ref)
        assert (err <= bound).all(), float((err / bound).max())
        err = np.abs(_bf16_model(q, k, v, scale, "one key dropped") - o_ref)
        assert not (err <= bound).all()


def test_bf16_bound_covers_rounding_errors_aligned_with_the_values():
    """Dividing by the sum of the rounded P moves O by sum_j w_j e_j (V_j - O),
    which can exceed u (A + |O|): here 2 keys of value 10 whose p round up
    and 63 keys of value 0 whose p round down (all p in [1, 2), so each
    rounding error is chosen by its p). The derived bound holds; a bound of
    u (A + |O|)(1 + 2^-6) would not."""
    u = 2.0**-8
    p = np.array([1 + 0.51 * 2.0**-7] * 2 + [1 + 1.49 * 2.0**-7] * 63)
    v = np.array([10.0] * 2 + [0.0] * 63)
    w = p / p.sum()
    o, a, m2 = w @ v, w @ np.abs(v), w @ (v * v)
    pr = oracle.bf16_round(p)
    got = oracle.bf16_round((pr @ v) / pr.sum())
    err = abs(got - o)
    narrow = u * (a + abs(o)) * (1 + 2.0**-6) + 2.0**-12 * a + 1e-6
    assert err > narrow
    bound = bf16_bound(np.array([[[[o]]]]), np.array([[[[a]]]]), 65, np.array([[[[m2]]]]))
    assert err <= float(bound.ravel()[0])

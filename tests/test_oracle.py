"""Pins of the fp64 attention oracle against things other than itself.

Each pin is a function of an attention implementation, so the same pins are
also run against copies of the oracle with a planted mistake (a transposed
operand, a wrong sign, a dropped key, a wrong normaliser, ...): every such
mutant must fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import random_qkv


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ------------------------------------------------------------------ pins
def pin_bruteforce(attn):
    """Against literal loops with correctly rounded sums."""
    for (B, H, N, d), seed in [((1, 1, 1, 1), 0), ((1, 1, 2, 2), 1), ((1, 2, 3, 5), 2),
                               ((1, 1, 17, 8), 3), ((2, 1, 33, 16), 4), ((1, 1, 65, 4), 5)]:
        q, k, v = _rand((B, H, N, d), seed), _rand((B, H, N, d), seed + 100), _rand((B, H, N, d), seed + 200)
        scale = 1.0 / math.sqrt(d)
        o, lse = attn(q, k, v, scale)
        ob, lb = oracle.attention_bruteforce(q, k, v, scale)
        if not (np.allclose(o, ob, rtol=0, atol=1e-12) and np.allclose(lse, lb, rtol=0, atol=1e-12)):
            return False
    return True


def pin_torch_sdpa(attn):
    """Against torch's float64 CPU scaled-dot-product attention (a library routine)."""
    for (B, H, N, d), seed in [((1, 2, 64, 64), 7), ((1, 2, 300, 128), 8)]:
        q, k, v = (_rand((B, H, N, d), seed + i) for i in range(3))
        scale = 1.0 / math.sqrt(d)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
        o, _ = attn(q, k, v, scale)
        if not np.allclose(o, ref, rtol=0, atol=1e-12):
            return False
    return True


def pin_single_token(attn):
    """N = 1: the only probability is 1, so O = V and lse = scale*<q,k>."""
    q, k, v = _rand((2, 3, 1, 16), 11), _rand((2, 3, 1, 16), 12), _rand((2, 3, 1, 16), 13)
    o, lse = attn(q, k, v, 0.25)
    return np.array_equal(o, v) and np.allclose(lse, 0.25 * (q * k).sum(-1), rtol=0, atol=1e-13)


def pin_two_tokens(attn):
    """N = 2: softmax of two logits is the logistic function of their difference."""
    q, k, v = _rand((1, 4, 2, 8), 21), _rand((1, 4, 2, 8), 22), _rand((1, 4, 2, 8), 23)
    scale = 0.7
    o, _ = attn(q, k, v, scale)
    for h in range(4):
        for i in range(2):
            delta = scale * (q[0, h, i] @ (k[0, h, 0] - k[0, h, 1]))
            sig = 1.0 / (1.0 + math.exp(-delta))
            ref = sig * v[0, h, 0] + (1.0 - sig) * v[0, h, 1]
            if not np.allclose(o[0, h, i], ref, rtol=0, atol=1e-14):
                return False
    return True


def pin_constant_values(attn):
    """V rows all equal c: O = c whatever the probabilities (they sum to 1)."""
    q, k = _rand((1, 2, 50, 8), 31), _rand((1, 2, 50, 8), 32)
    c = _rand((8,), 33)
    v = np.broadcast_to(c, (1, 2, 50, 8)).copy()
    o, _ = attn(q, k, v, 0.5)
    return np.allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


def pin_identical_keys(attn):
    """All keys equal: all logits of a row equal, p = 1/N, O = mean of V."""
    q, v = _rand((1, 2, 40, 8), 41), _rand((1, 2, 40, 8), 42)
    k = np.broadcast_to(_rand((1, 2, 1, 8), 43), (1, 2, 40, 8)).copy()
    o, lse = attn(q, k, v, 0.3)
    mean = v.mean(axis=2, keepdims=True)
    ok_o = np.allclose(o, np.broadcast_to(mean, o.shape), rtol=0, atol=1e-14)
    ok_l = np.allclose(lse, 0.3 * (q * k).sum(-1) + math.log(40), rtol=0, atol=1e-12)
    return ok_o and ok_l


def pin_vanishing_scale(attn):
    """scale -> 0: every logit -> 0, p -> 1/N, O -> mean of V."""
    q, k, v = _rand((1, 1, 37, 8), 51), _rand((1, 1, 37, 8), 52), _rand((1, 1, 37, 8), 53)
    o, _ = attn(q, k, v, 1e-30)
    return np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), rtol=0, atol=1e-14)


def pin_permutations(attn):
    """Joint permutation of K and V rows leaves O unchanged; permuting Q rows
    permutes O rows; adding one vector c to every key adds scale*<q_i,c> to
    every logit of row i and leaves O unchanged."""
    rng = np.random.default_rng(61)
    q, k, v = _rand((1, 2, 45, 8), 62), _rand((1, 2, 45, 8), 63), _rand((1, 2, 45, 8), 64)
    o, lse = attn(q, k, v, 0.4)
    pk = rng.permutation(45)
    o2, _ = attn(q, k[:, :, pk], v[:, :, pk], 0.4)
    pq = rng.permutation(45)
    o3, _ = attn(q[:, :, pq], k, v, 0.4)
    c = _rand((8,), 65)
    o4, lse4 = attn(q, k + c, v, 0.4)
    return (np.allclose(o, o2, rtol=0, atol=1e-13) and np.allclose(o[:, :, pq], o3, rtol=0, atol=1e-13)
            and np.allclose(o, o4, rtol=0, atol=1e-12)
            and np.allclose(lse4 - lse, 0.4 * (q @ c), rtol=0, atol=1e-12))


def pin_dominating_key(attn):
    """One key aligned with every query by a logit gap of ~100: O = V[j*]."""
    N, d = 70, 16
    u = np.sign(_rand((d,), 71))
    for j_star in (0, 33, 69):
        q = np.broadcast_to(2.5 * u, (1, 1, N, d)).copy()
        k = 0.01 * _rand((1, 1, N, d), 72)
        k[0, 0, j_star] = 2.5 * u
        v = _rand((1, 1, N, d), 73)
        o, _ = attn(q, k, v, 1.0)
        if not np.allclose(o, np.broadcast_to(v[:, :, j_star:j_star + 1], o.shape), rtol=0, atol=1e-12):
            return False
    return True


PINS = [pin_bruteforce, pin_torch_sdpa, pin_single_token, pin_two_tokens, pin_constant_values,
        pin_identical_keys, pin_vanishing_scale, pin_permutations, pin_dominating_key]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(oracle.attention)


def test_oracle_row_subset_and_blocking_exact():
    q, k, v = _rand((2, 2, 301, 16), 81), _rand((2, 2, 301, 16), 82), _rand((2, 2, 301, 16), 83)
    o, lse = oracle.attention(q, k, v, 0.25)
    o7, lse7 = oracle.attention(q, k, v, 0.25, block=7)
    rows = np.array([0, 5, 150, 299, 300])
    orow, lrow = oracle.attention(q, k, v, 0.25, rows=rows, block=2)
    assert np.allclose(o, o7, rtol=0, atol=1e-13) and np.allclose(lse, lse7, rtol=0, atol=1e-13)
    assert np.allclose(orow, o[:, :, rows], rtol=0, atol=1e-13)
    assert np.allclose(lrow, lse[:, :, rows], rtol=0, atol=1e-13)


def test_oracle_weighted_abs_and_row_sums():
    q, k, v = _rand((1, 2, 60, 8), 91), _rand((1, 2, 60, 8), 92), _rand((1, 2, 60, 8), 93)
    p = oracle.softmax_probabilities(q, k, 0.5)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert (p > 0).all()
    o, _, a = oracle.attention(q, k, v, 0.5, want_abs=True)
    assert np.allclose(a, p @ np.abs(v), rtol=0, atol=1e-13)
    assert np.allclose(o, p @ v, rtol=0, atol=1e-13)
    ones, _ = oracle.attention(q, k, np.ones_like(v), 0.5)
    assert np.allclose(ones, 1.0, rtol=0, atol=1e-14)


def test_oracle_weighted_second_moment():
    """M2 = sum_j p_ij v_jc^2, pinned by literal loops (math.fsum, no matrix
    product), the variance identity sum_j p_ij (v_jc - O_ic)^2 = M2 - O^2,
    a constant column (M2 = c^2) and a one-hot row (M2 = v_jc^2)."""
    q, k, v = _rand((1, 1, 12, 4), 94), _rand((1, 1, 12, 4), 95), _rand((1, 1, 12, 4), 96)
    o, _, m2 = oracle.attention(q, k, v, 0.7, want_sq=True)
    s = [[0.7 * math.fsum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(4)) for j in range(12)] for i in range(12)]
    for i in range(12):
        mx = max(s[i])
        w = [math.exp(x - mx) for x in s[i]]
        den = math.fsum(w)
        for c in range(4):
            sq = math.fsum(w[j] * v[0, 0, j, c] ** 2 for j in range(12)) / den
            var = math.fsum(w[j] * (v[0, 0, j, c] - o[0, 0, i, c]) ** 2 for j in range(12)) / den
            assert abs(m2[0, 0, i, c] - sq) <= 1e-13 * max(1.0, sq)
            assert abs((m2[0, 0, i, c] - o[0, 0, i, c] ** 2) - var) <= 1e-12
    vc = np.tile(np.array([2.0, -3.0, 0.5, 0.0]), (1, 1, 12, 1))
    _, _, a2, m2c = oracle.attention(q, k, vc, 0.7, want_abs=True, want_sq=True)
    assert np.allclose(m2c, vc[:, :, :1] ** 2, rtol=0, atol=1e-13)
    assert np.allclose(a2, np.abs(vc[:, :, :1]), rtol=0, atol=1e-13)
    kp = np.zeros((1, 1, 12, 4))
    kp[0, 0, 5, 0] = 1e3               # key 5 dominates every row with q[..., 0] > 0
    qp = np.abs(q) + 0.1
    _, _, m2p = oracle.attention(qp, kp, v, 1.0, want_sq=True)
    assert np.allclose(m2p, np.broadcast_to(v[:, :, 5:6] ** 2, m2p.shape), rtol=1e-12, atol=1e-12)


def test_oracle_accepts_bf16_tensors_exactly():
    q, k, v = random_qkv(1, 1, 20, 8, seed=3)
    o, _ = oracle.attention(q, k, v, 0.35)
    o2, _ = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.35)
    assert np.array_equal(o, o2)


# ------------------------------------------------------------------ planted mistakes
def _mutant(kind):
    def attn(q, k, v, scale, rows=None, block=512):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        s = np.einsum("bhid,bhjd->bhij", q, k) * scale
        if kind == "transposed_logits":
            s = np.swapaxes(s, -1, -2)
        if kind == "scale_twice":
            s = s * scale
        if kind == "scale_missing":
            s = s / scale
        m = s.max(-1, keepdims=True)
        e = np.exp(m - s) if kind == "wrong_sign" else np.exp(s - m)
        if kind == "dropped_last_key":
            e[..., -1] = 0.0
        den = e.sum(-1, keepdims=True)
        if kind == "mean_normaliser":
            den = np.full_like(den, e.shape[-1])
        if kind == "values_are_keys":
            o = (e @ k) / den
        elif kind == "values_transposed_heads":
            o = (e @ np.flip(v, axis=1)) / den
        elif kind == "max_not_readded_in_lse":
            o = (e @ v) / den
            return o, np.log(den[..., 0])
        elif kind == "lse_missing_log":
            o = (e @ v) / den
            return o, m[..., 0] + den[..., 0]
        else:
            o = (e @ v) / den
        return o, m[..., 0] + np.log(den[..., 0])
    return attn


MUTANTS = ["transposed_logits", "scale_twice", "scale_missing", "wrong_sign", "dropped_last_key",
           "mean_normaliser", "values_are_keys", "values_transposed_heads", "max_not_readded_in_lse",
           "lse_missing_log"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    attn = _mutant(kind)
    with np.errstate(all="ignore"):
        failed = [p.__name__ for p in PINS if not p(attn)]
    assert failed, f"mutant {kind} passed every pin"


def test_unmutated_reference_copy_passes():
    """The mutant harness itself, with no mutation, passes every pin."""
    attn = _mutant("none")
    assert all(p(attn) for p in PINS)

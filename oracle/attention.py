"""fp64 CPU oracle of dense, non-causal softmax attention.

What is computed
----------------
For every batch entry b and head h, over the N tokens of the joint
text+image sequence (text tokens first, then image tokens, then any
reference-image tokens):

    s_ij = scale * <Q[b,h,i,:], K[b,h,j,:]>
    p_ij = exp(s_ij - M_i) / sum_k exp(s_ik - M_i),   M_i = max_j s_ij
    O[b,h,i,:] = sum_j p_ij * V[b,h,j,:]

Sources and readings
--------------------
* The pages name the operation only as the DiT's dense (also called standard
  or traditional) BF16 attention, which takes about 60% of DiT kernel time at
  2048x2048 ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
  Blackwell GPUs", "Key takeaways"; Japanese summary, third paragraph;
  Italian commentary, section "NVFP4, attention e caching"). No formula is
  printed; the definition above is the standard scaled-dot-product softmax
  attention.
* Non-causal, no mask: the glossary of the same card describes the
  transformer as letting every token consider every other token. Its
  separate "earlier words" gloss of attention describes a causal language
  model and is not taken.
* Subtracting M_i is exact in real arithmetic; it keeps fp64 in range for
  peaked rows.
* ``lse_i = M_i + log(sum_j exp(s_ij - M_i))`` is the natural-log
  normaliser of row i.

This is the plain definition written out: a matrix product (a library
primitive) for the two contractions, nothing blocked beyond splitting query
rows into groups to bound memory (each output row depends on one query row
only, so the split is exact).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch/numpy tensor (bf16, fp32, fp64) to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, scale: float, rows=None, block: int = 512, want_abs: bool = False,
              want_sq: bool = False):
    """Return ``(O, lse)`` (then ``A`` if ``want_abs``, then ``M2`` if
    ``want_sq``) in float64.

    q, k, v: (B, H, N, d) arrays or tensors. ``rows``: optional index array
    of query rows to evaluate (the same rows for every (b, h)); the outputs
    then have R = len(rows) rows. ``A[b,h,i,c] = sum_j p_ij |V[b,h,j,c]|`` and
    ``M2[b,h,i,c] = sum_j p_ij V[b,h,j,c]^2`` are the weighted absolute value
    and second moment of V's column under row i's weights; they bound the
    effect of rounding p (test infrastructure, not part of the operation).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    assert k.shape == (B, H, N, d) and v.shape == (B, H, N, d)
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = idx.size
    out = np.empty((B, H, R, d))
    lse = np.empty((B, H, R))
    absw = np.empty((B, H, R, d)) if want_abs else None
    sqw = np.empty((B, H, R, d)) if want_sq else None
    for b in range(B):
        for h in range(H):
            kt = k[b, h].T
            vb = v[b, h]
            va = np.abs(vb) if want_abs else None
            vs = vb * vb if want_sq else None
            for r0 in range(0, R, block):
                sel = idx[r0:r0 + block]
                s = (q[b, h, sel] @ kt) * scale          # logits of these rows
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                den = e.sum(axis=1, keepdims=True)
                out[b, h, r0:r0 + sel.size] = (e @ vb) / den
                lse[b, h, r0:r0 + sel.size] = m[:, 0] + np.log(den[:, 0])
                if want_abs:
                    absw[b, h, r0:r0 + sel.size] = (e @ va) / den
                if want_sq:
                    sqw[b, h, r0:r0 + sel.size] = (e @ vs) / den
    res = (out, lse)
    if want_abs:
        res += (absw,)
    if want_sq:
        res += (sqw,)
    return res


def softmax_probabilities(q, k, scale: float) -> np.ndarray:
    """The (B, H, N, N) matrix p_ij itself (small inputs only)."""
    q, k = _f64(q), _f64(k)
    s = np.einsum("bhid,bhjd->bhij", q, k) * scale
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def attention_bruteforce(q, k, v, scale: float):
    """Literal loops over (b, h, i, j, c) with ``math.exp`` and ``math.fsum``.

    Independent second implementation for tiny inputs: no matrix product,
    every sum correctly rounded. Returns (O, lse) as nested float64 arrays."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    out = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            K = k[b, h].tolist()
            V = v[b, h].tolist()
            for i in range(N):
                qi = q[b, h, i].tolist()
                s = [scale * math.fsum(qi[c] * K[j][c] for c in range(d)) for j in range(N)]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                for c in range(d):
                    out[b, h, i, c] = math.fsum(w[j] * V[j][c] for j in range(N)) / den
                lse[b, h, i] = mx + math.log(den)
    return out, lse

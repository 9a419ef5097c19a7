"""fp64 CPU oracle of block-sparse attention (TEST INFRASTRUCTURE).

What is computed
----------------
Queries are grouped in blocks of ``q_block`` consecutive rows and keys in
blocks of ``kv_block`` consecutive tokens (the last block of each may be
short). Query block t of head (b, h) comes with a list of key blocks; S is
the set of keys in those blocks (keys past N do not exist). Every query row
i of block t attends to S only:

    s_ij = scale * <Q[b,h,i,:], K[b,h,j,:]>              for j in S
    O[b,h,i,:] = sum_{j in S} exp(s_ij - M_i) V[b,h,j,:] / sum_{j in S} exp(s_ij - M_i)
    lse_i = M_i + log(sum_{j in S} exp(s_ij - M_i)),      M_i = max_{j in S} s_ij

that is, softmax attention with the logits of keys outside S set to -inf.
An empty S gives O = 0 and lse = -inf.

Sources and readings
--------------------
* The pages report a sparse attention mode of the DiT (Sol-Attention at
  tau = 1.0, with the first 12 or 16 denoising steps dense) and its speed
  and image-distance figures (Japanese summary, third and fourth
  paragraphs). They do not say how blocks are chosen; only the
  execution given a choice is defined, and that is what this computes.
* Reading: "sparse" means that whole blocks of keys are skipped for a block
  of queries, and the softmax renormalises over the keys that remain (the
  plain meaning of attention restricted to a key subset). Block sizes are
  those of the GPU kernel's tiles (256 queries, 64 keys) by default.
* Reading: with no key left, the empty sum gives O = 0 and lse = log 0.
* The list is a set: order and repeats do not matter here.

Only the definition written out: one matrix product per group of rows (a
library primitive) and an explicit -inf mask.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64


def key_set(blocks_row, count, N: int, kv_block: int = 64) -> np.ndarray:
    """Boolean mask over the N keys: True for keys of the first ``count`` listed blocks."""
    mask = np.zeros(N, dtype=bool)
    for u in np.asarray(blocks_row)[:max(0, int(count))]:
        mask[int(u) * kv_block:min(N, (int(u) + 1) * kv_block)] = True
    return mask


def attention_blocksparse(q, k, v, scale: float, kv_blocks, kv_counts, *, q_block: int = 256,
                          kv_block: int = 64, rows=None, want_abs: bool = False):
    """Return ``(O, lse)`` (and ``A`` if ``want_abs``) in float64 for block-sparse attention.

    q, k, v: (B, H, N, d). kv_blocks: (B, H, nq, max_blocks) integer array,
    kv_counts: (B, H, nq), nq = ceil(N / q_block). ``rows``: optional sorted
    query-row indices to evaluate (the same for every (b, h)).
    ``A[b,h,i,c] = sum_{j in S} p_ij |V[b,h,j,c]|`` (0 for an empty S)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    kv_blocks = np.asarray(kv_blocks.cpu() if hasattr(kv_blocks, "cpu") else kv_blocks)
    kv_counts = np.asarray(kv_counts.cpu() if hasattr(kv_counts, "cpu") else kv_counts)
    B, H, N, d = q.shape
    nq = -(-N // q_block)
    assert kv_counts.shape == (B, H, nq) and kv_blocks.shape[:3] == (B, H, nq)
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, idx.size, d))
    lse = np.full((B, H, idx.size), -np.inf)
    absw = np.zeros((B, H, idx.size, d)) if want_abs else None
    for b in range(B):
        for h in range(H):
            for t in range(nq):
                pos = np.nonzero((idx >= t * q_block) & (idx < (t + 1) * q_block))[0]
                if pos.size == 0:
                    continue
                mask = key_set(kv_blocks[b, h, t], kv_counts[b, h, t], N, kv_block)
                if not mask.any():
                    continue                              # O = 0, lse = -inf
                s = (q[b, h, idx[pos]] @ k[b, h].T) * scale
                s[:, ~mask] = -np.inf
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)                         # exp(-inf) = 0 outside S
                den = e.sum(axis=1, keepdims=True)
                out[b, h, pos] = (e @ v[b, h]) / den
                lse[b, h, pos] = m[:, 0] + np.log(den[:, 0])
                if want_abs:
                    absw[b, h, pos] = (e @ np.abs(v[b, h])) / den
    if want_abs:
        return out, lse, absw
    return out, lse

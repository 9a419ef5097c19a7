"""fp64 emulation of the fp8-e4m3 attention pipeline.

Reading taken (the pages only report that FP8 attention exists and runs
about 1.08-1.18x faster end to end than BF16 attention, Japanese summary,
third paragraph; English card, "Key takeaways"): Q, K and V are each
quantised per tensor to e4m3 with an absmax scale, the logits are formed
from the e4m3 values and rescaled by dq*dk*scale, the softmax probabilities
p (relative to the row maximum) are multiplied by 2^8 and rounded to e4m3
before the second contraction, and the output is (P8 V8) * dv / (2^8 * l).
The pages leave l open. Two readings are provided: l from the unrounded p
(the default), or l from the rounded P8 themselves (``den_rounded=True``),
which makes every output row an exact convex combination of rows of V8. The
log-sum-exp returned is always the exact one, m + log(sum p).

Everything here is evaluated exactly in float64 apart from the two e4m3
roundings the pipeline itself prescribes (inputs, and P).
"""
from __future__ import annotations

import numpy as np

from .formats import e4m3_decode, e4m3_encode

P_SCALE = 256.0


def attention_fp8_pipeline(q8, k8, v8, dq, dk, dv, scale, rows=None, block=512,
                           p_scale=P_SCALE, round_p=True, den_rounded=False):
    """Return (O, lse) of the emulated fp8 pipeline, float64.

    q8, k8, v8: uint8 e4m3 codes of shape (B, H, N, d). ``round_p=False``
    skips the rounding of P (then this equals plain attention on the
    dequantised inputs)."""
    q = e4m3_decode(q8) * np.float64(dq)
    k = e4m3_decode(k8) * np.float64(dk)
    v = e4m3_decode(v8)
    return pipeline_on_values(q, k, v, dv, scale, rows=rows, block=block, p_scale=p_scale, round_p=round_p,
                              den_rounded=den_rounded)


def pipeline_on_values(q, k, v, dv, scale, rows=None, block=512, p_scale=P_SCALE, round_p=True,
                       den_rounded=False):
    """The pipeline after the inputs are dequantised: q, k, v float64 (B, H, N, d)
    values, dv the factor O carries. Shared by the per-tensor and the
    block-scaled (MX) input formats."""
    B, H, N, d = q.shape
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = idx.size
    out = np.empty((B, H, R, d))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            kt = k[b, h].T
            for r0 in range(0, R, block):
                sel = idx[r0:r0 + block]
                s = (q[b, h, sel] @ kt) * scale
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                den = p.sum(axis=1, keepdims=True)
                if round_p:
                    p8 = e4m3_decode(e4m3_encode(p * p_scale))
                    l8 = p8.sum(axis=1, keepdims=True) if den_rounded else p_scale * den
                    o = (p8 @ v[b, h]) * np.float64(dv) / l8
                else:
                    o = (p @ v[b, h]) * np.float64(dv) / den
                out[b, h, r0:r0 + sel.size] = o
                lse[b, h, r0:r0 + sel.size] = m[:, 0] + np.log(den[:, 0])
    return out, lse

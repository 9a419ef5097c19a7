"""MI355X (gfx950) dense joint text+image attention for diffusion transformers.

O = softmax(Q K^T * scale) V over the concatenated text and image tokens,
non-causal, computed by hand-written HIP kernels behind the C ABI of
``libditattn.so`` (declared in ``include/dit_attn.h``). The functions below
check torch tensors and pass their device addresses and the current stream
to the C entry points; PyTorch only provides device memory and streams.
"""
from __future__ import annotations

import math

from . import _lib
from ._lib import (DIT_ATTN_BF16, DIT_ATTN_EDEVICE, DIT_ATTN_EINVAL, DIT_ATTN_ELAUNCH, DIT_ATTN_FP8_E4M3,
                   DIT_ATTN_MX_ALONG_D, DIT_ATTN_MX_ALONG_TOKENS, DIT_ATTN_OK, DIT_ATTN_SPARSE_KV_BLOCK,
                   DIT_ATTN_SPARSE_Q_BLOCK, DIT_ATTN_EUNSUPPORTED, dit_attn_fwd, dit_attn_fwd_blocksparse,
                   dit_attn_fwd_ex, dit_attn_fwd_mx, dit_attn_fwd_strided, dit_attn_plan, dit_attn_quantize_e4m3,
                   dit_attn_quantize_mx, dit_attn_strerror, dit_attn_version, DitAttnPlan, DIT_ATTN_SCHED_SPLIT,
                   DIT_ATTN_SCHED_STREAMK, DIT_ATTN_SCHED_TILE)

__all__ = [
    "DitAttnError", "attention", "attention_blocksparse", "quantize_e4m3", "dit_attn_fwd", "dit_attn_fwd_ex",
    "dit_attn_fwd_strided", "dit_attn_fwd_blocksparse", "dit_attn_quantize_e4m3", "DIT_ATTN_SPARSE_Q_BLOCK",
    "DIT_ATTN_SPARSE_KV_BLOCK", "attention_mx", "quantize_mx", "dit_attn_fwd_mx", "dit_attn_quantize_mx",
    "DIT_ATTN_MX_ALONG_D", "DIT_ATTN_MX_ALONG_TOKENS", "dit_attn_plan", "DitAttnPlan", "DIT_ATTN_SCHED_TILE",
    "DIT_ATTN_SCHED_SPLIT", "DIT_ATTN_SCHED_STREAMK",
    "dit_attn_strerror", "dit_attn_version", "DIT_ATTN_BF16", "DIT_ATTN_FP8_E4M3", "DIT_ATTN_OK",
    "DIT_ATTN_EINVAL", "DIT_ATTN_EUNSUPPORTED", "DIT_ATTN_EDEVICE", "DIT_ATTN_ELAUNCH",
]


class DitAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dit_attn_strerror(status)} (status {status})")


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def attention(q, k, v, scale: float | None = None, *, out=None, lse=None, descale=None, stream=None):
    """Dense non-causal attention of (B, H, N, d) device tensors.

    bf16 inputs (d in {64, 128}) or float8_e4m3fn inputs (d = 128, with an
    optional device float32 ``descale`` tensor [dq, dk, dv]). q, k and v may
    be strided views (e.g. of a (B, N, H, d) or (B, N, 3, H, d) buffer, seen
    as (B, H, N, d)) as long as d is contiguous and the three share strides;
    ``out`` (default: a new contiguous bf16 tensor) may be strided the same
    way. Returns the bf16 output; writes the natural-log row normaliser into
    ``lse`` (float32 (B, H, N), contiguous) when given. Runs on ``stream``
    (default: torch's current stream) without synchronising."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one (B, H, N, d) shape")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.bfloat16:
        dtype = DIT_ATTN_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dtype = DIT_ATTN_FP8_E4M3
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v):
        if not t.is_cuda or t.stride(3) != 1:
            raise ValueError("q, k, v must be device tensors with a contiguous last dimension")
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k, v must share strides")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_cuda or out.stride(3) != 1:
        raise ValueError("out must be a bf16 device tensor of q's shape with a contiguous last dimension")
    if lse is not None and (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 (B, H, N) tensor")
    if descale is not None and (descale.numel() != 3 or descale.dtype != torch.float32 or not descale.is_cuda):
        raise ValueError("descale must be a float32 device tensor of 3 elements")
    st = dit_attn_fwd_strided(q, k, v, out, B, H, N, d, float(scale), dtype, q.stride()[:3], out.stride()[:3],
                              descale, lse, _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_fwd_strided")
    return out


def attention_blocksparse(q, k, v, kv_blocks, kv_counts, scale: float | None = None, *, out=None, lse=None,
                          stream=None):
    """Attention in which each block of 256 queries visits only listed blocks of 64 keys.

    q, k, v: bf16 (B, H, N, 128) device tensors, strided as for ``attention``.
    kv_counts: int32 device tensor (B, H, ceil(N / 256)), the number of key
    blocks listed for each query block; kv_blocks: int32 device tensor
    (B, H, ceil(N / 256), max_blocks) whose first count entries per row are
    strictly increasing key-block indices in [0, ceil(N / 64)). An empty list
    gives zero output rows (and -inf in ``lse``)."""
    import torch
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one (B, H, N, d) shape")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("block-sparse attention takes bf16 q, k, v")
    for t in (q, k, v):
        if not t.is_cuda or t.stride(3) != 1:
            raise ValueError("q, k, v must be device tensors with a contiguous last dimension")
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k, v must share strides")
    B, H, N, d = q.shape
    nq = -(-N // DIT_ATTN_SPARSE_Q_BLOCK)
    if (kv_counts.shape != (B, H, nq) or kv_counts.dtype != torch.int32 or not kv_counts.is_contiguous()
            or not kv_counts.is_cuda):
        raise ValueError(f"kv_counts must be a contiguous int32 device tensor of shape {(B, H, nq)}")
    if (kv_blocks.dim() != 4 or kv_blocks.shape[:3] != (B, H, nq) or kv_blocks.dtype != torch.int32
            or not kv_blocks.is_contiguous() or not kv_blocks.is_cuda):
        raise ValueError(f"kv_blocks must be a contiguous int32 device tensor of shape {(B, H, nq)} + (max_blocks,)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_cuda or out.stride(3) != 1:
        raise ValueError("out must be a bf16 device tensor of q's shape with a contiguous last dimension")
    if lse is not None and (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 (B, H, N) tensor")
    st = dit_attn_fwd_blocksparse(q, k, v, out, B, H, N, d, float(scale), DIT_ATTN_BF16, kv_blocks, kv_counts,
                                  kv_blocks.shape[3], q.stride()[:3], out.stride()[:3], lse,
                                  _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_fwd_blocksparse")
    return out


def quantize_mx(x, along: str, *, out=None, scales=None, stream=None):
    """Block-scaled e4m3 quantisation of a contiguous bf16 (B, H, N, d) device tensor.

    ``along`` is "d" (Q, K: scales (B, H, N, d/32)) or "tokens" (V: scales
    (B, H, ceil(N/32), 32, d/32)); returns (codes float8_e4m3fn, scales uint8)."""
    import torch
    if x.dim() != 4 or x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 (B, H, N, d) device tensor")
    B, H, N, d = x.shape
    if along == "d":
        ax, shape = DIT_ATTN_MX_ALONG_D, (B, H, N, d // 32)
    elif along == "tokens":
        ax, shape = DIT_ATTN_MX_ALONG_TOKENS, (B, H, -(-N // 32), 32, d // 32)
    else:
        raise ValueError('along must be "d" or "tokens"')
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if scales is None:
        scales = torch.empty(shape, dtype=torch.uint8, device=x.device)
    st = dit_attn_quantize_mx(x, B, H, N, d, ax, out, scales, _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_quantize_mx")
    return out, scales


def attention_mx(q8, q_scales, k8, k_scales, v8, v_scales, scale: float | None = None, *, out=None, lse=None,
                 stream=None):
    """Attention on block-scaled e4m3 inputs from ``quantize_mx`` (q, k along d, v along the tokens).

    Contiguous float8_e4m3fn (B, H, N, 128) device tensors; returns bf16 O."""
    import torch
    if q8.dim() != 4 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("q8, k8, v8 must share one (B, H, N, d) shape")
    for t in (q8, k8, v8):
        if t.dtype != torch.float8_e4m3fn or not t.is_cuda or not t.is_contiguous():
            raise ValueError("q8, k8, v8 must be contiguous float8_e4m3fn device tensors")
    B, H, N, d = q8.shape
    for t, shape in ((q_scales, (B, H, N, d // 32)), (k_scales, (B, H, N, d // 32)),
                     (v_scales, (B, H, -(-N // 32), 32, d // 32))):
        if tuple(t.shape) != shape or t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"scales must be contiguous uint8 device tensors of shape {shape}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    elif out.shape != q8.shape or out.dtype != torch.bfloat16 or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 device tensor of q8's shape")
    if lse is not None and (lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 (B, H, N) tensor")
    st = dit_attn_fwd_mx(q8, k8, v8, q_scales, k_scales, v_scales, out, B, H, N, d, float(scale), lse,
                         _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_fwd_mx")
    return out


def quantize_e4m3(x, *, out=None, descale=None, workspace=None, stream=None):
    """Per-tensor absmax quantisation of a bf16 device tensor to float8_e4m3fn.

    Returns (codes, descale) with ``descale`` a 1-element float32 device
    tensor holding 1/s. ``workspace`` is a 1-element int32 device tensor."""
    import torch
    if x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 device tensor")
    n = x.numel()
    if out is None:
        out = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device)
    if descale is None:
        descale = torch.empty(1, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(1, dtype=torch.int32, device=x.device)
    st = dit_attn_quantize_e4m3(x, n, out, descale, workspace, _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_quantize_e4m3")
    return out, descale

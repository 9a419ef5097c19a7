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
                   DIT_ATTN_EWORKSPACE, DIT_ATTN_NOALLOC_SCRATCH_BYTES, dit_attn_fwd_noalloc,
                   DIT_ATTN_MX_ALONG_D, DIT_ATTN_MX_ALONG_TOKENS, DIT_ATTN_OK, DIT_ATTN_SPARSE_KV_BLOCK,
                   DIT_ATTN_SPARSE_Q_BLOCK, DIT_ATTN_EUNSUPPORTED, dit_attn_fwd, dit_attn_fwd_blocksparse,
                   dit_attn_fwd_ex, dit_attn_fwd_mx, dit_attn_fwd_strided, dit_attn_mfma_ceiling, dit_attn_plan,
                   dit_attn_quantize_e4m3,
                   dit_attn_quantize_mx, dit_attn_strerror, dit_attn_version, DitAttnPlan, DIT_ATTN_SCHED_SPLIT,
                   DIT_ATTN_SCHED_STREAMK, DIT_ATTN_SCHED_TILE)

__all__ = [
    "DitAttnError", "attention", "attention_blocksparse", "quantize_e4m3", "dit_attn_fwd", "dit_attn_fwd_ex",
    "dit_attn_fwd_strided", "dit_attn_fwd_blocksparse", "dit_attn_quantize_e4m3", "DIT_ATTN_SPARSE_Q_BLOCK",
    "DIT_ATTN_SPARSE_KV_BLOCK", "attention_mx", "quantize_mx", "dit_attn_fwd_mx", "dit_attn_quantize_mx",
    "DIT_ATTN_MX_ALONG_D", "DIT_ATTN_MX_ALONG_TOKENS", "dit_attn_plan", "DitAttnPlan", "DIT_ATTN_SCHED_TILE",
    "DIT_ATTN_SCHED_SPLIT", "DIT_ATTN_SCHED_STREAMK",
    "dit_attn_strerror", "dit_attn_version", "DIT_ATTN_BF16", "DIT_ATTN_FP8_E4M3", "DIT_ATTN_OK",
    "DIT_ATTN_EINVAL", "DIT_ATTN_EUNSUPPORTED", "DIT_ATTN_EDEVICE", "DIT_ATTN_ELAUNCH", "DIT_ATTN_EWORKSPACE",
    "workspace_bytes", "dit_attn_fwd_noalloc", "DIT_ATTN_NOALLOC_SCRATCH_BYTES", "dit_attn_mfma_ceiling",
    "mfma_ceiling",
]


class DitAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {dit_attn_strerror(status)} (status {status})")


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check_buffer(t, name, shape, dtype, device, contiguous=True):
    """A caller-supplied buffer the kernels will read or write: a device
    tensor on ``device`` with this shape and dtype (contiguous unless the
    caller may pass a strided view). A host tensor's address would reach the
    kernels as a device pointer."""
    if t is None:
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a device tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(plan_args, workspace, device):
    """(workspace, bytes) for a call: the caller's uint8 device tensor, or a new
    one of the size dit_attn_plan asks for (allocated by torch; None if the
    fastest schedule needs none)."""
    import torch
    st, plan = dit_attn_plan(*plan_args)
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_plan")
    if workspace is None:
        if plan.workspace_wanted == 0:
            return None, 0
        workspace = torch.empty(plan.workspace_wanted, dtype=torch.uint8, device=device)
    elif (not workspace.is_cuda or workspace.device != device or workspace.dtype != torch.uint8
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 device tensor on the inputs' device")
    return workspace, workspace.numel()


def workspace_bytes(B, H, N, d, dtype=DIT_ATTN_BF16, *, lse=False, max_blocks=0) -> int:
    """Bytes of workspace the fastest schedule of a call of this shape uses on
    the current device (0 if it needs none)."""
    st, plan = dit_attn_plan(B, H, N, d, dtype, max_blocks, lse)
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_plan")
    return plan.workspace_wanted


def _check_qkv(q, k, v, dtypes):
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one (B, H, N, d) shape")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    if q.dtype not in dtypes:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v):
        if not t.is_cuda or t.stride(3) != 1:
            raise ValueError("q, k, v must be device tensors with a contiguous last dimension")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    if k.stride() != q.stride() or v.stride() != q.stride():
        raise ValueError("q, k, v must share strides")


def _output(out, q):
    import torch
    B, H, N, d = q.shape
    if out is None:
        return torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
    _check_buffer(out, "out", q.shape, torch.bfloat16, q.device, contiguous=False)
    if out.stride(3) != 1:
        raise ValueError("out must have a contiguous last dimension")
    return out


def attention(q, k, v, scale: float | None = None, *, out=None, lse=None, descale=None, workspace=None,
              stream=None):
    """Dense non-causal attention of (B, H, N, d) device tensors.

    bf16 inputs (d in {64, 128}) or float8_e4m3fn inputs (d = 128, with an
    optional device float32 ``descale`` tensor [dq, dk, dv]). q, k and v may
    be strided views (e.g. of a (B, N, H, d) or (B, N, 3, H, d) buffer, seen
    as (B, H, N, d)) as long as d is contiguous and the three share strides;
    ``out`` (default: a new contiguous bf16 tensor) may be strided the same
    way. Returns the bf16 output; writes the natural-log row normaliser into
    ``lse`` (float32 (B, H, N), contiguous) when given. ``workspace``: a uint8
    device tensor of at least ``workspace_bytes(...)`` bytes; by default one
    is taken from torch's allocator when the shape's fastest schedule needs
    it. Runs on ``stream`` (default: torch's current stream) without
    synchronising."""
    import torch
    _check_qkv(q, k, v, (torch.bfloat16, torch.float8_e4m3fn))
    dtype = DIT_ATTN_BF16 if q.dtype == torch.bfloat16 else DIT_ATTN_FP8_E4M3
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _output(out, q)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    _check_buffer(descale, "descale", (3,), torch.float32, q.device)
    ws, ws_bytes = _workspace((B, H, N, d, dtype, 0, lse is not None), workspace, q.device)
    st = dit_attn_fwd_strided(q, k, v, out, B, H, N, d, float(scale), dtype, q.stride()[:3], out.stride()[:3],
                              descale, lse, ws, ws_bytes, _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_fwd_strided")
    return out


def attention_blocksparse(q, k, v, kv_blocks, kv_counts, scale: float | None = None, *, out=None, lse=None,
                          workspace=None, stream=None):
    """Attention in which each block of 256 queries visits only listed blocks of 64 keys.

    q, k, v: bf16 (B, H, N, 128) device tensors, strided as for ``attention``.
    kv_counts: int32 device tensor (B, H, ceil(N / 256)), the number of key
    blocks listed for each query block; kv_blocks: int32 device tensor
    (B, H, ceil(N / 256), max_blocks) whose first count entries per row are
    strictly increasing key-block indices in [0, ceil(N / 64)). An empty list
    gives zero output rows (and -inf in ``lse``)."""
    import torch
    _check_qkv(q, k, v, (torch.bfloat16,))
    B, H, N, d = q.shape
    nq = -(-N // DIT_ATTN_SPARSE_Q_BLOCK)
    _check_buffer(kv_counts, "kv_counts", (B, H, nq), torch.int32, q.device)
    if kv_blocks.dim() != 4:
        raise ValueError(f"kv_blocks must have shape {(B, H, nq)} + (max_blocks,)")
    _check_buffer(kv_blocks, "kv_blocks", (B, H, nq, kv_blocks.shape[3]), torch.int32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = _output(out, q)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q.device)
    mb = kv_blocks.shape[3]
    ws, ws_bytes = _workspace((B, H, N, d, DIT_ATTN_BF16, mb, lse is not None), workspace, q.device)
    st = dit_attn_fwd_blocksparse(q, k, v, out, B, H, N, d, float(scale), DIT_ATTN_BF16, kv_blocks, kv_counts, mb,
                                  q.stride()[:3], out.stride()[:3], lse, ws, ws_bytes, _stream_handle(stream))
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
    _check_buffer(out, "out", x.shape, torch.float8_e4m3fn, x.device)
    if scales is None:
        scales = torch.empty(shape, dtype=torch.uint8, device=x.device)
    _check_buffer(scales, "scales", shape, torch.uint8, x.device)
    st = dit_attn_quantize_mx(x, B, H, N, d, ax, out, scales, _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_quantize_mx")
    return out, scales


def attention_mx(q8, q_scales, k8, k_scales, v8, v_scales, scale: float | None = None, *, out=None, lse=None,
                 workspace=None, stream=None):
    """Attention on block-scaled e4m3 inputs from ``quantize_mx`` (q, k along d, v along the tokens).

    Contiguous float8_e4m3fn (B, H, N, 128) device tensors; returns bf16 O."""
    import torch
    if q8.dim() != 4 or k8.shape != q8.shape or v8.shape != q8.shape:
        raise ValueError("q8, k8, v8 must share one (B, H, N, d) shape")
    for t in (q8, k8, v8):
        if t.dtype != torch.float8_e4m3fn or not t.is_cuda or not t.is_contiguous() or t.device != q8.device:
            raise ValueError("q8, k8, v8 must be contiguous float8_e4m3fn tensors on one device")
    B, H, N, d = q8.shape
    for t, nm, shape in ((q_scales, "q_scales", (B, H, N, d // 32)), (k_scales, "k_scales", (B, H, N, d // 32)),
                         (v_scales, "v_scales", (B, H, -(-N // 32), 32, d // 32))):
        if t is None:
            raise ValueError(f"{nm} is required")
        _check_buffer(t, nm, shape, torch.uint8, q8.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    _check_buffer(out, "out", q8.shape, torch.bfloat16, q8.device)
    _check_buffer(lse, "lse", (B, H, N), torch.float32, q8.device)
    ws, ws_bytes = _workspace((B, H, N, d, DIT_ATTN_FP8_E4M3, 0, lse is not None), workspace, q8.device)
    st = dit_attn_fwd_mx(q8, k8, v8, q_scales, k_scales, v_scales, out, B, H, N, d, float(scale), lse, ws, ws_bytes,
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
    _check_buffer(out, "out", x.shape, torch.float8_e4m3fn, x.device)
    if descale is None:
        descale = torch.empty(1, dtype=torch.float32, device=x.device)
    _check_buffer(descale, "descale", (1,), torch.float32, x.device)
    if workspace is None:
        workspace = torch.empty(1, dtype=torch.int32, device=x.device)
    _check_buffer(workspace, "workspace", (1,), torch.int32, x.device)
    st = dit_attn_quantize_e4m3(x, n, out, descale, workspace, _stream_handle(stream))
    if st != DIT_ATTN_OK:
        raise DitAttnError(st, "dit_attn_quantize_e4m3")
    return out, descale


def mfma_ceiling(dtype=DIT_ATTN_BF16, *, rounds=20000, reps=3, device=None):
    """The matrix-core rate the current card sustains on attention-like
    operands (dit_attn_mfma_ceiling): one warm-up launch, then ``reps`` timed
    launches on the current stream. Returns a dict with ``tflops`` (median
    launch), ``clock_mhz`` (shader clock over the product loops of that
    launch) and ``cycles_per_product`` (32 for bf16, 64 for e4m3 when the
    matrix cores never wait)."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    n_wg = torch.cuda.get_device_properties(dev).multi_processor_count
    record = torch.zeros(n_wg * 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    flop = n_wg * 4 * rounds * 16 * (32 * 32 * 64 * 2 if dtype == DIT_ATTN_FP8_E4M3 else 32 * 32 * 16 * 2)
    runs = []
    for i in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st, khz = dit_attn_mfma_ceiling(dtype, rounds, n_wg, record, record.numel() * 8, stream.cuda_stream)
        e1.record(stream)
        if st != DIT_ATTN_OK:
            raise DitAttnError(st, "dit_attn_mfma_ceiling")
        stream.synchronize()
        if i == 0:
            continue
        rec = record.view(-1, 2).double()
        cycles, ticks = rec[:, 0].sum().item(), rec[:, 1].sum().item()
        ms = e0.elapsed_time(e1)
        runs.append((flop / (ms * 1e-3) / 1e12, cycles / ticks * khz / 1000.0,
                     cycles / (n_wg * 4) / (rounds * 16)))
    runs.sort()
    tflops, mhz, cpp = runs[len(runs) // 2]
    return {"tflops": round(tflops, 1), "clock_mhz": round(mhz, 0), "cycles_per_product": round(cpp, 2),
            "rounds": rounds, "workgroups": n_wg}

"""ctypes binding of libditattn.so: the C entry points under the same names.

Argument marshalling only. Every step of the attention runs in the HIP
kernels behind the C ABI; nothing here computes. If the shared library is
missing the import of this module fails loudly: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libditattn.so")

DIT_ATTN_BF16 = 0
DIT_ATTN_FP8_E4M3 = 1
DIT_ATTN_OK = 0
DIT_ATTN_EINVAL = -1
DIT_ATTN_EUNSUPPORTED = -2
DIT_ATTN_EDEVICE = -3
DIT_ATTN_ELAUNCH = -4
DIT_ATTN_EWORKSPACE = -5

DIT_ATTN_SPARSE_Q_BLOCK = 256
DIT_ATTN_SPARSE_KV_BLOCK = 64
DIT_ATTN_MX_ALONG_D = 0
DIT_ATTN_MX_ALONG_TOKENS = 1

DIT_ATTN_SCHED_TILE = 0
DIT_ATTN_SCHED_SPLIT = 1
DIT_ATTN_SCHED_STREAMK = 2

DIT_ATTN_NOALLOC_SCRATCH_BYTES = 68157440

EXPORTED = ("dit_attn_fwd", "dit_attn_fwd_blocksparse", "dit_attn_fwd_ex", "dit_attn_fwd_mx", "dit_attn_fwd_noalloc",
            "dit_attn_fwd_strided", "dit_attn_mfma_ceiling",
            "dit_attn_plan", "dit_attn_quantize_e4m3", "dit_attn_quantize_mx", "dit_attn_strerror",
            "dit_attn_version")


class DitAttnPlan(ctypes.Structure):
    """dit_attn_plan_t."""
    _fields_ = [("schedule", ctypes.c_int32), ("workgroups", ctypes.c_int32), ("parts", ctypes.c_int32),
                ("split_tiles", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64),
                ("workspace_wanted", ctypes.c_int64), ("best_schedule", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m diffusion_transformer_attention_non_amd.build` "
                      "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _f, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
_lib.dit_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp]
_lib.dit_attn_fwd.restype = _i
_lib.dit_attn_fwd_ex.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp]
_lib.dit_attn_fwd_ex.restype = _i
_lib.dit_attn_fwd_strided.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _vp, _vp, _i64,
                                      _vp]
_lib.dit_attn_fwd_strided.restype = _i
_lib.dit_attn_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _vp, _vp, _vp]
_lib.dit_attn_fwd_noalloc.restype = _i
_lib.dit_attn_fwd_blocksparse.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _vp, _i,
                                          _vp, _vp, _vp, _vp, _i64, _vp]
_lib.dit_attn_fwd_blocksparse.restype = _i
_lib.dit_attn_fwd_mx.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _vp, _vp, _i64, _vp]
_lib.dit_attn_fwd_mx.restype = _i
_lib.dit_attn_quantize_mx.argtypes = [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]
_lib.dit_attn_quantize_mx.restype = _i
_lib.dit_attn_plan.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _i64, ctypes.POINTER(DitAttnPlan)]
_lib.dit_attn_plan.restype = _i
_lib.dit_attn_quantize_e4m3.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp]
_lib.dit_attn_quantize_e4m3.restype = _i
_lib.dit_attn_strerror.argtypes = [_i]
_lib.dit_attn_strerror.restype = ctypes.c_char_p
_lib.dit_attn_mfma_ceiling.argtypes = [_i, _i, _i, _vp, _i64, ctypes.POINTER(ctypes.c_int), _vp]
_lib.dit_attn_mfma_ceiling.restype = _i
_lib.dit_attn_version.argtypes = []
_lib.dit_attn_version.restype = _i


def _ptr(x):
    """Raw device address of a tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def dit_attn_fwd(q, k, v, o, B, H, N, d, scale, dtype, stream=None) -> int:
    return _lib.dit_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, scale, dtype, _ptr(stream))


def dit_attn_fwd_ex(q, k, v, o, B, H, N, d, scale, dtype, descale_qkv=None, lse=None, stream=None) -> int:
    return _lib.dit_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, scale, dtype,
                                _ptr(descale_qkv), _ptr(lse), _ptr(stream))


def _strides3(s):
    """(ctypes array that must outlive the call, its address) or (None, None)."""
    if s is None:
        return None, None
    arr = (ctypes.c_int64 * 3)(*[int(x) for x in s])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def dit_attn_fwd_strided(q, k, v, o, B, H, N, d, scale, dtype, qkv_strides=None, o_strides=None,
                         descale_qkv=None, lse=None, workspace=None, workspace_bytes=0, stream=None) -> int:
    qs, qp = _strides3(qkv_strides)
    os_, op = _strides3(o_strides)
    return _lib.dit_attn_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, scale, dtype, qp, op,
                                     _ptr(descale_qkv), _ptr(lse), _ptr(workspace), int(workspace_bytes),
                                     _ptr(stream))


def dit_attn_fwd_noalloc(q, k, v, o, B, H, N, d, scale, dtype, qkv_strides=None, o_strides=None,
                         descale_qkv=None, lse=None, stream=None) -> int:
    qs, qp = _strides3(qkv_strides)
    os_, op = _strides3(o_strides)
    return _lib.dit_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, scale, dtype, qp, op,
                                     _ptr(descale_qkv), _ptr(lse), _ptr(stream))


def dit_attn_fwd_blocksparse(q, k, v, o, B, H, N, d, scale, dtype, kv_blocks, kv_counts, max_blocks,
                             qkv_strides=None, o_strides=None, lse=None, workspace=None, workspace_bytes=0,
                             stream=None) -> int:
    qs, qp = _strides3(qkv_strides)
    os_, op = _strides3(o_strides)
    return _lib.dit_attn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, N, d, scale, dtype,
                                         _ptr(kv_blocks), _ptr(kv_counts), max_blocks, qp, op, _ptr(lse),
                                         _ptr(workspace), int(workspace_bytes), _ptr(stream))


def dit_attn_fwd_mx(q8, k8, v8, q_scales, k_scales, v_scales, o, B, H, N, d, scale, lse=None, workspace=None,
                    workspace_bytes=0, stream=None) -> int:
    return _lib.dit_attn_fwd_mx(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scales), _ptr(k_scales), _ptr(v_scales), _ptr(o),
                                B, H, N, d, scale, _ptr(lse), _ptr(workspace), int(workspace_bytes), _ptr(stream))


def dit_attn_quantize_mx(x, B, H, N, d, along, x8, scales, stream=None) -> int:
    return _lib.dit_attn_quantize_mx(_ptr(x), B, H, N, d, along, _ptr(x8), _ptr(scales), _ptr(stream))


def dit_attn_plan(B, H, N, d, dtype, max_blocks=0, lse=False, n_cu=0, workspace_bytes=0):
    """Returns (status, DitAttnPlan)."""
    plan = DitAttnPlan()
    st = _lib.dit_attn_plan(B, H, N, d, dtype, max_blocks, 1 if lse else 0, n_cu, int(workspace_bytes),
                            ctypes.byref(plan))
    return st, plan


def dit_attn_quantize_e4m3(x, n, x8, descale, amax_ws, stream=None) -> int:
    return _lib.dit_attn_quantize_e4m3(_ptr(x), n, _ptr(x8), _ptr(descale), _ptr(amax_ws), _ptr(stream))


def dit_attn_strerror(status: int) -> str:
    return _lib.dit_attn_strerror(status).decode()


def dit_attn_version() -> int:
    return _lib.dit_attn_version()


def dit_attn_mfma_ceiling(dtype, rounds, workgroups, record, record_bytes, stream=None):
    """Returns (status, wall-clock tick rate in kHz)."""
    khz = ctypes.c_int(0)
    st = _lib.dit_attn_mfma_ceiling(dtype, rounds, workgroups, _ptr(record), int(record_bytes), ctypes.byref(khz),
                                    _ptr(stream))
    return st, khz.value

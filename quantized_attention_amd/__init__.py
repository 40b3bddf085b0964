"""MI355X-native quantized attention forward (SageAttention2 INT8-QK / FP8-PV method).

Thin Python binding over the C ABI of ``libsage_attn.so`` (declared in
``include/sage_attn.h``).  Every step of the computation runs in the library's HIP
kernels; this module only marshals arguments.  PyTorch, where used, supplies device
memory and the current stream.

The raw entry points take integers (device addresses, sizes) and return the library's
status code; ``sage_attn`` is the convenience wrapper over torch tensors.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "SAGE_OK", "SAGE_ERR_INVALID_ARG", "SAGE_ERR_UNSUPPORTED", "SAGE_ERR_NO_MEMORY",
    "SAGE_ERR_LAUNCH", "SAGE_ERR_DEVICE", "SAGE_PATH_I8F8", "SAGE_PATH_MXFP4", "SAGE_QK_FP8", "SAGE_MX_P_TWO_LEVEL", "SAGE_SMOOTH_V", "SAGE_IN_BF16",
    "SAGE_IN_FP16", "SAGE_OUT_SAME", "SAGE_OUT_FP32", "SAGE_ACC_VALU", "SAGE_BQ", "SAGE_BK", "SageError",
    "library_path", "load_library", "sage_attn_fwd", "sage_attn_fwd_ws",
    "sage_attn_workspace_bytes", "sage_attn_quantize", "sage_attn_status_string",
    "sage_attn_version", "sage_attn_set_profile_events", "sage_attn", "QuantViews",
    "SageAttnShape", "sage_attn_fwd_ex", "sage_attn_workspace_bytes_ex", "sage_attn_quantize_ex",
    "SageAttnVarlenShape", "sage_attn_varlen_workspace_bytes", "sage_attn_varlen_fwd", "sage_attn_varlen",
    "SAGE_TRAIN_NO_SMOOTH_K", "SAGE_TRAIN_RECOMPUTE_DS", "SAGE_TRAIN_KEEP_QUANT", "sage_attn_train_workspace_bytes", "sage_attn_train_fwd", "sage_attn_train_bwd",
    "sage_attn_train_forward", "sage_attn_train_backward", "SageBwdAttention",
    "SAGE_NOALLOC_MAX_BYTES", "sage_attn_fwd_noalloc",
]

SAGE_OK = 0
SAGE_ERR_INVALID_ARG = -1
SAGE_ERR_UNSUPPORTED = -2
SAGE_ERR_NO_MEMORY = -3
SAGE_ERR_LAUNCH = -4
SAGE_ERR_DEVICE = -5

SAGE_PATH_I8F8 = 0x0000
SAGE_PATH_MXFP4 = 0x0001
SAGE_QK_FP8 = 0x0002
SAGE_MX_P_TWO_LEVEL = 0x0004
SAGE_SMOOTH_V = 0x0010
SAGE_IN_BF16 = 0x0000
SAGE_IN_FP16 = 0x0100
SAGE_OUT_SAME = 0x0000
SAGE_OUT_FP32 = 0x1000
SAGE_ACC_VALU = 0x2000
SAGE_TRAIN_NO_SMOOTH_K = 0x4000
SAGE_TRAIN_RECOMPUTE_DS = 0x8000
SAGE_TRAIN_KEEP_QUANT = 0x10000

SAGE_BQ = 128
SAGE_BK = 64
SAGE_NOALLOC_MAX_BYTES = 128 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libsage_attn.so")
_lib = None


class SageError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {sage_attn_status_string(status)} (status {status})")
        self.status = status


class QuantViews(ctypes.Structure):
    """Mirror of ``sage_quant_views`` (device pointers; 0 skips a field)."""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q_hat", "k_hat", "v_hat", "dq", "dk", "dv", "k_mean", "v_mean", "q_mean", "delta_s",
                 "mx_scales_q", "mx_scales_k", "mx_scales_v")]


class SageAttnShape(ctypes.Structure):
    """Mirror of ``sage_attn_shape`` (the extended entry points' shape, grouped heads included)."""
    _fields_ = [("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("N", ctypes.c_int),
                ("M", ctypes.c_int), ("d", ctypes.c_int), ("causal", ctypes.c_int),
                ("sm_scale", ctypes.c_float), ("variant", ctypes.c_uint)]


class SageAttnVarlenShape(ctypes.Structure):
    """Mirror of ``sage_attn_varlen_shape`` (a packed batch of variable-length sequences)."""
    _fields_ = [("batch", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("d", ctypes.c_int),
                ("total_q", ctypes.c_int), ("total_k", ctypes.c_int), ("max_seqlen_q", ctypes.c_int),
                ("max_seqlen_k", ctypes.c_int), ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("causal", ctypes.c_int), ("sm_scale", ctypes.c_float), ("variant", ctypes.c_uint)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsage_attn.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m quantized_attention_amd.build` "
                           "(the quantized attention has no non-HIP implementation)")
    L = ctypes.CDLL(_LIB_PATH)
    P, i, u, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_float, ctypes.c_size_t
    L.sage_attn_fwd.argtypes = [P, P, P, P, i, i, i, i, i, i, f, u, P]
    L.sage_attn_fwd.restype = i
    L.sage_attn_fwd_ws.argtypes = [P, P, P, P, i, i, i, i, i, i, f, u, P, sz, P]
    L.sage_attn_fwd_ws.restype = i
    L.sage_attn_workspace_bytes.argtypes = [i, i, i, i, i, i, u]
    L.sage_attn_workspace_bytes.restype = sz
    L.sage_attn_quantize.argtypes = [P, P, P, i, i, i, i, i, i, u, ctypes.POINTER(QuantViews), P]
    L.sage_attn_quantize.restype = i
    L.sage_attn_status_string.argtypes = [i]
    L.sage_attn_status_string.restype = ctypes.c_char_p
    L.sage_attn_set_profile_events.argtypes = [P, P]
    L.sage_attn_set_profile_events.restype = None
    L.sage_attn_version.argtypes = []
    L.sage_attn_version.restype = i
    SP = ctypes.POINTER(SageAttnShape)
    L.sage_attn_workspace_bytes_ex.argtypes = [SP]
    L.sage_attn_workspace_bytes_ex.restype = sz
    L.sage_attn_fwd_ex.argtypes = [SP, P, P, P, P, P, sz, P]
    L.sage_attn_fwd_ex.restype = i
    L.sage_attn_quantize_ex.argtypes = [SP, P, P, P, ctypes.POINTER(QuantViews), P]
    L.sage_attn_quantize_ex.restype = i
    VP = ctypes.POINTER(SageAttnVarlenShape)
    L.sage_attn_varlen_workspace_bytes.argtypes = [VP]
    L.sage_attn_varlen_workspace_bytes.restype = sz
    L.sage_attn_varlen_fwd.argtypes = [VP, P, P, P, P, P, sz, P]
    L.sage_attn_varlen_fwd.restype = i
    L.sage_attn_fwd_noalloc.argtypes = [SP, P, P, P, P, P]
    L.sage_attn_fwd_noalloc.restype = i
    L.sage_attn_train_workspace_bytes.argtypes = [SP]
    L.sage_attn_train_workspace_bytes.restype = sz
    L.sage_attn_train_fwd.argtypes = [SP, P, P, P, P, P, P, sz, P]
    L.sage_attn_train_fwd.restype = i
    L.sage_attn_train_bwd.argtypes = [SP, P, P, P, P, P, P, P, P, P, P, sz, P]
    L.sage_attn_train_bwd.restype = i
    _lib = L
    return L


# ---------------------------------------------------------------- raw C ABI (same names)
def sage_attn_fwd(q, k, v, out, B, H, N, M, d, causal, sm_scale, variant, stream) -> int:
    return load_library().sage_attn_fwd(q, k, v, out, B, H, N, M, d, int(causal), float(sm_scale),
                                        variant, stream)


def sage_attn_fwd_ws(q, k, v, out, B, H, N, M, d, causal, sm_scale, variant, workspace, ws_bytes,
                     stream) -> int:
    return load_library().sage_attn_fwd_ws(q, k, v, out, B, H, N, M, d, int(causal), float(sm_scale),
                                           variant, workspace, ws_bytes, stream)


def sage_attn_workspace_bytes(B, H, N, M, d, causal, variant) -> int:
    return load_library().sage_attn_workspace_bytes(B, H, N, M, d, int(causal), variant)


def sage_attn_quantize(q, k, v, B, H, N, M, d, causal, variant, views: QuantViews, stream) -> int:
    return load_library().sage_attn_quantize(q, k, v, B, H, N, M, d, int(causal), variant,
                                             ctypes.byref(views), stream)


def _shape_ptr(shape):
    return ctypes.byref(shape) if shape is not None else None


def sage_attn_workspace_bytes_ex(shape) -> int:
    return load_library().sage_attn_workspace_bytes_ex(_shape_ptr(shape))


def sage_attn_fwd_ex(shape, q, k, v, out, workspace, ws_bytes, stream) -> int:
    return load_library().sage_attn_fwd_ex(_shape_ptr(shape), q, k, v, out, workspace, ws_bytes, stream)


def sage_attn_quantize_ex(shape, q, k, v, views: QuantViews, stream) -> int:
    return load_library().sage_attn_quantize_ex(_shape_ptr(shape), q, k, v, ctypes.byref(views), stream)


def sage_attn_varlen_workspace_bytes(shape) -> int:
    return load_library().sage_attn_varlen_workspace_bytes(_shape_ptr(shape))


def sage_attn_varlen_fwd(shape, q, k, v, out, workspace, ws_bytes, stream) -> int:
    return load_library().sage_attn_varlen_fwd(_shape_ptr(shape), q, k, v, out, workspace, ws_bytes, stream)


def sage_attn_fwd_noalloc(shape, q, k, v, out, stream) -> int:
    return load_library().sage_attn_fwd_noalloc(_shape_ptr(shape), q, k, v, out, stream)


def sage_attn_train_workspace_bytes(shape) -> int:
    return load_library().sage_attn_train_workspace_bytes(_shape_ptr(shape))


def sage_attn_train_fwd(shape, q, k, v, out, lse, workspace, ws_bytes, stream) -> int:
    return load_library().sage_attn_train_fwd(_shape_ptr(shape), q, k, v, out, lse, workspace, ws_bytes, stream)


def sage_attn_train_bwd(shape, q, k, v, out, dout, lse, dq, dk, dv, workspace, ws_bytes, stream) -> int:
    return load_library().sage_attn_train_bwd(_shape_ptr(shape), q, k, v, out, dout, lse, dq, dk, dv, workspace,
                                              ws_bytes, stream)


def sage_attn_set_profile_events(start, stop) -> None:
    load_library().sage_attn_set_profile_events(start, stop)


def sage_attn_status_string(status: int) -> str:
    try:
        return load_library().sage_attn_status_string(status).decode()
    except RuntimeError:
        return f"status {status}"


def sage_attn_version() -> int:
    return load_library().sage_attn_version()


# ---------------------------------------------------------------- torch convenience
def _check_out(out, shape, dtype):
    """A caller's output buffer must be exactly what the library writes (shape and dtype)."""
    if tuple(out.shape) != tuple(shape) or out.dtype != dtype:
        raise ValueError(f"out must be {tuple(shape)} of {dtype}, got {tuple(out.shape)} of {out.dtype}")


def _check_device(ts, device):
    """Every tensor the library reads or writes: contiguous, on the GPU, on q's device."""
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.device != device:
            raise ValueError("tensors must be contiguous device tensors on q's device")


def _variant_for(q, smooth_v: bool, out_fp32: bool, acc_valu: bool = False, mxfp4: bool = False,
                 qk_fp8: bool = False, mx_p_two_level: bool = False) -> int:
    import torch
    if q.dtype == torch.bfloat16:
        var = SAGE_IN_BF16
    elif q.dtype == torch.float16:
        var = SAGE_IN_FP16
    else:
        raise TypeError(f"q, k, v must be bf16 or fp16, got {q.dtype}")
    if smooth_v:
        var |= SAGE_SMOOTH_V
    if out_fp32:
        var |= SAGE_OUT_FP32
    if acc_valu:
        var |= SAGE_ACC_VALU
    if mxfp4:
        var |= SAGE_PATH_MXFP4
    if qk_fp8:
        var |= SAGE_QK_FP8
    if mx_p_two_level:
        var |= SAGE_MX_P_TWO_LEVEL
    return var


def sage_attn(q, k, v, causal: bool = False, sm_scale: float | None = None, smooth_v: bool = False,
              out_fp32: bool = False, out=None, acc_valu: bool = False, mxfp4: bool = False,
              qk_fp8: bool = False, mx_p_two_level: bool = False):
    """softmax(Q K^T * sm_scale) V with the quantized method, for [B, H, N, d] tensors.

    q: [B, H, N, d], k/v: [B, Hkv, M, d] (Hkv divides H: query head h reads key/value head
    h // (H // Hkv)), all the same dtype (bf16/fp16), contiguous, on the current device.  causal: False/0 none, True/1 key t visible to query r iff t <= r, 2 iff
    t <= r + M - N (queries are the last N of M tokens).  Returns out [B, H, N, d] in the
    input dtype (FP32 with out_fp32).
    mxfp4 selects the MXFP4 variant (E2M1 operands with E8M0 block scales); qk_fp8 quantizes
    Q and K to E4M3 instead of INT8 (same groups, scale amax / 448); mx_p_two_level (with
    mxfp4) divides each row of a tile's P~ by rowmax / 6 before its E2M1 quantization.
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, T, d]")
    B, H, N, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, M, d) or tuple(v.shape) != (B, Hkv, M, d):
        raise ValueError("k and v must be [B, Hkv, M, d] matching q")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the query heads must be a multiple of the key/value heads")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    out_dtype = torch.float32 if out_fp32 else q.dtype
    if out is not None:
        _check_out(out, (B, H, N, d), out_dtype)
    _check_device((q, k, v) if out is None else (q, k, v, out), q.device)
    var = _variant_for(q, smooth_v, out_fp32, acc_valu, mxfp4, qk_fp8, mx_p_two_level)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    scale = float(sm_scale) if sm_scale is not None else 1.0 / math.sqrt(d)
    shape = SageAttnShape(B, H, Hkv, N, M, d, int(causal), scale, var)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = sage_attn_fwd_ex(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None, 0, stream)
    if rc != SAGE_OK:
        raise SageError(rc, "sage_attn_fwd_ex")
    return out


def sage_attn_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, causal: int = 0,
                     sm_scale: float | None = None, smooth_v: bool = False, out_fp32: bool = False, out=None,
                     mxfp4: bool = False, qk_fp8: bool = False):
    """The forward of a packed batch of variable-length sequences.

    q: [total_q, Hq, d], k/v: [total_k, Hkv, d] (same bf16/fp16 dtype, contiguous, on the
    device); cu_seqlens_q / cu_seqlens_k: int32 device tensors of batch + 1 offsets;
    max_seqlen_*: bounds on the sequence lengths.  Each sequence is computed as ``sage_attn``
    computes it alone; rows that see no key are 0.  Returns out [total_q, Hq, d].
    """
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [total, H, d]")
    total_q, H, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if tuple(k.shape) != (total_k, Hkv, d) or tuple(v.shape) != (total_k, Hkv, d):
        raise ValueError("k and v must be [total_k, Hkv, d] matching q")
    if Hkv < 1 or H % Hkv:
        raise ValueError("the query heads must be a multiple of the key/value heads")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1:
            raise ValueError("cu_seqlens must be int32 vectors")
    batch = cu_seqlens_q.numel() - 1
    if batch < 1 or cu_seqlens_k.numel() != batch + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold batch + 1 offsets")
    out_dtype = torch.float32 if out_fp32 else q.dtype
    if out is not None:
        _check_out(out, (total_q, H, d), out_dtype)
    _check_device((q, k, v, cu_seqlens_q, cu_seqlens_k) + (() if out is None else (out,)), q.device)
    var = _variant_for(q, smooth_v, out_fp32, False, mxfp4, qk_fp8)
    if out is None:
        out = torch.empty((total_q, H, d), dtype=out_dtype, device=q.device)
    scale = float(sm_scale) if sm_scale is not None else 1.0 / math.sqrt(d)
    shape = SageAttnVarlenShape(batch, H, Hkv, d, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k),
                                cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), int(causal), scale, var)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = sage_attn_varlen_fwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None, 0,
                                  stream)
    if rc != SAGE_OK:
        raise SageError(rc, "sage_attn_varlen_fwd")
    return out


# ---------------------------------------------------------------- SageBwd (training)
def _train_shape(q, k, v, causal, sm_scale, out_fp32, smooth_k, recompute_ds=False, keep=False):
    """The SageBwd shape of q [B, H, N, d] and k, v [B, Hkv, M, d]; shapes are checked here so
    that no mismatched buffer reaches the kernels (the library itself rejects Hkv != H)."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, T, d]")
    B, H, N, d = q.shape
    Hkv, M = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, M, d) or tuple(v.shape) != (B, Hkv, M, d):
        raise ValueError("k and v must be [B, H, M, d] matching q")
    if Hkv != H:
        raise ValueError("SageBwd needs as many key/value heads as query heads (grouped heads are not served)")
    var = (SAGE_IN_FP16 if q.dtype == torch.float16 else SAGE_IN_BF16) | (SAGE_OUT_FP32 if out_fp32 else 0)
    if not smooth_k:
        var |= SAGE_TRAIN_NO_SMOOTH_K
    if recompute_ds:
        var |= SAGE_TRAIN_RECOMPUTE_DS
    if keep:
        var |= SAGE_TRAIN_KEEP_QUANT
    scale = float(sm_scale) if sm_scale is not None else 1.0 / math.sqrt(d)
    return SageAttnShape(B, H, Hkv, N, M, d, int(causal), scale, var)


def _check_train_inputs(*ts):
    import torch
    for t in ts:
        if t.dtype not in (torch.bfloat16, torch.float16):
            raise TypeError("q, k, v, dout must be bf16 or fp16")
    if len({t.dtype for t in ts}) != 1:
        raise TypeError("q, k, v, dout must share a dtype")
    _check_device(ts, ts[0].device)


def _train_context(shape, device):
    """A workspace for one training step's two calls (SAGE_TRAIN_KEEP_QUANT): a uint8 tensor and its
    256-byte aligned pointer and size."""
    import torch
    n = sage_attn_train_workspace_bytes(shape)
    if n == 0:
        raise SageError(SAGE_ERR_INVALID_ARG, "sage_attn_train_workspace_bytes")
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    return ws, (ws.data_ptr() + 255) // 256 * 256, n


def sage_attn_train_forward(q, k, v, causal: int = 0, sm_scale: float | None = None, out_fp32: bool = False,
                            smooth_k: bool = True, keep: bool = False):
    """SageBwd forward: (out [B, H, N, d], lse [B, H, N] FP32) for q [B, H, N, d], k/v [B, H, M, d].
    keep: also return a context (a device workspace holding the INT8 Q, K, V) for
    sage_attn_train_backward(ctx=...), which then does not quantize q, k, v again
    (SAGE_TRAIN_KEEP_QUANT); q, k, v must not change in between."""
    import torch
    shape = _train_shape(q, k, v, causal, sm_scale, out_fp32, smooth_k, keep=keep)
    _check_train_inputs(q, k, v)
    B, H, N, d = q.shape
    out = torch.empty((B, H, N, d), dtype=torch.float32 if out_fp32 else q.dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ctx = _train_context(shape, q.device) if keep else None
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = sage_attn_train_fwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 ctx[1] if keep else None, ctx[2] if keep else 0, stream)
    if rc != SAGE_OK:
        raise SageError(rc, "sage_attn_train_fwd")
    return (out, lse, ctx) if keep else (out, lse)


def sage_attn_train_backward(q, k, v, out, dout, lse, causal: int = 0, sm_scale: float | None = None,
                             smooth_k: bool = True, recompute_ds: bool = False, ctx=None):
    """SageBwd backward: (dq, dk, dv) in FP32, from the forward's out (its dtype) and lse.
    recompute_ds: the dQ kernel recomputes dS instead of reading the dK/dV kernel's stored dS^
    codes (SAGE_TRAIN_RECOMPUTE_DS: slower, with a small workspace).  ctx: the context of
    sage_attn_train_forward(keep=True) on the same q, k, v (same causal, sm_scale, smooth_k and
    recompute_ds); the quantized inputs are then taken from it."""
    import torch
    keep = ctx is not None
    shape = _train_shape(q, k, v, causal, sm_scale, out.dtype == torch.float32, smooth_k, recompute_ds, keep)
    B, H, N, d = q.shape
    if tuple(dout.shape) != (B, H, N, d) or tuple(out.shape) != (B, H, N, d):
        raise ValueError("out and dout must be [B, H, N, d] like q")
    if out.dtype not in (q.dtype, torch.float32):
        raise TypeError("out must have q's dtype or float32 (the forward's output)")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 [B, H, N]")
    _check_train_inputs(q, k, v, dout)
    _check_device((out, lse), q.device)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    if keep and (ctx[0].device != q.device or ctx[2] < sage_attn_train_workspace_bytes(shape)):
        raise ValueError("ctx comes from a forward of another shape or device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = sage_attn_train_bwd(shape, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 ctx[1] if keep else None, ctx[2] if keep else 0, stream)
    if rc != SAGE_OK:
        raise SageError(rc, "sage_attn_train_bwd")
    return dq, dk, dv


def _sagebwd_function():
    import torch

    class SageBwdAttention(torch.autograd.Function):
        """softmax(Q K^T sm_scale) V with SageBwd's INT8 forward and backward, as a torch op.

        apply(q, k, v, causal=0, sm_scale=None); gradients come back in the input dtype."""

        @staticmethod
        def forward(ctx, q, k, v, causal=0, sm_scale=None):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            # the backward quantizes q, k, v again: holding the forward's workspace (the INT8 inputs
            # and, behind them, room for the backward's pair buffer) from each layer's forward to its
            # backward would cost more memory than the quantization costs time
            out, lse = sage_attn_train_forward(q, k, v, causal, sm_scale)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.causal, ctx.sm_scale = causal, sm_scale
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            dq, dk, dv = sage_attn_train_backward(q, k, v, out, dout.contiguous().to(q.dtype), lse, ctx.causal,
                                                  ctx.sm_scale)
            return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None

    return SageBwdAttention


def __getattr__(name):
    if name == "SageBwdAttention":
        return _sagebwd_function()
    raise AttributeError(name)

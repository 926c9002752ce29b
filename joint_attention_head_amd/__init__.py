"""Python binding of libfluxattn (FLUX joint-attention hot path on MI355X).

Thin ctypes layer: it checks dtypes, shapes and devices, allocates outputs
with torch when the caller passes none, and hands raw device pointers and the
current HIP stream to the C ABI declared in include/fluxattn.h.  All
arithmetic happens in the library's HIP kernels; there is no fallback, and
every entry point raises FluxAttnError when the library is missing or a call
is rejected.

Entry points (same names as the C ABI):
    fluxattn_qk_norm_rope_bf16(q, k, q_norm_w, k_norm_w, pos_ids, ...)
    fluxattn_qk_norm_rope_fp8(q, k, q_scale, k_scale, q_norm_w, k_norm_w, pos_ids, ...)
    fluxattn_forward_bf16(q, k, v, ...)
    fluxattn_forward_fp8(q, k, v, q_scale, k_scale, v_scale, ...)
    fluxattn_forward_fused_bf16(q, k, v, q_norm_w, pos_ids, ...)
    fluxattn_forward_fused_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, pos_ids, ...)
    fluxattn_joint_attention_bf16(q, k, v, q_norm_w, k_norm_w, pos_ids, ...)
    fluxattn_joint_attention_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, k_norm_w, pos_ids, ...)
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfluxattn.so")

HEAD_DIM = 128
ROPE_AXES = (16, 56, 56)
ROPE_THETA = 1e4
RMS_EPS = 1e-6

STATUS = {
    0: "FLUXATTN_OK",
    1: "FLUXATTN_ERR_NULL_POINTER",
    2: "FLUXATTN_ERR_INVALID_SHAPE",
    3: "FLUXATTN_ERR_MISALIGNED",
    4: "FLUXATTN_ERR_ALIASING",
    5: "FLUXATTN_ERR_NO_DEVICE",
    6: "FLUXATTN_ERR_HIP",
}

EXPORTS = (
    "fluxattn_qk_norm_rope_bf16",
    "fluxattn_qk_norm_rope_fp8",
    "fluxattn_forward_bf16",
    "fluxattn_forward_fp8",
    "fluxattn_forward_fused_bf16",
    "fluxattn_forward_fused_fp8",
    "fluxattn_joint_attention_bf16",
    "fluxattn_joint_attention_fp8",
    "fluxattn_status_string",
    "fluxattn_last_hip_error",
    "fluxattn_version",
)


class FluxAttnError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        self.status = status
        name = STATUS.get(status, f"status {status}")
        super().__init__(f"{name}{': ' + msg if msg else ''}")


_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f = ctypes.c_float

_SIGS = {
    "fluxattn_qk_norm_rope_bf16": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64,
                                   _i32, _i32, _i32, _f, _f, _p],
    "fluxattn_qk_norm_rope_fp8": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64,
                                  _i32, _i32, _i32, _f, _f, _p],
    "fluxattn_forward_bf16": [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p],
    "fluxattn_forward_fp8": [_p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _f, _p],
    "fluxattn_forward_fused_bf16": [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32, _i32,
                                    _f, _f, _f, _p],
    "fluxattn_forward_fused_fp8": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _i32,
                                   _i32, _f, _f, _f, _p],
    "fluxattn_joint_attention_bf16": [_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64,
                                      _i32, _i32, _i32, _f, _f, _f, _p],
    "fluxattn_joint_attention_fp8": [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                     _i64, _i32, _i32, _i32, _f, _f, _f, _p],
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises FluxAttnError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FluxAttnError(-1, f"{LIB_PATH} is missing; build it with "
                                    "`python -m joint_attention_head_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        l.fluxattn_status_string.argtypes = [ctypes.c_int]
        l.fluxattn_status_string.restype = ctypes.c_char_p
        l.fluxattn_last_hip_error.argtypes = []
        l.fluxattn_last_hip_error.restype = ctypes.c_int
        l.fluxattn_version.argtypes = []
        l.fluxattn_version.restype = ctypes.c_int
        _lib = l
    return _lib


def _check(status: int):
    if status != 0:
        l = lib()
        msg = l.fluxattn_status_string(status).decode()
        if status == 6:
            msg += f" (hipError_t {l.fluxattn_last_hip_error()})"
        raise FluxAttnError(status, msg)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _bhnd(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError(f"expected [B, H, N, D], got shape {tuple(q.shape)}")
    return tuple(q.shape)


def _ptr(t):
    return None if t is None else t.data_ptr()


def fluxattn_qk_norm_rope_bf16(q, k, q_norm_w, k_norm_w, pos_ids, q_out=None, k_out=None,
                               axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, stream=None):
    """RMSNorm + 3-axis RoPE of bf16 q, k [B,H,N,D]; returns (q_out, k_out).
    Pass q_out=q / k_out=k to work in place; q=None (with q_norm_w=None)
    processes the keys only and returns (None, k_out)."""
    B, H, N, D = _bhnd(k)
    _need(k, "k", torch.bfloat16)
    if q is not None:
        _need(q, "q", torch.bfloat16, k.shape)
        _need(q_norm_w, "q_norm_w", torch.float32, (D,))
        q_out = torch.empty_like(q) if q_out is None else q_out
        _need(q_out, "q_out", torch.bfloat16, k.shape)
    _need(k_norm_w, "k_norm_w", torch.float32, (D,))
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    k_out = torch.empty_like(k) if k_out is None else k_out
    _need(k_out, "k_out", torch.bfloat16, k.shape)
    _check(lib().fluxattn_qk_norm_rope_bf16(
        _ptr(q), k.data_ptr(), _ptr(q_out) if q is not None else None, k_out.data_ptr(),
        _ptr(q_norm_w) if q is not None else None, k_norm_w.data_ptr(), pos_ids.data_ptr(), B, H, N, D,
        axes[0], axes[1], axes[2], float(theta), float(eps), _stream(stream)))
    return (q_out if q is not None else None), k_out


def fluxattn_qk_norm_rope_fp8(q, k, q_scale, k_scale, q_norm_w, k_norm_w, pos_ids, q_out=None,
                              k_out=None, q_scale_out=None, k_scale_out=None, axes=ROPE_AXES,
                              theta=ROPE_THETA, eps=RMS_EPS, stream=None):
    """The prologue on float8_e4m3fn q, k with fp32 [B,H] scales; returns
    (q_out, k_out, q_scale_out, k_scale_out).  q=None (with q_scale and
    q_norm_w None) processes the keys only; the q entries are then None."""
    B, H, N, D = _bhnd(k)
    e4 = torch.float8_e4m3fn
    _need(k, "k", e4)
    _need(k_scale, "k_scale", torch.float32, (B, H))
    if q is not None:
        _need(q, "q", e4, k.shape)
        _need(q_scale, "q_scale", torch.float32, (B, H))
        _need(q_norm_w, "q_norm_w", torch.float32, (D,))
        q_out = torch.empty_like(q) if q_out is None else q_out
        q_scale_out = torch.empty_like(q_scale) if q_scale_out is None else q_scale_out
        _need(q_out, "q_out", e4, k.shape)
        _need(q_scale_out, "q_scale_out", torch.float32, (B, H))
    else:
        q_scale, q_out, q_scale_out, q_norm_w = None, None, None, None
    _need(k_norm_w, "k_norm_w", torch.float32, (D,))
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    k_out = torch.empty_like(k) if k_out is None else k_out
    k_scale_out = torch.empty_like(k_scale) if k_scale_out is None else k_scale_out
    _need(k_out, "k_out", e4, k.shape)
    _need(k_scale_out, "k_scale_out", torch.float32, (B, H))
    _check(lib().fluxattn_qk_norm_rope_fp8(
        _ptr(q), k.data_ptr(), _ptr(q_scale), k_scale.data_ptr(), _ptr(q_out), k_out.data_ptr(),
        _ptr(q_scale_out), k_scale_out.data_ptr(), _ptr(q_norm_w), k_norm_w.data_ptr(),
        pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta), float(eps),
        _stream(stream)))
    return q_out, k_out, q_scale_out, k_scale_out


def fluxattn_forward_bf16(q, k, v, o=None, softmax_scale=0.0, stream=None):
    """softmax(q k^T * scale) v over all tokens, bf16 [B,H,N,D]; returns o."""
    B, H, N, D = _bhnd(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, q.shape)
    o = torch.empty_like(q) if o is None else o
    _need(o, "o", torch.bfloat16, q.shape)
    _check(lib().fluxattn_forward_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       B, H, N, D, float(softmax_scale), _stream(stream)))
    return o


def fluxattn_forward_fp8(q, k, v, q_scale, k_scale, v_scale, o=None, softmax_scale=0.0, stream=None):
    """Joint attention on float8_e4m3fn q, k, v with fp32 [B,H] scales; bf16 o."""
    B, H, N, D = _bhnd(q)
    e4 = torch.float8_e4m3fn
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, e4, q.shape)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, (B, H))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    _need(o, "o", torch.bfloat16, q.shape)
    _check(lib().fluxattn_forward_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(),
                                      k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(),
                                      B, H, N, D, float(softmax_scale), _stream(stream)))
    return o


def joint_attention_bf16(q, k, v, q_norm_w, k_norm_w, pos_ids, axes=ROPE_AXES, theta=ROPE_THETA,
                         eps=RMS_EPS, stream=None):
    """Prologue then attention (the whole block) on bf16 inputs; returns o."""
    qn, kn = fluxattn_qk_norm_rope_bf16(q, k, q_norm_w, k_norm_w, pos_ids, axes=axes, theta=theta,
                                        eps=eps, stream=stream)
    return fluxattn_forward_bf16(qn, kn, v, stream=stream)


def joint_attention_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, k_norm_w, pos_ids,
                        axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, stream=None):
    """fp8 prologue then fp8 attention; returns bf16 o."""
    qn, kn, sq, sk = fluxattn_qk_norm_rope_fp8(q, k, q_scale, k_scale, q_norm_w, k_norm_w, pos_ids,
                                               axes=axes, theta=theta, eps=eps, stream=stream)
    return fluxattn_forward_fp8(qn, kn, v, sq, sk, v_scale, stream=stream)


def fluxattn_joint_attention_bf16(q, k, v, q_norm_w, k_norm_w, pos_ids, o=None, k_work=None,
                                  axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0,
                                  stream=None):
    """The whole block on raw bf16 q, k, v [B,H,N,D] in two launches: the
    keys' RMSNorm + RoPE into k_work (pass k_work=k to overwrite k), then
    attention that normalises and rotates the queries as it loads them.
    Returns o."""
    B, H, N, D = _bhnd(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, q.shape)
    _need(q_norm_w, "q_norm_w", torch.float32, (D,))
    _need(k_norm_w, "k_norm_w", torch.float32, (D,))
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty_like(q) if o is None else o
    k_work = torch.empty_like(k) if k_work is None else k_work
    _need(o, "o", torch.bfloat16, q.shape)
    _need(k_work, "k_work", torch.bfloat16, q.shape)
    _check(lib().fluxattn_joint_attention_bf16(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), k_work.data_ptr(), o.data_ptr(), q_norm_w.data_ptr(),
        k_norm_w.data_ptr(), pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta),
        float(eps), float(softmax_scale), _stream(stream)))
    return o


def fluxattn_joint_attention_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, k_norm_w, pos_ids,
                                 o=None, k_work=None, k_scale_work=None, axes=ROPE_AXES,
                                 theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0, stream=None):
    """The whole block on raw float8_e4m3fn q, k, v with fp32 [B,H] scales:
    the fp8 key prologue into (k_work, k_scale_work), then attention that
    normalises and rotates the queries as it loads them (kept in bf16).
    Returns bf16 o."""
    B, H, N, D = _bhnd(q)
    e4 = torch.float8_e4m3fn
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, e4, q.shape)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, (B, H))
    _need(q_norm_w, "q_norm_w", torch.float32, (D,))
    _need(k_norm_w, "k_norm_w", torch.float32, (D,))
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    k_work = torch.empty_like(k) if k_work is None else k_work
    k_scale_work = torch.empty_like(k_scale) if k_scale_work is None else k_scale_work
    _need(o, "o", torch.bfloat16, q.shape)
    _need(k_work, "k_work", e4, q.shape)
    _need(k_scale_work, "k_scale_work", torch.float32, (B, H))
    _check(lib().fluxattn_joint_attention_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), k_work.data_ptr(), k_scale_work.data_ptr(), o.data_ptr(),
        q_norm_w.data_ptr(), k_norm_w.data_ptr(), pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1],
        axes[2], float(theta), float(eps), float(softmax_scale), _stream(stream)))
    return o


def fluxattn_forward_fused_bf16(q, k, v, q_norm_w, pos_ids, o=None, axes=ROPE_AXES, theta=ROPE_THETA,
                                eps=RMS_EPS, softmax_scale=0.0, stream=None):
    """Attention on raw bf16 queries (RMSNorm + RoPE applied as they are
    loaded) against prepared keys k and values v; returns o."""
    B, H, N, D = _bhnd(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, torch.bfloat16, q.shape)
    _need(q_norm_w, "q_norm_w", torch.float32, (D,))
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty_like(q) if o is None else o
    _need(o, "o", torch.bfloat16, q.shape)
    _check(lib().fluxattn_forward_fused_bf16(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), q_norm_w.data_ptr(), pos_ids.data_ptr(),
        B, H, N, D, axes[0], axes[1], axes[2], float(theta), float(eps), float(softmax_scale),
        _stream(stream)))
    return o


def fluxattn_forward_fused_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, pos_ids, o=None,
                               axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0,
                               stream=None):
    """fp8 form of fluxattn_forward_fused_bf16 (E4M3 q raw, k prepared, v;
    fp32 [B,H] scales); returns bf16 o."""
    B, H, N, D = _bhnd(q)
    e4 = torch.float8_e4m3fn
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, e4, q.shape)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, (B, H))
    _need(q_norm_w, "q_norm_w", torch.float32, (D,))
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    _need(o, "o", torch.bfloat16, q.shape)
    _check(lib().fluxattn_forward_fused_fp8(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), o.data_ptr(), q_norm_w.data_ptr(), pos_ids.data_ptr(), B, H, N, D, axes[0],
        axes[1], axes[2], float(theta), float(eps), float(softmax_scale), _stream(stream)))
    return o

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
and the strided, multi-stream forms fluxattn_qk_norm_rope_ex_{bf16,fp8},
fluxattn_forward_ex_{bf16,fp8}, fluxattn_forward_fused_ex_{bf16,fp8} and
fluxattn_joint_attention_ex_{bf16,fp8}, which accept any [B,H,N,D] tensor
view whose last dimension is contiguous (for example q, k, v sliced out of a
packed [B,N,3,H,D] projection output) and per-stream norm weights [S, D]
with the streams' first tokens.  The attention _ex forms take an optional
key-range split (split=SplitWorkspace(...), see split_workspace()), whose
device workspace the binding allocates with torch, zeroed, like an output;
the library itself never allocates.
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
    7: "FLUXATTN_ERR_WORKSPACE",
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
    "fluxattn_qk_norm_rope_ex_bf16",
    "fluxattn_qk_norm_rope_ex_fp8",
    "fluxattn_forward_ex_bf16",
    "fluxattn_forward_ex_fp8",
    "fluxattn_joint_attention_ex_bf16",
    "fluxattn_joint_attention_ex_fp8",
    "fluxattn_forward_fused_ex_bf16",
    "fluxattn_forward_fused_ex_fp8",
    "fluxattn_split_workspace_bytes",
    "fluxattn_forward_fused_noalloc_bf16",
    "fluxattn_probe_mfma",
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



class Layout(ctypes.Structure):
    """fluxattn_layout: element strides of a [B,H,N,D] view (d contiguous)."""
    _fields_ = [("b_stride", ctypes.c_int64), ("h_stride", ctypes.c_int64), ("n_stride", ctypes.c_int64)]


class Streams(ctypes.Structure):
    """fluxattn_streams: 1..4 token streams given by their first tokens."""
    _fields_ = [("count", ctypes.c_int32), ("start", ctypes.c_int32 * 4)]


class Split(ctypes.Structure):
    """fluxattn_split: key-range split setting and the caller's workspace."""
    _fields_ = [("groups", ctypes.c_int32), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64)]


_L = Layout
_S = Streams
_SP = ctypes.POINTER(Split)

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
    "fluxattn_qk_norm_rope_ex_bf16": [_p, _L, _p, _L, _p, _L, _p, _L, _p, _p, _S, _p, _i64, _i64, _i64, _i64,
                                      _i32, _i32, _i32, _f, _f, _p],
    "fluxattn_qk_norm_rope_ex_fp8": [_p, _L, _p, _L, _p, _p, _p, _L, _p, _L, _p, _p, _p, _p, _S, _p, _i64, _i64,
                                     _i64, _i64, _i32, _i32, _i32, _f, _f, _p],
    "fluxattn_forward_ex_bf16": [_p, _L, _p, _L, _p, _L, _p, _L, _i64, _i64, _i64, _i64, _f, _SP, _p],
    "fluxattn_forward_ex_fp8": [_p, _L, _p, _L, _p, _L, _p, _p, _p, _p, _L, _i64, _i64, _i64, _i64, _f, _SP, _p],
    "fluxattn_forward_fused_ex_bf16": [_p, _L, _p, _L, _p, _L, _p, _L, _p, _S, _p, _i64, _i64, _i64, _i64,
                                       _i32, _i32, _i32, _f, _f, _f, _SP, _p],
    "fluxattn_forward_fused_ex_fp8": [_p, _L, _p, _L, _p, _L, _p, _p, _p, _p, _L, _p, _S, _p, _i64, _i64, _i64,
                                      _i64, _i32, _i32, _i32, _f, _f, _f, _SP, _p],
    "fluxattn_joint_attention_ex_bf16": [_p, _L, _p, _L, _p, _L, _p, _p, _L, _p, _p, _S, _p, _i64, _i64, _i64,
                                         _i64, _i32, _i32, _i32, _f, _f, _f, _SP, _p],
    "fluxattn_joint_attention_ex_fp8": [_p, _L, _p, _L, _p, _L, _p, _p, _p, _p, _p, _p, _L, _p, _p, _S, _p,
                                        _i64, _i64, _i64, _i64, _i32, _i32, _i32, _f, _f, _f, _SP, _p],
    "fluxattn_split_workspace_bytes": [_i64, _i64, _i64, _i64, _i32, ctypes.POINTER(ctypes.c_uint64)],
    "fluxattn_forward_fused_noalloc_bf16": [_p, _L, _p, _L, _p, _L, _p, _L, _p, _S, _p, _i64, _i64, _i64, _i64,
                                            _i32, _i32, _i32, _f, _f, _f, _i32, _p],
    "fluxattn_probe_mfma": [_i32, _i64, _i32, _p, ctypes.POINTER(ctypes.c_double), _p],
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
    normalises and rotates the queries as it loads them and re-encodes them
    in E4M3 per query.  Returns bf16 o."""
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


# ---- strided views and token streams


def fluxattn_split_workspace_bytes(B: int, H: int, N: int, groups: int = 0, D: int = HEAD_DIM) -> int:
    """Bytes of split workspace an attention launch over B*H heads of N
    tokens needs with this groups setting (0 when it would not be cut)."""
    n = ctypes.c_uint64(0)
    _check(lib().fluxattn_split_workspace_bytes(int(B), int(H), int(N), int(D), int(groups), ctypes.byref(n)))
    return int(n.value)


class SplitWorkspace:
    """A key-range split setting with its device workspace: `nbytes` zeroed
    bytes (torch memory of the binding, not of the library), reusable by any
    number of launches that do not overlap in time.  groups: 0 = one
    workgroup per compute unit, cut only where that balances the last round;
    > 0 = that many workgroups, always cut; < 0 = never cut."""

    def __init__(self, groups: int = 0, nbytes: int = 0, device=None):
        self.groups = int(groups)
        self.nbytes = int(nbytes)
        self.buffer = None
        if self.nbytes > 0:
            dev = torch.device("cuda") if device is None else torch.device(device)
            self.buffer = torch.zeros(self.nbytes, dtype=torch.uint8, device=dev)

    def as_struct(self) -> Split:
        ptr = None if self.buffer is None else self.buffer.data_ptr()
        return Split(self.groups, ptr, self.nbytes)

    def counts(self) -> torch.Tensor:
        """The arrival counts at the start of the workspace (int32), which
        every launch leaves at zero."""
        n = min(self.nbytes, 2 * 16384 * 4) // 4
        return self.buffer[:4 * n].view(torch.int32)


def split_workspace(B: int, H: int, N: int, groups: int = 0, device=None) -> SplitWorkspace:
    """A SplitWorkspace sized for attention over B*H heads of N tokens."""
    return SplitWorkspace(groups, fluxattn_split_workspace_bytes(B, H, N, groups), device)


def _split_arg(split):
    """ctypes argument of an optional split (None: the uncut launch)."""
    if split is None:
        return None
    if not isinstance(split, SplitWorkspace):
        raise TypeError("split must be a SplitWorkspace or None")
    return ctypes.byref(split.as_struct())


def layout_of(t: torch.Tensor) -> Layout:
    """The fluxattn_layout of a [B,H,N,D] tensor view (element strides)."""
    sb, sh, sn, sd = t.stride()
    if sd != 1 and t.shape[3] != 1:
        raise ValueError("the head dimension of a view must be contiguous")
    return Layout(sb, sh, sn)


def streams_of(starts) -> Streams:
    """fluxattn_streams from the first token of each stream, e.g. (0, 512)
    for 512 text tokens followed by the image tokens."""
    starts = [int(x) for x in starts]
    if not 1 <= len(starts) <= 4:
        raise ValueError("1 to 4 token streams")
    st = Streams()
    st.count = len(starts)
    for i, x in enumerate(starts):
        st.start[i] = x
    return st


def _need_view(t, name: str, dtype, shape):
    """Like _need for a strided [B,H,N,D] view; returns its layout."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return layout_of(t)


def _weights(w, name, n_streams, D):
    _need(w, name, torch.float32)
    if w.dim() == 1 and n_streams == 1:
        w = w.view(1, D)
    if tuple(w.shape) != (n_streams, D):
        raise ValueError(f"{name} must have shape ({n_streams}, {D}), got {tuple(w.shape)}")
    return w


def fluxattn_qk_norm_rope_ex_bf16(q, k, q_norm_w, k_norm_w, pos_ids, streams=(0,), q_out=None, k_out=None,
                                  axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, stream=None):
    """RMSNorm + RoPE of bf16 [B,H,N,D] views with one weight row per token
    stream (q_norm_w, k_norm_w: [S, D]; streams: the S first tokens).
    Outputs default to new contiguous tensors; pass q_out=q, k_out=k to work
    in place.  q=None processes the keys only.  Returns (q_out, k_out)."""
    shape = tuple(k.shape)
    B, H, N, D = _bhnd(k)
    st = streams_of(streams)
    lk = _need_view(k, "k", torch.bfloat16, shape)
    k_norm_w = _weights(k_norm_w, "k_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    k_out = torch.empty(shape, dtype=k.dtype, device=k.device) if k_out is None else k_out
    lko = _need_view(k_out, "k_out", torch.bfloat16, shape)
    lq = lqo = Layout(0, 0, 0)
    if q is not None:
        lq = _need_view(q, "q", torch.bfloat16, shape)
        q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
        q_out = torch.empty(shape, dtype=q.dtype, device=q.device) if q_out is None else q_out
        lqo = _need_view(q_out, "q_out", torch.bfloat16, shape)
    else:
        q_out, q_norm_w = None, None
    _check(lib().fluxattn_qk_norm_rope_ex_bf16(
        _ptr(q), lq, k.data_ptr(), lk, _ptr(q_out), lqo, k_out.data_ptr(), lko, _ptr(q_norm_w),
        k_norm_w.data_ptr(), st, pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta),
        float(eps), _stream(stream)))
    return q_out, k_out


def fluxattn_qk_norm_rope_ex_fp8(q, k, q_scale, k_scale, q_norm_w, k_norm_w, pos_ids, streams=(0,),
                                 q_out=None, k_out=None, q_scale_out=None, k_scale_out=None,
                                 axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, stream=None):
    """fp8 form of fluxattn_qk_norm_rope_ex_bf16; returns (q_out, k_out,
    q_scale_out, k_scale_out)."""
    shape = tuple(k.shape)
    B, H, N, D = _bhnd(k)
    e4 = torch.float8_e4m3fn
    st = streams_of(streams)
    lk = _need_view(k, "k", e4, shape)
    _need(k_scale, "k_scale", torch.float32, (B, H))
    k_norm_w = _weights(k_norm_w, "k_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    k_out = torch.empty(shape, dtype=e4, device=k.device) if k_out is None else k_out
    lko = _need_view(k_out, "k_out", e4, shape)
    k_scale_out = torch.empty_like(k_scale) if k_scale_out is None else k_scale_out
    _need(k_scale_out, "k_scale_out", torch.float32, (B, H))
    lq = lqo = Layout(0, 0, 0)
    if q is not None:
        lq = _need_view(q, "q", e4, shape)
        _need(q_scale, "q_scale", torch.float32, (B, H))
        q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
        q_out = torch.empty(shape, dtype=e4, device=q.device) if q_out is None else q_out
        lqo = _need_view(q_out, "q_out", e4, shape)
        q_scale_out = torch.empty_like(q_scale) if q_scale_out is None else q_scale_out
        _need(q_scale_out, "q_scale_out", torch.float32, (B, H))
    else:
        q_scale, q_out, q_scale_out, q_norm_w = None, None, None, None
    _check(lib().fluxattn_qk_norm_rope_ex_fp8(
        _ptr(q), lq, k.data_ptr(), lk, _ptr(q_scale), k_scale.data_ptr(), _ptr(q_out), lqo, k_out.data_ptr(),
        lko, _ptr(q_scale_out), k_scale_out.data_ptr(), _ptr(q_norm_w), k_norm_w.data_ptr(), st,
        pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta), float(eps), _stream(stream)))
    return q_out, k_out, q_scale_out, k_scale_out


def fluxattn_forward_ex_bf16(q, k, v, o=None, softmax_scale=0.0, split=None, stream=None):
    """Attention on bf16 [B,H,N,D] views; o defaults to a new contiguous
    tensor; split: optional SplitWorkspace.  Returns o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    lq = _need_view(q, "q", torch.bfloat16, shape)
    lk = _need_view(k, "k", torch.bfloat16, shape)
    lv = _need_view(v, "v", torch.bfloat16, shape)
    o = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lo = _need_view(o, "o", torch.bfloat16, shape)
    _check(lib().fluxattn_forward_ex_bf16(q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, o.data_ptr(),
                                          lo, B, H, N, D, float(softmax_scale), _split_arg(split),
                                          _stream(stream)))
    return o


def fluxattn_forward_ex_fp8(q, k, v, q_scale, k_scale, v_scale, o=None, softmax_scale=0.0, split=None,
                            stream=None):
    """fp8 form of fluxattn_forward_ex_bf16 (fp32 [B,H] scales); bf16 o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    e4 = torch.float8_e4m3fn
    lq = _need_view(q, "q", e4, shape)
    lk = _need_view(k, "k", e4, shape)
    lv = _need_view(v, "v", e4, shape)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, (B, H))
    o = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lo = _need_view(o, "o", torch.bfloat16, shape)
    _check(lib().fluxattn_forward_ex_fp8(q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, q_scale.data_ptr(),
                                         k_scale.data_ptr(), v_scale.data_ptr(), o.data_ptr(), lo, B, H, N, D,
                                         float(softmax_scale), _split_arg(split), _stream(stream)))
    return o


def fluxattn_joint_attention_ex_bf16(q, k, v, q_norm_w, k_norm_w, pos_ids, streams=(0,), o=None,
                                     k_work=None, axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS,
                                     softmax_scale=0.0, split=None, stream=None):
    """The whole block on raw bf16 [B,H,N,D] views with per-stream norm
    weights [S, D].  k_work (contiguous [B,H,N,D]) receives K'; o defaults
    to a new contiguous tensor.  Returns o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    st = streams_of(streams)
    lq = _need_view(q, "q", torch.bfloat16, shape)
    lk = _need_view(k, "k", torch.bfloat16, shape)
    lv = _need_view(v, "v", torch.bfloat16, shape)
    q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
    k_norm_w = _weights(k_norm_w, "k_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lo = _need_view(o, "o", torch.bfloat16, shape)
    k_work = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if k_work is None else k_work
    _need(k_work, "k_work", torch.bfloat16, shape)
    _check(lib().fluxattn_joint_attention_ex_bf16(
        q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, k_work.data_ptr(), o.data_ptr(), lo,
        q_norm_w.data_ptr(), k_norm_w.data_ptr(), st, pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1],
        axes[2], float(theta), float(eps), float(softmax_scale), _split_arg(split), _stream(stream)))
    return o


def fluxattn_joint_attention_ex_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, k_norm_w, pos_ids,
                                    streams=(0,), o=None, k_work=None, k_scale_work=None, axes=ROPE_AXES,
                                    theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0, split=None, stream=None):
    """fp8 form of fluxattn_joint_attention_ex_bf16; returns bf16 o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    e4 = torch.float8_e4m3fn
    st = streams_of(streams)
    lq = _need_view(q, "q", e4, shape)
    lk = _need_view(k, "k", e4, shape)
    lv = _need_view(v, "v", e4, shape)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, (B, H))
    q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
    k_norm_w = _weights(k_norm_w, "k_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lo = _need_view(o, "o", torch.bfloat16, shape)
    k_work = torch.empty(shape, dtype=e4, device=q.device) if k_work is None else k_work
    _need(k_work, "k_work", e4, shape)
    k_scale_work = torch.empty_like(k_scale) if k_scale_work is None else k_scale_work
    _need(k_scale_work, "k_scale_work", torch.float32, (B, H))
    _check(lib().fluxattn_joint_attention_ex_fp8(
        q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, q_scale.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), k_work.data_ptr(), k_scale_work.data_ptr(), o.data_ptr(), lo, q_norm_w.data_ptr(),
        k_norm_w.data_ptr(), st, pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta),
        float(eps), float(softmax_scale), _split_arg(split), _stream(stream)))
    return o


def fluxattn_forward_fused_ex_bf16(q, k, v, q_norm_w, pos_ids, streams=(0,), o=None, axes=ROPE_AXES,
                                   theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0, split=None, stream=None):
    """Attention on raw bf16 query views (RMSNorm + RoPE applied as they are
    loaded, per-stream weights [S, D]) against prepared key views k and
    value views v; split: optional SplitWorkspace.  Returns o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    st = streams_of(streams)
    lq = _need_view(q, "q", torch.bfloat16, shape)
    lk = _need_view(k, "k", torch.bfloat16, shape)
    lv = _need_view(v, "v", torch.bfloat16, shape)
    q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lo = _need_view(o, "o", torch.bfloat16, shape)
    _check(lib().fluxattn_forward_fused_ex_bf16(
        q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, o.data_ptr(), lo, q_norm_w.data_ptr(), st,
        pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta), float(eps),
        float(softmax_scale), _split_arg(split), _stream(stream)))
    return o


def fluxattn_forward_fused_ex_fp8(q, k, v, q_scale, k_scale, v_scale, q_norm_w, pos_ids, streams=(0,), o=None,
                                  axes=ROPE_AXES, theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0, split=None,
                                  stream=None):
    """fp8 form of fluxattn_forward_fused_ex_bf16 (E4M3 views, fp32 [B,H]
    scales); returns bf16 o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    e4 = torch.float8_e4m3fn
    st = streams_of(streams)
    lq = _need_view(q, "q", e4, shape)
    lk = _need_view(k, "k", e4, shape)
    lv = _need_view(v, "v", e4, shape)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _need(t, name, torch.float32, (B, H))
    q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    o = torch.empty(shape, dtype=torch.bfloat16, device=q.device) if o is None else o
    lo = _need_view(o, "o", torch.bfloat16, shape)
    _check(lib().fluxattn_forward_fused_ex_fp8(
        q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, q_scale.data_ptr(), k_scale.data_ptr(),
        v_scale.data_ptr(), o.data_ptr(), lo, q_norm_w.data_ptr(), st, pos_ids.data_ptr(), B, H, N, D, axes[0],
        axes[1], axes[2], float(theta), float(eps), float(softmax_scale), _split_arg(split), _stream(stream)))
    return o


def fluxattn_forward_fused_noalloc_bf16(q, k, v, q_norm_w, pos_ids, o, streams=(0,), axes=ROPE_AXES,
                                        theta=ROPE_THETA, eps=RMS_EPS, softmax_scale=0.0, groups=0, stream=None):
    """fluxattn_forward_fused_ex_bf16 with a split of `groups` workgroups in
    the library's static scratch (at most 256 workgroups): for code that must
    not allocate.  o is required (the binding allocates nothing here either).
    Returns o."""
    shape = tuple(q.shape)
    B, H, N, D = _bhnd(q)
    st = streams_of(streams)
    lq = _need_view(q, "q", torch.bfloat16, shape)
    lk = _need_view(k, "k", torch.bfloat16, shape)
    lv = _need_view(v, "v", torch.bfloat16, shape)
    q_norm_w = _weights(q_norm_w, "q_norm_w", st.count, D)
    _need(pos_ids, "pos_ids", torch.int32, (N, 3))
    lo = _need_view(o, "o", torch.bfloat16, shape)
    _check(lib().fluxattn_forward_fused_noalloc_bf16(
        q.data_ptr(), lq, k.data_ptr(), lk, v.data_ptr(), lv, o.data_ptr(), lo, q_norm_w.data_ptr(), st,
        pos_ids.data_ptr(), B, H, N, D, axes[0], axes[1], axes[2], float(theta), float(eps),
        float(softmax_scale), int(groups), _stream(stream)))
    return o


def fluxattn_probe_mfma(kind: str, iterations: int, workgroups: int, sink: torch.Tensor, stream=None) -> float:
    """Enqueue the matrix-core probe (include/fluxattn_probe.h): kind "bf16"
    (32x32x16), "fp8" (32x32x64) or "bf16_16x16x32"; sink a float32 device
    tensor of at least workgroups * 8 elements.  Returns the launch's matrix
    flops (time it with events)."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < 8 * workgroups:
        raise ValueError("sink needs workgroups * 8 elements")
    flops = ctypes.c_double(0.0)
    _check(lib().fluxattn_probe_mfma({"bf16": 0, "fp8": 1, "bf16_16x16x32": 2}[kind], int(iterations), int(workgroups),
                                     sink.data_ptr(), ctypes.byref(flops), _stream(stream)))
    return float(flops.value)

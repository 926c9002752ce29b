"""fp64 CPU oracle for the FLUX joint-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it, and it imports nothing from the
product path.

What it computes, in the order the method applies it:

1. decode of the stored inputs to fp64 (bf16 bit patterns; OCP E4M3 bytes
   times a per-(b,h) scale),
2. per-head RMS normalisation of queries and keys with learned weights,
3. a rotary position embedding whose head dimensions are split over the
   three position axes (t, h, w) of each token,
4. non-causal softmax(Q K^T / sqrt(d)) V over the merged text + image
   (+ reference image) token sequence.

Sources.  NVIDIA's blog post "Speed up image generation with FLUX 3 Image
Klein on NVIDIA Blackwell GPUs" states that the text, noisy-target and
optional reference-image streams are processed separately and then merged by
joint attention (section "Running FLUX 3 inference with TensorRT LLM
VisualGen"), and that the QKV projection's epilogue applies query/key
normalisation and RoPE (section "GEMM kernel optimization").  Its section
"Quantized and sparse attention" selects FP8 for queries/keys and values.
The pages give no formulas: the readings used for RMSNorm (eps inside the
square root), the axis split (16, 56, 56) with theta 1e4, adjacent-pair
rotation and the E4M3 format are the plain ones and are listed with the rest
of the readings in the design notes.

Everything is plain NumPy in float64 with no intermediate rounding; the only
blocking is over query rows, to keep the N x N score block in memory.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# 1. decoding of stored values
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.  A bf16 value is the upper
    16 bits of the IEEE binary32 value, so the decode is a shift."""
    b32 = (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16)
    with np.errstate(invalid="ignore"):   # NaN patterns stay NaN
        return b32.view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 bytes -> float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 encodes subnormals m/8 * 2^-6; the code with all exponent and
    mantissa bits set (0x7F / 0xFF) is NaN; there are no infinities, so the
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 7)
    sub = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def dequantize_e4m3(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """x[b,h,...] = e4m3(codes[b,h,...]) * scale[b,h]."""
    x = e4m3fn_to_f64(codes)
    s = np.asarray(scale, dtype=np.float64)
    return x * s.reshape(s.shape + (1,) * (x.ndim - s.ndim))


# --------------------------------------------------------------------------
# 2. per-head RMS normalisation
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """y = x * w / sqrt(mean_d(x^2) + eps) over the last (head) dimension."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * np.asarray(w, dtype=np.float64) / np.sqrt(ms + eps)


def stream_weights(w_rows, starts, N: int) -> np.ndarray:
    """Per-token RMSNorm weights [N, D] of a sequence made of token streams.

    The joint sequence is the text stream, then the target-image stream, then
    the optional reference-image stream; up to the joint attention each
    stream has its own projection and normalisation weights (blog post
    "Speed up image generation with FLUX 3 Image Klein on NVIDIA Blackwell
    GPUs", section "Running FLUX 3 inference with TensorRT LLM VisualGen").
    Stream s holds tokens [starts[s], starts[s+1]) (the last runs to N) and
    uses row w_rows[s].  rms_norm broadcasts the result over batch and heads.
    """
    w_rows = np.asarray(w_rows, dtype=np.float64)
    bounds = [int(x) for x in starts] + [N]
    assert w_rows.shape[0] == len(starts) and bounds[0] == 0
    out = np.empty((N, w_rows.shape[1]), dtype=np.float64)
    for s in range(len(starts)):
        out[bounds[s]:bounds[s + 1]] = w_rows[s]
    return out


# --------------------------------------------------------------------------
# 3. three-axis rotary position embedding
# --------------------------------------------------------------------------

def rope_frequencies(axes=(16, 56, 56), theta: float = 1e4):
    """Per axis a with d_a dims: omega_{a,j} = theta^(-2j/d_a), j < d_a/2."""
    return [np.power(float(theta), -2.0 * np.arange(d // 2) / d) for d in axes]


def rope(y: np.ndarray, pos_ids: np.ndarray, axes=(16, 56, 56),
         theta: float = 1e4) -> np.ndarray:
    """Rotate y[..., N, D] by the per-token angles of its (t, h, w) ids.

    The head dimension is split into contiguous blocks, one per axis in
    (t, h, w) order.  Inside axis a's block starting at offset o_a, the pair
    (y[o_a+2j], y[o_a+2j+1]) = (u, v) becomes
    (u cos phi - v sin phi, u sin phi + v cos phi) with phi = p_a * omega_{a,j}.
    """
    y = np.asarray(y, dtype=np.float64)
    pos = np.asarray(pos_ids, dtype=np.int64)
    assert pos.shape == (y.shape[-2], len(axes))
    assert sum(axes) == y.shape[-1]
    out = y.copy()
    off = 0
    for a, (d_a, omega) in enumerate(zip(axes, rope_frequencies(axes, theta))):
        phi = pos[:, a:a + 1].astype(np.float64) * omega[None, :]   # [N, d_a/2]
        c, s = np.cos(phi), np.sin(phi)
        u = y[..., off:off + d_a:2]
        v = y[..., off + 1:off + d_a:2]
        out[..., off:off + d_a:2] = u * c - v * s
        out[..., off + 1:off + d_a:2] = u * s + v * c
        off += d_a
    return out


def qk_prologue(q, k, w_q, w_k, pos_ids, axes=(16, 56, 56), theta=1e4,
                eps=1e-6):
    """RMSNorm then RoPE on queries and keys (values are left alone)."""
    qn = rope(rms_norm(q, w_q, eps), pos_ids, axes, theta)
    kn = rope(rms_norm(k, w_k, eps), pos_ids, axes, theta)
    return qn, kn


def fp8_prologue_out_scale(w: np.ndarray, D: int = 128) -> float:
    """Output scale of the fp8 prologue: sqrt(D) * max|w| / 448.

    |rms_norm(x)_d| <= sqrt(D) |w_d| because x_d^2 <= sum x^2 = D mean(x^2),
    and a rotation keeps each pair inside its own norm, so every prologue
    output divided by this scale lies in [-448, 448]."""
    return math.sqrt(D) * float(np.max(np.abs(np.asarray(w, np.float64)))) / E4M3_MAX


# --------------------------------------------------------------------------
# 4. non-causal softmax attention
# --------------------------------------------------------------------------

def attention(q, k, v, scale: float | None = None, rows=None,
              row_block: int = 1024) -> np.ndarray:
    """O = softmax(Q K^T * scale) V per (b, h), scale = 1/sqrt(d) by default.

    q, k, v: [B, H, N, D] (anything convertible to float64).  rows: optional
    1-D array of query indices; the output then has those rows only
    ([B, H, len(rows), D]).  Softmax is taken with the row maximum subtracted
    (an identity of the softmax, used so that exp cannot overflow).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    idx = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, H, idx.size, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kt = k[b, h].T
            for s0 in range(0, idx.size, row_block):
                r = idx[s0:s0 + row_block]
                s = (q[b, h, r] @ kt) * scale
                s -= s.max(axis=1, keepdims=True)
                p = np.exp(s)
                out[b, h, s0:s0 + r.size] = (p @ v[b, h]) / p.sum(axis=1, keepdims=True)
    return out


def joint_attention(q, k, v, w_q, w_k, pos_ids, axes=(16, 56, 56), theta=1e4,
                    eps=1e-6, scale=None, rows=None):
    """The whole block: prologue on Q and K, then attention over all tokens."""
    qn, kn = qk_prologue(q, k, w_q, w_k, pos_ids, axes, theta, eps)
    return attention(qn, kn, v, scale=scale, rows=rows)


def joint_attention_heads(q, k, v, w_q, w_k, pos_ids, heads, rows=None,
                          axes=(16, 56, 56), theta=1e4, eps=1e-6):
    """joint_attention restricted to a list of (b, h) pairs; returns
    [len(heads), len(rows) or N, D].  Used to check sampled outputs of large
    workloads one head at a time."""
    res = []
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        res.append(joint_attention(np.asarray(q[sl]), np.asarray(k[sl]),
                                   np.asarray(v[sl]), w_q, w_k, pos_ids,
                                   axes, theta, eps, rows=rows)[0, 0])
    return np.stack(res)

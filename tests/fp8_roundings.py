"""A CPU model of the roundings that the fp8 attention path is allowed
(test infrastructure: the parity tests use it to show where the fp8 error
comes from; it is not the oracle, and nothing of the HIP path is used).

The FP8 attention of the NVIDIA blog post "Speed up image generation with
FLUX 3 Image Klein on NVIDIA Blackwell GPUs" (section "Quantized and sparse
attention") runs both products on FP8 operands.  On the fused fp8 path of
this library that means three E4M3 roundings on top of the fp64 chain:

  K'   the key prologue's output, E4M3 codes of K' / s_k with the per-head
       scale s_k = sqrt(D) max|w_k| / 448 (the bound on |K'|);
  Q'   re-encoded per query: codes of Q' g / 2^e with g = c s_k,
       c = log2(e) / sqrt(D), and e the smallest integer that keeps the
       largest code within 448;
  P    E4M3 of 2^6 p relative to the row's shift (here the row maximum), so
       the largest p' is 2^6; the normaliser sums the rounded p'.

`fused_fp8_model` applies any subset of them to the oracle's own chain
(RMSNorm, RoPE, softmax attention) in fp64.  With none applied it is the
oracle's result; each one alone is a plain RNE encode of the values the
kernel encodes.  The kernel's running shift moves lazily (the largest p'
of a row lies between 2^6 and 2^8), which changes where values fall on the
E4M3 grid but not the size of the rounding, so the model predicts the
kernel's error statistics rather than its exact bits.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

E4M3_MAX = 448.0
LOG2E = math.log2(math.e)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest OCP E4M3 value (ties to even), as fp64."""
    assert np.all(np.abs(x) <= E4M3_MAX), "the model never encodes past the format's range"
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).double().numpy()


def fused_fp8_model(q, k, v, w_q_tok, w_k_tok, w_k_rows, pos, rounds=("k", "q", "p")):
    """Output [B, H, N, D] of the fused fp8 block on dequantised inputs q, k,
    v (fp64 [B, H, N, D]) with per-token norm weights [N, D], the key weight
    rows [S, D] (for the key scale) and ids [N, 3], with the named roundings
    applied."""
    D = q.shape[-1]
    c = LOG2E / math.sqrt(D)
    qp = oracle.rope(oracle.rms_norm(q, w_q_tok, 1e-6), pos)
    kp = oracle.rope(oracle.rms_norm(k, w_k_tok, 1e-6), pos)
    s_k = math.sqrt(D) * float(np.abs(w_k_rows).max()) / E4M3_MAX
    if "k" in rounds:
        kp = e4m3_round(kp / s_k) * s_k
    if "q" in rounds:
        g = c * s_k
        amax = np.abs(qp).max(axis=-1, keepdims=True)
        e = np.ceil(np.log2(amax * g / E4M3_MAX))
        qp = e4m3_round(qp * g / 2.0 ** e) * 2.0 ** e / g
    out = np.empty_like(q)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            x = c * (qp[b, h] @ kp[b, h].T)                  # base-2 logits
            p = np.exp2(x - x.max(axis=1, keepdims=True) + 6.0)
            if "p" in rounds:
                p = e4m3_round(p)
            out[b, h] = (p @ v[b, h]) / p.sum(axis=1, keepdims=True)
    return out


def case_inputs(inp, w_q_rows, w_k_rows, starts):
    """fp64 q, k, v and per-token weights of a workload's fp8 Inputs."""
    N = inp.q.shape[2]
    f64 = lambda t, s: oracle.torch_to_f64(t, s)
    return (f64(inp.q, inp.q_scale), f64(inp.k, inp.k_scale), f64(inp.v, inp.v_scale),
            oracle.stream_weights(w_q_rows, starts, N), oracle.stream_weights(w_k_rows, starts, N),
            inp.pos.numpy())

"""Bit-level conversion of CPU torch tensors into the oracle's fp64 arrays
(test infrastructure only).  The decode itself is the oracle's own: torch is
used only to expose the raw bytes."""
from __future__ import annotations

import numpy as np
import torch

from .fluxattn_oracle import bf16_bits_to_f64, dequantize_e4m3


def torch_to_f64(x: torch.Tensor, scale: torch.Tensor | None = None) -> np.ndarray:
    """bf16 / float8_e4m3fn (with per-(b,h) scale) / fp32 CPU tensor -> float64."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return bf16_bits_to_f64(x.view(torch.int16).numpy().view(np.uint16))
    if x.dtype == torch.float8_e4m3fn:
        codes = x.view(torch.uint8).numpy()
        s = np.ones(x.shape[:2]) if scale is None else scale.detach().cpu().double().numpy()
        return dequantize_e4m3(codes, s)
    return x.double().numpy()

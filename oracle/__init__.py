"""fp64 CPU oracle of the joint-attention hot path (test infrastructure only:
tests, the smoke check and the benchmark's CPU baseline may use it; the
product path never does)."""
from .fluxattn_oracle import (  # noqa: F401
    E4M3_MAX, attention, bf16_bits_to_f64, dequantize_e4m3, e4m3fn_to_f64,
    fp8_prologue_out_scale, joint_attention, joint_attention_heads,
    qk_prologue, rms_norm, rope, rope_frequencies, stream_weights,
)
from .convert import torch_to_f64  # noqa: F401

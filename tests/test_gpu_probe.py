"""The matrix-core probe (include/fluxattn_probe.h) on the GPU: it runs, its
flop count per round and wave is that of 8 MFMAs of 32x32xk (the 16x16x32
kind: 16 MFMAs, the same flops), and every wave leaves a finite sum in the
sink."""
import pytest
import torch

import joint_attention_head_amd as fa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,k", [("bf16", 16), ("fp8", 64), ("bf16_16x16x32", 16)])
def test_probe_runs_and_counts_flops(kind, k):
    wg = 16
    sink = torch.full((wg * 8,), float("nan"), dtype=torch.float32, device="cuda")
    flops = fa.fluxattn_probe_mfma(kind, 100, wg, sink)
    torch.cuda.synchronize()
    assert flops == 2.0 * 32 * 32 * k * 8 * 100 * 8 * wg
    assert torch.isfinite(sink).all()


def test_probe_rejects_bad_arguments():
    sink = torch.zeros(8, dtype=torch.float32, device="cuda")
    for kind, iters, wg in (("bf16", 0, 1), ("fp8", 1, 0), ("bf16", 1, 2)):
        with pytest.raises((fa.FluxAttnError, ValueError)):
            fa.fluxattn_probe_mfma(kind, iters, wg, sink)

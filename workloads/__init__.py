"""Seeded synthetic inputs for the FLUX joint-attention hot path.

This module is shared by the CPU oracle and the HIP path; it holds only the
workload shapes and the random-number recipe, none of the method's arithmetic
(no normalisation, no rotation, no attention, no fp8 decoding).

Workloads follow the token counts of FLUX-style MM-DiT generation: a text
stream of N_txt tokens followed by the latent-image patch grid (one token per
2x2 latent patch), and for image-to-image a second, reference-image grid.  The
merge of the streams into one sequence for joint attention is described in the
"Running FLUX 3 inference with TensorRT LLM VisualGen" section of the NVIDIA
blog post "Speed up image generation with FLUX 3 Image Klein on NVIDIA
Blackwell GPUs"; the pages print no activations, so standard-normal tensors of
the real shapes stand in for them.

Recipe (one torch CPU generator per call, seeded, drawn in this order):
  q, k, v      = randn(B, H, N, 128) fp32 each, then rounded to bf16
  w_q, w_k     = 1 + 0.1 * randn(128) fp32 each
fp8 workloads quantise q, k, v per (b, h) to OCP E4M3 with the amax scale
s[b, h] = max|x[b, h]| / 448 (torch's float8_e4m3fn cast does the rounding).
Position ids (t, h, w) are int32 [N, 3]: text tokens (0, 0, 0); target-image
tokens (0, r, c) in row-major patch order; reference-image tokens (1, r, c).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

HEAD_DIM = 128
ROPE_AXES = (16, 56, 56)
ROPE_THETA = 10000.0
RMS_EPS = 1e-6
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n_txt: int
    grid: tuple          # target-image patch grid (rows, cols)
    ref_grid: tuple | None
    dtype: str           # "bf16" or "fp8"
    seed: int = 0

    @property
    def N(self) -> int:
        n = self.n_txt + self.grid[0] * self.grid[1]
        if self.ref_grid is not None:
            n += self.ref_grid[0] * self.ref_grid[1]
        return n

    @property
    def flops(self) -> float:
        """Dense attention work 4*B*H*N^2*d (two N x N x d contractions)."""
        return 4.0 * self.B * self.H * self.N * self.N * HEAD_DIM


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, (16, 16), None, "bf16"),
    "flux_dev_512": Workload("flux_dev_512", 1, 24, 512, (32, 32), None, "bf16"),
    "flux_dev_1024": Workload("flux_dev_1024", 1, 24, 512, (64, 64), None, "bf16"),
    "t2i_2048_cfg": Workload("t2i_2048_cfg", 2, 24, 512, (128, 128), None, "bf16"),
    "i2i_2048": Workload("i2i_2048", 1, 24, 512, (128, 128), (128, 128), "fp8"),
}


def position_ids(n_txt: int, grid, ref_grid=None) -> np.ndarray:
    """int32 [N, 3] (t, h, w) ids: text, then target grid, then reference grid."""
    parts = [np.zeros((n_txt, 3), dtype=np.int32)]
    for t, g in ((0, grid), (1, ref_grid)):
        if g is None:
            continue
        r, c = np.meshgrid(np.arange(g[0]), np.arange(g[1]), indexing="ij")
        ids = np.stack([np.full(r.size, t), r.ravel(), c.ravel()], axis=1)
        parts.append(ids.astype(np.int32))
    return np.ascontiguousarray(np.concatenate(parts, axis=0))


def stream_starts(w: Workload) -> tuple:
    """First token of each stream in the joint sequence: text, target image
    and, when present, reference image."""
    starts = [0, w.n_txt]
    if w.ref_grid is not None:
        starts.append(w.n_txt + w.grid[0] * w.grid[1])
    return tuple(starts)


def stream_norm_weights(n_streams: int, seed: int = 0, D: int = HEAD_DIM):
    """Per-stream fp32 norm weights [S, D] for queries and keys, each row
    1 + 0.1*N(0,1) like the single-stream weights."""
    g = torch.Generator(device="cpu").manual_seed(1000 + seed)
    w_q = 1.0 + 0.1 * torch.randn(n_streams, D, generator=g, dtype=torch.float32)
    w_k = 1.0 + 0.1 * torch.randn(n_streams, D, generator=g, dtype=torch.float32)
    return w_q, w_k


def randn_qkv(B: int, H: int, N: int, seed: int = 0, D: int = HEAD_DIM):
    """fp32 q, k, v ~ N(0,1) and norm weights 1 + 0.1*N(0,1), in recipe order."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn(B, H, N, D, generator=g, dtype=torch.float32)
    k = torch.randn(B, H, N, D, generator=g, dtype=torch.float32)
    v = torch.randn(B, H, N, D, generator=g, dtype=torch.float32)
    w_q = 1.0 + 0.1 * torch.randn(D, generator=g, dtype=torch.float32)
    w_k = 1.0 + 0.1 * torch.randn(D, generator=g, dtype=torch.float32)
    return q, k, v, w_q, w_k


def quantize_e4m3_per_head(x: torch.Tensor):
    """x fp32 [B,H,N,D] -> (float8_e4m3fn tensor, fp32 scales [B,H]), amax/448."""
    amax = x.abs().amax(dim=(2, 3))
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (x / scale[:, :, None, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn), scale.contiguous()


@dataclasses.dataclass
class Inputs:
    """CPU tensors of one workload.  bf16: q,k,v bfloat16.  fp8: q,k,v
    float8_e4m3fn with per-(b,h) fp32 scales q_scale/k_scale/v_scale."""
    workload: Workload
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    w_q: torch.Tensor
    w_k: torch.Tensor
    pos: torch.Tensor
    q_scale: torch.Tensor | None = None
    k_scale: torch.Tensor | None = None
    v_scale: torch.Tensor | None = None


def make_inputs(w: Workload | str, seed: int | None = None) -> Inputs:
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed if seed is None else seed
    pos = torch.from_numpy(position_ids(w.n_txt, w.grid, w.ref_grid))
    q, k, v, w_q, w_k = randn_qkv(w.B, w.H, w.N, seed)
    if w.dtype == "bf16":
        return Inputs(w, q.to(torch.bfloat16), k.to(torch.bfloat16),
                      v.to(torch.bfloat16), w_q, w_k, pos)
    q8, sq = quantize_e4m3_per_head(q)
    del q
    k8, sk = quantize_e4m3_per_head(k)
    del k
    v8, sv = quantize_e4m3_per_head(v)
    return Inputs(w, q8, k8, v8, w_q, w_k, pos, sq, sk, sv)


def custom_workload(B, H, n_txt, grid, ref_grid=None, dtype="bf16", seed=0,
                    name="custom") -> Workload:
    return Workload(name, B, H, n_txt, tuple(grid),
                    None if ref_grid is None else tuple(ref_grid), dtype, seed)


def make_peaked_inputs(w: Workload | str, seed: int | None = None,
                       noise: float = 0.05) -> Inputs:
    """bf16 workload whose keys are the queries plus 0.05*N(0,1) noise, so
    each query's own key dominates its row of scores by about sqrt(d) logits."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    seed = w.seed if seed is None else seed
    pos = torch.from_numpy(position_ids(w.n_txt, w.grid, w.ref_grid))
    q, _, v, w_q, w_k = randn_qkv(w.B, w.H, w.N, seed)
    g = torch.Generator(device="cpu").manual_seed(seed + 1)
    k = q + noise * torch.randn(q.shape, generator=g, dtype=torch.float32)
    return Inputs(w, q.to(torch.bfloat16), k.to(torch.bfloat16),
                  v.to(torch.bfloat16), w_q, w_k, pos)

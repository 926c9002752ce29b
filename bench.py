#!/usr/bin/env python3
"""Joint-attention throughput on one MI355X.

One step = the whole hot path over one batch: per-head RMSNorm + 3-axis RoPE
of queries and keys, then non-causal softmax attention, on the 2048x2048
text-to-image workload with CFG (B=2, H=24, N = 512 text + 128x128 image
tokens = 16896, d=128, bf16), inputs already resident in HBM.  Default path
(--path fused): the keys-only prologue kernel, then the attention kernel
that normalises and rotates the queries as it loads them; --path unfused
runs the prologue on both and the plain attention kernel.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]

Prints one JSON line: TFLOP/s of the step (4*B*H*N^2*d per step), the
attention kernel's roofline fraction (its own average launch time from HIP
events on the launch stream), the same figures at N=4608 (FLUX-dev 1024x1024)
under "also", the fp8 path (E4M3 Q/K/V, fp8 matrix cores) on the 2048x2048
image-to-image workload (B=1, H=24, N = 512 + 2 x 128x128 = 33280) under
"fp8" with its roofline against the fp8 MFMA peak, every workload's forward
TFLOP/s and MFMA fraction under "all_configs", and the fp64 CPU oracle timed
on a bounded sample of the main workload under "cpu_baseline".  Each roofline
also carries the MFMA-busy fraction and sustained clock of its kernel from
the committed rocprofv3 counter summary ("counters", null once the kernel
source has changed since it was taken).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5033.2      # MI355X dense fp8 MFMA
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E
CSRC = os.path.join(ROOT, "joint_attention_head_amd", "csrc")
# rocprofv3 counter summaries of the attention kernels, and the sources each
# kernel is built from (a summary only counts while they are unchanged)
TRAFFIC = {
    "bf16": (os.path.join(ROOT, "profiles", "attn_fwd_bf16_t2i_2048_hbm_traffic.txt"),
             ("attention.hip", "attn_common.h", "fluxattn_internal.h")),
    "fp8": (os.path.join(ROOT, "profiles", "attn_fwd_fp8_i2i_2048_hbm_traffic.txt"),
            ("attention_fp8.hip", "attn_common.h", "fluxattn_internal.h")),
}


def kernel_source_hash(kind: str = "bf16") -> str:
    h = hashlib.sha256()
    for name in TRAFFIC[kind][1]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str, kind: str = "bf16"):
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, or None if the kernel source changed since it was taken or the
    summary covers the other kernel variant."""
    traffic_file = TRAFFIC[kind][0]
    if not os.path.exists(traffic_file):
        return None
    vals = {}
    with open(traffic_file) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kind) or vals.get("path", "unfused") != path:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


COUNTERS = os.path.join(ROOT, "profiles", "attn_fwd_mfma_valu_counters.txt")
COUNTER_KERNEL = {"bf16": "attn_fwd_kernel", "fp8": "attn_fwd_fp8_kernel"}


def measured_mfma_busy(kind: str = "bf16"):
    """MFMA-busy fraction and sustained clock of one attention kernel from the
    committed rocprofv3 counter summary, or None if that kernel's source
    changed since the counters were taken."""
    if not os.path.exists(COUNTERS):
        return None
    hashes, block, cur = {}, {}, None
    with open(COUNTERS) as f:
        for line in f:
            m = re.search(r"bf16 sha256_16 ([0-9a-f]+), fp8 sha256_16 ([0-9a-f]+)", line)
            if m:
                hashes = {"bf16": m.group(1), "fp8": m.group(2)}
            elif line.startswith("kernel:"):
                cur = line.split(":", 1)[1].strip()
                block[cur] = {}
            elif cur and ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                block[cur][k.strip()] = v.strip()
    vals = block.get(COUNTER_KERNEL[kind], {})
    if hashes.get(kind) != kernel_source_hash(kind):
        return None
    try:
        return {"mfma_busy_fraction": float(vals["mfma_busy_fraction"]), "clock_GHz": float(vals["clock_GHz"])}
    except (KeyError, ValueError):
        return None


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="t2i_2048_cfg")
    p.add_argument("--also", default="flux_dev_1024", help="second metric point ('' to skip)")
    p.add_argument("--fp8", default="i2i_2048", help="fp8 workload ('' to skip)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-all-configs", dest="all_configs", action="store_false",
                   help="skip the per-workload table (every workload's forward TFLOP/s and MFMA fraction)")
    p.add_argument("--cpu-heads", type=int, default=12, help="(b,h) heads in the CPU oracle sample")
    p.add_argument("--path", choices=("fused", "unfused"), default="fused")
    p.add_argument("--groups", type=int, default=0,
                   help="attention workgroup setting: 0 = one per compute unit, key ranges split where that "
                        "balances the last round (default); < 0 = never split; > 0 = that many workgroups")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB elementwise copy (HBM counter calibration)")
    return p.parse_args()


def run_gpu(name: str, steps: int, warmup: int, path: str = "fused"):
    import torch

    import joint_attention_head_amd as fa
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[name]
    inp = make_inputs(w)
    fp8 = w.dtype == "fp8"
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    w_q, w_k, pos = inp.w_q.to(dev), inp.w_k.to(dev), inp.pos.to(dev)
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    if fp8:
        sq, sk, sv = (t.to(dev) for t in (inp.q_scale, inp.k_scale, inp.v_scale))
        sqn, skn = torch.empty_like(sq), torch.empty_like(sk)
    stream = torch.cuda.current_stream()

    def prologue():
        if fp8 and path == "fused":
            fa.fluxattn_qk_norm_rope_fp8(None, k, None, sk, None, w_k, pos, k_out=kn, k_scale_out=skn, stream=stream)
        elif fp8:
            fa.fluxattn_qk_norm_rope_fp8(q, k, sq, sk, w_q, w_k, pos, q_out=qn, k_out=kn, q_scale_out=sqn,
                                         k_scale_out=skn, stream=stream)
        elif path == "fused":
            fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos, k_out=kn, stream=stream)
        else:
            fa.fluxattn_qk_norm_rope_bf16(q, k, w_q, w_k, pos, q_out=qn, k_out=kn, stream=stream)

    def attention():
        if fp8 and path == "fused":
            fa.fluxattn_forward_fused_fp8(q, kn, v, sq, skn, sv, w_q, pos, o=o, stream=stream)
        elif fp8:
            fa.fluxattn_forward_fp8(qn, kn, v, sqn, skn, sv, o=o, stream=stream)
        elif path == "fused":
            fa.fluxattn_forward_fused_bf16(q, kn, v, w_q, pos, o=o, stream=stream)
        else:
            fa.fluxattn_forward_bf16(qn, kn, v, o=o, stream=stream)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        prologue()
        if ev is not None:
            ev[1].record(stream)
        attention()
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pro = [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    fwd = [e[1].elapsed_time(e[2]) * 1e-3 for e in evs]
    span = evs[0][0].elapsed_time(evs[-1][2]) * 1e-3
    assert torch.isfinite(o).all().item()
    flops = w.flops
    # read + write K (fused path) or Q and K
    esize = 1 if fp8 else 2
    prologue_bytes = (2.0 if path == "fused" else 4.0) * w.B * w.H * w.N * 128 * esize
    attn_min_bytes = w.B * w.H * w.N * 128 * (3.0 * esize + 2)   # read Q, K, V, write bf16 O once
    t_fwd = sum(fwd) / len(fwd)
    t_pro = sum(pro) / len(pro)
    res = {
        "workload": w,
        "ms_per_step": wall / steps * 1e3,
        "gpu_span_ms_per_step": span / steps * 1e3,
        "value": flops / (wall / steps) / 1e12,
        "forward_ms": t_fwd * 1e3,
        "forward_tflops": flops / t_fwd / 1e12,
        "prologue_us": t_pro * 1e6,
        "prologue_gbs": prologue_bytes / t_pro / 1e9,
        "attn_min_bytes": attn_min_bytes,
        "flops": flops,
    }
    del q, k, v, qn, kn, o
    if fp8:
        del sq, sk, sv, sqn, skn
    torch.cuda.empty_cache()
    return res


def calibrate_copy():
    import torch
    n = 1 << 29                        # 2^29 bf16 = 1 GiB read + 1 GiB written
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"copy calibration: torch.neg over {n * 2} bytes read and {n * 2} written", file=sys.stderr)


def cpu_baseline(name: str, n_heads: int):
    import numpy as np

    import oracle
    from workloads import WORKLOADS, make_inputs
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = os.cpu_count() or 1
    w = WORKLOADS[name]
    inp = make_inputs(w)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][:n_heads]
    w_q, w_k, pos = inp.w_q.double().numpy(), inp.w_k.double().numpy(), inp.pos.numpy()
    t0 = time.perf_counter()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        q, k, v = (oracle.torch_to_f64(t[sl]) for t in (inp.q, inp.k, inp.v))
        out = oracle.joint_attention(q, k, v, w_q, w_k, pos)
        assert np.isfinite(out).all()
    dt = time.perf_counter() - t0
    flops = 4.0 * len(heads) * w.N * w.N * 128
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{len(heads)} of {w.B * w.H} (b,h) heads of {name} (N={w.N}), all query rows, "
                  f"prologue + attention in fp64 NumPy; {dt:.1f} s",
        "seconds": round(dt, 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    import joint_attention_head_amd as fa
    fa.fluxattn_set_forward_groups(args.groups)
    print(f"bench: {args.workload} steps={args.steps} warmup={args.warmup} groups={args.groups}",
          file=sys.stderr, flush=True)
    main_res = run_gpu(args.workload, args.steps, args.warmup, args.path)
    done = {args.workload: main_res}
    print(f"bench: {args.workload} forward {main_res['forward_ms']:.3f} ms", file=sys.stderr, flush=True)
    also = None
    if args.also:
        r = run_gpu(args.also, args.steps, args.warmup, args.path)
        done[args.also] = r
        w = r["workload"]
        also = {
            "workload": f"{w.name}: B={w.B} H={w.H} N={w.n_txt}+{w.grid[0]}x{w.grid[1]}={w.N} d=128 bf16",
            "value": round(r["value"], 2),
            "ms_per_step": round(r["ms_per_step"], 4),
            "forward_tflops": round(r["forward_tflops"], 2),
            "forward_frac_of_bf16_peak": round(r["forward_tflops"] / BF16_PEAK_TFLOPS, 4),
            "prologue_gbs": round(r["prologue_gbs"], 1),
        }
        print(f"bench: {args.also} forward {r['forward_ms']:.3f} ms", file=sys.stderr, flush=True)
    fp8 = None
    if args.fp8:
        r = run_gpu(args.fp8, args.steps, args.warmup, args.path)
        done[args.fp8] = r
        w = r["workload"]
        fp8 = {
            "workload": f"{w.name}: 2048x2048 image-to-image, B={w.B} H={w.H} "
                        f"N={w.n_txt}+{w.grid[0]}x{w.grid[1]}+{w.ref_grid[0]}x{w.ref_grid[1]}={w.N} d=128, "
                        "E4M3 q/k/v with per-(b,h) scales, bf16 output, prologue + attention",
            "value": round(r["value"], 2),
            "unit": "TFLOP/s",
            "ms_per_step": round(r["ms_per_step"], 4),
            "dtype": "fp8-e4m3",
            "roofline": {
                "kernel": "attn_fwd_fp8_kernel (E4M3 MFMA, %s)" % (
                    "fused query prologue" if args.path == "fused" else "plain"),
                "bound": "mfma",
                "achieved": round(r["forward_tflops"], 2),
                "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(r["forward_tflops"] / FP8_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.path, "fp8"),
                "launch_ms": round(r["forward_ms"], 4),
                "counters": measured_mfma_busy("fp8") if args.path == "fused" else None,
            },
            "prologue_gbs": round(r["prologue_gbs"], 1),
        }
        print(f"bench: {args.fp8} fp8 forward {r['forward_ms']:.3f} ms", file=sys.stderr, flush=True)
    all_configs = None
    if args.all_configs:
        from workloads import WORKLOADS
        all_configs = {}
        for name in WORKLOADS:
            r = done.get(name)
            if r is None:
                r = run_gpu(name, max(args.steps, 10), max(args.warmup, 3), args.path)
            w = r["workload"]
            peak = FP8_PEAK_TFLOPS if w.dtype == "fp8" else BF16_PEAK_TFLOPS
            all_configs[name] = {
                "B": w.B, "H": w.H, "N": w.N, "dtype": w.dtype,
                "value": round(r["value"], 2),
                "forward_ms": round(r["forward_ms"], 4),
                "forward_tflops": round(r["forward_tflops"], 2),
                "frac": round(r["forward_tflops"] / peak, 4),
                "prologue_gbs": round(r["prologue_gbs"], 1),
            }
            print(f"bench: {name} forward {r['forward_ms']:.4f} ms", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        calibrate_copy()
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 CPU oracle sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args.workload, args.cpu_heads)

    w = main_res["workload"]
    traffic = measured_traffic(args.path)
    line = {
        "metric": "joint-attention TFLOP/s and % MFMA peak at N=4608 and N=16896, 1 GPU",
        "value": round(main_res["value"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v, norm weights 1+0.1*N(0,1), FLUX (t,h,w) position ids",
        "config": {
            "workload": f"{w.name}: 2048x2048 text-to-image with CFG, B={w.B} H={w.H} "
                        f"N={w.n_txt}+{w.grid[0]}x{w.grid[1]}={w.N} d=128, prologue + attention",
            "path": args.path,
            "groups": args.groups,
            "B": w.B, "H": w.H, "N": w.N, "head_dim": 128,
        },
        "roofline": {
            "kernel": "attn_fwd_kernel (bf16, %s)" % ("fused query prologue" if args.path == "fused" else "plain"),
            "bound": "mfma",
            "achieved": round(main_res["forward_tflops"], 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(main_res["forward_tflops"] / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
            "launch_ms": round(main_res["forward_ms"], 4),
            "counters": measured_mfma_busy("bf16") if args.path == "fused" else None,
        },
        "prologue": {
            "kernel": "prologue_bf16_kernel (%s)" % ("keys only" if args.path == "fused" else "queries and keys"),
            "bound": "hbm",
            "achieved": round(main_res["prologue_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(main_res["prologue_gbs"] / HBM_PEAK_GBS, 4),
            "launch_us": round(main_res["prologue_us"], 2),
        },
        "also": also,
        "fp8": fp8,
        "all_configs": all_configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

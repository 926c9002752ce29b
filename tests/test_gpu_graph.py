"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph).

No entry point allocates, synchronises or reads a process-wide setting, so
the launches of a whole block, the key-range split with its caller
workspace included, can be captured once and replayed.  Each test captures
the block, then replays the graph several times with the program's own
eager work and synchronisations between replays, and checks every replay
bitwise against the eager result (and that the split leaves its arrival
counts at zero).
"""
import pytest
import torch

import joint_attention_head_amd as fa
from workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _flush(msg):
    print(msg, flush=True)


def prepared(B, H, n_txt, grid, dtype="bf16", seed=0):
    inp = make_inputs(custom_workload(B, H, n_txt, grid, None, dtype, seed))
    d = lambda t: t.to(DEV).contiguous()
    return inp, d


def capture(fn):
    """fn() captured on a side stream after one eager warm-up there."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def replay_and_check(g, outs, refs, ws=None, replays=4):
    for i in range(replays):
        for o in outs:
            o.view(torch.uint8).fill_(0xFF)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {i}"
        if ws is not None:
            assert not ws.counts().any(), f"replay {i}: arrival counts left non-zero"


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_block_with_split_replays_bitwise(dtype):
    """Keys-only prologue + fused attention with a split over 3 workgroups
    (B=1, H=2, N=1000: 8 query blocks cut in key ranges)."""
    _flush(f"graph capture, {dtype} block with split")
    inp, d = prepared(1, 2, 40, (24, 40), dtype, seed=3)
    B, H, N = inp.q.shape[:3]
    q, k, v, w_q, w_k, pos = (d(t) for t in (inp.q, inp.k, inp.v, inp.w_q, inp.w_k, inp.pos))
    kn = torch.empty_like(k)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    ws = fa.split_workspace(B, H, N, 3)
    assert ws.nbytes > 0
    if dtype == "fp8":
        sq, sk, sv = d(inp.q_scale), d(inp.k_scale), d(inp.v_scale)
        skn = torch.empty_like(sk)

        def block():
            fa.fluxattn_qk_norm_rope_fp8(None, k, None, sk, None, w_k, pos, k_out=kn, k_scale_out=skn)
            fa.fluxattn_forward_fused_ex_fp8(q, kn, v, sq, skn, sv, w_q, pos, o=o, split=ws)
    else:
        def block():
            fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos, k_out=kn)
            fa.fluxattn_forward_fused_ex_bf16(q, kn, v, w_q, pos, o=o, split=ws)
    block()
    torch.cuda.synchronize()
    ref, kref = o.clone(), kn.clone()
    g = capture(block)
    replay_and_check(g, [o, kn], [ref, kref], ws)


def test_noalloc_form_replays_bitwise():
    """The static-scratch form after its set-up call (made before capture)."""
    _flush("graph capture, no-alloc form")
    inp, d = prepared(1, 2, 40, (24, 40), "bf16", seed=5)
    q, k, v, w_q, w_k, pos = (d(t) for t in (inp.q, inp.k, inp.v, inp.w_q, inp.w_k, inp.pos))
    kn = fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos)[1]
    o = torch.empty_like(q)

    def block():
        fa.fluxattn_forward_fused_noalloc_bf16(q, kn, v, w_q, pos, o, groups=3)
    block()   # set-up on this device
    torch.cuda.synchronize()
    ref = o.clone()
    ws = fa.split_workspace(1, 2, q.shape[2], 3)
    want = fa.fluxattn_forward_fused_ex_bf16(q, kn, v, w_q, pos, split=ws)
    torch.cuda.synchronize()
    assert torch.equal(ref.view(torch.int16), want.view(torch.int16))
    g = capture(block)
    replay_and_check(g, [o], [ref])

"""fluxattn_forward_fused_noalloc_bf16 through the C ABI: the key-range
split in the library's static scratch instead of a caller workspace, for
code that must not allocate.  It must give bitwise the results of
fluxattn_forward_fused_ex_bf16 with a caller workspace and the same groups
(same kernels, same plan), call after call on the one shared scratch, and
refuse splits larger than the scratch before enqueueing anything."""
import numpy as np
import pytest
import torch

import joint_attention_head_amd as fa
import oracle
from workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_TOL = (2e-2, 2e-3)


def _flush(msg):
    print(msg, flush=True)


def f64(t):
    return oracle.torch_to_f64(t.detach().cpu().contiguous())


def prepared(B, H, n_txt, grid, seed):
    inp = make_inputs(custom_workload(B, H, n_txt, grid, None, "bf16", seed))
    q, k, v = (t.to(DEV) for t in (inp.q, inp.k, inp.v))
    w_q, w_k, pos = inp.w_q.to(DEV), inp.w_k.to(DEV), inp.pos.to(DEV)
    _, kn = fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos)
    return inp, q, kn, v, w_q, pos


def check_against_workspace_form(B, H, n_txt, grid, groups, seed, heads, rows):
    inp, q, kn, v, w_q, pos = prepared(B, H, n_txt, grid, seed)
    N = q.shape[2]
    ws = fa.split_workspace(B, H, N, groups)
    assert ws.nbytes > 0, "this launch is cut"
    ref = fa.fluxattn_forward_fused_ex_bf16(q, kn, v, w_q, pos, split=ws)
    o = torch.full_like(ref, float("nan"))
    _flush(f"noalloc B={B} H={H} N={N} groups={groups}")
    fa.fluxattn_forward_fused_noalloc_bf16(q, kn, v, w_q, pos, o, groups=groups)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
    w_qn, w_kn, posn = inp.w_q.double().numpy(), inp.w_k.double().numpy(), inp.pos.numpy()
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        want = oracle.joint_attention(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), w_qn, w_kn, posn,
                                      rows=rows)[0, 0]
        err = np.abs(f64(o[b, h])[rows] - want)
        _flush(f"  head ({b},{h}) vs oracle: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
        assert err.max() <= BF16_TOL[0] and err.mean() <= BF16_TOL[1]


def test_noalloc_matches_the_workspace_form_on_two_calls():
    """First call: B=1, H=24, N=5632 with the default setting (on 256
    compute units: 256 workgroups, the whole scratch); second call, smaller:
    B=1, H=2, N=1000 over 3 workgroups, on the scratch the first call left
    behind."""
    n = 512 + 64 * 80
    rows = np.unique((np.arange(0, n, 256)[:, None] + np.array([0, 130, 255])).ravel())
    check_against_workspace_form(1, 24, 512, (64, 80), 0, 0, [(0, 11), (0, 23)], rows)
    rows = np.arange(1000)
    check_against_workspace_form(1, 2, 40, (24, 40), 3, 4, [(0, 0), (0, 1)], rows)


def test_noalloc_refuses_a_split_beyond_the_scratch():
    """300 workgroups need more than the 256-workgroup scratch: refused
    before anything runs (the output keeps its contents)."""
    inp, q, kn, v, w_q, pos = prepared(1, 24, 512, (64, 80), 1)
    o = torch.full_like(q, 3.0)
    with pytest.raises(fa.FluxAttnError) as e:
        fa.fluxattn_forward_fused_noalloc_bf16(q, kn, v, w_q, pos, o, groups=300)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)


def test_noalloc_uncut_launch_uses_no_scratch():
    """A setting that does not cut runs the plain fused launch."""
    inp, q, kn, v, w_q, pos = prepared(1, 2, 40, (24, 40), 2)
    o = torch.empty_like(q)
    fa.fluxattn_forward_fused_noalloc_bf16(q, kn, v, w_q, pos, o, groups=-1)
    ref = fa.fluxattn_forward_fused_bf16(q, kn, v, w_q, pos)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), ref.view(torch.int16))

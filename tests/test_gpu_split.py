"""Key-range split of the attention launches, through the C ABI.

With G persistent workgroups each taking an equal share of the (query
block, key tile) pairs, a query block can be computed in several key
ranges whose partial results the last piece to finish merges, in a split
workspace the caller provides.  The split is forced here at sizes the fp64
oracle handles by setting G below or above the number of 256-query blocks;
every case spans several 64-key tiles, with a ragged last key tile and a
ragged last query block.  Checked: parity with the oracle (same tolerances
as the uncut launch), closeness to the uncut launch (a piece that starts
inside a block takes its first row shift from its own first tile, so its P
values are rounded relative to another shift: the two launches differ by
that rounding and fp32 summation order, far inside the oracle tolerance),
bitwise determinism (the merge sums the pieces in share order, so arrival
order does not matter), that a launch leaves the workspace's arrival counts
at zero, and that a short workspace is refused before anything runs.
"""
import numpy as np
import pytest
import torch

import joint_attention_head_amd as fa
import oracle
from workloads import custom_workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_TOL = (2e-2, 2e-3)
FP8_TOL = (4e-2, 4e-3)

# (B, H, text tokens, image grid): N = 1000 (8 query blocks, 16 key tiles,
# the last one 40 keys) and N = 667 (18 blocks, 11 tiles, the last 27 keys)
SHAPES = {"n1000": (1, 2, 40, (24, 40)), "n667": (2, 3, 7, (20, 33))}
# up to 7: whole rounds and a tail cut at most once per block; 12 and more:
# more workgroups than blocks, blocks cut into up to five pieces
GROUPS = (2, 3, 5, 7, 12, 20, 31)


def _flush(msg):
    print(msg, flush=True)


def workspace(inp, groups):
    B, H, N = inp.q.shape[:3]
    ws = fa.split_workspace(B, H, N, groups)
    assert groups <= 1 or ws.nbytes > 0, "forced settings always cut"
    return ws


def inputs(shape, dtype="bf16", seed=0):
    B, H, n_txt, grid = SHAPES[shape]
    return make_inputs(custom_workload(B, H, n_txt, grid, None, dtype, seed))


def dev(t):
    return t.to(DEV).contiguous()


def f64(t, scale=None):
    return oracle.torch_to_f64(t.cpu() if t.is_cuda else t, None if scale is None else scale.cpu())


def check_close(got, ref, tol, what):
    err = np.abs(got - ref)
    _flush(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert np.isfinite(got).all(), what
    assert err.max() <= tol[0], (what, err.max())
    assert err.mean() <= tol[1], (what, err.mean())


# split vs uncut launch: P rounding (bf16: 2^-9 relative, E4M3: 2^-4) of
# the same probabilities against another row shift
UNCUT_TOL = {"bf16": (4e-3, 2e-4), "fp8": (2e-2, 2e-3)}


def close_to_uncut(a, b, dtype, what):
    d = np.abs(f64(a) - f64(b))
    _flush(f"{what}: split vs uncut max diff {d.max():.3e} mean {d.mean():.3e}")
    assert d.max() <= UNCUT_TOL[dtype][0], what
    assert d.mean() <= UNCUT_TOL[dtype][1], what


def n_blocks(inp):
    B, H, N = inp.q.shape[:3]
    return B * H * ((N + 255) // 256)


def forward_bf16(inp, split=None):
    return fa.fluxattn_forward_ex_bf16(dev(inp.q), dev(inp.k), dev(inp.v), split=split)


def joint_bf16(inp, split=None):
    return fa.fluxattn_joint_attention_ex_bf16(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.w_q), dev(inp.w_k),
                                               dev(inp.pos), split=split)


def forward_fp8(inp, split=None):
    return fa.fluxattn_forward_ex_fp8(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.q_scale), dev(inp.k_scale),
                                      dev(inp.v_scale), split=split)


def joint_fp8(inp, split=None):
    return fa.fluxattn_joint_attention_ex_fp8(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.q_scale),
                                              dev(inp.k_scale), dev(inp.v_scale), dev(inp.w_q), dev(inp.w_k),
                                              dev(inp.pos), split=split)


def attention_ref(inp):
    if inp.q.dtype == torch.float8_e4m3fn:
        return oracle.attention(f64(inp.q, inp.q_scale), f64(inp.k, inp.k_scale), f64(inp.v, inp.v_scale))
    return oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v))


def joint_ref(inp):
    sc = lambda t, s: f64(t, s) if t.dtype == torch.float8_e4m3fn else f64(t)
    return oracle.joint_attention(sc(inp.q, inp.q_scale), sc(inp.k, inp.k_scale), sc(inp.v, inp.v_scale),
                                  inp.w_q.double().numpy(), inp.w_k.double().numpy(), inp.pos.numpy())


PATHS = {
    "forward_bf16": (forward_bf16, attention_ref, "bf16", BF16_TOL),
    "joint_fused_bf16": (joint_bf16, joint_ref, "bf16", BF16_TOL),
    "forward_fp8": (forward_fp8, attention_ref, "fp8", FP8_TOL),
    "joint_fused_fp8": (joint_fp8, joint_ref, "fp8", FP8_TOL),
}


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("path", list(PATHS))
def test_split_matches_oracle_and_uncut_launch(path, shape):
    run, ref_fn, dtype, tol = PATHS[path]
    inp = inputs(shape, dtype)
    ref = ref_fn(inp)
    whole = run(inp)
    for g in GROUPS:
        _flush(f"split {path} {shape} groups={g}")
        ws = workspace(inp, g)
        o = run(inp, ws)
        torch.cuda.synchronize()
        check_close(f64(o), ref, tol, f"split {path} {shape} G={g}")
        close_to_uncut(o, whole, dtype, f"split {path} {shape} G={g}")
        assert not ws.counts().any(), "arrival counts left non-zero"


def test_split_is_deterministic_and_leaves_counts_at_zero():
    a, b = inputs("n1000", seed=0), inputs("n1000", seed=5)
    ws = workspace(a, 3)
    o1 = forward_bf16(a, ws)
    ob = forward_bf16(b, ws)     # other inputs: stale counts would merge a's partials
    o2 = forward_bf16(a, ws)
    torch.cuda.synchronize()
    assert not ws.counts().any()
    check_close(f64(ob), attention_ref(b), BF16_TOL, "split second launch, other inputs")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_split_strided_layout():
    """The ex entry point on [B, N, H, D] storage (token-major), cut."""
    inp = inputs("n667")
    B, H, N, D = inp.q.shape
    tm = lambda t: t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3)
    q, k, v = tm(inp.q), tm(inp.k), tm(inp.v)
    o = torch.empty(B, N, H, D, dtype=torch.bfloat16, device=DEV).permute(0, 2, 1, 3)
    fa.fluxattn_forward_ex_bf16(q, k, v, o=o, split=workspace(inp, 5))
    torch.cuda.synchronize()
    check_close(f64(o), attention_ref(inp), BF16_TOL, "split strided n667 G=5")


def test_split_default_setting_cuts_three_rounds():
    """B=1, H=24, N = 512 + 64x80 = 5632: 528 query blocks, just over two
    rounds of 256 compute units, so the default setting (groups = 0) cuts
    the tail (one whole round, then 272 blocks shared by all workgroups).
    The workspace query says so, the result differs bitwise from the uncut
    launch (so the cut happened), stays close to it, and matches the oracle
    on rows of every query block of a whole-round head (0), the head where
    the tail starts (11) and the last head (23)."""
    w = custom_workload(1, 24, 512, (64, 80))
    inp = make_inputs(w)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 24 * ((w.N + 255) // 256)
    assert blocks >= 2 * cus and blocks % cus, (blocks, cus)   # the default rule cuts this shape
    ws = fa.split_workspace(1, 24, w.N, 0)
    assert ws.nbytes > 0
    o = forward_bf16(inp, ws)
    whole = forward_bf16(inp)
    torch.cuda.synchronize()
    assert not torch.equal(o.view(torch.int16), whole.view(torch.int16))
    close_to_uncut(o, whole, "bf16", "default setting N=5632")
    assert not ws.counts().any()
    rows = np.unique(np.concatenate([np.arange(0, w.N, 256)[:, None] + np.array([0, 97, 200, 255])]).ravel())
    rows = rows[rows < w.N]
    for h in (0, 11, 23):
        sl = (slice(0, 1), slice(h, h + 1))
        ref = oracle.attention(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), rows=rows)
        check_close(f64(o[sl])[:, :, rows], ref, BF16_TOL, f"default setting N=5632 head {h}")


def test_split_on_two_streams_at_once():
    """Cut launches on two streams that run at the same time, each with its
    own workspace, give bitwise the results of running them one after the
    other."""
    a, b = inputs("n1000", seed=0), inputs("n1000", seed=7)
    qa, ka, va = dev(a.q), dev(a.k), dev(a.v)
    qb, kb, vb = dev(b.q), dev(b.k), dev(b.v)
    wa, wb = workspace(a, 3), workspace(b, 3)
    ref_a = fa.fluxattn_forward_ex_bf16(qa, ka, va, split=wa)
    ref_b = fa.fluxattn_forward_ex_bf16(qb, kb, vb, split=wb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(4):
        with torch.cuda.stream(s1):
            oa = fa.fluxattn_forward_ex_bf16(qa, ka, va, split=wa)
        with torch.cuda.stream(s2):
            ob = fa.fluxattn_forward_ex_bf16(qb, kb, vb, split=wb)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa.view(torch.int16), ref_a.view(torch.int16))
        assert torch.equal(ob.view(torch.int16), ref_b.view(torch.int16))
    check_close(f64(ref_b), attention_ref(b), BF16_TOL, "split, second stream's inputs")


def test_split_many_pieces_flux_dev_512():
    """FLUX-dev 512x512 (B=1, H=24, N=1536: 144 query blocks of 24 key
    tiles) over 256 workgroups: more workgroups than blocks, every block cut
    into two or three pieces (shares of 13.5 tiles); close to the uncut
    launch, and the oracle on sampled rows of two heads.  (The default
    setting leaves this size uncut: measured faster.)"""
    inp = make_inputs(custom_workload(1, 24, 512, (32, 32)))
    o = forward_bf16(inp, workspace(inp, 256))
    whole = forward_bf16(inp)
    torch.cuda.synchronize()
    close_to_uncut(o, whole, "bf16", "256 workgroups N=1536")
    rows = np.unique(np.concatenate([np.arange(40), np.arange(1500, 1536), np.arange(0, 1536, 37)]))
    for h in (0, 23):
        sl = (slice(0, 1), slice(h, h + 1))
        ref = oracle.attention(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), rows=rows)
        check_close(f64(o[sl])[:, :, rows], ref, BF16_TOL, f"256 workgroups N=1536 head {h}")


def test_split_workspace_shared_across_group_counts():
    """Launches with different group counts share one workspace: a small
    count's partial slots must not land on the arrival counts a larger
    count expects at zero (G = 100 needs 200 counts, G = 5 ten).  G = 100
    also cuts each of the 8 blocks into about a dozen pieces."""
    inp = inputs("n1000")
    whole = forward_bf16(inp)
    ref = attention_ref(inp)
    ws = workspace(inp, 100)
    for g in (100, 5, 100, 5):
        ws.groups = g
        o = forward_bf16(inp, ws)
        torch.cuda.synchronize()
        check_close(f64(o), ref, BF16_TOL, f"shared workspace G={g}")
        close_to_uncut(o, whole, "bf16", f"shared workspace G={g}")


def test_short_or_missing_workspace_is_refused_before_launch():
    """A cut launch without enough workspace returns FLUXATTN_ERR_WORKSPACE
    and enqueues nothing (the output keeps its contents); a launch that is
    not cut needs none."""
    inp = inputs("n667")
    B, H, N = inp.q.shape[:3]
    need = fa.fluxattn_split_workspace_bytes(B, H, N, 5)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    o = torch.full(inp.q.shape, 7.0, dtype=torch.bfloat16, device=DEV)
    for ws in (fa.SplitWorkspace(5, 0), fa.SplitWorkspace(5, need - 256)):
        with pytest.raises(fa.FluxAttnError) as e:
            fa.fluxattn_forward_ex_bf16(q, k, v, o=o, split=ws)
        assert e.value.status == 7
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
    # uncut settings run without a workspace
    for g in (-1, 1):
        fa.fluxattn_forward_ex_bf16(q, k, v, o=o, split=fa.SplitWorkspace(g, 0))
    torch.cuda.synchronize()
    check_close(f64(o), attention_ref(inp), BF16_TOL, "uncut setting, no workspace")


def test_split_default_setting_between_one_and_two_rounds():
    """B=1, H=18, N = 512 + 64x64 = 4608: 324 query blocks, 1.27 rounds of
    256 compute units, the second round 27% full.  The default setting runs
    one whole round and cuts the other 68 blocks into pieces shared by all
    workgroups (shares of about 19 key tiles, so each block has several
    pieces).  It differs bitwise from the uncut launch (the cut happened),
    stays close to it, leaves the counts at zero and matches the oracle on
    rows of every query block of a whole-round head (0) and of the heads
    the tail covers (14, 17).  At H=24 (432 blocks, the second round 69%
    full) the default runs uncut."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"shape chosen for 256 compute units, device has {cus}")
    assert fa.split_workspace(1, 24, 4608, 0).nbytes == 0
    w = custom_workload(1, 18, 512, (64, 64))
    inp = make_inputs(w)
    ws = fa.split_workspace(1, 18, w.N, 0)
    assert ws.nbytes > 0
    o = forward_bf16(inp, ws)
    whole = forward_bf16(inp)
    torch.cuda.synchronize()
    assert not torch.equal(o.view(torch.int16), whole.view(torch.int16))
    close_to_uncut(o, whole, "bf16", "default setting H=18 N=4608")
    assert not ws.counts().any()
    rows = np.unique(np.concatenate([np.arange(0, w.N, 256)[:, None] + np.array([0, 131, 255])]).ravel())
    rows = rows[rows < w.N]
    for h in (0, 14, 17):
        sl = (slice(0, 1), slice(h, h + 1))
        ref = oracle.attention(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), rows=rows)
        check_close(f64(o[sl])[:, :, rows], ref, BF16_TOL, f"default setting H=18 N=4608 head {h}")

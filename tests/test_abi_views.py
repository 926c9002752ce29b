"""The strided, multi-stream entry points (*_ex) without a GPU: layout and
stream validation, the aliasing rules for views that share a packed QKV
tensor, and the binding's layout helpers.  Calls use fake device addresses
and never get past validation (a valid call stops at the device check)."""
import ctypes

import pytest
import torch

import joint_attention_head_amd as fa

OK, NULLP, SHAPE, ALIGN, ALIAS, NODEV, HIPERR, WORKSPACE = range(8)

B, H, N, D = 2, 3, 320, 128
WQ, WK, POS = 0x90000000, 0x90001000, 0x90002000
SQ, SK, SV, SQO, SKO, SKW = (0xA0000000 + 0x1000 * i for i in range(6))
KW = 0x70000000
# separate contiguous tensors
Q, K, V, O, QO, KO = (0x10000000 * (i + 1) for i in range(6))
# one packed [B, N, 3, H, D] projection output: q, k, v interleave per token
P = 0x80000000


def contig(h=H, n=N, d=D):
    return fa.Layout(h * n * d, n * d, d)


def packed(h=H, n=N, d=D):
    return fa.Layout(n * 3 * h * d, d, 3 * h * d)


def bnhd(h=H, n=N, d=D):
    return fa.Layout(n * h * d, d, h * d)


def has_gpu():
    try:
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="module")
def lib():
    if has_gpu():
        pytest.skip("a GPU is present: fake pointers must not reach a launch")
    return fa.lib()


def streams(*starts):
    return fa.streams_of(starts)


def prologue(lib, q=Q, lq=None, k=K, lk=None, qo=QO, lqo=None, ko=KO, lko=None, wq=WQ, wk=WK, st=None,
             n=N):
    lq, lk, lqo, lko = (x or contig(n=n) for x in (lq, lk, lqo, lko))
    st = st or streams(0)
    return lib.fluxattn_qk_norm_rope_ex_bf16(q, lq, k, lk, qo, lqo, ko, lko, wq, wk, st, POS, B, H, n, D,
                                             16, 56, 56, 1e4, 1e-6, None)


def prologue8(lib, q=Q, lq=None, k=K, lk=None, qo=QO, lqo=None, ko=KO, lko=None, sqo=SQO, sko=SKO, st=None):
    lq, lk, lqo, lko = (x or contig() for x in (lq, lk, lqo, lko))
    st = st or streams(0)
    return lib.fluxattn_qk_norm_rope_ex_fp8(q, lq, k, lk, SQ, SK, qo, lqo, ko, lko, sqo, sko, WQ, WK, st, POS,
                                            B, H, N, D, 16, 56, 56, 1e4, 1e-6, None)


def split_arg(split):
    return None if split is None else ctypes.byref(split)


def forward(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, o=O, lo=None, n=N, split=None):
    lq, lk, lv, lo = (x or contig(n=n) for x in (lq, lk, lv, lo))
    return lib.fluxattn_forward_ex_bf16(q, lq, k, lk, v, lv, o, lo, B, H, n, D, 0.0, split_arg(split), None)


def forward8(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, o=O, lo=None, split=None):
    lq, lk, lv, lo = (x or contig() for x in (lq, lk, lv, lo))
    return lib.fluxattn_forward_ex_fp8(q, lq, k, lk, v, lv, SQ, SK, SV, o, lo, B, H, N, D, 0.0, split_arg(split),
                                       None)


def fused(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, o=O, lo=None, wq=WQ, st=None, split=None):
    lq, lk, lv, lo = (x or contig() for x in (lq, lk, lv, lo))
    st = st or streams(0)
    return lib.fluxattn_forward_fused_ex_bf16(q, lq, k, lk, v, lv, o, lo, wq, st, POS, B, H, N, D, 16, 56, 56, 1e4,
                                              1e-6, 0.0, split_arg(split), None)


def fused8(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, o=O, lo=None, st=None, split=None):
    lq, lk, lv, lo = (x or contig() for x in (lq, lk, lv, lo))
    st = st or streams(0)
    return lib.fluxattn_forward_fused_ex_fp8(q, lq, k, lk, v, lv, SQ, SK, SV, o, lo, WQ, st, POS, B, H, N, D, 16,
                                             56, 56, 1e4, 1e-6, 0.0, split_arg(split), None)


def joint(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, kw=KW, o=O, lo=None, wq=WQ, wk=WK, st=None,
          split=None):
    lq, lk, lv, lo = (x or contig() for x in (lq, lk, lv, lo))
    st = st or streams(0)
    return lib.fluxattn_joint_attention_ex_bf16(q, lq, k, lk, v, lv, kw, o, lo, wq, wk, st, POS, B, H, N, D,
                                                16, 56, 56, 1e4, 1e-6, 0.0, split_arg(split), None)


def joint8(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, kw=KW, skw=SKW, o=O, lo=None, st=None, split=None):
    lq, lk, lv, lo = (x or contig() for x in (lq, lk, lv, lo))
    st = st or streams(0)
    return lib.fluxattn_joint_attention_ex_fp8(q, lq, k, lk, v, lv, SQ, SK, SV, kw, skw, o, lo, WQ, WK, st, POS,
                                               B, H, N, D, 16, 56, 56, 1e4, 1e-6, 0.0, split_arg(split), None)


def test_contiguous_layouts_and_one_stream_are_valid(lib):
    assert prologue(lib) == NODEV
    assert prologue8(lib) == NODEV
    assert forward(lib) == NODEV
    assert forward8(lib) == NODEV
    assert fused(lib) == NODEV
    assert fused8(lib) == NODEV
    assert joint(lib) == NODEV
    assert joint8(lib) == NODEV


def noalloc(lib, q=Q, lq=None, k=K, lk=None, v=V, lv=None, o=O, lo=None, st=None, groups=0):
    lq, lk, lv, lo = (x or contig() for x in (lq, lk, lv, lo))
    st = st or streams(0)
    return lib.fluxattn_forward_fused_noalloc_bf16(q, lq, k, lk, v, lv, o, lo, WQ, st, POS, B, H, N, D, 16, 56, 56,
                                                   1e4, 1e-6, 0.0, groups, None)


def test_noalloc_entry_point_validates_like_the_workspace_form(lib):
    """The static-scratch form runs every check of the fused _ex form before
    it looks up its scratch: without a GPU a valid call stops at the device
    check, and argument errors come first."""
    assert noalloc(lib) == NODEV
    assert noalloc(lib, groups=5) == NODEV
    assert noalloc(lib, groups=16385) == SHAPE
    assert noalloc(lib, q=None) == NULLP
    assert noalloc(lib, q=Q + 8) == ALIGN
    assert noalloc(lib, o=Q) == ALIAS
    assert noalloc(lib, lo=fa.Layout(0, 0, 64)) == SHAPE


def test_split_groups_are_validated_before_the_device(lib):
    """A split setting above 16384 workgroups is an invalid parameter;
    a valid one (even without a workspace) gets as far as the device check:
    the workspace is checked after it, against the device's plan."""
    for g, want in ((16385, SHAPE), (16384, NODEV), (5, NODEV), (0, NODEV), (-1, NODEV)):
        sp = fa.Split(g, None, 0)
        for call in (forward, forward8, fused, fused8, joint, joint8):
            assert call(lib, split=sp) == want, (call.__name__, g)


def test_packed_qkv_views_are_valid_and_disjoint(lib):
    e = 2 * H * D  # bytes between the q, k and v slices of one token row (bf16)
    lp = packed()
    assert forward(lib, q=P, lq=lp, k=P + e, lk=lp, v=P + 2 * e, lv=lp) == NODEV
    assert forward(lib, q=P, lq=lp, k=P + e, lk=lp, v=P + 2 * e, lv=lp, lo=bnhd()) == NODEV
    # prologue in place on the packed tensor: each output is its own input
    assert prologue(lib, q=P, lq=lp, k=P + e, lk=lp, qo=P, lqo=lp, ko=P + e, lko=lp) == NODEV
    # fp8 packed tensor: slices are H*D bytes apart
    e8 = H * D
    assert forward8(lib, q=P, lq=lp, k=P + e8, lk=lp, v=P + 2 * e8, lv=lp) == NODEV
    assert prologue8(lib, q=P, lq=lp, k=P + e8, lk=lp, qo=P, lqo=lp, ko=P + e8, lko=lp) == NODEV
    assert joint(lib, q=P, lq=lp, k=P + e, lk=lp, v=P + 2 * e, lv=lp) == NODEV
    assert joint8(lib, q=P, lq=lp, k=P + e8, lk=lp, v=P + 2 * e8, lv=lp) == NODEV


def test_overlapping_views_are_aliasing(lib):
    lp = packed()
    e = 2 * H * D
    # slices that overlap inside a token row
    assert prologue(lib, q=P, lq=lp, k=P + e - 16, lk=lp, qo=P, lqo=lp, ko=P + e - 16, lko=lp) == ALIAS
    # in place only with the same layout
    assert prologue(lib, q=P, lq=lp, k=P + e, lk=lp, qo=P, lqo=bnhd(), ko=P + e, lko=lp) == ALIAS
    # the output may not land inside the packed input
    assert forward(lib, q=P, lq=lp, k=P + e, lk=lp, v=P + 2 * e, lv=lp, o=P + 2 * e, lo=lp) == ALIAS
    # k_work is contiguous: in place needs a contiguous k
    assert joint(lib, q=P, lq=lp, k=P + e, lk=lp, v=P + 2 * e, lv=lp, kw=P + e) == ALIAS
    assert joint(lib, kw=K) == NODEV
    # views with different strides and overlapping extents are not proven apart
    assert forward(lib, o=Q + 4096, lo=bnhd()) == ALIAS


def test_per_stream_weights_extend_the_aliasing_ranges(lib):
    row = 4 * D  # bytes of one fp32 weight row
    # q_norm_w right before q_out: one row ends where q_out starts ...
    assert prologue(lib, wq=QO - row) == NODEV
    # ... two rows reach into it
    assert prologue(lib, wq=QO - row, st=streams(0, 100)) == ALIAS
    assert prologue(lib, wq=QO - 2 * row, st=streams(0, 100)) == NODEV
    assert prologue(lib, wq=QO - 2 * row, st=streams(0, 100, 200)) == ALIAS
    assert joint(lib, wq=O - row) == NODEV
    assert joint(lib, wq=O - row, st=streams(0, 64)) == ALIAS
    # fp8 scale outputs against the second weight row
    assert prologue8(lib, sqo=WQ + row) == NODEV
    assert prologue8(lib, sqo=WQ + row, st=streams(0, 64)) == ALIAS


def test_invalid_layouts(lib):
    c = contig()
    bad = [
        fa.Layout(c.b_stride, c.h_stride, D - 8),        # token rows overlap
        fa.Layout(c.b_stride, c.h_stride, D + 4),        # 8-byte row pitch breaks 16-byte alignment
        fa.Layout(-c.b_stride, c.h_stride, c.n_stride),  # negative stride
        fa.Layout(c.b_stride + 4, c.h_stride, D),        # batch stride not a 16-byte multiple
        fa.Layout(c.b_stride, c.h_stride, 1 << 29),      # padded head spans 2^32 bytes or more
    ]
    for l in bad:
        assert forward(lib, lq=l) == SHAPE, (l.b_stride, l.h_stride, l.n_stride)
        assert forward(lib, lk=l) == SHAPE
        assert forward(lib, lv=l) == SHAPE
        assert forward(lib, lo=l) == SHAPE
        assert prologue(lib, lk=l) == SHAPE
        assert prologue(lib, lqo=l) == SHAPE
        assert joint(lib, lq=l) == SHAPE
        assert joint8(lib, lv=l) == SHAPE
    # an output whose heads share memory is not one-to-one
    shared = fa.Layout(N * D, 0, D)
    assert forward(lib, lo=shared) == SHAPE
    assert prologue(lib, lko=shared) == SHAPE
    # ... while an input may broadcast over heads
    assert forward(lib, lk=shared) == NODEV
    # Within one head, the last row of the padded 256-row query block must
    # start below 2^32 bytes.  q broadcast over b and h, far from the rest:
    far = 0x1000000000
    rest = dict(lk=contig(n=257), lv=contig(n=257), lo=contig(n=257))
    r22 = fa.Layout(0, 0, (1 << 22) // 2)  # 2^22-byte token rows: 511 rows fit
    assert forward(lib, q=far, lq=r22, n=257, **rest) == NODEV
    r24 = fa.Layout(0, 0, (1 << 24) // 2)  # 2^24-byte rows: 511 rows do not
    assert forward(lib, q=far, lq=r24, n=257, **rest) == SHAPE
    # N = 200 pads to 256 rows: 255 rows of 2^24 bytes plus one row fit
    rest = dict(lk=contig(n=200), lv=contig(n=200), lo=contig(n=200))
    assert forward(lib, q=far, lq=r24, n=200, **rest) == NODEV


def test_invalid_streams(lib):
    for bad in (fa.Streams(0, (0, 0, 0, 0)), fa.Streams(5, (0, 1, 2, 3)), fa.Streams(2, (1, 5, 0, 0)),
                fa.Streams(3, (0, 200, 100, 0)), fa.Streams(2, (0, N + 1, 0, 0)), fa.Streams(2, (0, -1, 0, 0))):
        assert prologue(lib, st=bad) == SHAPE, list(bad.start)[:bad.count]
        assert prologue8(lib, st=bad) == SHAPE
        assert joint(lib, st=bad) == SHAPE
        assert joint8(lib, st=bad) == SHAPE
    # empty streams and a stream that starts at N are allowed
    assert prologue(lib, st=streams(0, 0, N)) == NODEV
    assert joint(lib, st=streams(0, 0, 100, N)) == NODEV
    # entries past count are ignored
    assert prologue(lib, st=fa.Streams(1, (0, -7, 99999, 3))) == NODEV


def test_null_and_alignment_rules_follow_the_contiguous_forms(lib):
    lp = packed()
    assert forward(lib, q=None) == NULLP
    assert joint(lib, kw=None) == NULLP
    assert prologue(lib, q=None, qo=None, wq=None) == NODEV  # keys only
    assert prologue(lib, q=None, qo=None) == NULLP
    assert forward(lib, q=P + 8, lq=lp) == ALIGN
    assert joint(lib, wq=WQ + 4) == ALIGN


def test_binding_layouts_of_torch_views():
    qkv = torch.empty(B, N, 3, H, D, dtype=torch.bfloat16)
    q = qkv[:, :, 0].permute(0, 2, 1, 3)
    k = qkv[:, :, 1].permute(0, 2, 1, 3)
    assert tuple(q.shape) == (B, H, N, D)
    lq = fa.layout_of(q)
    assert (lq.b_stride, lq.h_stride, lq.n_stride) == (N * 3 * H * D, D, 3 * H * D)
    assert k.data_ptr() - q.data_ptr() == H * D * 2
    c = fa.layout_of(torch.empty(B, H, N, D))
    assert (c.b_stride, c.h_stride, c.n_stride) == (H * N * D, N * D, D)
    with pytest.raises(ValueError):
        fa.layout_of(torch.empty(B, H, D, N).transpose(2, 3))
    s = fa.streams_of((0, 512))
    assert s.count == 2 and list(s.start)[:2] == [0, 512]
    with pytest.raises(ValueError):
        fa.streams_of(())
    with pytest.raises(ValueError):
        fa.fluxattn_forward_ex_bf16(q, k, k)   # CPU tensors

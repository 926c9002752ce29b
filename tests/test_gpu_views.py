"""Parity of the strided, multi-stream entry points (*_ex) on the GPU.

q, k and v are slices of one packed [B, N, 3, H, D] projection output (the
layout a fused QKV GEMM writes), outputs are contiguous or [B, N, H, D], and
the RMSNorm weights differ per token stream (text, target image, reference
image).  Each case is checked against the fp64 oracle with per-token weights
and, where the arithmetic is the same, bitwise against the contiguous entry
points on the same values.
"""
import numpy as np
import pytest
import torch

import joint_attention_head_amd as fa
import oracle
from workloads import custom_workload, make_inputs, stream_norm_weights, stream_starts

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_TOL = (2e-2, 2e-3)
FP8_TOL = (4e-2, 4e-3)


def _flush(msg):
    print(msg, flush=True)


def small(B, H, n_txt, grid, ref_grid=None, dtype="bf16", seed=0):
    w = custom_workload(B, H, n_txt, grid, ref_grid, dtype, seed)
    return w, make_inputs(w)


def f64(t, scale=None):
    return oracle.torch_to_f64(t.detach().cpu().contiguous(), None if scale is None else scale.cpu())


def dev(t):
    return t.to(DEV).contiguous()


def bits(t):
    return t.contiguous().view(torch.uint8)


def packed(q, k, v):
    """Packed [B, N, 3, H, D] device tensor and its [B, H, N, D] q, k, v views."""
    p = torch.stack([q, k, v], dim=2).permute(0, 3, 2, 1, 4).contiguous().to(DEV)
    return p, [p[:, :, i].permute(0, 2, 1, 3) for i in range(3)]


def bnhd_empty(B, H, N, D, dtype):
    """A [B, H, N, D] view of a fresh [B, N, H, D] tensor."""
    return torch.empty(B, N, H, D, dtype=dtype, device=DEV).permute(0, 2, 1, 3)


def check_close(got, ref, tol, what):
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    _flush(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), what
    assert err.max() <= tol[0], (what, err.max())
    assert err.mean() <= tol[1], (what, err.mean())
    return rel


def pair_norm(y):
    n = np.sqrt(y[..., 0::2] ** 2 + y[..., 1::2] ** 2)
    return np.repeat(n, 2, axis=-1)


CASES = {
    "t2i_77+256_B2": lambda: small(2, 3, 77, (16, 16)),
    "i2i_9+120+42": lambda: small(1, 2, 9, (10, 12), (6, 7), seed=1),
    "tiny_64+256": lambda: small(1, 2, 64, (16, 16), seed=2),
    "n65": lambda: small(2, 1, 1, (8, 8), seed=3),
}


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("case", list(CASES))
def test_forward_ex_bf16_packed_matches_contiguous_bitwise(case):
    _flush(f"forward_ex bf16 packed {case}")
    _, inp = CASES[case]()
    B, H, N, D = inp.q.shape
    p, (qv, kv, vv) = packed(inp.q, inp.k, inp.v)
    p_keep = p.clone()
    o_ref = fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k), dev(inp.v))
    o = fa.fluxattn_forward_ex_bf16(qv, kv, vv)
    o2 = fa.fluxattn_forward_ex_bf16(qv, kv, vv, o=bnhd_empty(B, H, N, D, torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(bits(o), bits(o_ref))
    assert torch.equal(bits(o2), bits(o_ref))
    assert torch.equal(bits(p), bits(p_keep))
    ref = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v))
    check_close(f64(o), ref, BF16_TOL, f"forward_ex bf16 {case}")


def test_forward_ex_bf16_bnhd_output_leaves_neighbours_alone():
    """Output into the even heads of a [B, N, 2H, D] buffer: the odd heads
    keep their contents."""
    _, inp = small(1, 2, 13, (9, 9), seed=5)
    B, H, N, D = inp.q.shape
    buf = torch.full((B, N, 2 * H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    o = buf[:, :, 0::2].permute(0, 2, 1, 3)
    fa.fluxattn_forward_ex_bf16(dev(inp.q), dev(inp.k), dev(inp.v), o=o)
    o_ref = fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    assert torch.equal(bits(o), bits(o_ref))
    assert torch.all(buf[:, :, 1::2] == 7.0)


def test_forward_ex_fp8_packed_matches_contiguous_bitwise():
    for case in ("t2i_77+256_B2", "i2i_9+120+42"):
        _flush(f"forward_ex fp8 packed {case}")
        w, _ = CASES[case]()
        inp = make_inputs(custom_workload(w.B, w.H, w.n_txt, w.grid, w.ref_grid, "fp8", w.seed))
        p, (qv, kv, vv) = packed(inp.q.view(torch.uint8), inp.k.view(torch.uint8), inp.v.view(torch.uint8))
        qv, kv, vv = (t.view(torch.float8_e4m3fn) for t in (qv, kv, vv))
        sc = [dev(s) for s in (inp.q_scale, inp.k_scale, inp.v_scale)]
        o_ref = fa.fluxattn_forward_fp8(dev(inp.q), dev(inp.k), dev(inp.v), *sc)
        o = fa.fluxattn_forward_ex_fp8(qv, kv, vv, *sc)
        torch.cuda.synchronize()
        assert torch.equal(bits(o), bits(o_ref))
        ref = oracle.attention(f64(inp.q, inp.q_scale), f64(inp.k, inp.k_scale), f64(inp.v, inp.v_scale))
        check_close(f64(o), ref, FP8_TOL, f"forward_ex fp8 {case}")


# ------------------------------------------------------------------ prologue

@pytest.mark.parametrize("case", ["t2i_77+256_B2", "i2i_9+120+42"])
def test_prologue_ex_bf16_streams_in_place_on_packed(case):
    _flush(f"prologue_ex bf16 streams {case}")
    w, inp = CASES[case]()
    starts = stream_starts(w)
    w_q, w_k = stream_norm_weights(len(starts), seed=w.seed)
    N = w.N
    p, (qv, kv, vv) = packed(inp.q, inp.k, inp.v)
    v_keep = vv.clone()
    fa.fluxattn_qk_norm_rope_ex_bf16(qv, kv, dev(w_q), dev(w_k), dev(inp.pos), streams=starts, q_out=qv, k_out=kv)
    torch.cuda.synchronize()
    assert torch.equal(bits(vv), bits(v_keep))
    wq_tok = oracle.stream_weights(w_q.double().numpy(), starts, N)
    wk_tok = oracle.stream_weights(w_k.double().numpy(), starts, N)
    rq, rk = oracle.qk_prologue(f64(inp.q), f64(inp.k), wq_tok, wk_tok, inp.pos.numpy())
    for got, ref, name in ((f64(qv), rq, "q"), (f64(kv), rk, "k")):
        bound = 2.0 ** -8 * np.abs(ref) + 4e-5 * np.maximum(pair_norm(ref), 1.0)
        bad = np.abs(got - ref) > bound
        _flush(f"  {name}: max_err={np.abs(got - ref).max():.3e} violations={bad.sum()}")
        assert not bad.any()
    # with every stream on the same weights the result is the one-stream call's
    same_q, same_k = w_q[:1].expand(len(starts), -1).contiguous(), w_k[:1].expand(len(starts), -1).contiguous()
    a_q, a_k = fa.fluxattn_qk_norm_rope_ex_bf16(dev(inp.q), dev(inp.k), dev(same_q), dev(same_k), dev(inp.pos),
                                                streams=starts)
    b_q, b_k = fa.fluxattn_qk_norm_rope_bf16(dev(inp.q), dev(inp.k), dev(w_q[0]), dev(w_k[0]), dev(inp.pos))
    torch.cuda.synchronize()
    assert torch.equal(bits(a_q), bits(b_q)) and torch.equal(bits(a_k), bits(b_k))


def test_prologue_ex_fp8_streams():
    w, _ = CASES["i2i_9+120+42"]()
    inp = make_inputs(custom_workload(w.B, w.H, w.n_txt, w.grid, w.ref_grid, "fp8", 7))
    starts = stream_starts(w)
    w_q, w_k = stream_norm_weights(len(starts), seed=7)
    w_k[2] *= 1.5  # the scale follows the largest weight of any stream
    qo, ko, sqo, sko = fa.fluxattn_qk_norm_rope_ex_fp8(dev(inp.q), dev(inp.k), dev(inp.q_scale), dev(inp.k_scale),
                                                       dev(w_q), dev(w_k), dev(inp.pos), streams=starts)
    torch.cuda.synchronize()
    wq_tok = oracle.stream_weights(w_q.double().numpy(), starts, w.N)
    wk_tok = oracle.stream_weights(w_k.double().numpy(), starts, w.N)
    rq, rk = oracle.qk_prologue(f64(inp.q, inp.q_scale), f64(inp.k, inp.k_scale), wq_tok, wk_tok, inp.pos.numpy())
    for got8, s_out, ref, wr, name in ((qo, sqo, rq, w_q, "q"), (ko, sko, rk, w_k, "k")):
        s_ref = oracle.fp8_prologue_out_scale(wr.double().numpy())
        np.testing.assert_allclose(s_out.cpu().double().numpy(), s_ref, rtol=1e-6)
        got = f64(got8, s_out)
        bound = 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * s_ref + 4e-5 * np.maximum(pair_norm(ref), 1.0)
        bad = np.abs(got - ref) > bound
        _flush(f"  fp8 {name}: max_err={np.abs(got - ref).max():.3e} violations={bad.sum()}")
        assert not bad.any()


# ------------------------------------------------------------------ the whole block

def joint_ref(inp, starts, w_q, w_k, fp8=False, heads=None, rows=None):
    N = inp.q.shape[2]
    wq_tok = oracle.stream_weights(w_q.double().numpy(), starts, N)
    wk_tok = oracle.stream_weights(w_k.double().numpy(), starts, N)
    pos = inp.pos.numpy()
    sc = lambda t, s, sl: f64(t[sl], s[sl] if fp8 else None)
    heads = heads or [(b, h) for b in range(inp.q.shape[0]) for h in range(inp.q.shape[1])]
    out = []
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        out.append(oracle.joint_attention(sc(inp.q, inp.q_scale, sl), sc(inp.k, inp.k_scale, sl),
                                          sc(inp.v, inp.v_scale, sl), wq_tok, wk_tok, pos, rows=rows)[0, 0])
    return np.stack(out)


@pytest.mark.parametrize("case", list(CASES))
def test_joint_ex_bf16_packed_streams_parity(case):
    _flush(f"joint_ex bf16 packed streams {case}")
    w, inp = CASES[case]()
    starts = stream_starts(w)
    w_q, w_k = stream_norm_weights(len(starts), seed=w.seed)
    p, (qv, kv, vv) = packed(inp.q, inp.k, inp.v)
    p_keep = p.clone()
    o = fa.fluxattn_joint_attention_ex_bf16(qv, kv, vv, dev(w_q), dev(w_k), dev(inp.pos), streams=starts)
    torch.cuda.synchronize()
    assert torch.equal(bits(p), bits(p_keep))
    B, H = inp.q.shape[:2]
    got = np.stack([f64(o[b, h]) for b in range(B) for h in range(H)])
    rel = check_close(got, joint_ref(inp, starts, w_q, w_k), BF16_TOL, f"joint_ex bf16 {case}")
    assert rel < 1e-2
    # one stream on the packed views: bitwise the contiguous whole-block call
    o1 = fa.fluxattn_joint_attention_ex_bf16(qv, kv, vv, dev(w_q[0]), dev(w_k[0]), dev(inp.pos),
                                             o=bnhd_empty(*inp.q.shape, torch.bfloat16))
    o_ref = fa.fluxattn_joint_attention_bf16(dev(inp.q), dev(inp.k), dev(inp.v), dev(w_q[0]), dev(w_k[0]),
                                             dev(inp.pos))
    torch.cuda.synchronize()
    assert torch.equal(bits(o1), bits(o_ref))


FP8_CASES = {
    "t2i_77+256_B2": (2, 3, 77, (16, 16), None),
    # three streams at N = 449: E4M3 Q', K' and P alone put the mean error
    # at about 2.8e-3 here (tests/test_fp8_rounding_model.py); the
    # 171-token sequence, where they alone exceed the tolerance, has its own
    # test below
    "i2i_9+320+120": (1, 2, 9, (16, 20), (10, 12)),
}


def test_joint_ex_fp8_packed_streams_parity():
    for case, (B, H, n_txt, grid, ref_grid) in FP8_CASES.items():
        _flush(f"joint_ex fp8 packed streams {case}")
        w = custom_workload(B, H, n_txt, grid, ref_grid, "fp8", 12)
        inp = make_inputs(w)
        starts = stream_starts(w)
        w_q, w_k = stream_norm_weights(len(starts), seed=w.seed)
        p, views = packed(inp.q.view(torch.uint8), inp.k.view(torch.uint8), inp.v.view(torch.uint8))
        qv, kv, vv = (t.view(torch.float8_e4m3fn) for t in views)
        sc = [dev(s) for s in (inp.q_scale, inp.k_scale, inp.v_scale)]
        o = fa.fluxattn_joint_attention_ex_fp8(qv, kv, vv, *sc, dev(w_q), dev(w_k), dev(inp.pos), streams=starts)
        torch.cuda.synchronize()
        B, H = inp.q.shape[:2]
        got = np.stack([f64(o[b, h]) for b in range(B) for h in range(H)])
        rel = check_close(got, joint_ref(inp, starts, w_q, w_k, fp8=True), FP8_TOL, f"joint_ex fp8 {case}")
        assert rel < 1e-1


def test_joint_ex_fp8_packed_streams_171_tokens_within_the_rounding_model():
    """The 171-token, three-stream fp8 sequence (9 text + 10x12 target +
    6x7 reference tokens).  The E4M3 roundings of K', Q' and P alone put its
    mean-abs error at about 4.3e-3, above the 4e-3 tolerance (the CPU model
    in tests/fp8_roundings.py, pinned in tests/test_fp8_rounding_model.py),
    so the kernel is held to that model: mean-abs within 10% of the
    model's, max-abs and relative L2 within the fp8 tolerance."""
    import fp8_roundings as fr
    w = custom_workload(1, 2, 9, (10, 12), (6, 7), "fp8", 12)
    _flush(f"joint_ex fp8 packed streams N={w.N}")
    inp = make_inputs(w)
    starts = stream_starts(w)
    w_q, w_k = stream_norm_weights(len(starts), seed=w.seed)
    p, views = packed(inp.q.view(torch.uint8), inp.k.view(torch.uint8), inp.v.view(torch.uint8))
    qv, kv, vv = (t.view(torch.float8_e4m3fn) for t in views)
    sc = [dev(s) for s in (inp.q_scale, inp.k_scale, inp.v_scale)]
    o = fa.fluxattn_joint_attention_ex_fp8(qv, kv, vv, *sc, dev(w_q), dev(w_k), dev(inp.pos), streams=starts)
    torch.cuda.synchronize()
    ref = joint_ref(inp, starts, w_q, w_k, fp8=True)
    q, k, v, wqt, wkt, pos = fr.case_inputs(inp, w_q.double().numpy(), w_k.double().numpy(), starts)
    model = fr.fused_fp8_model(q, k, v, wqt, wkt, w_k.double().numpy(), pos)[0]
    m_err = np.abs(model - ref)
    got = np.stack([f64(o[0, h]) for h in range(inp.q.shape[1])])
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    _flush(f"fp8 N={w.N}: kernel mean_abs={err.mean():.3e} max_abs={err.max():.3e} rel_l2={rel:.3e}; "
           f"rounding model mean_abs={m_err.mean():.3e} max_abs={m_err.max():.3e}")
    assert np.isfinite(got).all()
    assert err.mean() <= 1.1 * m_err.mean()
    assert err.max() <= FP8_TOL[0]
    assert rel < 1e-1


def test_joint_ex_bf16_t2i_2048_packed_streams_sampled():
    """The 2048x2048 text-to-image shape (B=2, H=24, N=512+16384) from a
    packed QKV tensor with text and image norm weights; sampled rows."""
    w = custom_workload(2, 24, 512, (128, 128), None, "bf16", 0)
    _flush(f"joint_ex bf16 t2i_2048 packed streams (N={w.N})")
    inp = make_inputs(w)
    starts = stream_starts(w)
    w_q, w_k = stream_norm_weights(len(starts), seed=0)
    p, (qv, kv, vv) = packed(inp.q, inp.k, inp.v)
    o = fa.fluxattn_joint_attention_ex_bf16(qv, kv, vv, dev(w_q), dev(w_k), dev(inp.pos), streams=starts)
    torch.cuda.synchronize()
    heads = [(0, 0), (1, 23)]
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(500, 530), np.arange(w.N - 32, w.N),
                                     rng.choice(w.N, 64, replace=False)]))
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    rel = check_close(got, joint_ref(inp, starts, w_q, w_k, heads=heads, rows=rows), BF16_TOL,
                      "joint_ex bf16 t2i_2048 sampled")
    assert rel < 1e-2

"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Small workloads are compared element by element; the 2048x2048 workloads
(N = 16896 bf16 and N = 33280 fp8) run in full on the GPU in the same launch
configuration the benchmark times and are compared on sampled (b, h, row)
outputs that the oracle computes one head at a time.  Tolerances for the
attention output are max-abs 2e-2 / mean-abs 2e-3 (bf16) and 4e-2 / 4e-3
(fp8); the prologue is held to its rounding bound (see each test).
"""
import functools
import math

import numpy as np
import pytest
import torch

import joint_attention_head_amd as fa
import oracle
from workloads import (ROPE_AXES, custom_workload, make_inputs, make_peaked_inputs)

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_TOL = (2e-2, 2e-3)
FP8_TOL = (4e-2, 4e-3)


def _flush(msg):
    print(msg, flush=True)


@functools.lru_cache(maxsize=4)
def inputs(name):
    return make_inputs(name)


def small(B, H, n_txt, grid, ref_grid=None, dtype="bf16", seed=0):
    return make_inputs(custom_workload(B, H, n_txt, grid, ref_grid, dtype, seed))


def dev(t):
    return t.to(DEV).contiguous()


def f64(t, scale=None):
    return oracle.torch_to_f64(t.cpu() if t.is_cuda else t,
                               None if scale is None else scale.cpu())


def check_close(got, ref, tol, what):
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    _flush(f"{what}: max_abs={err.max():.3e} mean_abs={err.mean():.3e} rel_l2={rel:.3e}")
    assert np.isfinite(got).all(), what
    assert err.max() <= tol[0], (what, err.max())
    assert err.mean() <= tol[1], (what, err.mean())
    return rel


def sample_rows(N, k=96, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(min(32, N)), np.arange(max(0, N - 48), N),
                           rng.choice(N, size=min(k, N), replace=False)])
    return np.unique(rows)


# ------------------------------------------------------------------ prologue

def prologue_ref(inp):
    if inp.q.dtype == torch.float8_e4m3fn:
        q, k = f64(inp.q, inp.q_scale), f64(inp.k, inp.k_scale)
    else:
        q, k = f64(inp.q), f64(inp.k)
    return oracle.qk_prologue(q, k, inp.w_q.double().numpy(), inp.w_k.double().numpy(),
                              inp.pos.numpy())


def pair_norm(y):
    n = np.sqrt(y[..., 0::2] ** 2 + y[..., 1::2] ** 2)
    return np.repeat(n, 2, axis=-1)


PROLOGUE_CASES = {
    "tiny": lambda: inputs("tiny"),
    "flux_dev_512": lambda: inputs("flux_dev_512"),
    "odd_77+256": lambda: small(1, 3, 77, (16, 16)),
    "ref_t1_tiny": lambda: small(2, 2, 7, (4, 5), (3, 4)),
}


@pytest.mark.parametrize("case", list(PROLOGUE_CASES))
def test_prologue_bf16_parity(case):
    _flush(f"prologue bf16 {case}")
    inp = PROLOGUE_CASES[case]()
    qo, ko = fa.fluxattn_qk_norm_rope_bf16(dev(inp.q), dev(inp.k), dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
    torch.cuda.synchronize()
    rq, rk = prologue_ref(inp)
    for got, ref, name in ((f64(qo), rq, "q"), (f64(ko), rk, "k")):
        # bf16 RNE (<= 2^-8 relative) plus fp32 angle / sum-of-squares error
        bound = 2.0 ** -8 * np.abs(ref) + 4e-5 * np.maximum(pair_norm(ref), 1.0)
        bad = np.abs(got - ref) > bound
        _flush(f"  {name}: max_err={np.abs(got - ref).max():.3e} violations={bad.sum()}")
        assert not bad.any()


def test_prologue_bf16_in_place_matches_out_of_place():
    inp = inputs("tiny")
    q, k = dev(inp.q), dev(inp.k)
    w_q, w_k, pos = dev(inp.w_q), dev(inp.w_k), dev(inp.pos)
    qo, ko = fa.fluxattn_qk_norm_rope_bf16(q, k, w_q, w_k, pos)
    q2, k2 = q.clone(), k.clone()
    fa.fluxattn_qk_norm_rope_bf16(q2, k2, w_q, w_k, pos, q_out=q2, k_out=k2)
    torch.cuda.synchronize()
    assert torch.equal(qo.view(torch.int16), q2.view(torch.int16))
    assert torch.equal(ko.view(torch.int16), k2.view(torch.int16))


def test_prologue_position_zero_is_norm_only_and_rms_invariant():
    inp = small(1, 2, 8, (8, 8))
    pos = torch.zeros_like(inp.pos)
    c = 0.75
    w = torch.full((128,), c)
    qo, ko = fa.fluxattn_qk_norm_rope_bf16(dev(inp.q), dev(inp.k), dev(w), dev(w), dev(pos))
    torch.cuda.synchronize()
    ref = oracle.rms_norm(f64(inp.q), np.full(128, c), 1e-6)
    got = f64(qo)
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    rms = np.sqrt(np.mean(f64(ko) ** 2, axis=-1))
    np.testing.assert_allclose(rms, c, rtol=4e-3)


@pytest.mark.parametrize("case", ["tiny_fp8", "ref_t1_fp8"])
def test_prologue_fp8_parity(case):
    _flush(f"prologue fp8 {case}")
    inp = small(1, 2, 64, (16, 16), None, "fp8") if case == "tiny_fp8" else \
        small(1, 3, 9, (5, 6), (4, 4), "fp8", seed=3)
    qo, ko, sqo, sko = fa.fluxattn_qk_norm_rope_fp8(dev(inp.q), dev(inp.k), dev(inp.q_scale),
                                                    dev(inp.k_scale), dev(inp.w_q), dev(inp.w_k),
                                                    dev(inp.pos))
    torch.cuda.synchronize()
    rq, rk = prologue_ref(inp)
    for got8, s_out, ref, w, name in ((qo, sqo, rq, inp.w_q, "q"), (ko, sko, rk, inp.w_k, "k")):
        s_ref = oracle.fp8_prologue_out_scale(w.double().numpy())
        np.testing.assert_allclose(s_out.cpu().double().numpy(), s_ref, rtol=1e-6)
        got = f64(got8, s_out)
        # E4M3 RNE: <= 2^-4 relative for normals, 2^-10 * scale for subnormals
        bound = 2.0 ** -4 * np.abs(ref) + 2.0 ** -10 * s_ref + 4e-5 * np.maximum(pair_norm(ref), 1.0)
        bad = np.abs(got - ref) > bound
        _flush(f"  {name}: max_err={np.abs(got - ref).max():.3e} violations={bad.sum()}")
        assert not bad.any()
        assert np.abs(got).max() <= 448 * float(s_out.max()) + 1e-6


def test_prologue_fp8_rows_at_the_bound():
    """Rows whose whole energy sits in one dim, with unit weights, position 0
    (no rotation) and eps = 0, normalise to exactly +-sqrt(D) max|w|, which
    the output scale sqrt(D) max|w| / 448 maps to +-448: the largest finite
    E4M3 value.  Every such code must come out as +-448 (0x7e / 0xfe), never
    NaN, whatever the fp32 rounding of the factors on the way."""
    _flush("prologue fp8 rows at the output bound")
    B, H, N, D = 1, 3, 96, 128
    k = torch.zeros(B, H, N, D)
    rows = torch.arange(N)
    dims = (7 * rows + 3) % D                        # even and odd dims, every pair
    codes = torch.tensor([192.0, -448.0, 0.5, -2.0 ** -6, 26.0, -3.25])
    for h in range(H):
        k[0, h, rows, dims] = codes[(rows + h) % len(codes)]
    k8 = k.to(torch.float8_e4m3fn)
    ks = torch.tensor([[0.5, 3.0, 1e-3]])
    w = torch.ones(D)
    pos = torch.zeros(N, 3, dtype=torch.int32)
    _, ko, _, sko = fa.fluxattn_qk_norm_rope_fp8(None, dev(k8), None, dev(ks), None, dev(w), dev(pos), eps=0.0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(float(sko[0, 0]), math.sqrt(D) / 448.0, rtol=1e-6)
    got = ko.cpu().view(torch.uint8)
    want = torch.where(k8.view(torch.uint8) == 0, 0, torch.where(k < 0, 0xFE, 0x7E)).to(torch.uint8)
    bad = int((got != want).sum())
    _flush(f"  codes off the bound: {bad}")
    assert bad == 0


# ------------------------------------------------------------------ forward

def run_forward_bf16(inp, **kw):
    return fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k), dev(inp.v), **kw)


FORWARD_CASES = {
    "tiny": lambda: inputs("tiny"),
    "flux_dev_512": lambda: inputs("flux_dev_512"),
    "odd_77+256": lambda: small(1, 3, 77, (16, 16)),
    "n1": lambda: small(1, 2, 1, (0, 0)),
    "n65": lambda: small(2, 1, 1, (8, 8)),
    "n129": lambda: small(1, 1, 1, (8, 16)),
    "peaked_1024": lambda: make_peaked_inputs("flux_dev_1024"),
}


@pytest.mark.parametrize("case", list(FORWARD_CASES))
def test_forward_bf16_parity(case):
    _flush(f"forward bf16 {case}")
    inp = FORWARD_CASES[case]()
    o = run_forward_bf16(inp)
    torch.cuda.synchronize()
    if inp.q.shape[2] > 2000:
        rows = sample_rows(inp.q.shape[2])
        ref = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v), rows=rows)
        got = f64(o)[:, :, rows]
    else:
        ref = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v))
        got = f64(o)
    rel = check_close(got, ref, BF16_TOL, f"forward bf16 {case}")
    assert rel < 1e-2


def test_forward_bf16_custom_scale():
    inp = small(1, 2, 5, (10, 10))
    o = run_forward_bf16(inp, softmax_scale=0.05)
    torch.cuda.synchronize()
    ref = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v), scale=0.05)
    check_close(f64(o), ref, BF16_TOL, "forward bf16 scale=0.05")


@pytest.mark.parametrize("growth", ["rising", "falling", "spike"])
def test_forward_bf16_logit_range_across_tiles(growth):
    """Scores whose scale changes from one 64-key tile to the next, so the
    running shift of the online softmax has to move by far more than the
    lazy threshold (rising: later tiles dominate by tens of log2 units;
    falling: the first tile dominates and later ones underflow towards 0;
    spike: one key tile far above everything before it)."""
    inp = small(1, 2, 37, (20, 20))          # N = 437: 7 key tiles, ragged
    N = inp.q.shape[2]
    f = torch.ones(N)
    tiles = torch.arange(N) // 64
    if growth == "rising":
        f = 1.0 + tiles.float()               # logit spread grows 7x
    elif growth == "falling":
        f = torch.where(tiles == 0, 6.0, 1.0)
    else:
        f = torch.where(tiles == 4, 9.0, 1.0)
    k = (inp.k.float() * f[None, None, :, None]).to(torch.bfloat16)
    o = fa.fluxattn_forward_bf16(dev(inp.q), dev(k), dev(inp.v))
    torch.cuda.synchronize()
    ref = oracle.attention(f64(inp.q), f64(k), f64(inp.v))
    rel = check_close(f64(o), ref, BF16_TOL, f"logit range {growth}")
    assert rel < 1e-2


def _tile_factors(N, growth, big):
    """Per-key factors that change the logit scale from one 64-key tile to
    the next (rising, falling: first tile dominates, spike: tile 4)."""
    tiles = torch.arange(N) // 64
    if growth == "rising":
        return 1.0 + (big - 1.0) / 6.0 * tiles.float()
    if growth == "falling":
        return torch.where(tiles == 0, big, 1.0)
    return torch.where(tiles == 4, big, 1.0)


def _q_prime(q, w_q, pos):
    """The queries' RMSNorm + RoPE, as the fused kernels apply them."""
    return oracle.rope(oracle.rms_norm(q, w_q.double().numpy(), 1e-6), pos.numpy())


LOG2E_OVER_SQRT_D = math.log2(math.e) / math.sqrt(128)


def _q_rounded_bf16(qp):
    """Q' as the fused bf16 kernel holds it: c Q' rounded once to bf16
    (c = log2 e / sqrt(d)), divided back by c in fp64."""
    c = LOG2E_OVER_SQRT_D
    return torch.from_numpy(qp * c).to(torch.bfloat16).double().numpy() / c


def _q_rounded_e4m3(qp, k_scale):
    """Q' as the fused fp8 kernel encodes it: per query, codes of Q' g / 2^e
    with g = c * (k scale) and e = ceil(log2(amax g / 448)), so that the
    largest code lies in (224, 448]; returned as codes * 2^e / g."""
    g = LOG2E_OVER_SQRT_D * k_scale.double().numpy()[:, :, None, None]
    amax = np.abs(qp).max(axis=-1, keepdims=True)
    e = np.ceil(np.log2(amax * g / 448.0))
    codes = torch.from_numpy(qp * g / 2.0 ** e).to(torch.float8_e4m3fn).double().numpy()
    return codes * 2.0 ** e / g


def _no_less_accurate(got, two_call, plain, what):
    """The fused path's error against the unrounded chain is within 1.5x
    (plus a rounding step of the output) of the error that the two-call
    path's one rounding of Q' alone gives, in max-abs and mean-abs."""
    e, e2 = np.abs(got - plain), np.abs(two_call - plain)
    _flush(f"{what} vs plain chain: max_abs={e.max():.3e} mean_abs={e.mean():.3e}; "
           f"two-call rounding alone: max_abs={e2.max():.3e} mean_abs={e2.mean():.3e}")
    assert e.max() <= 1.5 * e2.max() + 4e-3, what
    assert e.mean() <= 1.5 * e2.mean() + 2e-4, what


@pytest.mark.parametrize("growth", ["rising", "falling", "spike"])
def test_forward_fused_bf16_logit_range_across_tiles(growth):
    """The running shift of the fused kernel (whose QK^T accumulators start
    at -b) moving by tens of log2 units between key tiles.  At logits this
    large the one bf16 rounding of c Q' alone moves the weights by more
    than the tolerance, so the reference takes that rounding (of the
    oracle's Q') as its input."""
    inp = small(1, 2, 37, (20, 20))          # N = 437: 7 key tiles, ragged
    N = inp.q.shape[2]
    f = _tile_factors(N, growth, {"rising": 7.0, "falling": 6.0, "spike": 9.0}[growth])
    k = (inp.k.float() * f[None, None, :, None]).to(torch.bfloat16)
    o = fa.fluxattn_forward_fused_bf16(dev(inp.q), dev(k), dev(inp.v), dev(inp.w_q), dev(inp.pos))
    torch.cuda.synchronize()
    qp = _q_prime(f64(inp.q), inp.w_q, inp.pos)
    qr = _q_rounded_bf16(qp)
    ref = oracle.attention(qr, f64(k), f64(inp.v))
    rel = check_close(f64(o), ref, BF16_TOL, f"fused logit range {growth}")
    assert rel < 1e-2
    # against the plain chain (no rounding at all): no less accurate than
    # the two-call path's rounding of Q' itself to bf16 (the prologue's
    # output), which at these logits is also outside the tolerance
    plain = oracle.attention(qp, f64(k), f64(inp.v))
    two_call = oracle.attention(torch.from_numpy(qp).to(torch.bfloat16).double().numpy(), f64(k), f64(inp.v))
    _no_less_accurate(f64(o), two_call, plain, f"fused logit range {growth}")


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("growth", ["rising", "falling", "spike"])
def test_forward_fp8_logit_range_across_tiles(growth, fused):
    """The fp8 kernel's running shift (lane maximum test, rescale of O and of
    the matrix-core row sums) across tiles whose logit scale changes.  The
    factors are milder than in bf16: E4M3 keys carry a 2^-4 relative
    rounding, which at logits of tens of log2 units moves the softmax
    weights themselves; here the largest logits are about 15.  The fused
    form's reference takes the E4M3 re-encoding of the oracle's Q' (the
    per-query scale rule) as its input, for the same reason."""
    inp = small(1, 2, 37, (20, 20), None, "fp8", seed=3)
    N = inp.q.shape[2]
    f = _tile_factors(N, growth, 2.5)
    k_real = torch.from_numpy(f64(inp.k, inp.k_scale)).float() * f[None, None, :, None]
    amax = k_real.abs().amax(dim=(2, 3))
    sk = (amax / 448.0).contiguous()
    k8 = (k_real / sk[:, :, None, None]).clamp(-448, 448).to(torch.float8_e4m3fn)
    args = (dev(inp.q), dev(k8), dev(inp.v), dev(inp.q_scale), dev(sk), dev(inp.v_scale))
    if fused:
        o = fa.fluxattn_forward_fused_fp8(*args, dev(inp.w_q), dev(inp.pos))
        qp = _q_prime(f64(inp.q, inp.q_scale), inp.w_q, inp.pos)
        qr = _q_rounded_e4m3(qp, sk)
    else:
        o = fa.fluxattn_forward_fp8(*args)
        qr = f64(inp.q, inp.q_scale)
    torch.cuda.synchronize()
    ref = oracle.attention(qr, f64(k8, sk), f64(inp.v, inp.v_scale))
    rel = check_close(f64(o), ref, FP8_TOL, f"fp8 {'fused ' if fused else ''}logit range {growth}")
    assert rel < 1e-1
    if fused:
        # against the plain chain: no less accurate than the two-call path,
        # whose prologue stores Q' in E4M3 with the per-head output scale
        # sqrt(D) max|w| / 448
        plain = oracle.attention(qp, f64(k8, sk), f64(inp.v, inp.v_scale))
        s_out = math.sqrt(128) * float(inp.w_q.abs().max()) / 448.0
        q2 = torch.from_numpy(qp / s_out).to(torch.float8_e4m3fn).double().numpy() * s_out
        two_call = oracle.attention(q2, f64(k8, sk), f64(inp.v, inp.v_scale))
        _no_less_accurate(f64(o), two_call, plain, f"fp8 fused logit range {growth}")


def test_forward_bf16_invariants():
    inp = small(1, 2, 13, (10, 10))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    # V == 1 gives exactly 1
    o = fa.fluxattn_forward_bf16(q, k, torch.ones_like(v))
    # identical keys give the mean of V
    k_same = k[:, :, :1].expand_as(k).contiguous()
    o2 = fa.fluxattn_forward_bf16(q, k_same, v)
    # bitwise reproducible
    a = fa.fluxattn_forward_bf16(q, k, v)
    b = fa.fluxattn_forward_bf16(q, k, v)
    torch.cuda.synchronize()
    assert torch.all(o == 1.0)
    mean_v = f64(inp.v).mean(axis=2, keepdims=True)
    check_close(f64(o2), np.broadcast_to(mean_v, o2.shape), BF16_TOL, "identical keys")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_forward_bf16_writes_every_output_and_nothing_else():
    inp = small(1, 3, 50, (9, 7))
    B, H, N, D = inp.q.shape
    n = B * H * N * D
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    o = buf[guard:guard + n].view(B, H, N, D)
    fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k), dev(inp.v), o=o)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()


# Uncut launches run as a persistent grid of one workgroup per compute unit,
# each taking whole blocks of its XCD's range in turn.  Block counts above
# the compute units and not a multiple of 8 (uneven XCD ranges): 259 = 37
# heads x 7 blocks (N = 1792) and 513 = 3 x 19 x 9 (N = 2304).
PERSIST_SHAPES = {"nb259": (1, 37, 512, (32, 40)), "nb513": (3, 19, 512, (32, 56))}


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("shape", list(PERSIST_SHAPES))
def test_forward_persistent_grid_covers_every_block(shape, dtype):
    B, H, n_txt, grid = PERSIST_SHAPES[shape]
    _flush(f"persistent grid {shape} {dtype}")
    inp = small(B, H, n_txt, grid, None, dtype, seed=3)
    N, D = inp.q.shape[2], inp.q.shape[3]
    n = B * H * N * D
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    o = buf[guard:guard + n].view(B, H, N, D)
    if dtype == "bf16":
        fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k), dev(inp.v), o=o)
    else:
        fa.fluxattn_forward_fp8(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.q_scale), dev(inp.k_scale),
                                dev(inp.v_scale), o=o)
    torch.cuda.synchronize()
    # every block written, nothing outside
    assert torch.isfinite(o).all()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()
    # rows of every query block of the first, a middle and the last head
    rows = np.unique(np.concatenate([np.arange(0, N, 256)[:, None] + np.array([0, 77, 255])]).ravel())
    rows = rows[rows < N]
    tol = BF16_TOL if dtype == "bf16" else FP8_TOL
    for b, h in ((0, 0), (B // 2, H // 2), (B - 1, H - 1)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        if dtype == "bf16":
            ref = oracle.attention(f64(inp.q[sl]), f64(inp.k[sl]), f64(inp.v[sl]), rows=rows)
        else:
            ref = oracle.attention(f64(inp.q[sl], inp.q_scale[sl]), f64(inp.k[sl], inp.k_scale[sl]),
                                   f64(inp.v[sl], inp.v_scale[sl]), rows=rows)
        check_close(f64(o[sl])[:, :, rows], ref, tol, f"persistent grid {shape} {dtype} head ({b},{h})")


def test_forward_bf16_key_permutation_invariance():
    inp = small(1, 2, 11, (12, 12))
    perm = torch.randperm(inp.q.shape[2], generator=torch.Generator().manual_seed(1))
    a = run_forward_bf16(inp)
    b = fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k[:, :, perm]), dev(inp.v[:, :, perm]))
    torch.cuda.synchronize()
    check_close(f64(b), f64(a), BF16_TOL, "key permutation")


# ------------------------------------------------------------------ joint

def joint_ref(inp, heads=None, rows=None):
    sc = lambda t, s: f64(t, s) if t.dtype == torch.float8_e4m3fn else f64(t)
    w_q, w_k, pos = inp.w_q.double().numpy(), inp.w_k.double().numpy(), inp.pos.numpy()
    if heads is None:
        return oracle.joint_attention(sc(inp.q, inp.q_scale), sc(inp.k, inp.k_scale),
                                      sc(inp.v, inp.v_scale), w_q, w_k, pos, rows=rows)
    out = []
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        s = lambda x: None if x is None else x[sl]
        out.append(oracle.joint_attention(sc(inp.q[sl], s(inp.q_scale)), sc(inp.k[sl], s(inp.k_scale)),
                                          sc(inp.v[sl], s(inp.v_scale)), w_q, w_k, pos, rows=rows)[0, 0])
    return np.stack(out)


@pytest.mark.parametrize("name", ["tiny", "flux_dev_512", "flux_dev_1024"])
def test_joint_bf16_parity_full(name):
    _flush(f"joint bf16 {name}")
    inp = inputs(name)
    o = fa.joint_attention_bf16(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
    torch.cuda.synchronize()
    check_close(f64(o), joint_ref(inp), BF16_TOL, f"joint bf16 {name}")


def test_joint_bf16_parity_t2i_2048_sampled():
    _flush("joint bf16 t2i_2048_cfg (N=16896, B=2, H=24)")
    inp = inputs("t2i_2048_cfg")
    o = fa.joint_attention_bf16(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
    torch.cuda.synchronize()
    heads = [(0, 0), (1, 23), (0, 13)]
    rows = sample_rows(inp.q.shape[2])
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    rel = check_close(got, joint_ref(inp, heads, rows), BF16_TOL, "joint bf16 t2i sampled")
    assert rel < 1e-2
    # V == 1 on the full-size launch gives exactly 1 in bf16: l sums the
    # fp32 probabilities and P.V the bf16-rounded ones, so O / l is
    # sum(bf16(p)) / sum(p), within 2^-9 of 1, which the output rounding
    # takes to exactly 1 (the ratio itself is not 1 in fp32)
    ones = fa.fluxattn_forward_bf16(dev(inp.q), dev(inp.k), torch.ones_like(o))
    torch.cuda.synchronize()
    assert torch.all(ones == 1.0)


# Ragged edges at every boundary of the bf16 kernel's lane layout: a lane
# holds keys 16 kb + 4 g + r of each 64-key tile and the two query rows
# l % 16 and 16 + l % 16 of its wave's 32, so a last key tile ending at
# N mod 64 in {4, 15, 16, 17, 32, 48, 63} and a last query block ending at
# N mod 256 in {4, 15, 16, 17, 32, 48, 63, 240} cut those groups at
# different places (text tokens + an 8 x 8 image grid).  The fused form is
# held to the unrounded chain (RMSNorm + RoPE of the queries in fp64).
EDGE_N = (260, 272, 273, 288, 304, 319, 496, 783)


@pytest.mark.parametrize("fused", [False, True])
def test_forward_bf16_ragged_lane_edges(fused):
    for i, N in enumerate(EDGE_N):
        inp = small(1, 2, N - 64, (8, 8), seed=10 + i)
        assert inp.q.shape[2] == N
        if fused:
            o = fa.fluxattn_forward_fused_bf16(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.w_q), dev(inp.pos))
            ref = oracle.attention(_q_prime(f64(inp.q), inp.w_q, inp.pos), f64(inp.k), f64(inp.v))
        else:
            o = run_forward_bf16(inp)
            ref = oracle.attention(f64(inp.q), f64(inp.k), f64(inp.v))
        torch.cuda.synchronize()
        rel = check_close(f64(o), ref, BF16_TOL, f"forward bf16 {'fused ' if fused else ''}N={N}")
        assert rel < 1e-2


FUSED_CASES = {
    "tiny": lambda: inputs("tiny"),
    "flux_dev_512": lambda: inputs("flux_dev_512"),
    "odd_77+256": lambda: small(1, 3, 77, (16, 16)),
    "ref_t1": lambda: small(2, 2, 9, (10, 12), (6, 7)),
    "n65": lambda: small(2, 1, 1, (8, 8)),
}


@pytest.mark.parametrize("case", list(FUSED_CASES))
def test_joint_fused_bf16_parity(case):
    """Queries' RMSNorm + RoPE inside the attention kernel, keys' prologue
    into a separate buffer; against the whole fp64 chain."""
    _flush(f"joint fused bf16 {case}")
    inp = FUSED_CASES[case]()
    q, k = dev(inp.q), dev(inp.k)
    k_keep = k.clone()
    o = fa.fluxattn_joint_attention_bf16(q, k, dev(inp.v), dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
    torch.cuda.synchronize()
    assert torch.equal(k.view(torch.int16), k_keep.view(torch.int16))   # k untouched
    rel = check_close(f64(o), joint_ref(inp), BF16_TOL, f"joint fused bf16 {case}")
    assert rel < 1e-2


def test_joint_fused_bf16_in_place_and_matches_two_calls():
    inp = small(1, 2, 21, (12, 12))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w_q, w_k, pos = dev(inp.w_q), dev(inp.w_k), dev(inp.pos)
    two = fa.joint_attention_bf16(q, k, v, w_q, w_k, pos)
    sep = fa.fluxattn_joint_attention_bf16(q, k, v, w_q, w_k, pos)
    k2 = k.clone()
    inplace = fa.fluxattn_joint_attention_bf16(q, k2, v, w_q, w_k, pos, k_work=k2)
    kn = fa.fluxattn_qk_norm_rope_bf16(q, k, w_q, w_k, pos)[1]
    torch.cuda.synchronize()
    assert torch.equal(sep.view(torch.int16), inplace.view(torch.int16))
    assert torch.equal(k2.view(torch.int16), kn.view(torch.int16))      # k_work holds K'
    # same block up to where Q' is rounded: differences of a bf16 step at most
    check_close(f64(sep), f64(two), BF16_TOL, "fused vs two calls")


def test_keys_only_prologue_and_fused_forward_compose_the_joint_call():
    """keys-only prologue == the keys of the full prologue (bitwise), and
    keys-only prologue + fused forward == the joint entry point (bitwise)."""
    inp = small(1, 3, 13, (9, 11), (4, 5))
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w_q, w_k, pos = dev(inp.w_q), dev(inp.w_k), dev(inp.pos)
    _, k_full = fa.fluxattn_qk_norm_rope_bf16(q, k, w_q, w_k, pos)
    none, k_only = fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos)
    o_parts = fa.fluxattn_forward_fused_bf16(q, k_only, v, w_q, pos)
    o_joint = fa.fluxattn_joint_attention_bf16(q, k, v, w_q, w_k, pos)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(k_only.view(torch.int16), k_full.view(torch.int16))
    assert torch.equal(o_parts.view(torch.int16), o_joint.view(torch.int16))
    # fp8
    inp = small(1, 2, 13, (9, 11), None, "fp8", seed=6)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    sq, sk, sv = dev(inp.q_scale), dev(inp.k_scale), dev(inp.v_scale)
    w_q, w_k, pos = dev(inp.w_q), dev(inp.w_k), dev(inp.pos)
    _, k_full, _, sk_full = fa.fluxattn_qk_norm_rope_fp8(q, k, sq, sk, w_q, w_k, pos)
    _, k_only, _, sk_only = fa.fluxattn_qk_norm_rope_fp8(None, k, None, sk, None, w_k, pos)
    o_parts = fa.fluxattn_forward_fused_fp8(q, k_only, v, sq, sk_only, sv, w_q, pos)
    o_joint = fa.fluxattn_joint_attention_fp8(q, k, v, sq, sk, sv, w_q, w_k, pos)
    torch.cuda.synchronize()
    assert torch.equal(k_only.view(torch.uint8), k_full.view(torch.uint8))
    assert torch.equal(sk_only, sk_full)
    assert torch.equal(o_parts.view(torch.int16), o_joint.view(torch.int16))


def block_rows(N, offsets=(0, 101, 255)):
    """A few rows of every 256-query block: whatever blocks a launch cuts
    into key ranges, each of them is sampled."""
    rows = (np.arange(0, N, 256)[:, None] + np.asarray(offsets)[None, :]).ravel()
    return np.unique(np.concatenate([rows[rows < N], np.arange(min(32, N)), np.arange(max(0, N - 48), N)]))


def test_joint_fused_bf16_t2i_2048_sampled():
    """The launches the benchmark times at 2048x2048 text-to-image (B=2,
    H=24, N=16896): keys-only prologue, then the fused attention with the
    default key-range split (3168 query blocks on one workgroup per compute
    unit: 11 whole rounds, then a tail of 352 blocks in equal shares, most
    of them cut in two).  Checked on rows of every query block of a head of
    the whole rounds (0,0), of the head where the tail starts (1,18) and of
    the last head (1,23), against the whole fp64 chain."""
    _flush("joint fused bf16 t2i_2048_cfg (N=16896, B=2, H=24), benchmark launches")
    inp = inputs("t2i_2048_cfg")
    B, H, N = inp.q.shape[:3]
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w_q, w_k, pos = dev(inp.w_q), dev(inp.w_k), dev(inp.pos)
    ws = fa.split_workspace(B, H, N, 0)
    assert ws.nbytes > 0, "the default setting cuts this launch"
    _, kn = fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos)
    o = fa.fluxattn_forward_fused_ex_bf16(q, kn, v, w_q, pos, split=ws)
    torch.cuda.synchronize()
    assert not ws.counts().any()
    heads = [(0, 0), (1, 18), (1, 23)]
    rows = block_rows(N)
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    rel = check_close(got, joint_ref(inp, heads, rows), BF16_TOL, "joint fused bf16 t2i sampled (split)")
    assert rel < 1e-2
    # the whole-block entry point (uncut) agrees on the same rows
    o2 = fa.fluxattn_joint_attention_bf16(q, k, v, w_q, w_k, pos)
    torch.cuda.synchronize()
    got2 = np.stack([f64(o2[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    check_close(got2, joint_ref(inp, heads, rows), BF16_TOL, "joint fused bf16 t2i sampled (uncut)")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_joint_fused_flux_dev_1024_sampled(dtype):
    """The launches the benchmark times at FLUX-dev 1024x1024 (B=1, H=24,
    N = 512 + 64x64 = 4608), in both precisions: keys-only prologue, then
    the fused attention with the default split setting, which leaves this
    launch uncut: 432 query blocks on a persistent grid of one workgroup per
    compute unit, 176 workgroups taking a second block with a job start that
    overlaps the query transform with the first tile copies.  Rows of every
    query block of three heads against the whole fp64 chain."""
    _flush(f"joint fused {dtype} flux_dev_1024 (N=4608), benchmark launches")
    w = custom_workload(1, 24, 512, (64, 64), None, dtype)
    inp = make_inputs(w)
    B, H, N = inp.q.shape[:3]
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    w_q, w_k, pos = dev(inp.w_q), dev(inp.w_k), dev(inp.pos)
    ws = fa.split_workspace(B, H, N, 0)
    if dtype == "bf16":
        _, kn = fa.fluxattn_qk_norm_rope_bf16(None, k, None, w_k, pos)
        o = fa.fluxattn_forward_fused_ex_bf16(q, kn, v, w_q, pos, split=ws)
        tol, bound = BF16_TOL, 1e-2
    else:
        sq, sk, sv = dev(inp.q_scale), dev(inp.k_scale), dev(inp.v_scale)
        _, kn, _, skn = fa.fluxattn_qk_norm_rope_fp8(None, k, None, sk, None, w_k, pos)
        o = fa.fluxattn_forward_fused_ex_fp8(q, kn, v, sq, skn, sv, w_q, pos, split=ws)
        tol, bound = FP8_TOL, 1e-1
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 12), (0, 23)]
    rows = block_rows(N, offsets=(0, 255))
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    rel = check_close(got, joint_ref(inp, heads, rows), tol, f"joint fused {dtype} flux_dev_1024 sampled")
    assert rel < bound


def test_joint_fused_fp8_parity():
    """fp8 with the fused query prologue (Q' re-encoded in E4M3 per query
    inside the attention kernel) against the fp64 chain, and close to the
    two-call path, which reads Q' in E4M3 from the prologue."""
    for inp in (small(1, 2, 64, (16, 16), (8, 8), "fp8"), small(2, 1, 5, (16, 20), None, "fp8", seed=4)):
        args = (dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.q_scale), dev(inp.k_scale), dev(inp.v_scale),
                dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
        o = fa.fluxattn_joint_attention_fp8(*args)
        o2 = fa.joint_attention_fp8(*args)
        torch.cuda.synchronize()
        ref = joint_ref(inp)
        rel = check_close(f64(o), ref, FP8_TOL, f"joint fused fp8 N={inp.q.shape[2]}")
        assert rel < 1e-1
        check_close(f64(o2), ref, FP8_TOL, f"joint two-call fp8 N={inp.q.shape[2]}")
        # same operations, Q' encoded with a different scale: the two
        # results differ by fp8 rounding only
        assert np.abs(f64(o) - f64(o2)).mean() <= FP8_TOL[1]


def test_forward_fp8_parity_tiny_and_ragged():
    for inp in (small(1, 2, 64, (16, 16), None, "fp8"), small(1, 3, 77, (16, 16), None, "fp8", seed=2)):
        o = fa.fluxattn_forward_fp8(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.q_scale),
                                    dev(inp.k_scale), dev(inp.v_scale))
        torch.cuda.synchronize()
        ref = oracle.attention(f64(inp.q, inp.q_scale), f64(inp.k, inp.k_scale), f64(inp.v, inp.v_scale))
        check_close(f64(o), ref, FP8_TOL, f"forward fp8 N={inp.q.shape[2]}")


def test_joint_fp8_parity_tiny():
    inp = small(1, 2, 64, (16, 16), (8, 8), "fp8")
    o = fa.joint_attention_fp8(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.q_scale), dev(inp.k_scale),
                               dev(inp.v_scale), dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
    torch.cuda.synchronize()
    rel = check_close(f64(o), joint_ref(inp), FP8_TOL, "joint fp8 tiny")
    assert rel < 1e-1


def test_fp8_i2i_2048_sampled():
    _flush("fp8 i2i_2048 (N=33280, H=24)")
    inp = inputs("i2i_2048")
    B, H, N = inp.q.shape[:3]
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    sq, sk, sv = dev(inp.q_scale), dev(inp.k_scale), dev(inp.v_scale)
    heads = [(0, 0), (0, 17)]
    rows = sample_rows(inp.q.shape[2], k=64)
    # attention alone on the generated fp8 tensors
    o = fa.fluxattn_forward_fp8(q, k, v, sq, sk, sv)
    torch.cuda.synchronize()
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    ref = np.stack([oracle.attention(f64(inp.q[b:b + 1, h:h + 1], inp.q_scale[b:b + 1, h:h + 1]),
                                     f64(inp.k[b:b + 1, h:h + 1], inp.k_scale[b:b + 1, h:h + 1]),
                                     f64(inp.v[b:b + 1, h:h + 1], inp.v_scale[b:b + 1, h:h + 1]),
                                     rows=rows)[0, 0] for (b, h) in heads])
    check_close(got, ref, FP8_TOL, "forward fp8 i2i sampled")
    # the whole block
    o = fa.joint_attention_fp8(q, k, v, sq, sk, sv, dev(inp.w_q), dev(inp.w_k), dev(inp.pos))
    torch.cuda.synchronize()
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    rel = check_close(got, joint_ref(inp, heads, rows), FP8_TOL, "joint fp8 i2i sampled")
    assert rel < 1e-1
    # the launches the benchmark times: keys-only fp8 prologue, then the
    # fused attention with the default split (3120 query blocks: 11 whole
    # rounds, then a tail of 304 blocks, heads 21 (from block 86) to 23, in
    # equal shares); rows of every query block of a head of the whole
    # rounds and of two tail heads
    ws = fa.split_workspace(B, H, N, 0)
    assert ws.nbytes > 0, "the default setting cuts this launch"
    _, kn, _, skn = fa.fluxattn_qk_norm_rope_fp8(None, k, None, sk, None, dev(inp.w_k), dev(inp.pos))
    o = fa.fluxattn_forward_fused_ex_fp8(q, kn, v, sq, skn, sv, dev(inp.w_q), dev(inp.pos), split=ws)
    torch.cuda.synchronize()
    assert not ws.counts().any()
    heads = [(0, 0), (0, 21), (0, 23)]
    rows = block_rows(N, offsets=(0, 255))
    got = np.stack([f64(o[b, h, torch.from_numpy(rows)]) for (b, h) in heads])
    rel = check_close(got, joint_ref(inp, heads, rows), FP8_TOL, "joint fused fp8 i2i sampled (split)")
    assert rel < 1e-1

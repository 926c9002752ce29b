"""Pins of the fp64 CPU oracle against facts that do not come from the oracle:
closed forms, invariants, library routines in float64, brute force on tiny
inputs, and the OCP E4M3 encoding table.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden
from workloads import (ROPE_AXES, ROPE_THETA, custom_workload, make_inputs,
                       position_ids, quantize_e4m3_per_head)

AX = ROPE_AXES
TH = ROPE_THETA
EPS = 1e-6


# ----------------------------------------------------------------- decoding

def test_e4m3_decode_matches_spec_table():
    for code, val in read_golden("e4m3_special_values.txt"):
        got = oracle.e4m3fn_to_f64(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val), code
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_bf16_decode_matches_torch_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


# ----------------------------------------------------------------- RMSNorm

def test_rmsnorm_constant_row_closed_form():
    w = 1 + 0.1 * np.random.default_rng(1).standard_normal(128)
    for a in (3.0, -0.5, 1e-2):
        y = oracle.rms_norm(np.full(128, a), w, EPS)
        np.testing.assert_allclose(y, a * w / math.sqrt(a * a + EPS), rtol=1e-14)


def test_rmsnorm_eps_sits_inside_the_root():
    # mean(x^2) = eps: with eps inside the root the factor is 1/sqrt(2); with
    # eps added after the root it would be ~1, with no eps exactly 1.
    y = oracle.rms_norm(np.full(128, 1e-3), np.ones(128), 1e-6)
    np.testing.assert_allclose(y, 1e-3 / math.sqrt(2e-6), rtol=1e-14)
    np.testing.assert_allclose(y, 1 / math.sqrt(2), rtol=1e-14)


def test_rmsnorm_uniform_weight_rms_invariant():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 5, 128)) * rng.uniform(1e-3, 10, (3, 5, 1))
    c = 1.7
    y = oracle.rms_norm(x, np.full(128, c), EPS)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)),
                               c * np.sqrt(ms / (ms + EPS)), rtol=1e-13)


def test_rmsnorm_weight_is_per_dimension():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128)
    w = np.zeros(128)
    w[37] = 2.0
    y = oracle.rms_norm(x, w, EPS)
    assert np.count_nonzero(y) == 1 and y[37] != 0
    np.testing.assert_allclose(y[37], 2 * x[37] / math.sqrt(np.mean(x * x) + EPS), rtol=1e-14)


def test_stream_weights_brute_force_per_token():
    """Each token takes the weight row of the last stream starting at or
    before it; checked with plain loops, including empty streams."""
    rng = np.random.default_rng(4)
    D, N = 8, 11
    x = rng.standard_normal((2, 3, N, D))
    rows = 1 + 0.1 * rng.standard_normal((4, D))
    for starts in ((0,), (0, 4), (0, 4, 9), (0, 0, 5), (0, 3, 3, 11), (0, 11)):
        S = len(starts)
        got = oracle.rms_norm(x, oracle.stream_weights(rows[:S], starts, N), EPS)
        for b in range(2):
            for h in range(3):
                for n in range(N):
                    s = 0
                    for j in range(S):
                        if starts[j] <= n:
                            s = j
                    ss = 0.0
                    for d in range(D):
                        ss += x[b, h, n, d] ** 2
                    for d in range(D):
                        want = x[b, h, n, d] * rows[s, d] / math.sqrt(ss / D + EPS)
                        assert abs(got[b, h, n, d] - want) <= 1e-13 * max(1.0, abs(want))


def test_stream_weights_one_stream_is_the_shared_vector():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 2, 7, 128))
    w = 1 + 0.1 * rng.standard_normal(128)
    tok = oracle.stream_weights(w[None], (0,), 7)
    assert tok.shape == (7, 128) and np.array_equal(tok, np.broadcast_to(w, (7, 128)))
    np.testing.assert_array_equal(oracle.rms_norm(x, tok, EPS), oracle.rms_norm(x, w, EPS))


# ----------------------------------------------------------------- RoPE

def _basis(d):
    e = np.zeros((1, 1, 1, 128))
    e[..., d] = 1.0
    return e


def test_rope_frequency_ladder_fixture():
    om = oracle.rope_frequencies(AX, TH)
    by_dim = {16: om[0], 56: om[1]}
    np.testing.assert_array_equal(om[1], om[2])
    for d, j, val in read_golden("rope_frequency_ladder.txt"):
        np.testing.assert_allclose(by_dim[int(d)][int(j)], float(val), rtol=1e-14)


@pytest.mark.parametrize("pair_lo,pos", [(0, (1, 0, 0)), (16, (0, 1, 0)), (72, (0, 0, 1))])
def test_rope_first_pair_of_each_axis_rotates_by_one_radian(pair_lo, pos):
    # omega_{a,0} = 1, so id 1 on axis a rotates that axis's first pair by 1 rad
    p = np.array([pos], np.int32)
    y = oracle.rope(_basis(pair_lo), p, AX, TH)[0, 0, 0]
    exp = np.zeros(128)
    exp[pair_lo], exp[pair_lo + 1] = math.cos(1.0), math.sin(1.0)
    np.testing.assert_allclose(y, exp, atol=1e-15)
    # the second element of the pair goes to (-sin, cos): fixes the sign
    y = oracle.rope(_basis(pair_lo + 1), p, AX, TH)[0, 0, 0]
    exp = np.zeros(128)
    exp[pair_lo], exp[pair_lo + 1] = -math.sin(1.0), math.cos(1.0)
    np.testing.assert_allclose(y, exp, atol=1e-15)


def test_rope_axis_blocks_are_contiguous_t_h_w():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((1, 1, 3, 128))
    p = np.array([[5, 0, 0], [0, 7, 0], [0, 0, 9]], np.int32)
    r = oracle.rope(y, p, AX, TH)[0, 0]
    y = y[0, 0]
    changed = [np.nonzero(~np.isclose(r[i], y[i], rtol=0, atol=1e-15))[0] for i in range(3)]
    assert set(changed[0]) <= set(range(0, 16)) and len(changed[0]) > 8
    assert set(changed[1]) <= set(range(16, 72)) and len(changed[1]) > 40
    assert set(changed[2]) <= set(range(72, 128)) and len(changed[2]) > 40


def test_rope_pairs_are_adjacent_and_norm_preserving():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((2, 3, 10, 128))
    p = rng.integers(-50, 200, (10, 3)).astype(np.int32)
    r = oracle.rope(y, p, AX, TH)
    n_in = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    n_out = r[..., 0::2] ** 2 + r[..., 1::2] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)


def test_rope_position_zero_is_identity():
    rng = np.random.default_rng(6)
    y = rng.standard_normal((1, 2, 7, 128))
    r = oracle.rope(y, np.zeros((7, 3), np.int32), AX, TH)
    assert np.array_equal(r, y)


def test_rope_composition():
    rng = np.random.default_rng(7)
    y = rng.standard_normal((1, 1, 6, 128))
    a = rng.integers(0, 100, (6, 3)).astype(np.int32)
    b = rng.integers(0, 100, (6, 3)).astype(np.int32)
    two = oracle.rope(oracle.rope(y, a, AX, TH), b, AX, TH)
    one = oracle.rope(y, a + b, AX, TH)
    np.testing.assert_allclose(two, one, atol=1e-12)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 9, 128))
    k = rng.standard_normal((1, 1, 9, 128))
    p = position_ids(1, (2, 4))
    shift = p.copy()
    shift[:, 0] += 3
    shift[:, 1] += 11
    shift[:, 2] -= 5
    s0 = oracle.rope(q, p, AX, TH)[0, 0] @ oracle.rope(k, p, AX, TH)[0, 0].T
    s1 = oracle.rope(q, shift, AX, TH)[0, 0] @ oracle.rope(k, shift, AX, TH)[0, 0].T
    np.testing.assert_allclose(s1, s0, atol=1e-11)


def test_rope_matches_complex_rotation_brute_force():
    # independent construction: each pair as a complex number times e^{i phi}
    rng = np.random.default_rng(9)
    y = rng.standard_normal(128)
    pos = (3, 17, 42)
    out = [0.0] * 128
    off = 0
    for a, d in enumerate(AX):
        for j in range(d // 2):
            phi = pos[a] * TH ** (-2.0 * j / d)
            z = complex(y[off + 2 * j], y[off + 2 * j + 1]) * complex(math.cos(phi), math.sin(phi))
            out[off + 2 * j], out[off + 2 * j + 1] = z.real, z.imag
        off += d
    r = oracle.rope(y[None, None, None], np.array([pos], np.int32), AX, TH)[0, 0, 0]
    np.testing.assert_allclose(r, out, atol=1e-14)


def test_prologue_rms_invariant_survives_rope():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, 2, 12, 128))
    c = 0.8
    p = rng.integers(0, 64, (12, 3)).astype(np.int32)
    qn, kn = oracle.qk_prologue(x, x, np.full(128, c), np.full(128, c), p, AX, TH, EPS)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(qn * qn, axis=-1)),
                               c * np.sqrt(ms / (ms + EPS)), rtol=1e-13)


def test_fp8_prologue_scale_bounds_outputs():
    rng = np.random.default_rng(11)
    w = 1 + 0.1 * rng.standard_normal(128)
    s = oracle.fp8_prologue_out_scale(w)
    # one-hot rows put all the energy on one dimension: the worst case
    x = np.zeros((1, 1, 128, 128))
    x[0, 0, np.arange(128), np.arange(128)] = 5.0
    x = np.concatenate([x, rng.standard_normal((1, 1, 64, 128)) * 3], axis=2)
    p = rng.integers(0, 128, (x.shape[2], 3)).astype(np.int32)
    p[:128] = 0
    y = oracle.rope(oracle.rms_norm(x, w, EPS), p, AX, TH)
    ratio = np.abs(y) / s
    assert ratio.max() <= 448.0
    assert ratio.max() > 447.0   # the bound is reached by the one-hot row at id 0


# ----------------------------------------------------------------- attention

def _sdpa64(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()


def test_attention_matches_torch_sdpa_float64():
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((2, 3, 45, 128)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v, row_block=16),
                               _sdpa64(q, k, v), atol=1e-12)


def test_attention_row_subset_and_peaked_scores():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 2, 70, 128)) * 4
    k = q + 0.05 * rng.standard_normal(q.shape)
    v = rng.standard_normal(q.shape)
    rows = np.array([0, 13, 69])
    got = oracle.attention(q, k, v, rows=rows)
    np.testing.assert_allclose(got, _sdpa64(q, k, v)[:, :, rows], atol=1e-12)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(14)
    N, D = 5, 128
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    o = oracle.attention(q, k, v)[0, 0]
    for i in range(N):
        s = [math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(D)) / math.sqrt(D)
             for j in range(N)]
        e = [math.exp(x) for x in s]
        z = math.fsum(e)
        for d in range(D):
            ref = math.fsum(e[j] * v[0, 0, j, d] for j in range(N)) / z
            assert abs(o[i, d] - ref) < 1e-12


def test_attention_invariants():
    rng = np.random.default_rng(15)
    B, H, N, D = 1, 2, 33, 128
    q, k, v = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    # V == 1 -> 1
    np.testing.assert_allclose(oracle.attention(q, k, np.ones_like(v)), 1.0, atol=1e-14)
    # identical keys -> mean of V
    kk = np.broadcast_to(k[:, :, :1], k.shape)
    np.testing.assert_allclose(oracle.attention(q, kk, v),
                               np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), atol=1e-13)
    # zero queries -> mean of V
    np.testing.assert_allclose(oracle.attention(np.zeros_like(q), k, v),
                               np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), atol=1e-13)
    # N == 1 -> V
    np.testing.assert_allclose(oracle.attention(q[:, :, :1], k[:, :, :1], v[:, :, :1]),
                               v[:, :, :1], atol=1e-15)
    # linear in V
    v2 = rng.standard_normal(v.shape)
    np.testing.assert_allclose(oracle.attention(q, k, 2 * v - 3 * v2),
                               2 * oracle.attention(q, k, v) - 3 * oracle.attention(q, k, v2),
                               atol=1e-12)
    # key permutation invariance, query permutation equivariance
    perm = rng.permutation(N)
    np.testing.assert_allclose(oracle.attention(q, k[:, :, perm], v[:, :, perm]),
                               oracle.attention(q, k, v), atol=1e-13)
    np.testing.assert_allclose(oracle.attention(q[:, :, perm], k, v),
                               oracle.attention(q, k, v)[:, :, perm], atol=1e-13)


def test_joint_brute_force_tiny():
    """Whole chain in pure Python (fsum, complex rotation) on 6 tokens."""
    rng = np.random.default_rng(16)
    N, D = 6, 128
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    wq, wk = 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D)
    pos = np.array([[0, 0, 0], [0, 0, 0], [0, 0, 1], [0, 1, 0], [1, 1, 1], [2, 3, 5]], np.int32)

    def prologue(x, w, p):
        r = math.sqrt(math.fsum(t * t for t in x) / D + EPS)
        y = [x[d] * w[d] / r for d in range(D)]
        out, off = [0.0] * D, 0
        for a, da in enumerate(AX):
            for j in range(da // 2):
                z = complex(y[off + 2 * j], y[off + 2 * j + 1]) * \
                    complex(math.cos(p[a] * TH ** (-2 * j / da)), math.sin(p[a] * TH ** (-2 * j / da)))
                out[off + 2 * j], out[off + 2 * j + 1] = z.real, z.imag
            off += da
        return out

    Q = [prologue(q[0, 0, i], wq, pos[i]) for i in range(N)]
    K = [prologue(k[0, 0, i], wk, pos[i]) for i in range(N)]
    got = oracle.joint_attention(q, k, v, wq, wk, pos, AX, TH, EPS)[0, 0]
    for i in range(N):
        s = [math.fsum(Q[i][d] * K[j][d] for d in range(D)) / math.sqrt(D) for j in range(N)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        z = math.fsum(e)
        for d in range(D):
            assert abs(got[i, d] - math.fsum(e[j] * v[0, 0, j, d] for j in range(N)) / z) < 1e-12


def test_joint_heads_helper_matches_full():
    inp = make_inputs(custom_workload(1, 3, 5, (4, 4)))
    q, k, v = (oracle.torch_to_f64(t) for t in (inp.q, inp.k, inp.v))
    full = oracle.joint_attention(q, k, v, inp.w_q.numpy(), inp.w_k.numpy(), inp.pos.numpy())
    rows = np.array([0, 4, 20])
    part = oracle.joint_attention_heads(q, k, v, inp.w_q.numpy(), inp.w_k.numpy(),
                                        inp.pos.numpy(), [(0, 2), (0, 0)], rows=rows)
    np.testing.assert_allclose(part[0], full[0, 2, rows], atol=1e-14)
    np.testing.assert_allclose(part[1], full[0, 0, rows], atol=1e-14)


def test_identical_raw_keys_at_position_zero_give_mean_of_v():
    rng = np.random.default_rng(17)
    N = 20
    q = rng.standard_normal((1, 1, N, 128))
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, 128)), q.shape)
    v = rng.standard_normal(q.shape)
    w = 1 + 0.1 * rng.standard_normal(128)
    o = oracle.joint_attention(q, k, v, w, w, np.zeros((N, 3), np.int32))
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), atol=1e-13)


# ----------------------------------------------------------------- fp8

def test_fp8_path_reduces_to_bf16_with_unit_scales():
    # values representable in both formats, scale 1: identical decoded inputs
    rng = np.random.default_rng(18)
    grid = oracle.e4m3fn_to_f64(np.arange(0, 0x7E, dtype=np.uint8))
    vals = rng.choice(np.concatenate([grid, -grid]), size=(1, 2, 9, 128))
    t = torch.from_numpy(vals).to(torch.float8_e4m3fn)
    deq = oracle.torch_to_f64(t, torch.ones(1, 2))
    bf = oracle.torch_to_f64(torch.from_numpy(vals).to(torch.bfloat16))
    assert np.array_equal(deq, vals) and np.array_equal(bf, vals)


def test_generator_fp8_quantisation_is_decodable_within_e4m3_precision():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(1, 2, 50, 128, generator=g)
    x8, s = quantize_e4m3_per_head(x)
    deq = oracle.torch_to_f64(x8, s)
    err = np.abs(deq - x.double().numpy())
    bound = 2.0 ** -4 * np.abs(x.double().numpy()) + 2.0 ** -10 * s.double().numpy()[:, :, None, None]
    assert np.all(err <= bound)
    # the per-head amax maps to exactly 448
    assert np.allclose(np.abs(deq).max(axis=(2, 3)), s.double().numpy() * 448.0)


def test_position_ids_layout():
    p = position_ids(3, (2, 3), (2, 2))
    assert p.dtype == np.int32 and p.shape == (3 + 6 + 4, 3)
    assert np.array_equal(p[:3], np.zeros((3, 3)))
    assert np.array_equal(p[3:9], [[0, 0, 0], [0, 0, 1], [0, 0, 2], [0, 1, 0], [0, 1, 1], [0, 1, 2]])
    assert np.array_equal(p[9:], [[1, 0, 0], [1, 0, 1], [1, 1, 0], [1, 1, 1]])

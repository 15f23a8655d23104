"""Pins of the fp64 CPU oracle against closed forms, invariants and a library routine.

The pages give no worked numeric example for the attention layer, so each oracle
function is pinned by facts the mathematics fixes: special inputs whose result can
be written down by hand, invariants (norm preservation, permutation invariance,
all-equal keys), and a textbook special case (numpy float64 softmax(Q K^T) V).
Every plausible slip (a dropped eps, eps outside the square root, sum instead of
mean, a flipped rotation sign, a wrong frequency exponent, a transposed operand,
a missing softmax scale, tail rows leaking in) fails at least one test here.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O

D = 128
EPS = 1e-6
THETA = 1e4


def e(j, d=D, a=1.0):
    x = np.zeros(d)
    x[j] = a
    return x


# ----------------------------------------------------------------------------- bf16
def test_widen_bf16_exact_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F80, 0x0000, 0x8000], np.uint16)
    got = O.widen_bf16(bits)
    assert got[0] == 1.0
    assert got[1] == -2.0
    assert got[2] == 3.140625
    assert got[3] == 2.0 ** -133          # smallest subnormal
    assert math.isinf(got[4]) and got[4] > 0
    assert got[5] == 0.0 and got[6] == 0.0 and math.copysign(1, got[6]) < 0
    assert math.isnan(O.widen_bf16(np.array([0x7FC0], np.uint16))[0])


# -------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_single_channel_closed_form():
    # x = a e_k: mean square a^2/D, so y_k = a w_k / sqrt(a^2/D + eps), others 0.
    w = np.linspace(0.5, 1.5, D)
    a, k = 2.0, 5
    y = O.rmsnorm_row(e(k, a=a), w, EPS)
    expect = a * w[k] / math.sqrt(a * a / D + EPS)
    assert y[k] == pytest.approx(expect, rel=1e-14)
    assert np.count_nonzero(y) == 1


def test_rmsnorm_eps_inside_sqrt_added_to_mean_square():
    # mean square equal to eps: y = x / sqrt(2 eps) = 1e-3 / sqrt(2e-6) = 1/sqrt(2).
    y = O.rmsnorm_row(np.full(D, 1e-3), np.ones(D), EPS)
    np.testing.assert_allclose(y, 1 / math.sqrt(2), rtol=1e-13)


def test_rmsnorm_unit_rms_times_weight():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(D) * 3.0
    ms = np.mean(x * x)
    expect_rms = math.sqrt(ms / (ms + EPS))
    y1 = O.rmsnorm_row(x, np.ones(D), EPS)
    assert math.sqrt(np.mean(y1 * y1)) == pytest.approx(expect_rms, rel=1e-14)
    w = 1 + 0.1 * rng.standard_normal(D)
    yw = O.rmsnorm_row(x, w, EPS)
    np.testing.assert_allclose(yw / w, y1, rtol=1e-13)   # weight applies channel-wise
    np.testing.assert_allclose(y1 / x, y1[0] / x[0], rtol=1e-13)  # direction of x kept


def test_rmsnorm_scale_invariant_without_eps():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(D)
    w = 1 + 0.1 * rng.standard_normal(D)
    np.testing.assert_allclose(O.rmsnorm_row(37.5 * x, w, 0.0), O.rmsnorm_row(x, w, 0.0),
                               rtol=1e-13)


# ----------------------------------------------------------------------------- RoPE
@pytest.mark.parametrize("j", [0, 1, 17, 63])
@pytest.mark.parametrize("p", [1.0, 7.0, 1000.0, 87551.0])
def test_rope_1d_basis_closed_form(j, p):
    # R_p e_j = cos(p w_j) e_j + sin(p w_j) e_{j+64};  R_p e_{j+64} = -sin e_j + cos e_{j+64}
    # with w_j = theta^(-2j/D).
    w_j = THETA ** (-2.0 * j / D)
    c, s = math.cos(p * w_j), math.sin(p * w_j)
    y = O.rope_row(e(j), 0, [p], theta=THETA)
    expect = c * e(j) + s * e(j + 64)
    np.testing.assert_allclose(y, expect, atol=1e-12)
    y2 = O.rope_row(e(j + 64), 0, [p], theta=THETA)
    np.testing.assert_allclose(y2, -s * e(j) + c * e(j + 64), atol=1e-12)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(2).standard_normal(D)
    np.testing.assert_array_equal(O.rope_row(x, 0, [0.0]), x)
    np.testing.assert_array_equal(O.rope_row(x, 1, [0.0, 0.0, 0.0], (32, 48, 48)), x)


def _pairs(sections):
    if sections is None:
        return [(j, j + D // 2) for j in range(D // 2)]
    out, off = [], 0
    for ds in sections:
        out += [(off + j, off + j + ds // 2) for j in range(ds // 2)]
        off += ds
    return out


@pytest.mark.parametrize("mode,pos,sections", [
    (0, [12345.0], None), (1, [98.0, 11.0, 66.0], (32, 48, 48))])
def test_rope_preserves_norm_of_every_pair(mode, pos, sections):
    x = np.random.default_rng(3).standard_normal(D)
    y = O.rope_row(x, mode, pos, sections or (0, 0, 0))
    for a, b in _pairs(sections):
        assert math.hypot(y[a], y[b]) == pytest.approx(math.hypot(x[a], x[b]), rel=1e-12)


@pytest.mark.parametrize("mode,sections", [(0, (0, 0, 0)), (1, (32, 48, 48))])
def test_rope_composition(mode, sections):
    x = np.random.default_rng(4).standard_normal(D)
    a = [3.0, 5.0, 7.0]
    b = [11.0, 2.0, 40.0]
    ab = [u + v for u, v in zip(a, b)]
    y = O.rope_row(O.rope_row(x, mode, b, sections), mode, a, sections)
    np.testing.assert_allclose(y, O.rope_row(x, mode, ab, sections), atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    for p, r in [(100.0, 37.0), (58757.0, 3.0), (5.0, 9000.0)]:
        lhs = O.rope_row(q, 0, [p]) @ O.rope_row(k, 0, [r])
        rhs = O.rope_row(q, 0, [p - r]) @ k
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


@pytest.mark.parametrize("chan,section_off,ds,axis", [
    (1, 0, 32, 0), (15, 0, 32, 0), (32, 32, 48, 1), (40, 32, 48, 1), (81, 80, 48, 2),
    (103, 80, 48, 2)])
def test_rope_3axis_basis_closed_form(chan, section_off, ds, axis):
    pos = [9.0, 4.0, 61.0]
    j = chan - section_off
    w_j = THETA ** (-2.0 * j / ds)
    ang = pos[axis] * w_j
    y = O.rope_row(e(chan), 1, pos, (32, 48, 48))
    np.testing.assert_allclose(y, math.cos(ang) * e(chan) + math.sin(ang) * e(chan + ds // 2),
                               atol=1e-12)


def test_token_positions_1d_then_row_major_grid():
    r = O.make_rope(THETA, 512 + 7800, (32, 48, 48), (99, 12, 67))
    assert O.token_position(r, 0)[0] == 0
    m, p = O.token_position(r, 8311)
    assert m == 0 and p[0] == 8311
    m, p = O.token_position(r, 8312)
    assert m == 1 and list(p) == [0, 0, 0]
    m, p = O.token_position(r, 8312 + 804 * 5 + 67 * 3 + 7)
    assert m == 1 and list(p) == [5, 3, 7]
    m, p = O.token_position(r, 87499)          # video token 79,187: last of the clip
    assert m == 1 and list(p) == [98, 5, 60]
    with pytest.raises(ValueError):
        O.token_position(r, 8312 + 99 * 12 * 67)  # beyond the grid


# ------------------------------------------------------------------------ attention
def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_attention_all_keys_equal_gives_mean_of_values():
    N, H = 50, 2
    q = _rand((7, H, D), 10)
    k = np.broadcast_to(_rand((1, H, D), 11), (N, H, D)).copy()
    v = _rand((N, H, D), 12)
    out = O.attention(q, k, v, 1 / math.sqrt(D))
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(0), out.shape), rtol=1e-12,
                               atol=1e-14)


def test_attention_constant_values_and_single_key():
    q, k = _rand((5, 1, D), 13), _rand((40, 1, D), 14)
    v = np.full((40, 1, D), -0.625)
    np.testing.assert_allclose(O.attention(q, k, v, 0.1), -0.625, rtol=1e-14)
    v1 = _rand((1, 1, D), 15)
    np.testing.assert_allclose(O.attention(q, k[:1], v1, 0.1),
                               np.broadcast_to(v1, (5, 1, D)), rtol=1e-14)


def test_attention_two_keys_sigmoid_closed_form():
    # q = a e_0, k_0 = 0, k_1 = b e_0:  o = (v_0 + e^t v_1) / (1 + e^t), t = scale*a*b.
    a, b, scale = 1.5, 2.0, 1 / math.sqrt(D)
    q = e(0, a=a)[None, None]
    k = np.stack([np.zeros(D), e(0, a=b)])[:, None]
    v = _rand((2, 1, D), 16)
    t = scale * a * b
    expect = (v[0, 0] + math.exp(t) * v[1, 0]) / (1 + math.exp(t))
    np.testing.assert_allclose(O.attention(q, k, v, scale)[0, 0], expect, rtol=1e-13)


def test_attention_joint_key_value_permutation_invariance():
    N = 64
    q, k, v = _rand((9, 2, D), 17), _rand((N, 2, D), 18), _rand((N, 2, D), 19)
    perm = np.random.default_rng(20).permutation(N)
    np.testing.assert_allclose(O.attention(q, k[perm], v[perm], 0.09),
                               O.attention(q, k, v, 0.09), rtol=1e-12, atol=1e-14)


def test_attention_large_margin_selects_one_value():
    N = 20
    k = _rand((N, 1, D), 21) * 0.01
    k[7, 0] = e(3, a=40.0)
    q = e(3, a=40.0)[None, None]
    v = _rand((N, 1, D), 22)
    np.testing.assert_allclose(O.attention(q, k, v, 1.0)[0, 0], v[7, 0], rtol=1e-12)


def test_attention_matches_numpy_float64_library_softmax():
    R, N, H = 31, 300, 2
    q, k, v = _rand((R, H, D), 23), _rand((N, H, D), 24), _rand((N, H, D), 25)
    scale = 1 / math.sqrt(D)
    got = O.attention(q, k, v, scale, threads=3)
    for h in range(H):
        s = (q[:, h] @ k[:, h].T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ v[:, h]
        np.testing.assert_allclose(got[:, h], ref, rtol=1e-12, atol=1e-14)


def test_attention_zero_valid_keys_gives_zeros():
    q = _rand((3, 1, D), 26)
    out = O.attention(q, np.zeros((0, 1, D)), np.zeros((0, 1, D)), 0.1)
    assert np.all(out == 0.0)


# ------------------------------------------------------------- whole layer, by hand
ONE = 0x3F80  # bf16 1.0


def _bf16(x):
    """Exact bf16 bit patterns of values that bf16 represents exactly."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (b >> 16).astype(np.uint16)


def _four_token_case(q_chan, k_chan, v_chan=5, n=4, s_buf=6, rope=None, tail_nan=True):
    q = np.zeros((s_buf, 1, D), np.float32)
    k = np.zeros((s_buf, 1, D), np.float32)
    v = np.zeros((s_buf, 1, D), np.float32)
    for i in range(n):
        q[i, 0, q_chan] = 1.0
        k[i, 0, k_chan] = 1.0
        v[i, 0, v_chan] = i + 1.0
    qb, kb, vb = _bf16(q), _bf16(k), _bf16(v)
    if tail_nan:
        for t in (qb, kb, vb):
            t[n:] = 0x7FC0
    w = np.full(D, ONE, np.uint16)
    rope = rope or O.make_rope(THETA, n)
    return O.attn_layer(qb, kb, vb, n, w, w, EPS, rope, 1 / math.sqrt(D),
                        np.arange(s_buf)), n


def _softmax_mix(scores_row, vals):
    p = [math.exp(s) for s in scores_row]
    return sum(pi * vi for pi, vi in zip(p, vals)) / sum(p)


def test_layer_four_tokens_by_hand_cos_kernel():
    # Q_i = K_i = e_0, w = 1: RMSNorm gives sqrt(128)/sqrt(1 + 128 eps) e_0; RoPE with
    # w_0 = 1 gives c (cos i e_0 + sin i e_64); so s_ij = sqrt(128) cos(i-j) / (1 + 1.28e-4).
    out, n = _four_token_case(0, 0)
    c = math.sqrt(D) / (1 + D * EPS)
    for i in range(n):
        s = [c * math.cos(i - j) for j in range(n)]
        assert out[i, 0, 5] == pytest.approx(_softmax_mix(s, [1, 2, 3, 4]), rel=1e-12)
        assert np.count_nonzero(out[i, 0]) == 1
    assert np.all(out[n:] == 0.0)


def test_layer_four_tokens_by_hand_second_frequency():
    # Channel 1 rotates with w_1 = 1e4^(-1/64): s_ij = sqrt(128) cos((i-j) w_1) / (1+1.28e-4).
    out, n = _four_token_case(1, 1)
    c = math.sqrt(D) / (1 + D * EPS)
    w1 = THETA ** (-1.0 / 64)
    for i in range(n):
        s = [c * math.cos((i - j) * w1) for j in range(n)]
        assert out[i, 0, 5] == pytest.approx(_softmax_mix(s, [1, 2, 3, 4]), rel=1e-12)


def test_layer_four_tokens_by_hand_rotation_sign():
    # Q = e_0, K = e_64:  <R_i e_0, R_j e_64> = sin(i - j), so s_ij = sqrt(128) sin(i-j)/(1+1.28e-4).
    out, n = _four_token_case(0, 64)
    c = math.sqrt(D) / (1 + D * EPS)
    for i in range(n):
        s = [c * math.sin(i - j) for j in range(n)]
        assert out[i, 0, 5] == pytest.approx(_softmax_mix(s, [1, 2, 3, 4]), rel=1e-12)


def test_layer_3axis_by_hand_h_section():
    # All tokens on a (T, H, W) = (2, 2, 2) grid; channel 32 is the first pair of the
    # h section (frequency 1, partner 56): s_ij = sqrt(128) cos(h_i - h_j) / (1+1.28e-4).
    n = 8
    rope = O.make_rope(THETA, 0, (32, 48, 48), (2, 2, 2))
    out, _ = _four_token_case(32, 32, n=n, s_buf=10, rope=rope)
    c = math.sqrt(D) / (1 + D * EPS)
    hpos = [(i // 2) % 2 for i in range(n)]
    for i in range(n):
        s = [c * math.cos(hpos[i] - hpos[j]) for j in range(n)]
        assert out[i, 0, 5] == pytest.approx(_softmax_mix(s, list(range(1, n + 1))),
                                             rel=1e-12)


def test_layer_tail_rows_zero_and_tail_values_ignored():
    rng = np.random.default_rng(30)
    S, N, H = 40, 33, 2

    def draw():
        return _bf16((rng.standard_normal((S, H, D)).astype(np.float32).view(np.uint32)
                      & 0xFFFF0000).view(np.float32))

    q, k, v = draw(), draw(), draw()
    w = np.full(D, ONE, np.uint16)
    rope = O.make_rope(THETA, N)
    rows = np.arange(S)
    base = O.attn_layer(q, k, v, N, w, w, EPS, rope, 0.088, rows)
    for t in (q, k, v):
        t[N:] = 0x7FC0
    nan_tail = O.attn_layer(q, k, v, N, w, w, EPS, rope, 0.088, rows)
    np.testing.assert_array_equal(base, nan_tail)
    assert np.all(nan_tail[N:] == 0.0)
    assert np.all(np.isfinite(nan_tail))


def test_varlen_matches_numpy_library_on_bf16_inputs():
    rng = np.random.default_rng(31)
    S, N, H = 70, 61, 2

    def draw():
        return _bf16((rng.standard_normal((S, H, D)).astype(np.float32).view(np.uint32)
                      & 0xFFFF0000).view(np.float32))

    q, k, v = draw(), draw(), draw()
    scale = 1 / math.sqrt(D)
    got = O.attn_varlen(q, k, v, N, scale, np.arange(S))
    qf, kf, vf = (O.widen_bf16(t) for t in (q, k, v))
    for h in range(H):
        s = (qf[:N, h] @ kf[:N, h].T) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ vf[:N, h]
        np.testing.assert_allclose(got[:N, h], ref, rtol=1e-12, atol=1e-14)
    assert np.all(got[N:] == 0.0)


def test_prologue_per_head_weights_and_shared_weights_agree():
    rng = np.random.default_rng(32)
    S, H = 12, 3
    x = _bf16((rng.standard_normal((S, H, D)).astype(np.float32).view(np.uint32)
               & 0xFFFF0000).view(np.float32))
    wv = _bf16(((1 + 0.1 * rng.standard_normal(D)).astype(np.float32).view(np.uint32)
                & 0xFFFF0000).view(np.float32))
    rope = O.make_rope(THETA, S)
    shared = O.prologue(x, S, wv, EPS, rope, np.arange(S))
    per_head = O.prologue(x, S, np.tile(wv, H), EPS, rope, np.arange(S), w_head_stride=D)
    np.testing.assert_array_equal(shared, per_head)
    # composition: prologue == RoPE(RMSNorm(x)) row by row via the row-level functions
    xf = O.widen_bf16(x)
    wf = O.widen_bf16(wv)
    for t in (0, 5, 11):
        for h in range(H):
            y = O.rope_row(O.rmsnorm_row(xf[t, h], wf, EPS), 0, [float(t)])
            np.testing.assert_array_equal(shared[t, h], y)

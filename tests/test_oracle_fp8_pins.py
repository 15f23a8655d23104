"""Pins of the FP8 ("SAGE") oracle against definitions and closed forms, on the CPU.

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §4.3 and figure 6: Q, K, P and V are
quantized to FP8 for both attention products.  The format (OCP E4M3 "fn": bias 7,
3 mantissa bits, subnormals, largest finite 448) is pinned by brute force over its 254
finite values; the quantizer by its extremes and error bound and by exact rational
arithmetic on values at and next to E4M3 rounding midpoints; the attention by closed
forms (equal keys, one key, power-of-two scaling of a V channel, weights on either side
of a midpoint, the factor 256, the streamed tiles, Skip-Softmax decisions) and by its
distance from exact attention.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O


def e4m3_table():
    """All finite E4M3 values as (value, code) with the code's 3 mantissa bits."""
    out = []
    for sign in (0, 1):
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue  # NaN
                mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                out.append(((-1) ** sign * mag, (sign << 7) | (e << 3) | m))
    return out


TABLE = e4m3_table()

# Every step is fp64, so closed forms involving exp() and a carry between tiles hold to
# fp64 rounding.
CARRY_RTOL = 1e-12
VALUES = np.array(sorted({v for v, _ in TABLE}))
CODE_OF = {}
for v, c in TABLE:
    CODE_OF.setdefault(v, c)


def nearest_e4m3(x):
    """Brute force: the nearest finite E4M3 value, ties to the even code, saturating."""
    if x >= 448:
        return 448.0
    if x <= -448:
        return -448.0
    d = np.abs(VALUES - x)
    best = np.flatnonzero(d == d.min())
    if len(best) == 1:
        return float(VALUES[best[0]])
    even = [VALUES[i] for i in best if CODE_OF[VALUES[i]] % 2 == 0]
    return float(even[0])


def test_every_finite_e4m3_value_maps_to_itself():
    for v, _ in TABLE:
        assert O.e4m3(v) == v, v
    assert VALUES.max() == 448.0 and VALUES[VALUES > 0].min() == 2.0 ** -9


def test_e4m3_midpoints_tie_to_even_and_saturate():
    pos = VALUES[VALUES >= 0]
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        want = a if CODE_OF[a] % 2 == 0 else b
        assert O.e4m3(mid) == want, (a, b)
        assert O.e4m3(-mid) == -want
    for x in (448.0, 464.0, 500.0, 1e30):
        assert O.e4m3(x) == 448.0 and O.e4m3(-x) == -448.0
    assert math.isnan(O.e4m3(float("nan")))


def test_e4m3_matches_brute_force_on_random_values():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(3000) * s for s in (1e-3, 0.05, 1.0, 40.0, 300.0)])
    for x in xs:
        assert O.e4m3(float(x)) == nearest_e4m3(float(x)), x


def test_round_bf16_matches_brute_force():
    rng = np.random.default_rng(4)
    xs = np.concatenate([rng.standard_normal(4000) * s for s in (1e-30, 1e-3, 1.0, 1e5)])
    for x in xs:
        b = int(np.array([x], dtype=np.float32).view(np.uint32)[0] >> 16)
        cands = []
        for c in (b - 1, b, b + 1):
            val = float(np.array([c << 16], dtype=np.uint32).view(np.float32)[0])
            cands.append((abs(val - x), c & 1, c))
        cands.sort()
        want = cands[0][2] if cands[0][0] < cands[1][0] else min(cands[:2], key=lambda t: t[1])[2]
        assert O.round_bf16(float(x)) == want, x


def test_quantize_group_extremes_zero_and_error_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(500) * 3).astype(np.float32)
    codes, scale = O.quantize_group(x)
    i = int(np.argmax(np.abs(x)))
    assert abs(codes[i]) == 448.0 and np.sign(codes[i]) == np.sign(x[i])
    assert scale == pytest.approx(float(np.abs(x).max()) / 448.0, rel=0, abs=0)
    deq = codes * scale
    normal = np.abs(x) / scale >= 2.0 ** -6 * (1 + 1e-6)
    assert np.all(np.abs(deq - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] * (1 + 1e-6))
    assert np.all(np.abs(deq - x)[~normal] <= 2.0 ** -10 * scale * (1 + 1e-6))
    z, zs = O.quantize_group(np.zeros(7, dtype=np.float32))
    assert zs == 0.0 and np.all(z == 0)


def nearest_e4m3_exact(t: Fraction) -> float:
    """Brute force on an exact rational: the nearest finite E4M3 value, ties to the even
    code, saturating at +-448."""
    if t >= 448:
        return 448.0
    if t <= -448:
        return -448.0
    d = [abs(Fraction(float(v)) - t) for v in VALUES]
    m = min(d)
    best = [VALUES[i] for i, x in enumerate(d) if x == m]
    if len(best) == 1:
        return float(best[0])
    return float([v for v in best if CODE_OF[v] % 2 == 0][0])


def bf16_value(bits: int) -> float:
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def test_quantize_decision_is_the_exact_one():
    """The code of x in a group of maximum amax is the E4M3 rounding of the exact rational
    448 x / amax.  Checked with Python fractions on bf16 pairs built to hit E4M3 midpoints
    exactly (ties, which must go to the even code) and on their bf16 neighbours (one ulp
    away, which must go to the nearer code), for amax with mantissas that make 448/amax
    inexact in binary (3, 5, 7, 9, 11, 13 times a power of two) and exact (powers of
    two)."""
    pos = VALUES[VALUES > 0]
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    ties = 0
    checked = 0
    for amax in (1.5, 2.5, 3.5, 4.5, 5.5, 6.5, 0.75, 4.0, 1.0, 0.3125, 6.0, 7.0, 112.0):
        amax = bf16_value(O.round_bf16(amax))
        for mid in mids:
            x0 = mid * amax / 448.0
            b0 = O.round_bf16(x0)
            for bits in (b0 - 1, b0, b0 + 1):
                x = bf16_value(bits)
                if not (0 < x < amax):
                    continue
                t = Fraction(x) * 448 / Fraction(amax)
                codes, scale = O.quantize_group(np.array([amax, x], dtype=np.float32))
                assert codes[0] == 448.0 and scale == amax / 448.0
                assert codes[1] == nearest_e4m3_exact(t), (amax, x, t)
                checked += 1
                if any(t == Fraction(float(m)) for m in mids):
                    ties += 1
                codes, _ = O.quantize_group(np.array([-amax, -x], dtype=np.float32))
                assert codes[1] == -nearest_e4m3_exact(t)
    assert ties >= 20 and checked > 400, (ties, checked)


def bf16(x):
    """bf16 bit patterns (RNE) of a float array."""
    return np.array([O.round_bf16(float(v)) for v in np.ravel(x)], dtype=np.uint16).reshape(
        np.shape(x))


def test_equal_keys_give_mean_of_dequantized_values():
    rng = np.random.default_rng(7)
    S, N, H, D = 40, 37, 2, 128
    q = bf16(rng.standard_normal((S, H, D)))
    k = bf16(np.broadcast_to(rng.standard_normal((1, H, D)), (S, H, D)))
    v = bf16(rng.standard_normal((S, H, D)))
    out = O.attn_varlen_fp8(q, k, v, N, 1 / math.sqrt(D), np.arange(S))
    vf = np.array(v.astype(np.uint32) << 16, dtype=np.uint32).view(np.float32)
    for h in range(H):
        for c in range(D):
            codes, s = O.quantize_group(vf[:N, h, c])
            assert np.allclose(out[:N, h, c], np.mean(codes) * s, rtol=1e-12, atol=1e-15)
    assert np.all(out[N:] == 0)


def test_single_key_returns_its_dequantized_value():
    rng = np.random.default_rng(8)
    S, H, D = 5, 3, 128
    q, k, v = (bf16(rng.standard_normal((S, H, D))) for _ in range(3))
    out = O.attn_varlen_fp8(q, k, v, 1, 0.088, np.array([0, 3]))
    vf = np.array(v.astype(np.uint32) << 16, dtype=np.uint32).view(np.float32)
    for h in range(H):
        for c in range(D):
            codes, s = O.quantize_group(vf[:1, h, c])
            assert out[0, h, c] == codes[0] * s
    assert np.all(out[1] == 0)


def test_power_of_two_scaling_of_one_v_channel_is_isolated():
    """Per-channel V scales: multiplying channel 5 by 2^10 multiplies its output by 2^10
    exactly and leaves every other channel bit-identical."""
    rng = np.random.default_rng(9)
    S, N, H, D = 70, 70, 1, 128
    q, k = bf16(rng.standard_normal((S, H, D))), bf16(rng.standard_normal((S, H, D)))
    vv = rng.standard_normal((S, H, D))
    v1 = bf16(vv)
    vv2 = np.array(v1.astype(np.uint32) << 16, dtype=np.uint32).view(np.float32).astype(np.float64)
    vv2[:, :, 5] *= 1024.0
    v2 = bf16(vv2)
    rows = np.arange(N)
    a = O.attn_varlen_fp8(q, k, v1, N, 0.088, rows)
    b = O.attn_varlen_fp8(q, k, v2, N, 0.088, rows)
    assert np.array_equal(np.delete(a, 5, axis=2), np.delete(b, 5, axis=2))
    assert np.array_equal(a[:, :, 5] * 1024.0, b[:, :, 5])


def test_close_to_exact_attention_but_quantized():
    """FP8 keeps 4 significant bits (per-element relative error up to 2^-4 in Q, K, P and
    V), so the result must stay within 10 % relative L2 of exact attention on the same
    bf16 inputs, and must differ from it (the quantization is really applied)."""
    rng = np.random.default_rng(10)
    S, N, H, D = 300, 290, 2, 128
    q, k, v = (bf16(rng.standard_normal((S, H, D))) for _ in range(3))
    rows = np.arange(N)
    got = O.attn_varlen_fp8(q, k, v, N, 1 / math.sqrt(D), rows)
    ref = O.attn_varlen(q, k, v, N, 1 / math.sqrt(D), rows)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 1e-3 < rel < 0.1, rel


def test_layer_is_prologue_rounded_to_bf16_then_varlen():
    rng = np.random.default_rng(11)
    S, N, H, D = 48, 45, 2, 128
    q, k, v = (bf16(rng.standard_normal((S, H, D))) for _ in range(3))
    wq, wk = bf16(1 + 0.1 * rng.standard_normal(D)), bf16(1 + 0.1 * rng.standard_normal(D))
    rope = O.make_rope(1e4, N)
    rows = np.arange(S)
    got = O.attn_layer_fp8(q, k, v, N, wq, wk, 1e-6, rope, 0.088, rows)
    qn = np.zeros((S, H, D), dtype=np.uint16)
    kn = np.zeros((S, H, D), dtype=np.uint16)
    qn[:N] = bf16(O.prologue(q, N, wq, 1e-6, rope, np.arange(N)))
    kn[:N] = bf16(O.prologue(k, N, wk, 1e-6, rope, np.arange(N)))
    ref = O.attn_varlen_fp8(qn, kn, v, N, 0.088, rows)
    assert np.array_equal(got, ref)


def test_p_is_quantized_and_normalised_by_the_quantized_sum():
    """Two keys in one K block, one channel: K rows (1, 0.5) quantize to exactly 448 and
    224, Q = a e_0 to 448, so the scores are scale*a and scale*a/2.  With scale*a = 2 the
    gap is 1: the weights are 256 and E4M3(256/e) = 96 (256/e = 94.2), and with V = (1, 0)
    in every channel the output is exactly 256 / (256 + 96) (unquantized P would give
    256 / (256 + 94.2))."""
    S, N, H, D = 2, 2, 1, 128
    scale = 0.088
    a = 2.0 / scale
    q = np.zeros((S, H, D))
    q[:, 0, 0] = a
    k = np.zeros((S, H, D))
    k[0, 0, 0], k[1, 0, 0] = 1.0, 0.5
    v = np.zeros((S, H, D))
    v[0] = 1.0
    qb, kb, vb = bf16(q), bf16(k), bf16(v)
    a_b = float(np.array([int(qb[0, 0, 0]) << 16], dtype=np.uint32).view(np.float32)[0])
    assert 92.0 <= 256.0 * math.exp(-scale * a_b / 2) < 100.0  # still rounds to 96
    out = O.attn_varlen_fp8(qb, kb, vb, N, scale, np.array([0]))
    assert np.allclose(out[0, 0], 256.0 / 352.0, rtol=1e-14, atol=0)


def test_streamed_p_equals_global_max_when_the_max_is_in_the_first_tile():
    """The streamed weights use the running maximum of 64-key tiles; when every row's
    largest score is at key 0 the running maximum is the row maximum from the first tile
    on, so the result must equal the one-tile (global maximum) form bit for bit."""
    rng = np.random.default_rng(12)
    S, N, H, D = 200, 197, 2, 128
    q = bf16(np.abs(rng.standard_normal((S, H, D))))
    kk = 0.3 * rng.standard_normal((S, H, D))
    kk[0] = 10.0  # the largest score of every (positive) query row
    k = bf16(kk)
    v = bf16(rng.standard_normal((S, H, D)))
    rows = np.arange(N)
    tiled = O.attn_varlen_fp8(q, k, v, N, 0.088, rows)
    one_tile = O.attn_varlen_fp8(q, k, v, N, 0.088, rows, p_tile=10**9)
    assert np.array_equal(tiled, one_tile)


def test_streamed_p_two_tiles_closed_form():
    """Keys 0-63 (tile 0) score 1, key 64 (tile 1) scores 2; V is 1 on key 64 and 0
    elsewhere.  Tile 0's weights are quantized against its own maximum (256 each) and
    carried over by e^-1, so o = 256 / (64 * 256 / e + 256) = 1 / (64 / e + 1) in every
    channel; quantizing against the row maximum instead would give E4M3(256 / e) = 96
    per key and o = 256 / (64 * 96 + 256) = 0.04."""
    S, N, H, D = 65, 65, 1, 128
    scale = 0.125
    q = np.zeros((S, H, D))
    q[:, 0, 0] = 8.0  # scale * q = 1
    k = np.zeros((S, H, D))
    k[:64, 0, 0] = 1.0
    k[64, 0, 0] = 2.0
    v = np.zeros((S, H, D))
    v[64] = 1.0
    out = O.attn_varlen_fp8(bf16(q), bf16(k), bf16(v), N, scale, np.array([0, 64]))
    want = 1.0 / (64.0 / math.e + 1.0)
    assert np.allclose(out, want, rtol=CARRY_RTOL, atol=0)
    glob = O.attn_varlen_fp8(bf16(q), bf16(k), bf16(v), N, scale, np.array([0]), p_tile=10**9)
    assert np.allclose(glob, 0.04, rtol=1e-12, atol=0)


def _one_channel_case(n, kvals, vvals, scale=0.125):
    """Q = 8 e_0 (scale * q = 1), K = k_j e_0 (score k_j), V = v_j in every channel."""
    S, H, D = n, 1, 128
    q = np.zeros((S, H, D))
    q[:, 0, 0] = 8.0
    k = np.zeros((S, H, D))
    k[:, 0, 0] = kvals
    v = np.broadcast_to(np.asarray(vvals, dtype=np.float64)[:, None, None], (S, H, D)).copy()
    return bf16(q), bf16(k), bf16(v), scale


def test_skip_threshold_zero_is_dense():
    rng = np.random.default_rng(13)
    S, N, H, D = 200, 190, 2, 128
    q, k, v = (bf16(rng.standard_normal((S, H, D)) * s) for s in (3.0, 1.0, 1.0))
    rows = np.arange(N)
    dense = O.attn_varlen_fp8(q, k, v, N, 0.088, rows)
    assert np.array_equal(O.attn_varlen_fp8(q, k, v, N, 0.088, rows, skip_threshold=0.0), dense)
    with pytest.raises(ValueError):
        O.attn_varlen_fp8(q, k, v, N, 0.088, rows, skip_threshold=1.0)


def test_skip_single_key_tile_threshold_sides():
    """Tile 0: 64 keys of score 1 and V = 0; tile 1: one key of score 0 and V = 1.  Its
    factor against the running maximum is e^-1 = 0.367879: a threshold just above it
    (0.3680) drops the tile (output exactly 0), one just below (0.3678) keeps it (weight
    E4M3(256/e) = 96, output 96 / (64 * 256 + 96)).  The thresholds sit 3e-4 apart in
    log2 units from the factor, far above the fp32 rounding of the decision."""
    kv = [1.0] * 64 + [0.0]
    vv = [0.0] * 64 + [1.0]
    q, k, v, scale = _one_channel_case(65, kv, vv)
    rows = np.array([0, 64])
    dropped = O.attn_varlen_fp8(q, k, v, 65, scale, rows, skip_threshold=0.3680)
    kept = O.attn_varlen_fp8(q, k, v, 65, scale, rows, skip_threshold=0.3678)
    assert np.all(dropped == 0.0)
    assert np.allclose(kept, 96.0 / (64 * 256 + 96), rtol=1e-12, atol=0)


def test_skip_never_drops_a_tile_that_raises_the_maximum():
    kv = [1.0] * 64 + [2.0]
    vv = [0.0] * 64 + [1.0]
    q, k, v, scale = _one_channel_case(65, kv, vv)
    out = O.attn_varlen_fp8(q, k, v, 65, scale, np.array([0]), skip_threshold=0.99)
    assert np.allclose(out, 1.0 / (64.0 / math.e + 1.0), rtol=CARRY_RTOL, atol=0)


def test_skip_decides_against_the_running_maximum_before_the_tile():
    """Tiles of scores 1 (V = 1), 0 (V = 0) and one key of score 3 (V = 0), threshold 0.5.
    Tile 1 is dropped (e^-1 < 0.5 against the running maximum 1); tile 0 is kept although
    it is e^-2 below the row maximum, so o = 64 e^-2 / (64 e^-2 + 1).  Keeping tile 1
    would add 64 * 96 e^-2 to the normaliser; judging tile 0 against the row maximum
    would drop it and give 0."""
    kv = [1.0] * 64 + [0.0] * 64 + [3.0]
    vv = [1.0] * 64 + [0.0] * 65
    q, k, v, scale = _one_channel_case(129, kv, vv)
    out = O.attn_varlen_fp8(q, k, v, 129, scale, np.array([5]), skip_threshold=0.5)
    e2 = math.exp(-2.0)
    assert np.allclose(out, 64 * e2 / (64 * e2 + 1.0), rtol=CARRY_RTOL, atol=0)
    dense = O.attn_varlen_fp8(q, k, v, 129, scale, np.array([5]))
    assert np.allclose(dense, 64 * 256 * e2 / (64 * 256 * e2 + 64 * 96 * e2 + 256),
                       rtol=CARRY_RTOL, atol=0)


def _two_key_case(alpha, **kw):
    """Query alpha * e_0 against keys e_0 and 0 (one 16-key block, amax 1), V rows 0 and
    e_5.  The key-0 score exceeds the key-1 score (0) by alpha * scale exactly (the codes
    are 448 and 0, the scales alpha/448 and 1/448)."""
    D = 128
    q = np.zeros((2, 1, D))
    q[:, 0, 0] = alpha
    k = np.zeros((2, 1, D))
    k[0, 0, 0] = 1.0
    v = np.zeros((2, 1, D))
    v[1, 0, 5] = 1.0
    return O.attn_varlen_fp8(bf16(q), bf16(k), bf16(v), 2, 1 / math.sqrt(D), np.array([0]),
                             **kw)


def test_p_is_256_times_the_weight_down_to_the_smallest_subnormal():
    """P = E4M3(256 * 2^(x - m)): a key 17.47 log2 units below the maximum gets
    2^(8 - 17.47), 0.72 of the smallest E4M3 subnormal 2^-9, which rounds up to 2^-9, so
    o_5 = 2^-9 / (256 + 2^-9).  Any other power-of-two factor in
    front of the weights moves this key across the subnormal rounding point (at 128 it
    rounds to 0), so only the factor 256 gives this output."""
    out = _two_key_case(137.0)
    want = np.zeros(128)
    want[5] = 2.0 ** -9 / (256 + 2.0 ** -9)
    assert np.allclose(out[0, 0], want, rtol=1e-12, atol=0)


def test_weights_on_either_side_of_an_e4m3_midpoint():
    """Key 1's weight is 256 exp(-alpha / sqrt(128)).  alpha = 11.5625 gives 92.13, 0.14 %
    above the 88/96 midpoint 92, so the code is 96 and o_5 = 96 / 352; alpha = 11.6250
    gives 91.51, below it, so the code is 88 and o_5 = 88 / 344.  The two alphas are
    bf16 values, so the scores are exact."""
    for alpha, code in ((11.5625, 96.0), (11.625, 88.0)):
        w = 256.0 * math.exp(-alpha / math.sqrt(128))
        assert (w > 92.0) == (code == 96.0) and abs(w - 92.0) < 1.0
        out = _two_key_case(alpha)
        want = np.zeros(128)
        want[5] = code / (256.0 + code)
        assert np.allclose(out[0, 0], want, rtol=1e-14, atol=0), (alpha, out[0, 0, 5])


def test_skip_decision_at_a_fine_margin_from_its_threshold():
    """One key per tile; key 1 sits g = alpha / sqrt(128) nats below the maximum.  A
    threshold exp(-g + 1e-9) drops the tile (o_5 = 0), exp(-g - 1e-9) keeps it
    (o_5 = 96 / 352): the decision is taken on the exact scores, down to fp64 rounding."""
    g = 11.5625 / math.sqrt(128)
    out = _two_key_case(11.5625, p_tile=1, skip_threshold=math.exp(-g + 1e-9))
    assert out[0, 0, 5] == 0.0
    out = _two_key_case(11.5625, p_tile=1, skip_threshold=math.exp(-g - 1e-9))
    assert abs(out[0, 0, 5] - 96.0 / 352) <= 1e-15

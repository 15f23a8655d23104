"""Pins of the dense Skip-Softmax oracle (the "Skip-Softmax-only" control), on the CPU.

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §4.3 and figure 6: a tile-level decision
from the QK result drops the softmax and P x V work of unimportant tiles; a higher
threshold drops more.  Pinned by: threshold 0 equals the dense oracle (a separate
routine: two-pass softmax over all keys); tiles of equal keys are never dropped; a
single-key tile on either side of its factor against the running maximum (closed forms);
a tile that raises the maximum is kept at any threshold; the decision is taken against
the running maximum before the tile, not the row maximum (closed form); the result is a
softmax over the kept keys (against numpy on the kept set); the heaviest weight.
"""
import math

import numpy as np
import pytest

from oracle import oracle as O


def bf16(x):
    return np.array([O.round_bf16(float(v)) for v in np.ravel(x)], dtype=np.uint16).reshape(
        np.shape(x))


def widen(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def one_channel(kvals, vvals, scale=0.125):
    """Q = 8 e_0 (scale * q = 1), K = k_j e_0 (score k_j), V = v_j in every channel."""
    n = len(kvals)
    q = np.zeros((n, 1, 128))
    q[:, 0, 0] = 8.0
    k = np.zeros((n, 1, 128))
    k[:, 0, 0] = kvals
    v = np.broadcast_to(np.asarray(vvals, dtype=np.float64)[:, None, None], (n, 1, 128)).copy()
    return bf16(q), bf16(k), bf16(v), scale


def test_threshold_zero_is_dense_attention():
    rng = np.random.default_rng(21)
    S, N, H, D = 300, 290, 2, 128
    q, k, v = (bf16(rng.standard_normal((S, H, D)) * s) for s in (3.0, 1.0, 1.0))
    rows = np.arange(S)
    dense = O.attn_varlen(q, k, v, N, 0.088, rows)
    got = O.attn_varlen_skip(q, k, v, N, 0.088, rows, 0.0)
    assert np.allclose(got, dense, rtol=1e-12, atol=1e-15)
    assert np.all(got[N:] == 0)
    with pytest.raises(ValueError):
        O.attn_varlen_skip(q, k, v, N, 0.088, rows, 1.0)


def test_equal_keys_are_never_dropped():
    """All keys equal: every tile's maximum equals the running maximum (factor 1), so no
    threshold below 1 drops anything and the output is the mean of V."""
    rng = np.random.default_rng(22)
    S, N, H = 200, 200, 1
    q = bf16(rng.standard_normal((S, H, 128)))
    k = bf16(np.broadcast_to(rng.standard_normal((1, H, 128)), (S, H, 128)))
    v = bf16(rng.standard_normal((S, H, 128)))
    got = O.attn_varlen_skip(q, k, v, N, 0.088, np.arange(N), 0.9)
    assert np.allclose(got, widen(v)[:N].mean(0)[None], rtol=1e-12, atol=1e-14)


def test_single_key_tile_on_either_side_of_the_threshold():
    """Tile 0: 64 keys of score 1, V = 0; tile 1: one key of score 0, V = 1.  Its factor
    against the running maximum is e^-1 = 0.367879: 0.3680 drops it (output 0), 0.3678
    keeps it (output e^-1 / (64 + e^-1))."""
    q, k, v, scale = one_channel([1.0] * 64 + [0.0], [0.0] * 64 + [1.0])
    rows = np.array([0, 64])
    dropped = O.attn_varlen_skip(q, k, v, 65, scale, rows, 0.3680)
    kept = O.attn_varlen_skip(q, k, v, 65, scale, rows, 0.3678)
    assert np.all(dropped == 0.0)
    assert np.allclose(kept, math.exp(-1) / (64 + math.exp(-1)), rtol=1e-13, atol=0)


def test_a_tile_that_raises_the_maximum_is_kept():
    q, k, v, scale = one_channel([1.0] * 64 + [2.0], [0.0] * 64 + [1.0])
    out = O.attn_varlen_skip(q, k, v, 65, scale, np.array([0]), 0.99)
    assert np.allclose(out, 1.0 / (64 / math.e + 1.0), rtol=1e-13, atol=0)


def test_decision_against_the_running_maximum_before_the_tile():
    """Tiles of scores 1 (V = 1), 0 (V = 0) and one key of 3 (V = 0), threshold 0.5:
    tile 1 is dropped (e^-1 < 0.5 against the running maximum 1), tile 0 is kept although
    it is e^-2 below the row maximum: o = 64 e / (64 e + e^3) = 64 / (64 + e^2).  Judging
    tile 0 against the row maximum would drop it (o = 0); keeping tile 1 would give
    64 e / (64 e + 64 + e^3)."""
    q, k, v, scale = one_channel([1.0] * 64 + [0.0] * 64 + [3.0], [1.0] * 64 + [0.0] * 65)
    out = O.attn_varlen_skip(q, k, v, 129, scale, np.array([5]), 0.5)
    assert np.allclose(out, 64 / (64 + math.e ** 2), rtol=1e-13, atol=0)
    dense = O.attn_varlen_skip(q, k, v, 129, scale, np.array([5]), 0.0)
    assert np.allclose(dense, 64 * math.e / (64 * math.e + 64 + math.e ** 3), rtol=1e-13, atol=0)


def test_result_is_a_softmax_over_the_kept_keys():
    """Random peaked rows: the output equals numpy's softmax(s) V over the keys of the
    tiles the rule keeps (the kept set recomputed here from the scores), and the heaviest
    weight is that softmax's largest entry."""
    rng = np.random.default_rng(23)
    S, N, H, D = 700, 650, 1, 128
    q = bf16(rng.standard_normal((S, H, D)) * 4.0)
    k = bf16(rng.standard_normal((S, H, D)))
    v = bf16(rng.standard_normal((S, H, D)))
    lam = 0.05
    rows = np.arange(0, N, 7)
    got, wmax = O.attn_varlen_skip(q, k, v, N, 0.088, rows, lam, with_wmax=True)
    qf, kf, vf = widen(q)[:, 0], widen(k)[:N, 0], widen(v)[:N, 0]
    dropped_any = 0
    for r, i in enumerate(rows):
        s = 0.088 * (kf @ qf[i])
        keep = np.zeros(N, dtype=bool)
        m = -np.inf
        for t0 in range(0, N, 64):
            tmax = s[t0:t0 + 64].max()
            if t0 == 0 or not (tmax - m < math.log(lam)):
                keep[t0:t0 + 64] = True
                m = max(m, tmax)
        dropped_any += (~keep).sum() > 0
        p = np.exp(s[keep] - s[keep].max())
        p /= p.sum()
        assert np.allclose(got[r, 0], p @ vf[keep], rtol=1e-10, atol=1e-13)
        assert abs(wmax[r, 0] - p.max()) <= 1e-13
    assert dropped_any > 10


def test_layer_form_applies_the_fp64_prologue_first():
    rng = np.random.default_rng(24)
    S, N, H, D = 200, 190, 2, 128
    q, k, v = (bf16(rng.standard_normal((S, H, D))) for _ in range(3))
    wq, wk = bf16(1 + 0.1 * rng.standard_normal(D)), bf16(1 + 0.1 * rng.standard_normal(D))
    rope = O.make_rope(1e4, N)
    rows = np.arange(S)
    got = O.attn_layer_skip(q, k, v, N, wq, wk, 1e-6, rope, 0.088, rows, 0.0)
    dense = O.attn_layer(q, k, v, N, wq, wk, 1e-6, rope, 0.088, rows)
    assert np.allclose(got, dense, rtol=1e-12, atol=1e-15)

"""Pins of the block-step oracle (gated residual, LayerNorm, modulation) on the CPU.

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §3.2: the DiT's FP32 modulation,
normalization and residual steps are merged into one operation.  The reading (plain
adaLN): x <- x + gate * a; y = LayerNorm(x) * (1 + scale) + shift.  Pinned by closed
forms, invariances, a zero row, tail handling and an independent LayerNorm routine.
"""
import math

import numpy as np
import torch

from oracle import oracle as O


def bf16_bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def bf16_values(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def call(x, a=None, gate=None, shift=None, scale=None, n=None, eps=1e-6):
    S, C = x.shape
    shift = np.zeros(C) if shift is None else shift
    scale = np.zeros(C) if scale is None else scale
    return O.residual_norm_modulate(x, a, gate, shift, scale, S if n is None else n, eps)


def test_two_channel_closed_form():
    """x = (p, q): mean (p+q)/2, variance ((p-q)/2)^2, so n = +-h / sqrt(h^2 + eps) with
    h = (p-q)/2; then y = n (1 + scale) + shift."""
    x = np.array([[3.0, 1.0], [-2.0, 5.0]], dtype=np.float32)
    scale = np.array([0.5, -0.25], dtype=np.float32)
    shift = np.array([0.125, 2.0], dtype=np.float32)
    eps = 1e-3
    _, y = call(x, shift=shift, scale=scale, eps=eps)
    for t, (p, q) in enumerate(x.astype(np.float64)):
        h = (p - q) / 2
        n = np.array([h, -h]) / math.sqrt(h * h + eps)
        assert np.allclose(y[t], n * (1 + scale.astype(np.float64)) + shift, rtol=1e-14,
                           atol=1e-14)


def test_unmodulated_rows_have_zero_mean_and_known_second_moment():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((7, 96)) * 3 + 1.5).astype(np.float32)
    eps = 1e-2
    _, y = call(x, eps=eps)
    xd = x.astype(np.float64)
    var = xd.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-13)
    assert np.allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-12)


def test_shift_and_scale_invariance_of_the_norm():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    _, y0 = call(x, eps=0.0)
    _, y1 = call((x + np.float32(4.0)).astype(np.float32), eps=0.0)
    _, y2 = call((x * np.float32(8.0)).astype(np.float32), eps=0.0)  # exact power of two
    assert np.allclose(y0, y1, rtol=0, atol=2e-6)  # x + 4 rounds in fp32
    assert np.allclose(y0, y2, rtol=1e-13, atol=1e-13)


def test_modulation_is_the_affine_map_of_the_normalized_row():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 48)).astype(np.float32)
    scale = rng.standard_normal(48).astype(np.float32)
    shift = rng.standard_normal(48).astype(np.float32)
    _, n = call(x)
    _, y = call(x, shift=shift, scale=scale)
    assert np.allclose(y, n * (1 + scale.astype(np.float64)) + shift, rtol=1e-14, atol=1e-14)


def test_residual_that_cancels_the_row_leaves_shift():
    """a = -x (exact: x is drawn as bf16 values), gate 1: the updated row is exactly 0, its
    variance 0, so n = 0 and y = shift exactly; x_out is 0."""
    rng = np.random.default_rng(4)
    a = bf16_bits(rng.standard_normal((3, 32)))
    x = (-bf16_values(a)).astype(np.float32)
    shift = rng.standard_normal(32).astype(np.float32)
    scale = rng.standard_normal(32).astype(np.float32)
    x_out, y = call(x, a=a, gate=np.ones(32, np.float32), shift=shift, scale=scale)
    assert np.all(x_out == 0.0)
    assert np.array_equal(y, np.broadcast_to(shift.astype(np.float64), y.shape))


def test_gate_zero_none_and_one():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 40)).astype(np.float32)
    a = bf16_bits(rng.standard_normal((3, 40)))
    x0, y0 = call(x)
    xz, yz = call(x, a=a, gate=np.zeros(40, np.float32))
    assert np.array_equal(x0, xz) and np.array_equal(y0, yz)
    x1, y1 = call(x, a=a, gate=np.ones(40, np.float32))
    xn, yn = call(x, a=a, gate=None)
    assert np.array_equal(x1, xn) and np.array_equal(y1, yn)
    # gate 2 doubles the branch: x + 2a = (x + a) + a
    x2, _ = call(x, a=a, gate=np.full(40, 2.0, np.float32))
    assert np.allclose(x2 - x1, bf16_values(a), rtol=0, atol=1e-12)


def test_tail_rows_untouched_and_never_read():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((6, 16)).astype(np.float32)
    x[4:] = np.nan
    a = bf16_bits(rng.standard_normal((6, 16)))
    x_out, y = call(x, a=a, gate=np.ones(16, np.float32), n=4)
    assert np.all(np.isfinite(x_out[:4])) and np.all(np.isnan(x_out[4:]))
    assert np.all(y[4:] == 0.0) and np.all(np.isfinite(y[:4]))


def test_matches_torch_layer_norm_in_float64():
    """An independent implementation: torch's layer_norm (no affine) in float64, then the
    modulation."""
    rng = np.random.default_rng(7)
    C = 5376
    x = (rng.standard_normal((9, C)) * 4).astype(np.float32)
    a = bf16_bits(rng.standard_normal((9, C)))
    gate = (rng.standard_normal(C) * 0.3).astype(np.float32)
    shift = (rng.standard_normal(C) * 0.2).astype(np.float32)
    scale = (rng.standard_normal(C) * 0.2).astype(np.float32)
    x_out, y = call(x, a=a, gate=gate, shift=shift, scale=scale)
    r = torch.tensor(x.astype(np.float64)) + torch.tensor(gate.astype(np.float64)) * torch.tensor(
        bf16_values(a))
    ln = torch.nn.functional.layer_norm(r, (C,), eps=1e-6)
    want = ln * (1 + torch.tensor(scale.astype(np.float64))) + torch.tensor(
        shift.astype(np.float64))
    assert np.allclose(x_out, r.numpy(), rtol=0, atol=0)
    assert np.allclose(y, want.numpy(), rtol=1e-11, atol=1e-12)


def test_channel_permutation_equivariance():
    rng = np.random.default_rng(8)
    C = 50
    x = rng.standard_normal((3, C)).astype(np.float32)
    a = bf16_bits(rng.standard_normal((3, C)))
    gate, shift, scale = (rng.standard_normal(C).astype(np.float32) for _ in range(3))
    perm = rng.permutation(C)
    xo, y = call(x, a=a, gate=gate, shift=shift, scale=scale)
    xo2, y2 = call(x[:, perm], a=a[:, perm], gate=gate[perm], shift=shift[perm],
                   scale=scale[perm])
    assert np.array_equal(xo[:, perm], xo2)
    assert np.allclose(y[:, perm], y2, rtol=1e-13, atol=1e-13)

"""CPU pins of the FP8 comparison bar (parity_helpers.fp8_max_bar / assert_close_fp8).

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §4.3 and figure 6 (Q, K, P and V in FP8).

The bar must admit what a correct FP8 kernel can differ by (P codes one E4M3 step from
the oracle's where the exact argument lies near a rounding midpoint) and reject what a
wrong one would produce.  A relative change of 2^-12 in the softmax scale moves every P
argument by a tiny amount and nothing else (Q, K and V codes are unchanged), which flips
exactly the codes near midpoints: the bar must admit it.  Exact (unquantized) attention
and weights quantized against the row maximum instead of the streamed one must fail.
"""
import math

import numpy as np
import pytest

from long_sequence_attention_h3_amd import workloads as W
from oracle import oracle as O

from parity_helpers import MAX_ABS, assert_close_fp8, errors, fp8_max_bar


@pytest.fixture(scope="module")
def case():
    w = W.WORKLOADS[0]
    inp = W.generate(w, tail="nan")
    q, k, v = (W.bits(inp[x][0]) for x in ("q", "k", "v"))
    n = w.n_valid
    rows = np.arange(n)
    scale = 1.0 / math.sqrt(128)
    ref, wmax = O.attn_varlen_fp8(q, k, v, n, scale, rows, with_wmax=True)
    bar = fp8_max_bar(ref, wmax, inp["v"][0, :n].float().numpy())
    return q, k, v, n, rows, scale, ref, wmax, bar


def test_bar_formula():
    ref = np.array([[0.5, -2.0]])
    wmax = np.array([0.25, 0.5])
    v = np.array([[3.0, -4.0]])
    assert fp8_max_bar(ref, wmax, v) == MAX_ABS + 2.0 ** -3 * 0.5 * (4.0 + 2.0)
    # a Skip-Softmax threshold of 0.01 over 64-key tiles: 0.64 of the heaviest weight
    assert fp8_max_bar(ref, wmax, v, 0.01) == pytest.approx(MAX_ABS + 0.64 * 0.5 * 6.0)
    assert fp8_max_bar(ref, wmax, v, 0.001) == MAX_ABS + 2.0 ** -3 * 0.5 * 6.0


def test_wmax_is_the_heaviest_normalised_weight(case):
    """Every row's largest weight lies in (0, 1]; a single valid key weighs exactly 1."""
    *_, wmax, _ = case
    assert np.all(wmax > 0) and np.all(wmax <= 1)
    q, k, v, _, _, scale, *_ = case
    _, w1 = O.attn_varlen_fp8(q, k, v, 1, scale, np.array([0, 5]), with_wmax=True)
    assert np.all(w1[0] == 1.0) and np.all(w1[1] == 0.0)


def test_bar_admits_p_codes_one_step_apart(case):
    q, k, v, n, rows, scale, ref, _, bar = case
    got = O.attn_varlen_fp8(q, k, v, n, scale * (1 + 2.0 ** -12), rows)
    mx, _, rel = errors(got, ref)
    assert mx > 1e-4 and rel > 1e-3  # codes did flip
    assert_close_fp8(got, ref, bar, "scale x (1 + 2^-12)")


def test_bar_rejects_exact_attention(case):
    q, k, v, n, rows, scale, ref, _, bar = case
    exact = O.attn_varlen(q, k, v, n, scale, rows)
    with pytest.raises(AssertionError):
        assert_close_fp8(exact, ref, bar, "exact attention")


def test_bar_rejects_weights_against_the_row_maximum(case):
    q, k, v, n, rows, scale, ref, _, bar = case
    one_tile = O.attn_varlen_fp8(q, k, v, n, scale, rows, p_tile=10 ** 9)
    with pytest.raises(AssertionError):
        assert_close_fp8(one_tile, ref, bar, "one tile")

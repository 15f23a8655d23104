"""Workload table against the numbers the pages print (tests/golden/)."""
import json
import os

import numpy as np

from long_sequence_attention_h3_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "packed_sequence_shapes.json")


def test_full_size_workloads_match_pages_token_counts():
    facts = json.load(open(GOLDEN))["facts"]
    for cfg in (2, 3):
        w = W.WORKLOADS[cfg]
        assert w.n_valid == facts["valid_tokens"]
        assert w.seq_buf == facts["aligned_buffer_tokens"]
        assert w.head_dim == facts["head_projection_channels"]
        assert sum(w.segments) == w.n_valid
    assert W.WORKLOADS[3].heads * W.WORKLOADS[3].head_dim == facts["hidden_channels"]


def test_long_clip_grid_covers_video_tokens():
    w = W.WORKLOADS[4]
    video = w.n_valid - w.rope_n_1d
    assert video == w.segments[2] == 79188
    T, H, Wd = w.grid
    assert (T - 1) * H * Wd < video <= T * H * Wd
    assert sum(w.sections) == w.head_dim


def test_generator_is_seeded_and_fills_tail():
    w = W.Workload("t", heads=2, n_valid=10, seq_buf=16, seed=5)
    a = W.generate(w, tail="nan")
    b = W.generate(w, tail="nan")
    for name in ("q", "k", "v", "w_q", "w_k"):
        assert np.array_equal(W.bits(a[name]), W.bits(b[name]))
    qb = W.bits(a["q"])
    assert np.all(qb[0, 10:] == W.NAN_BF16_BITS)
    assert not np.any(qb[0, :10] == W.NAN_BF16_BITS)
    z = W.generate(w, tail="zero")
    assert np.all(W.bits(z["v"])[0, 10:] == 0)
    assert np.array_equal(W.bits(z["v"])[0, :10], W.bits(a["v"])[0, :10])


def test_sample_rows_include_segment_edges():
    w = W.WORKLOADS[1]
    rows = W.sample_rows(w, 100, seed=7)
    for r in (0, 299, 300, 2149, 2150, 8149):
        assert r in rows
    assert rows == sorted(set(rows)) and rows[-1] == w.n_valid - 1

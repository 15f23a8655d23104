"""GPU parity of dense (bf16) attention with Skip-Softmax, the "Skip-Softmax-only" control,
against its fp64 oracle.

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §4.3 and figure 6: a tile-level decision
from the QK result drops the softmax and P x V work of unimportant tiles.

Inputs carry frame-local structure (workloads.generate_local: tokens attend mostly
within their 804-token frame), since on N(0,1) inputs no tile is ever dropped.  The bar:
the layer's bf16 bar (mean |delta| <= 2e-3, relative L2 <= 1e-2, max |delta| <= 1.5e-2),
with the max bar widened by what one decision taken the other way at its threshold can
move (a tile of 64 keys, each weighing at most lambda times the heaviest weight W of the
checked rows: 64 lambda W R, R = max |V| + max |o|); the kernel decides on fp32 scores,
the oracle on exact ones.
"""
import math

import numpy as np
import pytest
import torch

from long_sequence_attention_h3_amd import binding as B
from long_sequence_attention_h3_amd import workloads as W
from oracle import oracle as O

from parity_helpers import (MAX_ABS, MEAN_ABS, REL_L2, assert_tail_zero, errors, gpu_rope,
                            oracle_rope, rows_of, say, scale_of, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def run(entry, w, d, lam, **kw):
    if entry == "layer":
        out = B.attn_layer_skip(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], d["n_valid"], w.eps,
                                gpu_rope(w), scale_of(w), lam, **kw)
    else:
        out = B.attn_varlen_skip(d["q"], d["k"], d["v"], d["n_valid"], scale_of(w), lam, **kw)
    torch.cuda.synchronize()
    return out


def oracle(entry, w, inp, rows, lam, batch=0):
    q, k, v = (W.bits(inp[x][batch]) for x in ("q", "k", "v"))
    n = inp["n_valid"][batch]
    if entry == "layer":
        ref, wmax = O.attn_layer_skip(q, k, v, n, W.bits(inp["w_q"]), W.bits(inp["w_k"]), w.eps,
                                      oracle_rope(w), scale_of(w), rows, lam, with_wmax=True)
    else:
        ref, wmax = O.attn_varlen_skip(q, k, v, n, scale_of(w), rows, lam, with_wmax=True)
    r = float(inp["v"][batch, :n].float().abs().max()) + float(np.abs(ref).max())
    return ref, MAX_ABS + 64 * lam * float(np.max(wmax)) * r


def check(got, ref, bar, label):
    assert np.all(np.isfinite(got)), label
    mx, mean, rel = errors(got, ref)
    say(f"  {label}: max|d|={mx:.3e} (bar {bar:.3e}) mean|d|={mean:.3e} relL2={rel:.3e}")
    assert mx <= bar and mean <= MEAN_ABS and rel <= REL_L2, label


def skip_rate(ws, x, n):
    counts = B.skip_counts(ws, x)
    waves = (n + 31) // 32
    tiles = (n + 63) // 64
    return int(counts.sum()), int(counts.sum()) / max(1, waves * (tiles - 1) * x.shape[-2])


@pytest.mark.parametrize("alpha,lam,entry", [(10.0, 0.01, "varlen"), (8.0, 0.001, "varlen"),
                                             (12.0, 0.01, "layer")])
def test_skip_matches_oracle(alpha, lam, entry, dev):
    w = W.WORKLOADS[1]
    inp = W.generate_local(w, alpha=alpha)
    d = to_dev(inp, dev)
    say(f"[bf16 skip] {entry} alpha={alpha} lambda={lam}")
    ws = torch.empty(B.workspace_size(d["q"]), dtype=torch.uint8, device=dev)
    out = run(entry, w, d, lam, workspace=ws)
    skipped, rate = skip_rate(ws, d["q"], w.n_valid)
    say(f"  {skipped} wave tiles skipped ({100 * rate:.1f} %)")
    assert_tail_zero(out, inp["n_valid"], entry)
    rows = np.arange(w.n_valid)
    ref, bar = oracle(entry, w, inp, rows, lam)
    check(rows_of(out, rows), ref, bar, f"{entry} skip {lam}")
    if alpha >= 10.0:
        assert rate > 0.1, rate  # whole wave tiles were skipped


def test_skip_full_length_sampled(dev):
    """The 6-head share at full length with frame-local structure, lambda = 0.01, on
    4,096 sampled rows per head."""
    w = W.WORKLOADS[2]
    inp = W.generate_local(w, alpha=12.0)
    d = to_dev(inp, dev)
    ws = torch.empty(B.workspace_size(d["q"]), dtype=torch.uint8, device=dev)
    out = run("layer", w, d, 0.01, workspace=ws)
    skipped, rate = skip_rate(ws, d["q"], w.n_valid)
    say(f"[bf16 skip] full length, lambda=0.01: {100 * rate:.1f} % of wave tiles skipped")
    assert_tail_zero(out, inp["n_valid"], "layer skip")
    rows = W.sample_rows(w, 4096, 50_002)
    ref, bar = oracle("layer", w, inp, rows, 0.01)
    check(rows_of(out, rows), ref, bar, "layer skip full length")
    assert rate > 0.1, rate


def test_skip_result_does_not_depend_on_row_grouping(dev):
    """Permuting the query rows (which regroups them into waves, changing which wave
    tiles are skipped whole) permutes the output bit for bit."""
    w = W.WORKLOADS[1]
    d = to_dev(W.generate_local(w, alpha=10.0), dev)
    n = w.n_valid
    out = run("varlen", w, d, 0.01)
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(78)).to(dev)
    qp = d["q"].clone()
    qp[0, :n] = d["q"][0, perm]
    outp = run("varlen", w, dict(d, q=qp), 0.01)
    assert torch.equal(outp[0, :n].view(torch.int16), out[0, perm].view(torch.int16))


@pytest.mark.parametrize("n_valid", [[1, 0], [65, 300], [320, 127]])
def test_skip_ragged_lengths_and_batches(n_valid, dev):
    w = W.Workload("edge_3h_320", heads=3, n_valid=max(n_valid), seq_buf=320, batch=2,
                   seed=60 + sum(n_valid))
    inp = W.generate(w, tail="nan", n_valid=n_valid)
    inp["q"] = (inp["q"].float() * 4).to(torch.bfloat16)  # peaked rows: tiles get dropped
    d = to_dev(inp, dev)
    for entry in ("varlen", "layer"):
        out = run(entry, w, d, 0.05)
        assert_tail_zero(out, n_valid, entry)
        for b, n in enumerate(n_valid):
            if n == 0:
                continue
            wb = W.Workload("edge", heads=3, n_valid=n, seq_buf=320)
            ref, bar = oracle(entry, wb, inp, np.arange(n), 0.05, batch=b)
            check(rows_of(out, np.arange(n), batch=b), ref, bar, f"{entry} skip N={n} b={b}")


def test_skip_threshold_checked_and_deterministic(dev):
    w = W.WORKLOADS[0]
    d = to_dev(W.generate_local(w, alpha=10.0), dev)
    a = run("layer", w, d, 0.01).view(torch.int16).clone()
    assert torch.equal(run("layer", w, d, 0.01).view(torch.int16), a)
    for bad in (0.0, -0.5, 1.0):
        with pytest.raises(B.H3Error):
            B.attn_varlen_skip(d["q"], d["k"], d["v"], d["n_valid"], scale_of(w), bad)

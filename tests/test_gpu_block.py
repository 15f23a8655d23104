"""GPU parity of h3_residual_norm_modulate (the DiT block steps around attention:
gated residual, LayerNorm, modulation) against the fp64 oracle.

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §3.2.

Bars (derived from the arithmetic):
- the updated residual stream x is one fp32 fused multiply-add x + gate * a of exact
  operands, so it must equal the oracle's exact value rounded to fp32 bit for bit;
- y is the normalized, modulated row rounded to bf16 after fp32 arithmetic (row sums of
  up to 8,192 terms, a reciprocal square root, two fused multiply-adds):
  |y - y_ref| <= 2^-8 |y_ref| + 1e-4 per element (round to nearest bf16 errs by up to
  half an ulp, 2^-8 relative at the bottom of a binade; the absolute term covers the
  fp32 arithmetic);
- rows [N, S): y is +0 and x keeps its bits (NaN tails included).
"""
import numpy as np
import pytest
import torch

from long_sequence_attention_h3_amd import binding as B
from long_sequence_attention_h3_amd import workloads as W
from oracle import oracle as O

from parity_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def check_rows(inp, x_gpu, y_gpu, rows, batch, mode, label):
    """Oracle on the given rows of one batch (the operation is row-independent)."""
    x = inp["x"][batch].numpy()[rows]
    a = bits16(inp["a"][batch])[rows] if mode != "plain" else None
    mod = lambda t: (t if t.dim() == 1 else t[batch]).numpy()  # noqa: E731
    gate = mod(inp["gate"]) if mode == "gated" else None
    x_ref, y_ref = O.residual_norm_modulate(x, a, gate, mod(inp["shift"]), mod(inp["scale"]),
                                            len(rows), 1e-6)
    xg = x_gpu[batch].cpu().numpy()[rows]
    yg = y_gpu[batch].float().cpu().numpy()[rows].astype(np.float64)
    x_exact = x_ref.astype(np.float32)
    mism = int(np.count_nonzero(xg.view(np.uint32) != x_exact.view(np.uint32)))
    err = np.abs(yg - y_ref)
    bound = 2.0 ** -8 * np.abs(y_ref) + 1e-4
    say(f"  {label}: x mismatches {mism} of {xg.size}; y max|d|={err.max():.3e} "
        f"worst ratio {(err / bound).max():.3f}")
    assert mism == 0
    assert np.all(err <= bound)


def run(inp, dev, mode):
    x = inp["x"].to(dev)
    a = inp["a"].to(dev) if mode != "plain" else None
    gate = inp["gate"].to(dev) if mode == "gated" else None
    y = torch.full(x.shape, 7.0, dtype=torch.bfloat16, device=dev)
    B.residual_norm_modulate(x, inp["shift"].to(dev), inp["scale"].to(dev), inp["n_valid"],
                             1e-6, a=a, gate=gate, y=y)
    torch.cuda.synchronize()
    return x.cpu(), y.cpu()


@pytest.mark.parametrize("hidden", [8, 128, 1000, 5376, 8192])
@pytest.mark.parametrize("mode", ["gated", "ungated", "plain"])
def test_block_small_matches_oracle(hidden, mode, dev):
    inp = W.generate_block(70, 65, hidden=hidden, seed=hidden + len(mode))
    say(f"[h3_residual_norm_modulate] S=70 N=65 hidden={hidden} {mode}")
    x_out, y = run(inp, dev, mode)
    check_rows(inp, x_out, y, np.arange(65), 0, mode, f"hidden {hidden} {mode}")
    assert int(torch.count_nonzero(y[0, 65:].view(torch.int16))) == 0
    assert torch.equal(x_out[0, 65:].view(torch.int32), inp["x"][0, 65:].view(torch.int32))
    if mode == "plain":
        assert torch.equal(x_out.view(torch.int32)[0, :65], inp["x"].view(torch.int32)[0, :65])


def test_block_full_length_sampled(dev):
    """The layer's size: 58,758 valid tokens of 58,816, hidden 5,376, gated residual;
    4,096 sampled rows (plus segment edges) against the oracle, x bit for bit and y
    within the bound; every tail row of y is +0."""
    inp = W.generate_block(58816, 58758, hidden=5376, seed=11)
    say("[h3_residual_norm_modulate] S=58816 N=58758 hidden=5376 gated")
    x_out, y = run(inp, dev, "gated")
    w = W.Workload("block", heads=42, n_valid=58758, seq_buf=58816)
    rows = np.asarray(W.sample_rows(w, 4096, 50_000))
    check_rows(inp, x_out, y, rows, 0, "gated", "full length, sampled rows")
    assert int(torch.count_nonzero(y[0, 58758:].view(torch.int16))) == 0


def test_block_batches_with_own_modulation(dev):
    inp = W.generate_block(300, [300, 17], hidden=384, batch=2, seed=5, per_batch_mod=True)
    say("[h3_residual_norm_modulate] two batches, per-batch gate/shift/scale")
    x_out, y = run(inp, dev, "gated")
    for b, n in enumerate(inp["n_valid"]):
        check_rows(inp, x_out, y, np.arange(n), b, "gated", f"batch {b} N={n}")
        assert int(torch.count_nonzero(y[b, n:].view(torch.int16))) == 0


def test_block_deterministic(dev):
    inp = W.generate_block(512, 500, hidden=5376, seed=3)
    outs = [run(inp, dev, "gated") for _ in range(2)]
    assert torch.equal(outs[0][0].view(torch.int32), outs[1][0].view(torch.int32))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))

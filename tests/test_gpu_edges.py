"""Edge cases of the C ABI on the GPU, each against the fp64 oracle or an exact property:
empty and one-token sequences, a valid length equal to the buffer, one key in the last
tile, many all-tail tiles, two batches of different lengths, a fused QKV buffer (row
stride 3*H*D), per-head norm weights, and the all-equal-keys property at full length."""
import numpy as np
import pytest
import torch

from long_sequence_attention_h3_amd import binding as B
from long_sequence_attention_h3_amd import workloads as W

from parity_helpers import (MAX_ABS, MEAN_ABS, REL_L2, assert_close, assert_tail_zero, errors,
                            gpu_layer, gpu_rope, gpu_varlen, oracle_layer, oracle_varlen,
                            rows_of, say, scale_of, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


def small(n, s, heads=3, seed=50, batch=1, **kw):
    return W.Workload(f"edge_{n}of{s}", heads=heads, n_valid=n, seq_buf=s, seed=seed,
                      batch=batch, **kw)


@pytest.mark.parametrize("n,s", [(1, 1), (1, 64), (64, 64), (65, 128), (127, 128),
                                 (300, 2000), (2048, 2048), (777, 1000)])
def test_ragged_lengths_match_oracle(n, s, dev):
    w = small(n, s)
    inp = W.generate(w, tail="nan")
    say(f"[edge] N={n} S={s}")
    for entry, run, orc in (("layer", gpu_layer, oracle_layer),
                            ("varlen", gpu_varlen, oracle_varlen)):
        out = run(w, to_dev(inp, dev))
        assert_tail_zero(out, inp["n_valid"], entry)
        rows = list(range(n))
        assert_close(rows_of(out, rows), orc(w, inp, rows), f"{entry} N={n} S={s}")


@pytest.mark.parametrize("entry", ["layer", "varlen"])
def test_single_token_returns_its_value_exactly(entry, dev):
    """N = 1: the one weight is exp2(0) = 1 in either form of the softmax (with prescaled
    K the score minus its own maximum is exactly 0), so the output is v_0 bit for bit."""
    w = small(1, 80, heads=4, seed=51)
    inp = W.generate(w, tail="nan")
    run = gpu_layer if entry == "layer" else gpu_varlen
    out = run(w, to_dev(inp, dev))
    assert torch.equal(out[0, 0].cpu().view(torch.int16), inp["v"][0, 0].view(torch.int16))
    assert_tail_zero(out, [1], f"{entry} N=1")


@pytest.mark.parametrize("entry", ["layer", "varlen"])
def test_empty_sequence_gives_zeros(entry, dev):
    w = small(0, 200, seed=52)
    inp = W.generate(w, tail="nan")
    run = gpu_layer if entry == "layer" else gpu_varlen
    out = run(w, to_dev(inp, dev), out=torch.full((1, 200, 3, 128), float("nan"),
                                                 dtype=torch.bfloat16, device=dev))
    assert_tail_zero(out, [0], f"{entry} N=0")


def test_two_batches_of_different_lengths(dev):
    w = small(700, 1024, heads=2, seed=53, batch=2, n_1d=1024)
    inp = W.generate(w, tail="nan", n_valid=[700, 1024])
    d = to_dev(inp, dev)
    say("[edge] batch 2, N = 700 and 1024")
    for entry, run, orc in (("layer", gpu_layer, oracle_layer),
                            ("varlen", gpu_varlen, oracle_varlen)):
        out = run(w, d)
        assert_tail_zero(out, inp["n_valid"], entry)
        for b, n in enumerate(inp["n_valid"]):
            rows = list(range(n))
            ref = orc(w, inp, rows, batch=b, n_valid=n) if entry == "layer" else \
                orc(w, inp, rows, batch=b)
            assert_close(rows_of(out, rows, batch=b), ref, f"{entry} batch {b}")


def test_fused_qkv_buffer_row_stride(dev):
    """Q, K and V as views of one [S, 3, H, D] buffer (row stride 3*H*D), output [S, H, D]."""
    w = small(900, 1000, heads=4, seed=54)
    inp = W.generate(w, tail="nan")
    qkv = torch.stack([inp["q"][0], inp["k"][0], inp["v"][0]], dim=1).to(dev)  # [S,3,H,D]
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    assert q.stride(0) == 3 * 4 * 128
    out = B.attn_layer(q, k, v, inp["w_q"].to(dev), inp["w_k"].to(dev), 900, w.eps,
                       gpu_rope(w), scale_of(w))
    torch.cuda.synchronize()
    rows = list(range(900))
    assert_close(rows_of(out.unsqueeze(0), rows), oracle_layer(w, inp, rows), "fused QKV")
    ref = gpu_layer(w, to_dev(inp, dev))
    assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16))


@pytest.mark.parametrize("scale", [None, 1e-11])
def test_layer_k_factor_and_extreme_scale(scale, dev):
    """The K tiles record the factor the layer stored K with: softmax_scale * log2(e)
    for ordinary scales, 1 when that factor would be below 2^-32 (K is then stored as
    given and the kernel applies the scale per score).  Either way the layer matches
    the oracle; at 1e-11 every score is ~0 and each row is the mean of V."""
    import struct

    from oracle import oracle as O
    from parity_helpers import oracle_rope
    w = small(700, 768, heads=2, seed=58)
    sc = scale_of(w) if scale is None else scale
    inp = W.generate(w, tail="nan")
    d = to_dev(inp, dev)
    say(f"[edge] layer K factor, softmax_scale {sc}")
    ws = torch.empty(B.workspace_size(d["q"]), dtype=torch.uint8, device=dev)
    out = B.attn_layer(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], 700, w.eps, gpu_rope(w),
                       sc, workspace=ws)
    torch.cuda.synchronize()
    factor = struct.unpack("<f", bytes(ws[260:264].cpu().tolist()))[0]
    c = float(np.float32(sc) * np.float32(1.4426950408889634))
    assert factor == (c if scale is None else 1.0), factor
    rows = list(range(700))
    ref = oracle_layer(w, inp, rows) if scale is None else O.attn_layer(
        W.bits(inp["q"][0]), W.bits(inp["k"][0]), W.bits(inp["v"][0]), 700, W.bits(inp["w_q"]),
        W.bits(inp["w_k"]), w.eps, oracle_rope(w), sc, np.asarray(rows))
    assert_close(rows_of(out, rows), ref, f"layer scale {sc}")
    assert_tail_zero(out, [700], "layer extreme scale")


def test_per_head_norm_weights(dev):
    """w_head_stride = D: head h uses its own weights; checked against the oracle run
    head by head with that head's weights."""
    from oracle import oracle as O
    w = small(500, 512, heads=3, seed=55)
    inp = W.generate(w, tail="nan")
    g = torch.Generator().manual_seed(56)
    wq = (1 + 0.3 * torch.randn((3, 128), generator=g)).to(torch.bfloat16)
    wk = (1 + 0.3 * torch.randn((3, 128), generator=g)).to(torch.bfloat16)
    d = to_dev(inp, dev)
    out = B.attn_layer(d["q"], d["k"], d["v"], wq.to(dev), wk.to(dev), 500, w.eps, gpu_rope(w),
                       scale_of(w))
    torch.cuda.synchronize()
    rows = np.arange(500)
    ref = O.attn_layer(W.bits(inp["q"][0]), W.bits(inp["k"][0]), W.bits(inp["v"][0]), 500,
                       W.bits(wq), W.bits(wk), w.eps,
                       O.make_rope(w.theta, 500), scale_of(w), rows, w_head_stride=128)
    assert_close(rows_of(out, rows), ref, "per-head weights")


def test_large_scores_mix_both_passes(dev):
    """Scores far above tile 0's row maximum.  Query rows [256, 512) scaled by 8 (their
    256-row workgroup must take the checked pass, the others the fast one) and key 1400
    scaled by 3 (the fast pass then runs with a running max below the true maximum);
    every row against the oracle.  The layer variant scales head 1's w_q by 8, so its
    logits are 8x the workload's, and compares with the plain fp64 oracle: head 0 at the
    layer's bar, head 1 at that bar with its absolute terms scaled by the logit factor
    (the products consume the normalised Q and K rounded to bf16, 2^-9 relative per
    element as in any bf16 attention, so the score errors and, to first order, the
    output errors grow with the logits; relative L2 keeps its 1e-2 gate)."""
    from oracle import oracle as O
    n, s = 1500, 1536
    w = small(n, s, heads=2, seed=57)
    inp = W.generate(w, tail="nan")
    inp["q"][0, 256:512] = (inp["q"][0, 256:512].float() * 8).to(torch.bfloat16)
    inp["k"][0, 1400] = (inp["k"][0, 1400].float() * 3).to(torch.bfloat16)
    d = to_dev(inp, dev)
    say("[edge] large scores, varlen")
    ws = torch.empty(B.workspace_size(d["q"]), dtype=torch.uint8, device=dev)
    out = gpu_varlen(w, d, workspace=ws)
    # rows [256, 512) of both heads were left to the checked pass in every key range,
    # every other workgroup was finished by the fast pass (this grid of 12 query blocks
    # splits its keys into several ranges)
    flags = B.pass_flags(ws, d["q"], n).cpu()
    assert flags.shape[2] == B.attn_splits(d["q"], n)[0] > 1
    want = torch.zeros_like(flags)
    want[:, :, :, 1] = 1
    assert torch.equal(flags, want), flags
    assert_tail_zero(out, [n], "large scores varlen")
    rows = list(range(n))
    assert_close(rows_of(out, rows), oracle_varlen(w, inp, rows), "large scores varlen")

    factor = 8.0
    wq = torch.stack([inp["w_q"], inp["w_q"]]).float()
    wq[1] *= factor
    wq = wq.to(torch.bfloat16)
    wk = torch.stack([inp["w_k"], inp["w_k"]])
    say("[edge] large scores, layer (head 1 w_q x 8)")
    out = B.attn_layer(d["q"], d["k"], d["v"], wq.to(dev), wk.to(dev), n, w.eps, gpu_rope(w),
                       scale_of(w))
    torch.cuda.synchronize()
    ref = O.attn_layer(W.bits(inp["q"][0]), W.bits(inp["k"][0]), W.bits(inp["v"][0]), n,
                       W.bits(wq), W.bits(wk), w.eps, O.make_rope(w.theta, n), scale_of(w),
                       np.asarray(rows), w_head_stride=128)
    got = rows_of(out, rows)
    assert_close(got[:, 0], ref[:, 0], "large scores layer, head 0")
    assert np.all(np.isfinite(got[:, 1]))
    mx, mean, rel = errors(got[:, 1], ref[:, 1])
    say(f"  large scores layer, head 1 (logits x8): max|d|={mx:.3e} mean|d|={mean:.3e} "
        f"relL2={rel:.3e}")
    assert mx <= factor * MAX_ABS and mean <= factor * MEAN_ABS and rel <= REL_L2


def test_equal_keys_give_mean_of_values_at_full_length(dev):
    """All valid K rows zero: every score is 0 after RMSNorm + RoPE, so each output row is
    the mean of the valid V rows (any Q) - a property that holds at any size."""
    w = W.WORKLOADS[2]
    inp = W.generate(w, tail="nan")
    inp["k"][0, : w.n_valid] = 0
    d = to_dev(inp, dev)
    say("[property] zero keys, full length")
    out = gpu_layer(w, d)
    mean = inp["v"][0, : w.n_valid].double().mean(0).numpy()            # [H, D]
    rows = W.sample_rows(w, 256, 7)
    got = rows_of(out, rows)
    assert_close(got, np.broadcast_to(mean, got.shape), "mean of V")

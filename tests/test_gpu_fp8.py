"""GPU parity of the FP8 ("SAGE") attention against the fp64 FP8 oracle.

Page: "vLLM-Omni 上的 MiniMax H3：从系统级优化到基于 FastVideo FastH3 的实时服务"
(Chinese translation of the vLLM blog post), §4.3 and figure 6.

- The FP8 operands the pre-pass writes (K codes with their 16-key block scales, V codes
  and the per-channel V maxima) are compared bit for bit with the oracle's quantizer
  (codes decoded from the OCP E4M3 definition, decided exactly in fp64; scales as fp32
  amax / 448).
- Outputs are compared with the oracle's fp64 FP8 attention (P quantized against the
  running maximum of 64-key tiles) at the FP8 bar of parity_helpers: mean |delta| <=
  2e-3 and relative L2 <= 1e-2 on the differences, and max |delta| <= 1.5e-2 plus what
  one P code one E4M3 step apart (2^-3 of a weight), or one Skip-Softmax decision at its
  threshold, can move on the heaviest normalised weight of the checked rows.
- Every row of the two small workloads; 4,096 sampled query rows per head on the three
  full-length ones.
- Edges: ragged and empty lengths, batches of different lengths, buffer tails of NaN.
"""
import math

import numpy as np
import pytest
import torch

from long_sequence_attention_h3_amd import binding as B
from long_sequence_attention_h3_amd import workloads as W
from oracle import oracle as O

from parity_helpers import (assert_close_fp8, assert_tail_zero, fp8_max_bar, gpu_rope,
                            oracle_rope, rows_of, say, scale_of, to_dev)

pytestmark = pytest.mark.gpu

TILE_BYTES = 19456
K_PITCH, V_PITCH, V_OFF = 144, 80, 9216
ROWS_PER_HEAD = {0: None, 1: None, 2: 4096, 3: 4096, 4: 4096}


def e4m3_values():
    """Value of every E4M3 byte (OCP "fn": bias 7, 0x7F / 0xFF are NaN)."""
    out = np.empty(256)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            out[c] = np.nan
        elif e == 0:
            out[c] = (m / 8) * 2.0 ** -6
        else:
            out[c] = (1 + m / 8) * 2.0 ** (e - 7)
        if s:
            out[c] = -out[c]
    return out


DECODE = e4m3_values()


def v_key(hh, b):
    """Key (within the tile) of byte 32 hh + b of a V channel row."""
    return 32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * hh + (b % 4)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a device"
    return torch.device("cuda:0")


_cache = {}


def inputs(cfg):
    if cfg not in _cache:
        _cache.clear()
        say(f"[inputs] workload {cfg} {W.WORKLOADS[cfg].name}")
        _cache[cfg] = W.generate(W.WORKLOADS[cfg], tail="nan")
    return _cache[cfg]


def gpu_varlen_fp8(w, d, **kw):
    out = B.attn_varlen_fp8(d["q"], d["k"], d["v"], d["n_valid"], scale_of(w), **kw)
    torch.cuda.synchronize()
    return out


def gpu_layer_fp8(w, d, **kw):
    out = B.attn_layer_fp8(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], d["n_valid"], w.eps,
                           gpu_rope(w), scale_of(w), **kw)
    torch.cuda.synchronize()
    return out


def oracle_fp8(w, inp, rows, entry, batch=0, skip=0.0, w_head_stride=0, w_q=None, w_k=None):
    """(output, max bar) of the FP8 oracle on the given rows."""
    q, k, v = (W.bits(inp[x][batch]) for x in ("q", "k", "v"))
    n = inp["n_valid"][batch]
    rows = np.asarray(rows, dtype=np.int64)
    if entry == "varlen":
        out, wmax = O.attn_varlen_fp8(q, k, v, n, scale_of(w), rows, skip_threshold=skip,
                                      with_wmax=True)
    else:
        wq = W.bits(inp["w_q"] if w_q is None else w_q)
        wk = W.bits(inp["w_k"] if w_k is None else w_k)
        out, wmax = O.attn_layer_fp8(q, k, v, n, wq, wk, w.eps, oracle_rope(w), scale_of(w),
                                     rows, w_head_stride=w_head_stride, skip_threshold=skip,
                                     with_wmax=True)
    v_valid = inp["v"][batch, :n].float().numpy()
    return out, fp8_max_bar(out, wmax, v_valid, skip)


@pytest.mark.parametrize("cfg", [0, 1])
def test_fp8_pack_matches_oracle_quantizer_bitwise(cfg, dev):
    w = W.WORKLOADS[cfg]
    inp = inputs(cfg)
    d = to_dev(inp, dev)
    say(f"[h3_kv_pack_fp8] workload {cfg} {w.name}")
    ws = B.kv_pack_fp8(d["k"], d["v"], d["n_valid"])
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    H, S, N, D = w.heads, w.seq_buf, w.n_valid, w.head_dim
    tph = (S + 63) // 64
    nt = (N + 63) // 64
    imgs = raw[:H * tph * TILE_BYTES].reshape(H, tph, TILE_BYTES)[:, :nt]
    vamax = raw[H * tph * TILE_BYTES:H * tph * TILE_BYTES + H * D * 4].view(np.float32)
    vamax = vamax.reshape(H, D)
    kf = inp["k"][0].float().numpy()
    vf = inp["v"][0].float().numpy()
    keys = nt * 64
    # K codes [H, keys, D] and block scales [H, nt, 4]
    kc = imgs[:, :, :64 * K_PITCH].reshape(H, nt, 64, K_PITCH)
    k_codes = kc[:, :, :, :D].reshape(H, keys, D)
    k_scales = kc[:, :, 0, D:D + 16].copy().view(np.float32).reshape(H, nt, 4)
    assert not np.any(kc[:, :, 1:, D:]), "K row pads must be zero"
    # V codes [H, keys, D] in key order
    vc = imgs[:, :, V_OFF:].reshape(H, nt, D, V_PITCH)
    assert not np.any(vc[:, :, :, 64:]), "V row pads must be zero"
    perm = np.array([v_key(hh, b) for hh in (0, 1) for b in range(32)])
    v_codes = np.zeros((H, nt, 64, D), dtype=np.uint8)
    v_codes[:, :, perm, :] = vc[:, :, :, :64].transpose(0, 1, 3, 2)
    v_codes = v_codes.reshape(H, keys, D)
    assert not np.any(k_codes[:, N:]) and not np.any(v_codes[:, N:]), "tail keys not zero"
    for h in range(H):
        for blk in range((N + 15) // 16):
            lo, hi = 16 * blk, min(N, 16 * blk + 16)
            codes, scale = O.quantize_group(kf[lo:hi, h, :])
            got = DECODE[k_codes[h, lo:hi]]
            assert np.array_equal(got, codes), (h, blk)
            assert k_scales[h, blk // 4, blk % 4] == np.float32(scale), (h, blk)
        for blk in range((N + 15) // 16, nt * 4):
            assert k_scales[h, blk // 4, blk % 4] == 0.0
        for c in range(D):
            codes, scale = O.quantize_group(vf[:N, h, c])
            assert vamax[h, c] == np.abs(vf[:N, h, c]).max(), (h, c)
            assert np.array_equal(DECODE[v_codes[h, :N, c]], codes), (h, c)
    say(f"  {H} heads x {nt} tiles: K/V codes, block scales and V maxima bit-exact")


CASES = [(cfg, entry) for cfg in (0, 1, 2, 3, 4) for entry in ("layer", "varlen")]


@pytest.mark.parametrize("cfg,entry", CASES)
def test_fp8_matches_oracle(cfg, entry, dev):
    w = W.WORKLOADS[cfg]
    inp = inputs(cfg)
    say(f"[h3_attn_{entry}_fp8] workload {cfg} {w.name} H={w.heads} N={w.n_valid} "
        f"S={w.seq_buf}")
    run = gpu_layer_fp8 if entry == "layer" else gpu_varlen_fp8
    out = run(w, to_dev(inp, dev))
    assert_tail_zero(out, inp["n_valid"], entry)
    per = ROWS_PER_HEAD[cfg]
    rows = list(range(w.n_valid)) if per is None else W.sample_rows(w, per, 30_000 + cfg)
    say(f"  oracle on {len(rows)} rows x {w.heads} heads")
    ref, bar = oracle_fp8(w, inp, rows, entry)
    assert_close_fp8(rows_of(out, rows), ref, bar, f"{entry}_fp8 cfg{cfg}")


def test_fp8_is_quantized_but_close_to_exact_attention(dev):
    """The FP8 path must really quantize (it differs from exact attention by more than
    bf16 rounding) and stay within FP8 accuracy of it (relative L2 below 0.1)."""
    w = W.WORKLOADS[0]
    inp = inputs(0)
    out = gpu_varlen_fp8(w, to_dev(inp, dev))
    rows = np.arange(w.n_valid)
    exact = O.attn_varlen(W.bits(inp["q"][0]), W.bits(inp["k"][0]), W.bits(inp["v"][0]),
                          w.n_valid, scale_of(w), rows)
    got = rows_of(out, rows)
    rel = np.linalg.norm(got - exact) / np.linalg.norm(exact)
    say(f"  fp8 vs exact attention: relL2={rel:.3e}")
    assert 1e-2 < rel < 0.1


@pytest.mark.parametrize("n_valid", [[1, 0], [17, 64], [65, 300], [320, 127]])
def test_fp8_ragged_lengths_and_batches(n_valid, dev):
    w = W.Workload("edge_3h_320", heads=3, n_valid=max(n_valid), seq_buf=320, batch=2,
                   seed=40 + sum(n_valid))
    inp = W.generate(w, tail="nan", n_valid=n_valid)
    say(f"[fp8 edges] n_valid={n_valid}")
    d = to_dev(inp, dev)
    for entry, run in (("varlen", gpu_varlen_fp8), ("layer", gpu_layer_fp8)):
        out = run(w, d)
        assert_tail_zero(out, n_valid, entry)
        for b, n in enumerate(n_valid):
            if n == 0:
                continue
            rows = list(range(n))
            wb = W.Workload("edge", heads=3, n_valid=n, seq_buf=320, n_1d=None)
            ref, bar = oracle_fp8(wb, inp, rows, entry, batch=b)
            assert_close_fp8(rows_of(out, rows, batch=b), ref, bar, f"{entry}_fp8 N={n} b={b}")


def test_fp8_single_key_returns_dequantized_value(dev):
    """N = 1: every output is the key's V code times its channel scale, up to the bf16
    rounding of the output."""
    w = W.Workload("one_key", heads=2, n_valid=1, seq_buf=64, seed=7)
    inp = W.generate(w, tail="nan")
    out = gpu_varlen_fp8(w, to_dev(inp, dev))
    vf = inp["v"][0, 0].float().numpy()
    want = np.empty_like(vf, dtype=np.float64)
    for h in range(2):
        for c in range(128):
            codes, scale = O.quantize_group(vf[h:h + 1, c])
            want[h, c] = codes[0] * scale
    got = out[0, 0].float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want))  # bf16 rounding only
    assert_tail_zero(out, [1], "one key")


def test_fp8_layer_equals_prologue_then_varlen_bitwise(dev):
    w = W.WORKLOADS[0]
    inp = inputs(0)
    d = to_dev(inp, dev)
    fused = gpu_layer_fp8(w, d)
    q2, k2 = B.qk_rmsnorm_rope(d["q"], d["k"], d["w_q"], d["w_k"], inp["n_valid"], w.eps,
                               gpu_rope(w))
    two = gpu_varlen_fp8(w, dict(d, q=q2, k=k2))
    assert torch.equal(fused.view(torch.int16), two.view(torch.int16))


def test_fp8_deterministic_and_tail_independent(dev):
    w = W.WORKLOADS[1]
    outs = []
    for tail in ("nan", "big", "nan"):
        d = to_dev(W.generate(w, tail=tail), dev)
        outs.append(gpu_layer_fp8(w, d).view(torch.int16).clone())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_fp8_packed_stages_match_one_call(dev):
    """h3_kv_pack_fp8 + h3_attn_packed_fp8 (twice, same workspace) equal h3_attn_layer_fp8."""
    w = W.WORKLOADS[0]
    inp = inputs(0)
    d = to_dev(inp, dev)
    one = gpu_layer_fp8(w, d)
    ws = B.kv_pack_fp8(d["k"], d["v"], d["n_valid"], w_k=d["w_k"], eps=w.eps, rope=gpu_rope(w))
    for _ in range(2):
        two = B.attn_packed_fp8(d["q"], ws, d["n_valid"], scale_of(w), w_q=d["w_q"], eps=w.eps,
                                rope=gpu_rope(w))
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16), two.view(torch.int16))


# ---------------------------------------------------------------- Skip-Softmax
def local_inputs(cfg, alpha, seed=None):
    w = W.WORKLOADS[cfg]
    say(f"[inputs] workload {cfg} {w.name} with frame-local structure, alpha={alpha}")
    return w, W.generate_local(w, alpha=alpha, seed=seed)


def skip_rate(ws, x, n_valid):
    counts = B.fp8_skip_counts(ws, x)
    waves = (n_valid + 31) // 32
    tiles = (n_valid + 63) // 64
    return int(counts.sum()), int(counts.sum()) / max(1, waves * (tiles - 1) * x.shape[-2])


@pytest.mark.parametrize("alpha,lam,entry", [(10.0, 0.01, "varlen"), (8.0, 0.001, "varlen"),
                                             (12.0, 0.01, "layer"), (12.0, 0.1, "layer")])
def test_fp8_skip_softmax_matches_oracle(alpha, lam, entry, dev):
    """Skip-Softmax against the oracle's per-row rule.  alpha = 10, lambda = 0.01 drops
    about half of the (row, tile) pairs and ~40 % of the wave tiles whole; alpha = 8,
    lambda = 0.001 drops a fifth of the pairs with rows of one wave disagreeing (P zeroed
    per row, almost no whole wave tile); on the layer path (RMSNorm shrinks the structure
    by ~1.3x) alpha = 12 drops ~40 % of the pairs and ~20 % of the wave tiles; lambda =
    0.1, the upper part of the bench's threshold sweep, drops more."""
    w, inp = local_inputs(1, alpha)
    d = to_dev(inp, dev)
    ws = torch.empty(B.workspace_size(d["q"], fp8=True), dtype=torch.uint8, device=dev)
    run = gpu_layer_fp8 if entry == "layer" else gpu_varlen_fp8
    out = run(w, d, workspace=ws, skip_threshold=lam)
    skipped, rate = skip_rate(ws, d["q"], w.n_valid)
    dense = run(w, d, skip_threshold=0.0)
    say(f"  {entry} lambda={lam}: {skipped} wave tiles skipped ({100 * rate:.1f} %)")
    assert_tail_zero(out, inp["n_valid"], entry)
    rows = np.arange(w.n_valid)
    ref, bar = oracle_fp8(w, inp, rows, entry, skip=lam)
    assert_close_fp8(rows_of(out, rows), ref, bar, f"{entry}_fp8 skip {lam}")
    assert not torch.equal(out.view(torch.int16), dense.view(torch.int16)), "nothing dropped"
    if alpha >= 10.0:
        assert rate > 0.1, rate  # whole wave tiles were skipped


def test_fp8_skip_result_does_not_depend_on_row_grouping(dev):
    """Each row's result depends on its own scores only: permuting the query rows (which
    regroups them into waves, changing which wave tiles are skipped whole) permutes the
    output bit for bit."""
    w, inp = local_inputs(1, 10.0)
    d = to_dev(inp, dev)
    n = w.n_valid
    out = gpu_varlen_fp8(w, d, skip_threshold=0.01)
    g = torch.Generator().manual_seed(77)
    perm = torch.randperm(n, generator=g).to(dev)
    qp = d["q"].clone()
    qp[0, :n] = d["q"][0, perm]
    outp = gpu_varlen_fp8(w, dict(d, q=qp), skip_threshold=0.01)
    assert torch.equal(outp[0, :n].view(torch.int16), out[0, perm].view(torch.int16))


def test_fp8_skip_counts_zero_when_dense_and_threshold_checked(dev):
    w, inp = local_inputs(0, 10.0)
    d = to_dev(inp, dev)
    ws = torch.empty(B.workspace_size(d["q"], fp8=True), dtype=torch.uint8, device=dev)
    gpu_varlen_fp8(w, d, workspace=ws, skip_threshold=0.01)
    assert skip_rate(ws, d["q"], w.n_valid)[0] > 0
    gpu_varlen_fp8(w, d, workspace=ws, skip_threshold=0.0)
    assert skip_rate(ws, d["q"], w.n_valid)[0] == 0
    for bad in (-0.5, 1.0):
        with pytest.raises(B.H3Error):
            B.attn_varlen_fp8(d["q"], d["k"], d["v"], d["n_valid"], scale_of(w),
                              skip_threshold=bad)


def test_fp8_skip_full_length_sampled(dev):
    """The 6-head share at full length with frame-local structure, lambda = 0.01, on
    4,096 sampled rows per head."""
    w, inp = local_inputs(2, 12.0)
    d = to_dev(inp, dev)
    ws = torch.empty(B.workspace_size(d["q"], fp8=True), dtype=torch.uint8, device=dev)
    out = gpu_layer_fp8(w, d, workspace=ws, skip_threshold=0.01)
    skipped, rate = skip_rate(ws, d["q"], w.n_valid)
    say(f"  layer_fp8 full length, lambda=0.01: {100 * rate:.1f} % of wave tiles skipped")
    rows = W.sample_rows(w, 4096, 40_002)
    ref, bar = oracle_fp8(w, inp, rows, "layer", skip=0.01)
    assert_close_fp8(rows_of(out, rows), ref, bar, "layer_fp8 skip full length")
    assert rate > 0.1, rate


# ---------------------------------------------------------------- layouts and large scores
def test_fp8_fused_qkv_buffer_row_stride(dev):
    """Q, K and V as views of one [S, 3, H, D] buffer (row stride 3*H*D): same result as
    contiguous inputs, bit for bit, and the oracle's."""
    w = W.Workload("qkv_4h_900of1000", heads=4, n_valid=900, seq_buf=1000, seed=54)
    inp = W.generate(w, tail="nan")
    qkv = torch.stack([inp["q"][0], inp["k"][0], inp["v"][0]], dim=1).to(dev)  # [S,3,H,D]
    q, k, v = qkv[:, 0], qkv[:, 1], qkv[:, 2]
    assert q.stride(0) == 3 * 4 * 128
    out = B.attn_layer_fp8(q, k, v, inp["w_q"].to(dev), inp["w_k"].to(dev), 900, w.eps,
                           gpu_rope(w), scale_of(w))
    torch.cuda.synchronize()
    ref = gpu_layer_fp8(w, to_dev(inp, dev))
    assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16))
    rows = list(range(900))
    ref, bar = oracle_fp8(w, inp, rows, "layer")
    assert_close_fp8(rows_of(out.unsqueeze(0), rows), ref, bar, "fused QKV fp8")


def test_fp8_per_head_norm_weights(dev):
    """w_head_stride = D: head h normalises with its own weights (then quantizes)."""
    w = W.Workload("heads_3h_500of512", heads=3, n_valid=500, seq_buf=512, seed=55)
    inp = W.generate(w, tail="nan")
    g = torch.Generator().manual_seed(56)
    wq = (1 + 0.3 * torch.randn((3, 128), generator=g)).to(torch.bfloat16)
    wk = (1 + 0.3 * torch.randn((3, 128), generator=g)).to(torch.bfloat16)
    d = to_dev(inp, dev)
    out = B.attn_layer_fp8(d["q"], d["k"], d["v"], wq.to(dev), wk.to(dev), 500, w.eps,
                           gpu_rope(w), scale_of(w))
    torch.cuda.synchronize()
    rows = np.arange(500)
    ref, bar = oracle_fp8(w, inp, rows, "layer", w_head_stride=128, w_q=wq, w_k=wk)
    assert_close_fp8(rows_of(out, rows), ref, bar, "per-head weights fp8")


def test_fp8_large_scores_raise_the_running_max_often(dev):
    """Raw Q scaled by 6 (scores std ~6): each row's running maximum is raised on many
    tiles, so O and the row sums are carried over repeatedly; tiles are quantized against
    very different maxima."""
    w = W.Workload("peaked_2h_2000of2048", heads=2, n_valid=2000, seq_buf=2048, seed=57)
    inp = W.generate(w, tail="nan")
    inp["q"] = (inp["q"].float() * 6.0).to(torch.bfloat16)  # the NaN tail stays NaN
    out = gpu_varlen_fp8(w, to_dev(inp, dev))
    rows = np.arange(2000)
    ref, bar = oracle_fp8(w, inp, rows, "varlen")
    assert_close_fp8(rows_of(out, rows), ref, bar, "peaked fp8")

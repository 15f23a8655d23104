"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI, run the
fp64 oracle on the same seeded inputs, compare.

Tolerance on bf16 attention outputs (the layer's stated bar): max |delta| <= 1.5e-2 and
mean |delta| <= 2e-3 against the fp64 oracle.  Because outputs at long sequence length
are small (std ~0.007 at N = 58,758), an all-zero output would miss that bar by only
2-3x, so every comparison also gates the relative L2 error at 1e-2 (a correct bf16
kernel sits near 3e-3).
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

from long_sequence_attention_h3_amd import binding as B
from long_sequence_attention_h3_amd import workloads as W
from oracle import oracle as O

MAX_ABS = 1.5e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def scale_of(w: W.Workload) -> float:
    return 1.0 / math.sqrt(w.head_dim)


def gpu_rope(w: W.Workload) -> B.Rope:
    return B.make_rope(w.theta, w.rope_n_1d, w.sections, w.grid)


def oracle_rope(w: W.Workload) -> O.Rope:
    return O.make_rope(w.theta, w.rope_n_1d, w.sections, w.grid)


def to_dev(inp: dict, dev) -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_layer(w: W.Workload, d: dict, **kw) -> torch.Tensor:
    out = B.attn_layer(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], d["n_valid"], w.eps,
                       gpu_rope(w), scale_of(w), **kw)
    torch.cuda.synchronize()
    return out


def gpu_varlen(w: W.Workload, d: dict, **kw) -> torch.Tensor:
    out = B.attn_varlen(d["q"], d["k"], d["v"], d["n_valid"], scale_of(w), **kw)
    torch.cuda.synchronize()
    return out


def rows_of(out: torch.Tensor, rows, batch: int = 0) -> np.ndarray:
    idx = torch.as_tensor(rows, dtype=torch.long, device=out.device)
    return out[batch].index_select(0, idx).float().cpu().numpy().astype(np.float64)


def oracle_layer(w: W.Workload, inp: dict, rows, batch: int = 0, n_valid=None):
    return O.attn_layer(W.bits(inp["q"][batch]), W.bits(inp["k"][batch]),
                        W.bits(inp["v"][batch]),
                        inp["n_valid"][batch] if n_valid is None else n_valid,
                        W.bits(inp["w_q"]), W.bits(inp["w_k"]), w.eps, oracle_rope(w),
                        scale_of(w), np.asarray(rows, dtype=np.int64))


def oracle_varlen(w: W.Workload, inp: dict, rows, batch: int = 0, n_valid=None):
    return O.attn_varlen(W.bits(inp["q"][batch]), W.bits(inp["k"][batch]),
                         W.bits(inp["v"][batch]),
                         inp["n_valid"][batch] if n_valid is None else n_valid, scale_of(w),
                         np.asarray(rows, dtype=np.int64))


def errors(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0, rel


def assert_close(got: np.ndarray, ref: np.ndarray, label: str):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    mx, mean, rel = errors(got, ref)
    say(f"  {label}: max|d|={mx:.3e} mean|d|={mean:.3e} relL2={rel:.3e} over {got.size} values")
    assert mx <= MAX_ABS, f"{label}: max|d| {mx:.3e} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{label}: mean|d| {mean:.3e} > {MEAN_ABS}"
    assert rel <= REL_L2, f"{label}: rel-L2 {rel:.3e} > {REL_L2}"
    return mx, mean, rel


def assert_tail_zero(out: torch.Tensor, n_valid, label: str):
    for b, n in enumerate(n_valid):
        tail = out[b, n:]
        if tail.numel():
            bits = tail.contiguous().view(torch.int16)
            assert int(torch.count_nonzero(bits)) == 0, f"{label}: tail rows not +0 (batch {b})"


def assert_close_allow(got: np.ndarray, ref: np.ndarray, allow: np.ndarray, label: str):
    """FP8 bars.  The mean and relative-L2 bars apply to the differences themselves; the
    max bar applies to the part of each difference beyond the oracle's allowance (P codes
    within the matrix cores' score error of an E4M3 rounding midpoint may come out one
    step apart, and the allowance is the most such codes can move each element).  Flips
    are rare and of either sign, so they leave the mean and L2 at bf16 level; a
    systematic error cannot hide in the allowance."""
    assert got.shape == ref.shape == allow.shape
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    d = np.abs(got - ref)
    raw_mx = float(d.max()) if d.size else 0.0
    mean = float(d.mean()) if d.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    eff = float(np.maximum(d - allow, 0.0).max()) if d.size else 0.0
    say(f"  {label}: max|d|={raw_mx:.3e} (beyond allowance {eff:.3e}) mean|d|={mean:.3e} "
        f"relL2={rel:.3e} over {got.size} values")
    assert eff <= MAX_ABS, f"{label}: max|d| beyond allowance {eff:.3e} > {MAX_ABS}"
    assert mean <= MEAN_ABS, f"{label}: mean|d| {mean:.3e} > {MEAN_ABS}"
    assert rel <= REL_L2, f"{label}: rel-L2 {rel:.3e} > {REL_L2}"
    return eff, mean, rel

"""Workload table and seeded synthetic input generator.

This module holds sizes, seeds and random draws only; none of the layer's
arithmetic lives here.  The tests and the benchmark use it to feed the same
inputs to the GPU library and to the CPU oracle.

Shapes follow the packed text+audio+video sequence of "vLLM-Omni 上的 MiniMax H3"
(Chinese translation of the vLLM blog post): §1 (one packed, jointly denoised
sequence), §3.1 (58,758 valid tokens in a 58,816-token aligned buffer; 128-channel
head projections against a 5,376-channel hidden state, i.e. 42 heads of 128).
The pages carry no tensors, so inputs are bf16 N(0, 1) draws of those shapes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

NAN_BF16_BITS = 0x7FC0  # quiet NaN


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    n_valid: int
    seq_buf: int
    segments: tuple = ()          # (text, audio, video) token counts, in packed order
    head_dim: int = 128
    eps: float = 1e-6
    theta: float = 10000.0
    # Tokens [0, n_1d) take 1-D RoPE; the rest (video) take 3-axis RoPE.
    n_1d: int | None = None       # None: every valid token is 1-D
    sections: tuple = (0, 0, 0)   # channel split (t, h, w) for 3-axis tokens
    grid: tuple = (0, 0, 0)       # (T, H, W) token grid for 3-axis tokens
    seed: int = 0
    batch: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def rope_n_1d(self) -> int:
        return self.n_valid if self.n_1d is None else self.n_1d

    @property
    def flops(self) -> float:
        """Attention FLOP of one call: two N x N x D products at 2 flop per MAC."""
        return 4.0 * self.batch * self.n_valid * self.n_valid * self.head_dim * self.heads


WORKLOADS = {
    0: Workload("tiny_2h_1000of1024", heads=2, n_valid=1000, seq_buf=1024, seed=0),
    1: Workload("mid_8h_8150of8192", heads=8, n_valid=8150, seq_buf=8192,
                segments=(300, 1850, 6000), seed=1),
    2: Workload("share_6h_58758of58816", heads=6, n_valid=58758, seq_buf=58816,
                segments=(512, 5246, 53000), seed=2),
    3: Workload("layer_42h_58758of58816", heads=42, n_valid=58758, seq_buf=58816,
                segments=(512, 5246, 53000), seed=3),
    4: Workload("long_42h_87500of87552", heads=42, n_valid=87500, seq_buf=87552,
                segments=(512, 7800, 79188), n_1d=512 + 7800, sections=(32, 48, 48),
                grid=(99, 12, 67), seed=4),
}


def tail_fill_bits(mode: str) -> int | None:
    """bf16 bit pattern written into the buffer tail: 'nan', 'big' (+3.0e4),
    'zero', or None (leave the N(0,1) draw in place)."""
    return {"nan": NAN_BF16_BITS, "big": 0x46EA, "zero": 0x0000, None: None}[mode]


def generate(w: Workload, tail: str | None = "nan", seed: int | None = None,
             n_valid: list | None = None) -> dict:
    """Seeded bf16 inputs on the CPU.

    Draw order from one ``torch.Generator`` seeded with ``seed`` (default
    ``w.seed``): Q, K, V as fp32 N(0,1) of shape [B, S, H, D] cast to bf16
    (round-to-nearest-even), then w_q = 1 + 0.1 * N(0,1) [D], then w_k likewise.
    Rows [N_b, S) of Q, K and V are then overwritten with ``tail``; ``n_valid`` gives
    N_b per batch (default: ``w.n_valid`` for every batch).
    """
    B, S, H, D = w.batch, w.seq_buf, w.heads, w.head_dim
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    out = {}
    for name in ("q", "k", "v"):
        out[name] = torch.randn((B, S, H, D), generator=g, dtype=torch.float32).to(
            torch.bfloat16)
    for name in ("w_q", "w_k"):
        out[name] = (1.0 + 0.1 * torch.randn((D,), generator=g, dtype=torch.float32)).to(
            torch.bfloat16)
    n_valid = [w.n_valid] * B if n_valid is None else list(n_valid)
    assert len(n_valid) == B and all(0 <= n <= S for n in n_valid)
    _fill_tail(out, tail, n_valid)
    out["n_valid"] = n_valid
    return out


def _fill_tail(out: dict, tail: str | None, n_valid: list):
    fill = tail_fill_bits(tail)
    if fill is not None:
        for name in ("q", "k", "v"):
            bits = out[name].view(torch.int16)
            for b in range(len(n_valid)):
                bits[b, n_valid[b]:] = torch.tensor(fill, dtype=torch.int32).to(torch.int16)


def generate_local(w: Workload, alpha: float = 10.0, frame: int = 804, tail: str | None = "nan",
                   seed: int | None = None) -> dict:
    """Seeded inputs with local structure, a stand-in for the peakier score distributions
    of a trained model: ``generate(w, tail=None, seed)`` (same draws), then one random
    unit direction per block of ``frame`` consecutive tokens and head is added with
    weight ``alpha`` to Q and K of every token of the block, rounded to bf16 again; V is
    unchanged.  The directions (fp32 N(0,1) [ceil(S / frame), H, 32] from a second
    generator seeded with seed + 1,000,003, normalised) occupy channels 48..63 and
    112..127 only: the 16 lowest-frequency pairs of the half-split rotary embedding,
    which turn by less than 1 radian over 804 positions, so the structure survives
    RoPE.  Tokens then attend mostly within their block (804 = 12 x 67 is one video
    frame of the long workload's grid).  Tail rows as in ``generate``."""
    base = w.seed if seed is None else seed
    out = generate(w, tail=None, seed=base)
    B, S, H, D = w.batch, w.seq_buf, w.heads, w.head_dim
    g = torch.Generator(device="cpu")
    g.manual_seed(base + 1_000_003)
    nblk = (S + frame - 1) // frame
    u = torch.randn((nblk, H, 32), generator=g, dtype=torch.float32)
    u = u / u.norm(dim=-1, keepdim=True)
    full = torch.zeros((nblk, H, D), dtype=torch.float32)
    full[:, :, D // 2 - 16:D // 2] = u[:, :, :16]
    full[:, :, D - 16:] = u[:, :, 16:]
    per_token = full.repeat_interleave(frame, dim=0)[:S]  # [S, H, D]
    for name in ("q", "k"):
        out[name] = (out[name].float() + alpha * per_token).to(torch.bfloat16)
    _fill_tail(out, tail, out["n_valid"])
    return out


def generate_block(seq_buf: int, n_valid, hidden: int = 5376, batch: int = 1, seed: int = 0,
                   tail: str | None = "nan", per_batch_mod: bool = False) -> dict:
    """Seeded inputs of the block steps around attention: the fp32 residual stream
    x = 0.5 + 2 N(0,1) [B, S, hidden], the branch output a = bf16(N(0,1)) of the same
    shape, then gate, shift and scale = 0.2 N(0,1) fp32 ([hidden], or [B, hidden] with
    ``per_batch_mod``), drawn in that order from one generator; rows [N_b, S) of x and a
    are overwritten with ``tail`` (x takes the fp32 pattern of the same value)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    B, S, C = batch, seq_buf, hidden
    out = {"x": 0.5 + 2.0 * torch.randn((B, S, C), generator=g, dtype=torch.float32),
           "a": torch.randn((B, S, C), generator=g, dtype=torch.float32).to(torch.bfloat16)}
    shape = (B, C) if per_batch_mod else (C,)
    for name in ("gate", "shift", "scale"):
        out[name] = 0.2 * torch.randn(shape, generator=g, dtype=torch.float32)
    n_valid = [n_valid] * B if isinstance(n_valid, int) else list(n_valid)
    assert len(n_valid) == B and all(0 <= n <= S for n in n_valid)
    fill = {"nan": float("nan"), "big": 3.0e4, "zero": 0.0, None: None}[tail]
    if fill is not None:
        for b in range(B):
            out["x"][b, n_valid[b]:] = fill
            out["a"][b, n_valid[b]:] = fill
    out["n_valid"] = n_valid
    return out


def bits(t: torch.Tensor):
    """Bit patterns of a CPU bf16 tensor as a numpy uint16 array (no copy of values)."""
    return t.contiguous().view(torch.int16).numpy().view("uint16")


def sample_rows(w: Workload, per_head: int, seed: int) -> "list[int]":
    """Query rows to check: ``per_head`` rows drawn uniformly without replacement from
    [0, N) with a fixed seed, plus rows 0 and N-1 and the first and last row of every
    packed segment.  Returned sorted; the same set serves every head."""
    import numpy as np

    n = w.n_valid
    rng = np.random.default_rng(seed)
    k = min(per_head, n)
    rows = set(rng.choice(n, size=k, replace=False).tolist()) if k > 0 else set()
    if n > 0:
        rows.update((0, n - 1))
    start = 0
    for seg in w.segments:
        if seg > 0:
            rows.update((start, start + seg - 1))
        start += seg
    return sorted(r for r in rows if 0 <= r < n)

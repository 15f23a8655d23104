#!/usr/bin/env python3
"""Benchmark of libh3attn on one MI355X.

One step = one h3_attn_layer call (K/V pre-pass + attention with the fused Q
prologue) over the 42-head x 58,758-valid-token packed buffer (58,816 rows) with
inputs already resident in HBM.  Prints one JSON line:

  value      attention TFLOP/s of the whole step, FLOP = 4 * N^2 * D * H
  roofline   the dominant kernel (attention, timed alone via h3_attn_packed with HIP
             events on the launch stream) against the bf16 dense MFMA peak
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the same workload
             (sampled query rows of every head), whose rows also gate parity: the check
             runs on the first h3_attn_layer call, before anything is timed, and a run
             that fails it prints a line with no `value` and exits non-zero
  kernels    the other kernels' achieved bandwidth (K/V pre-pass, standalone prologue, the
             fused residual + LayerNorm + modulation steps around attention)
  fp8        the FP8 (SAGE) variant on the same workload: h3_attn_layer_fp8 per step, its
             attention kernel alone (h3_attn_packed_fp8) against the FP8 dense MFMA peak,
             and its pre-pass; reported beside the bf16 headline, never as `value`.
             fp8.skip_softmax: the same step with Skip-Softmax (threshold 0.01) on these
             inputs and on frame-local inputs of the same shape, with the share of wave
             tiles skipped and the dense bf16 / dense FP8 times on those inputs, and a
             threshold sweep on the frame-local inputs (time, share skipped, distance of
             the output from dense FP8)
  skip_softmax_only  the Skip-Softmax-only control (h3_attn_layer_skip: dense bf16 with
             tile skipping, threshold 0.01) on these and on the frame-local inputs, with
             the same threshold sweep on the frame-local inputs
  per_workload  every workload size: h3_attn_layer and h3_attn_varlen TFLOP/s (median and
             min of 10 calls after 3 warm-up calls), the same for the FP8 calls,
             h3_qk_rmsnorm_rope GB/s, and (unless --no-cpu-baseline) `oracle`: the fp64
             oracle timed on every row of the short workloads and on 4,096 sampled rows
             per head of the long ones (with the full-layer time extrapolated), checked
             against the layer's output on those rows before the workload is timed (a
             workload that fails is not timed)
  sclk_mhz   the shader clock the driver reported right after the timed region

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3]
       python bench.py --only attn   (K/V pre-pass once, then one untimed and K timed
                                      attention launches only, with a JSON line of their
                                      HIP-event time: the run the kernel trace and the
                                      hardware counters are read from)
       python bench.py --only attn_fp8  (the same for the FP8 attention kernel)
       python bench.py --only prologue  (K launches each of the standalone prologue and
                                      the K/V pre-pass, timed the same way)
       python bench.py --only copy   (K copies of a 2 GiB buffer: a plain copy kernel of
                                      known size that calibrates those counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s + % bf16 MFMA peak, 42 heads x 58,758 valid tokens, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5033.2       # MI355X dense FP8 MFMA, published
SKIP_LAMBDA = 0.01             # Skip-Softmax threshold reported by the bench
SKIP_SWEEP = (0.01, 0.05, 0.1, 0.2)  # thresholds of the speed / accuracy sweep
LOCAL_ALPHA = 12.0             # strength of the frame-local input structure
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
KERNEL_SOURCES = ("long_sequence_attention_h3_amd/csrc/attention.hpp",
                  "long_sequence_attention_h3_amd/csrc/common.hpp",
                  "long_sequence_attention_h3_amd/csrc/prologue.hpp",
                  "long_sequence_attention_h3_amd/csrc/h3attn.hip")
FP8_KERNEL_SOURCES = KERNEL_SOURCES + ("long_sequence_attention_h3_amd/csrc/attention_fp8.hpp",)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_traffic.json")
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_traffic.json")


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(path: str = TRAFFIC_FILE, sources=KERNEL_SOURCES):
    """HBM bytes per attention launch from a committed rocprofv3 counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash(sources):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def sclk_mhz():
    """Current shader clock from the driver's DPM table (the level marked '*'), or None."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                for line in f:
                    if "*" in line:
                        return int("".join(ch for ch in line.split(":", 1)[1] if ch.isdigit()))
        except (OSError, ValueError, IndexError):
            continue
    return None


def call_times(torch, stream, fn, warmup: int = 3, reps: int = 10):
    """Per-call HIP-event times (ms) of `fn` on `stream` after `warmup` untimed calls."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def oracle_check(W, w, inp, out_rows, rows, scale):
    """The fp64 oracle of the layer on `rows` of every head, timed, against the GPU rows
    `out_rows` ([R, H, D] float64): seconds, fp64 rate and the parity figures."""
    import numpy as np
    from oracle import oracle as O
    threads = O.default_threads()
    orope = O.make_rope(w.theta, w.rope_n_1d, w.sections, w.grid)
    t0 = time.perf_counter()
    ref = O.attn_layer(W.bits(inp["q"][0]), W.bits(inp["k"][0]), W.bits(inp["v"][0]),
                       w.n_valid, W.bits(inp["w_q"]), W.bits(inp["w_k"]), w.eps, orope, scale,
                       np.asarray(rows, dtype=np.int64), threads=threads)
    t_cpu = time.perf_counter() - t0
    err = np.abs(out_rows - ref)
    rel = float(np.linalg.norm(out_rows - ref) / np.linalg.norm(ref))
    ok = bool(err.max() <= 1.5e-2 and err.mean() <= 2e-3 and rel <= 1e-2)
    flops = 4.0 * len(rows) * w.n_valid * w.head_dim * w.heads
    return {"rows_per_head": len(rows), "all_rows": len(rows) == w.n_valid,
            "threads": threads, "seconds": round(t_cpu, 3),
            "tflops_fp64": round(flops / t_cpu / 1e12, 6),
            "extrapolated_full_layer_s": round(t_cpu * w.n_valid / len(rows), 2),
            "max_abs": float(err.max()), "mean_abs": float(err.mean()), "rel_l2": rel,
            "ok": ok}


def per_workload(torch, B, W, dev, stream, oracle_rows=None, known=None):
    """h3_attn_layer / h3_attn_varlen TFLOP/s and prologue GB/s on every workload size;
    with `oracle_rows`, first the fp64 oracle timed on that many sampled rows per head
    (every row of the workloads with at most 8,192 valid tokens) and checked against the
    layer's output; a workload that fails the check is not timed.  `known`: {index:
    check} already made on the same inputs (the headline workload's)."""
    import statistics
    table = {}
    known = known or {}
    for idx, w in sorted(W.WORKLOADS.items()):
        inp = W.generate(w, tail="nan")
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        rope = B.make_rope(w.theta, w.rope_n_1d, w.sections, w.grid)
        scale = 1.0 / math.sqrt(w.head_dim)
        n = d["n_valid"]
        out = torch.empty_like(d["q"])
        ws = torch.empty(B.workspace_size(d["q"]), dtype=torch.uint8, device=dev)
        orc = known.get(idx)
        if orc is None and oracle_rows is not None:
            rows = (list(range(w.n_valid)) if w.n_valid <= 8192
                    else W.sample_rows(w, oracle_rows, 40_000 + idx))
            B.attn_layer(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], n, w.eps, rope, scale,
                         out=out, workspace=ws)
            idx_t = torch.as_tensor(rows, dtype=torch.long, device=dev)
            got = out[0].index_select(0, idx_t).double().cpu().numpy()
            orc = oracle_check(W, w, inp, got, rows, scale)
        if orc is not None:
            log(f"[bench] {w.name}: oracle {orc['seconds']}s on {orc['rows_per_head']} "
                f"rows/head, max {orc['max_abs']:.2e} mean {orc['mean_abs']:.2e} relL2 "
                f"{orc['rel_l2']:.2e} -> {'ok' if orc['ok'] else 'FAIL'}")
        del inp
        if orc is not None and not orc["ok"]:
            table[w.name] = {"heads": w.heads, "n_valid": w.n_valid, "seq_buf": w.seq_buf,
                             "oracle": orc, "timed": False}
            log(f"[bench] {w.name}: parity FAILED, not timed")
            del d, out, ws
            torch.cuda.empty_cache()
            continue
        ws8 = torch.empty(B.workspace_size(d["q"], fp8=True), dtype=torch.uint8, device=dev)
        q2, k2 = torch.empty_like(d["q"]), torch.empty_like(d["k"])
        row = {"heads": w.heads, "n_valid": w.n_valid, "seq_buf": w.seq_buf,
               "flop": w.flops}
        calls = {
            "h3_attn_layer": lambda: B.attn_layer(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], n,
                                                  w.eps, rope, scale, out=out, workspace=ws),
            "h3_attn_varlen": lambda: B.attn_varlen(d["q"], d["k"], d["v"], n, scale, out=out,
                                                    workspace=ws),
            "h3_attn_layer_fp8": lambda: B.attn_layer_fp8(d["q"], d["k"], d["v"], d["w_q"],
                                                          d["w_k"], n, w.eps, rope, scale,
                                                          out=out, workspace=ws8),
            "h3_attn_varlen_fp8": lambda: B.attn_varlen_fp8(d["q"], d["k"], d["v"], n, scale,
                                                            out=out, workspace=ws8),
        }
        for name, fn in calls.items():
            t = call_times(torch, stream, fn)
            med, mn = statistics.median(t), min(t)
            row[name] = {"ms_median": round(med, 4), "ms_min": round(mn, 4),
                         "tflops_median": round(w.flops / med / 1e9, 2),
                         "tflops_best": round(w.flops / mn / 1e9, 2),
                         "frac_bf16_peak_median": round(w.flops / med / 1e9 / PEAK_BF16_TFLOPS, 4)}
        t = call_times(torch, stream, lambda: B.qk_rmsnorm_rope(
            d["q"], d["k"], d["w_q"], d["w_k"], n, w.eps, rope, q_out=q2, k_out=k2))
        med = statistics.median(t)
        nbytes = 2 * 2 * w.batch * w.n_valid * w.heads * w.head_dim * 2
        row["h3_qk_rmsnorm_rope"] = {"ms_median": round(med, 4), "bytes": nbytes,
                                     "GB/s": round(nbytes / med / 1e6, 1)}
        if orc is not None:
            row["oracle"] = orc
        table[w.name] = row
        log(f"[bench] {w.name}: layer {row['h3_attn_layer']['tflops_median']} TFLOP/s, varlen "
            f"{row['h3_attn_varlen']['tflops_median']} TFLOP/s, layer_fp8 "
            f"{row['h3_attn_layer_fp8']['tflops_median']} TFLOP/s, prologue "
            f"{row['h3_qk_rmsnorm_rope']['GB/s']} GB/s")
        del d, out, ws, ws8, q2, k2
        torch.cuda.empty_cache()
    return table


def copy_only(torch, dev, steps: int) -> int:
    """A plain device-to-device copy of 2 GiB, `steps` times: 2 GiB read and 2 GiB
    written per launch, the known sizes the traffic counters are scaled by."""
    src = torch.ones(1 << 30, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    for i in range(steps):
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy {i + 1}/{steps} of {src.numel() * 2} bytes done")
    return 0


def workload_config(w) -> dict:
    return {"workload": w.name, "heads": w.heads, "head_dim": w.head_dim,
            "n_valid": w.n_valid, "seq_buf": w.seq_buf, "batch": w.batch,
            "entry": "h3_attn_layer", "rope": "1-D" if w.n_1d is None else "1-D+3-axis",
            "parallelism": "single GPU"}


def refusal(w, check: dict) -> str:
    """The one JSON line of a run whose parity check failed: nothing was timed, so there
    is no `value`."""
    return json.dumps({"metric": METRIC, "unit": "TFLOP/s", "n_gpus": 1, "data": "synthetic",
                       "config": workload_config(w), "parity": check,
                       "error": "h3_attn_layer does not match the fp64 oracle; not timed"})


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--cpu-rows-per-head", type=int, default=4096)
    ap.add_argument("--oracle-rows-per-head", type=int, default=4096,
                    help="sampled rows per head of the per-workload oracle check on the "
                         "long workloads (the short ones are checked on every row)")
    ap.add_argument("--no-per-workload", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large-scores", action="store_true",
                    help="skip the checked-pass measurement (keeps a kernel trace to the "
                         "headline's launches)")
    ap.add_argument("--only", choices=("all", "attn", "attn_fp8", "prologue", "copy"),
                    default="all")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}): the layer is "
              "measured on one GPU's share (a head-sharded multi-GPU layer is not implemented).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from long_sequence_attention_h3_amd import binding as B
    from long_sequence_attention_h3_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    if args.only == "copy":
        return copy_only(torch, dev, args.steps)
    w = W.WORKLOADS[args.workload]
    log(f"[bench] workload {args.workload} {w.name}: H={w.heads} N={w.n_valid} S={w.seq_buf}")
    t0 = time.time()
    inp = W.generate(w, tail="nan")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s")
    rope = B.make_rope(w.theta, w.rope_n_1d, w.sections, w.grid)
    scale = 1.0 / math.sqrt(w.head_dim)
    n = d["n_valid"]
    out = torch.empty_like(d["q"])
    ws = torch.empty(B.workspace_size(d["q"]), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        B.attn_layer(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], n, w.eps, rope, scale,
                     out=out, workspace=ws)

    def launches(name, fn, nbytes=None, flop=None, sources=KERNEL_SOURCES):
        """One untimed call, then args.steps calls bracketed by HIP events on the launch
        stream; returns the record of their average time (source_hash: of `sources`)."""
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn()
            log(f"[bench] {name} launch {i + 1}/{args.steps} issued")
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        rec = {"only": name, "workload": w.name, "launches_timed": args.steps,
               "launches_total": args.steps + 1, "ms_per_launch": round(ms, 4),
               "sclk_mhz": sclk_mhz(), "source_hash": source_hash(sources)}
        if flop is not None:
            rec["tflops"] = round(flop / ms / 1e9, 2)
            rec["frac_bf16_peak"] = round(flop / ms / 1e9 / PEAK_BF16_TFLOPS, 4)
        if nbytes is not None:
            rec["bytes"] = nbytes
            rec["GB/s"] = round(nbytes / ms / 1e6, 1)
        return rec

    if args.only == "attn":
        B.kv_pack(d["k"], d["v"], n, workspace=ws, w_k=d["w_k"], eps=w.eps, rope=rope,
                  softmax_scale=scale)
        rec = launches("attn", lambda: B.attn_packed(d["q"], ws, n, scale, w_q=d["w_q"],
                                                     eps=w.eps, rope=rope, out=out),
                       flop=w.flops)
        rec["kernels"] = "attn_fwd_kernel fast pass + checked pass per launch"
        print(json.dumps(rec), flush=True)
        return 0
    if args.only == "attn_fp8":
        ws8 = torch.empty(B.workspace_size(d["q"], fp8=True), dtype=torch.uint8, device=dev)
        B.kv_pack_fp8(d["k"], d["v"], n, workspace=ws8, w_k=d["w_k"], eps=w.eps, rope=rope)
        rec = launches("attn_fp8", lambda: B.attn_packed_fp8(d["q"], ws8, n, scale,
                                                             w_q=d["w_q"], eps=w.eps,
                                                             rope=rope, out=out),
                       flop=w.flops, sources=FP8_KERNEL_SOURCES)
        rec["frac_fp8_peak"] = round(rec["tflops"] / PEAK_FP8_TFLOPS, 4)
        print(json.dumps(rec), flush=True)
        return 0
    if args.only == "prologue":
        row_bytes = w.heads * w.head_dim * 2
        q2, k2 = torch.empty_like(d["q"]), torch.empty_like(d["k"])
        recs = [launches("qk_norm_rope_kernel", lambda: B.qk_rmsnorm_rope(
            d["q"], d["k"], d["w_q"], d["w_k"], n, w.eps, rope, q_out=q2, k_out=k2),
            nbytes=2 * 2 * w.n_valid * row_bytes)]
        tiles = (w.n_valid + 63) // 64
        recs.append(launches("kv_pack_kernel", lambda: B.kv_pack(
            d["k"], d["v"], n, workspace=ws, w_k=d["w_k"], eps=w.eps, rope=rope,
            softmax_scale=scale), nbytes=2 * w.n_valid * row_bytes + w.heads * tiles * 35840))
        for r in recs:
            print(json.dumps(r), flush=True)
        return 0

    # ---- parity first: the first h3_attn_layer call against the fp64 oracle on sampled
    # rows of every head (the CPU baseline's sample; 64 rows per head with
    # --no-cpu-baseline).  A failing configuration is not timed.
    step()
    torch.cuda.synchronize()
    layer_out = out.clone()
    rows = W.sample_rows(w, 64 if args.no_cpu_baseline else args.cpu_rows_per_head,
                         30_000 + args.workload)
    idx = torch.as_tensor(rows, dtype=torch.long, device=dev)
    got = layer_out[0].index_select(0, idx).double().cpu().numpy()
    log(f"[bench] oracle on {len(rows)} rows x {w.heads} heads before timing")
    check = oracle_check(W, w, inp, got, rows, scale)
    log(f"[bench] oracle {check['seconds']}s; parity max {check['max_abs']:.2e} mean "
        f"{check['mean_abs']:.2e} relL2 {check['rel_l2']:.2e} -> "
        f"{'ok' if check['ok'] else 'FAIL'}")
    if not check["ok"]:
        print(refusal(w, check), flush=True)
        return 1

    # ---- headline: K whole-layer steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    sclk = sclk_mhz()
    flops = w.flops
    value = flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] h3_attn_layer {ms_step:.3f} ms/step  {value:.1f} TFLOP/s "
        f"({100 * value / PEAK_BF16_TFLOPS:.1f}% of bf16 peak), wall {wall:.3f}s")
    assert torch.equal(out.view(torch.int16), layer_out.view(torch.int16)), \
        "timed calls differ from the checked call"

    # ---- dominant kernel alone: attention from packed K/V (fused Q prologue).  One call
    # is the fast pass plus the checked pass, which returns at once for workgroups the
    # fast pass finished (all of them on this workload); the events bracket both.
    B.kv_pack(d["k"], d["v"], n, workspace=ws, w_k=d["w_k"], eps=w.eps, rope=rope,
              softmax_scale=scale)
    for _ in range(2):
        B.attn_packed(d["q"], ws, n, scale, w_q=d["w_q"], eps=w.eps, rope=rope, out=out)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        B.attn_packed(d["q"], ws, n, scale, w_q=d["w_q"], eps=w.eps, rope=rope, out=out)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_attn = e0.elapsed_time(e1) / args.steps
    achieved = flops / (ms_attn * 1e-3) / 1e12
    assert torch.equal(out.view(torch.int16), layer_out.view(torch.int16)), \
        "two-stage call differs from h3_attn_layer"
    log(f"[bench] attention kernel {ms_attn:.3f} ms  {achieved:.1f} TFLOP/s")

    # ---- other kernels: K/V pre-pass and the standalone prologue (HBM-bound)
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    row_bytes = w.heads * w.head_dim * 2
    tiles = (w.n_valid + 63) // 64
    pack_bytes = 2 * w.n_valid * row_bytes + w.heads * tiles * 35840
    ms_pack = timed(lambda: B.kv_pack(d["k"], d["v"], n, workspace=ws, w_k=d["w_k"], eps=w.eps,
                                      rope=rope, softmax_scale=scale), args.steps)
    q2, k2 = torch.empty_like(d["q"]), torch.empty_like(d["k"])
    prol_bytes = 2 * 2 * w.n_valid * row_bytes
    ms_prol = timed(lambda: B.qk_rmsnorm_rope(d["q"], d["k"], d["w_q"], d["w_k"], n, w.eps,
                                              rope, q_out=q2, k_out=k2), args.steps)
    log(f"[bench] kv_pack {ms_pack:.3f} ms ({pack_bytes / ms_pack / 1e6:.0f} GB/s), "
        f"qk_rmsnorm_rope {ms_prol:.3f} ms ({prol_bytes / ms_prol / 1e6:.0f} GB/s)")

    # ---- large scores: Q/K weights x6 put every workgroup outside the fast pass's score
    # bound, so the checked pass (per-tile running max) does all the work
    large_scores = None
    if not args.no_large_scores:
        w_q6 = (d["w_q"].float() * 6.0).to(torch.bfloat16)
        w_k6 = (d["w_k"].float() * 6.0).to(torch.bfloat16)
        ms_big = timed(lambda: B.attn_layer(d["q"], d["k"], d["v"], w_q6, w_k6, n, w.eps, rope,
                                            scale, out=out, workspace=ws), args.steps)
        valid_blocks = (w.n_valid + 255) // 256
        big_checked = float(B.pass_flags(ws, d["q"], n)[..., :valid_blocks].float().mean())
        large_scores = {"weights": "w_q, w_k x 6", "ms_per_step": round(ms_big, 4),
                        "tflops": round(flops / ms_big / 1e9, 2),
                        "workgroups_in_checked_pass": round(big_checked, 4)}
        del w_q6, w_k6
        log(f"[bench] large scores (w x 6): h3_attn_layer {ms_big:.3f} ms "
            f"({flops / ms_big / 1e9:.1f} TFLOP/s), {100 * big_checked:.1f} % of workgroups "
            f"in the checked pass")

    # ---- the FP8 (SAGE) variant on the same workload
    ws8 = torch.empty(B.workspace_size(d["q"], fp8=True), dtype=torch.uint8, device=dev)
    out8 = torch.empty_like(d["q"])
    ms_layer8 = timed(lambda: B.attn_layer_fp8(d["q"], d["k"], d["v"], d["w_q"], d["w_k"], n,
                                               w.eps, rope, scale, out=out8, workspace=ws8),
                      args.steps)
    ms_pack8 = timed(lambda: B.kv_pack_fp8(d["k"], d["v"], n, workspace=ws8, w_k=d["w_k"],
                                           eps=w.eps, rope=rope), args.steps)
    ms_attn8 = timed(lambda: B.attn_packed_fp8(d["q"], ws8, n, scale, w_q=d["w_q"], eps=w.eps,
                                               rope=rope, out=out8), args.steps)
    pack8_bytes = 3 * w.n_valid * row_bytes + w.heads * tiles * 19456
    fp8 = {
        "entry": "h3_attn_layer_fp8",
        "dtype": "fp8 e4m3 products, fp32 accumulation, bf16 in/out",
        "ms_per_step": round(ms_layer8, 4),
        "tflops": round(flops / ms_layer8 / 1e9, 2),
        "speedup_over_bf16_step": round(ms_step / ms_layer8, 3),
        "attention_kernel": {"kernel": "attn_fp8_kernel", "ms": round(ms_attn8, 4),
                             "tflops": round(flops / ms_attn8 / 1e9, 2),
                             "frac_fp8_peak": round(flops / ms_attn8 / 1e9 / PEAK_FP8_TFLOPS, 4),
                             "peak": PEAK_FP8_TFLOPS,
                             "traffic": measured_traffic(FP8_TRAFFIC_FILE, FP8_KERNEL_SOURCES),
                             "source_hash": source_hash(FP8_KERNEL_SOURCES)},
        "pre_pass": {"kernels": "fill_zero_kernel + v_amax_kernel + kv_pack_fp8_kernel",
                     "ms": round(ms_pack8, 4), "bytes": pack8_bytes,
                     "GB/s": round(pack8_bytes / ms_pack8 / 1e6, 1)},
    }
    log(f"[bench] h3_attn_layer_fp8 {ms_layer8:.3f} ms/step ({fp8['tflops']} TFLOP/s), "
        f"attn_fp8_kernel {ms_attn8:.3f} ms ({fp8['attention_kernel']['tflops']} TFLOP/s, "
        f"{100 * fp8['attention_kernel']['frac_fp8_peak']:.1f}% of fp8 peak), pre-pass "
        f"{ms_pack8:.3f} ms")

    # ---- Skip-Softmax on the FP8 layer: these inputs, then frame-local ones
    wave_tiles = w.heads * ((w.n_valid + 31) // 32) * (tiles - 1)

    def skip_run(dd, lam):
        ms = timed(lambda: B.attn_layer_fp8(dd["q"], dd["k"], dd["v"], dd["w_q"], dd["w_k"], n,
                                            w.eps, rope, scale, out=out8, workspace=ws8,
                                            skip_threshold=lam), args.steps)
        skipped = int(B.fp8_skip_counts(ws8, dd["q"]).sum())
        return {"ms_per_step": round(ms, 4), "tflops_equiv": round(flops / ms / 1e9, 2),
                "wave_tiles_skipped": round(skipped / wave_tiles, 4)}

    skip = {"threshold": SKIP_LAMBDA, "rule": "per row, a 64-key tile after the first is "
            "dropped when exp(tile max - running max) < threshold",
            "this_workload": skip_run(d, SKIP_LAMBDA)}
    t0 = time.time()
    dl = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v)
          for k, v in W.generate_local(w, alpha=LOCAL_ALPHA).items()}
    log(f"[bench] frame-local inputs ready in {time.time() - t0:.1f}s")
    ms_bf16_local = timed(lambda: B.attn_layer(dl["q"], dl["k"], dl["v"], dl["w_q"], dl["w_k"], n,
                                               w.eps, rope, scale, out=out, workspace=ws),
                          args.steps)
    dense_local = skip_run(dl, 0.0)
    dense_out = out8[0, :w.n_valid].float()  # dense FP8 on the frame-local inputs

    def distance():
        """Relative L2 and max |difference| of the last FP8 output from dense FP8."""
        diff = out8[0, :w.n_valid].float() - dense_out
        return (round((diff.norm() / dense_out.norm()).item(), 5),
                round(diff.abs().max().item(), 5))

    # the threshold trades accuracy for speed: a sweep on the same inputs, each point with
    # its output's distance from dense FP8
    sweep = []
    skip_local = None
    for lam in SKIP_SWEEP:
        r = skip_run(dl, lam)
        if lam == SKIP_LAMBDA:
            skip_local = r
        rel, mx = distance()
        sweep.append({"threshold": lam, "ms_per_step": r["ms_per_step"],
                      "speedup_over_fp8_dense": round(dense_local["ms_per_step"] /
                                                      r["ms_per_step"], 3),
                      "wave_tiles_skipped": r["wave_tiles_skipped"],
                      "rel_l2_vs_fp8_dense": rel, "max_abs_vs_fp8_dense": mx})
    del dense_out
    assert skip_local is not None, "the sweep includes the reported threshold"
    skip["frame_local"] = {
        "inputs": f"workloads.generate_local(alpha={LOCAL_ALPHA}, frame=804): one direction "
                  "per 804-token block on the 16 lowest-frequency RoPE pairs",
        "bf16_dense_ms": round(ms_bf16_local, 4), "fp8_dense": dense_local,
        "fp8_skip": skip_local,
        "speedup_skip_over_fp8_dense": round(dense_local["ms_per_step"] /
                                             skip_local["ms_per_step"], 3),
        "speedup_skip_over_bf16_dense": round(ms_bf16_local / skip_local["ms_per_step"], 3),
        "threshold_sweep": sweep}
    fp8["skip_softmax"] = skip
    log(f"[bench] skip-softmax {SKIP_LAMBDA}: this workload {skip['this_workload']}; "
        f"frame-local bf16 {ms_bf16_local:.3f} ms, fp8 dense {dense_local['ms_per_step']} ms, "
        f"fp8 skip {skip_local['ms_per_step']} ms ({100 * skip_local['wave_tiles_skipped']:.1f} % "
        f"of wave tiles skipped)")

    # ---- the Skip-Softmax-only control: dense bf16 attention with Skip-Softmax, on these
    # inputs and on the frame-local ones, against dense bf16 on the same inputs
    def bf16_skip_run(dd, lam):
        ms = timed(lambda: B.attn_layer_skip(dd["q"], dd["k"], dd["v"], dd["w_q"], dd["w_k"], n,
                                             w.eps, rope, scale, lam, out=out, workspace=ws),
                   args.steps)
        skipped = int(B.skip_counts(ws, dd["q"]).sum())
        return {"ms_per_step": round(ms, 4), "tflops_equiv": round(flops / ms / 1e9, 2),
                "wave_tiles_skipped": round(skipped / wave_tiles, 4)}

    skip_only = {"threshold": SKIP_LAMBDA, "entry": "h3_attn_layer_skip",
                 "rule": skip["rule"] + " (dense bf16, exact running max of the kept tiles)",
                 "this_workload": bf16_skip_run(d, SKIP_LAMBDA),
                 "this_workload_bf16_dense_ms": round(ms_step, 4)}
    # dense bf16 on the frame-local inputs, the reference of the sweep's distances
    B.attn_layer(dl["q"], dl["k"], dl["v"], dl["w_q"], dl["w_k"], n, w.eps, rope, scale,
                 out=out, workspace=ws)
    dense16 = out[0, :w.n_valid].float()
    sweep16, sk_local = [], None
    for lam in SKIP_SWEEP:
        r = bf16_skip_run(dl, lam)
        if lam == SKIP_LAMBDA:
            sk_local = r
        diff = out[0, :w.n_valid].float() - dense16
        sweep16.append({"threshold": lam, "ms_per_step": r["ms_per_step"],
                        "speedup_over_bf16_dense": round(ms_bf16_local / r["ms_per_step"], 3),
                        "wave_tiles_skipped": r["wave_tiles_skipped"],
                        "rel_l2_vs_bf16_dense": round((diff.norm() / dense16.norm()).item(), 5),
                        "max_abs_vs_bf16_dense": round(diff.abs().max().item(), 5)})
        del diff
    del dense16
    skip_only["frame_local"] = {"bf16_dense_ms": round(ms_bf16_local, 4), "bf16_skip": sk_local,
                                "speedup_over_bf16_dense": round(ms_bf16_local /
                                                                 sk_local["ms_per_step"], 3),
                                "threshold_sweep": sweep16}
    log(f"[bench] skip-softmax-only (bf16) {SKIP_LAMBDA}: this workload "
        f"{skip_only['this_workload']}; frame-local {sk_local['ms_per_step']} ms "
        f"({100 * sk_local['wave_tiles_skipped']:.1f} % of wave tiles skipped) vs dense "
        f"{ms_bf16_local:.3f} ms")
    del ws8, out8, dl

    # ---- DiT block steps around attention: gated residual + LayerNorm + modulation on the
    # fp32 residual stream [N, 5,376] (after attention) and LayerNorm + modulation alone
    # (before it); HBM-bound
    blk_in = W.generate_block(w.seq_buf, w.n_valid, hidden=w.heads * w.head_dim, seed=11)
    bx = blk_in["x"].to(dev)
    ba = blk_in["a"].to(dev)
    bg, bsh, bsc = (blk_in[k].to(dev) for k in ("gate", "shift", "scale"))
    by = torch.empty(bx.shape, dtype=torch.bfloat16, device=dev)
    hid = w.heads * w.head_dim
    ms_blk = timed(lambda: B.residual_norm_modulate(bx, bsh, bsc, n, 1e-6, a=ba, gate=bg, y=by),
                   args.steps)
    ms_blk0 = timed(lambda: B.residual_norm_modulate(bx, bsh, bsc, n, 1e-6, y=by), args.steps)
    blk_bytes = w.n_valid * hid * (4 + 2 + 4 + 2) + (w.seq_buf - w.n_valid) * hid * 2
    blk0_bytes = w.n_valid * hid * (4 + 2) + (w.seq_buf - w.n_valid) * hid * 2
    log(f"[bench] residual_norm_modulate gated {ms_blk:.3f} ms ({blk_bytes / ms_blk / 1e6:.0f} "
        f"GB/s), norm+modulate {ms_blk0:.3f} ms ({blk0_bytes / ms_blk0 / 1e6:.0f} GB/s)")
    del bx, ba, bg, bsh, bsc, by, blk_in

    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": workload_config(w),
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "attn_fwd_kernel",
                     "kernel_ms": round(ms_attn, 4),
                     "timed": "h3_attn_packed: fast pass + checked pass, HIP events on "
                              "the launch stream"},
        "large_scores_checked_pass": large_scores,
        "kernels": {
            "kv_pack_kernel": {"ms": round(ms_pack, 4), "bytes": pack_bytes,
                               "GB/s": round(pack_bytes / ms_pack / 1e6, 1),
                               "frac_hbm": round(pack_bytes / ms_pack / 1e6 / PEAK_HBM_GBS, 4)},
            "qk_norm_rope_kernel": {"ms": round(ms_prol, 4), "bytes": prol_bytes,
                                    "GB/s": round(prol_bytes / ms_prol / 1e6, 1),
                                    "frac_hbm": round(prol_bytes / ms_prol / 1e6 /
                                                      PEAK_HBM_GBS, 4)},
            "residual_norm_modulate_kernel (gated residual, after attention)": {
                "ms": round(ms_blk, 4), "bytes": blk_bytes,
                "GB/s": round(blk_bytes / ms_blk / 1e6, 1),
                "frac_hbm": round(blk_bytes / ms_blk / 1e6 / PEAK_HBM_GBS, 4)},
            "residual_norm_modulate_kernel (norm + modulation, before attention)": {
                "ms": round(ms_blk0, 4), "bytes": blk0_bytes,
                "GB/s": round(blk0_bytes / ms_blk0 / 1e6, 1),
                "frac_hbm": round(blk0_bytes / ms_blk0 / 1e6 / PEAK_HBM_GBS, 4)},
        },
        "fp8": fp8,
        "skip_softmax_only": skip_only,
        "wall_s_timed_region": round(wall, 4),
        "sclk_mhz": sclk,
        "source_hash": source_hash(),
    }

    # ---- CPU baseline: the fp64 oracle's time on the sample checked before timing
    result["parity"] = {k: check[k] for k in ("rows_per_head", "max_abs", "mean_abs",
                                               "rel_l2", "ok")}
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        cpu_tflops = check["tflops_fp64"]
        result["cpu_baseline"] = {
            "value": cpu_tflops, "unit": "TFLOP/s", "cores": check["threads"],
            "kind": "oracle",
            "sample": f"{len(rows)} sampled query rows x {w.heads} heads of {w.name} "
                      f"(all {w.n_valid} keys each), fp64, {check['seconds']} s",
            "seconds": check["seconds"],
            "extrapolated_full_layer_s": check["extrapolated_full_layer_s"],
            "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "gpu_over_cpu": round(value / cpu_tflops, 1),
        }
    if not args.no_per_workload:
        del d, out, ws, q2, k2, layer_out
        torch.cuda.empty_cache()
        result["per_workload"] = per_workload(
            torch, B, W, dev, stream,
            None if args.no_cpu_baseline else args.oracle_rows_per_head,
            known=None if args.no_cpu_baseline else {args.workload: check})
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

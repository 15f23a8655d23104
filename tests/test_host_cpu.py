"""Host-side logic that needs no GPU: the binding fails loudly without the library, the
benchmark refuses more than one GPU, and committed counter summaries are used only for
the kernel sources they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_sequence_attention_h3_amd import binding as B  # noqa: E402


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "libh3attn.so"))
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_measured_traffic_needs_matching_sources(tmp_path):
    path = tmp_path / "traffic.json"
    good = {"source_hash": bench.source_hash(), "hbm_bytes_per_launch": 123}
    path.write_text(json.dumps(good))
    assert bench.measured_traffic(str(path)) == 123
    path.write_text(json.dumps(dict(good, source_hash="0" * 16)))
    assert bench.measured_traffic(str(path)) is None
    assert bench.measured_traffic(str(tmp_path / "absent.json")) is None
    path.write_text("not json")
    assert bench.measured_traffic(str(path)) is None


def test_source_hash_covers_every_kernel_source():
    assert bench.source_hash() == bench.source_hash()
    assert bench.source_hash() != bench.source_hash(bench.FP8_KERNEL_SOURCES)
    for rel in bench.FP8_KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, rel)), rel



def test_bench_oracle_check_gates_parity():
    """bench.oracle_check: the oracle's own rows pass the bar exactly, an all-zero output
    (which an N ~ 59k layer misses by only 2-3x on the absolute bounds) fails it."""
    import numpy as np
    from oracle import oracle as O
    from long_sequence_attention_h3_amd import workloads as W
    w = W.Workload("host_check_300of320", heads=2, n_valid=300, seq_buf=320, seed=9)
    inp = W.generate(w, tail="nan")
    rows = [0, 17, 299]
    scale = 1.0 / 128 ** 0.5
    ref = O.attn_layer(W.bits(inp["q"][0]), W.bits(inp["k"][0]), W.bits(inp["v"][0]), 300,
                       W.bits(inp["w_q"]), W.bits(inp["w_k"]), w.eps,
                       O.make_rope(w.theta, 300), scale, np.asarray(rows))
    good = bench.oracle_check(W, w, inp, ref, rows, scale)
    assert good["ok"] and good["max_abs"] == 0.0 and good["rows_per_head"] == 3
    assert not good["all_rows"] and good["extrapolated_full_layer_s"] >= good["seconds"]
    bad = bench.oracle_check(W, w, inp, np.zeros_like(ref), rows, scale)
    assert not bad["ok"]


def test_bench_refuses_to_report_a_value_when_parity_fails():
    """A failing parity check yields a JSON line with no `value` (and main returns 1
    before any timing); the check comes before the first timed event in main."""
    from long_sequence_attention_h3_amd import workloads as W
    w = W.WORKLOADS[3]
    bad = {"rows_per_head": 4096, "max_abs": 0.03, "mean_abs": 0.005, "rel_l2": 0.5,
           "ok": False}
    line = json.loads(bench.refusal(w, bad))
    assert "value" not in line and line["parity"]["ok"] is False
    assert line["config"]["workload"] == w.name and line["metric"] == bench.METRIC
    import inspect
    src = inspect.getsource(bench.main)
    check_at = src.index("check = oracle_check(")
    refuse_at = src.index("print(refusal(w, check)")
    headline = src.index("# ---- headline: K whole-layer steps")
    assert check_at < refuse_at < headline < src.index("e0.record(stream)", headline)
    assert "return 1" in src[refuse_at:refuse_at + 80]


def test_per_workload_skips_timing_of_a_failed_workload():
    import inspect
    src = inspect.getsource(bench.per_workload)
    assert src.index('if orc is not None and not orc["ok"]:') < src.index("call_times(")

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


"""Host-side logic of bench.py (no GPU): the one-GPU guard, the source hash that keys the committed HBM
byte counters, and the lookup of those counters."""
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_source_hash_ignores_comments_and_blank_lines(bench, tmp_path, monkeypatch):
    csrc = tmp_path / "attention_causal_gqa_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("int a = 1;  // first\n\nint b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash(["k.hip"])
    (csrc / "k.hip").write_text("// a new comment\nint a = 1;  // changed\nint b = 2;\n\n")
    assert bench.kernel_source_hash(["k.hip"]) == h0
    (csrc / "k.hip").write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash(["k.hip"]) != h0


def test_traffic_lookup_needs_workload_kernel_and_hash(bench, tmp_path, monkeypatch):
    f = tmp_path / "hbm_traffic.txt"
    f.write_text("# comment line\ntraffic 5 prefill_bf16_kernel 0123456789abcdef 215000000\n"
                 "traffic 5 decode_stream_kernel+decode_combine_kernel fedcba9876543210 1259840550\n")
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(f))
    assert bench.measured_traffic(5, "prefill_bf16_kernel", "0123456789abcdef") == 215000000
    assert bench.measured_traffic(5, "prefill_bf16_kernel", "fedcba9876543210") is None  # stale source
    assert bench.measured_traffic(3, "prefill_bf16_kernel", "0123456789abcdef") is None  # other workload
    assert bench.measured_traffic(5, "decode_stream_kernel+decode_combine_kernel", "fedcba9876543210") == 1259840550
    monkeypatch.setattr(bench, "PROFILE_COUNTERS", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic(5, "prefill_bf16_kernel", "0123456789abcdef") is None


def test_committed_traffic_lines_are_well_formed(bench):
    lines = [ln.split() for ln in open(bench.PROFILE_COUNTERS) if ln.startswith("traffic ")]
    assert lines, "no traffic lines in the committed counter summary"
    for parts in lines:
        assert len(parts) == 5
        assert int(parts[1]) in (3, 4, 5, 6, 7, 8, 9, 10, 11, 12)
        assert len(parts[3]) == 16 and int(parts[3], 16) >= 0
        assert int(parts[4]) > 0

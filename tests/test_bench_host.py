"""Host-side logic of bench.py (CPU only): the one-GPU guard, the rocprofv3
summaries, and the traffic record that is used only while the kernel sources
it was measured on are unchanged."""

import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _csrc_hash(name):
    path = os.path.join(ROOT, "fp8_block_scaled_quantize_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def test_traffic_record_follows_the_sources(tmp_path):
    rec = {"source_sha256_16": {"gemm.hip": _csrc_hash("gemm.hip"), "stream.hip": _csrc_hash("stream.hip")},
           "bytes_per_launch": {"k": 123}}
    p = tmp_path / "t.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), "k") == 123
    assert bench.measured_traffic(str(p), "other") is None
    rec["source_sha256_16"]["stream.hip"] = "0" * 16          # a source changed since the counters
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), "k") is None
    rec["source_sha256_16"] = {}                               # no source named: not trusted
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(p), "k") is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), "k") is None


def test_committed_traffic_records_name_their_sources():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.startswith("traffic_") and name.endswith(".json"):
            rec = json.load(open(os.path.join(ROOT, "profiles", name)))
            assert rec["source_sha256_16"], name
            assert rec["bytes_per_launch"], name


def test_summarize_trace_groups_by_kernel_and_grid(tmp_path, capsys):
    p = tmp_path / "trace.csv"
    p.write_text("Kernel_Name,Grid_Size,Start_Timestamp,End_Timestamp\n"
                 "void fp8bsq::a_kernel<1>(P),256,1000000,3000000\n"
                 "void fp8bsq::a_kernel<1>(P),256,5000000,9000000\n"
                 "void fp8bsq::a_kernel<1>(P),512,0,1000000\n")
    bench.summarize_trace(str(p))
    lines = [l for l in capsys.readouterr().out.splitlines() if "a_kernel" in l]
    assert len(lines) == 2
    first = lines[0].split()                                   # the largest total first
    assert first[-4:] == ["256", "2", "3.0000", "6.000"]
    assert lines[1].split()[-4:] == ["512", "1", "1.0000", "1.000"]


def test_summarize_counters_sums_per_dispatch(tmp_path, capsys):
    p = tmp_path / "pmc.csv"
    p.write_text("Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"
                 "1,fp8bsq::k<2>(P),64,FETCH_SIZE,10\n"
                 "1,fp8bsq::k<2>(P),64,FETCH_SIZE,5\n"      # two XCD rows of one dispatch
                 "2,fp8bsq::k<2>(P),64,FETCH_SIZE,25\n")
    bench.summarize_counters([str(p)])
    line = [l for l in capsys.readouterr().out.splitlines() if "FETCH_SIZE" in l][0]
    assert line.split()[-2:] == ["2", "20.0"]


@pytest.mark.parametrize("kind", ["quant_act", "quant_transpose", "quant_dual", "quant_weight",
                                  "quant_weight_nt", "quant_weight_stream"])
def test_every_quantizer_launch_has_a_stream_ceiling(kind):
    assert bench.STREAM_FOR[kind] in ("copy_nt", "read2_write1")


def test_launch_stats_mean_median_min():
    assert bench.launch_stats([3.0, 1.0, 2.0]) == {"ms": 2.0, "ms_median": 2.0, "ms_min": 1.0}
    assert bench.launch_stats([4.0, 1.0, 2.0, 3.0]) == {"ms": 2.5, "ms_median": 2.5, "ms_min": 1.0}
    assert bench.launch_stats([0.5]) == {"ms": 0.5, "ms_median": 0.5, "ms_min": 0.5}


def test_default_warmup_is_at_least_five(monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    args = bench.parse()
    assert args.warmup >= 5 and args.steps >= 20 and args.gpus == 1

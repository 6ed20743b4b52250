"""Host-side logic of bench.py, on the CPU: the one-GPU rule, the calibration of the
HBM-traffic summary on the weight-packing copy, and the source-hash check that keeps
counters taken on another kernel source out of the bench line."""

import json
import os
import subprocess
import sys

import pytest

import bench
from w8a8_quantized_decode_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PACK = "a8w8::(anonymous namespace)::pack_tiled_kernel(signed char const*, long, long, signed char*)"
GATEUP = "void a8w8::(anonymous namespace)::decode_kernel<2, 2, 1>(a8w8::StreamKArgs, a8w8::DecodeGeom)"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n")
        for name, grid, kib in rows:
            f.write(f'"{name}",{grid},{counter},{kib}\n')


def test_pmc_summary_calibrates_on_the_pack_copy(tmp_path, monkeypatch):
    cfg = synth.CONFIGS[2]
    nbytes = cfg.I * cfg.H            # one Gate weight: the pack reads and writes it once
    # FETCH_SIZE reports the copy at half its size, WRITE_SIZE at its size: factors 2 and 1
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(PACK, nbytes // 16, nbytes / 1024 / 2), (GATEUP, 1, 1000.0), (GATEUP, 1, 1002.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(PACK, nbytes // 16, nbytes / 1024), (GATEUP, 1, 10.0), (GATEUP, 1, 10.0)])
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "pmc.json"))
    monkeypatch.setattr(bench, "PMC_MD", str(tmp_path / "pmc.md"))
    bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), ["fetch", "write"], cfg)
    s = json.load(open(tmp_path / "pmc.json"))
    assert s["fetch_factor"] == pytest.approx(2.0)
    assert s["write_factor"] == pytest.approx(1.0)
    assert s["hbm_bytes_per_dispatch"] == round(1001.0 * 1024 * 2 + 10.0 * 1024)
    assert s["kernel_source_hash"] == bench.kernel_source_hash()
    # the bench line takes the traffic only while the kernel source is the one measured
    assert bench.measured_traffic(cfg) == s["hbm_bytes_per_dispatch"]
    s["kernel_source_hash"] = "0" * 16
    with open(tmp_path / "pmc.json", "w") as f:
        json.dump(s, f)
    assert bench.measured_traffic(cfg) is None


def test_kernel_hash_ignores_comments_but_not_code():
    a = "int x = 1;  // the count\n/* a block\n comment */ x += 2;\n"
    assert bench.code_text(a) == bench.code_text("int x = 1;\n\n    x += 2;")
    assert bench.code_text(a) != bench.code_text("int x = 1; x += 3;")
    files = {}
    for f in ("gemm_decode.hip", "gemm_streamk.hip", "device_common.h", "internal.h"):
        with open(os.path.join(bench.ROOT, "w8a8_quantized_decode_amd", "csrc", f)) as fh:
            files[f] = fh.read()
    h = bench.kernel_source_hash()
    assert bench.kernel_source_hash(lambda f: files[f] + "\n// a new remark\n") == h
    assert bench.kernel_source_hash(lambda f: files[f] + "\nint extra_symbol;\n") != h


def test_pmc_summary_rejects_a_copy_of_unknown_size(tmp_path, monkeypatch):
    cfg = synth.CONFIGS[2]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(PACK, 12345, 1.0), (GATEUP, 1, 1.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(PACK, 12345, 1.0), (GATEUP, 1, 1.0)])
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "pmc.json"))
    monkeypatch.setattr(bench, "PMC_MD", str(tmp_path / "pmc.md"))
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), ["f", "w"], cfg)
    assert not os.path.exists(tmp_path / "pmc.json")


def test_a_roofline_fraction_above_one_fails_the_run(capsys):
    """A fraction above 1 means the timed interval missed the kernel's work."""
    bench.emit({"metric": "m", "roofline": {"frac": 0.64}})
    with pytest.raises(SystemExit) as e:
        bench.emit({"metric": "m", "roofline": {"frac": 4.3}})
    assert e.value.code == 3
    assert capsys.readouterr().out.count('"metric"') == 2   # the line is still printed


def test_percentile_stats():
    s = bench.pct_stats(list(range(1, 101)))
    assert s["median"] == 50.5 and s["p10"] == 10.9 and s["p90"] == 90.1 and s["mean"] == 50.5

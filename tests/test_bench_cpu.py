"""Host logic of bench.py that runs without a GPU: the one-GPU contract, the source digest that
ties committed counter summaries to the kernels they were taken on, and the digest of rocprofv3
FETCH_SIZE / WRITE_SIZE files into per-launch HBM bytes (scaled by the copy calibration)."""

import csv
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
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_source_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    csrc = tmp_path / "block_scaled_fp4_plan_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "device.h").write_text("int a;  // note\n/* block\ncomment */ int b;\n")
    (csrc / "gemm.hip").write_text("int c;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    (csrc / "device.h").write_text("int a;\n\n  int    b;   // other note\n")
    assert bench.kernel_source_digest() == d0          # same code, other comments / spacing
    (csrc / "gemm.hip").write_text("int c2;\n")
    assert bench.kernel_source_digest() != d0          # a code change shows


def _write_counters(d, rows):
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, c, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_digest_counters_scales_by_the_copy_calibration(tmp_path):
    g1 = "void bfp4::(anonymous namespace)::moe_gemv_kernel<2, 1, 0, 2, 4>(bfp4::GemmArgs)"
    g2 = "void bfp4::(anonymous namespace)::moe_gemv_kernel<2, 1, 2, 2, 4>(bfp4::GemmArgs)"
    other = "void bfp4::(anonymous namespace)::moe_gemv16_kernel<2, 0, 2, true>(bfp4::GemmArgs)"
    # decode run: two dispatches of each GEMM (means 1500 and 300 KiB fetched), one unrelated
    _write_counters(tmp_path / "df", [(g1, "FETCH_SIZE", 1000), (g1, "FETCH_SIZE", 2000),
                                      (g2, "FETCH_SIZE", 300), (other, "FETCH_SIZE", 9e9)])
    _write_counters(tmp_path / "dw", [(g1, "WRITE_SIZE", 10), (g2, "WRITE_SIZE", 20),
                                      (g2, "WRITE_SIZE", 40)])
    # copy calibration: a 1 GiB copy reading as half its bytes fetched and all of them written
    _write_counters(tmp_path / "cf", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0)])
    _write_counters(tmp_path / "cw", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0)])
    out = tmp_path / "traffic.json"
    res = bench.digest_counters(["decode:%s:%s" % (tmp_path / "df", tmp_path / "dw"),
                                 "copy:%s:%s" % (tmp_path / "cf", tmp_path / "cw")],
                                out_path=str(out))
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    e1 = res["decode/gemm1_swiglu_decode"]
    assert e1["fetch_bytes"] == int(1500 * 1024 * 2.0) and e1["write_bytes"] == 10 * 1024
    assert e1["bytes_per_launch"] == e1["fetch_bytes"] + e1["write_bytes"]
    assert e1["dispatches"] == 2
    e2 = res["decode/gemm2_down_decode"]
    assert e2["fetch_bytes"] == int(300 * 1024 * 2.0) and e2["write_bytes"] == 30 * 1024
    on_disk = json.loads(out.read_text())
    assert on_disk["decode/gemm1_swiglu_decode"] == e1
    # the summary is reported only while the sources match the digest it was taken on
    assert bench.traffic_for("gemm1_swiglu_decode", "decode", path=str(out)) == \
        e1["bytes_per_launch"]
    on_disk["decode/gemm1_swiglu_decode"]["source_digest"] = "0" * 16
    out.write_text(json.dumps(on_disk))
    assert bench.traffic_for("gemm1_swiglu_decode", "decode", path=str(out)) is None


def test_digest_counters_needs_the_calibration(tmp_path):
    _write_counters(tmp_path / "df", [])
    _write_counters(tmp_path / "dw", [])
    with pytest.raises(SystemExit):
        bench.digest_counters(["decode:%s:%s" % (tmp_path / "df", tmp_path / "dw")],
                              out_path=str(tmp_path / "t.json"))


"""Host-side logic of bench.py, on the CPU: the one-GPU guard, workload
names, the roofline object's arithmetic and the traffic counters' scaling
(synthetic counter files; nothing is launched)."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,expect", [
    ("i8-8192", ("i8", 8192, 8192, 8192)),
    ("f16-512", ("f16", 512, 512, 512)),
    ("i4-2048", ("i4", 2048, 2048, 2048)),
    ("llm-16", ("dq", 16, 14336, 4096)),
    ("w8a8-128", ("w8", 128, 14336, 4096)),
    ("w8a8f-16", ("w8f", 16, 14336, 4096)),
    ("i8-1024x1024x8192", ("i8", 1024, 1024, 8192)),
    ("i8sk-512x2048x32768", ("i8", 512, 2048, 32768)),
    ("f16sk-300x520x8208", ("f16", 300, 520, 8208)),
    ("dqsk-256x4096x8192", ("dq", 256, 4096, 8192)),
    ("i4sk-4096", ("i4", 4096, 4096, 4096)),
])
def test_parse_workload(name, expect):
    assert bench.parse_workload(name) == expect


def test_split_kind():
    assert bench.split_kind("i8sk-512x2048x32768") == ("i8", True)
    assert bench.split_kind("i4sk-4096") == ("i4", True)
    assert bench.split_kind("i8-8192") == ("i8", False)
    assert bench.split_kind("llm-128") == ("llm", False)


@pytest.mark.parametrize("name", ["bf16-8192", "i8-1x2", "llm-1x2x3", "i8sk-1x2x", "i8-8192-1", "i8-x"])
def test_unknown_workload_is_rejected(name):
    with pytest.raises(SystemExit):
        bench.parse_workload(name)


def _workload(name, kind, M, N, K, in_bytes, out_bytes):
    return SimpleNamespace(name=name, kind=kind, M=M, N=N, K=K, in_bytes=in_bytes,
                           out_bytes=out_bytes, ops=2 * M * N * K)


def test_roofline_mfma_bound_int8_8192(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "none.json"))
    n = 8192
    w = _workload("i8-8192", "i8", n, n, n, 2 * n * n, 4 * n * n)
    r = bench.roofline(w, {"kernel_ms_avg": 0.5})
    # 2 n^3 ops in 0.5 ms against 5033.2 TOP/s
    achieved = 2 * n ** 3 / 0.5e-3 / 1e12
    assert r["bound"] == "mfma" and r["unit"] == "TOP/s"
    assert r["achieved"] == pytest.approx(achieved, abs=0.05)
    assert r["frac"] == pytest.approx(achieved / 5033.2, abs=1e-4)
    assert r["traffic"] is None
    assert r["algorithmic_bytes"] == 6 * n * n


def test_roofline_hbm_bound_llm_16(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "none.json"))
    M, N, K = 16, 14336, 4096
    w = _workload("llm-16", "dq", M, N, K, M * K + N * K + 4 * (M + N), 4 * M * N)
    r = bench.roofline(w, {"kernel_ms_avg": 0.014})
    gbs = (w.in_bytes + w.out_bytes) / 0.014e-3 / 1e9
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(gbs, abs=0.05)
    assert r["frac"] == pytest.approx(gbs / 8000.0, abs=1e-4)


def test_roofline_fp16_uses_its_own_peak(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "none.json"))
    n = 8192
    w = _workload("f16-8192", "f16", n, n, n, 4 * n * n, 4 * n * n)
    r = bench.roofline(w, {"kernel_ms_avg": 0.9})
    assert r["peak"] == 2516.6 and r["unit"] == "TFLOP/s"


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for k, c, v in rows:
            wr.writerow({"Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_write_traffic_scales_by_the_copy_and_checks_the_hash(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cfetch, cwrite = tmp_path / "cf.csv", tmp_path / "cw.csv"
    rows_f, rows_w = [], []
    for i, k in enumerate(bench.TRAFFIC_KERNELS.values()):
        for v in (100.0 * (i + 1), 101.0 * (i + 1), 102.0 * (i + 1)):   # median: 101 (i + 1)
            rows_f.append((k, "FETCH_SIZE", v))
            rows_w.append((k, "WRITE_SIZE", 2 * v))
    _counter_csv(fetch, rows_f)
    _counter_csv(write, rows_w)
    # a 256 MiB copy whose counters read half (fetch) and all (write) of it
    _counter_csv(cfetch, [(copy, "FETCH_SIZE", 131072.0)] * 3)
    _counter_csv(cwrite, [(copy, "WRITE_SIZE", 262144.0)] * 3)
    rec = bench.write_traffic(str(fetch), str(write), str(cfetch), str(cwrite), 256)
    assert json.loads(out.read_text()) == rec
    first = rec["i8-8192"]
    assert first["fetch_scale"] == 2.0 and first["write_scale"] == 1.0
    assert first["fetch_bytes"] == int(101.0 * 1024 * 2.0)
    assert first["write_bytes"] == int(202.0 * 1024 * 1.0)
    assert first["kernel_source_hash"] == bench.kernel_source_hash()
    # the roofline reports the traffic while the sources still hash the same
    n = 8192
    w = _workload("i8-8192", "i8", n, n, n, 2 * n * n, 4 * n * n)
    assert bench.roofline(w, {"kernel_ms_avg": 0.5})["traffic"] == first["fetch_bytes"] + first["write_bytes"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.roofline(w, {"kernel_ms_avg": 0.5})["traffic"] is None


def test_default_cache_state():
    # the LLM and W8A8 weights stream cold (rotating copies); the rest warm
    assert bench.default_cache("llm-16") == "cold"
    assert bench.default_cache("w8a8-128") == "cold"
    assert bench.default_cache("w8a8f-16") == "cold"
    for name in ("i8-512", "f16-8192", "i4-2048", "i8sk-300x520x8208", "dq-256x4096x8192"):
        assert bench.default_cache(name) == "warm", name
    # enough copies to exceed the 256 MB Infinity Cache
    assert bench.COLD_ROTATION_BYTES > 256 * 10 ** 6

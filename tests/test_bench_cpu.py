"""Host logic of bench.py, without a GPU: kernel names from profiler output,
the refusal of more than one GPU, and the HBM traffic computed from counter
summaries with the copy-kernel calibration."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,key", [
    ("_ZN4attn15attn_fwd_kernelIDF16bfLi64ELi4ELi64ELi1ELb0EEEvPKT_", "fwd"),
    ("void attn::attn_bwd_dkdv_kernel<__bf16, float, 64, 64, 1, false, 1>(__bf16 const*)", "dkdv"),
    ("void attn::attn_bwd_dkdv_pair_kernel<__bf16, float, 128, 1, false>(__bf16 const*)", "dkdv"),
    ("void attn::attn_bwd_dq_kernel<__bf16, float, 64, 32, 1, false, true>(__bf16 const*)", "dq_delta"),
    ("void attn::attn_bwd_dq_kernel<__bf16, float, 64, 32, 1, false, false>(__bf16 const*)", "dq"),
    ("_ZN4attn18attn_bwd_dq_kernelIDF16bfLi64ELi32ELi1ELb0ELb1EEEvPKT_", "dq_delta"),
    ("void attn::attn_bwd_preprocess_kernel<__bf16, float, 64>(float const*)", "pre"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", "copy"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>", None),
])
def test_kernel_key(name, key):
    assert bench.kernel_key(name) == key


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counters(directory, counter, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, name, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_counters_with_calibration(tmp_path, monkeypatch):
    """The calibration copy reads and writes 256 MiB; its counters read half of
    that on FETCH_SIZE and all of it on WRITE_SIZE, so a kernel's counts are
    divided by 0.5 and 1.0.  Per-dispatch values are the sum over the
    counter's instances (several rows per dispatch), averaged over dispatches."""
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    dkdv = "void attn::attn_bwd_dkdv_kernel<__bf16, float, 64, 64, 1, false, 1>(x)"
    _counters(tmp_path / "f", "FETCH_SIZE", [(1, neg, 65536.0), (1, neg, 65536.0),
                                              (2, dkdv, 40000.0), (2, dkdv, 2000.0), (3, dkdv, 42000.0)])
    _counters(tmp_path / "w", "WRITE_SIZE", [(1, neg, 262144.0), (2, dkdv, 66000.0), (3, dkdv, 66000.0)])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "sources_digest", lambda: "test")
    rec = bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "lm237m_ctx1024", 256)
    assert rec["calibration"]["fetch_factor"] == pytest.approx(0.5)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    k = rec["kernels"]["lm237m_ctx1024"]["dkdv"]
    assert k["raw_fetch_kib"] == pytest.approx(42000.0)
    assert k["fetch_bytes"] == pytest.approx(42000.0 * 1024 / 0.5)
    assert k["write_bytes"] == pytest.approx(66000.0 * 1024)
    assert k["bytes_per_launch"] == pytest.approx(k["fetch_bytes"] + k["write_bytes"])
    with open(tmp_path / "profiles" / "traffic.json") as f:
        assert json.load(f)["sources_digest"] == "test"


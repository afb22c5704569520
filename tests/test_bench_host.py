"""Host-side logic of bench.py, on the CPU: the roofline arithmetic, the
algorithmic work counts against the block's published sizes, the rocprofv3
counter summaries (fed synthetic counter files) and the one-GPU guard."""

import csv
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_picks_the_binding_resource():
    # 8 GB and 1 GFLOP in 2 ms: HBM-bound, 4 TB/s = half of the 8 TB/s peak
    r = bench.roofline(8e9, 1e9, 2e-3, "bf16")
    assert (r["bound"], r["unit"], r["achieved"], r["frac"]) == ("hbm", "GB/s", 4000.0, 0.5)
    # 1 GB and 2.5 TFLOP in 2 ms: matrix-core-bound, 1250 of 2500 TFLOP/s
    r = bench.roofline(1e9, 2.5e12, 2e-3, "bf16", traffic=123)
    assert (r["bound"], r["unit"], r["achieved"], r["frac"]) == ("mfma", "TFLOP/s", 1250.0, 0.5)
    assert r["traffic"] == 123
    # fp8 takes its own peak
    assert bench.roofline(1e9, 5e12, 2e-3, "fp8")["frac"] == 0.5


def test_work_counts_match_the_block_sizes():
    cfg = workloads.workload("decode")
    H, I = cfg["hidden"], cfg["intermediate"]
    # about 39M parameters per expert (three 2560 x 5120 matrices)
    assert 3 * H * I == 39_321_600
    # every expert active: about 20 GB of bf16 expert weights, plus x, out and W_r
    lb, lf = bench.layer_work(cfg, 256)
    weights = 256 * 3 * H * I * 2
    assert weights == 20_132_659_200
    assert lb == weights + 2 * cfg["T"] * H * 2 + 256 * H * 4
    # the gate/up launch reads two of the three matrices of each active expert
    gb, gf = bench.gateup_work(cfg, 222)
    assert gb - 222 * 2 * H * I * 2 == cfg["T"] * H * 2 + cfg["T"] * 8 * I * 2
    # flops: 2 per multiply-add, 8 experts per token, gate and up of I x H each
    assert gf == 2 * cfg["T"] * 8 * 2 * I * H
    assert lf == 1.5 * gf  # the down projection adds half again
    # fp8: one byte per weight, e4m3 x in, fp32 h out
    f8 = workloads.workload("fp8")
    b8, _ = bench.gateup_work(f8, 256)
    assert b8 == 256 * 2 * H * I + f8["T"] * H + f8["T"] * 8 * I * 4


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    keys = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=keys)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(keys, r)))


GATEUP = "void beam::gemm_dma_kernel<0, 256>(beam::GemmArgs)"
DOWN = "void beam::gemm_dma_kernel<1, 256>(beam::GemmArgs)"
COPY = "__amd_rocclr_copyBuffer"


@pytest.fixture
def sandbox(tmp_path, monkeypatch):
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda paths=None: "0123456789abcdef")
    return tmp_path


def test_traffic_summary_scales_by_the_copy(sandbox, monkeypatch):
    # the copy reads 524288 KiB of FETCH_SIZE for 1 GiB (factor 2) and writes
    # 1048576 KiB (factor 1); two gate/up dispatches average 3000 and 1000 KiB
    _write_counters(sandbox / "f", [(1, COPY, "FETCH_SIZE", 524288, 0, 1),
                                    (2, GATEUP, "FETCH_SIZE", 2900, 0, 1),
                                    (3, GATEUP, "FETCH_SIZE", 3100, 0, 1),
                                    (4, DOWN, "FETCH_SIZE", 99999, 0, 1)])
    _write_counters(sandbox / "w", [(1, COPY, "WRITE_SIZE", 1048576, 0, 1),
                                    (2, GATEUP, "WRITE_SIZE", 1000, 0, 1),
                                    (3, GATEUP, "WRITE_SIZE", 1000, 0, 1)])
    bench.write_traffic(str(sandbox / "f"), str(sandbox / "w"), "decode")
    assert bench.stored_figure("decode") == (3000 * 2 + 1000) * 1024
    # counters taken on other kernel sources are not used
    monkeypatch.setattr(bench, "kernel_source_sha", lambda paths=None: "fedcba9876543210")
    assert bench.stored_figure("decode") is None


def test_mfma_summary(sandbox):
    # 1 ms dispatches; GRBM_GUI_ACTIVE 2e6 cycles on each of the 8 XCDs: 2 GHz;
    # half of the 1024 SIMDs' cycles with the matrix core busy
    cyc = 2e6
    rows = []
    for d, (kern, busy) in enumerate([(GATEUP, 0.5), (GATEUP, 0.5), (DOWN, 0.25)]):
        t0 = 10_000_000 * d
        for name, v in (("GRBM_GUI_ACTIVE", 8 * cyc), ("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * cyc * busy),
                        ("SQ_INSTS_MFMA", 1000), ("SQ_BUSY_CU_CYCLES", 256 * cyc * 0.9)):
            rows.append((d, kern, name, v, t0, t0 + 1_000_000))
    _write_counters(sandbox / "m", rows)
    bench.write_mfma(str(sandbox / "m"), "skewed")
    assert bench.stored_figure("skewed", "mfma", key="gateup_mfma_busy") == pytest.approx(0.5)
    assert bench.stored_figure("skewed", "mfma", key="gateup_clock_ghz") == pytest.approx(2.0)
    assert bench.stored_figure("skewed", "mfma", key="down_mfma_busy") == pytest.approx(0.25)
    assert bench.stored_figure("skewed", "mfma", key="gateup_cu_busy") == pytest.approx(0.9)
    assert bench.stored_figure("skewed", "mfma", key="gateup_mfma_insts") == 1000


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

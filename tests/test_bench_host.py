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
    # and the x rows; the h rows it writes are design overhead, not counted
    gb, gf = bench.gateup_work(cfg, 222)
    assert gb - 222 * 2 * H * I * 2 == cfg["T"] * H * 2
    # flops: 2 per multiply-add, 8 experts per token, gate and up of I x H each
    assert gf == 2 * cfg["T"] * 8 * 2 * I * H
    assert lf == 1.5 * gf  # the down projection adds half again
    db, df = bench.down_work(cfg, 222)
    assert db == 222 * H * I * 2 and df == gf / 2
    # gate/up + down weights are the layer's weights
    assert gb + db - cfg["T"] * H * 2 == 222 * 3 * H * I * 2
    # fp8: one byte per weight, e4m3 x codes in
    f8 = workloads.workload("fp8")
    b8, _ = bench.gateup_work(f8, 256)
    assert b8 == 256 * 2 * H * I + f8["T"] * H


def test_design_overhead_counts_the_round_trips():
    # prefill: h (bf16) and y (bf16) each written once and read once
    p = workloads.workload("prefill")
    P, H, I = p["T"] * 8, p["hidden"], p["intermediate"]
    o = bench.design_overhead(p)
    assert o["h_round_trip"] == 2 * P * I * 2 and o["y_round_trip"] == 2 * P * H * 2
    assert o["total"] == o["h_round_trip"] + o["y_round_trip"]
    # the skewed workload's overhead is about 4 GB, the prefill one's about 1 GB
    assert 0.9e9 < o["total"] < 1.1e9
    assert 3.9e9 < bench.design_overhead(workloads.workload("skewed"))["total"] < 4.3e9
    # quantised weights add the E4M3 codes of x and h
    f = bench.design_overhead(workloads.workload("fp8"))
    assert f["x_codes"] == 2 * 8192 * H and f["h_codes"] == 2 * 8192 * 8 * I
    assert f["h_round_trip"] == 2 * 8192 * 8 * I * 2  # h is stored as bf16 there too


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
                                    (4, DOWN, "FETCH_SIZE", 500, 0, 1)])
    _write_counters(sandbox / "w", [(1, COPY, "WRITE_SIZE", 1048576, 0, 1),
                                    (2, GATEUP, "WRITE_SIZE", 1000, 0, 1),
                                    (3, GATEUP, "WRITE_SIZE", 1000, 0, 1),
                                    (4, DOWN, "WRITE_SIZE", 300, 0, 1)])
    bench.write_traffic(str(sandbox / "f"), str(sandbox / "w"), "decode")
    assert bench.stored_figure("decode") == (3000 * 2 + 1000) * 1024
    assert bench.stored_figure("decode", key="down_hbm_bytes_per_launch") == (500 * 2 + 300) * 1024
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


def test_counter_summaries_match_the_mixed_fp8_kernel(sandbox):
    """The fp8 GEMMs at 256-row tiles are gemm_dma8_mixed_kernel<0> / <1>
    (no second template argument): the parsers must still tell gate/up from
    down."""
    gu = "void beam::gemm_dma8_mixed_kernel<0>(beam::GemmArgs)"
    dn = "void beam::gemm_dma8_mixed_kernel<1>(beam::GemmArgs)"
    _write_counters(sandbox / "f", [(1, COPY, "FETCH_SIZE", 524288, 0, 1),
                                    (2, gu, "FETCH_SIZE", 1000, 0, 1),
                                    (3, dn, "FETCH_SIZE", 400, 0, 1)])
    _write_counters(sandbox / "w", [(1, COPY, "WRITE_SIZE", 1048576, 0, 1),
                                    (2, gu, "WRITE_SIZE", 100, 0, 1),
                                    (3, dn, "WRITE_SIZE", 50, 0, 1)])
    bench.write_traffic(str(sandbox / "f"), str(sandbox / "w"), "fp8")
    assert bench.stored_figure("fp8") == (1000 * 2 + 100) * 1024
    assert bench.stored_figure("fp8", key="down_hbm_bytes_per_launch") == (400 * 2 + 50) * 1024
    assert bench.gateup_kernel(workloads.workload("fp8")) == "gemm_dma8_mixed_kernel<0>"


def test_gateup_kernel_follows_the_launcher_rules():
    """The kernel named for the roofline is the one the library picks: bf16
    weights stream up to 16 rows per expert on average, MXFP4 up to 12 (32-row
    tiles above 8), packed fp8 never."""
    import bench
    import workloads
    d = workloads.workload("decode")
    assert bench.gateup_kernel(d).startswith("gemm_stream_kernel<0, unsigned short, false, true")
    assert bench.gateup_kernel(dict(d, T=600)) == "gemm_dma_kernel<0, 128>"
    assert bench.gateup_kernel(workloads.workload("prefill")) == "gemm_dma_kernel<0, 256>"
    m = workloads.workload("mxfp4")
    assert bench.gateup_kernel(m) == "gemm_stream4_kernel<0, 8, 4, 1>"
    assert bench.gateup_kernel(dict(m, T=350)) == "gemm_stream4_kernel<0, 4, 2, 2>"
    assert bench.gateup_kernel(dict(m, T=400)) == "gemm_dma4_kernel<0, 128>"
    f = workloads.workload("fp8")
    assert bench.gateup_kernel(dict(f, T=64)) == "gemm_dma8_kernel<0, 128>"


def test_shard_traffic_takes_the_32_row_stream_launches(sandbox):
    """In the decode run that carries the expert-shard line, the shard's
    launches are the 32-row streaming kernels and the decode ones the 16-row
    kernels: the ep_shard summary must take only the former."""
    dec_g = "void beam::gemm_stream_kernel<0, unsigned short, false, true, 8, 2, 1>(beam::GemmArgs)"
    dec_d = "void beam::gemm_stream_kernel<1, unsigned short, false, true, 8, 2, 1>(beam::GemmArgs)"
    sh_g = "void beam::gemm_stream_kernel<0, unsigned short, false, true, 2, 2, 2>(beam::GemmArgs)"
    sh_d = "void beam::gemm_stream_kernel<1, unsigned short, false, true, 2, 2, 2>(beam::GemmArgs)"
    for d, c in (("f", "FETCH_SIZE"), ("w", "WRITE_SIZE")):
        _write_counters(sandbox / d, [(1, COPY, c, 524288 if c == "FETCH_SIZE" else 1048576, 0, 1),
                                      (2, dec_g, c, 9000, 0, 1), (3, dec_d, c, 8000, 0, 1),
                                      (4, sh_g, c, 700, 0, 1), (5, sh_d, c, 300, 0, 1),
                                      (6, sh_g, c, 900, 0, 1)])
    bench.write_traffic(str(sandbox / "f"), str(sandbox / "w"), "ep_shard")
    assert bench.stored_figure("ep_shard") == (800 * 2 + 800) * 1024
    assert bench.stored_figure("ep_shard", key="down_hbm_bytes_per_launch") == (300 * 2 + 300) * 1024
    text = open(os.path.join(bench.ROOT, "profiles", "gateup_ep_shard_counters.txt")).read()
    assert "--workload decode" in text and "--no-shard" not in text


def test_every_global_name_main_uses_exists():
    """bench.main() only runs on a GPU machine; a name it calls that the module no
    longer defines would only show there. Every global it (and the functions
    it calls) loads must resolve in the module or the builtins."""
    import builtins
    import dis
    import types

    seen, todo, missing = set(), [bench.main], []
    while todo:
        fn = todo.pop()
        if fn in seen:
            continue
        seen.add(fn)
        codes = [fn.__code__]
        while codes:
            code = codes.pop()
            codes += [c for c in code.co_consts if isinstance(c, types.CodeType)]
            for ins in dis.get_instructions(code):
                if ins.opname != "LOAD_GLOBAL":
                    continue
                name = ins.argval
                obj = getattr(bench, name, getattr(builtins, name, None))
                if obj is None and not hasattr(bench, name):
                    missing.append((fn.__name__, name))
                elif isinstance(obj, types.FunctionType) and obj.__module__ == bench.__name__:
                    todo.append(obj)
    assert not missing, missing

#!/usr/bin/env python3
"""Benchmark of the Beam sparse-MoE block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

One step is one beam_moe_forward call over one batch of synthetic tokens,
with the expert weights in the packed (MFMA fragment) layout made once at
load time by beam_moe_pack_weights:
router logits, group-limited selection, permutation, both grouped expert
GEMMs and the combine. Inputs and the 20 GB of expert weights are resident
in HBM before the timed region. The default workload is Beam's decode shape
(T = 64 tokens, hidden 5120, 256 experts x SwiGLU 2560, bf16 weights); the
same line carries the prefill shape (T = 4096, balanced routing) under
"prefill", the skewed routing (T = 16384, +0.5 bias on 8 experts) under
"skewed" and the fp8 experts (T = 8192) under "fp8", each measured the
same way.

Timing: W untimed warm-up steps, then K steps back to back between two
synchronisations, each bracketed by a pair of HIP events on the stream the
library launches on. ms_per_step is the median of the K per-step times
(ms_per_step_mean: the K steps' total over K). Kernel launch times come
from separate passes in which the library records events around its
launches, so the timed steps carry no per-kernel events.

Printed fields beyond the usual ones:
* roofline: the dominant kernel (the gate/up grouped GEMM); achieved =
  algorithmic bytes (or flops) per launch / average launch time. Bytes are
  the method's own: the gate and up weights of the active experts and the
  token rows the launch reads (x, or its E4M3 codes with quantised
  weights); flops = 4 * (T * top_k) * hidden * intermediate. The bound is
  whichever of HBM (8 TB/s) and dense MFMA (bf16 2.5 PFLOP/s, fp8 5.0
  PFLOP/s) takes longer for those figures. traffic: HBM bytes per launch
  from the committed rocprofv3 counter summary for this kernel and
  workload, scaled by the copy-kernel calibration stored with it; null when
  the summary is missing or was taken from other kernel sources.
  down_roofline: the same for the down GEMM (its weights of the active
  experts).
* layer: the whole step against the block's algorithmic bytes (weights of
  the active experts, x, out, the router weights) and flops;
  design_overhead_bytes lists what the implementation moves beyond them
  (the h and y round trips between the kernels, the E4M3 codes of x and h).
* cpu_baseline: the oracle (numpy float64) on a bounded sample of the same
  workload, on this machine's host cores, median of 3 runs.

Other modes: --workload tiny|decode|prefill|skewed|fp8 picks the timed
workload; --calibrate-copy runs one plain device copy of 1 GiB before the
timed region (for counter calibration); --summarize DIR prints a summary of
a rocprofv3 output directory (kernel stats or counter collection);
--traffic FETCH_DIR WRITE_DIR --workload W writes the counter summary that
the traffic field reads (W = ep_shard: the expert-shard line's launches in
a decode run).
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at Beam shape (T=64 decode, T=4096 prefill) + % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
# bytes per weight: MXFP4 is half a byte plus one scale byte per 32 weights
WEIGHT_BYTES = {"bf16": 2, "fp8": 1, "mxfp4": 0.5 + 1 / 32}
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}
KERNEL_SOURCES = ["group_limited_routing_amd/csrc/expert_gemm.hip",
                  "group_limited_routing_amd/csrc/common.h"]
WGRAD_SOURCES = ["group_limited_routing_amd/csrc/backward.hip",
                 "group_limited_routing_amd/csrc/common.h"]
COPY_CAL_KIB = 1 << 20          # the calibration copy moves 1 GiB each way



def progress(msg):
    """One line on stderr per phase, so that long runs show where they are."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)

def gateup_kernel(cfg):
    """Name of the kernel the library launches for the gate/up pass of this
    workload with packed weights (same rules as its launcher)."""
    pairs = cfg["T"] * cfg["top_k"]
    xt = "float" if cfg["x_dtype"] == "f32" else "unsigned short"
    fp8 = cfg["w_dtype"] == "fp8"
    E = cfg["n_experts"]
    if cfg["w_dtype"] == "mxfp4":
        if pairs <= 12 * E:  # streamed: 16-row tiles up to 8 rows per expert, else 32
            return "gemm_stream4_kernel<0, 8, 4, 1>" if pairs <= 8 * E else "gemm_stream4_kernel<0, 4, 2, 2>"
        return f"gemm_dma4_kernel<0, {256 if pairs >= 96 * E else 128}>"
    if not fp8 and pairs <= 16 * E:  # packed fp8 weights always take the DMA variant
        return f"gemm_stream_kernel<0, {xt}, false, true, ...>"
    dma = fp8 or xt == "unsigned short"
    bm = 256 if pairs >= (96 if dma else 192) * cfg["n_experts"] else 128
    if cfg["hidden"] % 256:
        bm = 128
    if fp8:
        # 256-row tiles: mixed heights (512 rows for experts beyond 256)
        return "gemm_dma8_mixed_kernel<0>" if bm == 256 else f"gemm_dma8_kernel<0, {bm}>"
    if dma:
        return f"gemm_dma_kernel<0, {bm}>"
    return f"gemm_wide_kernel<0, {xt}, false, {bm}>"


def kernel_source_sha(paths=KERNEL_SOURCES):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def describe(cfg):
    wdesc = {"fp8": "fp8 e4m3 weights, per-row scales",
             "mxfp4": "MXFP4 weights (e2m1, e8m0 scale per 32), e4m3 activations"}.get(
                 cfg["w_dtype"], "bf16 weights")
    return (f"{cfg['name']}: T={cfg['T']} tokens, hidden {cfg['hidden']}, {cfg['n_experts']} experts "
            f"x SwiGLU {cfg['intermediate']}, {wdesc}, x {cfg['x_dtype']}, group-limited top-{cfg['top_k']} "
            f"({cfg['n_group']} groups, keep {cfg['topk_group']}), scale {cfg['routed_scaling_factor']}")


# Bytes per element of the intermediate h as the gate/up launch stores it
# (bf16 with every weight type; quantised weights add one E4M3 code per
# element, counted as h_codes).
H_STORE_BYTES = 2


def quantised(cfg):
    return cfg["w_dtype"] in ("fp8", "mxfp4")


def gateup_work(cfg, active):
    """Algorithmic bytes and flops of one gate/up launch: the gate and up
    weights of the active experts and the token rows read (x, or its E4M3
    codes with quantised weights). The h rows it writes for the down pass
    are design overhead (design_overhead)."""
    T, H, I, k = cfg["T"], cfg["hidden"], cfg["intermediate"], cfg["top_k"]
    wb = WEIGHT_BYTES[cfg["w_dtype"]]
    xb = 4 if cfg["x_dtype"] == "f32" else 2
    x_read = T * H * (1 if quantised(cfg) else xb)
    bytes_ = int(active * 2 * I * H * wb) + x_read
    flops = 4.0 * T * k * H * I
    return bytes_, flops


def down_work(cfg, active):
    """Algorithmic bytes and flops of one down launch: the down weights of
    the active experts (its h input and y output are design overhead)."""
    T, H, I, k = cfg["T"], cfg["hidden"], cfg["intermediate"], cfg["top_k"]
    return int(active * I * H * WEIGHT_BYTES[cfg["w_dtype"]]), 2.0 * T * k * H * I


def design_overhead(cfg):
    """Bytes the implementation moves beyond the block's algorithmic ones:
    h written by the gate/up launch and read back, y (the scaled expert
    outputs, bf16) written by the down launch and read by the combine; with
    quantised weights also the E4M3 codes of x and of h (written, read)."""
    T, H, I, k = cfg["T"], cfg["hidden"], cfg["intermediate"], cfg["top_k"]
    P = T * k
    out = {"h_round_trip": 2 * P * I * H_STORE_BYTES, "y_round_trip": 2 * P * H * 2}
    if quantised(cfg):
        out["x_codes"] = 2 * T * H
        out["h_codes"] = 2 * P * I
    out["total"] = sum(out.values())
    return out


def layer_work(cfg, active):
    """Algorithmic bytes and flops of the whole block (weights of active
    experts + x + out + router weight; expert and router flops)."""
    T, H, I, k, E = cfg["T"], cfg["hidden"], cfg["intermediate"], cfg["top_k"], cfg["n_experts"]
    wb = WEIGHT_BYTES[cfg["w_dtype"]]
    xb = 4 if cfg["x_dtype"] == "f32" else 2
    bytes_ = int(active * 3 * I * H * wb) + 2 * T * H * xb + E * H * 4
    flops = 6.0 * T * k * H * I
    return bytes_, flops


def roofline(bytes_, flops, seconds, wdt, traffic=None):
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS[wdt] * 1e12)
    if t_hbm >= t_mfma:
        ach = bytes_ / seconds / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}
    ach = flops / seconds / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_TFLOPS[wdt],
            "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS[wdt], 4), "traffic": traffic}


def stored_figure(workload, name="gateup", sources=KERNEL_SOURCES, key="hbm_bytes_per_launch"):
    """A figure from a committed counter summary profiles/<name>_<workload>_counters.txt
    (by default the HBM bytes per gate/up launch), or None: missing, or the
    counters were taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{name}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha") != kernel_source_sha(sources):
        return None
    try:
        v = float(vals[key])
    except (KeyError, ValueError):
        return None
    return int(v) if key.endswith("hbm_bytes_per_launch") else v


class Bench:
    def __init__(self, cfg, dev, weights=None, packed=None):
        import torch
        import group_limited_routing_amd as gl
        import workloads
        self.torch, self.gl = torch, gl
        self.cfg = cfg
        x, rw, b = workloads.make_small_inputs(cfg, 0)
        self.x, self.rw, self.b = x.to(dev), rw.to(dev), b.to(dev)
        self.w = weights if weights is not None else workloads.make_expert_weights(cfg, 0, dev)
        # the MFMA fragment copy the timed forward reads (packed once, at load)
        mx = self.w["w_gate"].dtype == torch.uint8
        self.pw = packed if packed is not None else {
            k: gl.pack_weights(self.w[k]) for k in ("w_gate", "w_up", "w_down")}
        w = self.w
        self.scales = None
        if w["w_gate"].dtype == torch.float8_e4m3fn:
            self.scales = (w["w_gate_scale"], w["w_up_scale"], w["w_down_scale"])
        elif mx:  # MXFP4: the block scales are packed like the codes
            self.scales = tuple(gl.pack_mx_scales(w[k + "_scale"]) for k in ("w_gate", "w_up", "w_down"))
        xdt = self.x.dtype
        wdt = w["w_gate"].dtype
        c = gl.make_config(cfg["hidden"], cfg["intermediate"], cfg["n_experts"], cfg["n_group"],
                           cfg["topk_group"], cfg["top_k"], cfg["routed_scaling_factor"], xdt, wdt,
                           packed=True)
        self.ws = torch.empty(gl.workspace_bytes(c, cfg["T"]), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(self.x)
        r = gl.route(self.x, self.rw, self.b, n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                     top_k=cfg["top_k"], return_counts=True, workspace=self.ws)
        cnt = r["expert_counts"].cpu()
        self.active = int((cnt > 0).sum())
        self.max_over_mean = float(cnt.max().item() / cnt.float().mean().item())
        self.residual = None

    def use_residual(self, step):
        """Time the block with its fused residual-stream step from now on."""
        import workloads
        stream, gain = workloads.make_residual_inputs(self.cfg, 0)
        dev = self.x.device
        self.residual = (stream.to(dev), gain.to(dev), step)

    def step(self):
        w = self.pw
        kw = dict(scales=self.scales, packed=True, n_group=self.cfg["n_group"],
                  topk_group=self.cfg["topk_group"], top_k=self.cfg["top_k"],
                  routed_scaling_factor=self.cfg["routed_scaling_factor"], out=self.out,
                  workspace=self.ws)
        if self.residual is None:
            self.gl.forward(self.x, self.rw, self.b, w["w_gate"], w["w_up"], w["w_down"], **kw)
        else:
            s, g, k = self.residual
            self.gl.forward_residual(self.x, self.rw, self.b, w["w_gate"], w["w_up"],
                                     w["w_down"], s, g, k, **kw)

    def routed_forward(self):
        """One forward of the timed configuration that also returns its routing."""
        w = self.pw
        out, r = self.gl.forward(self.x, self.rw, self.b, w["w_gate"], w["w_up"], w["w_down"],
                                 scales=self.scales, packed=True, n_group=self.cfg["n_group"],
                                 topk_group=self.cfg["topk_group"], top_k=self.cfg["top_k"],
                                 routed_scaling_factor=self.cfg["routed_scaling_factor"],
                                 workspace=self.ws, return_routing=True)
        self.torch.cuda.synchronize()
        return out, r

    def run(self, steps, warmup):
        torch, gl = self.torch, self.gl
        for _ in range(warmup):
            self.step()
        per, total, wall = timed_steps(torch, self.step, steps)
        # the two GEMM launches, in a separate pass with the library's events
        # around them (the timed steps above carry none)
        gl.profile_begin(["gateup", "down"])
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        prof = gl.profile_end()
        # per-stage breakdown from a short pass with events on every stage
        gl.profile_begin()
        for _ in range(min(steps, 10)):
            self.step()
        torch.cuda.synchronize()
        stages = {k: round(v[0] / v[1], 4) for k, v in gl.profile_end().items()}
        return {"ms_per_step": statistics.median(per), "ms_per_step_mean": total / steps,
                "wall_s": wall, "gateup_ms": prof["gateup"][0] / prof["gateup"][1],
                "down_ms": prof["down"][0] / prof["down"][1], "stages_ms": stages}


def timed_steps(torch, step, steps):
    """Run `steps` steps back to back between two synchronisations, each
    bracketed by HIP events on the current stream (where the library
    launches). Returns (per-step ms list, total ms, wall seconds)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    return per, ev[0][0].elapsed_time(ev[-1][1]), wall


def backward_work(cfg, active):
    """Bytes each backward stage moves by design (weights of the active
    experts, its input and output tensors) and its flops."""
    T, H, I, k, E = cfg["T"], cfg["hidden"], cfg["intermediate"], cfg["top_k"], cfg["n_experts"]
    P = T * k
    w = active * I * H * 2          # one bf16 matrix of every active expert
    return {
        "bwd_gateup": (2 * w + T * H * 2 + P * 2 * I * 4 + P * I * 2, 4.0 * P * H * I),
        "bwd_down": (w + T * H * 2 + P * 2 * I * 4 + P * 2 * I * 2 + 2 * P * I * 2, 2.0 * P * H * I),
        "bwd_dx": (2 * w + P * 2 * I * 2 + P * H * 2, 4.0 * P * H * I),
        "bwd_wgrad": (3 * E * H * I * 2 + 3 * P * H * 2 + 3 * P * I * 2, 6.0 * P * H * I),
    }


class BackwardBench:
    """The backward pass (gradients of x, the router and the expert weights)
    on a workload's inputs, with a seeded N(0, 1) output gradient."""

    def __init__(self, cfg, dev, weights, packed=None):
        import torch
        import group_limited_routing_amd as gl
        import workloads
        self.torch, self.gl, self.cfg = torch, gl, cfg
        x, rw, b = workloads.make_small_inputs(cfg, 0)
        self.x, self.rw, self.b = x.to(dev), rw.to(dev), b.to(dev)
        self.dout = workloads.normal((cfg["T"], cfg["hidden"]), 1.0, 0, "dout").to(torch.bfloat16).to(dev)
        w = weights
        fwd = packed if packed is not None else {
            k: gl.pack_weights(w[k]) for k in ("w_gate", "w_up")}
        self.pw = {"w_gate": fwd["w_gate"], "w_up": fwd["w_up"],
                   "w_gate_t": gl.pack_weights_transposed(w["w_gate"]),
                   "w_up_t": gl.pack_weights_transposed(w["w_up"]),
                   "w_down_t": gl.pack_weights_transposed(w["w_down"])}
        c = gl.make_config(cfg["hidden"], cfg["intermediate"], cfg["n_experts"], cfg["n_group"],
                           cfg["topk_group"], cfg["top_k"], cfg["routed_scaling_factor"],
                           torch.bfloat16, torch.bfloat16, packed=True)
        self.ws = torch.empty(gl.backward_workspace_bytes(c, cfg["T"], True), dtype=torch.uint8,
                              device=dev)
        r = gl.route(self.x, self.rw, self.b, n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                     top_k=cfg["top_k"], return_counts=True)
        self.active = int((r["expert_counts"].cpu() > 0).sum())

    def step(self):
        p = self.pw
        return self.gl.backward(self.x, self.rw, self.b, p["w_gate"], p["w_up"], p["w_gate_t"],
                                p["w_up_t"], p["w_down_t"], self.dout, weight_grads=True,
                                n_group=self.cfg["n_group"], topk_group=self.cfg["topk_group"],
                                top_k=self.cfg["top_k"],
                                routed_scaling_factor=self.cfg["routed_scaling_factor"],
                                workspace=self.ws)

    def run(self, steps, warmup):
        torch, gl = self.torch, self.gl
        for _ in range(warmup):
            self.step()
        per, _, _ = timed_steps(torch, self.step, steps)
        ms = statistics.median(per)
        gl.profile_begin()
        for _ in range(min(steps, 5)):
            self.step()
        torch.cuda.synchronize()
        prof = gl.profile_end()
        per_step = {k: round(v[0] / min(steps, 5), 4) for k, v in prof.items()}
        return ms, per_step


def backward_line(cfg, dev, weights, steps, packed=None):
    bb = BackwardBench(cfg, dev, weights, packed)
    ms, per_step = bb.run(steps, 2)
    work = backward_work(cfg, bb.active)
    # roofline of the longest stage (its launches in one step)
    name = max(work, key=lambda k: per_step.get(k, 0.0))
    by, fl = work[name]
    traffic = None
    if name == "bwd_wgrad":
        traffic = stored_figure("backward", "wgrad", WGRAD_SOURCES, "hbm_bytes_per_step")
    rl = roofline(by, fl, per_step[name] / 1e3, "bf16", traffic)
    out = {"workload": f"backward of {describe(cfg)}; gradients of x, the router and all "
                       "expert weights (bf16), output gradient N(0, 1)",
           "value": round(cfg["T"] / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
           "steps": steps, "active_experts": bb.active,
           "roofline": dict(rl, stage=name, launch_ms=per_step[name], algorithmic_bytes=by,
                            algorithmic_flops=fl),
           "stages_ms_per_step": per_step}
    del bb
    return out


def ep_shard_line(dev, bench, gpus=8, steps=50):
    """One of `gpus` expert shards at Beam's decode shape: the tokens of
    `gpus` x 64-token decode batches are routed over all experts and this
    shard (experts 0 .. 256 / gpus - 1, its weights only) runs its share."""
    import torch
    import group_limited_routing_amd as gl
    import workloads
    cfg = dict(workloads.workload("decode"), T=64 * gpus)
    e1 = cfg["n_experts"] // gpus
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, 0))
    w = {k: bench.pw[k][:e1] for k in ("w_gate", "w_up", "w_down")}
    r = gl.route(x, rw, b, return_counts=True)
    cnt = r["expert_counts"].cpu()[:e1]
    active, pairs = int((cnt > 0).sum()), int(cnt.sum())
    c = gl.make_config(cfg["hidden"], cfg["intermediate"], x_dtype=x.dtype, w_dtype=w["w_gate"].dtype,
                       packed=True)
    ws = torch.empty(gl.workspace_bytes(c, cfg["T"]), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    def step():
        gl.forward_shard(x, rw, b, 0, e1, w["w_gate"], w["w_up"], w["w_down"], packed=True,
                         out=out, workspace=ws)
    for _ in range(5):
        step()
    per, _, _ = timed_steps(torch, step, steps)
    ms = statistics.median(per)
    gl.profile_begin(["gateup"])
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = gl.profile_end()
    gu_ms = prof["gateup"][0] / prof["gateup"][1]
    H, I = cfg["hidden"], cfg["intermediate"]
    gb = active * 2 * I * H * 2 + cfg["T"] * H * 2
    return {"workload": f"expert shard 0-{e1 - 1} of {gpus} at decode: {cfg['T']} tokens "
                        f"({gpus} x 64) routed over all experts, this shard's {pairs} pairs "
                        f"on {active} active experts, bf16 weights (its {e1} experts only)",
            "ms_per_step": round(ms, 4), "steps": steps,
            "roofline": dict(roofline(gb, 4.0 * pairs * H * I, gu_ms / 1e3, "bf16",
                                      traffic=stored_figure("ep_shard")),
                             kernel="gate/up", launch_ms=round(gu_ms, 4), algorithmic_bytes=gb)}


def blas_threads():
    """Threads of the BLAS library numpy calls (0 if it cannot be told)."""
    try:
        from threadpoolctl import threadpool_info
        return sum(i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas")
    except Exception:  # threadpoolctl missing or unable to inspect the library
        return 0


def cpu_baseline(cfg, bench, n_tokens, runs=3):
    """The oracle on the first n_tokens tokens of the same inputs (float64),
    timed `runs` times (the median is reported); then the timed
    configuration's routing and outputs on those tokens compared with the
    oracle's. Returns (baseline, parity)."""
    import numpy as np
    import torch
    import oracle
    tok = np.arange(n_tokens)
    x64 = bench.x[:n_tokens].cpu().double().numpy()
    rw64 = bench.rw.cpu().double().numpy()
    b64 = bench.b.cpu().double().numpy()
    r = oracle.route(x64, rw64, b64, cfg["n_group"], cfg["topk_group"], cfg["top_k"])
    need = sorted(set(int(e) for e in np.unique(r["idx"])))
    fp8 = cfg["w_dtype"] == "fp8"
    mx = cfg["w_dtype"] == "mxfp4"
    host = {}
    for e in need:  # copy the needed experts to host memory before timing
        host[e] = {k: bench.w[k][e].cpu() for k in ("w_gate", "w_up", "w_down")}
        if fp8 or mx:
            for k in ("w_gate", "w_up", "w_down"):
                host[e][k + "_scale"] = bench.w[k + "_scale"][e].cpu()

    def get(e):
        if mx:
            return tuple(oracle.mxfp4.dequantize(host[e][k].numpy(), host[e][k + "_scale"].numpy())
                         for k in ("w_gate", "w_up", "w_down"))
        if fp8:
            return tuple(oracle.e4m3.decode(host[e][k].view(torch.uint8).numpy())
                         * host[e][k + "_scale"].double().numpy()[:, None]
                         for k in ("w_gate", "w_up", "w_down"))
        return tuple(host[e][k].double().numpy() for k in ("w_gate", "w_up", "w_down"))

    times = []
    xall = bench.x.cpu().double().numpy()
    for _ in range(runs):
        t0 = time.perf_counter()
        ref, _ = oracle.forward_tokens(tok, xall, rw64, b64, get, n_group=cfg["n_group"],
                                       topk_group=cfg["topk_group"], top_k=cfg["top_k"],
                                       routed_scaling_factor=cfg["routed_scaling_factor"],
                                       fp8=fp8 or mx)
        times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    base = {"value": round(n_tokens / dt, 3), "unit": "tokens/s",
            "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "blas_threads": blas_threads(),
            "sample": f"first {n_tokens} tokens of the {cfg['name']} workload ({len(need)} experts), "
                      f"float64 numpy, median of {runs} runs: {dt:.1f} s "
                      f"(runs {', '.join(f'{t:.1f}' for t in times)} s)"}
    # the timed forward's routing and output on the same tokens against the
    # oracle's: expert indices outside the near-tie band (margin < 1e-6) must
    # agree, outputs are compared where the routing agrees
    out, gr = bench.routed_forward()
    gidx = gr["topk_idx"][:n_tokens].cpu().numpy().astype(np.int64)
    near = r["margin"] < 1e-6
    same = np.all(gidx == r["idx"], axis=1)
    got = out[:n_tokens].cpu().double().numpy()[same]
    want = ref[same]
    d = got - want
    row_inf = np.abs(want).max(axis=1)
    parity = {"tokens": n_tokens,
              "routing_mismatches": int(np.sum(~same & ~near)),
              "near_ties": int(near.sum()),
              "outputs_compared": int(same.sum()),
              "max_rel": float(np.max(np.abs(d).max(axis=1) / np.where(row_inf > 0, row_inf, 1.0)))
              if same.any() else None,
              "normwise": float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-300))
              if same.any() else None,
              "bars": {"max_rel": 2e-2, "normwise": 5e-3}}
    return base, parity


def summarize(d):
    """Print kernel statistics / counters found under a rocprofv3 output dir."""
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"# kernel stats: {os.path.relpath(path, d)}")
        with open(path) as f:
            rows = list(csv.DictReader(f))
        print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
        for r in rows:
            print(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.1f} {float(r['MinNs']) / 1e3:>10.1f} "
                  f"{float(r['MaxNs']) / 1e3:>10.1f} {float(r['Percentage']):>6.2f}  {r['Name'][:110]}")
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        print(f"# counters: {os.path.relpath(path, d)}")
        agg = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"][:110], r["Counter_Name"])
                a = agg.setdefault(key, [0.0, 0])
                a[0] += float(r["Counter_Value"])
                a[1] += 1
        print(f"{'dispatches':>10} {'mean_per_dispatch':>20}  counter  kernel")
        for (kname, cname), (tot, n) in sorted(agg.items()):
            print(f"{n:>10} {tot / n:>20.1f}  {cname}  {kname}")


def _counter_rows(d):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


MFMA_COUNTERS = "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_BUSY_CU_CYCLES"
N_SIMDS = 1024  # 256 CUs x 4 SIMDs
N_XCDS = 8      # GRBM_GUI_ACTIVE sums one count per XCD


def write_mfma(pmc_dir, workload):
    """Matrix-core utilisation of the two expert GEMM launches from one
    rocprofv3 --pmc pass (MFMA_COUNTERS) over `bench.py --workload W`:
    per kernel the mean dispatch duration, the shader clock (GRBM_GUI_ACTIVE
    per XCD over the duration), the fraction of SIMD cycles the matrix core
    was busy (SQ_VALU_MFMA_BUSY_CYCLES over SIMDs x cycles) and the MFMA
    instructions per dispatch."""
    import re
    rows = _counter_rows(pmc_dir)
    pat = re.compile(r"beam::gemm_\w+<([01])[,>]")
    per = {}
    for r in rows:
        m = pat.search(r["Kernel_Name"])
        if not m:
            continue
        k = per.setdefault(m.group(1), {"name": r["Kernel_Name"], "ids": {}, "c": {}})
        did = r["Dispatch_Id"]
        if did not in k["ids"]:
            k["ids"][did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        k["c"][r["Counter_Name"]] = k["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if "0" not in per:
        raise SystemExit(f"no gate/up GEMM dispatches under {pmc_dir}")
    lines = []
    for mode, label in (("0", "gateup"), ("1", "down")):
        if mode not in per:
            continue
        k = per[mode]
        n = len(k["ids"])
        dur = sum(k["ids"].values()) / n
        c = {name: v / n for name, v in k["c"].items()}
        cyc = c["GRBM_GUI_ACTIVE"] / N_XCDS
        lines += [f"{label}_kernel = {k['name']}",
                  f"{label}_dispatches = {n}",
                  f"{label}_duration_ms = {dur * 1e3:.4f}",
                  f"{label}_clock_ghz = {cyc / dur / 1e9:.3f}",
                  f"{label}_mfma_busy = {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMDS * cyc):.4f}",
                  f"{label}_mfma_insts = {c['SQ_INSTS_MFMA']:.0f}",
                  f"{label}_cu_busy = {c['SQ_BUSY_CU_CYCLES'] / (256 * cyc):.4f}"]
    cmd = (f"cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {MFMA_COUNTERS} "
           "--kernel-include-regex 'gemm' -d <dir> -o run --output-format csv "
           f"-- python3 /root/repo/bench.py --workload {workload} --steps 3 --warmup 1 --no-prefill "
           "--no-residual --no-backward --no-shard --no-fp8 --no-cpu-baseline")
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}_counters.txt")
    with open(path, "w") as fh:
        fh.write(f"# Matrix-core utilisation of the expert GEMMs, workload {workload}, one MI355X\n")
        fh.write(f"# command: {cmd}\n")
        fh.write(f"#   python3 bench.py --mfma <dir> --workload {workload}\n")
        fh.write("# clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES /\n")
        fh.write("# (1024 SIMDs x clock cycles); cu_busy = SQ_BUSY_CU_CYCLES / (256 CUs x clock cycles)\n")
        fh.write("\n".join(lines) + "\n")
        fh.write(f"kernel_source_sha = {kernel_source_sha()}\n")
    print(open(path).read())


def write_wgrad_traffic(fetch_dir, write_dir):
    """HBM bytes of the backward's weight-gradient launches per step (three
    launches, per-dispatch counters scaled as in write_traffic), from passes
    over the default decode run with its backward line."""
    out = {}
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _counter_rows(d)
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        wg = [r for r in rows if "gemm_wgrad_kernel" in r["Kernel_Name"]]
        if not wg:
            raise SystemExit(f"no weight-gradient dispatches in {d}")
        out[name] = {"copy_kib": copy, "factor": COPY_CAL_KIB / copy,
                     "kib": sum(float(r["Counter_Value"]) for r in wg) / len(wg), "n": len(wg),
                     "kernel": wg[0]["Kernel_Name"]}
    f, w = out["fetch"], out["write"]
    per_launch = (f["kib"] * f["factor"] + w["kib"] * w["factor"]) * 1024
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} -d <dir> -o run --output-format csv "
           "-- python3 /root/repo/bench.py --steps 3 --warmup 1 --no-prefill --no-residual "
           "--no-shard --no-fp8 --no-cpu-baseline --calibrate-copy --backward-steps 2")
    path = os.path.join(ROOT, "profiles", "wgrad_backward_counters.txt")
    with open(path, "w") as fh:
        fh.write("# HBM traffic of the backward's weight-gradient GEMMs (prefill shape, all\n"
                 "# expert weights), one MI355X\n# commands (one counter per pass):\n")
        fh.write("#   " + cmd.format(c="FETCH_SIZE") + "\n")
        fh.write("#   " + cmd.format(c="WRITE_SIZE") + "\n")
        fh.write("#   python3 bench.py --wgrad-traffic <fetch dir> <write dir>\n")
        fh.write(f"kernel = {f['kernel']}\n")
        fh.write(f"dispatches = {f['n']}\n")
        fh.write(f"fetch_kib_per_dispatch = {f['kib']:.1f}\n")
        fh.write(f"write_kib_per_dispatch = {w['kib']:.1f}\n")
        fh.write(f"fetch_factor = {f['factor']:.4f}\n")
        fh.write(f"write_factor = {w['factor']:.4f}\n")
        fh.write(f"hbm_bytes_per_launch = {per_launch:.0f}\n")
        fh.write(f"hbm_bytes_per_step = {3 * per_launch:.0f}\n")
        fh.write(f"kernel_source_sha = {kernel_source_sha(WGRAD_SOURCES)}\n")
    print(open(path).read())


def write_traffic(fetch_dir, write_dir, workload):
    """Turn one FETCH_SIZE pass and one WRITE_SIZE pass (rocprofv3 --pmc, KiB per
    dispatch) over `bench.py --workload W --no-prefill --calibrate-copy` into
    HBM bytes per launch of the gate/up and of the down GEMM. Each counter is
    scaled by what it reads for the 1 GiB device copy made before the timed
    region (the largest copyBuffer dispatch of the run)."""
    import re
    pats = {"gateup": re.compile(r"beam::gemm_\w+<0[,>]"), "down": re.compile(r"beam::gemm_\w+<1[,>]")}
    run = (f"--workload {workload} --steps 3 --warmup 1 --no-prefill --no-residual --no-backward "
           "--no-shard --no-fp8 --no-cpu-baseline --calibrate-copy")
    if workload == "ep_shard":
        # the decode run with its expert-shard line: the shard's 512 tokens
        # (about 15 rows per expert) take the 32-row streaming kernels, the
        # 64 decode tokens the 16-row ones
        pats = {"gateup": re.compile(r"beam::gemm_stream_kernel<0, .*, 2>\("),
                "down": re.compile(r"beam::gemm_stream_kernel<1, .*, 2>\(")}
        run = ("--workload decode --steps 3 --warmup 1 --no-prefill --no-residual --no-backward "
               "--no-fp8 --no-cpu-baseline --calibrate-copy")
    out = {}
    for name, d in (("fetch", fetch_dir), ("write", write_dir)):
        rows = _counter_rows(d)
        copy = max(float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
        out[name] = {"copy_kib": copy, "factor": COPY_CAL_KIB / copy}
        for stage, pat in pats.items():
            sel = [r for r in rows if pat.search(r["Kernel_Name"])]
            kernels = sorted({r["Kernel_Name"] for r in sel})
            if len(kernels) != 1:
                raise SystemExit(f"expected one {stage} kernel in {d}, found {kernels}")
            out[name][stage] = {"kib": sum(float(r["Counter_Value"]) for r in sel) / len(sel),
                                "n": len(sel), "kernel": kernels[0]}
    f, w = out["fetch"], out["write"]
    hbm = {st: (f[st]["kib"] * f["factor"] + w[st]["kib"] * w["factor"]) * 1024 for st in pats}
    cmd = ("cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc {c} --kernel-include-regex 'gemm|copyBuffer' "
           f"-d <dir> -o run --output-format csv -- python3 /root/repo/bench.py {run}")
    path = os.path.join(ROOT, "profiles", f"gateup_{workload}_counters.txt")
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of the gate/up and down grouped GEMMs, workload {workload}, one MI355X\n")
        fh.write("# commands (one counter per pass):\n")
        fh.write("#   " + cmd.format(c="FETCH_SIZE") + "\n")
        fh.write("#   " + cmd.format(c="WRITE_SIZE") + "\n")
        fh.write(f"#   python3 bench.py --traffic <fetch dir> <write dir> --workload {workload}\n")
        fh.write("# calibration: a 1 GiB device copy reads and writes 1048576 KiB\n")
        fh.write(f"kernel = {f['gateup']['kernel']}\n")
        fh.write(f"dispatches = {f['gateup']['n']}\n")
        fh.write(f"fetch_kib_per_dispatch = {f['gateup']['kib']:.1f}\n")
        fh.write(f"write_kib_per_dispatch = {w['gateup']['kib']:.1f}\n")
        fh.write(f"down_kernel = {f['down']['kernel']}\n")
        fh.write(f"down_fetch_kib_per_dispatch = {f['down']['kib']:.1f}\n")
        fh.write(f"down_write_kib_per_dispatch = {w['down']['kib']:.1f}\n")
        fh.write(f"copy_fetch_kib = {f['copy_kib']:.1f}\n")
        fh.write(f"copy_write_kib = {w['copy_kib']:.1f}\n")
        fh.write(f"fetch_factor = {f['factor']:.4f}\n")
        fh.write(f"write_factor = {w['factor']:.4f}\n")
        fh.write(f"hbm_bytes_per_launch = {hbm['gateup']:.0f}\n")
        fh.write(f"down_hbm_bytes_per_launch = {hbm['down']:.0f}\n")
        fh.write(f"kernel_source_sha = {kernel_source_sha()}\n")
    print(open(path).read())


def workload_line(cfg, bench, steps, warmup):
    """Time one workload (Bench.run) and report it: throughput, the gate/up
    and down launches against their rooflines, the whole layer, and the
    stored rocprofv3 figures for its kernels."""
    res = bench.run(steps, warmup)
    wdt = "fp8" if quantised(cfg) else "bf16"
    name = cfg["name"]
    gb, gf = gateup_work(cfg, bench.active)
    db, df = down_work(cfg, bench.active)
    lb, lf = layer_work(cfg, bench.active)
    step_s = res["ms_per_step"] / 1e3
    rl = roofline(gb, gf, res["gateup_ms"] / 1e3, wdt, stored_figure(name))
    drl = roofline(db, df, res["down_ms"] / 1e3, wdt,
                   stored_figure(name, key="down_hbm_bytes_per_launch"))
    return {
        "workload": describe(cfg),
        "value": round(cfg["T"] / step_s, 1), "unit": "tokens/s",
        "ms_per_step": round(res["ms_per_step"], 4),
        "ms_per_step_mean": round(res["ms_per_step_mean"], 4),
        "steps": steps, "warmup": warmup,
        "dtype": "mxfp4 x e4m3" if cfg["w_dtype"] == "mxfp4" else wdt,
        "active_experts": bench.active, "max_over_mean_load": round(bench.max_over_mean, 4),
        "roofline": dict(rl, kernel=gateup_kernel(cfg), launch_ms=round(res["gateup_ms"], 4),
                         algorithmic_bytes=gb, algorithmic_flops=gf,
                         mfma_busy=stored_figure(name, "mfma", key="gateup_mfma_busy"),
                         clock_ghz=stored_figure(name, "mfma", key="gateup_clock_ghz")),
        "down_roofline": dict(drl, launch_ms=round(res["down_ms"], 4), algorithmic_bytes=db,
                              algorithmic_flops=df,
                              mfma_busy=stored_figure(name, "mfma", key="down_mfma_busy"),
                              clock_ghz=stored_figure(name, "mfma", key="down_clock_ghz")),
        "layer": {"pct_hbm": round(lb / step_s / 1e9 / HBM_PEAK_GBS, 4),
                  "pct_mfma": round(lf / step_s / 1e12 / MFMA_PEAK_TFLOPS[wdt], 4),
                  "algorithmic_bytes": lb, "flops": lf,
                  "design_overhead_bytes": design_overhead(cfg),
                  "stages_ms": res["stages_ms"]},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode",
                    choices=["tiny", "decode", "prefill", "skewed", "fp8", "mxfp4", "mxfp4_prefill",
                             "ep_shard"])
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill and skewed lines (decode runs)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the fp8 line (decode runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-residual", action="store_true",
                    help="skip timing the block with its fused residual step")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward pass at the prefill shape")
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--no-shard", action="store_true",
                    help="skip timing one expert shard of 8 at the decode shape")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens the oracle runs on (default: 64, MXFP4 weights 4; ~10-30 s)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma", metavar="PMC_DIR")
    ap.add_argument("--wgrad-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()

    if args.summarize:
        summarize(args.summarize)
        return 0
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.workload)
        return 0
    if args.workload == "ep_shard":
        raise SystemExit("--workload ep_shard only names the counter summary of --traffic; the "
                         "expert-shard line runs with the decode workload")
    if args.wgrad_traffic:
        write_wgrad_traffic(args.wgrad_traffic[0], args.wgrad_traffic[1])
        return 0
    if args.mfma:
        write_mfma(args.mfma, args.workload)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py measures one GPU: the library has no cross-GPU exchange (one expert "
              "shard's compute is timed on one GPU in the ep_shard line); run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import workloads
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = workloads.workload(args.workload)
    progress(f"{args.workload}: inputs and weights")
    bench = Bench(cfg, dev)
    progress(f"{args.workload}: {args.warmup} warmup + {args.steps} timed steps")
    main_line = workload_line(cfg, bench, args.steps, args.warmup)
    line = {
        "metric": METRIC,
        "value": main_line["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_line["ms_per_step"],
        "ms_per_step_mean": main_line["ms_per_step_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_line["dtype"],
        "data": "synthetic",
        "device": {"name": torch.cuda.get_device_name(0),
                   "arch": torch.cuda.get_device_properties(0).gcnArchName,
                   "hip": torch.version.hip, "host_cores": len(os.sched_getaffinity(0))},
        "config": {"workload": describe(cfg), "T": cfg["T"], "hidden": cfg["hidden"],
                   "intermediate": cfg["intermediate"], "n_experts": cfg["n_experts"],
                   "n_group": cfg["n_group"], "topk_group": cfg["topk_group"], "top_k": cfg["top_k"],
                   "active_experts": bench.active, "max_over_mean_load": round(bench.max_over_mean, 4),
                   "parallelism": "single GPU"},
        "roofline": main_line["roofline"],
        "down_roofline": main_line["down_roofline"],
        "layer": main_line["layer"],
    }
    if not args.no_residual:
        # the same block with the fused post-norm + depth-scaled residual step
        # (the MoE of the last layer: step 105)
        bench.use_residual(105)
        progress("fused residual step")
        rres = bench.run(min(args.steps, 50), 3)
        bench.residual = None
        line["fused_residual"] = {
            "step": 105, "ms_per_step": round(rres["ms_per_step"], 4),
            "value": round(cfg["T"] / (rres["ms_per_step"] / 1e3), 1), "unit": "tokens/s",
            "combine_ms": rres["stages_ms"].get("combine"),
            "plain_combine_ms": main_line["layer"]["stages_ms"].get("combine")}
    if args.workload == "decode" and not args.no_prefill:
        for name, steps in (("prefill", args.prefill_steps), ("skewed", args.prefill_steps)):
            progress(name)
            wb = Bench(workloads.workload(name), dev, weights=bench.w, packed=bench.pw)
            line[name] = workload_line(wb.cfg, wb, steps, 3)
            del wb
            torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_shard:
        progress("expert shard")
        line["ep_shard"] = ep_shard_line(dev, bench)
    if args.workload == "decode" and not args.no_backward:
        progress("backward")
        line["backward"] = backward_line(workloads.workload("prefill"), dev, bench.w,
                                         args.backward_steps, bench.pw)
        torch.cuda.empty_cache()
    if args.workload == "decode" and not args.no_fp8:
        progress("fp8: weights")
        fcfg = workloads.workload("fp8")
        fb = Bench(fcfg, dev)
        progress("fp8")
        line["fp8"] = workload_line(fcfg, fb, args.prefill_steps, 3)
        del fb
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        n_cpu = args.cpu_tokens or (4 if cfg["w_dtype"] == "mxfp4" else 64)
        progress(f"cpu baseline: the oracle on {min(n_cpu, cfg['T'])} tokens")
        line["cpu_baseline"], line["parity_sample"] = cpu_baseline(cfg, bench, min(n_cpu, cfg["T"]))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

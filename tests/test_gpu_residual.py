"""GPU parity of the fused residual step (beam_moe_forward_residual) against
the oracle: the oracle's MoE output, then oracle.residual.residual_update
(post-norm RMSNorm with gain and eps, depth-scaled residual at step k).

The same output criteria as the block itself (max over tokens of the
row-relative inf-norm error <= 2e-2, normwise <= 5e-3): RMSNorm is scale
invariant, so the relative error of the normalised block output is that of
the block output, and the stream term adds only the output rounding.
"""

import json

import numpy as np
import pytest
import torch

import oracle
import workloads
import group_limited_routing_amd as gl
from parity import (check_outputs, check_routing, guarded_out, guarded_workspace,
                    oracle_reference, packed_copy)

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(T, H, I, x_dtype="bf16", w_dtype="bf16"):
    cfg = dict(workloads.BEAM)
    cfg.update(T=T, hidden=H, intermediate=I, x_dtype=x_dtype, w_dtype=w_dtype, bias="normal")
    return cfg


def _scales(w):
    if w["w_gate"].dtype in (torch.float8_e4m3fn, torch.uint8):
        return (w["w_gate_scale"], w["w_up_scale"], w["w_down_scale"])
    return None


def _run(name, cfg, seed, step, eps=1e-6, packed=False, in_place=False, tokens=None):
    dev = _dev()
    x, rw, b = workloads.make_small_inputs(cfg, seed)
    x, rw, b = x.to(dev), rw.to(dev), b.to(dev)
    stream, gain = workloads.make_residual_inputs(cfg, seed)
    stream, gain = stream.to(dev), gain.to(dev)
    w = workloads.make_expert_weights(cfg, seed, dev)
    gw = packed_copy(w) if packed else w
    stream64 = stream.cpu().double().numpy()
    print(f"\n[residual] {name}: T={cfg['T']} H={cfg['hidden']} I={cfg['intermediate']} "
          f"step={step} eps={eps}", flush=True)
    ws = guarded_workspace(x, gw, cfg)
    og, gout = guarded_out(x)
    out, r = gl.forward_residual(x, rw, b, gw["w_gate"], gw["w_up"], gw["w_down"], stream, gain,
                                 step, norm_eps=eps, scales=_scales(gw),
                                 packed=gw.get("packed", False), out=stream if in_place else gout,
                                 return_routing=True, workspace=ws.view)
    torch.cuda.synchronize()
    ws.check()
    og.check()
    if in_place:
        assert out.data_ptr() == stream.data_ptr()
    T = cfg["T"]
    x64 = x.cpu().double().numpy()
    ora = oracle.route(x64, rw.cpu().double().numpy(), b.cpu().double().numpy(), cfg["n_group"],
                       cfg["topk_group"], cfg["top_k"])
    rep = {"T": T, "H": cfg["hidden"], "step": step, "eps": eps}
    near = check_routing(r, ora, cfg, rep)
    toks = np.arange(T) if tokens is None else tokens
    moe = oracle_reference(toks, x, rw, b, w, cfg, r["topk_idx"].cpu().numpy(), near)
    ref = oracle.residual.residual_update(stream64[toks], moe, gain.cpu().double().numpy(), eps,
                                          step)
    got = out[torch.as_tensor(toks, device=dev)].cpu().double().numpy()
    check_outputs(got, ref, rep)
    rep["block_out_mean_square"] = float(np.mean(moe * moe))
    print(f"[residual] {name}: " + json.dumps(rep), flush=True)
    del w, gw
    torch.cuda.empty_cache()
    return out, r


def test_residual_tiny_fp32_stream():
    """x and the stream fp32 (T=128, H=256, I=128), step 3."""
    _run("tiny f32", workloads.workload("tiny"), 0, 3)


def test_residual_bf16_in_place_ragged():
    """bf16 stream updated in place; H=384 leaves most of the workgroup's
    lanes without a chunk; a late step (the MoE of the last of 52 layers)."""
    _run("ragged in place", _case(300, 384, 256), 3, 105, in_place=True)


def test_residual_eps_matters():
    """eps of the order of the block output's mean square, so that its
    place inside the square root is tested (the default eps is far below)."""
    _run("large eps", _case(200, 512, 256), 8, 7, eps=3e-3)


def test_residual_fp8_packed():
    _run("fp8 packed", _case(200, 512, 256, w_dtype="fp8"), 6, 11, packed=True)


def test_residual_widest_row():
    """hidden 16384, the largest row the fused step takes: every lane holds
    its full 8 chunks."""
    _run("H=16384", _case(8, 16384, 128), 9, 2)


def test_residual_matches_unfused_routing():
    """Routing of the fused call equals the plain forward's, and the block
    output of the plain forward pushed through the oracle's residual step
    (in fp64) is within the output rounding of the fused result."""
    dev = _dev()
    cfg = _case(256, 1024, 512)
    x, rw, b = workloads.make_small_inputs(cfg, 21)
    x, rw, b = x.to(dev), rw.to(dev), b.to(dev)
    stream, gain = workloads.make_residual_inputs(cfg, 21)
    stream, gain = stream.to(dev), gain.to(dev)
    w = workloads.make_expert_weights(cfg, 21, dev)
    print("\n[residual] fused vs plain forward: T=256 H=1024 I=512", flush=True)
    plain, r0 = gl.forward(x, rw, b, w["w_gate"], w["w_up"], w["w_down"], return_routing=True)
    fused, r1 = gl.forward_residual(x, rw, b, w["w_gate"], w["w_up"], w["w_down"], stream, gain,
                                    9, return_routing=True)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_w", "expert_counts"):
        assert torch.equal(r0[k], r1[k]), k
    ref = oracle.residual.residual_update(stream.cpu().double().numpy(),
                                          plain.cpu().double().numpy(),
                                          gain.cpu().double().numpy(), 1e-6, 9)
    # the plain output is rounded to bf16 before the oracle's step; the
    # fused step never rounds the block output
    rep = {}
    check_outputs(fused.cpu().double().numpy(), ref, rep)
    assert rep["normwise"] <= 2e-3, rep
    print("[residual] fused vs plain: " + json.dumps(rep), flush=True)


@pytest.mark.parametrize("wl", ["decode", "mxfp4"])
def test_residual_full_decode_shape(wl):
    """Beam's decode shape (T=64, H=5120, I=2560) with packed weights, step
    105; the outputs of every token against the oracle."""
    cfg = workloads.workload(wl)
    _run(f"{wl} full shape", cfg, 0, 105, packed=True)

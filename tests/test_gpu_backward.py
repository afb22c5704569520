"""GPU parity of the backward pass (beam_moe_backward), the transposed weight
packing and the bias step, against the oracle (oracle/backward.py).

The GPU recomputes the routing with the forward's kernels; near-tie tokens
(oracle margin < 1e-6) are given the GPU's choice on the oracle side, as in
the forward's parity tests. Gradients are compared with the criteria of
``check_grad`` below.
"""

import json

import numpy as np
import pytest
import torch

import oracle
import workloads
import group_limited_routing_amd as gl
from parity import (Guarded, check_routing, coverage_report, expert_getter, output_errors,
                    tile_cover)

pytestmark = pytest.mark.gpu

# dx and the weight gradients pass through bf16-stored intermediates (dg and
# du, the per-slot input-gradient rows, the transposed operands) with fp32
# arithmetic in between; each bf16 rounding adds a relative error of at most
# 2^-9, so they are held to the forward's bars (row max-relative 2e-2,
# normwise 5e-3). The router gradient is computed from fp32 values only
# (g and u are kept in fp32, h . q and dz are fp32 sums; x, dout and the
# weights are exact bf16 inputs), so its error is fp32 accumulation error:
# bars 1e-4 row max-relative and 1e-5 normwise.
BARS = {"dx": (2e-2, 5e-3), "d_w_gate": (2e-2, 5e-3), "d_w_up": (2e-2, 5e-3),
        "d_w_down": (2e-2, 5e-3), "d_router_w": (1e-4, 1e-5)}


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(T, H, I):
    cfg = dict(workloads.BEAM)
    cfg.update(T=T, hidden=H, intermediate=I, x_dtype="bf16", w_dtype="bf16", bias="normal")
    return cfg


def check_grad(name, got, ref, rep):
    max_rel, normwise = output_errors(got, ref)
    rep[name] = {"max_rel": max_rel, "normwise": normwise}
    bmax, bnorm = BARS[name]
    if bmax is not None:
        assert max_rel <= bmax, (name, max_rel)
    assert normwise <= bnorm, (name, normwise)


def _packed(w):
    return {"w_gate": gl.pack_weights(w["w_gate"]), "w_up": gl.pack_weights(w["w_up"]),
            "w_gate_t": gl.pack_weights_transposed(w["w_gate"]),
            "w_up_t": gl.pack_weights_transposed(w["w_up"]),
            "w_down_t": gl.pack_weights_transposed(w["w_down"])}


def _run(cfg, x, rw, b, pw, dout, weight_grads=True):
    """beam_moe_backward on a guarded workspace of exactly the size it asks for."""
    c = gl.make_config(x.shape[1], pw["w_gate"].shape[1], cfg["n_experts"], cfg["n_group"],
                       cfg["topk_group"], cfg["top_k"], cfg["routed_scaling_factor"],
                       torch.bfloat16, torch.bfloat16, packed=True)
    ws = Guarded(gl.backward_workspace_bytes(c, x.shape[0], weight_grads), x.device,
                 "backward workspace")
    g = gl.backward(x, rw, b, pw["w_gate"], pw["w_up"], pw["w_gate_t"], pw["w_up_t"],
                    pw["w_down_t"], dout, weight_grads=weight_grads, n_group=cfg["n_group"],
                    topk_group=cfg["topk_group"], top_k=cfg["top_k"],
                    routed_scaling_factor=cfg["routed_scaling_factor"], workspace=ws.view)
    torch.cuda.synchronize()
    ws.check()
    return g


def _routing(cfg, x, rw, b, rep):
    r = gl.route(x, rw, b, n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                 top_k=cfg["top_k"], return_counts=True)
    torch.cuda.synchronize()
    x64 = x.cpu().double().numpy()
    ora = oracle.route(x64, rw.cpu().double().numpy(), b.cpu().double().numpy(), cfg["n_group"],
                       cfg["topk_group"], cfg["top_k"])
    near = check_routing(r, ora, cfg, rep)
    idx = ora["idx"].copy()
    idx[near] = r["topk_idx"].cpu().numpy()[near]
    return idx, r


def _full_compare(name, cfg, seed):
    dev = _dev()
    print(f"\n[backward] {name}: T={cfg['T']} H={cfg['hidden']} I={cfg['intermediate']}", flush=True)
    x, rw, b = workloads.make_small_inputs(cfg, seed)
    x, rw, b = x.to(dev), rw.to(dev), b.to(dev)
    dout = workloads.normal((cfg["T"], cfg["hidden"]), 1.0, seed, "dout").to(torch.bfloat16).to(dev)
    w = workloads.make_expert_weights(cfg, seed, dev)
    pw = _packed(w)
    g = _run(cfg, x, rw, b, pw, dout)
    rep = {"T": cfg["T"]}
    idx, r = _routing(cfg, x, rw, b, rep)
    ref = oracle.backward.backward(x.cpu().double().numpy(), rw.cpu().double().numpy(),
                                   b.cpu().double().numpy(), expert_getter(w),
                                   dout.cpu().double().numpy(), cfg["n_group"], cfg["topk_group"],
                                   cfg["top_k"], cfg["routed_scaling_factor"], routing=idx)
    check_grad("dx", g["dx"].cpu().double().numpy(), ref["dx"], rep)
    check_grad("d_router_w", g["d_router_w"].cpu().double().numpy(), ref["d_router_w"], rep)
    chosen = sorted(ref["d_w_gate"])
    for name_ in ("d_w_gate", "d_w_up", "d_w_down"):
        got = g[name_].cpu().double().numpy()
        check_grad(name_, np.concatenate([got[e] for e in chosen]),
                   np.concatenate([ref[name_][e] for e in chosen]), rep)
        # experts no token chose get zeros
        unchosen = [e for e in range(cfg["n_experts"]) if e not in ref[name_]]
        assert all(not got[e].any() for e in unchosen), name_
    rep["unchosen_experts"] = cfg["n_experts"] - len(chosen)
    print(f"[backward] {name}: " + json.dumps(rep), flush=True)
    return g


def test_backward_small_128_row_tiles():
    """T=300, H=512, I=256: about 9 rows per expert, 128-row tiles, ragged;
    some experts unchosen."""
    _full_compare("small", _case(300, 512, 256), 31)


def test_backward_256_row_tiles():
    """About 100 rows per expert: 256-row tiles with partly live waves and
    experts whose rows cross several 32-row segments."""
    _full_compare("256 rows", _case(3200, 256, 256), 32)


def test_backward_single_token_and_empty():
    """T=1 (eight experts with one row each, the rest zero) and T=0."""
    _full_compare("T=1", _case(1, 256, 256), 34)
    dev = _dev()
    cfg = _case(1, 256, 256)
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, 34))
    pw = _packed(workloads.make_expert_weights(cfg, 34, dev))
    g = _run(cfg, x[:0], rw, b, pw, torch.empty((0, 256), dtype=torch.bfloat16, device=dev))
    assert g["dx"].shape == (0, 256)


def test_backward_without_weight_grads_matches():
    dev = _dev()
    cfg = _case(200, 512, 512)
    x, rw, b = workloads.make_small_inputs(cfg, 33)
    x, rw, b = x.to(dev), rw.to(dev), b.to(dev)
    dout = workloads.normal((200, 512), 1.0, 33, "dout").to(torch.bfloat16).to(dev)
    pw = _packed(workloads.make_expert_weights(cfg, 33, dev))
    g1 = _run(cfg, x, rw, b, pw, dout, weight_grads=True)
    g2 = _run(cfg, x, rw, b, pw, dout, weight_grads=False)
    g3 = _run(cfg, x, rw, b, pw, dout, weight_grads=True)
    assert g2["d_w_gate"] is None
    assert torch.equal(g1["dx"], g2["dx"]) and torch.equal(g1["d_router_w"], g2["d_router_w"])
    for k in ("dx", "d_router_w", "d_w_gate", "d_w_up", "d_w_down"):
        assert torch.equal(g1[k], g3[k]), k  # deterministic


def test_pack_weights_transposed_matches_definition():
    dev = _dev()
    w = workloads.normal((3, 256, 192), 1.0, 0, "pack_t").to(torch.bfloat16).to(dev)
    got = gl.pack_weights_transposed(w)
    ref = gl.pack_weights(w.transpose(1, 2).contiguous())
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_update_bias_matches_oracle():
    dev = _dev()
    rng = np.random.default_rng(5)
    b = rng.normal(size=256).astype(np.float32) * 0.01
    counts = rng.integers(0, 300, size=256).astype(np.int32)
    counts[:3] = int(np.round(counts.mean()))  # likely near the mean
    counts[3] = 0
    bt = torch.tensor(b, device=dev)
    gl.update_bias(bt, torch.tensor(counts, device=dev), 1e-3)
    torch.cuda.synchronize()
    ref = oracle.backward.bias_step(b.astype(np.float64), counts, np.float64(np.float32(1e-3)))
    np.testing.assert_array_equal(bt.cpu().numpy(), ref.astype(np.float32))
    # balanced load: no change
    bt2 = torch.tensor(b, device=dev)
    gl.update_bias(bt2, torch.full((256,), 7, dtype=torch.int32, device=dev), 0.5)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bt2.cpu().numpy(), b)


def test_backward_prefill_full_shape():
    """Beam's prefill shape (T=4096, H=5120, I=2560, balanced bias): dx on
    a token set that holds the first, the last and a random row of every
    M-tile of every expert (the oracle with all their experts), and the
    complete weight gradients of eight experts (the busiest, the least busy
    and six spread over the groups; the oracle runs only those experts,
    whose weight gradients need no other expert)."""
    dev = _dev()
    cfg = workloads.workload("prefill")
    x, rw, b = workloads.make_small_inputs(cfg, 0)
    x, rw, b = x.to(dev), rw.to(dev), b.to(dev)
    dout = workloads.normal((cfg["T"], cfg["hidden"]), 1.0, 0, "dout").to(torch.bfloat16).to(dev)
    w = workloads.make_expert_weights(cfg, 0, dev)
    pw = _packed(w)
    print("\n[backward] prefill full shape: T=4096", flush=True)
    g = _run(cfg, x, rw, b, pw, dout)
    del pw
    torch.cuda.empty_cache()
    rep = {"T": cfg["T"]}
    idx, r = _routing(cfg, x, rw, b, rep)
    E = cfg["n_experts"]
    x64 = x.cpu().double().numpy()
    rw64 = rw.cpu().double().numpy()
    b64 = b.cpu().double().numpy()
    d64 = dout.cpu().double().numpy()
    gidx = r["topk_idx"].cpu().numpy()
    toks = tile_cover(gidx, E, 128, seed=7)
    cov = coverage_report(toks, gidx, E)
    rep.update(cov)
    for bm in (128, 256):
        assert cov[f"tiles_covered_{bm}"] == cov[f"tiles_total_{bm}"], cov
    rep["dx_tokens"] = int(len(toks))
    ref = oracle.backward.backward(x64[toks], rw64, b64, expert_getter(w), d64[toks], 8, 4, 8, 2.5,
                                   routing=idx[toks], weight_grads=False)
    check_grad("dx", g["dx"][torch.as_tensor(toks, device=dev)].cpu().double().numpy(), ref["dx"], rep)
    cnt = r["expert_counts"].cpu().numpy()
    live = np.nonzero(cnt)[0]
    experts = sorted({int(cnt.argmax()), int(live[np.argmin(cnt[live])]), 0, 37, 77, 130, 201, 255})
    tk = np.nonzero(np.any(np.isin(idx, experts), axis=1))[0]
    refe = oracle.backward.backward(x64[tk], rw64, b64, expert_getter(w), d64[tk], 8, 4, 8, 2.5,
                                    routing=idx[tk], only_experts=set(experts))
    for name_ in ("d_w_gate", "d_w_up", "d_w_down"):
        got = np.concatenate([g[name_][e].cpu().double().numpy() for e in experts])
        check_grad(name_, got, np.concatenate([refe[name_][e] for e in experts]), rep)
    rep["weight_grad_experts"] = {int(e): int(cnt[e]) for e in experts}
    print("[backward] prefill full shape: " + json.dumps(rep), flush=True)
    del w, g
    torch.cuda.empty_cache()

"""GPU parity of one expert shard's share of the block (beam_moe_forward_shard),
the compute that expert parallelism puts on each device: every shard's
partial output against the oracle run with only that shard's experts (the
others' weights zero), and the sum over a partition of the experts ("fake
expert parallelism" on one GPU) against the oracle's full block.
"""

import json

import numpy as np
import pytest
import torch

import oracle
import workloads
import group_limited_routing_amd as gl
from parity import (check_outputs, check_routing, expert_getter, guarded_out, guarded_workspace,
                    oracle_reference, packed_copy, run_forward)

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(T, H, I, w_dtype="bf16", x_dtype="bf16"):
    cfg = dict(workloads.BEAM)
    cfg.update(T=T, hidden=H, intermediate=I, x_dtype=x_dtype, w_dtype=w_dtype, bias="normal")
    return cfg


def _slice(w, e0, e1):
    """The shard's weights (and scales): experts e0 .. e1 - 1, contiguous."""
    out = {k: v[e0:e1].contiguous() for k, v in w.items() if torch.is_tensor(v)}
    if "packed" in w:
        out["packed"] = w["packed"]
    return out


def _shard_forward(x, rw, b, w, cfg, e0, e1):
    sw = _slice(w, e0, e1)
    scales = None
    if sw["w_gate"].dtype in (torch.float8_e4m3fn, torch.uint8):
        scales = (sw["w_gate_scale"], sw["w_up_scale"], sw["w_down_scale"])
    ws = guarded_workspace(x, sw, cfg)
    og, out = guarded_out(x)
    out, r = gl.forward_shard(x, rw, b, e0, e1, sw["w_gate"], sw["w_up"], sw["w_down"],
                              scales=scales, packed=sw.get("packed", False),
                              n_group=cfg["n_group"], topk_group=cfg["topk_group"],
                              top_k=cfg["top_k"],
                              routed_scaling_factor=cfg["routed_scaling_factor"],
                              return_routing=True, workspace=ws.view, out=out)
    torch.cuda.synchronize()
    ws.check()
    og.check()
    return out, r


def _restricted_getter(w, e0, e1):
    """The oracle's experts with every expert outside [e0, e1) zeroed."""
    get = expert_getter(w)
    cache = {}

    def g(e):
        if e0 <= e < e1:
            return get(e)
        if "zero" not in cache:
            cache["zero"] = tuple(np.zeros_like(m) for m in get(e0))
        return cache["zero"]
    return g


def _run(name, cfg, seed, bounds, packed, tokens=None):
    dev = _dev()
    print(f"\n[shard] {name}: T={cfg['T']} shards {bounds}", flush=True)
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, seed))
    w = workloads.make_expert_weights(cfg, seed, dev)
    gw = packed_copy(w) if packed else w
    _, r = run_forward(x, rw, b, gw, cfg)
    x64, rw64, b64 = (t.cpu().double().numpy() for t in (x, rw, b))
    ora = oracle.route(x64, rw64, b64, cfg["n_group"], cfg["topk_group"], cfg["top_k"])
    rep = {"T": cfg["T"], "shards": len(bounds) - 1}
    near = check_routing(r, ora, cfg, rep)
    idx = r["topk_idx"].cpu().numpy()
    toks = np.arange(cfg["T"]) if tokens is None else tokens
    fp8 = cfg["w_dtype"] in ("fp8", "mxfp4")
    total = torch.zeros((cfg["T"], cfg["hidden"]), dtype=torch.float64)
    for e0, e1 in zip(bounds[:-1], bounds[1:]):
        part, rs = _shard_forward(x, rw, b, gw, cfg, e0, e1)
        for k in ("topk_idx", "topk_w", "expert_counts"):
            assert torch.equal(rs[k], r[k]), k
        # tokens with no expert in the shard get exact zeros
        none = ~np.any((idx >= e0) & (idx < e1), axis=1)
        assert not part[torch.as_tensor(np.nonzero(none)[0], device=dev)].any()
        total += part.cpu().double()
        sel = np.array([t for t in toks if not none[t]])
        forced = ora["idx"].copy()
        forced[near] = idx[near]
        ref, _ = oracle.forward(x64[sel], rw64, b64, _restricted_getter(w, e0, e1),
                                cfg["n_group"], cfg["topk_group"], cfg["top_k"],
                                cfg["routed_scaling_factor"], routing=forced[sel], fp8=fp8)
        check_outputs(part[torch.as_tensor(sel, device=dev)].cpu().double().numpy(), ref, rep,
                      f"shard{e0}_")
    ref_full = oracle_reference(toks, x, rw, b, w, cfg, idx, near)
    check_outputs(total.numpy()[toks], ref_full, rep, "sum_")
    print(f"[shard] {name}: " + json.dumps(rep), flush=True)


def test_shards_bf16_eight_way():
    _run("bf16 8 shards", _case(300, 512, 256), 41, list(range(0, 257, 32)), packed=False)


def test_shards_bf16_packed_decode_batch():
    """Eight shards of 32 experts at a decode-sized batch (about 6 rows per
    expert): 16-row streaming tiles with 2 fragments per wave and the deeper
    register ring that narrow waves take."""
    _run("bf16 packed decode batch", _case(200, 1024, 512), 45, list(range(0, 257, 32)), packed=True)


def test_shards_bf16_packed_uneven():
    _run("bf16 packed uneven", _case(1000, 512, 256), 42, [0, 1, 100, 255, 256], packed=True)


def test_shards_fp8_packed():
    _run("fp8 packed 4 shards", _case(200, 512, 256, "fp8"), 43, [0, 64, 128, 192, 256], packed=True)


def test_shards_mxfp4():
    _run("mxfp4 2 shards", _case(64, 512, 512, "mxfp4"), 44, [0, 128, 256], packed=True)


def test_shard_decode_eight_gpus_full_shape():
    """One of 8 shards at Beam's shape for 8 GPUs x 64 decode tokens (T=512
    routed tokens, experts 0-31), packed bf16 weights: the shard's partial
    output on every token with an expert in the shard against the oracle
    with that shard's experts, and exact zeros on the other tokens."""
    dev = _dev()
    cfg = dict(workloads.workload("decode"), T=512)
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, 0))
    w = workloads.make_expert_weights(cfg, 0, dev, experts=range(32))
    pw = packed_copy(_slice(w, 0, 32))
    sw = dict(pw)
    print("\n[shard] decode 8 GPUs: T=512 experts 0-31", flush=True)
    part, r = gl.forward_shard(x, rw, b, 0, 32, sw["w_gate"], sw["w_up"], sw["w_down"],
                               packed=True, return_routing=True)
    torch.cuda.synchronize()
    idx = r["topk_idx"].cpu().numpy()
    x64, rw64, b64 = (t.cpu().double().numpy() for t in (x, rw, b))
    ora = oracle.route(x64, rw64, b64)
    rep = {"T": 512}
    near = check_routing(r, ora, cfg, rep)
    forced = ora["idx"].copy()
    forced[near] = idx[near]
    hit = np.nonzero(np.any(idx < 32, axis=1))[0]
    miss = np.nonzero(~np.any(idx < 32, axis=1))[0]
    if len(miss):
        assert not part[torch.as_tensor(miss, device=dev)].any()
    ref, _ = oracle.forward(x64[hit], rw64, b64, _restricted_getter(w, 0, 32), 8, 4, 8, 2.5,
                            routing=forced[hit])
    check_outputs(part[torch.as_tensor(hit, device=dev)].cpu().double().numpy(), ref, rep)
    rep["tokens_with_shard_experts"] = int(len(hit))
    print("[shard] decode 8 GPUs: " + json.dumps(rep), flush=True)
    del w, pw, sw
    torch.cuda.empty_cache()

"""GPU parity: the HIP path (through the C ABI) against the oracle.

Small shapes are compared on every token; they span several M-tiles and
column tiles and have ragged tails (T, rows per expert and tiles not
multiples of the tile sizes), and they exercise both expert-GEMM variants
(weight streaming for few rows per expert, LDS tiles for many) and both
weight formats. The named Beam workloads (decode T=64, prefill T=4096,
skewed T=16384, fp8 T=8192, MXFP4 T=64 and T=4096) run at full size in the
same launch configuration the benchmark times: routing is compared on every
token, and the outputs on every token at decode and, above that, on a set of
tokens that holds the first, the last and a random row of every M-tile of
every expert (tiles of 128 sorted rows, which also covers every 256-row
tile), which the oracle computes one expert at a time. Each report prints
the covered and total tile counts, and the test asserts they are equal.
"""

import json

import numpy as np
import pytest
import torch

import oracle
import workloads
import group_limited_routing_amd as gl
from parity import (check_logits, check_outputs, check_routing, coverage_report, oracle_reference,
                    run_forward, output_errors, packed_copy, tile_cover)

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _case(T, H, I, x_dtype="bf16", w_dtype="bf16", bias="normal", seed=0, **routing):
    cfg = dict(workloads.BEAM)
    cfg.update(T=T, hidden=H, intermediate=I, x_dtype=x_dtype, w_dtype=w_dtype, bias=bias)
    cfg.update(routing)
    return cfg


def _inputs(cfg, seed, dev, experts=None):
    x, rw, b = workloads.make_small_inputs(cfg, seed)
    w = workloads.make_expert_weights(cfg, seed, dev, experts=experts)
    return x.to(dev), rw.to(dev), b.to(dev), w


def _report(name, rep):
    print(f"\n[parity] {name}: " + json.dumps(rep), flush=True)


def _full_compare(name, cfg, seed=0, packed=False):
    """Every token against the oracle (the oracle always reads the row-major
    weights; the GPU optionally their packed copy)."""
    dev = _dev()
    x, rw, b, w = _inputs(cfg, seed, dev)
    out, r = run_forward(x, rw, b, packed_copy(w) if packed else w, cfg)
    x64 = x.cpu().double().numpy()
    rw64 = rw.cpu().double().numpy()
    ora = oracle.route(x64, rw64, b.cpu().double().numpy(), cfg["n_group"], cfg["topk_group"],
                       cfg["top_k"])
    rep = {"T": cfg["T"], "H": cfg["hidden"], "I": cfg["intermediate"]}
    near = check_routing(r, ora, cfg, rep)
    check_logits(r["router_logits"], x64, rw64, ora["z"])
    tokens = np.arange(cfg["T"])
    ref = oracle_reference(tokens, x, rw, b, w, cfg, r["topk_idx"].cpu().numpy(), near)
    check_outputs(out.cpu().double().numpy(), ref, rep)
    _report(name, rep)
    return out, r


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_workload(seed):
    """T=128, H=256, I=128, x and out fp32, bf16 experts."""
    cfg = workloads.workload("tiny")
    _full_compare(f"tiny seed {seed}", cfg, seed)


LAYOUTS = [pytest.param(False, id="rowmajor"), pytest.param(True, id="packed")]


@pytest.mark.parametrize("packed", LAYOUTS)
def test_ragged_stream_variant(packed):
    cfg = _case(300, 384, 256)          # 2400 pairs: streaming GEMMs; H % 256 != 0
    _full_compare("ragged stream", cfg, 3, packed)


@pytest.mark.parametrize("packed", LAYOUTS)
def test_stream_variant_wide(packed):
    cfg = _case(150, 1024, 512)         # widths that take the 8-fragment waves
    _full_compare("stream wide", cfg, 13, packed)


# Between 8 and 16 rows per expert on average the streaming variants take
# 32-row M-tiles (two row blocks per weight fragment): experts of 17-32 rows
# in one tile, hot experts over many tiles with a ragged last one.
@pytest.mark.parametrize("name,T,H,I,x_dtype,w_dtype,bias,packed", [
    ("bf16 wide", 450, 1024, 512, "bf16", "bf16", "normal", False),
    ("bf16 packed hot", 400, 512, 256, "bf16", "bf16", "hot", True),
    ("fp32 x", 400, 256, 128, "f32", "bf16", "normal", True),
    ("fp8 rowmajor", 400, 512, 256, "bf16", "fp8", "normal", False),
    ("fp8 rowmajor hot", 400, 512, 256, "bf16", "fp8", "hot", False),
    ("mxfp4", 350, 512, 1024, "bf16", "mxfp4", "normal", True),
    ("mxfp4 hot", 370, 1024, 512, "bf16", "mxfp4", "hot", True),
])
def test_stream_variant_two_row_blocks(name, T, H, I, x_dtype, w_dtype, bias, packed):
    cfg = _case(T, H, I, x_dtype=x_dtype, w_dtype=w_dtype, bias=bias)
    assert 8 * 256 < T * 8 <= (12 if w_dtype == "mxfp4" else 16) * 256
    out, r = _full_compare("stream 32-row " + name, cfg, 31, packed)
    cnt = r["expert_counts"].cpu().numpy()
    assert (cnt > 16).sum() >= 4  # experts that a 16-row tile list splits
    if bias == "hot":
        assert cnt[:8].min() > 4 * 32  # hot experts span several 32-row tiles


@pytest.mark.parametrize("packed", LAYOUTS)
def test_ragged_tiled_variant(packed):
    cfg = _case(1000, 512, 384)         # 8000 pairs: LDS-tiled GEMMs, ragged tiles
    _full_compare("ragged tiled", cfg, 4, packed)


@pytest.mark.parametrize("packed", LAYOUTS)
def test_fp32_x_tiled_variant(packed):
    cfg = _case(700, 256, 128, x_dtype="f32")
    _full_compare("fp32 x tiled", cfg, 5, packed)


def test_wide_variant_256_rows():
    cfg = _case(6500, 256, 256)         # ~203 rows per expert: 256-row tiles, ragged
    _full_compare("wide 256", cfg, 14, True)


@pytest.mark.parametrize("packed", LAYOUTS)
def test_fp8_stream_variant(packed):
    # row-major fp8 weights stream; packed ones take the DMA variant at any batch
    cfg = _case(200, 512, 256, w_dtype="fp8")
    _full_compare("fp8 stream", cfg, 6, packed)


@pytest.mark.parametrize("T", [1, 64, 500])
def test_fp8_packed_decode_batches_take_the_dma_variant(T):
    """Packed fp8 weights never stream: one to a few rows per expert in
    128-row DMA tiles (most of each tile's rows absent)."""
    cfg = _case(T, 512, 256, w_dtype="fp8")
    _full_compare(f"fp8 packed T={T}", cfg, 37, True)


@pytest.mark.parametrize("packed", LAYOUTS)
def test_fp8_tiled_variant(packed):
    cfg = _case(900, 384, 256, w_dtype="fp8")
    _full_compare("fp8 tiled", cfg, 7, packed)


def test_dma_variant_short_reduction():
    # hidden 128: the gate/up reduction is 4 steps, shorter than the distance
    # at which the next tile's first stages are loaded
    cfg = _case(3000, 128, 256)
    _full_compare("dma short K", cfg, 17, True)


def test_fp8_dma_variant_128_rows():
    cfg = _case(1000, 512, 256, w_dtype="fp8")   # ~31 rows per expert; down N = 512
    _full_compare("fp8 dma 128", cfg, 15, True)


def test_fp8_dma_variant_256_rows():
    # ~100 rows per expert: 256-row tiles with partly live waves; the down
    # pass has K = 128 (one fp8 step, shorter than the load-ahead distance)
    cfg = _case(3200, 512, 128, w_dtype="fp8")
    _full_compare("fp8 dma 256", cfg, 16, True)


def test_fp8_mixed_tile_heights():
    # about 256 rows per expert (as at the fp8 workload's T = 8192): experts
    # beyond 256 rows run 512-row tiles, the others 256-row tiles, in one launch
    cfg = _case(8192, 256, 256, w_dtype="fp8")
    out, r = _full_compare("fp8 mixed tiles", cfg, 27, True)
    cnt = r["expert_counts"].cpu().numpy()
    assert (cnt > 256).sum() >= 32 and (cnt <= 256).sum() >= 32, cnt


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_hidden_not_a_multiple_of_256_at_many_rows(w_dtype):
    # packed weights, about 100 rows per expert, hidden 384: the down pass
    # runs the 128-row tiled kernel (256-column tiles do not divide 384), so
    # the shared tile list must hold 128-row tiles for both passes
    cfg = _case(3200, 384, 256, w_dtype=w_dtype)
    _full_compare(f"hidden 384 packed {w_dtype}", cfg, 28, True)


@pytest.mark.parametrize("T", [255, 256, 257, 512])
def test_routing_paths_at_the_single_chunk_boundary(T):
    # up to 256 tokens: split-K fp32 router logits and the one-launch
    # permutation; from 257: the split-weight bf16 router and per-chunk
    # histogram, scan and scatter
    cfg = _case(T, 512, 256)
    _full_compare(f"boundary T={T}", cfg, 23, True)


def test_mxfp4_stream_variant():
    cfg = _case(200, 512, 1024, w_dtype="mxfp4")   # ragged M-tiles, 4-bit weights
    _full_compare("mxfp4 stream", cfg, 18, True)


def test_mxfp4_dma_variant_128_rows():
    # ~47 rows per expert: the MXFP4 DMA variant with 128-row tiles
    cfg = _case(1500, 1024, 512, w_dtype="mxfp4")
    _full_compare("mxfp4 dma 128", cfg, 19, True)


def test_mxfp4_dma_variant_256_rows():
    # ~100 rows per expert: 256-row tiles, partly live waves, 4 scale groups
    cfg = _case(3200, 512, 512, w_dtype="mxfp4")
    _full_compare("mxfp4 dma 256", cfg, 20, True)


def test_mxfp4_pack_layouts():
    """Packed MXFP4 codes and scale bytes equal their documented layouts,
    built here with torch views (an independent formulation)."""
    dev = _dev()
    E, R, C = 2, 32, 1024
    g = torch.Generator(device=dev).manual_seed(3)
    codes = torch.randint(0, 256, (E, R, C // 2), generator=g, device=dev, dtype=torch.uint8)
    sc = torch.randint(0, 256, (E, R, C // 32), generator=g, device=dev, dtype=torch.uint8)
    pc, ps = gl.pack_weights(codes), gl.pack_mx_scales(sc)
    torch.cuda.synchronize()
    # codes: 128 weights (64 bytes) per row per step, lane l = r % 16 + 16 * (chunk of 16 bytes)
    ref = codes.view(E, R // 16, 16, C // 128, 4, 16).permute(0, 1, 3, 4, 2, 5).contiguous()
    assert torch.equal(pc.view(-1), ref.view(-1))
    # scales: block b of row r -> ((r/16)*(C/512) + b/16)*256 + (r%16 + 16*(b%4))*4 + (b%16)/4
    ref = sc.view(E, R // 16, 16, C // 512, 4, 4).permute(0, 1, 3, 5, 2, 4).contiguous()
    assert torch.equal(ps.view(-1), ref.view(-1))


@pytest.mark.parametrize("dtype,S", [(torch.bfloat16, 32), (torch.float8_e4m3fn, 128)])
def test_pack_layout_matches_definition(dtype, S):
    """The packed copy equals the documented layout, built here with a torch
    view/permute of the row-major tensor (an independent formulation)."""
    dev = _dev()
    E, R, C = 3, 48, 384
    g = torch.Generator(device=dev).manual_seed(1)
    w = torch.randn((E, R, C), generator=g, device=dev).to(dtype)
    p = gl.pack_weights(w)
    torch.cuda.synchronize()
    L = S // 4
    ref = w.view(torch.uint8 if dtype != torch.bfloat16 else torch.int16)
    ref = ref.view(E, R // 16, 16, C // S, 4, L).permute(0, 1, 3, 4, 2, 5).contiguous().view(E, R, C)
    got = p.view(ref.dtype)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("n_group,topk_group,top_k", [(1, 1, 8), (8, 8, 8), (64, 16, 8), (8, 4, 1),
                                                      (16, 3, 12), (4, 2, 32)])
def test_group_parameters(n_group, topk_group, top_k):
    cfg = _case(260, 256, 128, n_group=n_group, topk_group=topk_group, top_k=top_k)
    _full_compare(f"groups {n_group}/{topk_group}/{top_k}", cfg, 8)


def test_all_keys_equal_tie_rule():
    """Router weight 0 and bias 0: every key is 0.5, so every token takes
    experts 0..7 (groups 0..3, lower index first) with weight 1/8."""
    dev = _dev()
    cfg = _case(50, 256, 128)
    x, rw, b, w = _inputs(cfg, 9, dev)
    rw.zero_()
    b.zero_()
    out, r = run_forward(x, rw, b, w, cfg)
    idx = r["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, np.tile(np.arange(8), (50, 1)))
    assert torch.all(r["topk_w"] == 0.125)
    cnt = r["expert_counts"].cpu().numpy()
    assert cnt[:8].tolist() == [50] * 8 and cnt[8:].sum() == 0


@pytest.mark.parametrize("T", [64, 300])
@pytest.mark.parametrize("dup", ["same_lane", "next_lane", "other_group"])
def test_exact_ties_go_to_the_lower_index(T, dup):
    """Experts with identical router rows and biases have identical keys, on
    the GPU as in the oracle: pairs inside one lane's four experts (2i, 2i+1),
    in neighbouring lanes of a group (8g + i, 8g + 4 + i), or in different
    groups (e, e + 128, which also ties the group scores). Every tie goes to
    the lower index, so the GPU's experts equal the oracle's on every token.
    The seed leaves no near tie between different keys."""
    dev = _dev()
    cfg = _case(T, 256, 128)
    x, rw, b, w = _inputs(cfg, 24, dev)
    e = torch.arange(256, device=dev)
    src = {"same_lane": e // 2, "next_lane": (e // 8) * 4 + e % 4, "other_group": e % 128}[dup]
    rw = rw[src].contiguous()
    b = b[src].contiguous()
    out, r = run_forward(x, rw, b, w, cfg)
    ora = oracle.route(x.cpu().double().numpy(), rw.cpu().double().numpy(),
                       b.cpu().double().numpy(), cfg["n_group"], cfg["topk_group"], cfg["top_k"])
    idx = r["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, ora["idx"])
    np.testing.assert_allclose(r["topk_w"].cpu().numpy(), ora["w"], rtol=1e-5, atol=1e-6)
    # the ties are real: some token chose both members of a duplicated pair
    assert any(len(set(src[torch.as_tensor(row, device=dev)].tolist())) < 8 for row in idx)


def test_route_entry_point_matches_forward():
    dev = _dev()
    cfg = _case(333, 512, 128)
    x, rw, b, w = _inputs(cfg, 10, dev)
    out, r = run_forward(x, rw, b, w, cfg)
    rr = gl.route(x, rw, b, return_logits=True, return_counts=True)
    torch.cuda.synchronize()
    assert torch.equal(rr["topk_idx"], r["topk_idx"])
    assert torch.equal(rr["topk_w"], r["topk_w"])
    assert torch.equal(rr["router_logits"], r["router_logits"])
    assert torch.equal(rr["expert_counts"], r["expert_counts"])


def test_deterministic_and_token_permutation():
    dev = _dev()
    cfg = _case(600, 256, 128)
    x, rw, b, w = _inputs(cfg, 11, dev)
    o1, r1 = run_forward(x, rw, b, w, cfg)
    o2, r2 = run_forward(x, rw, b, w, cfg)
    assert torch.equal(o1, o2) and torch.equal(r1["topk_idx"], r2["topk_idx"])
    perm = torch.randperm(600, generator=torch.Generator().manual_seed(0)).to(dev)
    o3, r3 = run_forward(x[perm].contiguous(), rw, b, w, cfg)
    assert torch.equal(r3["topk_idx"], r1["topk_idx"][perm])
    assert torch.equal(o3, o1[perm])


def test_single_token_and_empty():
    dev = _dev()
    cfg = _case(1, 256, 128)
    _full_compare("T=1", cfg, 12)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    xs, rw, b, w = _inputs(cfg, 12, dev)
    out = gl.forward(x, rw, b, w["w_gate"], w["w_up"], w["w_down"])
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


# ------------------------------------------------- many M-tiles per expert, every token
@pytest.mark.parametrize("w_dtype,I,packed", [("bf16", 256, False), ("bf16", 256, True),
                                              ("fp8", 256, False), ("fp8", 256, True),
                                              ("mxfp4", 512, True)])
def test_hot_experts_span_many_mtiles(w_dtype, I, packed):
    """The skewed routing (+0.5 bias on experts 0..7, all in group 0) at a
    small width: each hot expert gets about two thirds of the 4000 tokens,
    so its rows span 11 M-tiles of 256 (22 of 128). The tile order then runs
    several full blocks of M-tiles and a partial last block per expert, and
    every token's output is compared with the oracle."""
    cfg = _case(4000, 512, I, w_dtype=w_dtype, bias="hot")
    out, r = _full_compare(f"hot experts {w_dtype} I={I}" + (" packed" if packed else ""), cfg,
                           25, packed)
    cnt = r["expert_counts"].cpu().numpy()
    assert cnt[:8].min() >= 9 * 256, cnt[:8]


# ---------------------------------------------------------------- full Beam shape
@pytest.fixture(scope="module")
def beam_bf16_weights():
    dev = _dev()
    cfg = workloads.workload("decode")
    w = workloads.make_expert_weights(cfg, 0, dev)
    torch.cuda.synchronize()
    yield w
    del w
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def beam_bf16_packed(beam_bf16_weights):
    pw = packed_copy(beam_bf16_weights)
    torch.cuda.synchronize()
    yield pw
    del pw
    torch.cuda.empty_cache()


def _full_shape(name, wl, variants, oracle_weights, extra=None, all_tokens=False):
    """Run the workload's forward once per weight variant (label, weights):
    routing compared on every token (and equal across the variants); the
    outputs of every variant on the compared tokens against one oracle pass
    (all tokens, or a set covering every M-tile of every expert)."""
    dev = _dev()
    cfg = workloads.workload(wl)
    T, E = cfg["T"], cfg["n_experts"]
    print(f"\n[parity] {name}: T={T} variants {[v[0] for v in variants]}", flush=True)
    x, rw, b = workloads.make_small_inputs(cfg, 0)
    x, rw, b = x.to(dev), rw.to(dev), b.to(dev)
    runs = []
    for label, w in variants:
        out, r = run_forward(x, rw, b, w, cfg)
        runs.append((label, out, r))
    r0 = runs[0][2]
    for label, _, r in runs[1:]:
        for k in ("topk_idx", "topk_w", "expert_counts", "router_logits"):
            assert torch.equal(r[k], r0[k]), (label, k)
    x64 = x.cpu().double().numpy()
    rw64 = rw.cpu().double().numpy()
    ora = oracle.route(x64, rw64, b.cpu().double().numpy(), cfg["n_group"], cfg["topk_group"],
                       cfg["top_k"])
    rep = {"T": T}
    near = check_routing(r0, ora, cfg, rep)
    gidx = r0["topk_idx"].cpu().numpy()
    cnt = r0["expert_counts"].cpu().numpy()
    rep["active_experts"] = int((cnt > 0).sum())
    rep["max_over_mean"] = float(cnt.max() / cnt.mean())
    if all_tokens:
        tokens = np.arange(T)
    else:
        tokens = np.union1d(tile_cover(gidx, E, 128, seed=T), np.nonzero(near)[0])
    cov = coverage_report(tokens, gidx, E)
    rep.update(cov)
    for bm in (128, 256):
        assert cov[f"tiles_covered_{bm}"] == cov[f"tiles_total_{bm}"], cov
    rep["compared_tokens"] = int(len(tokens))
    ref = oracle_reference(tokens, x, rw, b, oracle_weights, cfg, gidx, near)
    sel = torch.as_tensor(tokens, device=dev)
    for label, out, _ in runs:
        check_outputs(out[sel].cpu().double().numpy(), ref, rep, label + "_")
    if extra:
        extra(rep, cnt)
    _report(name, rep)


def test_beam_decode_full_shape(beam_bf16_weights, beam_bf16_packed):
    """T=64: every token, row-major and packed weights."""
    _full_shape("decode T=64", "decode",
                [("rowmajor", beam_bf16_weights), ("packed", beam_bf16_packed)],
                beam_bf16_weights, all_tokens=True)


def test_beam_prefill_full_shape(beam_bf16_weights, beam_bf16_packed):
    def balanced(rep, cnt):
        assert rep["max_over_mean"] <= 1.05
    _full_shape("prefill T=4096", "prefill",
                [("rowmajor", beam_bf16_weights), ("packed", beam_bf16_packed)],
                beam_bf16_weights, balanced)


def test_beam_skewed_full_shape(beam_bf16_weights, beam_bf16_packed):
    def skewed(rep, cnt):
        assert cnt[:8].min() >= 4 * cnt.mean()   # the +0.5 bias makes experts 0-7 hot
        assert int(cnt.sum()) == 8 * 16384
    _full_shape("skewed T=16384", "skewed",
                [("rowmajor", beam_bf16_weights), ("packed", beam_bf16_packed)],
                beam_bf16_weights, skewed)


def test_beam_mxfp4_decode_full_shape():
    dev = _dev()
    cfg = workloads.workload("mxfp4")
    w = workloads.make_expert_weights(cfg, 0, dev)
    pw = packed_copy(w)
    torch.cuda.synchronize()
    try:
        _full_shape("mxfp4 decode T=64", "mxfp4", [("packed", pw)], w, all_tokens=True)
    finally:
        del w, pw
        torch.cuda.empty_cache()


def test_beam_mxfp4_prefill_full_shape():
    dev = _dev()
    cfg = workloads.workload("mxfp4_prefill")
    w = workloads.make_expert_weights(cfg, 0, dev)
    pw = packed_copy(w)
    torch.cuda.synchronize()
    try:
        _full_shape("mxfp4 prefill T=4096", "mxfp4_prefill", [("packed", pw)], w)
    finally:
        del w, pw
        torch.cuda.empty_cache()


def test_beam_fp8_full_shape():
    dev = _dev()
    cfg = workloads.workload("fp8")
    w8 = workloads.make_expert_weights(cfg, 0, dev)
    pw8 = packed_copy(w8)
    torch.cuda.synchronize()
    try:
        _full_shape("fp8 T=8192", "fp8", [("rowmajor", w8), ("packed", pw8)], w8)
    finally:
        del w8, pw8
        torch.cuda.empty_cache()

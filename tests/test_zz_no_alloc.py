"""beam_moe_forward_noalloc (the library's static per-GPU scratch instead of a
workspace) against beam_moe_forward (a caller's workspace) through the C ABI:
the same kernels, so outputs and routing must be equal bit for bit. Two
calls in a row, the second with fewer tokens, so the second runs on scratch
that still holds the first call's contents. Then the largest batch the
scratch holds at Beam's decode shape. Output buffers are filled with NaN
before each call, so nothing stale can pass."""

import pytest
import torch

import workloads
import group_limited_routing_amd as gl
from parity import packed_copy

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def _scales(w):
    if w["w_gate"].dtype in (torch.float8_e4m3fn, torch.uint8):
        return (w["w_gate_scale"], w["w_up_scale"], w["w_down_scale"])
    return None


def _compare(x, rw, b, w, T):
    """One beam_moe_forward and one beam_moe_forward_noalloc on the first T tokens."""
    dev = x.device
    xs = x[:T].contiguous()
    ref, r = gl.forward(xs, rw, b, w["w_gate"], w["w_up"], w["w_down"], scales=_scales(w),
                        packed=w.get("packed", False), return_routing=True, return_logits=True)
    E = rw.shape[0]
    out = torch.full_like(xs, float("nan"))
    idx = torch.full((T, 8), -1, dtype=torch.int32, device=dev)
    tw = torch.full((T, 8), float("nan"), dtype=torch.float32, device=dev)
    cnt = torch.full((E,), -1, dtype=torch.int32, device=dev)
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device=dev)
    gl.forward_noalloc(xs, rw, b, w["w_gate"], w["w_up"], w["w_down"], out=out,
                       scales=_scales(w), packed=w.get("packed", False), topk_idx=idx, topk_w=tw,
                       expert_counts=cnt, router_logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(idx, r["topk_idx"]) and torch.equal(tw, r["topk_w"])
    assert torch.equal(cnt, r["expert_counts"]) and torch.equal(logits, r["router_logits"])


@pytest.mark.parametrize("w_dtype,I,packed", [("bf16", 256, False), ("bf16", 256, True),
                                              ("fp8", 256, True), ("mxfp4", 512, True)])
def test_noalloc_matches_forward_twice(w_dtype, I, packed):
    dev = _dev()
    cfg = dict(workloads.BEAM, T=300, hidden=512, intermediate=I, x_dtype="bf16",
               w_dtype=w_dtype, bias="normal")
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, 71))
    w = workloads.make_expert_weights(cfg, 71, dev)
    if packed:
        w = packed_copy(w)
    print(f"\n[noalloc] {w_dtype} I={I} packed={packed}: T=300 then T=37", flush=True)
    _compare(x, rw, b, w, 300)   # more than one permutation chunk
    _compare(x, rw, b, w, 37)    # fewer tokens on the scratch the first call left


def test_noalloc_largest_decode_batch_at_beam_shape():
    """T=256 at hidden 5120, intermediate 2560 (bf16 experts, packed): the
    largest batch the 64 MiB scratch holds; then T=64."""
    dev = _dev()
    cfg = workloads.workload("decode")
    cfg = dict(cfg, T=256)
    assert gl.workspace_bytes(gl.make_config(5120, 2560, packed=True), 256) <= gl.NOALLOC_MAX_BYTES
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, 0))
    w = packed_copy(workloads.make_expert_weights(cfg, 0, dev))
    print("\n[noalloc] decode shape: T=256 then T=64", flush=True)
    _compare(x, rw, b, w, 256)
    _compare(x, rw, b, w, 64)
    del w
    torch.cuda.empty_cache()

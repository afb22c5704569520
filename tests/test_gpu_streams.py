"""Calls on a side stream (``stream=``) with no workspace or outputs passed:
the binding allocates them from that stream's pool, so a block it frees on
return is not handed to work on another stream while the side stream's
kernels still use it. Between the calls the default stream allocates and
overwrites memory of the workspace's size; every result must still equal
the eager result on the default stream bit for bit (the kernels are
deterministic)."""

import pytest
import torch

import workloads
import group_limited_routing_amd as gl
from parity import packed_copy

pytestmark = pytest.mark.gpu


def _setup(T, seed):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    cfg = dict(workloads.BEAM, T=T, hidden=512, intermediate=256, x_dtype="bf16", w_dtype="bf16",
               bias="normal")
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, seed))
    w = workloads.make_expert_weights(cfg, seed, dev)
    return dev, cfg, x, rw, b, w


def _scribble(dev, nbytes):
    """Default-stream work that allocates and overwrites nbytes."""
    junk = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    junk.fill_(0xA5)
    return junk


def test_forward_on_side_stream_allocates_there():
    dev, cfg, x, rw, b, w = _setup(3000, 61)
    pw = packed_copy(w)
    c = gl.make_config(512, 256, x_dtype=torch.bfloat16, w_dtype=torch.bfloat16, packed=True)
    nbytes = gl.workspace_bytes(c, cfg["T"])
    eager = gl.forward(x, rw, b, pw["w_gate"], pw["w_up"], pw["w_down"], packed=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs, keep = [], []
    for _ in range(4):
        outs.append(gl.forward(x, rw, b, pw["w_gate"], pw["w_up"], pw["w_down"], packed=True,
                               stream=side))
        keep.append(_scribble(dev, nbytes))
    side.synchronize()
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, eager), f"call {i}"


def test_backward_on_side_stream_allocates_there():
    dev, cfg, x, rw, b, w = _setup(1000, 62)
    pw = {"w_gate": gl.pack_weights(w["w_gate"]), "w_up": gl.pack_weights(w["w_up"]),
          "w_gate_t": gl.pack_weights_transposed(w["w_gate"]),
          "w_up_t": gl.pack_weights_transposed(w["w_up"]),
          "w_down_t": gl.pack_weights_transposed(w["w_down"])}
    dout = workloads.normal((cfg["T"], 512), 1.0, 62, "dout").to(torch.bfloat16).to(dev)
    c = gl.make_config(512, 256, x_dtype=torch.bfloat16, w_dtype=torch.bfloat16, packed=True)
    nbytes = gl.backward_workspace_bytes(c, cfg["T"], True)

    def call(stream=None):
        return gl.backward(x, rw, b, pw["w_gate"], pw["w_up"], pw["w_gate_t"], pw["w_up_t"],
                           pw["w_down_t"], dout, weight_grads=True, stream=stream)

    eager = call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    res, keep = [], []
    for _ in range(3):
        res.append(call(side))
        keep.append(_scribble(dev, nbytes))
    side.synchronize()
    torch.cuda.synchronize()
    for i, g in enumerate(res):
        for k in ("dx", "d_router_w", "d_w_gate", "d_w_up", "d_w_down"):
            assert torch.equal(g[k], eager[k]), (i, k)

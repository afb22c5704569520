"""The forward pass captured in a HIP graph: the library allocates nothing,
synchronises nothing and issues no memset, so a caller can capture a whole
call (routing, permutation, GEMMs, combine) on its stream and replay it.
Every replay, with eager work and synchronisations in between, must equal
the eager result bit for bit (the kernels are deterministic)."""

import pytest
import torch

import workloads
import group_limited_routing_amd as gl
from parity import packed_copy

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T", [64, 1000])
def test_forward_replays_equal_eager(T):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    cfg = dict(workloads.BEAM, T=T, hidden=512, intermediate=256, x_dtype="bf16", w_dtype="bf16",
               bias="normal")
    x, rw, b = (t.to(dev) for t in workloads.make_small_inputs(cfg, 51))
    w = packed_copy(workloads.make_expert_weights(cfg, 51, dev))
    c = gl.make_config(512, 256, x_dtype=torch.bfloat16, w_dtype=torch.bfloat16, packed=True)
    ws = torch.empty(gl.workspace_bytes(c, T), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)

    def call():
        gl.forward(x, rw, b, w["w_gate"], w["w_up"], w["w_down"], packed=True, out=out,
                   workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(4):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)

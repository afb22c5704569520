"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments before any HIP call (so these run with
no GPU). Fake, never-dereferenced pointer values stand in for device memory.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")

gl = pytest.importorskip("group_limited_routing_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gl.LIB_PATH):
        pytest.skip("libbeam_moe.so not built")
    return gl.lib()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_moe_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert declared == sorted(gl.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(8):
        txt = gl.status_string(s)
        assert txt and txt != "unknown status"
    assert gl.status_string(99) == "unknown status"


FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _fwd(L, cfg, T, ptrs=None, ws_bytes=1 << 40, **over):
    p = dict(x=FAKE, rw=FAKE, b=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, sg=None, su=None, sd=None,
             out=FAKE, idx=None, w=None, cnt=None, logits=None, ws=FAKE)
    p.update(over)
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.beam_moe_forward(ctypes.byref(cfg) if cfg is not None else None, T, v(p["x"]),
                              v(p["rw"]), v(p["b"]), v(p["wg"]), v(p["wu"]), v(p["wd"]),
                              v(p["sg"]), v(p["su"]), v(p["sd"]), v(p["out"]), v(p["idx"]),
                              v(p["w"]), v(p["cnt"]), v(p["logits"]), v(p["ws"]), ws_bytes, None)


def _route(L, cfg, T, ws_bytes=1 << 40, **over):
    p = dict(x=FAKE, rw=FAKE, b=FAKE, idx=FAKE, w=FAKE, logits=None, cnt=None, ws=FAKE)
    p.update(over)
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.beam_moe_route(ctypes.byref(cfg), T, v(p["x"]), v(p["rw"]), v(p["b"]), v(p["idx"]),
                            v(p["w"]), v(p["logits"]), v(p["cnt"]), v(p["ws"]), ws_bytes, None)


def beam_cfg(**kw):
    c = gl.make_config(5120, 2560)
    for k, val in kw.items():
        setattr(c, k, val)
    return c


def test_config_checks(L):
    bad = [dict(n_experts=128), dict(n_group=3), dict(n_group=128), dict(n_group=0),
           dict(topk_group=0), dict(topk_group=9), dict(top_k=0), dict(top_k=33),
           dict(n_group=64, topk_group=1, top_k=5), dict(routed_scaling_factor=float("inf"))]
    for kw in bad:
        assert _fwd(L, beam_cfg(**kw), 8) == gl.BEAM_ERR_CONFIG, kw
        assert _route(L, beam_cfg(**kw), 8) == gl.BEAM_ERR_CONFIG, kw
    for kw in [dict(x_dtype=2), dict(x_dtype=7), dict(w_dtype=0)]:
        assert _fwd(L, beam_cfg(**kw), 8) == gl.BEAM_ERR_DTYPE, kw
    for kw in [dict(hidden=5000), dict(hidden=0), dict(intermediate=100), dict(hidden=65536 + 128)]:
        assert _fwd(L, beam_cfg(**kw), 8) == gl.BEAM_ERR_SHAPE, kw
    assert _fwd(L, None, 8) == gl.BEAM_ERR_NULL


def test_token_count_checks(L):
    c = beam_cfg()
    assert _fwd(L, c, -1) == gl.BEAM_ERR_SHAPE
    assert _fwd(L, c, (1 << 22) + 1) == gl.BEAM_ERR_SHAPE
    # T == 0 is a no-op that does not look at the pointers
    assert _fwd(L, c, 0, x=None, out=None, ws=None) == gl.BEAM_OK
    assert _route(L, c, 0, x=None, idx=None, w=None, ws=None) == gl.BEAM_OK


def test_pointer_checks(L):
    c = beam_cfg()
    for name in ["x", "rw", "b", "wg", "wu", "wd", "out"]:
        assert _fwd(L, c, 8, **{name: None}) == gl.BEAM_ERR_NULL, name
    for name in ["x", "rw", "b", "idx", "w"]:
        assert _route(L, c, 8, **{name: None}) == gl.BEAM_ERR_NULL, name
    assert _fwd(L, c, 8, ws=None) == gl.BEAM_ERR_WORKSPACE
    for name in ["x", "rw", "b", "wg", "wu", "wd", "out", "idx", "w", "cnt", "logits", "ws"]:
        assert _fwd(L, c, 8, **{name: FAKE + 4}) == gl.BEAM_ERR_ALIGN, name
    for name in ["x", "rw", "b", "idx", "w", "cnt", "logits", "ws"]:
        assert _route(L, c, 8, **{name: FAKE + 8}) == gl.BEAM_ERR_ALIGN, name


def test_fp8_needs_scales(L):
    c = beam_cfg(w_dtype=gl.BEAM_FP8_E4M3)
    assert _fwd(L, c, 8) == gl.BEAM_ERR_DTYPE
    assert _fwd(L, c, 8, sg=FAKE, su=FAKE) == gl.BEAM_ERR_DTYPE
    assert _fwd(L, c, 8, sg=FAKE, su=FAKE, sd=FAKE + 4) == gl.BEAM_ERR_ALIGN


def test_mxfp4_checks(L):
    """MXFP4 weights: packed layout only, hidden and intermediate multiples of
    512, block scales required; packing needs 512-weight rows."""
    mx = gl.BEAM_MXFP4
    assert _fwd(L, beam_cfg(w_dtype=mx), 8) == gl.BEAM_ERR_CONFIG            # row-major
    ok = beam_cfg(w_dtype=mx, w_layout=gl.BEAM_LAYOUT_PACKED)
    assert _fwd(L, ok, 8) == gl.BEAM_ERR_DTYPE                                 # no scales
    assert _fwd(L, ok, 8, sg=FAKE, su=FAKE, sd=FAKE + 8) == gl.BEAM_ERR_ALIGN
    for kw in [dict(hidden=5120 - 128), dict(intermediate=2560 + 256)]:
        c = beam_cfg(w_dtype=mx, w_layout=gl.BEAM_LAYOUT_PACKED, **kw)
        assert _fwd(L, c, 8, sg=FAKE, su=FAKE, sd=FAKE) == gl.BEAM_ERR_SHAPE, kw
    f = gl.workspace_bytes(beam_cfg(w_dtype=gl.BEAM_FP8_E4M3), 64)
    assert gl.workspace_bytes(ok, 64) == f  # the E4M3 activation buffers of the fp8 path
    v = ctypes.c_void_p
    pk = L.beam_moe_pack_weights
    for dt in (gl.BEAM_MXFP4, gl.BEAM_E8M0):
        assert pk(v(FAKE), v(FAKE), 256, 2560, 5120 - 128, dt, None) == gl.BEAM_ERR_SHAPE
        assert pk(v(FAKE), v(FAKE), 256, 2568, 5120, dt, None) == gl.BEAM_ERR_SHAPE
    assert pk(v(FAKE), v(FAKE), 256, 2560, 5120, 5, None) == gl.BEAM_ERR_DTYPE


def _fwd_res(L, cfg, T, res, **over):
    p = dict(x=FAKE, rw=FAKE, b=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, out=FAKE, ws=FAKE)
    p.update(over)
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.beam_moe_forward_residual(ctypes.byref(cfg), T, v(p["x"]), v(p["rw"]), v(p["b"]),
                                       v(p["wg"]), v(p["wu"]), v(p["wd"]), None, None, None,
                                       None if res is None else ctypes.byref(res), v(p["out"]),
                                       None, None, None, None, v(p["ws"]), 1 << 40, None)


def test_residual_checks(L):
    """The fused residual step: step >= 2, a finite eps >= 0, hidden <= 16384,
    its two pointers present and aligned; T == 0 still a no-op."""
    c = beam_cfg()
    R = lambda **kw: gl.BeamMoeResidual(**dict(dict(stream_in=FAKE, norm_weight=FAKE,
                                                    norm_eps=1e-6, step=5), **kw))
    assert _fwd_res(L, c, 8, None) == gl.BEAM_ERR_NULL
    for kw in [dict(step=1), dict(step=0), dict(step=-3), dict(norm_eps=-1e-6),
               dict(norm_eps=float("nan")), dict(norm_eps=float("inf"))]:
        assert _fwd_res(L, c, 8, R(**kw)) == gl.BEAM_ERR_CONFIG, kw
        assert _fwd_res(L, c, 0, R(**kw)) == gl.BEAM_ERR_CONFIG, kw
    assert _fwd_res(L, beam_cfg(hidden=16384 + 128), 8, R()) == gl.BEAM_ERR_SHAPE
    assert _fwd_res(L, c, 8, R(stream_in=None)) == gl.BEAM_ERR_NULL
    assert _fwd_res(L, c, 8, R(norm_weight=None)) == gl.BEAM_ERR_NULL
    assert _fwd_res(L, c, 8, R(stream_in=FAKE + 2)) == gl.BEAM_ERR_ALIGN
    assert _fwd_res(L, c, 8, R(norm_weight=FAKE + 4)) == gl.BEAM_ERR_ALIGN
    assert _fwd_res(L, c, 8, R(), out=None) == gl.BEAM_ERR_NULL
    assert _fwd_res(L, c, 0, R(stream_in=None, norm_weight=None), x=None, out=None,
                    ws=None) == gl.BEAM_OK


def _bwd(L, cfg, T, grads, **over):
    p = dict(x=FAKE, rw=FAKE, b=FAKE, wg=FAKE, wu=FAKE, wgt=FAKE, wut=FAKE, wdt=FAKE, dout=FAKE,
             ws=FAKE)
    p.update(over)
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.beam_moe_backward(ctypes.byref(cfg), T, v(p["x"]), v(p["rw"]), v(p["b"]), v(p["wg"]),
                               v(p["wu"]), v(p["wgt"]), v(p["wut"]), v(p["wdt"]), v(p["dout"]),
                               None if grads is None else ctypes.byref(grads), v(p["ws"]),
                               1 << 40, None)


def test_backward_checks(L):
    """Backward: bf16 tokens and packed bf16 weights only, hidden and
    intermediate multiples of 256, dx required, weight gradients all or none."""
    c = beam_cfg(w_layout=gl.BEAM_LAYOUT_PACKED)
    G = lambda **kw: gl.BeamMoeGrads(**dict(dict(dx=FAKE, d_router_w=FAKE), **kw))
    assert _bwd(L, beam_cfg(), 8, G()) == gl.BEAM_ERR_CONFIG                       # row-major
    assert _bwd(L, beam_cfg(w_layout=1, x_dtype=gl.BEAM_F32), 8, G()) == gl.BEAM_ERR_DTYPE
    assert _bwd(L, beam_cfg(w_layout=1, w_dtype=gl.BEAM_FP8_E4M3), 8, G()) == gl.BEAM_ERR_DTYPE
    assert _bwd(L, beam_cfg(w_layout=1, hidden=5120 + 128), 8, G()) == gl.BEAM_ERR_SHAPE
    assert _bwd(L, beam_cfg(w_layout=1, intermediate=2560 - 128), 8, G()) == gl.BEAM_ERR_SHAPE
    assert _bwd(L, c, 8, None) == gl.BEAM_ERR_NULL
    assert _bwd(L, c, 8, G(dx=None)) == gl.BEAM_ERR_NULL
    assert _bwd(L, c, 8, G(d_w_gate=FAKE, d_w_up=FAKE)) == gl.BEAM_ERR_NULL      # two of three
    for name in ["x", "rw", "b", "wg", "wu", "wgt", "wut", "wdt", "dout"]:
        assert _bwd(L, c, 8, G(), **{name: None}) == gl.BEAM_ERR_NULL, name
        assert _bwd(L, c, 8, G(), **{name: FAKE + 4}) == gl.BEAM_ERR_ALIGN, name
    assert _bwd(L, c, 8, G(d_router_w=FAKE + 4)) == gl.BEAM_ERR_ALIGN
    assert _bwd(L, c, 8, G(), ws=None) == gl.BEAM_ERR_WORKSPACE
    assert _bwd(L, c, 0, G(), x=None, ws=None) == gl.BEAM_OK
    assert _bwd(L, c, -1, G()) == gl.BEAM_ERR_SHAPE
    # workspace: more with the weight gradients' transposed operands; 0 outside the scope
    a = gl.backward_workspace_bytes(c, 4096, False)
    b = gl.backward_workspace_bytes(c, 4096, True)
    assert 0 < a < b
    assert gl.backward_workspace_bytes(beam_cfg(), 4096, False) == 0
    v = ctypes.c_void_p
    pt = L.beam_moe_pack_weights_transposed
    assert pt(v(FAKE), v(FAKE), 256, 2560, 5120, gl.BEAM_FP8_E4M3, None) == gl.BEAM_ERR_DTYPE
    assert pt(v(FAKE), v(FAKE), 256, 2560 + 32, 5120, gl.BEAM_BF16, None) == gl.BEAM_ERR_SHAPE
    assert pt(None, v(FAKE), 256, 2560, 5120, gl.BEAM_BF16, None) == gl.BEAM_ERR_NULL
    assert pt(v(FAKE), v(FAKE + 8), 256, 2560, 5120, gl.BEAM_BF16, None) == gl.BEAM_ERR_ALIGN
    ub = L.beam_moe_update_bias
    assert ub(None, v(FAKE), 256, 1e-3, None) == gl.BEAM_ERR_NULL
    assert ub(v(FAKE), v(FAKE), 128, 1e-3, None) == gl.BEAM_ERR_CONFIG
    assert ub(v(FAKE), v(FAKE), 256, float("nan"), None) == gl.BEAM_ERR_CONFIG
    assert ub(v(FAKE + 4), v(FAKE), 256, 1e-3, None) == gl.BEAM_ERR_ALIGN


def test_shard_checks(L):
    """Expert shard: 0 <= begin < end <= 256; otherwise the forward's checks."""
    c = beam_cfg()
    v = lambda a: None if a is None else ctypes.c_void_p(a)

    def shard(b, e, T=8, **over):
        p = dict(x=FAKE, rw=FAKE, b=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, out=FAKE, ws=FAKE)
        p.update(over)
        return L.beam_moe_forward_shard(ctypes.byref(c), T, v(p["x"]), v(p["rw"]), v(p["b"]), b, e,
                                        v(p["wg"]), v(p["wu"]), v(p["wd"]), None, None, None,
                                        v(p["out"]), None, None, None, v(p["ws"]), 1 << 40, None)
    for b, e in [(-1, 32), (0, 0), (32, 32), (64, 32), (0, 257), (255, 300)]:
        assert shard(b, e) == gl.BEAM_ERR_CONFIG, (b, e)
    assert shard(0, 32, out=None) == gl.BEAM_ERR_NULL
    assert shard(0, 32, wg=FAKE + 4) == gl.BEAM_ERR_ALIGN
    assert shard(224, 256, T=0, x=None, out=None, ws=None) == gl.BEAM_OK


def test_workspace_size(L):
    c = beam_cfg()
    need = gl.workspace_bytes(c, 64)
    assert need > 0
    assert _fwd(L, c, 64, ws_bytes=need - 1) == gl.BEAM_ERR_WORKSPACE
    assert _route(L, c, 64, ws_bytes=need - 1) == gl.BEAM_ERR_WORKSPACE
    # grows with T; the bf16 SwiGLU and expert-output buffers dominate at large T
    sizes = [gl.workspace_bytes(c, T) for T in (1, 64, 4096, 16384)]
    assert sizes == sorted(sizes)
    T = 16384
    assert sizes[-1] >= T * 8 * (2560 + 5120) * 2
    assert sizes[-1] < T * 8 * (2560 + 5120) * 2 * 1.1
    assert gl.workspace_bytes(c, -1) == 0
    assert gl.workspace_bytes(beam_cfg(n_group=3), 64) == 0
    f8 = gl.workspace_bytes(beam_cfg(w_dtype=gl.BEAM_FP8_E4M3), 64)
    assert f8 > 0


def test_layout_and_pack_checks(L):
    assert _fwd(L, beam_cfg(w_layout=2), 8) == gl.BEAM_ERR_CONFIG
    v = ctypes.c_void_p
    pk = L.beam_moe_pack_weights
    assert pk(None, v(FAKE), 256, 2560, 5120, gl.BEAM_BF16, None) == gl.BEAM_ERR_NULL
    assert pk(v(FAKE), v(FAKE), 256, 2560, 5120, gl.BEAM_F32, None) == gl.BEAM_ERR_DTYPE
    for E, R, C in [(0, 2560, 5120), (256, 2568, 5120), (256, 2560, 5000), (256, 0, 5120),
                    (1 << 20, 2560, 5120)]:
        assert pk(v(FAKE), v(FAKE), E, R, C, gl.BEAM_BF16, None) == gl.BEAM_ERR_SHAPE, (E, R, C)
    assert pk(v(FAKE + 8), v(FAKE), 256, 2560, 5120, gl.BEAM_BF16, None) == gl.BEAM_ERR_ALIGN


def test_library_links_every_kernel(L):
    """Every kernel launched by the library has its host launch stub in the
    .so and nothing of the library is left undefined (a kernel whose host-side
    instantiation fails would otherwise leave a launch that never happens)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    und = subprocess.run([nm, "-DC", "--undefined-only", gl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert "beam::" not in und, [ln for ln in und.splitlines() if "beam::" in ln]
    syms = subprocess.run([nm, "-C", gl.LIB_PATH], capture_output=True, text=True, check=True).stdout
    for kernel in ["gemm_dma4_kernel", "router_logits_kernel", "router_split_kernel", "router_x3_kernel", "select_kernel", "perm_hist_kernel", "perm_scan_kernel",
                   "perm_scatter_kernel", "gemm_stream_kernel", "gemm_tiled_kernel",
                   "gemm_wide_kernel", "gemm_dma_kernel", "gemm_dma8_kernel", "gemm_stream4_kernel",
                   "combine_kernel", "combine_residual_kernel", "combine_shard_kernel", "pack_mx_scales_kernel",
                   "segment_cols_kernel", "gather_t_kernel", "zero_pads_kernel",
                   "token_grad_kernel", "router_grad_kernel", "gemm_wgrad_kernel",
                   "pack_t_kernel", "bias_step_kernel", "quant_x_kernel",
                   "quant_h_kernel", "pack_kernel"]:
        assert f"__device_stub__{kernel}" in syms, kernel


def _noalloc(L, cfg, T, **over):
    p = dict(x=FAKE, rw=FAKE, b=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, sg=None, su=None, sd=None,
             out=FAKE, idx=None, w=None, cnt=None, logits=None)
    p.update(over)
    v = lambda a: None if a is None else ctypes.c_void_p(a)
    return L.beam_moe_forward_noalloc(ctypes.byref(cfg) if cfg is not None else None, T,
                                      v(p["x"]), v(p["rw"]), v(p["b"]), v(p["wg"]), v(p["wu"]),
                                      v(p["wd"]), v(p["sg"]), v(p["su"]), v(p["sd"]),
                                      v(p["out"]), v(p["idx"]), v(p["w"]), v(p["cnt"]),
                                      v(p["logits"]), None)


def test_noalloc_checks_run_before_any_hip_call(L):
    """beam_moe_forward_noalloc: the forward's checks, then the scratch limit,
    all before its first HIP call. This machine has no GPU, so a HIP call
    would return BEAM_ERR_HIP: the statuses below show the checks came
    first."""
    c = beam_cfg()
    assert gl.NOALLOC_MAX_BYTES == 64 << 20
    assert _noalloc(L, c, 0, x=None, out=None) == gl.BEAM_OK
    assert _noalloc(L, None, 8) == gl.BEAM_ERR_NULL
    assert _noalloc(L, beam_cfg(n_group=3), 8) == gl.BEAM_ERR_CONFIG
    assert _noalloc(L, c, -1) == gl.BEAM_ERR_SHAPE
    for name in ["x", "rw", "b", "wg", "wu", "wd", "out"]:
        assert _noalloc(L, c, 8, **{name: None}) == gl.BEAM_ERR_NULL, name
    assert _noalloc(L, c, 8, out=FAKE + 4) == gl.BEAM_ERR_ALIGN
    assert _noalloc(L, beam_cfg(w_dtype=gl.BEAM_FP8_E4M3), 8) == gl.BEAM_ERR_DTYPE
    # the scratch holds the workspace of every batch up to 256 tokens at
    # Beam's shape, bf16 / fp8 / MXFP4 experts; beyond it the call refuses
    for wdt in (gl.BEAM_BF16, gl.BEAM_FP8_E4M3):
        assert gl.workspace_bytes(beam_cfg(w_dtype=wdt), 256) <= gl.NOALLOC_MAX_BYTES
    big = next(T for T in range(256, 4096) if gl.workspace_bytes(c, T) > gl.NOALLOC_MAX_BYTES)
    assert _noalloc(L, c, big) == gl.BEAM_ERR_WORKSPACE
    assert _noalloc(L, c, 1 << 20) == gl.BEAM_ERR_WORKSPACE

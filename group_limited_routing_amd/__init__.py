"""Beam sparse-MoE block on MI355X (gfx950): Python binding of libbeam_moe.so.

Argument marshalling only. Every step of the block (router logits, group-
limited selection, permutation, expert GEMMs, combine) runs in the HIP
kernels behind the C ABI declared in include/beam_moe.h; torch supplies
device memory and the current stream. If the library is missing the calls
raise instead of falling back to anything else.

Names follow the Beam model doc's config fields: n_group, topk_group,
routed_scaling_factor (transformers model doc "Beam", "Overview").

Streams: every call takes ``stream`` (default: the current stream of the
tensors' device) and enqueues its kernels there. Tensors a call allocates
(outputs, and the workspace when none is passed) come from that stream's
pool of torch's caching allocator, so a block freed on return is reused only
by later work on the same stream, which runs after the kernels that used it.
A caller that passes its own workspace or outputs owns their stream
ordering, as for any torch tensor used on a side stream.
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbeam_moe.so")

BEAM_OK, BEAM_ERR_NULL, BEAM_ERR_CONFIG, BEAM_ERR_SHAPE = 0, 1, 2, 3
BEAM_ERR_DTYPE, BEAM_ERR_ALIGN, BEAM_ERR_WORKSPACE, BEAM_ERR_HIP = 4, 5, 6, 7
BEAM_F32, BEAM_BF16, BEAM_FP8_E4M3, BEAM_MXFP4, BEAM_E8M0 = 0, 1, 2, 3, 4
BEAM_LAYOUT_ROW_MAJOR, BEAM_LAYOUT_PACKED = 0, 1

EXPORTED = ("beam_moe_workspace_bytes", "beam_moe_route", "beam_moe_forward",
            "beam_moe_forward_residual", "beam_moe_status_string", "beam_moe_profile_begin",
            "beam_moe_profile_end", "beam_moe_pack_weights", "beam_moe_backward_workspace_bytes",
            "beam_moe_backward", "beam_moe_pack_weights_transposed", "beam_moe_update_bias",
            "beam_moe_forward_shard", "beam_moe_forward_noalloc")

# Scratch size of beam_moe_forward_noalloc (BEAM_MOE_NOALLOC_MAX_BYTES in the header)
NOALLOC_MAX_BYTES = 64 << 20

STAGES = ("router_logits", "select", "perm_hist", "perm_scan", "perm_scatter", "quant_x",
          "gateup", "quant_h", "down", "combine", "bwd_gateup", "bwd_down", "bwd_dx",
          "bwd_token", "bwd_router", "bwd_transpose", "bwd_wgrad")


class BeamMoeConfig(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("x_dtype", ctypes.c_int32),
        ("w_dtype", ctypes.c_int32),
        ("w_layout", ctypes.c_int32),
    ]


class BeamMoeResidual(ctypes.Structure):
    _fields_ = [
        ("stream_in", ctypes.c_void_p),
        ("norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("step", ctypes.c_int32),
    ]


class BeamMoeGrads(ctypes.Structure):
    _fields_ = [
        ("dx", ctypes.c_void_p),
        ("d_router_w", ctypes.c_void_p),
        ("d_w_gate", ctypes.c_void_p),
        ("d_w_up", ctypes.c_void_p),
        ("d_w_down", ctypes.c_void_p),
    ]


class BeamMoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status}: {status_string(status)}")


_lib = None


def lib():
    """The loaded C library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with "
                              "`python -m group_limited_routing_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        cfgp = ctypes.POINTER(BeamMoeConfig)
        L.beam_moe_workspace_bytes.argtypes = [cfgp, i32]
        L.beam_moe_workspace_bytes.restype = sz
        L.beam_moe_route.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_route.restype = ctypes.c_int
        L.beam_moe_forward.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, sz, vp]
        L.beam_moe_forward.restype = ctypes.c_int
        L.beam_moe_forward_residual.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.POINTER(BeamMoeResidual), vp, vp, vp, vp,
                                                vp, vp, sz, vp]
        L.beam_moe_forward_residual.restype = ctypes.c_int
        L.beam_moe_status_string.argtypes = [i32]
        L.beam_moe_status_string.restype = ctypes.c_char_p
        L.beam_moe_profile_begin.argtypes = [ctypes.c_uint32]
        L.beam_moe_profile_begin.restype = ctypes.c_int
        L.beam_moe_profile_end.argtypes = [vp, vp]
        L.beam_moe_profile_end.restype = ctypes.c_int
        L.beam_moe_pack_weights.argtypes = [vp, vp, i32, i32, i32, i32, vp]
        L.beam_moe_pack_weights.restype = ctypes.c_int
        L.beam_moe_forward_shard.argtypes = [cfgp, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_forward_shard.restype = ctypes.c_int
        L.beam_moe_forward_noalloc.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, vp, vp]
        L.beam_moe_forward_noalloc.restype = ctypes.c_int
        L.beam_moe_backward_workspace_bytes.argtypes = [cfgp, i32, i32]
        L.beam_moe_backward_workspace_bytes.restype = sz
        L.beam_moe_backward.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        ctypes.POINTER(BeamMoeGrads), vp, sz, vp]
        L.beam_moe_backward.restype = ctypes.c_int
        L.beam_moe_pack_weights_transposed.argtypes = [vp, vp, i32, i32, i32, i32, vp]
        L.beam_moe_pack_weights_transposed.restype = ctypes.c_int
        L.beam_moe_update_bias.argtypes = [vp, vp, i32, ctypes.c_float, vp]
        L.beam_moe_update_bias.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status):
    return lib().beam_moe_status_string(int(status)).decode()


_X_DTYPES = {torch.float32: BEAM_F32, torch.bfloat16: BEAM_BF16}
# uint8 weight tensors are MXFP4 codes (two E2M1 values per byte)
_W_DTYPES = {torch.bfloat16: BEAM_BF16, torch.float8_e4m3fn: BEAM_FP8_E4M3,
             torch.uint8: BEAM_MXFP4}


def make_config(hidden, intermediate, n_experts=256, n_group=8, topk_group=4, top_k=8,
                routed_scaling_factor=2.5, x_dtype=torch.bfloat16, w_dtype=torch.bfloat16,
                packed=False):
    if x_dtype not in _X_DTYPES or w_dtype not in _W_DTYPES:
        raise TypeError(f"unsupported dtypes x={x_dtype} w={w_dtype}")
    return BeamMoeConfig(hidden, intermediate, n_experts, n_group, topk_group, top_k,
                         routed_scaling_factor, _X_DTYPES[x_dtype], _W_DTYPES[w_dtype],
                         BEAM_LAYOUT_PACKED if packed else BEAM_LAYOUT_ROW_MAJOR)


def pack_weights(w, out=None, stream=None):
    """MFMA-fragment copy of row-major expert weights w [E, R, C] (bf16 or
    float8_e4m3fn; uint8 = MXFP4 codes [E, R, C/2]); pass the result to
    forward(..., packed=True)."""
    if w.dim() != 3 or not w.is_contiguous() or w.dtype not in _W_DTYPES:
        raise ValueError("pack_weights needs a contiguous [E, rows, cols] bf16/fp8/MXFP4 tensor")
    s = _target(w.device, stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty_like(w)
    E, R, C = w.shape
    if w.dtype == torch.uint8:
        C *= 2  # weights per row
    st = lib().beam_moe_pack_weights(_ptr(w), _ptr(out), E, R, C, _W_DTYPES[w.dtype],
                                     _handle(s))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_pack_weights")
    return out


def pack_mx_scales(s, out=None, stream=None):
    """Packed copy of row-major MXFP4 scale bytes s [E, R, C/32] (uint8, E8M0)."""
    if s.dim() != 3 or not s.is_contiguous() or s.dtype != torch.uint8:
        raise ValueError("pack_mx_scales needs a contiguous [E, rows, cols/32] uint8 tensor")
    ts = _target(s.device, stream)
    if out is None:
        with torch.cuda.stream(ts):
            out = torch.empty_like(s)
    E, R, B = s.shape
    st = lib().beam_moe_pack_weights(_ptr(s), _ptr(out), E, R, 32 * B, BEAM_E8M0, _handle(ts))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_pack_weights")
    return out


def workspace_bytes(cfg, T):
    return int(lib().beam_moe_workspace_bytes(ctypes.byref(cfg), int(T)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, shape, dtypes, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _workspace(cfg, T, device, workspace):
    """The caller's workspace, or a new one (call it under the target stream)."""
    need = workspace_bytes(cfg, T)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def _target(device, stream):
    """The torch stream a call runs on: ``stream``, else the device's current one."""
    return stream if stream is not None else torch.cuda.current_stream(device)


def _handle(s):
    return ctypes.c_void_p(s.cuda_stream)


def route(x, router_w, expert_bias, *, n_group=8, topk_group=4, top_k=8,
          return_logits=False, return_counts=False, workspace=None, stream=None):
    """Router only. Returns dict(topk_idx [T, k] int32, topk_w [T, k] fp32,
    router_logits [T, E] fp32 or None, expert_counts [E] int32 or None)."""
    T, H = x.shape
    E = router_w.shape[0]
    dev = x.device
    _check(x, "x", (T, H), (torch.float32, torch.bfloat16), dev)
    _check(router_w, "router_w", (E, H), (torch.float32,), dev)
    _check(expert_bias, "expert_bias", (E,), (torch.float32,), dev)
    cfg = make_config(H, 128, E, n_group, topk_group, top_k, 1.0, x.dtype, torch.bfloat16)
    s = _target(dev, stream)
    with torch.cuda.stream(s):
        idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
        logits = torch.empty((T, E), dtype=torch.float32, device=dev) if return_logits else None
        counts = torch.empty((E,), dtype=torch.int32, device=dev) if return_counts else None
        ws = _workspace(cfg, T, dev, workspace)
    st = lib().beam_moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                              _ptr(idx), _ptr(w), _ptr(logits), _ptr(counts), _ptr(ws),
                              ws.numel(), _handle(s))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_route")
    return {"topk_idx": idx, "topk_w": w, "router_logits": logits, "expert_counts": counts}


def forward(x, router_w, expert_bias, w_gate, w_up, w_down, *, scales=None, n_group=8,
            topk_group=4, top_k=8, routed_scaling_factor=2.5, out=None, return_routing=False,
            return_logits=False, workspace=None, stream=None, packed=False):
    """The whole MoE block. ``scales`` = (w_gate_scale, w_up_scale, w_down_scale)
    for fp8 weights (fp32 per row) and MXFP4 weights (uint8 codes, with the
    E8M0 block scales from pack_mx_scales); ``packed`` says the weights come
    from pack_weights() (required for MXFP4).
    Returns out [T, H] (x's dtype), or (out, routing dict) with
    ``return_routing`` or ``return_logits``."""
    return _forward(x, router_w, expert_bias, w_gate, w_up, w_down, None, scales, n_group,
                    topk_group, top_k, routed_scaling_factor, out, return_routing,
                    return_logits, workspace, stream, packed)


def forward_residual(x, router_w, expert_bias, w_gate, w_up, w_down, stream_in, norm_weight,
                     step, *, norm_eps=1e-6, scales=None, n_group=8, topk_group=4, top_k=8,
                     routed_scaling_factor=2.5, out=None, return_routing=False,
                     return_logits=False, workspace=None, stream=None, packed=False):
    """The MoE block and its residual-stream step at sublayer step ``step``:
    returns sqrt((step-1)/step) * stream_in + RMSNorm(block output) / sqrt(step)
    (RMSNorm with gain ``norm_weight`` [H] fp32 and ``norm_eps``), x's dtype.
    ``out`` may be ``stream_in`` itself. Other arguments as for forward()."""
    T, H = x.shape
    _check(stream_in, "stream_in", (T, H), (x.dtype,), x.device)
    _check(norm_weight, "norm_weight", (H,), (torch.float32,), x.device)
    res = BeamMoeResidual(stream_in.data_ptr(), norm_weight.data_ptr(), float(norm_eps),
                          int(step))
    return _forward(x, router_w, expert_bias, w_gate, w_up, w_down, res, scales, n_group,
                    topk_group, top_k, routed_scaling_factor, out, return_routing,
                    return_logits, workspace, stream, packed)


def forward_noalloc(x, router_w, expert_bias, w_gate, w_up, w_down, *, out, scales=None,
                    n_group=8, topk_group=4, top_k=8, routed_scaling_factor=2.5, topk_idx=None,
                    topk_w=None, expert_counts=None, router_logits=None, stream=None,
                    packed=False):
    """The whole MoE block through beam_moe_forward_noalloc: the library's
    static per-GPU scratch instead of a workspace. Every output is the
    caller's (``out`` [T, H] in x's dtype, and optionally topk_idx [T, k]
    int32, topk_w [T, k] fp32, expert_counts [E] int32, router_logits [T, E]
    fp32), so the call allocates nothing. Calls that overlap on one GPU
    race on the shared scratch. Other arguments as for forward()."""
    T, H = x.shape
    E = router_w.shape[0]
    I = w_gate.shape[1]
    dev = x.device
    mx = w_gate.dtype == torch.uint8
    d = 2 if mx else 1
    wdt = (torch.bfloat16, torch.float8_e4m3fn, torch.uint8)
    _check(x, "x", (T, H), (torch.float32, torch.bfloat16), dev)
    _check(router_w, "router_w", (E, H), (torch.float32,), dev)
    _check(expert_bias, "expert_bias", (E,), (torch.float32,), dev)
    _check(w_gate, "w_gate", (E, I, H // d), wdt, dev)
    _check(w_up, "w_up", (E, I, H // d), (w_gate.dtype,), dev)
    _check(w_down, "w_down", (E, H, I // d), (w_gate.dtype,), dev)
    _check(out, "out", (T, H), (x.dtype,), dev)
    for t, name, shape, dt in ((topk_idx, "topk_idx", (T, top_k), torch.int32),
                               (topk_w, "topk_w", (T, top_k), torch.float32),
                               (expert_counts, "expert_counts", (E,), torch.int32),
                               (router_logits, "router_logits", (T, E), torch.float32)):
        if t is not None:
            _check(t, name, shape, (dt,), dev)
    sg = su = sd = None
    if w_gate.dtype in (torch.float8_e4m3fn, torch.uint8):
        if scales is None:
            raise ValueError("quantised weights need (w_gate_scale, w_up_scale, w_down_scale)")
        sg, su, sd = scales
    cfg = make_config(H, I, E, n_group, topk_group, top_k, routed_scaling_factor, x.dtype,
                      w_gate.dtype, packed)
    st = lib().beam_moe_forward_noalloc(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w),
                                        _ptr(expert_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                        _ptr(sg), _ptr(su), _ptr(sd), _ptr(out), _ptr(topk_idx),
                                        _ptr(topk_w), _ptr(expert_counts), _ptr(router_logits),
                                        _handle(_target(dev, stream)))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_forward_noalloc")
    return out


def forward_shard(x, router_w, expert_bias, expert_begin, expert_end, w_gate, w_up, w_down, *,
                  scales=None, n_group=8, topk_group=4, top_k=8, routed_scaling_factor=2.5,
                  out=None, return_routing=False, workspace=None, stream=None, packed=False):
    """One expert shard's share of the block: the weights (and scales) hold
    experts [expert_begin, expert_end) only; returns the partial output
    [T, H] (x's dtype) whose sum over a partition of the experts is the block
    output. Other arguments as for forward()."""
    return _forward(x, router_w, expert_bias, w_gate, w_up, w_down, None, scales, n_group,
                    topk_group, top_k, routed_scaling_factor, out, return_routing, False,
                    workspace, stream, packed, shard=(int(expert_begin), int(expert_end)))


def _forward(x, router_w, expert_bias, w_gate, w_up, w_down, res, scales, n_group, topk_group,
             top_k, routed_scaling_factor, out, return_routing, return_logits, workspace,
             stream, packed, shard=None):
    T, H = x.shape
    E = router_w.shape[0]
    n_w = E if shard is None else shard[1] - shard[0]  # experts held by the weight arrays
    I = w_gate.shape[1]
    dev = x.device
    wdt = (torch.bfloat16, torch.float8_e4m3fn, torch.uint8)
    mx = w_gate.dtype == torch.uint8
    d = 2 if mx else 1  # MXFP4: two codes per byte
    _check(x, "x", (T, H), (torch.float32, torch.bfloat16), dev)
    _check(router_w, "router_w", (E, H), (torch.float32,), dev)
    _check(expert_bias, "expert_bias", (E,), (torch.float32,), dev)
    _check(w_gate, "w_gate", (n_w, I, H // d), wdt, dev)
    _check(w_up, "w_up", (n_w, I, H // d), (w_gate.dtype,), dev)
    _check(w_down, "w_down", (n_w, H, I // d), (w_gate.dtype,), dev)
    sg = su = sd = None
    if w_gate.dtype in (torch.float8_e4m3fn, torch.uint8):
        if scales is None:
            raise ValueError("quantised weights need (w_gate_scale, w_up_scale, w_down_scale)")
        sg, su, sd = scales
        if mx:
            _check(sg, "w_gate_scale", (n_w, I, H // 32), (torch.uint8,), dev)
            _check(su, "w_up_scale", (n_w, I, H // 32), (torch.uint8,), dev)
            _check(sd, "w_down_scale", (n_w, H, I // 32), (torch.uint8,), dev)
        else:
            _check(sg, "w_gate_scale", (n_w, I), (torch.float32,), dev)
            _check(su, "w_up_scale", (n_w, I), (torch.float32,), dev)
            _check(sd, "w_down_scale", (n_w, H), (torch.float32,), dev)
    cfg = make_config(H, I, E, n_group, topk_group, top_k, routed_scaling_factor, x.dtype,
                      w_gate.dtype, packed)
    if out is not None:
        _check(out, "out", (T, H), (x.dtype,), dev)
    s = _target(dev, stream)
    idx = w = counts = logits = None
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty((T, H), dtype=x.dtype, device=dev)
        if return_routing:
            idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
            w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
            counts = torch.empty((E,), dtype=torch.int32, device=dev)
        if return_logits:
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        ws = _workspace(cfg, T, dev, workspace)
    if shard is not None:
        st = lib().beam_moe_forward_shard(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w),
                                          _ptr(expert_bias), shard[0], shard[1], _ptr(w_gate),
                                          _ptr(w_up), _ptr(w_down), _ptr(sg), _ptr(su), _ptr(sd),
                                          _ptr(out), _ptr(idx), _ptr(w), _ptr(counts), _ptr(ws),
                                          ws.numel(), _handle(s))
        where = "beam_moe_forward_shard"
    elif res is None:
        st = lib().beam_moe_forward(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w),
                                    _ptr(expert_bias), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                                    _ptr(sg), _ptr(su), _ptr(sd), _ptr(out), _ptr(idx), _ptr(w),
                                    _ptr(counts), _ptr(logits), _ptr(ws), ws.numel(),
                                    _handle(s))
        where = "beam_moe_forward"
    else:
        st = lib().beam_moe_forward_residual(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w),
                                             _ptr(expert_bias), _ptr(w_gate), _ptr(w_up),
                                             _ptr(w_down), _ptr(sg), _ptr(su), _ptr(sd),
                                             ctypes.byref(res), _ptr(out), _ptr(idx), _ptr(w),
                                             _ptr(counts), _ptr(logits), _ptr(ws), ws.numel(),
                                             _handle(s))
        where = "beam_moe_forward_residual"
    if st != BEAM_OK:
        raise BeamMoeError(st, where)
    if return_routing or return_logits:
        return out, {"topk_idx": idx, "topk_w": w, "expert_counts": counts,
                     "router_logits": logits}
    return out


def pack_weights_transposed(w, out=None, stream=None):
    """[E, rows, cols] bf16 expert matrices -> the packed layout of their
    transposes (what backward() takes as w_gate_t, w_up_t, w_down_t)."""
    if w.dtype != torch.bfloat16 or w.dim() != 3 or not w.is_contiguous():
        raise ValueError("expects a contiguous [E, rows, cols] bf16 tensor")
    E, R, C = w.shape
    s = _target(w.device, stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((E, C, R), dtype=w.dtype, device=w.device)
    st = lib().beam_moe_pack_weights_transposed(_ptr(w), _ptr(out), E, R, C, BEAM_BF16,
                                                _handle(s))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_pack_weights_transposed")
    return out


def backward_workspace_bytes(cfg, T, weight_grads):
    return int(lib().beam_moe_backward_workspace_bytes(ctypes.byref(cfg), int(T), int(bool(weight_grads))))


def backward(x, router_w, expert_bias, w_gate, w_up, w_gate_t, w_up_t, w_down_t, dout, *,
             weight_grads=False, router_grad=True, n_group=8, topk_group=4, top_k=8,
             routed_scaling_factor=2.5, workspace=None, stream=None):
    """Gradients of sum(dout * forward(...)) (bf16 x and dout, packed bf16
    weights: w_gate, w_up from pack_weights, the *_t from
    pack_weights_transposed). Returns dict(dx [T, H] bf16, d_router_w [E, H]
    fp32 or None, d_w_gate / d_w_up [E, I, H] and d_w_down [E, H, I] bf16
    with ``weight_grads``, else None)."""
    T, H = x.shape
    E = router_w.shape[0]
    I = w_gate.shape[1]
    dev = x.device
    _check(x, "x", (T, H), (torch.bfloat16,), dev)
    _check(dout, "dout", (T, H), (torch.bfloat16,), dev)
    _check(router_w, "router_w", (E, H), (torch.float32,), dev)
    _check(expert_bias, "expert_bias", (E,), (torch.float32,), dev)
    for name, t, shape in (("w_gate", w_gate, (E, I, H)), ("w_up", w_up, (E, I, H)),
                           ("w_gate_t", w_gate_t, (E, H, I)), ("w_up_t", w_up_t, (E, H, I)),
                           ("w_down_t", w_down_t, (E, I, H))):
        _check(t, name, shape, (torch.bfloat16,), dev)
    cfg = make_config(H, I, E, n_group, topk_group, top_k, routed_scaling_factor, x.dtype,
                      torch.bfloat16, packed=True)
    need = backward_workspace_bytes(cfg, T, weight_grads)
    if need == 0 and T > 0:
        raise BeamMoeError(BEAM_ERR_CONFIG, "beam_moe_backward_workspace_bytes")
    s = _target(dev, stream)
    dwg = dwu = dwd = None
    with torch.cuda.stream(s):
        dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        drw = torch.empty((E, H), dtype=torch.float32, device=dev) if router_grad else None
        if weight_grads:
            dwg = torch.empty((E, I, H), dtype=torch.bfloat16, device=dev)
            dwu = torch.empty((E, I, H), dtype=torch.bfloat16, device=dev)
            dwd = torch.empty((E, H, I), dtype=torch.bfloat16, device=dev)
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    grads = BeamMoeGrads(dx.data_ptr(), drw.data_ptr() if drw is not None else None,
                         dwg.data_ptr() if dwg is not None else None,
                         dwu.data_ptr() if dwu is not None else None,
                         dwd.data_ptr() if dwd is not None else None)
    st = lib().beam_moe_backward(ctypes.byref(cfg), T, _ptr(x), _ptr(router_w), _ptr(expert_bias),
                                 _ptr(w_gate), _ptr(w_up), _ptr(w_gate_t), _ptr(w_up_t),
                                 _ptr(w_down_t), _ptr(dout), ctypes.byref(grads), _ptr(workspace),
                                 workspace.numel(), _handle(s))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_backward")
    return {"dx": dx, "d_router_w": drw, "d_w_gate": dwg, "d_w_up": dwu, "d_w_down": dwd}


def update_bias(expert_bias, expert_counts, gamma, stream=None):
    """One load-balancing step of the selection bias, in place:
    b[e] += gamma * sign(mean(counts) - counts[e])."""
    dev = expert_bias.device
    _check(expert_bias, "expert_bias", (256,), (torch.float32,), dev)
    _check(expert_counts, "expert_counts", (256,), (torch.int32,), dev)
    st = lib().beam_moe_update_bias(_ptr(expert_bias), _ptr(expert_counts), 256, float(gamma),
                                    _handle(_target(dev, stream)))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_update_bias")
    return expert_bias


def profile_begin(stages=STAGES):
    """Start timing the named stages of every following route/forward call."""
    mask = 0
    for name in stages:
        mask |= 1 << STAGES.index(name)
    st = lib().beam_moe_profile_begin(mask)
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_profile_begin")


def profile_end():
    """Stop timing; returns {stage: (total_ms, launches)} for timed stages."""
    n = len(STAGES)
    tot = (ctypes.c_float * n)()
    cnt = (ctypes.c_int32 * n)()
    st = lib().beam_moe_profile_end(ctypes.cast(tot, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p))
    if st != BEAM_OK:
        raise BeamMoeError(st, "beam_moe_profile_end")
    return {STAGES[i]: (float(tot[i]), int(cnt[i])) for i in range(n) if cnt[i] > 0}

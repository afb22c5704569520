"""Oracle: routed SwiGLU experts and the weighted combine (float64, numpy).

Test infrastructure only; see the package docstring.

Beam launch post, "Mixture of Experts": each of the 256 experts is a SwiGLU
MLP with intermediate size 2560 (about 39M parameters: three 5120 x 2560
matrices), a token runs through the 8 experts its router chose, the expert
outputs are combined with the normalised router weights and the result is
scaled by 2.5; there is no shared expert. Section "Residual Stream": the
SwiGLU product is computed in fp32 (here float64, which is at least as
precise). transformers model doc "Beam", "Overview": the MoE output is scaled
by ``routed_scaling_factor``.

Expert e is y = W_down[e] @ (silu(W_gate[e] @ x) * (W_up[e] @ x)) with
silu(v) = v / (1 + e^-v) and no linear biases. Matrices are stored [out, in]:
w_gate and w_up [E, I, H], w_down [E, H, I].

Experts may be given as three arrays or as a callable ``get_expert(e)`` that
returns (w_gate[e], w_up[e], w_down[e]); the callable form lets a caller
stream one expert at a time at the full 20 GB layer size.
"""

import numpy as np

from .routing import route, weights_for
from . import bf16, e4m3


def silu(v):
    """silu(v) = v * sigmoid(v) = v / (1 + e^-v), float64, overflow-safe."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))
    ev = np.exp(v[~pos])
    out[~pos] = v[~pos] * ev / (1.0 + ev)
    return out


def expert_ffn(x_rows, w_gate_e, w_up_e, w_down_e, quantize_h=False):
    """One SwiGLU expert on a block of rows: [n, H] -> [n, H] (float64).

    ``quantize_h`` (fp8 and MXFP4 experts only) takes the [n, I]
    intermediate as it is stored, bf16 (``bf16.round_to_bf16``), through
    per-row E4M3 quantise/dequantise before the down projection.
    """
    xr = np.asarray(x_rows, dtype=np.float64)
    g = xr @ np.asarray(w_gate_e, dtype=np.float64).T
    u = xr @ np.asarray(w_up_e, dtype=np.float64).T
    h = silu(g) * u
    if quantize_h:
        h = e4m3.fake_quantize_rows(bf16.round_to_bf16(h))
    return h @ np.asarray(w_down_e, dtype=np.float64).T


def _expert_getter(experts):
    if callable(experts):
        return experts
    wg, wu, wd = experts
    return lambda e: (wg[e], wu[e], wd[e])


def _combine(x, idx, w, routed_scaling_factor, get_expert, fp8):
    """out[t] = sum_j rsf * w[t, j] * FFN_{idx[t, j]}(x[t]), float64.

    Tokens are gathered per expert (the sparse dispatch). With ``fp8`` the
    expert input rows are the per-token E4M3 quantise/dequantise of x and the
    intermediate is quantised per (token, slot) row.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    xin = e4m3.fake_quantize_rows(x) if fp8 else x
    out = np.zeros((T, H), dtype=np.float64)
    for e in np.unique(idx):
        tok, slot = np.nonzero(idx == e)
        wg, wu, wd = get_expert(int(e))
        y = expert_ffn(xin[tok], wg, wu, wd, quantize_h=fp8)
        coef = routed_scaling_factor * w[tok, slot]
        np.add.at(out, tok, coef[:, None] * y)
    return out


def forward(x, router_w, expert_bias, experts, n_group=8, topk_group=4, top_k=8,
            routed_scaling_factor=2.5, routing=None, fp8=False):
    """The whole block: route every token, run its experts, combine.

    ``routing`` optionally forces the expert choice ([T, top_k] indices); the
    weights are then the normalised unbiased scores of those experts. Used to
    check tokens whose selection lies within rounding distance of a tie.
    Returns (out [T, H] float64, the routing dict of :func:`route`).
    """
    r = route(x, router_w, expert_bias, n_group, topk_group, top_k)
    if routing is not None:
        r["idx"] = np.asarray(routing, dtype=np.int64)
        r["w"] = weights_for(r["s"], r["idx"])
    out = _combine(x, r["idx"], r["w"], routed_scaling_factor, _expert_getter(experts), fp8)
    return out, r


def forward_tokens(tokens, x, router_w, expert_bias, experts, **kw):
    """:func:`forward` on a subset of token rows (routing is per token).

    Returns (out [len(tokens), H], routing dict for those tokens).
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    routing = kw.pop("routing", None)
    if routing is not None:
        routing = np.asarray(routing)[tokens]
    return forward(np.asarray(x)[tokens], router_w, expert_bias, experts, routing=routing, **kw)


def dense_forward(x, router_w, expert_bias, experts, n_experts, n_group=8, topk_group=4,
                  top_k=8, routed_scaling_factor=2.5):
    """Every expert on every token, masked by the routing: an independent check
    of the sparse dispatch and combine.

    out[t] = sum over all e of M[t, e] * rsf * W[t, e] * FFN_e(x[t]), where M is
    1 on the chosen experts and W holds their normalised weights.
    """
    x = np.asarray(x, dtype=np.float64)
    r = route(x, router_w, expert_bias, n_group, topk_group, top_k)
    T = x.shape[0]
    M = np.zeros((T, n_experts))
    Wd = np.zeros((T, n_experts))
    rows = np.arange(T)[:, None]
    M[rows, r["idx"]] = 1.0
    Wd[rows, r["idx"]] = r["w"]
    get = _expert_getter(experts)
    out = np.zeros_like(x)
    for e in range(n_experts):
        wg, wu, wd = get(e)
        out += (M[:, e] * routed_scaling_factor * Wd[:, e])[:, None] * expert_ffn(x, wg, wu, wd)
    return out, r

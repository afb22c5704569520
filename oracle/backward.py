"""Oracle: gradients of the MoE block, and the load-balancing bias step.

Test infrastructure only; see the package docstring.

The block is the one of :mod:`oracle.experts` (Beam launch post, "Mixture of
Experts"): out[t] = rsf * sum_j w[t, j] * y_{e_j}(x[t]), with
y_e(x) = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)), w[t, j] = s[t, e_j] /
sum_i s[t, e_i] and s = sigmoid(W_r x). The launch post's section
"Post-training Beam" trains the model with GRPO under expert parallelism and
full recomputation, with bf16 gradients ("GRPO with Miles"), and fine-tunes
rank-16 adapters on the expert layers ("Training with LoRA"); both need this
block's backward pass. The pages state no formula for it, so it is the chain
rule applied to the forward, written out step by step in reverse order:

* the expert choice is piecewise constant in its inputs, so it carries no
  gradient: the selection bias gets none, and the router gets its gradient
  only through the normalised weights of the chosen experts;
* grad of w[t, j]: dw = rsf * <dout[t], y_{e_j}(x[t])>;
* through the normalisation w_j = s_j / S (S = sum of the chosen s):
  ds_j = (dw_j - sum_i w_i dw_i) / S;
* through the sigmoid: dz_j = ds_j * s_j * (1 - s_j); every other logit's
  gradient is 0; d W_r = dz^T x, and dz W_r adds to dx;
* inside expert e, for its rows: gy = rsf * w * dout (the gradient of y),
  dh = gy W_down, du = dh * silu(g), dg = dh * u * silu'(g) with
  silu'(g) = sigmoid(g) * (1 + g * (1 - sigmoid(g))); dx += dg W_gate +
  du W_up; d W_down = gy^T h, d W_gate = dg^T x, d W_up = du^T x.

The bias step: the model doc ("Overview") says a learned per-expert bias
balances the load in place of an auxiliary loss, and the launch post says the
routing follows DeepSeek-V3's scheme. That scheme's published rule (its
auxiliary-loss-free balancing) moves every bias by a fixed step against its
expert's excess load: b_e <- b_e + gamma * sign(mean load - load_e). The
pages do not print the rule or gamma (parity unpinned for that reading; the
arithmetic of the step is pinned).
"""

import numpy as np

from .routing import route, sigmoid, weights_for
from .experts import silu, _expert_getter


def dsilu(g):
    """silu'(g) = sigmoid(g) * (1 + g * (1 - sigmoid(g))), float64."""
    g = np.asarray(g, dtype=np.float64)
    sg = sigmoid(g)
    return sg * (1.0 + g * (1.0 - sg))


def backward(x, router_w, expert_bias, experts, dout, n_group=8, topk_group=4, top_k=8,
             routed_scaling_factor=2.5, routing=None, weight_grads=True, only_experts=None):
    """Gradients of L = sum(dout * out) for the block's forward.

    ``experts`` as for :func:`oracle.experts.forward` (three arrays or a
    callable ``get_expert(e)``); ``routing`` optionally forces the expert
    choice. Returns a dict:

    * ``dx`` [T, H], ``d_router_w`` [E, H];
    * ``d_w_gate``, ``d_w_up``, ``d_w_down``: {expert: array} for every
      expert some token chose (the others' gradients are 0), when
      ``weight_grads``;
    * ``dw`` [T, top_k] (gradient of the normalised weights), ``ds`` and
      ``dz`` [T, top_k] (of the chosen scores and logits);
    * ``route``: the routing dict of :func:`oracle.routing.route`.

    ``only_experts`` (a set of expert indices) runs only those experts: their
    weight gradients are complete (they depend on no other expert), while
    dx, dw and the router gradient then lack the other experts' terms.
    """
    x = np.asarray(x, dtype=np.float64)
    W_r = np.asarray(router_w, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    rsf = float(routed_scaling_factor)
    T, H = x.shape
    E = W_r.shape[0]
    r = route(x, W_r, expert_bias, n_group, topk_group, top_k)
    if routing is not None:
        r["idx"] = np.asarray(routing, dtype=np.int64)
        r["w"] = weights_for(r["s"], r["idx"])
    idx, w = r["idx"], r["w"]
    get = _expert_getter(experts)

    dx = np.zeros((T, H))
    dw = np.zeros(idx.shape)
    grads = {"d_w_gate": {}, "d_w_up": {}, "d_w_down": {}}
    for e in np.unique(idx):
        if only_experts is not None and int(e) not in only_experts:
            continue
        tok, slot = np.nonzero(idx == e)
        wg, wu, wd = (np.asarray(m, dtype=np.float64) for m in get(int(e)))
        xr = x[tok]
        g = xr @ wg.T
        u = xr @ wu.T
        a = silu(g)
        h = a * u
        y = h @ wd.T
        dw[tok, slot] = rsf * np.sum(dout[tok] * y, axis=1)
        gy = (rsf * w[tok, slot])[:, None] * dout[tok]
        dh = gy @ wd
        du = dh * a
        dg = dh * u * dsilu(g)
        np.add.at(dx, tok, dg @ wg + du @ wu)
        if weight_grads:
            grads["d_w_down"][int(e)] = gy.T @ h
            grads["d_w_gate"][int(e)] = dg.T @ xr
            grads["d_w_up"][int(e)] = du.T @ xr

    s_sel = np.take_along_axis(r["s"], idx, axis=1)
    S = s_sel.sum(axis=1, keepdims=True)
    ds = (dw - np.sum(w * dw, axis=1, keepdims=True)) / S
    dz = ds * s_sel * (1.0 - s_sel)
    dz_full = np.zeros((T, E))
    np.put_along_axis(dz_full, idx, dz, axis=1)
    dx += dz_full @ W_r
    out = {"dx": dx, "d_router_w": dz_full.T @ x, "dw": dw, "ds": ds, "dz": dz, "route": r}
    if weight_grads:
        out.update(grads)
    return out


def bias_step(expert_bias, counts, gamma):
    """One balancing step: b_e + gamma * sign(mean(counts) - counts[e]) (float64)."""
    c = np.asarray(counts, dtype=np.float64)
    return np.asarray(expert_bias, dtype=np.float64) + gamma * np.sign(c.mean() - c)

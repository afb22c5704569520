"""Pins of the oracle's backward pass and balancing step (oracle/backward.py).

* central finite differences of L = sum(dout * out), with the oracle's own
  forward, for every parameter of a tiny block (the expert choice is checked
  to stay fixed under each perturbation);
* torch.autograd in float64 through an independently written torch forward
  of the block (the expert choice fixed to the oracle's);
* closed forms: the normalised weights do not change when all chosen scores
  are scaled, so sum_j s_j ds_j = 0; with one expert per token the weight is
  always 1 and the router gets no gradient; the gradients are linear in dout.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob


def _problem(T, H, I, E, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, H))
    rw = rng.normal(size=(E, H)) * scale / np.sqrt(H)
    b = rng.normal(size=E) * 0.01
    wg = rng.normal(size=(E, I, H)) * 0.3
    wu = rng.normal(size=(E, I, H)) * 0.3
    wd = rng.normal(size=(E, H, I)) * 0.3
    dout = rng.normal(size=(T, H))
    return x, rw, b, wg, wu, wd, dout


TINY = dict(n_group=4, topk_group=2, top_k=4, routed_scaling_factor=2.5)


def _loss(x, rw, b, wg, wu, wd, dout, idx0):
    out, r = oracle.forward(x, rw, b, (wg, wu, wd), **TINY)
    assert np.array_equal(r["idx"], idx0), "perturbation changed the expert choice"
    return float(np.sum(out * dout))


def test_finite_differences_every_parameter():
    x, rw, b, wg, wu, wd, dout = _problem(3, 8, 4, 16, 0)
    g = ob.backward(x, rw, b, (wg, wu, wd), dout, **TINY)
    idx0 = g["route"]["idx"]
    # every input with a gradient (the bias has none: it enters the selection only)
    params = {"x": x, "rw": rw, "wg": wg, "wu": wu, "wd": wd}
    expect = {"x": g["dx"], "rw": g["d_router_w"]}
    for key, name in (("wg", "d_w_gate"), ("wu", "d_w_up"), ("wd", "d_w_down")):
        full = np.zeros_like(params[key])
        for e, m in g[name].items():
            full[e] = m
        expect[key] = full
    h = 1e-6
    for key, arr in params.items():
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + h
            lp = _loss(x, rw, b, wg, wu, wd, dout, idx0)
            arr[i] = old - h
            lm = _loss(x, rw, b, wg, wu, wd, dout, idx0)
            arr[i] = old
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(expect[key], fd, rtol=1e-6, atol=1e-7, err_msg=key)


def _torch_forward(x, rw, wg, wu, wd, idx, rsf):
    """The block in torch with a fixed expert choice ``idx`` [T, k]."""
    s = torch.sigmoid(x @ rw.T)
    s_sel = torch.gather(s, 1, idx)
    w = s_sel / s_sel.sum(dim=1, keepdim=True)
    g = torch.einsum("tkih,th->tki", wg[idx], x)
    u = torch.einsum("tkih,th->tki", wu[idx], x)
    h = torch.nn.functional.silu(g) * u
    y = torch.einsum("tkhi,tki->tkh", wd[idx], h)
    return rsf * torch.einsum("tk,tkh->th", w, y)


@pytest.mark.parametrize("seed", [1, 2])
def test_matches_torch_autograd(seed):
    T, H, I, E = 16, 32, 16, 32
    x, rw, b, wg, wu, wd, dout = _problem(T, H, I, E, seed, scale=3.0)
    kw = dict(n_group=8, topk_group=4, top_k=8, routed_scaling_factor=2.5)
    g = ob.backward(x, rw, b, (wg, wu, wd), dout, **kw)
    tens = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True)
            for k, v in dict(x=x, rw=rw, wg=wg, wu=wu, wd=wd).items()}
    idx = torch.tensor(g["route"]["idx"])
    out = _torch_forward(tens["x"], tens["rw"], tens["wg"], tens["wu"], tens["wd"], idx, 2.5)
    out.backward(torch.tensor(dout))
    np.testing.assert_allclose(g["dx"], tens["x"].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["d_router_w"], tens["rw"].grad.numpy(), rtol=1e-10, atol=1e-12)
    for key, name in (("wg", "d_w_gate"), ("wu", "d_w_up"), ("wd", "d_w_down")):
        ref = tens[key].grad.numpy()
        chosen = set(int(e) for e in np.unique(g["route"]["idx"]))
        for e in range(E):
            if e in chosen:
                np.testing.assert_allclose(g[name][e], ref[e], rtol=1e-10, atol=1e-12)
            else:
                assert e not in g[name] and np.all(ref[e] == 0)


def test_weight_normalisation_is_scale_invariant():
    x, rw, b, wg, wu, wd, dout = _problem(32, 16, 8, 32, 3, scale=2.0)
    g = ob.backward(x, rw, b, (wg, wu, wd), dout, n_group=8, topk_group=4, top_k=8)
    s_sel = np.take_along_axis(g["route"]["s"], g["route"]["idx"], axis=1)
    lhs = np.sum(s_sel * g["ds"], axis=1)
    assert np.all(np.abs(lhs) <= 1e-12 * np.sum(np.abs(s_sel * g["ds"]), axis=1) + 1e-15)
    assert np.max(np.abs(g["ds"])) > 1e-3  # not vacuous


def test_single_expert_gives_no_router_gradient():
    x, rw, b, wg, wu, wd, dout = _problem(8, 16, 8, 32, 4, scale=2.0)
    g = ob.backward(x, rw, b, (wg, wu, wd), dout, n_group=8, topk_group=4, top_k=1)
    assert np.all(g["route"]["w"] == 1.0)
    assert np.all(g["dz"] == 0.0) and np.all(g["d_router_w"] == 0.0)
    # dx is then the expert path alone: rsf * J_e^T dout
    e = g["route"]["idx"][:, 0]
    for t in range(8):
        xt = x[t]
        gg = wg[e[t]] @ xt
        uu = wu[e[t]] @ xt
        dh = 2.5 * (wd[e[t]].T @ dout[t])
        sg = 1.0 / (1.0 + np.exp(-gg))
        dgg = dh * uu * sg * (1.0 + gg * (1.0 - sg))
        duu = dh * gg * sg
        np.testing.assert_allclose(g["dx"][t], wg[e[t]].T @ dgg + wu[e[t]].T @ duu, rtol=1e-12)


def test_linear_in_dout():
    x, rw, b, wg, wu, wd, d1 = _problem(16, 16, 8, 32, 5, scale=2.0)
    d2 = np.random.default_rng(9).normal(size=d1.shape)
    kw = dict(n_group=8, topk_group=4, top_k=8)
    g1 = ob.backward(x, rw, b, (wg, wu, wd), d1, **kw)
    g2 = ob.backward(x, rw, b, (wg, wu, wd), d2, **kw)
    g3 = ob.backward(x, rw, b, (wg, wu, wd), 2.0 * d1 - 3.0 * d2, **kw)
    for k in ("dx", "d_router_w"):
        np.testing.assert_allclose(g3[k], 2.0 * g1[k] - 3.0 * g2[k], rtol=1e-10, atol=1e-12)


def test_bias_step():
    b = np.array([0.1, -0.2, 0.0, 0.05])
    got = ob.bias_step(b, np.array([1, 3, 2, 2]), 1e-3)
    np.testing.assert_array_equal(got, b + 1e-3 * np.array([1.0, -1.0, 0.0, 0.0]))
    # balanced load leaves the bias alone
    np.testing.assert_array_equal(ob.bias_step(b, np.full(4, 7), 0.5), b)


def test_dsilu_closed_form():
    g = np.linspace(-20, 20, 2001)
    h = 1e-6
    fd = (oracle.experts.silu(g + h) - oracle.experts.silu(g - h)) / (2 * h)
    np.testing.assert_allclose(ob.dsilu(g), fd, rtol=1e-7, atol=1e-9)
    assert ob.dsilu(0.0) == 0.5


def test_only_experts_keeps_their_weight_gradients():
    x, rw, b, wg, wu, wd, dout = _problem(24, 16, 8, 32, 6, scale=2.0)
    kw = dict(n_group=8, topk_group=4, top_k=8)
    full = ob.backward(x, rw, b, (wg, wu, wd), dout, **kw)
    chosen = sorted(full["d_w_gate"])
    sub = set(chosen[::3])
    part = ob.backward(x, rw, b, (wg, wu, wd), dout, only_experts=sub, **kw)
    assert set(part["d_w_gate"]) == sub
    for name in ("d_w_gate", "d_w_up", "d_w_down"):
        for e in sub:
            np.testing.assert_array_equal(part[name][e], full[name][e])

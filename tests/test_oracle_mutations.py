"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of an oracle function (on the CPU,
by monkeypatching) and checks that at least one pin then fails. This shows
that the pins constrain the oracle rather than restate it.
"""

import numpy as np
import pytest

import oracle
import oracle.experts as ox
import oracle.routing as orr
from oracle import e4m3

import oracle.backward as ob
import test_oracle_backward as tb
import test_oracle_e4m3 as te
import test_oracle_experts as tx
import test_oracle_routing as tr


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def _group_scores_max(key, n_group):
    T, E = key.shape
    return np.asarray(key).reshape(T, n_group, E // n_group).max(axis=2)


def _group_scores_top3(key, n_group):
    T, E = key.shape
    b = np.sort(np.asarray(key).reshape(T, n_group, E // n_group), axis=2)
    return b[:, :, -1] + b[:, :, -2] + b[:, :, -3]


def _order_unstable(values):
    # ties to the higher index
    v = np.asarray(values)
    return np.argsort(-v[:, ::-1], axis=1, kind="stable")[:, :] * -1 + (v.shape[1] - 1)


def test_group_score_as_max_is_caught(monkeypatch):
    monkeypatch.setattr(orr, "group_scores", _group_scores_max)
    assert _fails(tr.test_golden_group_score_is_top2_sum) or _fails(tr.test_bruteforce_group_subsets_full_shape)


def test_group_score_top3_is_caught(monkeypatch):
    monkeypatch.setattr(orr, "group_scores", _group_scores_top3)
    assert _fails(tr.test_bruteforce_group_subsets_full_shape)


def test_tie_to_higher_index_is_caught(monkeypatch):
    monkeypatch.setattr(orr, "_order_desc", _order_unstable)
    assert _fails(tr.test_all_equal_keys_tie_rule)


def test_bias_in_weights_is_caught(monkeypatch):
    real = orr.route

    def route_bias_in_w(x, rw, b, n_group=8, topk_group=4, top_k=8):
        r = real(x, rw, b, n_group, topk_group, top_k)
        k = np.take_along_axis(r["key"], r["idx"], 1)
        r["w"] = k / k.sum(1, keepdims=True)
        return r

    monkeypatch.setattr(orr, "route", route_bias_in_w)
    monkeypatch.setattr(oracle, "route", route_bias_in_w)
    assert _fails(tr.test_forced_set_by_bias)


def test_outside_groups_zeroed_is_caught(monkeypatch):
    real = orr.select_from_keys

    def zero_fill(key, n_group, topk_group, top_k):
        r = real(key, n_group, topk_group, top_k)
        masked = np.where(np.isfinite(r["masked_key"]), r["masked_key"], 0.0)
        r["idx"] = np.argsort(-masked, axis=1, kind="stable")[:, :top_k]
        return r

    monkeypatch.setattr(oracle, "select_from_keys", zero_fill)
    assert _fails(tr.test_outside_kept_groups_never_chosen_even_with_negative_keys)


def test_missing_scale_is_caught(monkeypatch):
    real = ox._combine
    monkeypatch.setattr(ox, "_combine", lambda x, idx, w, rsf, g, fp8: real(x, idx, w, 1.0, g, fp8))
    assert _fails(tx.test_identical_experts_closed_form)


def test_silu_sign_is_caught(monkeypatch):
    monkeypatch.setattr(ox, "silu", lambda v: np.asarray(v) / (1.0 + np.exp(np.asarray(v))))
    assert _fails(tx.test_expert_matches_torch_swiglu)


def test_gate_up_swapped_is_caught(monkeypatch):
    real = ox.expert_ffn
    monkeypatch.setattr(oracle, "expert_ffn", lambda x, g, u, d, quantize_h=False: real(x, u, g, d, quantize_h))
    assert _fails(tx.test_expert_matches_torch_swiglu)


def test_round_half_up_is_caught(monkeypatch):
    real_rint = np.rint

    class NP:
        def __getattr__(self, k):
            if k == "rint":
                return lambda a: np.floor(np.asarray(a) + 0.5)
            return getattr(np, k)

    monkeypatch.setattr(e4m3, "np", NP())
    assert _fails(te.test_midpoints_against_torch)
    assert real_rint is np.rint


def test_wrong_exponent_bias_is_caught(monkeypatch):
    real_decode = e4m3.decode
    monkeypatch.setattr(e4m3, "decode", lambda c: real_decode(c) * 2.0)
    assert _fails(te.test_known_codes)


def test_backward_silu_derivative_as_sigmoid_is_caught(monkeypatch):
    monkeypatch.setattr(ob, "dsilu", orr.sigmoid)
    assert _fails(tb.test_finite_differences_every_parameter)
    assert _fails(tb.test_matches_torch_autograd, 1)


def test_backward_sigmoid_slope_dropped_is_caught(monkeypatch):
    # the router gradient computed from ds instead of dz (the sigmoid's slope
    # s (1 - s) left out)
    real = ob.backward

    def no_slope(x, router_w, *a, **k):
        out = real(x, router_w, *a, **k)
        ds_full = np.zeros((out["ds"].shape[0], np.asarray(router_w).shape[0]))
        np.put_along_axis(ds_full, out["route"]["idx"], out["ds"], axis=1)
        out["d_router_w"] = ds_full.T @ np.asarray(x)
        return out

    monkeypatch.setattr(ob, "backward", no_slope)
    assert _fails(tb.test_finite_differences_every_parameter)
    assert _fails(tb.test_matches_torch_autograd, 2)


def test_row_quantiser_dividing_by_the_scale_is_caught(monkeypatch):
    """Quantising a row as e4m3(v / fp32(amax / 448)) instead of
    e4m3(v * fp32(448 / amax))."""
    def quantize_rows_div(v):
        v32 = np.asarray(v, dtype=np.float32)
        amax = np.max(np.abs(v32), axis=1)
        zero = amax == 0
        safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
        scale = (safe / np.float32(e4m3.FP8_MAX)).astype(np.float32)
        codes = e4m3.encode((v32 / scale[:, None]).astype(np.float32).astype(np.float64))
        codes[zero, :] = 0
        return codes, np.where(zero, np.float32(1.0), scale).astype(np.float32)
    monkeypatch.setattr(e4m3, "quantize_rows", quantize_rows_div)
    assert _fails(te.test_quantize_rows_multiplies_by_the_fp32_reciprocal)


def test_quantised_h_without_bf16_storage_is_caught(monkeypatch):
    """Quantising the fp32 intermediate directly instead of its stored bf16
    values."""
    import oracle.bf16 as ob16
    import test_oracle_bf16 as tb16
    monkeypatch.setattr(ob16, "round_to_bf16", lambda v: np.asarray(v, dtype=np.float64))
    assert _fails(tb16.test_quantised_expert_quantises_the_stored_bf16_h)

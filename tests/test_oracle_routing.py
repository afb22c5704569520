"""Pins of the oracle's routing against what the pages and mathematics fix.

Rule (Beam launch post, "Mixture of Experts"; model doc "Beam", "Overview"):
sigmoid scores, 8 groups of 32 ranked by the sum of their two best keys, keep
4 groups, top 8 experts inside them, normalised weights. The checks here do
not reuse the oracle's sort code: brute force enumerates subsets with
itertools, hand-built cases come from tests/golden/, and invariants are
counted directly.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.routing import counts, weights_for
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(seed=0):
    cfg = workloads.workload("tiny")
    x, rw, b = workloads.make_small_inputs(cfg, seed)
    return cfg, x.double().numpy(), rw.double().numpy(), b.double().numpy()


# ---------------------------------------------------------------- P-a invariants
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants_tiny(seed):
    cfg, x, rw, b = _tiny(seed)
    r = oracle.route(x, rw, b, cfg["n_group"], cfg["topk_group"], cfg["top_k"])
    idx, w = r["idx"], r["w"]
    T, k = idx.shape
    assert k == 8
    gs = cfg["n_experts"] // cfg["n_group"]
    for t in range(T):
        chosen = idx[t].tolist()
        assert len(set(chosen)) == 8, "exactly 8 distinct experts"
        groups = {e // gs for e in chosen}
        assert len(groups) <= 4, "experts drawn from at most 4 groups"
        assert groups <= set(r["kept_groups"][t].tolist()), "all from kept groups"
        keys = r["key"][t, chosen]
        assert np.all(np.diff(keys) <= 0), "ordered by key descending"
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose((2.5 * w).sum(axis=1), 2.5, rtol=0, atol=1e-12)
    assert np.all(w > 0) and np.all(w < 1)
    c = counts(idx, cfg["n_experts"])
    assert c.sum() == 8 * T


# ---------------------------------------------------------------- P-b brute force
def _brute_top2(vals):
    """Largest sum of two distinct entries (enumerate all pairs)."""
    return max(vals[i] + vals[j] for i, j in itertools.combinations(range(len(vals)), 2))


def _brute_select(key_row, n_group, topk_group, top_k):
    """Brute-force group-limited selection of one token.

    Group score = the largest pair sum in the group; kept groups = the
    topk_group-subset with the largest total group score; chosen experts = the
    top_k-subset of candidates with the largest total key.
    """
    E = len(key_row)
    gs = E // n_group
    gscore = [_brute_top2(key_row[g * gs:(g + 1) * gs]) for g in range(n_group)]
    best_groups = max(itertools.combinations(range(n_group), topk_group),
                      key=lambda sub: sum(gscore[g] for g in sub))
    cand = [e for g in best_groups for e in range(g * gs, (g + 1) * gs)]
    best_experts = max(itertools.combinations(cand, top_k), key=lambda sub: sum(key_row[e] for e in sub))
    return set(best_groups), set(best_experts)


def test_bruteforce_group_subsets_full_shape():
    """Full Beam shape: the kept groups maximise the summed group score over all
    C(8, 4) = 70 group subsets."""
    cfg, x, rw, b = _tiny(0)
    r = oracle.route(x, rw, b, 8, 4, 8)
    key = r["key"]
    for t in range(key.shape[0]):
        gscore = [_brute_top2(key[t, g * 32:(g + 1) * 32]) for g in range(8)]
        best = max(itertools.combinations(range(8), 4), key=lambda sub: sum(gscore[g] for g in sub))
        assert set(best) == set(r["kept_groups"][t].tolist())
        np.testing.assert_allclose(r["group_score"][t], gscore, rtol=0, atol=1e-15)


@pytest.mark.parametrize("E,n_group,topk_group,top_k", [(32, 8, 4, 8), (16, 4, 2, 4), (24, 6, 3, 5)])
def test_bruteforce_expert_subsets_reduced(E, n_group, topk_group, top_k):
    """Reduced shapes through the oracle's general parameters: the whole
    selection equals exhaustive search over group subsets and expert subsets
    (E=32: C(16, 8) = 12,870 expert subsets per token)."""
    rng = np.random.default_rng(E)
    T, H = 12, 16
    x = rng.standard_normal((T, H))
    rw = rng.standard_normal((E, H)) / math.sqrt(H)
    b = rng.standard_normal(E) * 0.01
    r = oracle.route(x, rw, b, n_group, topk_group, top_k)
    for t in range(T):
        groups, experts = _brute_select(list(r["key"][t]), n_group, topk_group, top_k)
        assert set(r["kept_groups"][t].tolist()) == groups
        assert set(r["idx"][t].tolist()) == experts


# ---------------------------------------------------------------- P-c special cases
def test_group_limit_inactive_equals_plain_topk():
    """kg = G (or G = 1): the group limit does nothing, so the choice is the plain
    top-8 of s + b; checked against torch.topk (a different library routine)."""
    import torch
    cfg, x, rw, b = _tiny(3)
    for n_group, topk_group in [(8, 8), (1, 1)]:
        r = oracle.route(x, rw, b, n_group, topk_group, 8)
        key = torch.from_numpy(r["key"])
        vals, ref = torch.topk(key, 8, dim=1, largest=True, sorted=True)
        assert np.array_equal(np.sort(r["idx"], axis=1), np.sort(ref.numpy(), axis=1))
        np.testing.assert_array_equal(np.take_along_axis(r["key"], r["idx"], 1), vals.numpy())


def test_top1_weight_is_exactly_one():
    cfg, x, rw, b = _tiny(4)
    r = oracle.route(x, rw, b, 8, 4, 1)
    assert np.all(r["w"] == 1.0)


def test_forced_set_by_bias():
    """+10 on 8 experts spread over 3 groups forces exactly those 8; the weights
    still come from the unbiased sigmoid scores."""
    cfg, x, rw, b = _tiny(5)
    forced = [3, 17, 40, 41, 42, 100, 101, 127]  # groups 0, 1, 3
    b2 = b.copy()
    b2[forced] += 10.0
    r = oracle.route(x, rw, b2, 8, 4, 8)
    for t in range(x.shape[0]):
        assert set(r["idx"][t].tolist()) == set(forced)
    s = r["s"]
    sel = np.take_along_axis(s, r["idx"], 1)
    np.testing.assert_allclose(r["w"], sel / sel.sum(1, keepdims=True), rtol=1e-15)
    # the bias does not leak into the weights: they differ from normalised keys
    keys = np.take_along_axis(r["key"], r["idx"], 1)
    assert not np.allclose(r["w"], keys / keys.sum(1, keepdims=True))


def test_all_equal_keys_tie_rule():
    """W_r = 0, b = 0: every key is sigmoid(0) = 0.5, all group scores tie, so the
    lower-index rule keeps groups 0-3 and chooses experts 0-7 with weight 1/8."""
    T, H, E = 5, 8, 256
    x = np.ones((T, H))
    r = oracle.route(x, np.zeros((E, H)), np.zeros(E), 8, 4, 8)
    assert np.all(r["s"] == 0.5)
    for t in range(T):
        assert r["kept_groups"][t].tolist() == [0, 1, 2, 3]
        assert r["idx"][t].tolist() == list(range(8))
    assert np.all(r["w"] == 0.125)
    assert np.all(r["margin"] == 0.0)


def test_golden_group_score_is_top2_sum():
    with open(os.path.join(GOLDEN, "group_limit_case.json")) as f:
        g = json.load(f)
    key = np.full((1, g["n_experts"]), g["background_key"])
    for e, v in g["set_keys"].items():
        key[0, int(e)] = v
    r = oracle.select_from_keys(key, g["n_group"], g["topk_group"], g["top_k"])
    assert r["kept_groups"][0].tolist() == g["expected_kept_groups"]
    assert r["idx"][0].tolist() == g["expected_idx"]
    assert sorted(r["kept_groups"][0].tolist()) != g["expected_if_group_score_were_max_key_kept_groups"]


def test_outside_kept_groups_never_chosen_even_with_negative_keys():
    """Keys inside kept groups can be negative (b < -s); experts outside the
    kept groups must still never be chosen (they are excluded, not zeroed)."""
    E = 256
    key = np.full((1, E), -0.5)
    key[0, 0:2] = [0.9, 0.8]        # group 0 wins on its top-2 sum
    key[0, 32:34] = [0.7, 0.6]      # group 1
    key[0, 64:66] = [0.5, 0.4]      # group 2
    key[0, 96:98] = [0.3, 0.2]      # group 3
    r = oracle.select_from_keys(key, 8, 4, 8)
    chosen = set(r["idx"][0].tolist())
    assert chosen == {0, 1, 32, 33, 64, 65, 96, 97}
    r = oracle.select_from_keys(key, 8, 4, 10)   # must now take -0.5 keys from kept groups
    assert all(e // 32 in {0, 1, 2, 3} for e in r["idx"][0])


# ---------------------------------------------------------------- sigmoid
def test_sigmoid_values():
    s = oracle.sigmoid(np.array([0.0, 800.0, -800.0, 1.0, -1.0]))
    assert s[0] == 0.5 and s[1] == 1.0 and s[2] == 0.0
    assert abs(s[3] + s[4] - 1.0) < 1e-16
    assert abs(s[3] - 0.7310585786300049) < 1e-15  # 1/(1+1/e), from tables


# ---------------------------------------------------------------- P-g equivariance
def test_equivariance():
    cfg, x, rw, b = _tiny(6)
    r = oracle.route(x, rw, b, 8, 4, 8)
    rng = np.random.default_rng(0)
    perm = rng.permutation(x.shape[0])
    rp = oracle.route(x[perm], rw, b, 8, 4, 8)
    assert np.array_equal(rp["idx"], r["idx"][perm])
    # relabel experts inside every group and relabel whole groups
    gperm = rng.permutation(8)
    inner = np.stack([rng.permutation(32) for _ in range(8)])
    new_of_old = np.empty(256, dtype=np.int64)
    for g in range(8):
        for i in range(32):
            new_of_old[g * 32 + i] = gperm[g] * 32 + inner[g, i]
    rw2 = np.empty_like(rw)
    b2 = np.empty_like(b)
    rw2[new_of_old] = rw
    b2[new_of_old] = b
    r2 = oracle.route(x, rw2, b2, 8, 4, 8)
    assert np.array_equal(np.sort(r2["idx"], 1), np.sort(new_of_old[r["idx"]], 1))
    np.testing.assert_allclose(np.sort(r2["w"], 1), np.sort(r["w"], 1), rtol=1e-14)


def test_near_tie_margin():
    """The margin is the distance to the nearest different selection."""
    E = 256
    key = np.linspace(0, 1, E)[None, :].copy()
    r = oracle.select_from_keys(key, 8, 4, 8)
    gs = r["group_score"][0]
    srt = np.sort(gs)[::-1]
    kept_keys = np.sort(r["masked_key"][0][np.isfinite(r["masked_key"][0])])[::-1]
    assert r["margin"][0] == pytest.approx(min(srt[3] - srt[4], kept_keys[7] - kept_keys[8]), abs=0)

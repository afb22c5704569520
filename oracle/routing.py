"""Oracle: group-limited sigmoid routing (float64, numpy).

Test infrastructure only; see the package docstring.

The routing rule is stated in the Beam launch post, section "Mixture of
Experts", and in the transformers model doc "Beam", section "Overview":

1. score every expert with a sigmoid of its router logit;
2. split the experts into ``n_group`` groups (Beam: 8 groups of 32) and
   score each group by the sum of its two largest scores;
3. keep the ``topk_group`` best groups (Beam: 4);
4. choose the ``top_k`` best experts inside the kept groups (Beam: 8);
5. normalise the chosen experts' weights.

The per-expert bias of the model doc balances load by changing which
experts are chosen; it is added to the score for steps 2-4 only (the
"selection key"), and the weights of step 5 use the unbiased sigmoid.
"""

import numpy as np


def sigmoid(z):
    """s = 1 / (1 + e^(-z)), elementwise, float64.

    Beam launch post, "Mixture of Experts": experts are scored with a
    sigmoid. Written in the form that never overflows for large |z|.
    """
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def group_scores(key, n_group):
    """Sum of the two largest keys in each contiguous block of experts.

    ``key`` is [T, E]; group g holds experts g*E/n_group .. (g+1)*E/n_group-1
    (contiguous blocks, the plainest reading of "split into 8 groups of 32").
    Returns [T, n_group] float64.
    """
    key = np.asarray(key, dtype=np.float64)
    T, E = key.shape
    gs = E // n_group
    if gs * n_group != E or gs < 2:
        raise ValueError("n_experts must split into groups of at least 2")
    blocks = np.sort(key.reshape(T, n_group, gs), axis=2)  # ascending
    return blocks[:, :, -1] + blocks[:, :, -2]


def _order_desc(values):
    """Indices that order each row by value descending, ties to the lower index.

    A stable ascending sort of the negated values keeps equal values in index
    order, so the lower index comes first among equals.
    """
    return np.argsort(-values, axis=1, kind="stable")


def select_from_keys(key, n_group, topk_group, top_k):
    """Group-limited top-k on precomputed selection keys.

    ``key`` [T, E] float64. Returns a dict:

    * ``idx`` [T, top_k] int64: chosen experts ordered by key descending,
      equal keys by index ascending;
    * ``group_score`` [T, n_group]; ``kept_groups`` [T, topk_group] (best
      first, equal scores to the lower group index);
    * ``masked_key`` [T, E]: the key inside kept groups, -inf elsewhere;
    * ``margin`` [T]: the smaller of (4th minus 5th group score) and (8th
      minus 9th candidate key), i.e. how far the token is from a different
      selection; +inf where a boundary does not exist.
    """
    key = np.asarray(key, dtype=np.float64)
    T, E = key.shape
    gs = E // n_group
    if not (1 <= topk_group <= n_group):
        raise ValueError("topk_group out of range")
    if not (1 <= top_k <= topk_group * gs):
        raise ValueError("top_k out of range")
    gsc = group_scores(key, n_group)
    gorder = _order_desc(gsc)
    kept = gorder[:, :topk_group]

    group_of_expert = np.arange(E) // gs
    keep_mask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep_mask, kept, True, axis=1)
    cand = keep_mask[:, group_of_expert]  # [T, E]
    masked = np.where(cand, key, -np.inf)

    eorder = _order_desc(masked)
    idx = eorder[:, :top_k]

    sorted_g = np.take_along_axis(gsc, gorder, axis=1)
    if topk_group < n_group:
        gmargin = sorted_g[:, topk_group - 1] - sorted_g[:, topk_group]
    else:
        gmargin = np.full(T, np.inf)
    sorted_k = np.take_along_axis(masked, eorder, axis=1)
    if top_k < topk_group * gs:
        kmargin = sorted_k[:, top_k - 1] - sorted_k[:, top_k]
    else:
        kmargin = np.full(T, np.inf)
    return {
        "idx": idx,
        "group_score": gsc,
        "kept_groups": kept,
        "masked_key": masked,
        "margin": np.minimum(gmargin, kmargin),
    }


def route(x, router_w, expert_bias, n_group=8, topk_group=4, top_k=8):
    """Full router: logits, sigmoid, biased selection, normalised weights.

    x [T, H], router_w [E, H] (row e is expert e's router vector),
    expert_bias [E]. All are upcast to float64 (exact for bf16 and fp32).

    Returns the dict of :func:`select_from_keys` plus
    ``z`` [T, E] (pre-sigmoid router logits, the values the model doc's
    "Notes" section says are returned on request), ``s`` [T, E] sigmoid
    scores, ``key`` = s + bias, and ``w`` [T, top_k]: the chosen experts'
    unbiased scores divided by their sum (launch post, "Mixture of
    Experts": normalised router weights). The 2.5 scale is not applied
    here; see :func:`oracle.experts.forward`.
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(router_w, dtype=np.float64)
    b = np.asarray(expert_bias, dtype=np.float64)
    z = x @ W.T
    s = sigmoid(z)
    key = s + b[None, :]
    r = select_from_keys(key, n_group, topk_group, top_k)
    s_sel = np.take_along_axis(s, r["idx"], axis=1)
    r["w"] = s_sel / s_sel.sum(axis=1, keepdims=True)
    r["z"] = z
    r["s"] = s
    r["key"] = key
    return r


def weights_for(s, idx):
    """Normalised weights of a given (possibly forced) selection ``idx``."""
    s_sel = np.take_along_axis(np.asarray(s, dtype=np.float64), np.asarray(idx), axis=1)
    return s_sel / s_sel.sum(axis=1, keepdims=True)


def counts(idx, n_experts):
    """Tokens per expert: counts[e] = number of (t, j) with idx[t, j] == e."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=n_experts).astype(np.int64)

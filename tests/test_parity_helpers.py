"""Host logic of the parity tests (no GPU): the sorted order rebuilt from a
routing, the M-tile coverage of a token sample, and the decode tables that
stand in for the oracle's per-weight decoders."""

import numpy as np
import pytest
import torch

import oracle
from parity import (GUARD, Guarded, coverage_report, e4m3_dequantize, expert_rows, mx_dequantize,
                    tile_cover, tiles_covered)


def _routing(T, E=256, k=8, hot=(), seed=0):
    """A random routing with distinct experts per token; tokens pick the
    experts in ``hot`` with probability about 2/3 each."""
    rng = np.random.default_rng(seed)
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        chosen = [e for e in hot if rng.random() < 2 / 3][:k]
        rest = rng.permutation(np.setdiff1d(np.arange(E), chosen))[:k - len(chosen)]
        idx[t] = rng.permutation(np.concatenate([chosen, rest]).astype(np.int64))
    return idx


def test_expert_rows_is_the_stable_sorted_order():
    idx = _routing(300)
    rows = expert_rows(idx, 256)
    assert sum(len(r) for r in rows) == idx.size
    for e, r in enumerate(rows):
        assert np.all(np.diff(r) > 0)  # ascending tokens, each once
        assert np.array_equal(r, np.nonzero(np.any(idx == e, axis=1))[0])


def test_tile_cover_reaches_every_tile_of_hot_experts():
    idx = _routing(4000, hot=range(8), seed=1)
    toks = tile_cover(idx, 256, 128, seed=3)
    rows = expert_rows(idx, 256)
    assert max(len(r) for r in rows[:8]) > 9 * 256  # many M-tiles per hot expert
    rep = coverage_report(toks, idx, 256, bms=(16, 128, 256))
    assert rep["tiles_covered_128"] == rep["tiles_total_128"]
    assert rep["tiles_covered_256"] == rep["tiles_total_256"]
    # 16-row tiles are finer than the sample: some are missed (the count is real)
    assert rep["tiles_covered_16"] < rep["tiles_total_16"]
    # first and last row of every 128-row block are in the sample
    pick = set(toks.tolist())
    for r in rows:
        for m0 in range(0, len(r), 128):
            assert r[m0] in pick and r[min(m0 + 128, len(r)) - 1] in pick


def test_tiles_covered_counts_a_missing_tile():
    idx = _routing(2000, hot=range(4), seed=2)
    toks = set(tile_cover(idx, 256, 128, seed=0).tolist())
    rows = expert_rows(idx, 256)
    r0 = rows[0]
    # drop every token of expert 0's third 128-row block
    gone = set(r0[256:384].tolist())
    left = np.array(sorted(toks - gone))
    c, t = tiles_covered(left, idx, 256, 128)
    assert c <= t - 1


def test_decode_tables_equal_the_oracle_decoders():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, size=(64, 512), dtype=np.uint8)
    sc = rng.random(64).astype(np.float32)
    got = e4m3_dequantize(codes, sc)
    want = oracle.e4m3.decode(codes) * sc.astype(np.float64)[:, None]
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.nan_to_num(got), np.nan_to_num(want))
    packed = rng.integers(0, 256, size=(32, 256), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(32, 16), dtype=np.uint8)
    assert np.array_equal(mx_dequantize(packed, scales), oracle.mxfp4.dequantize(packed, scales))


def test_guarded_buffer_catches_writes_outside_it():
    g = Guarded(1000, "cpu", "ws")
    assert g.view.numel() == 1000 and g.view.data_ptr() % 256 == g.full.data_ptr() % 256
    g.view.fill_(7)  # anything inside is fine
    g.check()
    for where in (GUARD - 1, GUARD + 1000):
        h = Guarded(1000, "cpu", "ws")
        h.full[where] = 0
        with pytest.raises(AssertionError):
            h.check()
    t = Guarded(8 * 6 * 2, "cpu", "out").tensor((8, 6), torch.bfloat16)
    assert t.shape == (8, 6) and t.dtype == torch.bfloat16

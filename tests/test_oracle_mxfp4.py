"""Pins of the oracle's MXFP4 codec (OCP microscaling FP4, E2M1 elements with
an E8M0 scale per block of 32) and of the checkpoint quantiser in
``workloads`` that produces the 4-bit test weights."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import mxfp4

# The 16 E2M1 values as tabulated in the OCP MX format specification
# (codes 0..7 positive, 8..15 the same magnitudes negated).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_code_table():
    vals = mxfp4.decode_e2m1(np.arange(16))
    assert np.array_equal(vals, np.array(E2M1_TABLE))
    assert np.array_equal(np.signbit(vals), np.arange(16) >= 8)


def test_e8m0_scales():
    assert mxfp4.decode_e8m0(127) == 1.0
    assert mxfp4.decode_e8m0(0) == 2.0 ** -127
    assert mxfp4.decode_e8m0(254) == 2.0 ** 127
    assert mxfp4.decode_e8m0(130) == 8.0
    assert np.isnan(mxfp4.decode_e8m0(255))


@pytest.mark.parametrize("v,expected", [
    # midpoints between neighbours go to the even code
    (0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),
    # just off the midpoints go to the nearer value
    (0.2500001, 0.5), (0.7499999, 0.5), (4.9999, 4.0), (5.0001, 6.0),
    # saturation, and the sign of small values
    (6.0, 6.0), (7.9, 6.0), (1e30, 6.0), (-0.1, -0.0), (-5.5, -6.0),
])
def test_e2m1_rounding_cases(v, expected):
    got = mxfp4.decode_e2m1(mxfp4.encode_e2m1(v))
    assert got == expected and np.signbit(got) == np.signbit(expected), (v, got)


def test_e2m1_nearest_on_a_fine_grid():
    """Every rounding is to a nearest representable value (within half the
    local spacing), and exact representable values round-trip."""
    v = np.arange(-8 * 256, 8 * 256 + 1) / 256.0
    q = mxfp4.decode_e2m1(mxfp4.encode_e2m1(v))
    mags = np.array(E2M1_TABLE[:8])
    clipped = np.clip(v, -6.0, 6.0)
    dist = np.abs(np.abs(clipped)[:, None] - mags[None, :]).min(axis=1)
    assert np.allclose(np.abs(q - clipped), dist, atol=0)
    for m in mags:
        assert mxfp4.decode_e2m1(mxfp4.encode_e2m1(m)) == m
        assert mxfp4.decode_e2m1(mxfp4.encode_e2m1(-m)) == -m


@pytest.mark.parametrize("amax,exp_code,top", [
    (1.0, 125, 4.0),      # 2^0 -> exponent -2, 1.0 / 0.25 = 4
    (6.0, 127, 6.0),      # largest E2M1 value at scale 1
    (7.9, 127, 6.0),      # top of the binade saturates at 6
    (8.0, 128, 4.0),      # next binade
    (0.05, 120, 6.0),     # floor(log2 0.05) = -5 -> exponent -7; 0.05 * 128 = 6.4 -> 6
    (3.0 * 2.0 ** -100, 26, 6.0),  # floor(log2) = -99 -> exponent -101
])
def test_block_exponent_rule(amax, exp_code, top):
    w = np.zeros((1, 32))
    w[0, 5] = amax
    w[0, 6] = -amax / 3.0
    codes, sc = mxfp4.quantize_blocks(w)
    assert sc[0, 0] == exp_code
    assert mxfp4.decode_e2m1(codes[0, 5]) == top
    assert mxfp4.decode_e2m1(codes[0, 6]) < 0


def test_zero_block_and_nibble_order():
    w = np.zeros((2, 64))
    w[1, 33] = 1.0      # second block of row 1, odd element -> high nibble of byte 16
    codes, sc = mxfp4.quantize_blocks(w)
    assert sc[0, 0] == 0 and sc[0, 1] == 0 and sc[1, 0] == 0
    packed = mxfp4.pack_nibbles(codes)
    assert packed.shape == (2, 32)
    assert packed[1, 16] == (codes[1, 33] << 4) and codes[1, 33] == 6  # 1.0 = 4.0 (code 6) x 0.25
    assert np.array_equal(mxfp4.unpack_nibbles(packed), codes)
    deq = mxfp4.dequantize(packed, sc)
    assert deq[1, 33] == 1.0 and np.count_nonzero(deq) == 1


def test_dequantize_error_bound():
    """Quantisation error of a block is at most one unit of its top binade's
    spacing (2^e, saturation included) and half that below the top binade."""
    rng = np.random.default_rng(0)
    w = rng.normal(0.0, 0.02, size=(16, 256))
    codes, sc = mxfp4.quantize_blocks(w)
    deq = mxfp4.dequantize(mxfp4.pack_nibbles(codes), sc)
    scale = np.repeat(mxfp4.decode_e8m0(sc), 32, axis=1)
    err = np.abs(deq - w)
    assert np.all(err <= 2.0 * scale + 1e-300)
    assert np.all(np.abs(deq) <= 6.0 * scale)


def test_checkpoint_quantiser_matches_oracle():
    """The torch quantiser that writes the 4-bit test weights agrees code for
    code with the oracle's (random rows and hand-made edge blocks)."""
    w = workloads.normal((48, 512), 0.02, 7, "mx")
    w[0, :32] = 0.0                                   # zero block
    w[1, :32] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)  # ties at scale 1
    w[1, 32:64] = 8.0                                 # one binade up
    w[2, :32] = -torch.linspace(0, 7.9, 32)           # saturation, negative
    packed, sc = workloads.mxfp4_quantize(w)
    codes_o, sc_o = mxfp4.quantize_blocks(w.double().numpy())
    assert np.array_equal(sc.numpy(), sc_o)
    assert np.array_equal(packed.numpy(), mxfp4.pack_nibbles(codes_o))


def test_mxfp4_workload_weights_shapes():
    cfg = dict(workloads.workload("mxfp4"), hidden=512, intermediate=512)
    w = workloads.make_expert_weights(cfg, 0, "cpu", experts=[3])
    assert w["w_gate"].shape == (256, 512, 256) and w["w_gate"].dtype == torch.uint8
    assert w["w_down_scale"].shape == (256, 512, 16)
    deq = mxfp4.dequantize(w["w_up"][3].numpy(), w["w_up_scale"][3].numpy())
    ref = workloads.normal((512, 512), 0.02, 0, "w_up", 3).double().numpy()
    assert np.max(np.abs(deq - ref)) < 0.02

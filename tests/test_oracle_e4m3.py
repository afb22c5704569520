"""Pins of the oracle's E4M3 codec (OCP 8-bit float, 4 exponent / 3 mantissa
bits, bias 7, no infinity, largest finite 448).

Checks: known codes from the format definition, round trip of all 256 codes,
and round-to-nearest-even at every midpoint against torch's CPU
float8_e4m3fn cast (a separate implementation), after clamping to +-448.
"""

import numpy as np
import torch

from oracle import e4m3


def test_known_codes():
    assert e4m3.decode(np.array([0x00]))[0] == 0.0
    assert e4m3.decode(np.array([0x01]))[0] == 2.0 ** -9       # smallest subnormal
    assert e4m3.decode(np.array([0x07]))[0] == 7 * 2.0 ** -9    # largest subnormal
    assert e4m3.decode(np.array([0x08]))[0] == 2.0 ** -6        # smallest normal
    assert e4m3.decode(np.array([0x38]))[0] == 1.0
    assert e4m3.decode(np.array([0x7E]))[0] == 448.0
    assert np.isnan(e4m3.decode(np.array([0x7F]))[0])
    assert e4m3.decode(np.array([0xB8]))[0] == -1.0
    assert e4m3.encode(np.array([448.0, 1000.0, -1e9]))[:].tolist() == [0x7E, 0x7E, 0xFE]


def test_roundtrip_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    finite = ~np.isnan(e4m3.decode(codes))
    assert finite.sum() == 254
    back = e4m3.encode(e4m3.decode(codes[finite]))
    assert np.array_equal(back, codes[finite])


def _torch_cast(v):
    t = torch.from_numpy(np.clip(v, -448.0, 448.0).astype(np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_midpoints_against_torch():
    codes = np.arange(0, 0x7F, dtype=np.uint8)  # non-negative finite codes
    vals = e4m3.decode(codes)
    mids = (vals[:-1] + vals[1:]) / 2
    m32 = mids.astype(np.float32)
    nudged = np.concatenate([mids, np.nextafter(m32, np.float32(0)).astype(np.float64),
                             np.nextafter(m32, np.float32(1e9)).astype(np.float64)])
    probe = np.concatenate([vals, nudged, -vals, -nudged])
    probe = probe[np.abs(probe) <= 448.0]
    # midpoints have at most 5 significant bits, so they are exact in fp32,
    # and the nudges are one fp32 ulp, so both casts see the same value
    assert np.array_equal(mids.astype(np.float32).astype(np.float64), mids)
    p32 = probe.astype(np.float32).astype(np.float64)
    mine = e4m3.encode(p32)
    ref = _torch_cast(p32)
    # +0 and -0 may differ only in the sign bit
    same = (mine == ref) | ((e4m3.decode(mine) == 0) & (e4m3.decode(ref) == 0))
    assert same.all(), p32[~same][:10]


def test_random_values_against_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-12, 6, 200000))).astype(np.float32).astype(np.float64)
    v = np.clip(v, -448, 448)
    assert np.array_equal(e4m3.encode(v), _torch_cast(v))


def test_quantize_rows():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((6, 300)).astype(np.float32)
    v[2] = 0.0
    codes, scale = e4m3.quantize_rows(v)
    assert scale.dtype == np.float32
    assert scale[2] == 1.0 and np.all(codes[2] == 0)
    deq = e4m3.decode(codes) * scale[:, None].astype(np.float64)
    for r in [0, 1, 3, 4, 5]:
        amax = np.abs(v[r]).max()
        # the largest element maps to (within rounding) the largest code
        assert np.abs(e4m3.decode(codes[r])).max() == 448.0
        assert scale[r] == np.float32(np.float32(amax) / np.float32(448.0))
        # relative error of a 3-bit mantissa: at most 2^-4 of the value for
        # normals, plus the subnormal spacing scaled back
        err = np.abs(deq[r] - v[r])
        bound = np.maximum(np.abs(v[r]) * 2.0 ** -4, 2.0 ** -10 * scale[r]) * 1.0001
        assert np.all(err <= bound)


def _rows_where_the_readings_differ(rng, n_rows):
    """Rows [amax, v] (amax the row's largest magnitude) with v within a few
    fp32 ulps of where an E4M3 rounding boundary falls, found by search."""
    mids = (e4m3.decode(np.arange(0, 0x7E, dtype=np.uint8)) +
            e4m3.decode(np.arange(1, 0x7F, dtype=np.uint8))) / 2
    rows = []
    while len(rows) < n_rows:
        amax = np.float32(np.exp(rng.uniform(-4, 4)))
        inv = np.float32(448.0) / amax
        scale = amax / np.float32(448.0)
        m = mids[rng.integers(8, len(mids))]
        v0 = np.float32(m / np.float64(inv))
        for k in range(-8, 9):
            v = np.float32(v0 + np.float32(k) * np.spacing(v0))
            if not 0 < v < amax:
                continue
            p1, p2 = np.float32(v * inv), np.float32(v / scale)
            if (p1 - m) * (p2 - m) <= 0 and p1 != p2:
                rows.append([amax, v])
                break
    return np.array(rows, dtype=np.float32)


def test_quantize_rows_multiplies_by_the_fp32_reciprocal():
    """The row reading: codes = e4m3(fp32(v * fp32(448 / amax))), the same
    correctly rounded fp32 steps the GPU takes. Dividing by the stored scale
    fp32(amax / 448) is a plausible other reading that rounds differently
    near code boundaries; on rows built to sit there, the oracle must give
    the multiply path's codes. Both paths are computed with torch's float32
    arithmetic and torch's float8_e4m3fn cast, independently of the oracle's
    own encoder, and they do disagree on these rows."""
    v = _rows_where_the_readings_differ(np.random.default_rng(7), 64)
    t = torch.from_numpy(v)
    amax = t.abs().amax(dim=1)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    scale = amax / torch.tensor(448.0, dtype=torch.float32)
    mul = (t * inv[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    div = (t / scale[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (mul != div).any(axis=1).sum() >= 32   # the readings really differ here
    codes, sc = e4m3.quantize_rows(v)
    assert np.array_equal(codes, mul)
    assert np.array_equal(sc, scale.numpy())

"""Oracle: the OCP FP8 E4M3 ("e4m3fn") codec and row quantisation.

Test infrastructure only; see the package docstring.

The pages say only that an FP8 checkpoint of Beam exists (launch post,
"Mixture of Experts" and "Hardware requirements"); they give no layout. The
format used here is the OCP 8-bit floating point E4M3 encoding, written from
its definition:

* bit layout S EEEE MMM, exponent bias 7;
* E = 0: subnormal, value (-1)^S * M * 2^-9;
* E = 1..15: normal, value (-1)^S * 2^(E-7) * (1 + M/8), except that
  E = 15, M = 7 is NaN (there is no infinity); the largest finite value is
  therefore 2^8 * 1.75 = 448.

Encoding rounds to the nearest representable value, ties to the even
mantissa, and saturates finite overflow to +-448.

Row quantisation (the reading adopted for per-token activations and the
per-row intermediate): amax = max |v| over the row; if amax is 0 the scale is
1 and every code is 0; otherwise inv = fp32(448 / amax), the codes are
encode(fp32(v * inv)) and the stored scale is fp32(amax / 448). The scalar
operations are correctly rounded fp32 operations, the same ones a GPU
performs, so both sides take the same decision on the same fp32 value.
"""

import numpy as np

FP8_MAX = 448.0


def decode(codes):
    """Value of each uint8 code (float64). NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    nrm = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    val = np.where(e == 0, sub, nrm)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def round_to_e4m3(v):
    """Nearest E4M3 value to each element of ``v`` (float64 in, float64 out).

    Round to nearest, ties to even mantissa; finite values beyond 448 in
    magnitude saturate to +-448.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    out = np.zeros_like(a)
    nz = a > 0
    # floor(log2 a) from the binary exponent: a = f * 2^ex with f in [0.5, 1)
    _, ex = np.frexp(a[nz])
    e_unb = np.maximum(ex - 1, -6)  # below 2^-6 the spacing is fixed (subnormals)
    quantum = np.ldexp(1.0, (e_unb - 3).astype(np.int64))  # 3 mantissa bits
    n = np.rint(a[nz] / quantum)  # np.rint rounds half to even
    out[nz] = n * quantum
    out = np.minimum(out, FP8_MAX)
    return np.copysign(out, v)


def encode(v):
    """uint8 E4M3 codes of ``v`` (round to nearest even, saturate to 448)."""
    r = round_to_e4m3(v)
    a = np.abs(r)
    sign = np.where(np.signbit(r), 0x80, 0).astype(np.int64)
    codes = np.zeros(a.shape, dtype=np.int64)
    sub = (a > 0) & (a < 2.0 ** -6)
    codes = np.where(sub, np.rint(a / 2.0 ** -9).astype(np.int64), codes)
    nrm = a >= 2.0 ** -6
    safe = np.where(nrm, a, 1.0)
    _, ex = np.frexp(safe)
    e = ex - 1  # unbiased exponent
    mant = np.rint((safe / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    codes = np.where(nrm, ((e + 7) << 3) | mant, codes)
    return (codes | sign).astype(np.uint8)


def quantize_rows(v):
    """Per-row E4M3 quantisation; returns (codes uint8 [R, C], scale fp32 [R]).

    See the module docstring for the arithmetic. The dequantised rows are
    ``decode(codes) * scale[:, None]``.
    """
    v32 = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v32), axis=1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    inv = (np.float32(FP8_MAX) / safe).astype(np.float32)
    prod = (v32 * inv[:, None]).astype(np.float32)
    codes = encode(prod.astype(np.float64))
    codes[zero, :] = 0
    scale = np.where(zero, np.float32(1.0), (safe / np.float32(FP8_MAX)).astype(np.float32))
    return codes, scale.astype(np.float32)


def fake_quantize_rows(v):
    """Quantise then dequantise each row (float64 result)."""
    codes, scale = quantize_rows(v)
    return decode(codes) * scale.astype(np.float64)[:, None]

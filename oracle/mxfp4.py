"""Oracle: the OCP microscaling FP4 format (MXFP4) for expert weights.

Test infrastructure only; see the package docstring.

The launch post ("Introducing Beam", sections "Mixture of Experts" and
"Hardware requirements") names a 4-bit expert checkpoint as the practical way
to serve the model on one node, in NVIDIA's NVFP4 format. The MI355X matrix
cores take the OCP MX formats natively, so the 4-bit reading here is OCP
MXFP4, written from the format definition:

* element E2M1: bit layout S EE M, exponent bias 1; E = 0: subnormal value
  (-1)^S * M * 0.5; E = 1..3: (-1)^S * 2^(E-1) * (1 + M/2). The magnitudes are
  0, 0.5, 1, 1.5, 2, 3, 4, 6; there is no infinity or NaN;
* a block of 32 consecutive elements along the reduction dimension shares one
  E8M0 scale: an 8-bit biased exponent, value 2^(code - 127); code 255 is NaN;
* quantising a block: amax = max |v|; the shared exponent is
  floor(log2(amax)) - 2 (2 = the exponent of E2M1's largest binade, so the
  largest element lands in [4, 8) before rounding); each element is v / 2^e
  rounded to the nearest E2M1 value, ties to the even code, magnitudes
  beyond 6 saturating to 6. An all-zero block takes the smallest scale code.

Storage: codes two to a byte, element 2j in the low nibble and 2j + 1 in the
high nibble; one scale byte per block.
"""

import numpy as np

E2M1_MAX = 6.0
BLOCK = 32
_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def decode_e2m1(codes):
    """Value of each 4-bit code (0..15), float64, from the bit-layout formula."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    sub = m * 0.5
    nrm = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64))
    return sign * np.where(e == 0, sub, nrm)


def decode_e8m0(codes):
    """Value of each scale byte: 2^(code - 127); 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, (c - 127).astype(np.int64))
    return np.where(c == 255, np.nan, v)


def encode_e2m1(v):
    """Nearest E2M1 code to each value (already divided by the block scale).

    Ties go to the even code (mantissa bit 0); magnitudes beyond 6 saturate.
    Returns uint8 codes 0..15 (sign in bit 3; -0 keeps its sign bit).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E2M1_MAX)
    # distance to every magnitude; the nearest wins, a tie picks the even code
    d = np.abs(a[..., None] - _MAGNITUDES)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    codes = np.arange(8)
    # among the tied candidates prefer an even code; there is at most one of each parity
    even_pick = np.where(cand & (codes % 2 == 0), codes, 99).min(axis=-1)
    any_pick = np.where(cand, codes, 99).min(axis=-1)
    mag = np.where(even_pick < 99, even_pick, any_pick)
    return (mag | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def quantize_blocks(w):
    """MXFP4 of a [rows, K] array (K a multiple of 32), float64 in.

    Returns (codes [rows, K] uint8 one code per element, scale codes
    [rows, K/32] uint8).
    """
    w = np.asarray(w, dtype=np.float64)
    rows, K = w.shape
    assert K % BLOCK == 0
    blocks = w.reshape(rows, K // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    nz = amax > 0
    exp = np.zeros(amax.shape, dtype=np.int64)
    _, ex = np.frexp(amax[nz])          # amax = f * 2^ex, f in [0.5, 1)
    exp[nz] = (ex - 1) - 2              # floor(log2 amax) - 2
    exp = np.where(nz, exp, -127)
    exp = np.clip(exp, -127, 127)
    scale = np.ldexp(1.0, exp)
    codes = encode_e2m1(blocks / scale[..., None]).reshape(rows, K)
    return codes, (exp + 127).astype(np.uint8)


def pack_nibbles(codes):
    """[rows, K] codes -> [rows, K/2] bytes, element 2j in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """[rows, K/2] bytes -> [rows, K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequantize(packed, scales):
    """Weights of a [rows, K/2] packed code matrix with [rows, K/32] scale
    codes, float64 [rows, K] (exact: every E2M1 value times a power of two)."""
    vals = decode_e2m1(unpack_nibbles(packed))
    rows, K = vals.shape
    s = decode_e8m0(scales)
    return (vals.reshape(rows, K // BLOCK, BLOCK) * s[..., None]).reshape(rows, K)

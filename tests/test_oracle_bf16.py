"""Pins of the oracle's bf16 storage rounding and of its place in the
quantised expert: the intermediate h is stored as bf16 and the per-row E4M3
quantisation starts from the stored values."""

import numpy as np
import torch

import oracle
from oracle.bf16 import round_to_bf16


def test_matches_torch_bfloat16_cast():
    """torch's float32 -> bfloat16 conversion (round to nearest even) is the
    library routine the definition reduces to, over a wide range of
    magnitudes and on exact ties of both parities."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))
    want = torch.from_numpy(v).float().to(torch.bfloat16).double().numpy()
    assert np.array_equal(round_to_bf16(v), want)
    # fp32 patterns whose low 16 bits are exactly half a bf16 step
    hi = rng.integers(0x0080, 0x7F00, size=4096, dtype=np.uint32)
    bits = (hi << np.uint32(16)) | np.uint32(0x8000)
    ties = bits.view(np.float32).astype(np.float64)
    want = torch.from_numpy(ties).float().to(torch.bfloat16).double().numpy()
    got = round_to_bf16(ties)
    assert np.array_equal(got, want)
    up = (hi & 1) == 1  # odd kept bit: the tie goes up to the even neighbour
    assert np.all(got[up] > ties[up]) and np.all(got[~up] < ties[~up])


def test_closed_forms():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(10_000)
    r = round_to_bf16(v)
    assert np.array_equal(round_to_bf16(r), r)  # bf16 values are fixed points
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    # nearest: within half a bf16 step (2^-8 relative to the leading bit)
    assert np.all(np.abs(r - v) <= np.abs(v) * 2.0 ** -8 * (1 + 1e-12))
    for x in (0.0, 1.0, -2.5, 3.0 * 2.0 ** -100, 448.0):
        assert round_to_bf16(x) == x


def test_rounds_to_fp32_first():
    """h leaves an fp32 computation: float64 inputs are rounded to fp32
    before bf16. A value above a bf16 midpoint by less than half an fp32
    step becomes the midpoint in fp32, which then ties to even (down here);
    rounding the float64 value directly would go up."""
    mid = 1.0 + 2.0 ** -8                    # halfway between bf16 1 and 1 + 2^-7
    v = mid + 2.0 ** -30                     # below half an fp32 step (2^-24) above it
    assert np.float32(v) == np.float32(mid)
    assert round_to_bf16(v) == 1.0


def _midpoint_rows(rng, n):
    """Rows of h targets that sit within half a bf16 step above a midpoint
    of two E4M3 codes whose lower code is even, plus 448 so that the row
    scale is exactly 1: bf16 storage turns each into the midpoint, a tie that
    goes down to the even code, while quantising the fp32 value would round
    it up."""
    rows = []
    for _ in range(n):
        row = [448.0]
        for _ in range(31):
            e = int(rng.integers(-3, 8))                  # 2^e in [1/8, 128]
            m = 2 * int(rng.integers(0, 4))               # even mantissa of the lower code
            lo = (1.0 + m / 8.0) * 2.0 ** e
            mid = lo + 2.0 ** (e - 4)                     # halfway to the next code
            t = mid + float(rng.uniform(0.05, 0.45)) * 2.0 ** (e - 7)  # < half a bf16 step
            row.append(float(np.float32(t)) * (1 if rng.random() < 0.5 else -1))
        rows.append(row)
    return np.array(rows, dtype=np.float64)


def test_quantised_expert_quantises_the_stored_bf16_h():
    """The quantised expert's intermediate equals, value for value, torch's
    own chain: fp32 h -> bfloat16 -> times fp32(448 / amax) -> float8_e4m3fn
    -> times the row scale. The rows are built so that quantising the fp32
    values instead gives other codes. An expert with silu(g) = 1 to float64
    precision and an identity down projection exposes h directly."""
    rng = np.random.default_rng(3)
    t = _midpoint_rows(rng, 16)                           # [16, 32] target h values
    n, I = t.shape
    x = np.ones((n, 1))
    big = 60.0                                            # silu(60) = 60 (1 - 9e-27)
    w_gate = np.full((I, 1), big)
    out = []
    for row in t:
        w_up = (row / big)[:, None]                       # u = h / silu(g)
        out.append(oracle.expert_ffn(x[:1], w_gate, w_up, np.eye(I), quantize_h=True)[0])
    got = np.array(out)
    h = torch.from_numpy(t).float()
    hb = h.to(torch.bfloat16).float()
    amax = hb.abs().amax(dim=1)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    scale = amax / torch.tensor(448.0, dtype=torch.float32)
    q = (hb * inv[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).float()
    want = (q.double() * scale.double()[:, None]).numpy()
    assert np.array_equal(got, want)
    # quantising the fp32 values instead disagrees on these rows
    q32 = (h * (torch.tensor(448.0) / h.abs().amax(dim=1))[:, None]).clamp(-448, 448)
    q32 = q32.to(torch.float8_e4m3fn).float().double().numpy()
    assert (q32 != q.double().numpy()).sum() == 16 * 31  # every value but the 448s

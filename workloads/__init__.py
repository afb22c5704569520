"""Seeded synthetic inputs for the Beam sparse-MoE block.

Shared by the tests, the benchmark and the oracle's checks; it holds none of
the block's arithmetic (no routing, no expert math), only random draws,
dtype conversion to the storage formats, and the named workloads.

Every tensor has its own torch.Generator, seeded from (seed, tensor name,
expert index), so any single expert can be regenerated alone. Small tensors
(x, router weights, bias) are always drawn on the CPU so that they are the
same whichever device holds the experts; the expert weights are drawn on the
device that will hold them (20 GB of bf16 at the full layer shape).

Distributions: x ~ N(0, 1); router weight ~ N(0, 1/H) (variance 1/H, so the
logits have unit variance); expert bias ~ N(0, 0.01^2) (standard deviation
0.01); expert weights ~ N(0, 0.02^2) (standard deviation 0.02). bf16 values
are the round-to-nearest-even images of the fp32 draws.
"""

import hashlib
import math
import os

import torch

# Beam's MoE layer shape (launch post "Mixture of Experts"; model doc "Beam",
# "Overview"): hidden 5120, 256 experts in 8 groups of 32, keep 4 groups,
# 8 experts per token, SwiGLU intermediate 2560, output scale 2.5.
BEAM = dict(hidden=5120, intermediate=2560, n_experts=256, n_group=8, topk_group=4,
            top_k=8, routed_scaling_factor=2.5)

# Named workloads. "bias": normal = N(0, 0.01^2) per expert; hot = +0.5 on
# experts 0..7 (all in group 0) and N(0, 0.01^2) elsewhere; balanced = a
# stored bias that spreads this exact token set to max/mean load <= 1.05.
WORKLOADS = {
    "tiny": dict(T=128, hidden=256, intermediate=128, x_dtype="f32", w_dtype="bf16", bias="normal"),
    "decode": dict(T=64, x_dtype="bf16", w_dtype="bf16", bias="normal"),
    "prefill": dict(T=4096, x_dtype="bf16", w_dtype="bf16", bias="balanced"),
    "skewed": dict(T=16384, x_dtype="bf16", w_dtype="bf16", bias="hot"),
    "fp8": dict(T=8192, x_dtype="bf16", w_dtype="fp8", bias="normal"),
    "mxfp4": dict(T=64, x_dtype="bf16", w_dtype="mxfp4", bias="normal"),
    "mxfp4_prefill": dict(T=4096, x_dtype="bf16", w_dtype="mxfp4", bias="balanced"),
}

DATA_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "data")


def workload(name):
    """Full parameter dict of a named workload (Beam shape unless overridden)."""
    cfg = dict(BEAM)
    cfg.update(WORKLOADS[name])
    cfg["name"] = name
    return cfg


def derive_seed(seed, name, index=0):
    """A 63-bit generator seed from (seed, tensor name, index)."""
    h = hashlib.blake2b(f"{seed}/{name}/{index}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def generator(seed, name, index=0, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, name, index))
    return g


def normal(shape, std, seed, name, index=0, device="cpu"):
    """fp32 draws from N(0, std^2)."""
    g = generator(seed, name, index, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def balanced_bias_path(T, seed):
    return os.path.join(DATA_DIR, f"balanced_bias_T{T}_seed{seed}.txt")


def load_bias_file(path):
    """Read a stored bias: one float.hex() value per non-comment line."""
    vals = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float.fromhex(line))
    return torch.tensor(vals, dtype=torch.float32)


def make_small_inputs(cfg, seed=0):
    """x, router_w, expert_bias (CPU tensors) for a workload dict.

    x is fp32 for x_dtype "f32" and bf16 for "bf16".
    """
    T, H, E = cfg["T"], cfg["hidden"], cfg["n_experts"]
    x = normal((T, H), 1.0, seed, "x")
    if cfg["x_dtype"] == "bf16":
        x = x.to(torch.bfloat16)
    router_w = normal((E, H), math.sqrt(1.0 / H), seed, "router_w")
    kind = cfg.get("bias", "normal")
    if kind == "balanced":
        path = balanced_bias_path(T, seed)
        if not os.path.exists(path):
            raise FileNotFoundError(f"no stored balanced bias for T={T} seed={seed}: {path}")
        bias = load_bias_file(path)
        assert bias.numel() == E
    else:
        bias = normal((E,), 0.01, seed, "expert_bias")
        if kind == "hot":
            bias[0:8] = 0.5
    return x, router_w, bias


def make_residual_inputs(cfg, seed=0):
    """stream_in [T, H] (x's dtype) and the post-norm gain [H] fp32 (CPU
    tensors) for the fused residual step. The stream is unit-RMS noise (the
    scale of a stream of unit-RMS contributions after the depth scaling); the
    gain is uniform in [0.5, 1.5]."""
    T, H = cfg["T"], cfg["hidden"]
    stream = normal((T, H), 1.0, seed, "stream_in")
    if cfg["x_dtype"] == "bf16":
        stream = stream.to(torch.bfloat16)
    g = torch.rand((H,), generator=generator(seed, "norm_weight"), dtype=torch.float32)
    return stream, g + 0.5


# E2M1 magnitudes and the midpoints between neighbours (storage format of the
# 4-bit checkpoint: OCP MXFP4, blocks of 32 along the reduction dimension).
_E2M1_MID = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]


def mxfp4_quantize(w):
    """OCP MXFP4 of an fp32 [rows, K] tensor (K a multiple of 32), as stored
    in the checkpoint: (codes [rows, K/2] uint8, element 2j in the low nibble;
    scale codes [rows, K/32] uint8, E8M0). Block exponent floor(log2 amax) - 2;
    elements rounded to the nearest E2M1 value, ties to the even code,
    saturating at 6; an all-zero block takes scale code 0."""
    rows, K = w.shape
    b = w.reshape(rows, K // 32, 32)
    amax = b.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)  # amax = m * 2^ex, m in [0.5, 1)
    e = torch.where(amax > 0, ex.to(torch.int64) - 3, torch.full_like(ex, -127, dtype=torch.int64))
    e = e.clamp(-127, 127)
    scaled = b / torch.ldexp(torch.ones_like(amax), e.to(torch.float32))[..., None]
    a = scaled.abs().clamp(max=6.0)
    mid = torch.tensor(_E2M1_MID, dtype=torch.float32, device=w.device)
    idx = torch.bucketize(a, mid)  # number of midpoints below a (a tie counts as below)
    tie = (idx < len(_E2M1_MID)) & (a == mid[idx.clamp(max=len(_E2M1_MID) - 1)])
    idx = torch.where(tie & (idx % 2 == 1), idx + 1, idx)  # ties to the even code
    codes = (idx | torch.where(torch.signbit(scaled), 8, 0)).to(torch.uint8).reshape(rows, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8)


def make_expert_weights(cfg, seed=0, device="cpu", experts=None):
    """Expert weights in storage format on ``device``.

    bf16: dict(w_gate [E, I, H], w_up [E, I, H], w_down [E, H, I]) bf16.
    fp8: the same shapes as torch.float8_e4m3fn codes plus per-output-row
    fp32 scales w_gate_scale [E, I], w_up_scale [E, I], w_down_scale [E, H];
    each row was quantised from its N(0, 0.02^2) draw with scale amax/448
    (checkpoint preparation, done with torch's own fp8 cast).
    mxfp4: codes [E, I, H/2] / [E, H, I/2] uint8 (two E2M1 codes per byte)
    plus E8M0 block scales w_*_scale [E, I, H/32] / [E, H, I/32] uint8
    (``mxfp4_quantize`` of the same N(0, 0.02^2) draws).
    ``experts`` restricts generation to a list of expert indices (the other
    rows are left zero), for tests that only need a few experts.
    """
    E, H, I = cfg["n_experts"], cfg["hidden"], cfg["intermediate"]
    if cfg["w_dtype"] == "mxfp4":
        shapes = {"w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}
        out = {}
        for k, (R, C) in shapes.items():
            out[k] = torch.zeros((E, R, C // 2), dtype=torch.uint8, device=device)
            out[k + "_scale"] = torch.zeros((E, R, C // 32), dtype=torch.uint8, device=device)
        ids = range(E) if experts is None else experts
        for e in ids:
            for k, s in shapes.items():
                w = normal(s, 0.02, seed, k, e, device)
                out[k][e], out[k + "_scale"][e] = mxfp4_quantize(w)
                del w
        return out
    fp8 = cfg["w_dtype"] == "fp8"
    store = torch.float8_e4m3fn if fp8 else torch.bfloat16
    shapes = {"w_gate": (I, H), "w_up": (I, H), "w_down": (H, I)}
    out = {k: torch.zeros((E,) + s, dtype=store, device=device) for k, s in shapes.items()}
    if fp8:
        for k, s in shapes.items():
            out[k + "_scale"] = torch.ones((E, s[0]), dtype=torch.float32, device=device)
    ids = range(E) if experts is None else experts
    for e in ids:
        for k, s in shapes.items():
            w = normal(s, 0.02, seed, k, e, device)
            if fp8:
                amax = w.abs().amax(dim=1)
                scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
                out[k][e] = (w / scale[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
                out[k + "_scale"][e] = scale
            else:
                out[k][e] = w.to(torch.bfloat16)
            del w
    return out

"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle.

Criteria (they restate the targets for this block):
* expert indices bit-exact, in order, for every token whose oracle margin to
  a different selection is at least NEAR_TIE (1e-6); tokens below it are
  counted and reported, their GPU choice is checked to lie within the band,
  and their outputs are checked against the oracle run with the GPU's choice;
* per-expert token counts exact (against the oracle's counts when no token
  is a near tie, and against the GPU's own indices always);
* routing weights within 1e-6 + 1e-5 relative (fp32 vs float64 arithmetic);
* outputs: max over tokens of ||out_t - ref_t||_inf / ||ref_t||_inf <= 2e-2
  and ||out - ref||_F / ||ref||_F <= 5e-3.
"""

import numpy as np
import torch

import oracle
from oracle.routing import counts as oracle_counts
import group_limited_routing_amd as gl

NEAR_TIE = 1e-6
MAX_REL = 2e-2
NORMWISE = 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy() if t.dtype != torch.float8_e4m3fn else None


def is_mxfp4(w):
    return w["w_gate"].dtype == torch.uint8


def packed_copy(w):
    """The same weights in the MFMA fragment layout (made by the library);
    MXFP4 scale bytes are packed too."""
    pw = dict(w)
    for k in ("w_gate", "w_up", "w_down"):
        pw[k] = gl.pack_weights(w[k])
        if is_mxfp4(w):
            pw[k + "_scale"] = gl.pack_mx_scales(w[k + "_scale"])
    pw["packed"] = True
    return pw


GUARD = 4096       # canary bytes before and after a guarded buffer
CANARY = 0xA5


class Guarded:
    """nbytes of device memory with GUARD canary bytes on both sides. The
    library is handed ``view`` (256-byte aligned) and told its exact size;
    ``check()`` after the call asserts that no byte outside it changed."""

    def __init__(self, nbytes, device, what):
        self.n, self.what = int(nbytes), what
        self.full = torch.full((self.n + 2 * GUARD,), CANARY, dtype=torch.uint8, device=device)
        self.view = self.full[GUARD:GUARD + self.n]

    def tensor(self, shape, dtype):
        return self.view.view(dtype).view(shape)

    def check(self):
        if self.full.is_cuda:
            torch.cuda.synchronize()
        head, tail = self.full[:GUARD], self.full[GUARD + self.n:]
        assert bool((head == CANARY).all()), f"{self.what}: bytes written before its start"
        assert bool((tail == CANARY).all()), f"{self.what}: bytes written past its end"


def guarded_workspace(x, w, cfg):
    """A guarded workspace of exactly the size the library asks for."""
    c = gl.make_config(x.shape[1], w["w_gate"].shape[1], cfg["n_experts"], cfg["n_group"],
                       cfg["topk_group"], cfg["top_k"], cfg["routed_scaling_factor"], x.dtype,
                       w["w_gate"].dtype, w.get("packed", False))
    return Guarded(gl.workspace_bytes(c, x.shape[0]), x.device, "workspace")


def guarded_out(x):
    g = Guarded(x.numel() * x.element_size(), x.device, "out")
    return g, g.tensor(tuple(x.shape), x.dtype)


def run_forward(x, rw, b, w, cfg, **kw):
    """beam_moe_forward with routing outputs, on a guarded workspace and a
    guarded output buffer (checked after the call)."""
    scales = None
    if w["w_gate"].dtype in (torch.float8_e4m3fn, torch.uint8):
        scales = (w["w_gate_scale"], w["w_up_scale"], w["w_down_scale"])
    ws = guarded_workspace(x, w, cfg)
    og, out = guarded_out(x)
    out, r = gl.forward(x, rw, b, w["w_gate"], w["w_up"], w["w_down"], scales=scales,
                        packed=w.get("packed", False),
                        n_group=cfg["n_group"], topk_group=cfg["topk_group"], top_k=cfg["top_k"],
                        routed_scaling_factor=cfg["routed_scaling_factor"], return_routing=True,
                        return_logits=True, workspace=ws.view, out=out, **kw)
    torch.cuda.synchronize()
    ws.check()
    og.check()
    return out, r


# Decode tables: the oracle's own decoders applied once to every code, then
# indexed with torch's multithreaded CPU gather (the same values as calling
# the decoders on each weight, many times faster at 13M weights per matrix).
_E4M3_TABLE = None
_MX_TABLES = None


def _e4m3_table():
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = oracle.e4m3.decode(np.arange(256, dtype=np.uint8))
    return _E4M3_TABLE


def _mx_tables():
    """(byte -> (value of the low nibble, value of the high nibble), E8M0 byte -> scale)."""
    global _MX_TABLES
    if _MX_TABLES is None:
        b = np.arange(256)
        pair = np.stack([oracle.mxfp4.decode_e2m1(b & 0xF), oracle.mxfp4.decode_e2m1(b >> 4)], axis=1)
        _MX_TABLES = (pair, oracle.mxfp4.decode_e8m0(b))
    return _MX_TABLES


def e4m3_dequantize(codes, scales):
    """oracle.e4m3.decode(codes) * scales[:, None] through the decode table
    (codes uint8 [R, C], per-row scales [R]; CPU tensors or arrays)."""
    tab = torch.from_numpy(_e4m3_table())
    c = torch.as_tensor(codes).to(torch.int64)
    return (tab[c] * torch.as_tensor(scales).to(torch.float64)[:, None]).numpy()


def mx_dequantize(packed, scales):
    """oracle.mxfp4.dequantize through the decode tables."""
    pair, e8 = (torch.from_numpy(t) for t in _mx_tables())
    p = torch.as_tensor(packed).to(torch.int64)
    v = pair[p].reshape(p.shape[0], -1)
    R, K = v.shape
    sc = e8[torch.as_tensor(scales).to(torch.int64)]
    return (v.reshape(R, K // 32, 32) * sc[..., None]).reshape(R, K).numpy()


def expert_getter(w):
    """get_expert(e) for the oracle: one expert copied to the host, float64
    (fp8 weights dequantised with their per-row scales, MXFP4 weights with
    their block scales; the row-major copies)."""
    fp8 = w["w_gate"].dtype == torch.float8_e4m3fn
    mx = is_mxfp4(w)
    loaded = [0]

    def get(e):
        loaded[0] += 1
        if loaded[0] % 64 == 0:  # progress of a long full-shape reference
            print(f"[oracle] {loaded[0]} experts loaded", flush=True)
        mats = []
        for k in ("w_gate", "w_up", "w_down"):
            m = w[k][e].to("cpu")
            if mx:
                mats.append(mx_dequantize(m, w[k + "_scale"][e].to("cpu")))
            elif fp8:
                mats.append(e4m3_dequantize(m.view(torch.uint8), w[k + "_scale"][e].to("cpu")))
            else:
                mats.append(m.to(torch.float64).numpy())
        return tuple(mats)

    return get


def expert_rows(idx, E):
    """The sorted order of the expert GEMMs, rebuilt from the routing: expert
    e's rows are the tokens that chose it, in ascending token order (the
    permutation is stable by token). Returns a list of E int arrays."""
    idx = np.asarray(idx)
    T, k = idx.shape
    tok = np.repeat(np.arange(T), k)
    e = idx.reshape(-1)
    order = np.lexsort((tok, e))
    counts = np.bincount(e, minlength=E)
    return np.split(tok[order], np.cumsum(counts)[:-1])


def tile_cover(idx, E, bm=128, seed=0):
    """Tokens whose outputs include, for every expert and every M-tile of
    ``bm`` sorted rows, the tile's first row, its last row and one seeded
    random row. With bm = 128 this also covers every 256-row tile (two
    128-row blocks, one per half of the tile's waves)."""
    rng = np.random.default_rng(seed)
    pick = set()
    for rows in expert_rows(idx, E):
        n = len(rows)
        for m0 in range(0, n, bm):
            m1 = min(m0 + bm, n) - 1
            for q in (m0, m1, int(rng.integers(m0, m1 + 1))):
                pick.add(int(rows[q]))
    return np.array(sorted(pick), dtype=np.int64)


def tiles_covered(tokens, idx, E, bm):
    """(covered, total): M-tiles of ``bm`` sorted rows (expert by expert)
    holding at least one row of ``tokens``, counted independently of how
    the tokens were chosen."""
    tokens = set(int(t) for t in tokens)
    covered = total = 0
    for rows in expert_rows(idx, E):
        for m0 in range(0, len(rows), bm):
            total += 1
            covered += any(int(t) in tokens for t in rows[m0:m0 + bm])
    return covered, total


def coverage_report(tokens, idx, E, bms=(128, 256)):
    rep = {}
    for bm in bms:
        c, t = tiles_covered(tokens, idx, E, bm)
        rep[f"tiles_covered_{bm}"] = c
        rep[f"tiles_total_{bm}"] = t
    return rep


def check_routing(gpu_r, ora, cfg, report):
    """Compare GPU routing with the oracle's. Returns the near-tie token mask."""
    idx = gpu_r["topk_idx"].cpu().numpy().astype(np.int64)
    wts = gpu_r["topk_w"].cpu().numpy().astype(np.float64)
    near = ora["margin"] < NEAR_TIE
    far = ~near
    mism = np.nonzero(np.any(idx[far] != ora["idx"][far], axis=1))[0]
    assert mism.size == 0, f"{mism.size} routing mismatches outside the near-tie band: tokens {np.nonzero(far)[0][mism][:10]}"
    np.testing.assert_allclose(wts[far], ora["w"][far], rtol=1e-5, atol=1e-6)
    E = cfg["n_experts"]
    gs = E // cfg["n_group"]
    for t in np.nonzero(near)[0]:
        chosen = idx[t]
        assert len(set(chosen.tolist())) == cfg["top_k"]
        assert len({int(e) // gs for e in chosen}) <= cfg["topk_group"]
        key = ora["key"][t]
        gsc = ora["group_score"][t]
        kth = np.sort(ora["masked_key"][t])[::-1][cfg["top_k"] - 1]
        gth = np.sort(gsc)[::-1][cfg["topk_group"] - 1]
        for e in chosen:
            assert key[e] >= kth - NEAR_TIE and gsc[e // gs] >= gth - NEAR_TIE, (t, e)
    cnt = gpu_r["expert_counts"].cpu().numpy().astype(np.int64)
    assert np.array_equal(cnt, oracle_counts(idx, E)), "counts disagree with the GPU's own indices"
    if not near.any():
        assert np.array_equal(cnt, oracle_counts(ora["idx"], E)), "counts differ from the oracle"
    report["near_ties"] = int(near.sum())
    report["tokens"] = int(len(near))
    return near


def check_logits(gpu_logits, x64, rw64, z_ora):
    z = gpu_logits.cpu().numpy().astype(np.float64)
    # fp32 accumulation of H products: bound the error by a multiple of the
    # unit roundoff times the sum of |products| (generous, but it is the
    # logits' absolute scale that decides the selection, checked exactly).
    absum = np.abs(x64) @ np.abs(rw64).T
    tol = 64 * 2.0 ** -24 * absum + 1e-7
    assert np.all(np.abs(z - z_ora) <= tol), float(np.max(np.abs(z - z_ora) / tol))


def output_errors(out, ref):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = out - ref
    row_inf = np.abs(ref).max(axis=1)
    max_rel = float(np.max(np.abs(d).max(axis=1) / np.where(row_inf > 0, row_inf, 1.0)))
    normwise = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    return max_rel, normwise


def check_outputs(out_gpu, ref, report, label=""):
    max_rel, normwise = output_errors(out_gpu, ref)
    report[label + "max_rel"] = max_rel
    report[label + "normwise"] = normwise
    assert max_rel <= MAX_REL, (label, max_rel)
    assert normwise <= NORMWISE, (label, normwise)


def oracle_reference(tokens, x, rw, b, w, cfg, gpu_idx, near):
    """Oracle outputs for `tokens`; near-tie tokens use the GPU's selection."""
    x64 = x.detach().cpu().to(torch.float64).numpy()
    rw64 = rw.detach().cpu().to(torch.float64).numpy()
    b64 = b.detach().cpu().to(torch.float64).numpy()
    r = oracle.route(x64[tokens], rw64, b64, cfg["n_group"], cfg["topk_group"], cfg["top_k"])
    forced = r["idx"].copy()
    nt = near[tokens]
    forced[nt] = gpu_idx[tokens][nt]
    # fp8 and MXFP4 weights: the expert inputs are E4M3-quantised per row
    fp8 = w["w_gate"].dtype in (torch.float8_e4m3fn, torch.uint8)
    out, _ = oracle.forward(x64[tokens], rw64, b64, expert_getter(w), cfg["n_group"],
                            cfg["topk_group"], cfg["top_k"], cfg["routed_scaling_factor"],
                            routing=forced, fp8=fp8)
    return out

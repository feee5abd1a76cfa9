"""Helpers shared by the parity tests: inputs with routing margins, device upload,
sampling of bucket positions, and the comparison bounds.

Tolerances (for floating-point outputs):
  * per-row relative L2:   ||got - ref||_2 / ||ref||_2 <= 2e-3
  * elementwise:           |got - ref| <= 2e-2 * (1 + |ref|)
  * gate weights:          |got - ref| <= 1e-5
Integer and index outputs (top-k ids, counts, offsets, perm, inv_perm) must match exactly.

Reading for h (the one bf16 rounding point): the GPU computes the pre-rounding value
a = silu(g) * u in fp32, so near a bf16 midpoint it may round to the other neighbour than
the oracle's fp64 value does. A GPU h element is accepted if it is a faithful rounding of
the oracle's fp64 a, widened by the fp32 accumulation bound of its inputs:
  |h_gpu - a| < ulp_bf16(a) + slack,
  slack = 16 * 2^-24 * (sum_i |wg_i x_i| |silu'(g) u| + sum_i |wu_i x_i| |silu(g)|) + 2^-20 |a|
and at most 1% of elements may differ from the oracle's own rounding. y and out are then
judged against the oracle evaluated at the GPU's h.
"""
from __future__ import annotations

import numpy as np

import synth
from oracle import codecs, moe as omoe

REL_L2 = 2e-3
ELEM = 2e-2
W_ABS = 1e-5
MARGIN = 1e-4


def margin_fixed_x(cfg: synth.Config, layer: int = 0, T: int | None = None,
                   max_attempts: int = 50):
    """Activations whose oracle logits have every gap among the top k+1 above MARGIN.

    Returns (x bits [T, H], number of rows redrawn).
    """
    x = synth.make_x(cfg, layer, T)
    wr = synth.make_router(cfg, layer)
    bias = synth.make_bias(cfg)
    redrawn = 0

    def bad_rows(xx):
        L = omoe.router_logits(xx, wr, bias)
        s = -np.sort(-L, axis=1)[:, :min(cfg.k + 1, cfg.E)]
        if s.shape[1] < 2:                   # E = 1: nothing to order
            return np.zeros(0, dtype=np.int64)
        gaps = s[:, :-1] - s[:, 1:]
        return np.nonzero(gaps.min(axis=1) <= MARGIN)[0]

    bad = bad_rows(x)
    attempt = 0
    while bad.size:
        attempt += 1
        if attempt > max_attempts:
            raise RuntimeError("could not reach the routing margin")
        for t in bad:
            x[t] = synth.redraw_x_row(cfg, layer, int(t), attempt)
        redrawn += bad.size
        bad = bad[bad_rows(x[bad])]
    return x, redrawn


def make_case(cfg: synth.Config, layer: int = 0, T: int | None = None):
    """A synth layer whose x has been margin-fixed."""
    L = synth.make_layer(cfg, layer, T)
    L.x, _ = margin_fixed_x(cfg, layer, T)
    return L


def to_device(L: synth.Layer, device="cuda"):
    import torch
    import quantized_routed_expert_gemv_amd as qm
    pool = qm.Pool.from_canonical(L.cfg.fmt, L.cfg.H, L.cfg.I, L.planes, device=device)
    x = torch.from_numpy(L.x.view(np.int16)).to(device).view(torch.bfloat16)
    wr = torch.from_numpy(L.wr.view(np.int16)).to(device).view(torch.bfloat16)
    bias = None if L.bias is None else torch.from_numpy(L.bias).to(device)
    sm = torch.from_numpy(L.slot_map).to(device)
    return pool, x, wr, bias, sm


def h_bits(t):
    """bf16 device tensor -> uint16 numpy bits."""
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------------------- bounds


def rel_l2_rows(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / np.maximum(den, 1e-300)


def assert_close_rows(got, ref, what, rows=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2_rows(got, ref)
    e = np.abs(got - ref) / (1.0 + np.abs(ref))
    assert r.max() <= REL_L2, f"{what}: max per-row rel L2 {r.max():.3e} > {REL_L2}"
    assert e.max() <= ELEM, f"{what}: max elementwise err/(1+|ref|) {e.max():.3e} > {ELEM}"
    return r.max(), e.max()


def _ulp_bf16(a):
    a = np.abs(a)
    _, ex = np.frexp(np.maximum(a, 2.0 ** -126))
    return np.ldexp(1.0, ex - 8)


def check_h(h_gpu_bits, a_ref, slack):
    """Faithful-rounding check of h (see the module docstring). Returns the mismatch fraction."""
    hv = codecs.bf16_decode(h_gpu_bits)
    href = codecs.bf16_round(a_ref)
    assert np.all(np.isfinite(hv)), "h: non-finite"
    bound = _ulp_bf16(a_ref) + slack
    bad = np.abs(hv - a_ref) >= bound
    assert not bad.any(), (f"h: {int(bad.sum())} elements not a faithful rounding; worst "
                           f"|h-a|/bound = {(np.abs(hv - a_ref) / bound).max():.3f}")
    frac = float(np.mean(hv != href))
    assert frac <= 0.01, f"h: {frac:.4%} of elements differ from the oracle's rounding"
    return frac


def _accumulated_magnitude(fmt, planes, name, s, W):
    """|term| per weight of the sums the kernels accumulate in fp32: |w| for MXFP4 and Q8_0;
    for Q4_K and Q5_K the kernels sum x q and x over a block, scaled by a = d sc and by
    c = dmin m, so the magnitude is a q + |c|. Q6_K: per 16-element half, x q and x scaled
    by a = d sc, the latter times 32: |a| (q + 32)."""
    if fmt not in ("q4_k", "q5_k", "q6_k"):
        return np.abs(W)
    codes = planes[name + "_q"][s]
    if fmt == "q6_k":
        q = codecs.q6_k_codes(codes).astype(np.float64)
        K = q.shape[1]
        sp = np.asarray(planes[name + "_s"][s], dtype=np.uint8)
        sc = sp[:, :K // 16].view(np.int8).astype(np.float64)
        d = codecs.fp16_decode(np.ascontiguousarray(sp[:, K // 16:K // 16 + K // 128]).view(np.uint16))
        a = np.abs(np.repeat(d, 16, axis=1) * sc)
        return np.repeat(a, 16, axis=1) * (q + 32)
    if fmt == "q5_k":
        q = codecs.q5_k_codes(codes).astype(np.float64)
    else:
        q = np.empty((codes.shape[0], 2 * codes.shape[1]))
        q[:, 0::2] = codes & 15
        q[:, 1::2] = codes >> 4
    K = q.shape[1]
    sc, m, d, dmin = codecs.q4_k_fields(planes[name + "_s"][s], K)
    a = np.abs(np.repeat(d, 8, axis=1) * sc)
    c = np.repeat(dmin, 8, axis=1) * m
    return np.repeat(a, 32, axis=1) * q + np.repeat(np.abs(c), 32, axis=1)


def h_slack(planes, fmt, slot_map, x_bits, k, offsets, perm, positions, a_ref):
    """The fp32 accumulation slack of each h element at the given positions."""
    offsets = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    K = x_bits.shape[1]
    xa = np.abs(codecs.bf16_decode(x_bits))
    x_all = codecs.bf16_decode(x_bits)
    E = offsets.size - 1
    I = planes["gate_q"].shape[1]
    slack = np.zeros((len(positions), I))
    pos_index = {int(p): i for i, p in enumerate(positions)}
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sel = [p for p in range(lo, hi) if p in pos_index]
        if not sel:
            continue
        s = int(slot_map[e])
        Wg = codecs.dequant(fmt, planes["gate_q"][s], planes["gate_s"][s])
        Wu = codecs.dequant(fmt, planes["up_q"][s], planes["up_s"][s])
        toks = perm[sel] // k
        Sg = xa[toks] @ _accumulated_magnitude(fmt, planes, "gate", s, Wg).T
        Su = xa[toks] @ _accumulated_magnitude(fmt, planes, "up", s, Wu).T
        g = x_all[toks] @ Wg.T
        u = x_all[toks] @ Wu.T
        sig = 1.0 / (1.0 + np.exp(-g))
        dsilu = sig * (1.0 + g * (1.0 - sig))
        # fp32 accumulation error of a K-term dot product: ~u * sum|w x| with u = 2^-24,
        # taken 16x as a high-probability bound (the worst case K*u*sum|w x| is vacuous)
        err_g = 16 * 2.0 ** -24 * Sg
        err_u = 16 * 2.0 ** -24 * Su
        sl = err_g * np.abs(dsilu * u) + err_u * np.abs(g * sig) + 2.0 ** -20 * np.abs(g * sig * u)
        for j, p in enumerate(sel):
            slack[pos_index[p]] = sl[j]
    return slack


def sample_positions(offsets, n_uniform=512, seed=0, tile=128):
    """Bucket positions to check at large sizes: every position of experts with < 16 pairs,
    the first/last and tile-boundary positions of every non-empty expert, plus a seeded
    uniform sample."""
    offsets = np.asarray(offsets, dtype=np.int64)
    n = int(offsets[-1])
    rng = np.random.default_rng(seed)
    pos = set()
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        if hi - lo < 16:
            pos.update(range(lo, hi))
        else:
            for d in (0, 1, tile - 1, tile, tile + 1, hi - lo - 2, hi - lo - 1):
                if 0 <= d < hi - lo:
                    pos.add(lo + d)
    if n:
        pos.update(rng.choice(n, size=min(n_uniform, n), replace=False).tolist())
    return np.array(sorted(pos), dtype=np.int64)


def sample_tokens(ids, E, n_uniform=512, seed=0):
    """Tokens to check at large sizes: all tokens of experts with < 16 tokens, the first
    and last token of every other expert, plus a seeded uniform sample."""
    T, k = ids.shape
    counts = np.bincount(ids.ravel(), minlength=E)
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(T, size=min(n_uniform, T), replace=False).tolist())
    small = np.nonzero((counts > 0) & (counts < 16))[0]
    for e in range(E):
        ts = np.nonzero((ids == e).any(axis=1))[0]
        if ts.size == 0:
            continue
        if e in small:
            toks.update(ts.tolist())
        else:
            toks.update([int(ts[0]), int(ts[-1])])
    return np.array(sorted(toks), dtype=np.int64)

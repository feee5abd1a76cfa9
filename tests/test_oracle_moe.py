"""Pins for the oracle's layer functions (CPU only).

Each pin checks the oracle against something that is not the oracle:
  * brute force with Python loops and math.fsum on tiny shapes, decoding weights
    through the spec's E2M1 value table (independent of the oracle's bit formula);
  * exact integer arithmetic (Q8_0 with d = 1 and integer activations);
  * library routines: numpy's stable argsort for bucketing, torch's float64 silu and
    softmax for the textbook special cases (E = 1, k = 1 is a dense SwiGLU FFN; k = E
    is a full softmax mixture of every expert);
  * invariants that the layer's definition fixes (each token appears k times,
    counts sum to T*k, gate weights sum to 1, ties go to the lower index).
"""
import math
import os

import numpy as np
import pytest

import synth
from oracle import codecs, moe


def _e2m1_table(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "e2m1_table.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


def _bf16(bits):
    return float((np.uint32(bits) << np.uint32(16)).view(np.float32))


def _brute_weight(table, fmt, q, s, r, i):
    if fmt == "mxfp4":
        byte = int(q[r, i // 2])
        c = (byte >> 4) if (i % 2) else (byte & 0xF)
        return table[c] * math.ldexp(1.0, int(s[r, i // 32]) - 127)
    d = float(np.uint16(s[r, i // 32]).view(np.float16))
    return d * int(q[r, i])


def _brute_layer(L: synth.Layer, table):
    """The whole layer with Python loops + math.fsum, from the definitions."""
    cfg = L.cfg
    T, H, I, E, k = L.x.shape[0], cfg.H, cfg.I, cfg.E, cfg.k
    x = [[_bf16(L.x[t, h]) for h in range(H)] for t in range(T)]
    wr = [[_bf16(L.wr[e, h]) for h in range(H)] for e in range(E)]
    out = []
    for t in range(T):
        logit = [math.fsum(x[t][h] * wr[e][h] for h in range(H)) +
                 (float(L.bias[e]) if L.bias is not None else 0.0) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-logit[e], e))[:k]
        z = [math.exp(logit[e] - logit[order[0]]) for e in order]
        wts = [v / math.fsum(z) for v in z]
        acc = [0.0] * H
        for j, e in enumerate(order):
            s = int(L.slot_map[e])
            W = {}
            for name, rows, K in (("gate", I, H), ("up", I, H), ("down", H, I)):
                q, sc = getattr(L, name + "_q")[s], getattr(L, name + "_s")[s]
                W[name] = [[_brute_weight(table, cfg.fmt, q, sc, r, i) for i in range(K)]
                           for r in range(rows)]
            hrow = []
            for r in range(I):
                g = math.fsum(W["gate"][r][i] * x[t][i] for i in range(H))
                u = math.fsum(W["up"][r][i] * x[t][i] for i in range(H))
                a = g / (1.0 + math.exp(-g)) * u
                hrow.append(a)
            y = [math.fsum(W["down"][r][i] * hrow_rounded for i, hrow_rounded in
                           enumerate(codecs.bf16_round(np.array(hrow)))) for r in range(H)]
            acc = [acc[r] + wts[j] * y[r] for r in range(H)]
        out.append((order, wts, acc))
    return out


@pytest.mark.parametrize("fmt", ["mxfp4", "q8_0"])
def test_layer_matches_brute_force_on_tiny_shapes(fmt, golden_dir):
    table = _e2m1_table(golden_dir)
    cfg = synth.Config("brute", 3, 64, 32, 4, 2, fmt, 1.1 if fmt == "q8_0" else None,
                       "perm", 9 if fmt == "mxfp4" else 10, 1)
    L = synth.make_layer(cfg)
    ref = moe.layer(L.planes, fmt, L.slot_map, L.wr, L.bias, L.x, cfg.k)
    brute = _brute_layer(L, table)
    for t, (order, wts, acc) in enumerate(brute):
        assert list(ref["ids"][t]) == order
        np.testing.assert_allclose(ref["w"][t], wts, rtol=1e-14, atol=0)
        np.testing.assert_allclose(ref["out"][t], acc, rtol=1e-12, atol=1e-12 * max(map(abs, acc)))


def test_q8_0_exact_integer_case():
    """d = 1.0 and integer activations: g and u are exact integers on any exact path."""
    rng = np.random.default_rng(3)
    I, H = 32, 64
    q = rng.integers(-127, 128, size=(I, H), dtype=np.int8)
    d = np.full((I, H // 32), 0x3C00, dtype=np.uint16)        # fp16 1.0
    xi = rng.integers(-4, 5, size=H)
    W = codecs.dequant_q8_0(q, d)
    g = W @ xi.astype(np.float64)
    gi = q.astype(np.int64) @ xi.astype(np.int64)
    assert np.array_equal(g, gi.astype(np.float64))


def test_one_hot_row_selects_a_weight_column():
    cfg = synth.config("tiny", T=4)
    L = synth.make_layer(cfg)
    i = 37
    x = np.zeros((1, cfg.H), dtype=np.uint16)
    x[0, i] = 0x3F80                                          # bf16 1.0
    slot = int(L.slot_map[0])
    Wg = codecs.dequant_mxfp4(L.gate_q[slot], L.gate_s[slot])
    Wu = codecs.dequant_mxfp4(L.up_q[slot], L.up_s[slot])
    offsets = np.array([0] + [1] * cfg.E)                       # one pair, in expert 0
    perm = np.array([0])
    h, y, a = moe.expert_ffn(L.planes, "mxfp4", L.slot_map, x, 1, offsets, perm)
    g, u = Wg[:, i], Wu[:, i]
    np.testing.assert_array_equal(a[0], g / (1 + np.exp(-g)) * u)


def test_dense_special_case_e1_k1_matches_torch_swiglu():
    torch = pytest.importorskip("torch")
    cfg = synth.Config("dense", 5, 64, 96, 1, 1, "mxfp4", None, "identity", 11, 1)
    L = synth.make_layer(cfg)
    ref = moe.layer(L.planes, "mxfp4", L.slot_map, L.wr, None, L.x, 1)
    assert np.all(ref["ids"] == 0) and np.all(ref["w"] == 1.0)
    x = torch.from_numpy(codecs.bf16_decode(L.x))
    Wg = torch.from_numpy(codecs.dequant_mxfp4(L.gate_q[0], L.gate_s[0]))
    Wu = torch.from_numpy(codecs.dequant_mxfp4(L.up_q[0], L.up_s[0]))
    Wd = torch.from_numpy(codecs.dequant_mxfp4(L.down_q[0], L.down_s[0]))
    a = torch.nn.functional.silu(x @ Wg.T) * (x @ Wu.T)
    np.testing.assert_allclose(ref["a"], a.numpy(), rtol=1e-12, atol=1e-15)
    # h is the nearest bf16 to a: no bf16 value is closer
    hv = codecs.bf16_decode(ref["h"])
    an = a.numpy()
    up = codecs.bf16_decode((ref["h"].astype(np.int32) + 1).astype(np.uint16))
    dn = codecs.bf16_decode((ref["h"].astype(np.int32) - 1).astype(np.uint16))
    assert np.all(np.abs(hv - an) <= np.abs(up - an)) and np.all(np.abs(hv - an) <= np.abs(dn - an))
    out = torch.from_numpy(hv) @ Wd.T
    np.testing.assert_allclose(ref["out"], out.numpy(), rtol=1e-12, atol=1e-12)


def test_k_equals_e_is_a_full_softmax_mixture():
    torch = pytest.importorskip("torch")
    cfg = synth.Config("mix", 6, 64, 32, 4, 4, "q8_0", 1.2, "perm", 12, 1)
    L = synth.make_layer(cfg)
    ref = moe.layer(L.planes, "q8_0", L.slot_map, L.wr, L.bias, L.x, cfg.k)
    x = torch.from_numpy(codecs.bf16_decode(L.x))
    logits = x @ torch.from_numpy(codecs.bf16_decode(L.wr)).T + torch.from_numpy(
        L.bias.astype(np.float64))
    p = torch.softmax(logits, dim=1)
    total = torch.zeros(cfg.T, cfg.H, dtype=torch.float64)
    for e in range(cfg.E):
        s = int(L.slot_map[e])
        Wg = torch.from_numpy(codecs.dequant_q8_0(L.gate_q[s], L.gate_s[s]))
        Wu = torch.from_numpy(codecs.dequant_q8_0(L.up_q[s], L.up_s[s]))
        Wd = torch.from_numpy(codecs.dequant_q8_0(L.down_q[s], L.down_s[s]))
        a = torch.nn.functional.silu(x @ Wg.T) * (x @ Wu.T)
        h = torch.from_numpy(codecs.bf16_round(a.numpy()))
        total += p[:, e:e + 1] * (h @ Wd.T)
    np.testing.assert_allclose(ref["out"], total.numpy(), rtol=1e-10,
                               atol=1e-10 * float(total.abs().max()))
    # every token routes to every expert
    assert np.array_equal(np.sort(ref["ids"], axis=1), np.tile(np.arange(cfg.E), (cfg.T, 1)))


def test_routing_invariants_and_brute_force_sort():
    cfg = synth.config("qwen_a3b_prefill", T=200)
    x, wr, bias = synth.make_x(cfg), synth.make_router(cfg), synth.make_bias(cfg)
    ids, w, L = moe.route(x, wr, bias, cfg.k)
    for t in range(cfg.T):
        want = sorted(range(cfg.E), key=lambda e: (-L[t, e], e))[:cfg.k]
        assert list(ids[t]) == want
        assert len(set(ids[t])) == cfg.k
        assert abs(w[t].sum() - 1.0) <= 1e-12
        assert np.all(np.diff(w[t]) <= 0)
    counts, offsets, perm, inv = moe.bucket(ids, cfg.E)
    assert counts.sum() == cfg.T * cfg.k and offsets[-1] == cfg.T * cfg.k
    # each token appears exactly k times across the buckets
    assert np.array_equal(np.bincount(perm // cfg.k, minlength=cfg.T), np.full(cfg.T, cfg.k))


def test_router_logits_brute_force():
    cfg = synth.config("tiny", T=3)
    x, wr = synth.make_x(cfg), synth.make_router(cfg)
    L = moe.router_logits(x, wr)
    for t in range(cfg.T):
        for e in range(cfg.E):
            want = math.fsum(_bf16(x[t, h]) * _bf16(wr[e, h]) for h in range(cfg.H))
            assert abs(L[t, e] - want) <= 1e-15 * max(1.0, abs(want)) * cfg.H


def test_ties_go_to_the_lower_index():
    L = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0],
                  [-0.0, 0.0, -1.0, 5.0, np.nan]])
    ids, w = moe.topk_softmax(L, 3)
    assert ids[0].tolist() == [1, 2, 4]
    assert ids[1].tolist() == [0, 1, 2]
    assert ids[2].tolist() == [3, 0, 1]         # -0 == +0, NaN counts as -inf
    np.testing.assert_allclose(w[1], [1 / 3] * 3, rtol=1e-15)


@pytest.mark.parametrize("T,k,E,seed", [(1, 4, 32, 0), (64, 2, 8, 1), (1000, 8, 128, 2),
                                        (16384, 4, 32, 3), (0, 2, 8, 4)])
def test_bucket_matches_numpy_stable_argsort(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, inv = moe.bucket(ids, E)
    flat = ids.ravel()
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(inv[perm], np.arange(T * k))


def test_slot_map_indirection_in_oracle():
    """Moving experts to other slots (and the map with them) leaves every output equal."""
    cfg = synth.config("tiny", T=8)
    L = synth.make_layer(cfg)
    ref = moe.layer(L.planes, "mxfp4", L.slot_map, L.wr, None, L.x, cfg.k)
    rng = np.random.default_rng(4)
    sigma = rng.permutation(cfg.E)                 # new slot of old slot s is sigma[s]
    planes2 = {n: np.empty_like(a) for n, a in L.planes.items()}
    for n, a in L.planes.items():
        planes2[n][sigma] = a
    sm2 = sigma[L.slot_map].astype(np.int32)
    got = moe.layer(planes2, "mxfp4", sm2, L.wr, None, L.x, cfg.k)
    assert np.array_equal(got["out"], ref["out"])


def test_zipf_bias_skews_the_load():
    cfg = synth.config("gptoss_prefill", T=2048)
    bias = synth.make_bias(cfg)
    ids, _, _ = moe.route(synth.make_x(cfg), synth.make_router(cfg), bias, cfg.k)
    counts = np.bincount(ids.ravel(), minlength=cfg.E)
    # the expert with the largest prior (r = 1, bias 0) is the busiest
    assert int(np.argmax(counts)) == int(np.argmax(bias))
    assert counts.max() > 4 * np.median(counts)


# ----------------------------------------------------------- resident hits and misses

def _routing(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    return ids


def test_miss_list_with_no_misses_and_with_every_expert_missing():
    T, k, E = 13, 3, 9
    ids = _routing(T, k, E, 1)
    counts, offsets, perm, inv = moe.bucket(ids, E)
    nonempty = int((counts > 0).sum())
    pos, mop, cnt = moe.miss_list(np.arange(E), offsets, perm)
    assert pos.size == 0 and np.all(mop == -1)
    assert cnt.tolist() == [T * k, 0, nonempty, 0]
    pos, mop, cnt = moe.miss_list(np.full(E, moe.SLOT_MISS), offsets, perm)
    assert np.array_equal(pos, np.arange(T * k))
    assert np.array_equal(mop, inv)          # every pair's index is its bucket position
    assert cnt.tolist() == [0, T * k, 0, nonempty]


@pytest.mark.parametrize("seed", [2, 3, 4])
def test_miss_list_matches_brute_force(seed):
    T, k, E = 37, 4, 16
    ids = _routing(T, k, E, seed)
    rng = np.random.default_rng(seed + 100)
    slot_map = rng.permutation(E).astype(np.int32)
    slot_map[rng.choice(E, size=5, replace=False)] = moe.SLOT_MISS
    counts, offsets, perm, inv = moe.bucket(ids, E)
    pos, mop, cnt = moe.miss_list(slot_map, offsets, perm)
    missed_pairs = [p for p in range(T * k) if slot_map[ids.flat[p]] == moe.SLOT_MISS]
    assert sorted(inv[p] for p in missed_pairs) == pos.tolist()
    for p in range(T * k):
        if p in missed_pairs:
            assert pos[mop[p]] == inv[p]
        else:
            assert mop[p] == -1
    used = set(ids.flat)
    assert cnt.tolist() == [T * k - len(missed_pairs), len(missed_pairs),
                            sum(1 for e in used if slot_map[e] != moe.SLOT_MISS),
                            sum(1 for e in used if slot_map[e] == moe.SLOT_MISS)]


def test_resident_combine_plus_merged_misses_is_the_full_combine():
    T, k, E, H = 21, 3, 8, 17
    ids = _routing(T, k, E, 5)
    rng = np.random.default_rng(6)
    w = rng.random((T, k))
    counts, offsets, perm, inv = moe.bucket(ids, E)
    y = rng.standard_normal((T * k, H))
    slot_map = np.arange(E, dtype=np.int32)
    slot_map[[1, 4, 6]] = moe.SLOT_MISS
    pos, mop, _ = moe.miss_list(slot_map, offsets, perm)
    part = moe.combine_hits(y, inv, w, T, k, mop)
    merged = moe.merge_misses(part, y[pos], mop, w, T, k)
    full = moe.combine(y, inv, w, T, k)
    assert np.allclose(merged, full, rtol=1e-13, atol=1e-13)
    # and the resident part alone is the mixture with the missed terms dropped
    y0 = y.copy()
    y0[pos] = 0.0
    assert np.allclose(part, moe.combine(y0, inv, w, T, k), rtol=1e-13, atol=1e-13)


def test_oracle_refuses_a_non_resident_slot():
    cfg = synth.config("tiny", T=4)
    L = synth.make_layer(cfg)
    ids, _, _ = moe.route(L.x, L.wr, None, cfg.k)
    counts, offsets, perm, _ = moe.bucket(ids, cfg.E)
    sm = L.slot_map.copy()
    sm[int(ids[0, 0])] = moe.SLOT_MISS
    with pytest.raises(ValueError):
        moe.expert_ffn(L.planes, cfg.fmt, sm, L.x, cfg.k, offsets, perm)


# ------------------------------------------------------------------ staged prefill

@pytest.mark.parametrize("seed,n_stage", [(1, 16), (2, 3), (3, 0), (4, 7)])
def test_stage_plan_matches_brute_force(seed, n_stage):
    E = 16
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 3, size=E)
    slot_map = np.full(E, moe.SLOT_MISS, dtype=np.int32)
    resident = rng.choice(E, size=5, replace=False)
    slot_map[resident] = np.arange(5)
    first = 5
    sm, copy_list, cnt = moe.stage_plan(counts, slot_map, first, n_stage)
    want = sorted(e for e in range(E) if counts[e] > 0 and e not in set(resident.tolist()))
    staged = want[:n_stage]
    assert copy_list.tolist() == staged
    assert cnt.tolist() == [len(staged), len(want) - len(staged)]
    for e in range(E):
        if e in staged:
            assert sm[e] == first + staged.index(e)
        else:
            assert sm[e] == slot_map[e]
    # the window's slots are distinct, inside the window, and increase with the expert index
    ws = [int(sm[e]) for e in staged]
    assert ws == list(range(first, first + len(staged)))


def _resident_and_backing(L, E, resident):
    """Backing store indexed by expert, and a pool whose first slots hold `resident`."""
    backing = {n: a[L.slot_map] for n, a in L.planes.items()}
    S = len(resident) + E
    pool = {n: np.zeros((S,) + a.shape[1:], dtype=a.dtype) for n, a in backing.items()}
    slot_map = np.full(E, moe.SLOT_MISS, dtype=np.int32)
    for i, e in enumerate(resident):
        slot_map[e] = i
        for n in pool:
            pool[n][i] = backing[n][e]
    return backing, pool, slot_map


def test_staged_pool_gives_the_all_resident_layer():
    """Staging every used non-resident expert and rewriting the map reproduces, exactly, the
    layer computed with every expert resident."""
    cfg = synth.config("tiny", T=32)
    L = synth.make_layer(cfg)
    resident = [1, 4, 6]
    backing, pool, slot_map = _resident_and_backing(L, cfg.E, resident)
    ids, _, _ = moe.route(L.x, L.wr, None, cfg.k)
    counts, _, _, _ = moe.bucket(ids, cfg.E)
    first = len(resident)
    sm, copy_list, cnt = moe.stage_plan(counts, slot_map, first, cfg.E)
    assert cnt[1] == 0 and cnt[0] == int(((counts > 0) & (slot_map == moe.SLOT_MISS)).sum())
    staged = moe.stage_copy(pool, backing, copy_list, first)
    got = moe.layer(staged, cfg.fmt, sm, L.wr, None, L.x, cfg.k)
    ref = moe.layer(L.planes, cfg.fmt, L.slot_map, L.wr, None, L.x, cfg.k)
    assert np.array_equal(got["out"], ref["out"])
    assert np.array_equal(got["h"], ref["h"])


def test_window_overflow_takes_the_miss_path():
    """With a window smaller than the batch needs, the experts left out stay non-resident;
    their pairs computed elsewhere and merged give the full layer."""
    cfg = synth.config("tiny", T=32)
    L = synth.make_layer(cfg)
    backing, pool, slot_map = _resident_and_backing(L, cfg.E, [0, 5])
    ids, w, _ = moe.route(L.x, L.wr, None, cfg.k)
    counts, offsets, perm, inv = moe.bucket(ids, cfg.E)
    sm, copy_list, cnt = moe.stage_plan(counts, slot_map, 2, 2)
    assert cnt[0] == 2 and cnt[1] > 0
    staged = moe.stage_copy(pool, backing, copy_list, 2)
    pos, mop, mcnt = moe.miss_list(sm, offsets, perm)
    assert mcnt[3] == cnt[1]
    # resident and staged pairs from the pool; missed pairs from the backing store
    ident = np.arange(cfg.E, dtype=np.int32)
    _, y_all, _ = moe.expert_ffn(backing, cfg.fmt, ident, L.x, cfg.k, offsets, perm)
    hit_pos = np.setdiff1d(np.arange(perm.size), pos)
    _, y_hit, _ = moe.expert_ffn(staged, cfg.fmt, np.where(sm < 0, 0, sm), L.x, cfg.k,
                                 offsets, perm, hit_pos)
    y = np.where(np.isnan(y_hit), 0.0, y_hit)
    part = moe.combine_hits(y, inv, w, cfg.T, cfg.k, mop)
    merged = moe.merge_misses(part, y_all[pos], mop, w, cfg.T, cfg.k)
    assert np.allclose(merged, moe.combine(y_all, inv, w, cfg.T, cfg.k), rtol=1e-12,
                       atol=1e-12)


# ------------------------------------------------------------------ Q4_K experts

def test_q4_k_layer_equals_the_q8_0_layer_of_the_same_weights():
    """Q4_K experts whose scales are d = 1, sc = 1 and whose mins are 0 carry the integer
    weights q in 0..15; the same integers as Q8_0 codes with d = 1 give the same layer."""
    cfg = synth.config("tiny_q4k", T=8)
    L = synth.make_layer(cfg)
    one = np.float16(1.0).view(np.uint16)
    planes4, planes8 = {}, {}
    for n in ("gate", "up", "down"):
        codes = L.planes[n + "_q"]                          # [S, rows, K/2]
        S, rows, half = codes.shape
        K = 2 * half
        nb, ns = K // 32, K // 256
        sc = np.zeros((S, rows, 2 * nb + 4 * ns), dtype=np.uint8)
        sc[..., 0:2 * nb:2] = 1                              # sc_b = 1, m_b = 0
        sup = np.zeros((S, rows, ns, 2), dtype=np.uint16)
        sup[..., 0] = one                                    # d = 1, dmin = 0
        sc[..., 2 * nb:] = sup.reshape(S, rows, 2 * ns).view(np.uint8)
        planes4[n + "_q"], planes4[n + "_s"] = codes, sc
        q8 = np.empty((S, rows, K), dtype=np.int8)
        q8[..., 0::2] = codes & 15
        q8[..., 1::2] = codes >> 4
        planes8[n + "_q"] = q8
        planes8[n + "_s"] = np.full((S, rows, nb), one, dtype=np.uint16)
    a = moe.layer(planes4, "q4_k", L.slot_map, L.wr, None, L.x, cfg.k)
    b = moe.layer(planes8, "q8_0", L.slot_map, L.wr, None, L.x, cfg.k)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["out"], b["out"])


def test_q6_k_layer_equals_the_q8_0_layer_of_the_same_weights():
    """Q6_K experts with d = 1 and every sub-block scale 1 carry the integer weights q - 32;
    the same integers as Q8_0 codes with d = 1 give the same layer."""
    cfg = synth.config("tiny_q6k", T=8)
    L = synth.make_layer(cfg)
    one = np.float16(1.0).view(np.uint16)
    planes6, planes8 = {}, {}
    for n in ("gate", "up", "down"):
        codes = L.planes[n + "_q"]                          # [S, rows, K/2 + K/4]
        S, rows, nbytes = codes.shape
        K = nbytes * 4 // 3
        sc = np.ones((S, rows, K // 16), dtype=np.uint8)
        d = np.full((S, rows, K // 256), one, dtype=np.uint16)
        planes6[n + "_q"] = codes
        planes6[n + "_s"] = np.concatenate([sc, d.view(np.uint8)], axis=2)
        lo, hi = codes[..., :K // 2], codes[..., K // 2:]
        q = np.empty((S, rows, K), dtype=np.int64)
        q[..., 0::2] = lo & 15
        q[..., 1::2] = lo >> 4
        for i in range(4):
            q[..., i::4] += 16 * ((hi >> (2 * i)) & 3)
        planes8[n + "_q"] = (q - 32).astype(np.int8)
        planes8[n + "_s"] = np.full((S, rows, K // 32), one, dtype=np.uint16)
    with np.errstate(over="ignore"):   # integer weights: silu meets exp of large -g (-> 0)
        a = moe.layer(planes6, "q6_k", L.slot_map, L.wr, None, L.x, cfg.k)
        b = moe.layer(planes8, "q8_0", L.slot_map, L.wr, None, L.x, cfg.k)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["out"], b["out"])

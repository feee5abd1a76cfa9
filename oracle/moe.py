"""The routed MoE FFN layer as plain fp64 definitions.

TEST INFRASTRUCTURE: part of the CPU oracle (see oracle/__init__.py for who may use it).

What the layer is, from the pages:
  * tinyserve README, "How it works" item 2: each selected expert's forward is a gate,
    an up and a down projection computed on the native quantized bytes;
  * tinyserve README, "How it works" item 3: experts are reached through a GPU slot map;
  * tinyserve README, "How it works" item 6: tokens are grouped by expert so that each
    expert's weights are loaded once;
  * llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution",
    original post: the router stays on the GPU, the selected expert IDs are served from
    a resident pool, and the weighted outputs are merged; its "Formal gate results"
    follow-up: router output -> mapping rewrite -> grouped quantized matmul.
The pages give no formulas. The definitions written out here are the plain reading
of that structure:
  logits   L[t,e] = sum_h x[t,h] Wr[e,h] + b[e]
  top-k    the k largest L[t,:], ordered by (-L, e): ties go to the lower expert index
  weights  w[t,j] = exp(L_j - L_0) / sum_{i<k} exp(L_i - L_0)  (softmax over the k chosen)
  bucket   pairs p = t*k + j grouped by expert, ascending p inside each expert
  expert   g = Wg x, u = Wu x, h = bf16_RNE(silu(g) * u), y = Wd h, silu(z) = z / (1 + e^-z)
  combine  out[t] = sum_{j<k} w[t,j] * y[pair (t, j)]
  misses   an expert whose slot is SLOT_MISS is not resident: its pairs are listed (in bucket
           order) for computation elsewhere, the resident pairs are combined, and the
           missed pairs' outputs are merged afterwards, per token in j order
  staging  the batch's used, non-resident experts are copied into a window of staging
           slots (in increasing expert index) and the slot map is rewritten to point at
           them before the grouped expert matmul
All arithmetic is fp64; the one rounding is h to bf16, taken directly from fp64.
"""
from __future__ import annotations

import numpy as np

from . import codecs


# ------------------------------------------------------------------------------ route


def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray, bias=None) -> np.ndarray:
    """L = x Wr^T (+ b) in fp64: [T, H] bf16 bits x [E, H] bf16 bits -> [T, E]."""
    x = codecs.bf16_decode(x_bits)
    wr = codecs.bf16_decode(wr_bits)
    L = x @ wr.T
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return L


def topk_softmax(L: np.ndarray, k: int):
    """Per row: the k largest logits by (-L, index), and the softmax over those k.

    Returns ids int32 [T, k] and weights fp64 [T, k]. NaN logits count as -inf.
    """
    L = np.where(np.isnan(L), -np.inf, L)
    T, E = L.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -L[t]))          # primary key -L, then index
        sel = order[:k]
        ids[t] = sel
        z = np.exp(L[t, sel] - L[t, sel[0]])
        w[t] = z / z.sum()
    return ids, w


def route(x_bits, wr_bits, bias, k):
    """Router + top-k + softmax. Returns (ids [T,k] int32, w [T,k] fp64, logits [T,E])."""
    L = router_logits(x_bits, wr_bits, bias)
    ids, w = topk_softmax(L, k)
    return ids, w, L


# ----------------------------------------------------------------------------- bucket


def bucket(ids: np.ndarray, E: int):
    """Counting sort of the pairs p = t*k + j by expert, keeping ascending p within an expert.

    Returns counts [E], offsets [E+1] (exclusive scan, offsets[E] = T*k),
    perm [T*k] (perm[pos] = p) and inv_perm [T*k] (inv_perm[p] = pos), all int32.
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    n = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:E].copy()
    perm = np.empty(n, dtype=np.int64)
    for p in range(n):
        e = flat[p]
        perm[fill[e]] = p
        fill[e] += 1
    inv_perm = np.empty(n, dtype=np.int64)
    inv_perm[perm] = np.arange(n)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), inv_perm.astype(np.int32))


# ------------------------------------------------------------------------- expert FFN


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def _slot_weights(planes, fmt, slot, name):
    if slot < 0:
        raise ValueError(f"slot {slot}: a non-resident expert has no weights in the pool")
    return codecs.dequant(fmt, planes[name + "_q"][slot], planes[name + "_s"][slot])


def expert_ffn(planes: dict, fmt: str, slot_map, x_bits, k: int, offsets, perm,
               positions=None):
    """Gate/up/SwiGLU/down for the bucketed pairs.

    planes: the pool in canonical layout, indexed by slot (see synth).
    positions: bucket positions to compute (default: all). Results for other positions
    are left as NaN (h as 0) so a partial evaluation cannot be mistaken for a full one.
    Returns (h_bits uint16 [T*k, I], y fp64 [T*k, H], a fp64 [T*k, I]) where a is the
    pre-rounding silu(g)*u.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    n = perm.size
    E = offsets.size - 1
    I = planes["gate_q"].shape[1]
    want = _wanted(n, positions)
    x_all = codecs.bf16_decode(x_bits)
    h_bits = np.zeros((n, I), dtype=np.uint16)
    a = np.full((n, I), np.nan)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pos = np.arange(lo, hi)[want[lo:hi]]
        if pos.size == 0:
            continue
        slot = int(slot_map[e])
        xe = x_all[perm[pos] // k]                          # [n_e, H]
        Wg = _slot_weights(planes, fmt, slot, "gate")       # [I, H]
        g = xe @ Wg.T
        del Wg
        Wu = _slot_weights(planes, fmt, slot, "up")
        u = xe @ Wu.T
        del Wu
        a[pos] = silu(g) * u
        h_bits[pos] = codecs.bf16_bits(codecs.bf16_round(a[pos]))
    y = down_proj(planes, fmt, slot_map, h_bits, offsets, positions)
    return h_bits, y, a


def down_proj(planes: dict, fmt: str, slot_map, h_bits, offsets, positions=None):
    """y[pos] = W_down[slot_map[e]] h[pos] in fp64 for the bucketed rows of h (bf16 bits).

    Used on the oracle's own h, and to judge a down projection at another party's h.
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    n = int(offsets[-1])
    E = offsets.size - 1
    H = planes["down_q"].shape[1]
    want = _wanted(n, positions)
    y = np.full((n, H), np.nan)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        pos = np.arange(lo, hi)[want[lo:hi]]
        if pos.size == 0:
            continue
        Wd = _slot_weights(planes, fmt, int(slot_map[e]), "down")   # [H, I]
        y[pos] = codecs.bf16_decode(np.asarray(h_bits)[pos]) @ Wd.T
    return y


def _wanted(n, positions):
    want = np.zeros(n, dtype=bool)
    want[np.arange(n) if positions is None else np.asarray(positions, dtype=np.int64)] = True
    return want


# ---------------------------------------------------------------------------- combine


def combine(y: np.ndarray, inv_perm, w: np.ndarray, T: int, k: int, tokens=None):
    """out[t] = sum_{j<k} w[t,j] * y[inv_perm[t*k + j]], summed in j order, fp64.

    tokens: which tokens to compute (default all); other rows are NaN.
    """
    inv_perm = np.asarray(inv_perm, dtype=np.int64)
    H = y.shape[1]
    out = np.full((T, H), np.nan)
    ts = range(T) if tokens is None else tokens
    for t in ts:
        acc = np.zeros(H)
        for j in range(k):
            acc = acc + float(w[t, j]) * y[inv_perm[t * k + j]]
        out[t] = acc
    return out


# ------------------------------------------------------------------------------ layer


def layer(planes: dict, fmt: str, slot_map, wr_bits, bias, x_bits, k: int):
    """The whole layer on every token. Returns a dict of every intermediate."""
    T = x_bits.shape[0]
    E = wr_bits.shape[0]
    ids, w, L = route(x_bits, wr_bits, bias, k)
    counts, offsets, perm, inv_perm = bucket(ids, E)
    h, y, a = expert_ffn(planes, fmt, slot_map, x_bits, k, offsets, perm)
    out = combine(y, inv_perm, w, T, k)
    return dict(logits=L, ids=ids, w=w, counts=counts, offsets=offsets, perm=perm,
                inv_perm=inv_perm, a=a, h=h, y=y, out=out)


# -------------------------------------------------------------- resident hits and misses
#
# llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution",
# original post: the selected expert IDs are split into resident hits, served from the GPU
# pool, and misses, computed elsewhere; the weighted outputs are then merged. The same post
# proposes public hit/miss counters.

SLOT_MISS = -1


def miss_list(slot_map, offsets, perm):
    """The pairs routed to non-resident experts (slot_map[e] == SLOT_MISS).

    Returns (miss_pos, miss_of_pair, counters):
      miss_pos      int32 [n_miss]: their bucket positions, increasing (expert by expert)
      miss_of_pair  int32 [T*k]: for pair p = t*k + j, its index in miss_pos, or -1
      counters      int32 [4]: resident pairs, missed pairs, resident experts with pairs,
                    non-resident experts with pairs
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    E = offsets.size - 1
    n = perm.size
    miss_pos = []
    hit_e = miss_e = 0
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        if int(slot_map[e]) == SLOT_MISS:
            miss_pos.extend(range(lo, hi))
            miss_e += 1
        else:
            hit_e += 1
    miss_pos = np.array(miss_pos, dtype=np.int32)
    miss_of_pair = np.full(n, -1, dtype=np.int32)
    for i, pos in enumerate(miss_pos):
        miss_of_pair[perm[pos]] = i
    counters = np.array([n - miss_pos.size, miss_pos.size, hit_e, miss_e], dtype=np.int32)
    return miss_pos, miss_of_pair, counters


def combine_hits(y: np.ndarray, inv_perm, w: np.ndarray, T: int, k: int, miss_of_pair):
    """out[t] = sum over the resident pairs j of w[t,j] * y[inv_perm[t*k + j]], j order."""
    inv_perm = np.asarray(inv_perm, dtype=np.int64)
    out = np.zeros((T, y.shape[1]))
    for t in range(T):
        for j in range(k):
            p = t * k + j
            if miss_of_pair[p] < 0:
                out[t] = out[t] + float(w[t, j]) * y[inv_perm[p]]
    return out


def merge_misses(out: np.ndarray, y_miss: np.ndarray, miss_of_pair, w: np.ndarray, T: int,
                 k: int):
    """out[t] + sum over the missed pairs j (in j order) of w[t,j] * y_miss[miss_of_pair[p]]."""
    res = np.array(out, dtype=np.float64, copy=True)
    for t in range(T):
        for j in range(k):
            m = int(miss_of_pair[t * k + j])
            if m >= 0:
                res[t] = res[t] + float(w[t, j]) * y_miss[m]
    return res


# ------------------------------------------------------------------ staged prefill
#
# llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution",
# "Formal gate results": for a large prefill batch, the unique experts the router picked
# are packed, copied in bulk into shared staging windows of GPU slots, the mapping is
# rewritten to those slots, and the grouped quantized matmul runs on the rewritten map.
# tinyserve README, "How it works" item 6: each expert of the batch is loaded once.
# Reading: the experts to stage are the used (count > 0) experts whose slot is SLOT_MISS;
# they take the window's slots in increasing expert index; experts beyond the window's
# size stay SLOT_MISS (their pairs then take the miss path above).


def stage_plan(counts, slot_map, first_slot: int, n_stage: int):
    """Staging plan of one batch.

    Returns (slot_map_out, copy_list, counters):
      slot_map_out int32 [E]: resident experts and unused experts unchanged; the i-th staged
                   expert (increasing index) maps to slot first_slot + i
      copy_list    int32 [n_staged]: the staged experts, in slot order
      counters     int32 [2]: experts staged, used non-resident experts left out (window full)
    """
    counts = np.asarray(counts, dtype=np.int64)
    out = np.array(slot_map, dtype=np.int32, copy=True)
    need = [e for e in range(counts.size) if counts[e] > 0 and int(slot_map[e]) == SLOT_MISS]
    staged = need[:n_stage]
    for i, e in enumerate(staged):
        out[e] = first_slot + i
    copy_list = np.array(staged, dtype=np.int32)
    counters = np.array([len(staged), len(need) - len(staged)], dtype=np.int32)
    return out, copy_list, counters


def stage_copy(planes: dict, backing: dict, copy_list, first_slot: int) -> dict:
    """The pool after the copy: slot first_slot + i holds every plane of expert copy_list[i]
    taken from the backing store (indexed by expert); every other slot is unchanged."""
    res = {n: np.array(a, copy=True) for n, a in planes.items()}
    for i, e in enumerate(copy_list):
        for n in res:
            res[n][first_slot + i] = backing[n][int(e)]
    return res

"""Resident hits and misses on the GPU (moe_miss_list, moe_merge_misses and the layer with
non-resident experts), through the C ABI, against the CPU oracle.

llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution",
original post: the chosen experts that sit in the GPU pool are served there, the others are
computed elsewhere, and the weighted outputs are merged.
"""
import numpy as np
import pytest

import synth
from oracle import codecs, moe as omoe

from parity import W_ABS, assert_close_rows, make_case, rel_l2_rows, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import quantized_routed_expert_gemv_amd as qm  # noqa: E402


def _random_routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    counts, offsets, perm, inv = omoe.bucket(ids, E)
    return ids, offsets, perm, inv


def _gpu_miss_list(slot_map, offsets, perm, k):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    mp, mop, cnt = qm.miss_list(dev(slot_map), dev(offsets), dev(perm), k)
    torch.cuda.synchronize()
    return mp.cpu().numpy(), mop.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("T,E,k,frac,seed", [
    (64, 8, 2, 0.5, 1),        # small
    (1, 32, 4, 0.5, 2),        # one decode token
    (8192, 128, 8, 0.3, 3),    # many pairs: the list loops over the workgroup
    (300, 256, 8, 0.9, 4),     # the largest expert count
    (64, 8, 2, 0.0, 5),        # every expert resident
    (64, 8, 2, 1.0, 6),        # none resident
])
def test_miss_list_matches_oracle(T, E, k, frac, seed):
    print(f"miss list T={T} E={E} k={k} frac={frac}", flush=True)
    ids, offsets, perm, inv = _random_routing(T, E, k, seed)
    rng = np.random.default_rng(100 + seed)
    slot_map = rng.permutation(E).astype(np.int32)
    slot_map[rng.random(E) < frac] = qm.SLOT_MISS
    mp, mop, cnt = _gpu_miss_list(slot_map, offsets, perm, k)
    rp, rmop, rcnt = omoe.miss_list(slot_map, offsets, perm)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(mp, rp)
    assert np.array_equal(mop, rmop)


def test_miss_list_without_tokens():
    E, k = 8, 2
    slot_map = np.full(E, qm.SLOT_MISS, dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    mp, mop, cnt = _gpu_miss_list(slot_map, offsets, np.zeros(0, dtype=np.int32), k)
    assert mp.size == 0 and mop.size == 0 and np.array_equal(cnt, [0, 0, 0, 0])


def _close(got, ref, rel):
    """|got - ref| <= rel * (|ref| + max|ref|): sums of the same terms in another order."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return bool(np.all(np.abs(got - ref) <= rel * (np.abs(ref) + np.abs(ref).max())))


@pytest.mark.parametrize("T,k,H", [(5, 4, 256), (70000, 2, 32)])   # the latter > grid.y limit
def test_merge_misses_matches_oracle(T, k, H):
    print(f"merge T={T} k={k} H={H}", flush=True)
    rng = np.random.default_rng(T)
    out0 = rng.standard_normal((T, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    missed = rng.random(T * k) < 0.4
    mop = np.full(T * k, -1, dtype=np.int32)
    mop[missed] = rng.permutation(int(missed.sum())).astype(np.int32)
    y_miss = rng.standard_normal((int(missed.sum()), H)).astype(np.float32)
    out = torch.from_numpy(out0.copy()).cuda()
    qm.merge_misses(out, torch.from_numpy(y_miss).cuda(), torch.from_numpy(mop).cuda(),
                    torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ref = omoe.merge_misses(out0.astype(np.float64), y_miss.astype(np.float64), mop,
                            w.astype(np.float64), T, k)
    assert _close(out.cpu().numpy(), ref, 1e-6)


def _layer(pool, sm, wr, bias, x, k, path):
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ws = qm.layer(pool, sm, wr, bias, x, k, err_flags=err, path=path)
    torch.cuda.synchronize()
    return out.cpu().numpy(), {n: t.cpu() for n, t in ws.intermediates().items()}, \
        int(err.item())


CASES = [
    # fused decode (routing finished in the gate/up kernel), full gpt-oss shape
    ("gptoss_decode_t1", None, qm.PATH_AUTO),
    ("gptoss_decode_t4", None, qm.PATH_AUTO),
    # Q8_0 decode
    ("mixtral_q8_decode", dict(T=3, H=512, I=1024), qm.PATH_AUTO),
    # GEMV path over bucketed pairs (more tokens than the fused decode takes)
    ("tiny", dict(T=17), qm.PATH_GEMV),
    # grouped GEMM
    ("tiny", dict(T=130), qm.PATH_GROUPED),
    ("qwen_a3b_decode", dict(T=64, H=512), qm.PATH_GROUPED),
]


@pytest.mark.parametrize("name,over,path", CASES)
def test_layer_with_non_resident_experts(name, over, path):
    """Experts marked SLOT_MISS: no flag; their h and y rows are zero; every resident pair is
    bit-identical to the all-resident layer; out is the weighted sum of the resident pairs;
    the GPU miss list equals the oracle's; and merging expert outputs computed elsewhere for
    the missed pairs gives the full layer."""
    cfg = synth.config(name, **over) if over else synth.CONFIGS[name]
    print(f"misses {cfg.name} T={cfg.T} H={cfg.H} path={path}", flush=True)
    T, k, E = cfg.T, cfg.k, cfg.E
    L = make_case(cfg)
    ids, w, _ = omoe.route(L.x, L.wr, L.bias, k)
    counts, offsets, perm, inv = omoe.bucket(ids, E)
    # every other chosen expert is non-resident (so tokens mix hits and misses)
    chosen = np.unique(ids)
    missing = chosen[::2]
    pool, x, wr, bias, sm = to_device(L)
    sm_miss = sm.clone()
    sm_miss[torch.from_numpy(missing.astype(np.int64)).cuda()] = qm.SLOT_MISS
    slot_miss = sm_miss.cpu().numpy()

    out_full, im_full, err_full = _layer(pool, sm, wr, bias, x, k, path)
    out_hit, im, err = _layer(pool, sm_miss, wr, bias, x, k, path)
    assert err_full == 0 and err == 0
    assert np.array_equal(im["ids"].numpy(), ids)
    for n, ref in (("offsets", offsets), ("perm", perm), ("inv_perm", inv)):
        assert np.array_equal(im[n].numpy(), ref), n

    rp, rmop, rcnt = omoe.miss_list(slot_miss, offsets, perm)
    assert rcnt[1] > 0 and (rcnt[0] > 0 or T * k == rcnt[1])
    missed = np.zeros(T * k, dtype=bool)
    missed[rp] = True
    y_full, y = im_full["y"].numpy(), im["y"].numpy()
    assert np.all(y[missed] == 0) and torch.all(im["h"][torch.from_numpy(missed)].float() == 0)
    assert np.array_equal(y[~missed], y_full[~missed])

    wg = im["w"].numpy()
    assert np.abs(wg - w).max() <= W_ABS
    hits_ref = omoe.combine_hits(y.astype(np.float64), inv, wg, T, k, rmop)
    assert _close(out_hit, hits_ref, 1e-5)

    # the GPU miss list over the GPU's own bucketing
    mp, mop, cnt = qm.miss_list(sm_miss, im["offsets"].cuda(), im["perm"].cuda(), k)
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(mp.cpu().numpy(), rp)
    assert np.array_equal(mop.cpu().numpy(), rmop)

    # (a) the misses' outputs from the all-resident layer: merged = the full layer
    out_a = torch.from_numpy(out_hit).cuda()
    y_miss = torch.from_numpy(np.ascontiguousarray(y_full[rp])).cuda()
    qm.merge_misses(out_a, y_miss, mop, im["w"].cuda())
    torch.cuda.synchronize()
    out_a = out_a.cpu().numpy()
    assert _close(out_a, omoe.merge_misses(out_hit, y_full[rp].astype(np.float64), rmop, wg,
                                           T, k), 1e-6)
    assert _close(out_a, out_full, 1e-5)

    # (b) the misses computed by the oracle, as a host would: merged = the pure oracle layer
    positions = np.arange(T * k)
    _, _, a_ref = omoe.expert_ffn(L.planes, cfg.fmt, L.slot_map, L.x, k, offsets, perm,
                                  positions)
    y_pure = omoe.down_proj(L.planes, cfg.fmt, L.slot_map,
                            codecs.bf16_bits(codecs.bf16_round(a_ref)), offsets, positions)
    out_b = torch.from_numpy(out_hit).cuda()
    qm.merge_misses(out_b, torch.from_numpy(np.ascontiguousarray(y_pure[rp], dtype=np.float32))
                    .cuda(), mop, im["w"].cuda())
    torch.cuda.synchronize()
    out_pure = omoe.combine(y_pure, inv, w, T, k)
    r = rel_l2_rows(out_b.cpu().numpy(), out_pure).max()
    assert_close_rows(out_b.cpu().numpy(), out_pure, "merged out")
    print(f"  pairs {T * k}: {rcnt[0]} resident, {rcnt[1]} missed; merged vs oracle L2 "
          f"{r:.2e}", flush=True)

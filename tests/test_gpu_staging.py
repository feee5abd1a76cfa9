"""Staged prefill on the GPU (moe_stage_plan, moe_stage_copy, and the layer on the rewritten
map), through the C ABI, against the CPU oracle.

llama.cpp discussion "fixed GPU expert working set with Native CPU miss execution",
"Formal gate results": the batch's unique experts are copied into shared staging windows,
the mapping is rewritten to those slots, and the grouped quantized matmul runs on it.
"""
import numpy as np
import pytest

import synth
from oracle import moe as omoe

from parity import assert_close_rows, make_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import quantized_routed_expert_gemv_amd as qm  # noqa: E402

PLANES = ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("E,n_stage,seed", [(8, 8, 1), (32, 5, 2), (128, 40, 3), (256, 0, 4),
                                            (256, 256, 5), (256, 17, 6)])
def test_stage_plan_matches_oracle(E, n_stage, seed):
    print(f"stage plan E={E} window={n_stage}", flush=True)
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 3, size=E).astype(np.int32)
    slot_map = np.full(E, qm.SLOT_MISS, dtype=np.int32)
    res = rng.choice(E, size=E // 3, replace=False)
    slot_map[res] = rng.permutation(E // 3)
    first = E // 3
    sm, cl, cnt = qm.stage_plan(_dev(counts), _dev(slot_map), first, n_stage)
    rsm, rcl, rcnt = omoe.stage_plan(counts, slot_map, first, n_stage)
    torch.cuda.synchronize()
    cnt = cnt.cpu().numpy()
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(sm.cpu().numpy(), rsm)
    assert np.array_equal(cl.cpu().numpy()[:cnt[0]], rcl)
    # in place
    smi = _dev(slot_map)
    qm.stage_plan(_dev(counts), smi, first, n_stage, slot_map_out=smi)
    torch.cuda.synchronize()
    assert np.array_equal(smi.cpu().numpy(), rsm)


def _setup(cfg, resident, window):
    """Backing store (slot = expert), and a pool whose first slots hold `resident` and whose
    window slots hold some other expert's bytes (so a missing copy cannot pass)."""
    L = make_case(cfg)
    E = cfg.E
    by_expert = {n: a[L.slot_map] for n, a in L.planes.items()}
    backing = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I, by_expert)
    S = len(resident) + window
    filler = [resident[i] if i < len(resident) else (i * 7 + 3) % E for i in range(S)]
    pool = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I,
                                  {n: a[filler] for n, a in by_expert.items()})
    slot_map = np.full(E, qm.SLOT_MISS, dtype=np.int32)
    slot_map[resident] = np.arange(len(resident), dtype=np.int32)
    L.by_expert = by_expert
    L.pool_planes = {n: a[filler] for n, a in by_expert.items()}
    return L, backing, pool, slot_map


def _slot_bytes(pool, n, s):
    b = pool.planes[n].numel() // pool.n_slots
    return pool.planes[n][s * b:(s + 1) * b]


CASES = [
    # name, overrides, resident experts, window, path
    ("tiny", dict(T=130), [1, 4], 6, qm.PATH_GROUPED),
    ("tiny", dict(T=130), [1, 4], 2, qm.PATH_GROUPED),          # window too small
    ("mixtral_q8_prefill", dict(T=96, H=512, I=1024), [0], 7, qm.PATH_GROUPED),
    ("qwen_a3b_prefill", dict(T=512, H=512), list(range(0, 128, 3)), 80, qm.PATH_GROUPED),
    ("gptoss_prefill", None, list(range(0, 32, 3)), 21, qm.PATH_AUTO),   # full size
    ("gptoss_decode_t4", None, [], 4, qm.PATH_AUTO),            # decode: nothing resident
]


@pytest.mark.parametrize("name,over,resident,window,path", CASES)
def test_staged_layer_equals_the_all_resident_layer(name, over, resident, window, path):
    """Plan (bit-exact against the oracle), copy (bytes equal to the backing store's), then
    the layer on the rewritten map: bit-identical to the layer with every expert resident
    when the window holds every needed expert; otherwise the experts left out take the miss
    path and merging their outputs gives the same layer."""
    cfg = synth.config(name, **over) if over else synth.CONFIGS[name]
    print(f"staging {cfg.name} T={cfg.T} H={cfg.H} resident={len(resident)} window={window}",
          flush=True)
    T, k, E = cfg.T, cfg.k, cfg.E
    L, backing, pool, slot_map = _setup(cfg, resident, window)
    x = torch.from_numpy(L.x.view(np.int16)).cuda().view(torch.bfloat16)
    wr = torch.from_numpy(L.wr.view(np.int16)).cuda().view(torch.bfloat16)
    bias = None if L.bias is None else torch.from_numpy(L.bias).cuda()
    ident = torch.arange(E, dtype=torch.int32, device="cuda")
    out_full, ws = qm.layer(backing, ident, wr, bias, x, k, path=path)
    im = {n: t.cpu() for n, t in ws.intermediates().items()}
    y_full = im["y"].numpy()
    counts = ws.intermediates()["counts"]

    first = len(resident)
    sm, cl, cnt = qm.stage_plan(counts, _dev(slot_map), first, window)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    qm.stage_copy(pool, backing, cl, cnt, first, window, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    rsm, rcl, rcnt = omoe.stage_plan(im["counts"].numpy(), slot_map, first, window)
    cnt = cnt.cpu().numpy()
    assert np.array_equal(cnt, rcnt) and np.array_equal(sm.cpu().numpy(), rsm)
    assert np.array_equal(cl.cpu().numpy()[:cnt[0]], rcl)
    for i, e in enumerate(rcl):
        for n in PLANES:
            assert torch.equal(_slot_bytes(pool, n, first + i), _slot_bytes(backing, n, int(e))), \
                (i, int(e), n)

    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ws2 = qm.layer(pool, sm, wr, bias, x, k, err_flags=err, path=path)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    if rcnt[1] == 0:
        assert torch.equal(out, out_full)
        if T * k <= 512:
            # the oracle layer on the oracle's staged pool and rewritten map
            staged = omoe.stage_copy(L.pool_planes, L.by_expert, rcl, first)
            ref = omoe.layer(staged, cfg.fmt, rsm, L.wr, L.bias, L.x, k)["out"]
            assert_close_rows(out.cpu().numpy(), ref, "out")
    else:
        mp, mop, mcnt = qm.miss_list(sm, ws2.intermediates()["offsets"],
                                     ws2.intermediates()["perm"], k)
        assert int(mcnt[3].item()) == rcnt[1]
        y_miss = torch.from_numpy(np.ascontiguousarray(y_full[mp.cpu().numpy()])).cuda()
        qm.merge_misses(out, y_miss, mop, ws2.intermediates()["w"])
        torch.cuda.synchronize()
        ref = out_full.cpu().numpy().astype(np.float64)
        got = out.cpu().numpy()
        assert np.all(np.abs(got - ref) <= 1e-5 * (np.abs(ref) + np.abs(ref).max()))
    print(f"  staged {cnt[0]} experts, left out {cnt[1]}", flush=True)


def test_copy_of_an_expert_outside_the_backing_store_sets_the_flag():
    cfg = synth.config("tiny", T=4)
    L, backing, pool, slot_map = _setup(cfg, [0], 2)
    before = {n: t.clone() for n, t in pool.planes.items()}
    cl = _dev([cfg.E + 3, 0])
    cnt = _dev([1, 0])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    qm.stage_copy(pool, backing, cl, cnt, 1, 2, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    for n, t in pool.planes.items():
        assert torch.equal(t, before[n])


def test_staged_layers_with_the_copy_on_a_second_stream():
    """Staging overlapped with compute: three layers, each with its own pool and window; each
    layer's plan and copy run on a second stream (default priority) one layer ahead, planned
    from a count of one per expert, and the compute stream waits on an event before the
    layer's expert FFN. Every layer equals its all-resident layer bit for bit."""
    cfg = synth.config("qwen_a3b_prefill", T=384, H=512)
    E, k, T = cfg.E, cfg.k, cfg.T
    resident = list(range(0, E, 3))
    window = E - len(resident)
    first = len(resident)
    compute, copier = torch.cuda.Stream(), torch.cuda.Stream()
    every = torch.ones(E, dtype=torch.int32, device="cuda")
    layers = []
    for l in range(3):
        L, backing, pool, slot_map = _setup_layer(cfg, l, resident, window)
        layers.append((L, backing, pool, _dev(slot_map)))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    maps, ready, outs = [], [], []
    with torch.cuda.stream(copier):
        for L, backing, pool, smr in layers:
            sm, cl, cnt = qm.stage_plan(every, smr, first, window, stream=copier)
            qm.stage_copy(pool, backing, cl, cnt, first, window, err_flags=err, stream=copier)
            ev = torch.cuda.Event()
            ev.record(copier)
            maps.append(sm)
            ready.append(ev)
    with torch.cuda.stream(compute):
        for (L, backing, pool, smr), sm, ev in zip(layers, maps, ready):
            x = torch.from_numpy(L.x.view(np.int16)).cuda().view(torch.bfloat16)
            wr = torch.from_numpy(L.wr.view(np.int16)).cuda().view(torch.bfloat16)
            bias = None if L.bias is None else torch.from_numpy(L.bias).cuda()
            compute.wait_event(ev)
            out, _ = qm.layer(pool, sm, wr, bias, x, k, err_flags=err, path=qm.PATH_GROUPED,
                              stream=compute)
            ident = torch.arange(E, dtype=torch.int32, device="cuda")
            full, _ = qm.layer(backing, ident, wr, bias, x, k, path=qm.PATH_GROUPED,
                               stream=compute)
            outs.append((out, full))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for i, (out, full) in enumerate(outs):
        assert torch.equal(out, full), f"layer {i}"


def _setup_layer(cfg, layer, resident, window):
    """_setup for another layer of the workload (its own experts, input and slot map)."""
    L = synth.make_layer(cfg, layer)
    from parity import margin_fixed_x
    L.x, _ = margin_fixed_x(cfg, layer)
    E = cfg.E
    by_expert = {n: a[L.slot_map] for n, a in L.planes.items()}
    backing = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I, by_expert)
    S = len(resident) + window
    filler = [resident[i] if i < len(resident) else (i * 7 + 3) % E for i in range(S)]
    pool = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I,
                                  {n: a[filler] for n, a in by_expert.items()})
    slot_map = np.full(E, qm.SLOT_MISS, dtype=np.int32)
    slot_map[resident] = np.arange(len(resident), dtype=np.int32)
    return L, backing, pool, slot_map

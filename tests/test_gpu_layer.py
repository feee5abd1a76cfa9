"""GPU parity of the fused layer (moe_layer) against the CPU oracle, through the C ABI.

Small workloads are checked on every token; the full-size prefill workloads are checked
bit-exactly on routing and bucketing for every token, and numerically on a stratified
sample (every token of experts with < 16 tokens, tile-boundary rows, 512 seeded tokens),
in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

import synth
from oracle import codecs, moe as omoe

from parity import (W_ABS, _ulp_bf16, assert_close_rows, check_h, h_slack, make_case,
                    rel_l2_rows, sample_tokens, to_device)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import quantized_routed_expert_gemv_amd as qm  # noqa: E402


def run_layer(cfg, path=qm.PATH_AUTO, layer=0, sample=False):
    L = make_case(cfg, layer)
    k, E, T = cfg.k, cfg.E, cfg.T
    pool, x, wr, bias, sm = to_device(L)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ws = qm.layer(pool, sm, wr, bias, x, k, err_flags=err, path=path)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = {n: t.cpu() for n, t in ws.intermediates().items()}
    out = out.cpu().numpy()

    ids, w, _ = omoe.route(L.x, L.wr, L.bias, k)
    counts, offsets, perm, inv = omoe.bucket(ids, E)
    assert np.array_equal(got["ids"].numpy(), ids)
    assert np.abs(got["w"].numpy() - w).max() <= W_ABS
    for n, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv_perm", inv)):
        assert np.array_equal(got[n].numpy(), ref), n

    toks = sample_tokens(ids, E) if sample else np.arange(T)
    positions = np.sort(inv.reshape(T, k)[toks].ravel())
    hb = got["h"].view(torch.int16).numpy().view(np.uint16)
    _, _, a_ref = omoe.expert_ffn(L.planes, cfg.fmt, L.slot_map, L.x, k, offsets, perm, positions)
    a = a_ref[positions]
    off = np.abs(codecs.bf16_decode(hb[positions]) - a) >= _ulp_bf16(a)
    slack = np.zeros_like(a)
    rows = np.nonzero(off.any(axis=1))[0]
    if rows.size:
        slack[rows] = h_slack(L.planes, cfg.fmt, L.slot_map, L.x, k, offsets, perm,
                              positions[rows], a_ref)
    frac = check_h(hb[positions], a, slack)
    y_gh = omoe.down_proj(L.planes, cfg.fmt, L.slot_map, hb, offsets, positions)
    ry, ey = assert_close_rows(got["y"].numpy()[positions], y_gh[positions], "y")
    out_ref = omoe.combine(y_gh, inv, w, T, k, tokens=toks)
    ro, eo = assert_close_rows(out[toks], out_ref[toks], "out")
    # end to end against the pure oracle (its own h) -- reported, judged on the L2 bound
    y_pure = omoe.down_proj(L.planes, cfg.fmt, L.slot_map,
                            codecs.bf16_bits(codecs.bf16_round(a_ref)), offsets, positions)
    out_pure = omoe.combine(y_pure, inv, w, T, k, tokens=toks)
    rp = rel_l2_rows(out[toks], out_pure[toks]).max()
    print(f"  {cfg.name} T={T}: h mismatch {frac:.2e}; y L2 {ry:.2e} elem {ey:.2e}; "
          f"out L2 {ro:.2e} elem {eo:.2e}; vs pure oracle L2 {rp:.2e}", flush=True)
    assert rp <= 2e-3
    return L, out, got


SMALL = [("tiny", qm.PATH_AUTO), ("tiny", qm.PATH_GEMV), ("gptoss_decode_t1", qm.PATH_AUTO),
         ("gptoss_decode_t4", qm.PATH_AUTO), ("gptoss_decode_t4", qm.PATH_GROUPED),
         ("mixtral_q8_decode", qm.PATH_AUTO), ("qwen_a3b_decode", qm.PATH_AUTO),
         ("tiny_q4k", qm.PATH_AUTO), ("tiny_q4k", qm.PATH_GEMV),
         ("qwen_a3b_q4k_decode", qm.PATH_AUTO), ("mixtral_q4k_decode", qm.PATH_AUTO),
         ("tiny_q5k", qm.PATH_AUTO), ("tiny_q5k", qm.PATH_GEMV),
         ("qwen_a3b_q5k_decode", qm.PATH_AUTO), ("mixtral_q5k_decode", qm.PATH_AUTO),
         ("tiny_q6k", qm.PATH_AUTO), ("tiny_q6k", qm.PATH_GEMV),
         ("qwen_a3b_q6k_decode", qm.PATH_AUTO), ("mixtral_q6k_decode", qm.PATH_AUTO)]


@pytest.mark.parametrize("name,path", SMALL)
def test_layer_parity_small(name, path):
    print(f"layer {name} path={path}", flush=True)
    run_layer(synth.CONFIGS[name], path)


PERSISTENT = [("gptoss_decode_t1", None), ("gptoss_decode_t4", None), ("gptoss_decode_t4", 2),
              ("gptoss_decode_t4", 3), ("qwen_a3b_decode", None), ("mixtral_q8_decode", None),
              ("mixtral_q8_decode", 3), ("qwen_a3b_q4k_decode", None),
              ("mixtral_q5k_decode", None), ("qwen_a3b_q6k_decode", None), ("tiny", 4)]


@pytest.mark.parametrize("name,T", PERSISTENT)
def test_layer_parity_persistent_decode(name, T):
    """The persistent decode layer (routing, gate/up, down and combine in one kernel after
    the router's partials) against the oracle."""
    cfg = synth.config(name) if T is None else synth.config(name, T=T)
    print(f"layer {name} T={cfg.T} persistent", flush=True)
    run_layer(cfg, qm.PATH_PERSISTENT)


def test_layer_persistent_invalid_slot_and_repeat():
    """Persistent path: an out-of-range slot sets bit 0 (bit 1, a timed-out hand-off, must
    stay clear), contributes nothing, and repeated runs on one workspace are bit-identical."""
    cfg = synth.config("gptoss_decode_t4", T=2, H=256, I=512)
    L = make_case(cfg)
    ids, w, _ = omoe.route(L.x, L.wr, L.bias, cfg.k)
    pool, x, wr, bias, sm = to_device(L)
    sm_bad = sm.clone()
    sm_bad[int(ids[0, 0])] = cfg.E + 5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ws = qm.layer(pool, sm_bad, wr, bias, x, cfg.k, err_flags=err, path=qm.PATH_PERSISTENT)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    ref = out.clone()
    for _ in range(3):
        err.zero_()
        o, _ = qm.layer(pool, sm_bad, wr, bias, x, cfg.k, workspace=ws, err_flags=err,
                        path=qm.PATH_PERSISTENT)
        torch.cuda.synchronize()
        assert int(err.item()) == 1 and torch.equal(o, ref)


@pytest.mark.parametrize("T", [2, 3])
def test_layer_parity_decode_two_and_three_tokens(T):
    """Decode with fewer tokens than the 4-token kernel's rows (MXFP4 runs them on MFMA with
    the empty token rows of A zeroed)."""
    print(f"layer gptoss_decode_t4 T={T}", flush=True)
    run_layer(synth.config("gptoss_decode_t4", T=T))


def test_layer_parity_decode_last_of_24_layers():
    print("layer gptoss_decode_t1 layer 23", flush=True)
    run_layer(synth.CONFIGS["gptoss_decode_t1"], layer=23)


@pytest.mark.parametrize("name", ["gptoss_prefill", "qwen_a3b_prefill", "mixtral_q8_prefill",
                                  "qwen_a3b_q4k_prefill", "qwen_a3b_q5k_prefill",
                                  "qwen_a3b_q6k_prefill"])
def test_layer_parity_full_size_prefill(name):
    print(f"layer {name} (full size, sampled)", flush=True)
    run_layer(synth.CONFIGS[name], sample=True)


@pytest.mark.parametrize("T", [2, 17, 130, 257])
def test_layer_ragged_tails(T):
    print(f"layer tiny T={T}", flush=True)
    run_layer(synth.config("tiny", T=T))


def test_layer_dense_and_full_mixture_special_cases():
    for cfg in (synth.Config("dense1", 40, 256, 512, 1, 1, "mxfp4", None, "identity", 21, 1),
                synth.Config("allk", 24, 256, 512, 8, 8, "q8_0", 1.1, "perm", 22, 1),
                synth.Config("q8tiny", 70, 256, 512, 8, 2, "q8_0", None, "perm", 23, 1)):
        print(f"layer {cfg.name}", flush=True)
        run_layer(cfg)


@pytest.mark.parametrize("cfg", [
    # 256 experts: four logits per lane in the top-k; 8 experts chosen
    synth.Config("e256_t1", 1, 256, 512, 256, 8, "mxfp4", 1.2, "perm", 31, 1),
    # 100 and 200 experts: the last of two / four logits per lane only partly used
    synth.Config("e100_t1", 1, 256, 512, 100, 6, "mxfp4", 1.1, "perm", 38, 1),
    synth.Config("e200_t1_q8", 1, 256, 512, 200, 8, "q8_0", None, "perm", 39, 1),
    # 4 tokens x 8 choices = 32 pairs, 64 experts (256 logits): the fused decode limits
    synth.Config("e64_t4_k8", 4, 512, 256, 64, 8, "mxfp4", 1.1, "perm", 32, 1),
    # 3 tokens (a partly used 4-token pass), Q8_0
    synth.Config("q8_t3", 3, 256, 512, 16, 3, "q8_0", None, "perm", 33, 1),
    # 2 tokens sharing experts (8 experts, 6 choices each)
    synth.Config("shared_t2", 2, 256, 256, 8, 6, "mxfp4", None, "perm", 34, 1),
    # past the fused decode's activation limit (H > 4096): split router finished by its own
    # kernel, then the GEMV path; 256 experts, top-8
    synth.Config("h7168_e256_t1", 1, 7168, 512, 256, 8, "mxfp4", 1.2, "perm", 35, 1),
    synth.Config("h6144_t4_q8", 4, 6144, 256, 16, 4, "q8_0", None, "perm", 36, 1),
    synth.Config("h7168_t2_q6k", 2, 7168, 512, 64, 6, "q6_k", None, "perm", 37, 1),
    # one Q8_0 token at the gpt-oss shape: 45 chunks per row, two batches of 6 per wave
    synth.Config("gptoss_q8_t1", 1, 2880, 2880, 32, 4, "q8_0", None, "perm", 40, 1),
    # long MXFP4 down rows on the ticket-combining down kernel: 64 chunks per row, one batch
    # of 16 per wave (one token), and 56 chunks, four batches of 14 (four tokens)
    synth.Config("i8192_t1", 1, 256, 8192, 8, 2, "mxfp4", None, "perm", 41, 1),
    synth.Config("i7168_t4", 4, 256, 7168, 8, 2, "mxfp4", None, "perm", 42, 1),
])
def test_layer_decode_routing_edge_cases(cfg):
    """Shapes at the edges of the decode path that finishes the routing in the gate/up
    kernel (up to 4 tokens, up to 256 (token, expert) logits, up to 32 pairs)."""
    print(f"layer {cfg.name}", flush=True)
    run_layer(cfg)


@pytest.mark.parametrize("E,k,tied", [
    (40, 4, (3, 17, 33)),                  # one key per lane
    (100, 6, (5, 64, 70, 99)),             # two per lane, the second slot partly used
    (200, 8, (1, 66, 130, 197)),           # four per lane, the last slot partly used
    (256, 8, (0, 63, 64, 127, 128, 255)),  # every slot's first and last lane
])
def test_layer_one_token_ties_across_lanes_and_slots(E, k, tied):
    """One token whose top logit is shared by several experts spread over the lanes and
    key slots of the in-kernel top-k: the tied experts come first, lowest index first, and
    the layer's routing equals the stand-alone route's bit for bit."""
    print(f"layer ties E={E} k={k}", flush=True)
    cfg = synth.Config(f"ties_e{E}", 1, 256, 256, E, k, "mxfp4", None, "perm", 41, 1)
    L = synth.make_layer(cfg)
    top = int(np.argmax(omoe.router_logits(L.x, L.wr, None)[0]))
    for e in tied:
        L.wr[e] = L.wr[top]
    ids_ref, w_ref, _ = omoe.route(L.x, L.wr, None, k)
    lg = np.sort(omoe.router_logits(L.x, L.wr, None)[0])[::-1]
    # the tie is exact; every other gap among the top k + 1 keeps the routing margin
    others = np.diff(np.unique(lg[: k + 1]))
    assert len(set(tied) | {top}) <= k and np.all(np.abs(others) > 1e-4)
    assert list(ids_ref[0, : len(set(tied) | {top})]) == sorted(set(tied) | {top})
    pool, x, wr, bias, sm = to_device(L)
    out, ws = qm.layer(pool, sm, wr, None, x, k)
    ids_s, w_s = qm.route(x, wr, None, k)
    torch.cuda.synchronize()
    got = ws.intermediates()
    assert np.array_equal(got["ids"].cpu().numpy(), ids_ref)
    assert torch.equal(got["ids"].cpu(), ids_s.cpu()) and torch.equal(got["w"].cpu(), w_s.cpu())
    assert np.abs(got["w"].cpu().numpy() - w_ref).max() <= W_ABS
    counts, offsets, perm, inv = omoe.bucket(ids_ref, E)
    for n, ref in (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv_perm", inv)):
        assert np.array_equal(got[n].cpu().numpy(), ref), n


@pytest.mark.parametrize("cfg", [
    # the small-batch down + combine kernel is sized by the most pairs one expert can hold
    # (its token count T, rounded up to 1, 2, 4 or 8); these cover each bound partly used
    synth.Config("np8_t6_k1", 6, 256, 512, 8, 1, "mxfp4", 1.1, "perm", 51, 1),
    synth.Config("np8_t8_k1_q8", 8, 256, 256, 4, 1, "q8_0", None, "perm", 52, 1),
    synth.Config("np4_t3_k2", 3, 512, 256, 16, 2, "mxfp4", None, "perm", 53, 1),
    synth.Config("np2_t2_k3_q6k", 2, 256, 512, 6, 3, "q6_k", None, "perm", 54, 1),
])
def test_layer_small_batch_down_pair_bounds(cfg):
    """Layers whose down projection runs the fused small-batch down + combine kernel with
    each of its per-expert pair bounds, against the oracle."""
    print(f"layer {cfg.name}", flush=True)
    run_layer(cfg)


def test_layer_decode_invalid_slot_sets_flag_and_zeroes():
    """A slot outside the pool: the flag is set and that expert adds nothing."""
    cfg = synth.config("gptoss_decode_t4", T=2, H=256, I=512)
    L = make_case(cfg)
    ids, w, _ = omoe.route(L.x, L.wr, L.bias, cfg.k)
    pool, x, wr, bias, sm = to_device(L)
    bad_e = int(ids[0, 0])
    sm_bad = sm.clone()
    sm_bad[bad_e] = cfg.E + 5
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out, ws = qm.layer(pool, sm_bad, wr, bias, x, cfg.k, err_flags=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    im = {n: t.cpu() for n, t in ws.intermediates().items()}
    counts, offsets, perm, inv = omoe.bucket(ids, cfg.E)
    lo, hi = offsets[bad_e], offsets[bad_e + 1]
    assert torch.all(im["h"][lo:hi].float() == 0) and torch.all(im["y"][lo:hi] == 0)
    # every other pair is as in the valid layer, and out is their weighted sum
    ref, ws2 = qm.layer(pool, sm, wr, bias, x, cfg.k)
    torch.cuda.synchronize()
    y_ok = ws2.intermediates()["y"].cpu().numpy()
    keep = np.ones(perm.size, dtype=bool)
    keep[lo:hi] = False
    assert np.array_equal(im["y"].numpy()[keep], y_ok[keep])
    y0 = y_ok.copy()
    y0[~keep] = 0.0
    wg = im["w"].numpy()
    exp = np.zeros((cfg.T, cfg.H), dtype=np.float64)
    for t in range(cfg.T):
        for j in range(cfg.k):
            exp[t] += np.float64(wg[t, j]) * y0[inv[t * cfg.k + j]]
    assert np.allclose(out.cpu().numpy(), exp, rtol=1e-5, atol=1e-5)


def test_layer_empty_input_is_a_no_op():
    cfg = synth.config("tiny", T=0)
    L = synth.make_layer(cfg)
    pool, x, wr, bias, sm = to_device(L)
    out, _ = qm.layer(pool, sm, wr, None, x, cfg.k)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.H)


def test_slot_map_permutation_invariance_bit_exact():
    cfg = synth.CONFIGS["qwen_a3b_decode"]
    cfg = synth.config("qwen_a3b_decode", T=8)
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    rng = np.random.default_rng(7)
    sigma = rng.permutation(cfg.E)
    planes2 = {}
    for n, a in L.planes.items():
        b = np.empty_like(a)
        b[sigma] = a
        planes2[n] = b
    pool2 = qm.Pool.from_canonical(cfg.fmt, cfg.H, cfg.I, planes2)
    sm2 = torch.from_numpy(sigma[L.slot_map].astype(np.int32)).cuda()
    for path in (qm.PATH_GEMV, qm.PATH_GROUPED):
        o1, _ = qm.layer(pool, sm, wr, bias, x, cfg.k, path=path)
        o2, _ = qm.layer(pool2, sm2, wr, bias, x, cfg.k, path=path)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", ["gptoss_decode_t4", "tiny"])
def test_layer_repeat_runs_are_bit_identical(name):
    cfg = synth.CONFIGS[name]
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    ref, ws = qm.layer(pool, sm, wr, bias, x, cfg.k)
    ref = ref.clone()
    for _ in range(3):
        o, _ = qm.layer(pool, sm, wr, bias, x, cfg.k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref)


def test_layer_in_a_hip_graph_matches_eager():
    cfg = synth.CONFIGS["gptoss_decode_t1"]
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    ws = qm.Workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k)
    out = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    eager, _ = qm.layer(pool, sm, wr, bias, x, cfg.k, workspace=ws)
    eager = eager.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        qm.layer(pool, sm, wr, bias, x, cfg.k, out=out, workspace=ws, stream=s)   # warm up
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            qm.layer(pool, sm, wr, bias, x, cfg.k, out=out, workspace=ws, stream=s)
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        # eager work between replays
        o2, _ = qm.layer(pool, sm, wr, bias, x, cfg.k)
        torch.cuda.synchronize()
        assert torch.equal(o2, eager)


def _stages(pool, sm, wr, bias, x, k, path):
    ids, w = qm.route(x, wr, bias, k)
    counts, offsets, perm, inv = qm.bucket(ids, wr.shape[0])
    h, y = qm.expert_ffn(pool, sm, x, k, offsets, perm, path=path)
    return qm.combine(y, inv, w), ids, w, perm, h, y


@pytest.mark.parametrize("name,T,path", [("gptoss_decode_t4", 1, qm.PATH_GEMV),
                                         ("gptoss_decode_t4", 2, qm.PATH_GEMV),
                                         ("gptoss_decode_t4", 3, qm.PATH_GEMV),
                                         ("gptoss_decode_t4", 4, qm.PATH_GEMV),
                                         ("qwen_a3b_decode", 16, qm.PATH_GEMV),
                                         ("mixtral_q8_decode", 3, qm.PATH_GEMV),
                                         ("tiny", 12, qm.PATH_GROUPED),
                                         ("tiny", 64, qm.PATH_AUTO)])
def test_layer_equals_its_stages_bit_exact(name, T, path):
    """The fused call (router finished and bucketed by one kernel) equals the stage calls."""
    cfg = synth.config(name, T=T)
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    ref, ids, w, perm, h, y = _stages(pool, sm, wr, bias, x, cfg.k, path)
    out, ws = qm.layer(pool, sm, wr, bias, x, cfg.k, path=path)
    torch.cuda.synchronize()
    im = ws.intermediates()
    assert torch.equal(im["ids"], ids) and torch.equal(im["w"], w)
    assert torch.equal(im["perm"], perm)
    assert torch.equal(im["h"], h) and torch.equal(im["y"], y)
    assert torch.equal(out, ref)


def test_layer_timed_equals_layer_and_records_events():
    cfg = synth.CONFIGS["gptoss_decode_t1"]
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    ref, ws = qm.layer(pool, sm, wr, bias, x, cfg.k)
    ref = ref.clone()
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    out = torch.empty_like(ref)
    call = qm.LayerCall(pool, sm, wr, bias, x, cfg.k, out, ws, events=ev)
    for _ in range(3):
        call()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert ev[0].elapsed_time(ev[1]) > 0


def test_workspace_reuse_across_batch_sizes():
    """One workspace, sized for the largest T, serves smaller batches in turn."""
    cfg = synth.config("qwen_a3b_decode", T=16)
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    ws = qm.Workspace(16, cfg.H, cfg.I, cfg.E, cfg.k)
    for T in (16, 1, 5, 16, 2):
        fresh, _ = qm.layer(pool, sm, wr, bias, x[:T].contiguous(), cfg.k)
        got, _ = qm.layer(pool, sm, wr, bias, x[:T].contiguous(), cfg.k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, fresh), T

"""GPU parity of each stage against the CPU oracle, through the C ABI.

route: top-k ids bit-exact, gate weights within 1e-5 (inputs have a routing margin).
bucket: counts, offsets, perm, inv_perm bit-exact.
expert FFN: h a faithful bf16 rounding (<= 1% off the oracle's rounding), y within
tolerance of the oracle's down projection at the GPU's h; both schedules (GEMV, grouped).
combine: within tolerance of the oracle's combine of the GPU's y.
"""
import numpy as np
import pytest

import synth
from oracle import moe as omoe

from parity import (W_ABS, assert_close_rows, check_h, h_bits, h_slack, make_case,
                    margin_fixed_x, sample_positions, to_device)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import quantized_routed_expert_gemv_amd as qm  # noqa: E402


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.view(dtype)


# ------------------------------------------------------------------------------- route

ROUTE_CASES = [("tiny", None), ("tiny", 1), ("tiny", 17), ("gptoss_decode_t1", None),
               ("gptoss_decode_t4", None), ("mixtral_q8_decode", None), ("qwen_a3b_decode", None),
               ("qwen_a3b_decode", 16), ("qwen_a3b_decode", 64), ("qwen_a3b_decode", 65),
               ("gptoss_prefill", None), ("mixtral_q8_prefill", None), ("qwen_a3b_prefill", None)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_parity(name, T):
    cfg = synth.CONFIGS[name]
    print(f"route {name} T={T}", flush=True)
    x, redrawn = margin_fixed_x(cfg, 0, T)
    wr, bias = synth.make_router(cfg), synth.make_bias(cfg)
    ids_ref, w_ref, _ = omoe.route(x, wr, bias, cfg.k)
    ids, w = qm.route(_t(x.view(np.int16), torch.bfloat16), _t(wr.view(np.int16), torch.bfloat16),
                      None if bias is None else _t(bias), cfg.k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(ids, ids_ref), f"{np.sum(ids != ids_ref)} ids differ"
    assert np.abs(w - w_ref).max() <= W_ABS
    assert np.abs(w.sum(axis=1) - 1).max() <= 1e-6


def test_route_ties_go_to_lower_index():
    # identical router rows make exactly tied logits
    cfg = synth.config("tiny", T=32)
    x = synth.make_x(cfg)
    wr = synth.make_router(cfg)
    wr[5] = wr[2]
    wr[7] = wr[2]
    ids_ref, w_ref, _ = omoe.route(x, wr, None, 3)
    ids, w = qm.route(_t(x.view(np.int16), torch.bfloat16), _t(wr.view(np.int16), torch.bfloat16),
                      None, 3)
    ids = ids.cpu().numpy()
    # tokens whose top-3 holds a tied pair: the order is (2, 5, 7) in that order
    for t in range(cfg.T):
        row = list(ids[t])
        tied = [e for e in row if e in (2, 5, 7)]
        assert tied == sorted(tied)
    np.testing.assert_array_equal(np.sort(ids, axis=1), np.sort(ids_ref, axis=1))


# ------------------------------------------------------------------------------ bucket

@pytest.mark.parametrize("T,k,E,seed", [(1, 4, 32, 0), (4, 4, 32, 1), (64, 2, 8, 2), (1, 8, 128, 3),
                                        (1024, 4, 32, 4), (1025, 4, 32, 5), (16384, 4, 32, 6),
                                        (8192, 8, 128, 7), (4096, 2, 8, 8), (3000, 8, 256, 9),
                                        (5, 1, 1, 10), (7, 8, 8, 11)])
def test_bucket_parity(T, k, E, seed):
    print(f"bucket T={T} k={k} E={E}", flush=True)
    rng = np.random.default_rng(seed)
    # Zipf-skewed choices (some experts empty, one huge) plus the uniform case
    p = 1.0 / np.arange(1, E + 1) ** (1.3 if seed % 2 else 0.0)
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    ref = omoe.bucket(ids, E)
    got = qm.bucket(_t(ids), E)
    for name, a, b in zip(("counts", "offsets", "perm", "inv_perm"), got, ref):
        assert np.array_equal(a.cpu().numpy(), b), name


def test_bucket_empty():
    counts, offsets, perm, inv = qm.bucket(torch.zeros((0, 2), dtype=torch.int32, device="cuda"), 8)
    assert counts.cpu().numpy().tolist() == [0] * 8
    assert offsets.cpu().numpy().tolist() == [0] * 9


def test_bucket_is_deterministic():
    rng = np.random.default_rng(1)
    ids = np.stack([rng.permutation(128)[:8] for _ in range(8192)]).astype(np.int32)
    a = [t.cpu().numpy() for t in qm.bucket(_t(ids), 128)]
    for _ in range(3):
        b = [t.cpu().numpy() for t in qm.bucket(_t(ids), 128)]
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


# --------------------------------------------------------------------------- expert FFN

FFN_CASES = [
    ("tiny", 1, qm.PATH_GEMV), ("tiny", 3, qm.PATH_GEMV), ("tiny", 16, qm.PATH_GEMV),
    ("tiny", 64, qm.PATH_GEMV), ("tiny", 64, qm.PATH_GROUPED), ("tiny", 3, qm.PATH_GROUPED),
    ("tiny", 300, qm.PATH_GROUPED),
    ("gptoss_decode_t1", None, qm.PATH_GEMV), ("gptoss_decode_t4", None, qm.PATH_GEMV),
    ("gptoss_decode_t4", None, qm.PATH_GROUPED),
    ("qwen_a3b_decode", None, qm.PATH_GEMV), ("qwen_a3b_decode", 40, qm.PATH_GROUPED),
    ("mixtral_q8_decode", None, qm.PATH_GEMV), ("mixtral_q8_decode", 3, qm.PATH_GEMV),
    ("mixtral_q8_decode", 24, qm.PATH_GROUPED),
    # Q4_K: GEMV (1, 3 and 16 tokens), grouped GEMM, ragged expert sizes
    ("tiny_q4k", 1, qm.PATH_GEMV), ("tiny_q4k", 3, qm.PATH_GEMV), ("tiny_q4k", 16, qm.PATH_GEMV),
    ("tiny_q4k", 64, qm.PATH_GROUPED), ("tiny_q4k", 300, qm.PATH_GROUPED),
    ("qwen_a3b_q4k_decode", None, qm.PATH_GEMV), ("qwen_a3b_q4k_decode", 40, qm.PATH_GROUPED),
    ("mixtral_q4k_decode", None, qm.PATH_GEMV), ("mixtral_q4k_decode", 24, qm.PATH_GROUPED),
    # Q5_K: the same paths
    ("tiny_q5k", 1, qm.PATH_GEMV), ("tiny_q5k", 3, qm.PATH_GEMV), ("tiny_q5k", 16, qm.PATH_GEMV),
    ("tiny_q5k", 64, qm.PATH_GROUPED), ("tiny_q5k", 300, qm.PATH_GROUPED),
    ("qwen_a3b_q5k_decode", None, qm.PATH_GEMV), ("qwen_a3b_q5k_decode", 40, qm.PATH_GROUPED),
    ("mixtral_q5k_decode", None, qm.PATH_GEMV), ("mixtral_q5k_decode", 24, qm.PATH_GROUPED),
    # Q6_K: the same paths
    ("tiny_q6k", 1, qm.PATH_GEMV), ("tiny_q6k", 3, qm.PATH_GEMV), ("tiny_q6k", 16, qm.PATH_GEMV),
    ("tiny_q6k", 64, qm.PATH_GROUPED), ("tiny_q6k", 300, qm.PATH_GROUPED),
    ("qwen_a3b_q6k_decode", None, qm.PATH_GEMV), ("qwen_a3b_q6k_decode", 40, qm.PATH_GROUPED),
    ("mixtral_q6k_decode", None, qm.PATH_GEMV), ("mixtral_q6k_decode", 24, qm.PATH_GROUPED),
]


def run_ffn_case(cfg, T, path, n_sample=None):
    L = make_case(cfg, 0, T)
    k = cfg.k
    ids, _, _ = omoe.route(L.x, L.wr, L.bias, k)
    counts, offsets, perm, inv = omoe.bucket(ids, cfg.E)
    pool, x, wr, bias, sm = to_device(L)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    h, y = qm.expert_ffn(pool, sm, x, k, _t(offsets), _t(perm), err_flags=err, path=path)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    hb, yg = h_bits(h), y.cpu().numpy()
    positions = (np.arange(perm.size) if n_sample is None
                 else sample_positions(offsets, n_uniform=n_sample))
    h_ref, _, a_ref = omoe.expert_ffn(L.planes, cfg.fmt, L.slot_map, L.x, k, offsets, perm,
                                      positions)
    a = a_ref[positions]
    # the slack is only needed where the plain faithful test fails; compute it there
    from parity import _ulp_bf16
    from oracle import codecs
    off = np.abs(codecs.bf16_decode(hb[positions]) - a) >= _ulp_bf16(a)
    slack = np.zeros_like(a)
    rows = np.nonzero(off.any(axis=1))[0]
    if rows.size:
        slack[rows] = h_slack(L.planes, cfg.fmt, L.slot_map, L.x, k, offsets, perm,
                              positions[rows], a_ref)
    frac = check_h(hb[positions], a, slack)
    y_at_gpu_h = omoe.down_proj(L.planes, cfg.fmt, L.slot_map, hb, offsets, positions)
    r, e = assert_close_rows(yg[positions], y_at_gpu_h[positions], "y")
    print(f"  h mismatch {frac:.2e}, y rel L2 {r:.2e}, elem {e:.2e}", flush=True)
    return L, ids, offsets, perm, inv, hb, yg


@pytest.mark.parametrize("name,T,path", FFN_CASES)
def test_expert_ffn_parity(name, T, path):
    cfg = synth.config(name) if T is None else synth.config(name, T=T)
    print(f"ffn {name} T={cfg.T} path={path}", flush=True)
    run_ffn_case(cfg, None, path)


def test_expert_ffn_invalid_slot_sets_flag_and_zeroes():
    cfg = synth.config("tiny", T=16)
    L = make_case(cfg)
    ids, _, _ = omoe.route(L.x, L.wr, None, cfg.k)
    counts, offsets, perm, inv = omoe.bucket(ids, cfg.E)
    pool, x, wr, bias, sm = to_device(L)
    bad_e = int(np.argmax(counts))
    sm_bad = sm.clone()
    sm_bad[bad_e] = cfg.E + 3          # outside the pool
    for path in (qm.PATH_GEMV, qm.PATH_GROUPED):
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        h, y = qm.expert_ffn(pool, sm_bad, x, cfg.k, _t(offsets), _t(perm), err_flags=err, path=path)
        torch.cuda.synchronize()
        assert int(err.item()) & 1
        lo, hi = offsets[bad_e], offsets[bad_e + 1]
        assert torch.all(y[lo:hi] == 0) and torch.all(h[lo:hi].float() == 0)
        # other experts unaffected
        h2, y2 = qm.expert_ffn(pool, sm, x, cfg.k, _t(offsets), _t(perm), path=path)
        keep = np.ones(perm.size, dtype=bool)
        keep[lo:hi] = False
        assert torch.equal(y[keep], y2[keep])


# ----------------------------------------------------------------------------- combine

@pytest.mark.parametrize("T,k,H", [(1, 4, 2880), (64, 2, 256), (1000, 8, 2048), (3, 1, 32),
                                   (70000, 2, 32)])   # more tokens than a launch's grid.y
def test_combine_parity(T, k, H):
    rng = np.random.default_rng(T)
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    inv = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    ref = omoe.combine(y.astype(np.float64), inv, w.astype(np.float64), T, k)
    out = qm.combine(_t(y), _t(inv), _t(w)).cpu().numpy()
    assert_close_rows(out, ref, "out")
    # summed in j order in fp32: equal to a sequential fp32 evaluation
    seq = np.zeros((T, H), dtype=np.float32)
    for j in range(k):
        seq = (w[:, j:j + 1] * y[inv.reshape(T, k)[:, j]] + seq).astype(np.float32)
    np.testing.assert_allclose(out, seq, rtol=1e-6, atol=1e-6)


def test_expert_ffn_grouped_past_2e32_h_elements():
    """The grouped GEMM's gathered rows past 2^32 elements of h: Q8_0 experts of the
    Mixtral shape's I = 14336 with H = 256 and 150,016 tokens x top-2 = 300,032 pairs, so
    bucket positions from 299,594 on start past element 2^32 of h. Checked on sampled
    positions, among them the last 64, through a compacted oracle bucketing (the oracle
    of the sampled pairs only)."""
    cfg = synth.config("mixtral_q8_prefill", T=150016, H=256)
    k = cfg.k
    print(f"ffn past 2^32 h elements: T={cfg.T} H={cfg.H} I={cfg.I} pairs={cfg.T * k}",
          flush=True)
    L = make_case(cfg)
    ids, _, _ = omoe.route(L.x, L.wr, None, k)
    counts, offsets, perm, inv = omoe.bucket(ids, cfg.E)
    n = perm.size
    first_wrap = (1 << 32) // cfg.I + 1
    assert n > first_wrap + 64
    pool, x, wr, bias, sm = to_device(L)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    h, y = qm.expert_ffn(pool, sm, x, k, _t(offsets), _t(perm), err_flags=err,
                         path=qm.PATH_GROUPED)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    positions = np.union1d(sample_positions(offsets, n_uniform=96),
                           np.r_[np.arange(n - 64, n), first_wrap - 2, first_wrap - 1,
                                 first_wrap, first_wrap + 1]).astype(np.int64)
    pt = torch.from_numpy(positions).cuda()
    hb = h_bits(h[pt])
    yg = y[pt].cpu().numpy()
    del h, y
    # the sampled pairs as a bucketing of their own: same experts, same tokens, in order
    perm_s = perm[positions].astype(np.int32)
    exp_of_pos = np.searchsorted(offsets, positions, side="right") - 1
    off_s = np.zeros(cfg.E + 1, dtype=np.int64)
    off_s[1:] = np.cumsum(np.bincount(exp_of_pos, minlength=cfg.E))
    h_ref, _, a_ref = omoe.expert_ffn(L.planes, cfg.fmt, L.slot_map, L.x, k, off_s, perm_s)
    from parity import _ulp_bf16
    from oracle import codecs
    off = np.abs(codecs.bf16_decode(hb) - a_ref) >= _ulp_bf16(a_ref)
    slack = np.zeros_like(a_ref)
    rows = np.nonzero(off.any(axis=1))[0]
    if rows.size:
        slack[rows] = h_slack(L.planes, cfg.fmt, L.slot_map, L.x, k, off_s, perm_s, rows,
                              a_ref)
    frac = check_h(hb, a_ref, slack)
    y_at_gpu_h = omoe.down_proj(L.planes, cfg.fmt, L.slot_map, hb, off_s)
    r, e = assert_close_rows(yg, y_at_gpu_h, "y")
    print(f"  {positions.size} positions, h mismatch {frac:.2e}, y rel L2 {r:.2e}, elem {e:.2e}",
          flush=True)

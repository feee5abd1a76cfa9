"""moe_layer_noalloc (the fused layer on the library's static device workspace) against
moe_layer with a caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, each equal to moe_layer's output bit for bit (the same kernels run on the
same inputs), plus the size limit."""
import numpy as np
import pytest

import synth

from parity import make_case, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)
import quantized_routed_expert_gemv_amd as qm  # noqa: E402


def _pair(cfg, path):
    L = make_case(cfg)
    pool, x, wr, bias, sm = to_device(L)
    err_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    err_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref, _ = qm.layer(pool, sm, wr, bias, x, cfg.k, err_flags=err_a, path=path)
    # poison the output so a call that writes nothing cannot pass
    out = torch.full_like(ref, float("nan"))
    got = qm.layer_noalloc(pool, sm, wr, bias, x, cfg.k, out=out, err_flags=err_b, path=path)
    torch.cuda.synchronize()
    assert int(err_a.item()) == 0 and int(err_b.item()) == 0
    return ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("big,small,path", [
    (("gptoss_decode_t4", 4), ("gptoss_decode_t1", 1), qm.PATH_AUTO),
    (("qwen_a3b_decode", 16), ("qwen_a3b_decode", 1), qm.PATH_AUTO),
    (("tiny", 300), ("tiny", 17), qm.PATH_GROUPED),
    (("mixtral_q8_decode", 3), ("mixtral_q8_decode", 1), qm.PATH_GEMV),
])
def test_noalloc_matches_layer_twice(big, small, path):
    for name, T in (big, small):
        cfg = synth.config(name, T=T)
        print(f"noalloc {name} T={T} path={path}", flush=True)
        ref, got = _pair(cfg, path)
        assert np.array_equal(ref, got), (
            f"{name} T={T}: {int(np.sum(ref != got))} outputs differ from moe_layer")


def test_noalloc_refuses_oversized_layer():
    cfg = synth.config("gptoss_prefill", T=4096)
    need = qm.layer_workspace(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k).total
    assert need > qm.NOALLOC_WS_BYTES
    pool = qm.Pool.empty(cfg.fmt, cfg.E, cfg.H, cfg.I)
    x = torch.zeros((cfg.T, cfg.H), dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros((cfg.E, cfg.H), dtype=torch.bfloat16, device="cuda")
    sm = torch.arange(cfg.E, dtype=torch.int32, device="cuda")
    with pytest.raises(qm.MoeError, match="static workspace"):
        qm.layer_noalloc(pool, sm, wr, None, x, cfg.k)

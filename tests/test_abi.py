"""The C-ABI library loads, exports every entry point include/moe.h declares, and rejects
bad arguments on the host before anything reaches the GPU (CPU only: no call here
launches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_routed_expert_gemv_amd", "libmoe.so")
HDR = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2


def _declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_layer_calls():
    names = _declared()
    for n in ("moe_route", "moe_bucket", "moe_expert_ffn", "moe_combine", "moe_layer",
              "moe_pool_pack", "moe_layer_workspace"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"


def test_binding_covers_every_declared_symbol():
    pytest.importorskip("torch")
    import quantized_routed_expert_gemv_amd as qm
    assert sorted(qm.EXPORTED) == _declared()


class Pool(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32)] + [(n, ctypes.c_void_p) for n in
                                          ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")]


class Ws(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("total", "topk_ids", "topk_w", "counts", "offsets",
                                               "perm", "inv_perm", "h", "y", "scratch", "act",
                                               "sync")]


def _setup(lib):
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_plane_bytes.restype = ctypes.c_size_t
    lib.moe_route_scratch_bytes.restype = ctypes.c_size_t
    lib.moe_bucket_scratch_bytes.restype = ctypes.c_size_t
    return lib


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced by the checks below
MISALIGNED = ctypes.c_void_p(0x10004)


def test_status_strings(lib):
    _setup(lib)
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(1) == b"MOE_ERR_INVALID_ARG"
    assert lib.moe_status_string(3) == b"MOE_ERR_HIP"


def test_plane_bytes(lib):
    _setup(lib)
    # MXFP4: 16 code bytes + 1 scale byte per 32 weights; Q8_0: 32 + 2
    assert lib.moe_plane_bytes(1, 2880, 2880, 0) == 2880 * 2880 // 2
    assert lib.moe_plane_bytes(1, 2880, 2880, 1) == 2880 * 90
    assert lib.moe_plane_bytes(2, 14336, 4096, 0) == 14336 * 4096
    assert lib.moe_plane_bytes(2, 14336, 4096, 1) == 14336 * 128 * 2
    assert lib.moe_plane_bytes(7, 16, 32, 0) == 0
    # Q4_K: 16 code bytes per block; 2 scale bytes per block + 4 per 256-element super-block
    assert lib.moe_plane_bytes(3, 768, 2048, 0) == 768 * 2048 // 2
    assert lib.moe_plane_bytes(3, 768, 2048, 1) == 768 * (64 * 2 + 8 * 4)
    assert lib.moe_plane_bytes(3, 768, 2080, 1) == 0                    # K % 256
    # Q5_K: Q4_K's planes plus 4 bytes of high bits per block in the code plane
    assert lib.moe_plane_bytes(4, 768, 2048, 0) == 768 * 64 * (16 + 4)
    assert lib.moe_plane_bytes(4, 768, 2048, 1) == 768 * (64 * 2 + 8 * 4)
    # Q6_K: 8 bytes of 2-bit high parts per block; d in a 4-byte record per super-block
    assert lib.moe_plane_bytes(5, 768, 2048, 0) == 768 * 64 * (16 + 8)
    assert lib.moe_plane_bytes(5, 768, 2048, 1) == 768 * (64 * 2 + 8 * 4)


def test_route_argument_checks(lib):
    _setup(lib)
    f = lib.moe_route
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 3 + \
                 [ctypes.c_size_t, ctypes.c_void_p]
    # k > E, k > 8, H not a multiple of 32, E > 256, T < 0
    for T, H, E, k in ((1, 64, 4, 5), (1, 64, 16, 9), (1, 48, 8, 2), (1, 64, 300, 2),
                       (-1, 64, 8, 2), (1, 64, 8, 0)):
        assert f(FAKE, FAKE, None, T, H, E, k, FAKE, FAKE, None, 0, None) == INVALID
        assert lib.moe_last_error()
    # NULL / misaligned activations
    assert f(None, FAKE, None, 4, 64, 8, 2, FAKE, FAKE, None, 0, None) == INVALID
    assert b"x" in lib.moe_last_error()
    assert f(MISALIGNED, FAKE, None, 4, 64, 8, 2, FAKE, FAKE, None, 0, None) == INVALID
    # T = 0: nothing to do
    assert f(None, None, None, 0, 64, 8, 2, None, None, None, 0, None) == OK
    # up to 4 tokens: the reduction is split into min(32, H/64) slices whose partial
    # logits [slices][T][E] fp32 live in the scratch
    assert lib.moe_route_scratch_bytes(1, 2880, 32) == 32 * 1 * 32 * 4
    assert lib.moe_route_scratch_bytes(4, 256, 8) == 4 * 4 * 8 * 4
    # 5..16 tokens with E <= 128 are routed by one workgroup: no scratch
    assert lib.moe_route_scratch_bytes(8, 2880, 32) == 0
    # with more experts the reduction is split across workgroups: scratch required
    need = lib.moe_route_scratch_bytes(1, 2880, 256)
    assert need > 0
    assert f(FAKE, FAKE, None, 1, 2880, 256, 4, FAKE, FAKE, None, 0, None) == INVALID
    assert f(FAKE, FAKE, None, 1, 2880, 256, 4, FAKE, FAKE, FAKE, need - 1, None) == INVALID


def test_bucket_argument_checks(lib):
    _setup(lib)
    f = lib.moe_bucket
    f.argtypes = [ctypes.c_void_p] + [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5 + \
                 [ctypes.c_size_t, ctypes.c_void_p]
    assert f(FAKE, 4, 9, 16, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    assert f(FAKE, 4, 2, 8, None, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    need = lib.moe_bucket_scratch_bytes(16384, 4, 32)
    assert need > 0 and lib.moe_bucket_scratch_bytes(1, 4, 32) == 0
    assert f(FAKE, 16384, 4, 32, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID


def _pool(fmt=1, n_slots=4, H=64, I=32):
    p = Pool(fmt, n_slots, H, I, *([0x10000] * 6))
    return p


def test_ffn_and_layer_argument_checks(lib):
    _setup(lib)
    f = lib.moe_expert_ffn
    f.argtypes = [ctypes.POINTER(Pool), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 5 + [ctypes.c_int32,
                                                                             ctypes.c_void_p]
    p = _pool()
    p.fmt = 9
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == UNSUPPORTED
    p = _pool(I=40)
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    p = _pool(fmt=3, H=256, I=32)                  # Q4_K needs I % 256 == 0 too
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    p = _pool(n_slots=0)
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    p = _pool()
    p.down_s = None
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID
    p = _pool()
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 7, None) == INVALID
    assert f(ctypes.byref(p), FAKE, 4, FAKE, 2, 2, FAKE, FAKE, None, FAKE, None, 0, None) == INVALID
    assert f(None, FAKE, 4, FAKE, 2, 2, FAKE, FAKE, FAKE, FAKE, None, 0, None) == INVALID

    g = lib.moe_layer
    g.argtypes = [ctypes.POINTER(Pool)] + [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 3 + \
                 [ctypes.c_void_p] * 2 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p]
    ws = Ws()
    lib.moe_layer_workspace.argtypes = [ctypes.c_int32] * 5 + [ctypes.POINTER(Ws)]
    assert lib.moe_layer_workspace(3, 64, 32, 4, 2, ctypes.byref(ws)) == OK
    assert ws.total >= 3 * 2 * (32 * 2 + 64 * 4)
    for name in ("topk_ids", "topk_w", "counts", "offsets", "perm", "inv_perm", "h", "y", "scratch",
                 "act", "sync"):
        assert getattr(ws, name) % 256 == 0
    # workspace too small
    assert g(ctypes.byref(p), FAKE, FAKE, None, FAKE, 3, 4, 2, FAKE, FAKE, ws.total - 1, None, 0,
             None) == INVALID
    # workspace misaligned (needs 256)
    assert g(ctypes.byref(p), FAKE, FAKE, None, FAKE, 3, 4, 2, FAKE, ctypes.c_void_p(0x10010),
             ws.total, None, 0, None) == INVALID
    # T = 0 is a no-op
    assert g(ctypes.byref(p), None, None, None, None, 0, 4, 2, None, None, 0, None, 0, None) == OK


def test_miss_argument_checks(lib):
    _setup(lib)
    f = lib.moe_miss_list
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 4
    # E > 256, k > E, k > 8, T < 0
    for T, E, k in ((4, 300, 2), (4, 4, 5), (4, 16, 9), (-1, 8, 2)):
        assert f(FAKE, E, FAKE, FAKE, T, k, FAKE, FAKE, FAKE, None) == INVALID
    # NULL or misaligned outputs and inputs
    assert f(FAKE, 8, FAKE, FAKE, 4, 2, FAKE, None, FAKE, None) == INVALID
    assert b"miss_of_pair" in lib.moe_last_error()
    assert f(FAKE, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, None, None) == INVALID
    assert f(MISALIGNED, 8, FAKE, FAKE, 4, 2, FAKE, FAKE, FAKE, None) == INVALID
    g = lib.moe_merge_misses
    g.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 3 + [ctypes.c_void_p]
    # H not a multiple of 32, k outside [1, 8]
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 2, 48, None) == INVALID
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 9, 64, None) == INVALID
    assert g(FAKE, None, FAKE, FAKE, 4, 2, 64, None) == INVALID
    assert b"y_miss" in lib.moe_last_error()
    # T = 0: nothing to do
    assert g(None, None, None, None, 0, 2, 64, None) == OK


def test_stage_argument_checks(lib):
    _setup(lib)
    f = lib.moe_stage_plan
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ctypes.c_int32] * 3 + \
                 [ctypes.c_void_p] * 4
    assert f(FAKE, FAKE, 300, 0, 4, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 8, -1, 4, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 8, 0, -2, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 8, 0, 4, FAKE, FAKE, None, None) == INVALID
    assert b"counters" in lib.moe_last_error()
    g = lib.moe_stage_copy
    g.argtypes = [ctypes.POINTER(Pool)] * 2 + [ctypes.c_void_p] * 2 + [ctypes.c_int32] * 2 + \
                 [ctypes.c_void_p] * 2
    pool, back = _pool(n_slots=8), _pool(n_slots=4)
    # the window must fit in the pool
    assert g(ctypes.byref(pool), ctypes.byref(back), FAKE, FAKE, 6, 3, None, None) == INVALID
    assert g(ctypes.byref(pool), ctypes.byref(back), FAKE, FAKE, -1, 2, None, None) == INVALID
    # backing store of another format or shape
    other = _pool(fmt=2, n_slots=4)
    assert g(ctypes.byref(pool), ctypes.byref(other), FAKE, FAKE, 4, 4, None, None) == INVALID
    other = _pool(n_slots=4, I=64)
    assert g(ctypes.byref(pool), ctypes.byref(other), FAKE, FAKE, 4, 4, None, None) == INVALID
    assert g(ctypes.byref(pool), ctypes.byref(back), None, FAKE, 4, 4, None, None) == INVALID
    # an empty window enqueues nothing
    assert g(ctypes.byref(pool), ctypes.byref(back), None, None, 4, 0, None, None) == OK


def test_pack_argument_checks(lib):
    _setup(lib)
    f = lib.moe_pool_pack
    f.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 5
    assert f(1, 1, 24, 64, FAKE, FAKE, FAKE, FAKE, None) == INVALID     # rows % 16
    assert f(1, 1, 32, 48, FAKE, FAKE, FAKE, FAKE, None) == INVALID     # K % 32
    assert f(9, 1, 32, 64, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    assert f(3, 1, 32, 64, FAKE, FAKE, FAKE, FAKE, None) == INVALID     # Q4_K: K % 256
    assert f(2, 1, 32, 64, FAKE, ctypes.c_void_p(0x10001), FAKE, FAKE, None) == INVALID
    assert f(1, 0, 32, 64, None, None, None, None, None) == OK


def test_workspace_layout_struct_matches_library(lib):
    """moe_layer_workspace writes exactly len(Ws._fields_) size_t values (no more)."""
    SENT = 0xDEADBEEFCAFE
    buf = (ctypes.c_size_t * 32)(*([SENT] * 32))
    lib.moe_layer_workspace.argtypes = [ctypes.c_int32] * 5 + [ctypes.c_void_p]
    assert lib.moe_layer_workspace(3, 64, 32, 4, 2, ctypes.cast(buf, ctypes.c_void_p)) == OK
    n = len(Ws._fields_)
    assert all(buf[i] != SENT for i in range(n))
    assert all(buf[i] == SENT for i in range(n, 32))
    pytest.importorskip("torch")
    import quantized_routed_expert_gemv_amd as qm
    assert [f[0] for f in qm.WsLayout._fields_] == [f[0] for f in Ws._fields_]



def test_activation_extent_limit(lib):
    """x [T x H] and h [T*k x I] must each hold fewer than 2^35 elements (the grouped GEMM
    addresses gathered rows as 32-bit indices of 16-byte units); past that the layer, the
    expert FFN and the workspace query refuse on the host."""
    _setup(lib)
    ws = Ws()
    lib.moe_layer_workspace.argtypes = [ctypes.c_int32] * 5 + [ctypes.POINTER(Ws)]
    # h: T*k*I = 2^35 exactly (T = 2^20, k = 2, I = 2^14) is refused; one token less fits
    assert lib.moe_layer_workspace(1 << 20, 256, 1 << 14, 8, 2, ctypes.byref(ws)) == INVALID
    assert b"T*k*I" in lib.moe_last_error()
    assert lib.moe_layer_workspace((1 << 20) - 1, 256, 1 << 14, 8, 2, ctypes.byref(ws)) == OK
    # x: T*H = 2^35 (T = 2^23, H = 4096), with h small enough (I = 32, k = 1)
    assert lib.moe_layer_workspace(1 << 23, 4096, 32, 8, 1, ctypes.byref(ws)) == INVALID
    assert b"T*H" in lib.moe_last_error()
    f = lib.moe_expert_ffn
    f.argtypes = [ctypes.POINTER(Pool), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 5 + [ctypes.c_int32,
                                                                             ctypes.c_void_p]
    p = _pool(fmt=2, n_slots=8, H=256, I=1 << 14)
    assert f(ctypes.byref(p), FAKE, 8, FAKE, 1 << 20, 2, FAKE, FAKE, FAKE, FAKE, None, 0,
             None) == INVALID
    g = lib.moe_layer
    g.argtypes = [ctypes.POINTER(Pool)] + [ctypes.c_void_p] * 4 + [ctypes.c_int32] * 3 + \
                 [ctypes.c_void_p] * 2 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                          ctypes.c_void_p]
    assert g(ctypes.byref(p), FAKE, FAKE, None, FAKE, 1 << 20, 8, 2, FAKE, FAKE, 1 << 62, None,
             0, None) == INVALID
    assert b"T*k*I" in lib.moe_last_error()

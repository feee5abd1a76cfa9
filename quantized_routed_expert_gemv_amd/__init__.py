"""Python binding of libmoe.so, the routed MoE FFN layer for MI355X (gfx950).

Argument marshalling only: every function takes torch tensors (device memory and
streams come from PyTorch), checks dtypes and shapes, and calls the same-named C entry
point declared in include/moe.h. All arithmetic runs in the library's HIP kernels; there
is no fallback. If the library has not been built, importing this package raises.

    import quantized_routed_expert_gemv_amd as moe
    pool = moe.Pool.from_canonical("mxfp4", H, I, planes)   # planes indexed by slot
    out = moe.layer(pool, slot_map, w_router, bias, x, k)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MXFP4, Q8_0, Q4_K, Q5_K, Q6_K = 1, 2, 3, 4, 5
PATH_AUTO, PATH_GEMV, PATH_GROUPED, PATH_PERSISTENT = 0, 1, 2, 3
SLOT_MISS = -1      # slot_map value of an expert that is not in the pool (MOE_SLOT_MISS)
_FMT = {"mxfp4": MXFP4, "q8_0": Q8_0, "q4_k": Q4_K, "q5_k": Q5_K, "q6_k": Q6_K}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python quantized_routed_expert_gemv_amd/build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t


class PoolStruct(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("n_slots", _i32), ("H", _i32), ("I", _i32),
                ("gate_q", _p), ("gate_s", _p), ("up_q", _p), ("up_s", _p),
                ("down_q", _p), ("down_s", _p)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, _sz) for n in ("total", "topk_ids", "topk_w", "counts", "offsets", "perm",
                                   "inv_perm", "h", "y", "scratch", "act", "sync")]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_plane_bytes = _sig("moe_plane_bytes", _sz, _i32, _i32, _i32, _i32)
_pool_pack = _sig("moe_pool_pack", _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _p, _p)
_route_scratch = _sig("moe_route_scratch_bytes", _sz, _i32, _i32, _i32)
_route = _sig("moe_route", _i32, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _p, _p, _sz, _p)
_bucket_scratch = _sig("moe_bucket_scratch_bytes", _sz, _i32, _i32, _i32)
_bucket = _sig("moe_bucket", _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p, _p, _sz, _p)
_ffn = _sig("moe_expert_ffn", _i32, ctypes.POINTER(PoolStruct), _p, _i32, _p, _i32, _i32, _p,
            _p, _p, _p, _p, _i32, _p)
_gate_up = _sig("moe_expert_gate_up", _i32, ctypes.POINTER(PoolStruct), _p, _i32, _p, _i32,
                _i32, _p, _p, _p, _p, _i32, _p)
_down = _sig("moe_expert_down", _i32, ctypes.POINTER(PoolStruct), _p, _i32, _i32, _i32, _p, _p,
             _p, _p, _i32, _p)
_combine = _sig("moe_combine", _i32, _p, _p, _p, _i32, _i32, _i32, _p, _p)
_miss_list = _sig("moe_miss_list", _i32, _p, _i32, _p, _p, _i32, _i32, _p, _p, _p, _p)
_merge_misses = _sig("moe_merge_misses", _i32, _p, _p, _p, _p, _i32, _i32, _i32, _p)
_stage_plan = _sig("moe_stage_plan", _i32, _p, _p, _i32, _i32, _i32, _p, _p, _p, _p)
_stage_copy = _sig("moe_stage_copy", _i32, ctypes.POINTER(PoolStruct), ctypes.POINTER(PoolStruct),
                   _p, _p, _i32, _i32, _p, _p)
_ws = _sig("moe_layer_workspace", _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(WsLayout))
_layer = _sig("moe_layer", _i32, ctypes.POINTER(PoolStruct), _p, _p, _p, _p, _i32, _i32, _i32,
              _p, _p, _sz, _p, _i32, _p)
_layer_timed = _sig("moe_layer_timed", _i32, ctypes.POINTER(PoolStruct), _p, _p, _p, _p, _i32,
                    _i32, _i32, _p, _p, _sz, _p, _i32, _p, _p, _p)
_layer_noalloc = _sig("moe_layer_noalloc", _i32, ctypes.POINTER(PoolStruct), _p, _p, _p, _p,
                      _i32, _i32, _i32, _p, _p, _i32, _p)
_status_string = _sig("moe_status_string", ctypes.c_char_p, _i32)
_last_error = _sig("moe_last_error", ctypes.c_char_p)

EXPORTED = ("moe_plane_bytes", "moe_pool_pack", "moe_route_scratch_bytes", "moe_route",
            "moe_bucket_scratch_bytes", "moe_bucket", "moe_expert_ffn", "moe_expert_gate_up",
            "moe_expert_down", "moe_combine", "moe_miss_list", "moe_merge_misses",
            "moe_stage_plan", "moe_stage_copy",
            "moe_layer_workspace", "moe_layer", "moe_layer_timed", "moe_layer_noalloc",
            "moe_status_string", "moe_last_error")

NOALLOC_WS_BYTES = 32 << 20   # MOE_NOALLOC_WS_BYTES


def _check(status: int):
    if status != 0:
        raise MoeError(status, f"{_status_string(status).decode()}: {_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: must be a contiguous device tensor")


# ---------------------------------------------------------------------------- pool


def plane_bytes(fmt: str, rows: int, K: int, scales: bool) -> int:
    return _plane_bytes(_FMT[fmt], rows, K, int(scales))


class Pool:
    """Resident expert pool in the library's tiled layout (six device byte tensors)."""

    def __init__(self, fmt: str, n_slots: int, H: int, I: int, planes: dict):
        self.fmt, self.n_slots, self.H, self.I = fmt, n_slots, H, I
        self.planes = planes
        self.struct = PoolStruct(_FMT[fmt], n_slots, H, I,
                                 *[planes[n].data_ptr() for n in
                                   ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s")])

    @classmethod
    def empty(cls, fmt: str, n_slots: int, H: int, I: int, device="cuda"):
        planes = {}
        for n, rows, K in (("gate", I, H), ("up", I, H), ("down", H, I)):
            planes[n + "_q"] = torch.empty(n_slots * plane_bytes(fmt, rows, K, False),
                                           dtype=torch.uint8, device=device)
            planes[n + "_s"] = torch.empty(n_slots * plane_bytes(fmt, rows, K, True),
                                           dtype=torch.uint8, device=device)
        return cls(fmt, n_slots, H, I, planes)

    @classmethod
    def from_canonical(cls, fmt: str, H: int, I: int, planes: dict, device="cuda", stream=None):
        """planes: name -> array [S, rows, ...] in the canonical layout (numpy or torch)."""
        n_slots = int(planes["gate_q"].shape[0])
        pool = cls.empty(fmt, n_slots, H, I, device)
        for n, rows, K in (("gate", I, H), ("up", I, H), ("down", H, I)):
            q = torch.as_tensor(planes[n + "_q"]).contiguous().view(torch.uint8).to(device)
            s = torch.as_tensor(planes[n + "_s"]).contiguous()
            s = (s.view(torch.int16) if s.dtype == torch.uint16 else s).view(torch.uint8).to(device)
            pool_pack(fmt, n_slots, rows, K, q, s, pool.planes[n + "_q"], pool.planes[n + "_s"],
                      stream)
        return pool


def pool_pack(fmt, n_mats, rows, K, src_q, src_s, dst_q, dst_s, stream=None):
    _check(_pool_pack(_FMT[fmt], n_mats, rows, K, _ptr(src_q), _ptr(src_s), _ptr(dst_q),
                      _ptr(dst_s), _stream(stream)))


# --------------------------------------------------------------------------- stages


def route_scratch_bytes(T: int, H: int, E: int) -> int:
    return _route_scratch(T, H, E)


def bucket_scratch_bytes(T: int, k: int, E: int) -> int:
    return _bucket_scratch(T, k, E)


def _scratch(nbytes, device):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device) if nbytes else None


def route(x, w_router, bias, k: int, ids=None, w=None, scratch=None, stream=None):
    """x bf16 [T, H], w_router bf16 [E, H], bias fp32 [E] or None -> (ids int32 [T,k], w fp32 [T,k])."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_router, torch.bfloat16, (E, H), "w_router")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if ids is None:
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    ns = route_scratch_bytes(T, H, E)
    if scratch is None:
        scratch = _scratch(ns, x.device)
    _check(_route(_ptr(x), _ptr(w_router), _ptr(bias), T, H, E, k, _ptr(ids), _ptr(w),
                  _ptr(scratch), scratch.numel() if scratch is not None else 0, _stream(stream)))
    return ids, w


def bucket(ids, E: int, counts=None, offsets=None, perm=None, inv_perm=None, scratch=None,
           stream=None):
    """ids int32 [T, k] -> (counts [E], offsets [E+1], perm [T*k], inv_perm [T*k]) int32."""
    T, k = ids.shape
    _need(ids, torch.int32, (T, k), "ids")
    dev = ids.device
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if offsets is None:
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    if perm is None:
        perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)[:T * k]
    if inv_perm is None:
        inv_perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)[:T * k]
    ns = bucket_scratch_bytes(T, k, E)
    if scratch is None:
        scratch = _scratch(ns, dev)
    _check(_bucket(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv_perm),
                   _ptr(scratch), scratch.numel() if scratch is not None else 0, _stream(stream)))
    return counts, offsets, perm, inv_perm


def expert_ffn(pool: Pool, slot_map, x, k: int, offsets, perm, err_flags=None, path=PATH_AUTO,
               stream=None):
    """-> (h bf16 [T*k, I], y fp32 [T*k, H]), both in bucket order."""
    T, H = x.shape
    E = slot_map.shape[0]
    _need(x, torch.bfloat16, (T, pool.H), "x")
    _need(slot_map, torch.int32, (E,), "slot_map")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    dev = x.device
    h = torch.empty((max(T * k, 1), pool.I), dtype=torch.bfloat16, device=dev)[:T * k]
    y = torch.empty((max(T * k, 1), pool.H), dtype=torch.float32, device=dev)[:T * k]
    _check(_ffn(ctypes.byref(pool.struct), _ptr(slot_map), E, _ptr(x), T, k, _ptr(offsets),
                _ptr(perm), _ptr(h), _ptr(y), _ptr(err_flags), path, _stream(stream)))
    return h, y


def expert_gate_up(pool: Pool, slot_map, x, k: int, offsets, perm, h=None, err_flags=None,
                   path=PATH_AUTO, stream=None):
    """-> h bf16 [T*k, I] in bucket order (gate, up and SwiGLU)."""
    T = x.shape[0]
    E = slot_map.shape[0]
    _need(x, torch.bfloat16, (T, pool.H), "x")
    if h is None:
        h = torch.empty((max(T * k, 1), pool.I), dtype=torch.bfloat16, device=x.device)[:T * k]
    _check(_gate_up(ctypes.byref(pool.struct), _ptr(slot_map), E, _ptr(x), T, k, _ptr(offsets),
                    _ptr(perm), _ptr(h), _ptr(err_flags), path, _stream(stream)))
    return h


def expert_down(pool: Pool, slot_map, T: int, k: int, offsets, h, y=None, err_flags=None,
                path=PATH_AUTO, stream=None):
    """h bf16 [T*k, I] -> y fp32 [T*k, H] in bucket order."""
    E = slot_map.shape[0]
    _need(h, torch.bfloat16, (T * k, pool.I), "h")
    if y is None:
        y = torch.empty((max(T * k, 1), pool.H), dtype=torch.float32, device=h.device)[:T * k]
    _check(_down(ctypes.byref(pool.struct), _ptr(slot_map), E, T, k, _ptr(offsets), _ptr(h),
                 _ptr(y), _ptr(err_flags), path, _stream(stream)))
    return y


def combine(y, inv_perm, w, out=None, stream=None):
    """y fp32 [T*k, H], inv_perm int32 [T*k], w fp32 [T, k] -> out fp32 [T, H]."""
    T, k = w.shape
    H = y.shape[1]
    _need(y, torch.float32, (T * k, H), "y")
    _need(w, torch.float32, (T, k), "w")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=y.device)
    _check(_combine(_ptr(y), _ptr(inv_perm), _ptr(w), T, k, H, _ptr(out), _stream(stream)))
    return out


def miss_list(slot_map, offsets, perm, k: int, stream=None):
    """Pairs routed to non-resident experts (slot_map == SLOT_MISS).

    slot_map int32 [E], offsets int32 [E+1], perm int32 [T*k] ->
    (miss_pos int32 [n_miss], miss_of_pair int32 [T*k], counters int32 [4]); the count
    n_miss (= counters[1]) is read back to size miss_pos, which synchronises the stream.
    """
    E = slot_map.shape[0]
    n = perm.shape[0]
    T = n // k
    dev = slot_map.device
    miss_pos = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    miss_of_pair = torch.empty(max(n, 1), dtype=torch.int32, device=dev)
    counters = torch.empty(4, dtype=torch.int32, device=dev)
    _check(_miss_list(_ptr(slot_map), E, _ptr(offsets), _ptr(perm), T, k, _ptr(miss_pos),
                      _ptr(miss_of_pair), _ptr(counters), _stream(stream)))
    n_miss = int(counters[1].item())
    return miss_pos[:n_miss], miss_of_pair[:n], counters


def merge_misses(out, y_miss, miss_of_pair, w, stream=None):
    """out fp32 [T, H] += w[t,j] * y_miss[miss_of_pair[t*k+j]] over missed pairs, j order."""
    T, k = w.shape
    H = out.shape[1]
    _need(out, torch.float32, (T, H), "out")
    _need(w, torch.float32, (T, k), "w")
    if y_miss.shape[0] == 0:
        return out
    _need(y_miss, torch.float32, (y_miss.shape[0], H), "y_miss")
    _check(_merge_misses(_ptr(out), _ptr(y_miss), _ptr(miss_of_pair), _ptr(w), T, k, H,
                         _stream(stream)))
    return out


def stage_plan(counts, slot_map, first_slot: int, n_stage: int, slot_map_out=None,
               copy_list=None, counters=None, stream=None):
    """Staging window plan (mapping rewrite) of one batch.

    counts int32 [E], slot_map int32 [E] -> (slot_map_out int32 [E], copy_list int32 [E],
    counters int32 [2]); copy_list[:counters[0]] are the staged experts in slot order.
    Nothing is read back: the copy takes copy_list and counters on the device.
    """
    E = slot_map.shape[0]
    _need(counts, torch.int32, (E,), "counts")
    _need(slot_map, torch.int32, (E,), "slot_map")
    dev = slot_map.device
    if slot_map_out is None:
        slot_map_out = torch.empty(E, dtype=torch.int32, device=dev)
    if copy_list is None:
        copy_list = torch.empty(E, dtype=torch.int32, device=dev)
    if counters is None:
        counters = torch.empty(2, dtype=torch.int32, device=dev)
    _check(_stage_plan(_ptr(counts), _ptr(slot_map), E, first_slot, n_stage,
                       _ptr(slot_map_out), _ptr(copy_list), _ptr(counters), _stream(stream)))
    return slot_map_out, copy_list, counters


def stage_copy(pool: Pool, backing: Pool, copy_list, counters, first_slot: int,
               max_copies: int, err_flags=None, stream=None):
    """Copy the planned experts from `backing` (slot = expert) into the pool's window."""
    _check(_stage_copy(ctypes.byref(pool.struct), ctypes.byref(backing.struct), _ptr(copy_list),
                       _ptr(counters), first_slot, max_copies, _ptr(err_flags),
                       _stream(stream)))


def _event_handles(events):
    """Raw hipEvent_t handles of a (begin, end) pair: ints (handles) or torch.cuda.Event.
    torch creates its underlying event on first record, so such events are recorded once
    (on the current stream) first."""
    hs = []
    for ev in events:
        if isinstance(ev, int):
            hs.append(ctypes.c_void_p(ev))
            continue
        if ev.cuda_event == 0:
            ev.record()
        hs.append(ctypes.c_void_p(ev.cuda_event))
    return tuple(hs)


def layer_workspace(T: int, H: int, I: int, E: int, k: int) -> WsLayout:
    L = WsLayout()
    _check(_ws(T, H, I, E, k, ctypes.byref(L)))
    return L


class Workspace:
    """A device workspace for moe_layer plus typed views of its intermediates."""

    def __init__(self, T, H, I, E, k, device="cuda"):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.layout = layer_workspace(T, H, I, E, k)
        self.buf = torch.empty(max(self.layout.total, 256), dtype=torch.uint8, device=device)

    def view(self, name, dtype, shape):
        off = getattr(self.layout, name)
        n = 1
        for d in shape:
            n *= d
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        return self.buf[off:off + nbytes].view(dtype).view(shape)

    def scratch(self):
        n = self.layout.act - self.layout.scratch
        return self.buf[self.layout.scratch:self.layout.act] if n > 0 else None

    def intermediates(self):
        T, k, E, H, I = self.T, self.k, self.E, self.H, self.I
        return dict(ids=self.view("topk_ids", torch.int32, (T, k)),
                    w=self.view("topk_w", torch.float32, (T, k)),
                    counts=self.view("counts", torch.int32, (E,)),
                    offsets=self.view("offsets", torch.int32, (E + 1,)),
                    perm=self.view("perm", torch.int32, (T * k,)),
                    inv_perm=self.view("inv_perm", torch.int32, (T * k,)),
                    h=self.view("h", torch.bfloat16, (T * k, I)),
                    y=self.view("y", torch.float32, (T * k, H)))


def layer(pool: Pool, slot_map, w_router, bias, x, k: int, out=None, workspace=None,
          err_flags=None, path=PATH_AUTO, stream=None, events=None):
    """The fused layer: x bf16 [T, H] -> out fp32 [T, H]. Returns (out, workspace).

    events: optional (begin, end) pair of timing events recorded on the stream around the
    gate/up launch (moe_layer_timed)."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, (T, pool.H), "x")
    _need(w_router, torch.bfloat16, (E, pool.H), "w_router")
    _need(slot_map, torch.int32, (E,), "slot_map")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = Workspace(T, pool.H, pool.I, E, k, x.device)
    args = (ctypes.byref(pool.struct), _ptr(slot_map), _ptr(w_router), _ptr(bias), _ptr(x),
            T, E, k, _ptr(out), _ptr(workspace.buf), workspace.buf.numel(), _ptr(err_flags),
            path, _stream(stream))
    if events is None:
        _check(_layer(*args))
    else:   # (begin, end) torch.cuda.Event pair recorded around the gate/up launch
        _check(_layer_timed(*args, *_event_handles(events)))
    return out, workspace


def layer_noalloc(pool: Pool, slot_map, w_router, bias, x, k: int, out=None, err_flags=None,
                  path=PATH_AUTO, stream=None):
    """moe_layer_noalloc: the fused layer with the library's static device workspace
    (no workspace argument). x bf16 [T, H] -> out fp32 [T, H]."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, (T, pool.H), "x")
    _need(w_router, torch.bfloat16, (E, pool.H), "w_router")
    _need(slot_map, torch.int32, (E,), "slot_map")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(out, torch.float32, (T, pool.H), "out")
    _check(_layer_noalloc(ctypes.byref(pool.struct), _ptr(slot_map), _ptr(w_router), _ptr(bias),
                          _ptr(x), T, E, k, _ptr(out), _ptr(err_flags), path, _stream(stream)))
    return out


class LayerCall:
    """A moe_layer (or moe_layer_timed) call with its arguments marshalled once.

    For loops that launch the same layer many times: calling the object enqueues the layer
    on `stream` with no per-call argument conversion. The tensors must stay alive.
    """

    def __init__(self, pool: Pool, slot_map, w_router, bias, x, k: int, out, workspace,
                 err_flags=None, path=PATH_AUTO, stream=None, events=None):
        T = x.shape[0]
        E = w_router.shape[0]
        _need(x, torch.bfloat16, (T, pool.H), "x")
        _need(w_router, torch.bfloat16, (E, pool.H), "w_router")
        _need(slot_map, torch.int32, (E,), "slot_map")
        _need(out, torch.float32, (T, pool.H), "out")
        self._keep = (pool, slot_map, w_router, bias, x, out, workspace, err_flags, events)
        args = (ctypes.byref(pool.struct), _ptr(slot_map), _ptr(w_router), _ptr(bias), _ptr(x),
                T, E, k, _ptr(out), _ptr(workspace.buf), workspace.buf.numel(), _ptr(err_flags),
                path, _stream(stream))
        if events is None:
            self._fn, self._args = _layer, args
        else:
            self._fn = _layer_timed
            self._args = args + _event_handles(events)

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            _check(st)


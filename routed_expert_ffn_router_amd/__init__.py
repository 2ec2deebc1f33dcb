"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every entry point takes torch tensors that live on the GPU, passes their
device pointers and the current HIP stream to the C ABI, and raises
``MoeError`` on a non-OK status.  All computation happens in libmoe's HIP
kernels; there is no fallback path.  torch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

FMT_BF16, FMT_Q2K, FMT_VQ2, FMT_MXFP4 = 0, 1, 2, 3
ROUTE_SOFTMAX_TOPK, ROUTE_HASH = 0, 1
ACT_BF16, ACT_MXFP8 = 0, 1
ACT_TRACE = 0x100  # with ACT_MXFP8 in expert_ffn: keep the fp32 SwiGLU output
OK, EINVAL, EUNSUPPORTED, ENOSPC, EHIP = 0, -1, -2, -3, -4


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class Weights(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n_experts", C.c_int32), ("rows", C.c_int32),
                ("cols", C.c_int32), ("data", C.c_void_p), ("scales", C.c_void_p),
                ("codebook", C.c_void_p)]


class Layer(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("I_shared", C.c_int32), ("route_mode", C.c_int32), ("w_router", C.c_void_p),
                ("gate", Weights), ("up", Weights), ("down", Weights),
                ("shared_gate", C.c_void_p), ("shared_up", C.c_void_p),
                ("shared_down", C.c_void_p), ("act_fmt", C.c_int32),
                ("steer_dir", C.c_void_p), ("steer_alpha", C.c_float)]


class SideStream(C.Structure):
    _fields_ = [("stream", C.c_void_p), ("fork", C.c_void_p), ("join", C.c_void_p)]


class ExpertCache(C.Structure):
    _fields_ = [("n_slots", C.c_int32), ("slot_gate", Weights), ("slot_up", Weights),
                ("slot_down", Weights), ("state", C.c_void_p)]


class Mark(C.Structure):
    _fields_ = [("start", C.c_void_p), ("stop", C.c_void_p), ("name", C.c_char_p)]


_lib = None


def build():
    """Compile libmoe.so for gfx950 (hipcc)."""
    from . import buildlib
    return buildlib.build()


def lib():
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoe.so is not built ({LIB_PATH}); run "
                              "routed_expert_ffn_router_amd.build()")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        L.moe_last_error.restype = C.c_char_p
        L.moe_abi_version.restype = i32
        L.moe_route_workspace.restype = sz
        L.moe_route_workspace.argtypes = [i32, i32]
        L.moe_route.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_dispatch_workspace.restype = sz
        L.moe_dispatch_workspace.argtypes = [i32, i32, i32]
        L.moe_dispatch.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_check_buckets.argtypes = [i32, i32, i32, i32, vp, vp, vp]
        L.moe_expert_ffn_workspace.restype = sz
        L.moe_expert_ffn_workspace.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
        L.moe_expert_ffn.argtypes = [i32, i32, i32, vp, C.POINTER(Weights), C.POINTER(Weights),
                                     C.POINTER(Weights), i32, vp, vp, i32, vp, vp, sz, vp]
        L.moe_mxfp8_quantize.argtypes = [i32, i32, vp, vp, vp, vp]
        L.moe_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, C.c_float, vp, vp, vp]
        L.moe_expert_ffn_a8_layout.argtypes = [i32, i32, i32, i32, i32, C.POINTER(sz),
                                               C.POINTER(sz), C.POINTER(sz)]
        L.moe_forward_workspace.restype = sz
        L.moe_forward_workspace.argtypes = [C.POINTER(Layer), i32]
        L.moe_forward.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                  C.POINTER(SideStream), vp]
        L.moe_dequantize.argtypes = [C.POINTER(Weights), i32, i64, i64, vp, vp]
        L.moe_forward_marked.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                         C.POINTER(Mark), i32, C.POINTER(i32), vp]
        L.moe_forward_static.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_cache_state_ints.restype = sz
        L.moe_cache_state_ints.argtypes = [i32, i32]
        L.moe_cache_reset.argtypes = [C.POINTER(ExpertCache), i32, vp]
        L.moe_forward_cached.argtypes = [C.POINTER(Layer), C.POINTER(ExpertCache), i32, vp, vp, vp,
                                         vp, vp, vp, vp, vp, sz, vp]
        L.moe_probe_read_blocks.restype = i32
        L.moe_probe_read_blocks.argtypes = [sz]
        L.moe_probe_hbm_read.argtypes = [vp, sz, vp, vp]
        L.moe_probe_mfma.argtypes = [i32, i32, i32, vp, C.POINTER(C.c_double), vp]
        _lib = L
    return _lib


def abi_version() -> int:
    return lib().moe_abi_version()


def _check(rc):
    if rc != OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


BF16 = (torch.bfloat16, torch.int16)  # bf16 values, or their bit patterns


def _dev(t, dtype, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
    if not ok:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------
# weights on the device
# --------------------------------------------------------------------------

class DeviceProj:
    """One projection of E experts in device memory (see include/moe.h)."""

    def __init__(self, fmt, E, N, K, data, scales=None, codebook=None):
        self.fmt, self.E, self.N, self.K = fmt, E, N, K
        self.data, self.scales, self.codebook = data, scales, codebook
        self.c = Weights(fmt, E, N, K, _ptr(data), _ptr(scales), _ptr(codebook))

    @classmethod
    def upload(cls, p, device="cuda", codebook=None):
        """From a host projection with numpy fields fmt/E/N/K/data/scales/codebook."""
        data = torch.from_numpy(p.data.reshape(-1).view("uint8").copy()).to(device)
        scales = None
        if p.scales is not None:
            scales = torch.from_numpy(p.scales.reshape(-1).view("uint8").copy()).to(device)
        cb = codebook
        if cb is None and p.codebook is not None:
            cb = torch.from_numpy(p.codebook.reshape(-1).view("uint8").copy()).to(device)
        return cls(p.fmt, p.E, p.N, p.K, data, scales, cb)

    def clone(self):
        return DeviceProj(self.fmt, self.E, self.N, self.K, self.data.clone(),
                          None if self.scales is None else self.scales.clone(), self.codebook)

    def nbytes_per_expert(self):
        n = self.data.numel() // self.E
        if self.scales is not None:
            n += self.scales.numel() // self.E
        return n


class DeviceLayer:
    """A whole MoE layer in device memory, with its moe_layer descriptor."""

    def __init__(self, H, I, E, k, route_mode, w_router, gate, up, down,
                 shared_gate=None, shared_up=None, shared_down=None, act=ACT_BF16,
                 steer_dir=None, steer_alpha=0.0):
        self.H, self.I, self.E, self.k, self.route_mode = H, I, E, k, route_mode
        self.act = act
        self.w_router, self.gate, self.up, self.down = w_router, gate, up, down
        self.shared_gate, self.shared_up, self.shared_down = shared_gate, shared_up, shared_down
        self.steer_dir, self.steer_alpha = _dev(steer_dir, torch.float32, "steer_dir"), steer_alpha
        self.I_shared = 0 if shared_gate is None else shared_gate.shape[0]
        self.c = Layer(H, I, E, k, self.I_shared, route_mode, _ptr(w_router), gate.c, up.c, down.c,
                       _ptr(shared_gate), _ptr(shared_up), _ptr(shared_down), act,
                       _ptr(steer_dir), float(steer_alpha))

    @classmethod
    def upload(cls, layer, route_mode=ROUTE_SOFTMAX_TOPK, device="cuda", act=ACT_BF16):
        """From a host layer (fields spec, w_router, gate, up, down, shared_*, codebook)."""
        s = layer.spec

        def u16(a):
            return None if a is None else torch.from_numpy(a.view("int16").copy()).to(device)

        cb = None
        if layer.codebook is not None:
            cb = torch.from_numpy(layer.codebook.reshape(-1).view("uint8").copy()).to(device)
        return cls(s.H, s.I, s.E, s.k, route_mode, u16(layer.w_router),
                   DeviceProj.upload(layer.gate, device, cb if layer.gate.fmt == FMT_VQ2 else None),
                   DeviceProj.upload(layer.up, device, cb if layer.up.fmt == FMT_VQ2 else None),
                   DeviceProj.upload(layer.down, device, cb if layer.down.fmt == FMT_VQ2 else None),
                   u16(layer.shared_gate), u16(layer.shared_up), u16(layer.shared_down), act)

    def clone(self):
        """An independent copy of every weight (distinct device memory)."""
        cl = lambda t: None if t is None else t.clone()
        return DeviceLayer(self.H, self.I, self.E, self.k, self.route_mode, cl(self.w_router),
                           self.gate.clone(), self.up.clone(), self.down.clone(),
                           cl(self.shared_gate), cl(self.shared_up), cl(self.shared_down),
                           self.act, cl(self.steer_dir), self.steer_alpha)

    def with_route_mode(self, mode):
        return DeviceLayer(self.H, self.I, self.E, self.k, mode, self.w_router, self.gate,
                           self.up, self.down, self.shared_gate, self.shared_up, self.shared_down,
                           self.act, self.steer_dir, self.steer_alpha)

    def with_act(self, act):
        """The same weights with another activation format (MOE_ACT_*)."""
        return DeviceLayer(self.H, self.I, self.E, self.k, self.route_mode, self.w_router,
                           self.gate, self.up, self.down, self.shared_gate, self.shared_up,
                           self.shared_down, act, self.steer_dir, self.steer_alpha)

    def with_steering(self, steer_dir, steer_alpha):
        """The same weights with an activation-steering direction (fp32 [H] on
        the device, or None) and strength."""
        return DeviceLayer(self.H, self.I, self.E, self.k, self.route_mode, self.w_router,
                           self.gate, self.up, self.down, self.shared_gate, self.shared_up,
                           self.shared_down, self.act, steer_dir, steer_alpha)

    def forward_workspace(self, T):
        return lib().moe_forward_workspace(C.byref(self.c), T)


# --------------------------------------------------------------------------
# entry points
# --------------------------------------------------------------------------

def route(x, w_router, k, mode=ROUTE_SOFTMAX_TOPK, logits_in=None, token_ids=None,
          want_logits=True):
    """moe_route -> (topk_idx int32 [T,k], topk_w fp32 [T,k], logits fp32 [T,E] or None)."""
    dev = (x if x is not None else logits_in).device
    if logits_in is not None:
        T, E = logits_in.shape
        H = 0 if x is None else x.shape[1]
    else:
        T, H = x.shape
        E = w_router.shape[0]
    _dev(x, BF16, "x")
    _dev(w_router, BF16, "w_router")
    _dev(logits_in, torch.float32, "logits_in")
    _dev(token_ids, torch.int64, "token_ids")
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    lo = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    ws = None if want_logits else _ws(lib().moe_route_workspace(T, E), dev)
    _check(lib().moe_route(mode, T, H, E, k, _ptr(x), _ptr(w_router), _ptr(logits_in),
                           _ptr(token_ids), _ptr(idx), _ptr(w), _ptr(lo), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream()))
    return idx, w, lo


def check_buckets(T, E, k, n_rows, expert_offsets, sorted_token=None, slot_pos=None):
    """moe_check_buckets on host int32 arrays (numpy): expert_offsets [E+1],
    sorted_token [n_rows], slot_pos [T*k]; raises MoeError on a malformed
    bucketing."""
    import numpy as np

    def host(a, n, name):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=np.int32)
        if a.size != n:
            raise ValueError(f"{name}: {a.size} values, expected {n}")
        return a

    off = host(expert_offsets, E + 1, "expert_offsets")
    st = host(sorted_token, n_rows, "sorted_token")
    sp = host(slot_pos, T * k, "slot_pos")
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    _check(lib().moe_check_buckets(T, E, k, n_rows, ptr(off), ptr(st), ptr(sp)))


def dispatch(topk_idx, E):
    """moe_dispatch -> (expert_offsets [E+1], sorted_token, sorted_slot, slot_pos) int32."""
    _dev(topk_idx, torch.int32, "topk_idx")
    T, k = topk_idx.shape
    dev = topk_idx.device
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    st = torch.empty(T * k, dtype=torch.int32, device=dev)
    ss = torch.empty(T * k, dtype=torch.int32, device=dev)
    sp = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = _ws(lib().moe_dispatch_workspace(T, E, k), dev)
    _check(lib().moe_dispatch(T, E, k, _ptr(topk_idx), _ptr(off), _ptr(st), _ptr(ss), _ptr(sp),
                              _ptr(ws), ws.numel(), _stream()))
    return off, st, ss, sp


def expert_ffn(x, gate, up, down, expert_offsets=None, sorted_token=None, n_rows=None,
               act=ACT_BF16, keep_ws=False):
    """moe_expert_ffn -> y_rows fp32 [n_rows, H] (dense over x when offsets is None);
    with keep_ws, (y_rows, workspace)."""
    _dev(x, BF16, "x")
    _dev(expert_offsets, torch.int32, "expert_offsets")
    _dev(sorted_token, torch.int32, "sorted_token")
    T, H = x.shape
    I = gate.N
    if n_rows is None:
        n_rows = T if expert_offsets is None else sorted_token.numel()
    y = torch.empty((n_rows, H), dtype=torch.float32, device=x.device)
    ws = _ws(lib().moe_expert_ffn_workspace(T, n_rows, gate.E, H, I, gate.fmt, down.fmt, act),
             x.device)
    _check(lib().moe_expert_ffn(T, H, I, _ptr(x), C.byref(gate.c), C.byref(up.c), C.byref(down.c),
                                act, _ptr(expert_offsets), _ptr(sorted_token), n_rows, _ptr(y),
                                _ptr(ws), ws.numel(), _stream()))
    return (y, ws) if keep_ws else y


def a8_intermediate(ws, T, n_rows, E, H, I):
    """The MX-FP8 SwiGLU output a MOE_ACT_MXFP8 moe_expert_ffn call left in its
    workspace `ws`: (E4M3 codes uint8 [n_rows, I], E8M0 scales uint8 [n_rows, I/32],
    fp32 values they were quantized from [n_rows, I] -- meaningful when the call
    had ACT_TRACE)."""
    co, so, fo = C.c_size_t(0), C.c_size_t(0), C.c_size_t(0)
    _check(lib().moe_expert_ffn_a8_layout(T, n_rows, E, H, I, C.byref(co), C.byref(so),
                                          C.byref(fo)))
    codes = ws[co.value:co.value + n_rows * I].view(n_rows, I)
    scales = ws[so.value:so.value + n_rows * (I // 32)].view(n_rows, I // 32)
    vals = ws[fo.value:fo.value + 4 * n_rows * I].view(torch.float32).view(n_rows, I)
    return codes, scales, vals


def mxfp8_quantize(x):
    """moe_mxfp8_quantize -> (E4M3 codes uint8 [rows, K], E8M0 scales uint8 [rows, K/32])."""
    _dev(x, BF16, "x")
    rows, K = x.shape
    q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    sc = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    _check(lib().moe_mxfp8_quantize(rows, K, _ptr(x), _ptr(q), _ptr(sc), _stream()))
    return q, sc


def combine(y_rows, slot_pos, topk_w, shared_y=None, want_bf16=False, steer_dir=None,
            steer_alpha=0.0):
    """moe_combine -> (out fp32 [T, H], out bf16 bits [T, H] or None)."""
    _dev(y_rows, torch.float32, "y_rows")
    _dev(slot_pos, torch.int32, "slot_pos")
    _dev(topk_w, torch.float32, "topk_w")
    _dev(shared_y, torch.float32, "shared_y")
    _dev(steer_dir, torch.float32, "steer_dir")
    T, k = topk_w.shape
    H = y_rows.shape[1]
    out = torch.empty((T, H), dtype=torch.float32, device=y_rows.device)
    ob = torch.empty((T, H), dtype=torch.int16, device=y_rows.device) if want_bf16 else None
    _check(lib().moe_combine(T, H, k, _ptr(y_rows), _ptr(slot_pos), _ptr(topk_w), _ptr(shared_y),
                             _ptr(steer_dir), float(steer_alpha), _ptr(out), _ptr(ob),
                             _stream()))
    return out, ob


class Forward:
    """moe_forward on a DeviceLayer with preallocated outputs and workspace.

    With side_stream (the default) it owns a second torch stream and two
    events that moe_forward uses for the shared expert above one token."""

    def __init__(self, layer, T, device="cuda", want_bf16=False, side_stream=True):
        self.layer, self.T = layer, T
        self.out = torch.empty((T, layer.H), dtype=torch.float32, device=device)
        self.out_bf16 = torch.empty((T, layer.H), dtype=torch.int16, device=device) if want_bf16 else None
        self.idx = torch.empty((T, layer.k), dtype=torch.int32, device=device)
        self.w = torch.empty((T, layer.k), dtype=torch.float32, device=device)
        self.ws = _ws(layer.forward_workspace(T), device)
        self.side = None
        if side_stream:
            self._side_stream = torch.cuda.Stream(device=device)
            self._fork = torch.cuda.Event()
            self._join = torch.cuda.Event()
            # torch creates the HIP events on first record
            self._fork.record(self._side_stream)
            self._join.record(self._side_stream)
            self.side = SideStream(self._side_stream.cuda_stream, self._fork.cuda_event,
                                   self._join.cuda_event)

    def __call__(self, x, logits_in=None, token_ids=None, layer=None):
        L = self.layer if layer is None else layer
        _dev(x, BF16, "x")
        _dev(logits_in, torch.float32, "logits_in")
        _dev(token_ids, torch.int64, "token_ids")
        _check(lib().moe_forward(C.byref(L.c), self.T, _ptr(x), _ptr(logits_in), _ptr(token_ids),
                                 _ptr(self.out), _ptr(self.out_bf16), _ptr(self.idx), _ptr(self.w),
                                 _ptr(self.ws), self.ws.numel(),
                                 None if self.side is None else C.byref(self.side), _stream()))
        return self.out


    def marked(self, x, events, logits_in=None, token_ids=None, layer=None):
        """moe_forward_marked: `events` is a list of (start, stop) torch.cuda.Event
        pairs (already recorded once, so that the HIP events exist); kernel i
        records pair i at its own start and end.  Returns the kernel names."""
        L = self.layer if layer is None else layer
        marks = (Mark * len(events))(*[Mark(a.cuda_event, b.cuda_event, None) for a, b in events])
        n = C.c_int(0)
        _check(lib().moe_forward_marked(C.byref(L.c), self.T, _ptr(x), _ptr(logits_in),
                                        _ptr(token_ids), _ptr(self.out), _ptr(self.out_bf16),
                                        _ptr(self.idx), _ptr(self.w), _ptr(self.ws), self.ws.numel(),
                                        marks, len(events), C.byref(n), _stream()))
        return [marks[i].name.decode() for i in range(n.value)]


class CachedLayer:
    """A layer whose routed experts live in pinned host memory, with a pool of
    n_slots expert slots in device memory and the cache state
    (moe_expert_cache); forward() runs moe_forward_cached on one token."""

    def __init__(self, host, n_slots, device="cuda", route_mode=ROUTE_SOFTMAX_TOPK):
        s = host.spec
        dev = torch.device(device)

        def pinned(a):
            return torch.from_numpy(a.reshape(-1).view("uint8").copy()).pin_memory()

        cb = None
        if host.codebook is not None:
            cb = torch.from_numpy(host.codebook.reshape(-1).view("uint8").copy()).to(dev)
        projs, slots = [], []
        for p in (host.gate, host.up, host.down):
            c = cb if p.fmt == FMT_VQ2 else None
            hd = pinned(p.data)
            hs = None if p.scales is None else pinned(p.scales)
            projs.append(DeviceProj(p.fmt, p.E, p.N, p.K, hd, hs, c))
            sd = torch.empty(hd.numel() // p.E * n_slots, dtype=torch.uint8, device=dev)
            ss = None if hs is None else torch.empty(hs.numel() // p.E * n_slots,
                                                     dtype=torch.uint8, device=dev)
            slots.append(DeviceProj(p.fmt, n_slots, p.N, p.K, sd, ss, c))

        def u16(a):
            return None if a is None else torch.from_numpy(a.view("int16").copy()).to(dev)

        self.layer = DeviceLayer(s.H, s.I, s.E, s.k, route_mode, u16(host.w_router), *projs,
                                 u16(host.shared_gate), u16(host.shared_up),
                                 u16(host.shared_down))
        self.slots = slots
        self.n_slots, self.E = n_slots, s.E
        self.state = torch.empty(int(lib().moe_cache_state_ints(s.E, n_slots)),
                                 dtype=torch.int32, device=dev)
        self.c = ExpertCache(n_slots, slots[0].c, slots[1].c, slots[2].c, _ptr(self.state))
        self.f = Forward(self.layer, 1, dev, side_stream=False)
        self.reset()

    def reset(self):
        """moe_cache_reset: no expert resident."""
        _check(lib().moe_cache_reset(C.byref(self.c), self.E, _stream()))

    def __call__(self, x, logits_in=None, token_ids=None):
        """moe_forward_cached -> the layer's output fp32 [1, H] (and .idx, .w)."""
        _dev(x, BF16, "x")
        _dev(logits_in, torch.float32, "logits_in")
        _dev(token_ids, torch.int64, "token_ids")
        f = self.f
        _check(lib().moe_forward_cached(C.byref(self.layer.c), C.byref(self.c), x.shape[0],
                                        _ptr(x), _ptr(logits_in), _ptr(token_ids), _ptr(f.out),
                                        None, _ptr(f.idx), _ptr(f.w), _ptr(f.ws), f.ws.numel(),
                                        _stream()))
        return f.out

    @property
    def idx(self):
        return self.f.idx

    @property
    def w(self):
        return self.f.w

    def resident(self):
        """Host copy of the expert -> slot map (-1: not resident)."""
        return self.state[4:4 + self.E].cpu().numpy()

    def counts(self):
        """(hits, misses) so far."""
        h = self.state[2:4].cpu().numpy()
        return int(h[0]), int(h[1])


def forward_static(layer, x, out, idx, w, logits_in=None, token_ids=None, out_bf16=None):
    """moe_forward_static into preallocated outputs (out fp32 [T, H], idx int32
    [T, k], w fp32 [T, k]): no workspace, no allocation."""
    _dev(x, BF16, "x")
    _dev(logits_in, torch.float32, "logits_in")
    _dev(token_ids, torch.int64, "token_ids")
    _check(lib().moe_forward_static(C.byref(layer.c), x.shape[0], _ptr(x), _ptr(logits_in),
                                    _ptr(token_ids), _ptr(out), _ptr(out_bf16), _ptr(idx),
                                    _ptr(w), _stream()))
    return out


def forward(layer, x, logits_in=None, token_ids=None):
    """moe_forward -> (out fp32 [T, H], topk_idx, topk_w)."""
    f = Forward(layer, x.shape[0], x.device)
    f(x, logits_in, token_ids)
    return f.out, f.idx, f.w


def dequantize(proj, expert=0, w0=0, count=None):
    """moe_dequantize -> fp32 weights [w0, w0+count) of one expert's flattened matrix."""
    if count is None:
        count = proj.N * proj.K - w0
    out = torch.empty(count, dtype=torch.float32, device=proj.data.device)
    _check(lib().moe_dequantize(C.byref(proj.c), expert, w0, count, _ptr(out), _stream()))
    return out


# --------------------------------------------------------------------------
# measurement probes (include/moe_probe.h)
# --------------------------------------------------------------------------

PROBE_BF16, PROBE_F16, PROBE_F8F4, PROBE_BF16_32, PROBE_F16_32 = 0, 1, 2, 3, 4


def probe_sink_words(nbytes):
    """uint32 words of sink that probe_hbm_read needs for an nbytes buffer."""
    return int(lib().moe_probe_read_blocks(nbytes))


def probe_hbm_read(buf, sink):
    """moe_probe_hbm_read: stream-read the whole of `buf` (a GPU tensor)."""
    _check(lib().moe_probe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                    _stream()))


def probe_mfma(kind, blocks, iters, sink):
    """moe_probe_mfma -> the flops the launch performs."""
    fl = C.c_double(0.0)
    _check(lib().moe_probe_mfma(kind, blocks, iters, _ptr(sink), C.byref(fl), _stream()))
    return fl.value

"""ctypes wrapper of the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, the package smoke check and
bench.py's CPU-baseline leg, never by the GPU library.  Arguments are the
numpy arrays produced by ``synth``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "moe_oracle.c")


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no FP contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
             "-Wall", "-Wno-unknown-pragmas", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Proj(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("E", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
                ("data", C.c_void_p), ("scales", C.c_void_p), ("codebook", C.c_void_p)]


class Layer(C.Structure):
    _fields_ = [("H", C.c_int32), ("I", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("I_shared", C.c_int32), ("route_mode", C.c_int32),
                ("w_router", C.c_void_p), ("gate", Proj), ("up", Proj), ("down", Proj),
                ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
                ("steer_dir", C.c_void_p), ("steer_alpha", C.c_float)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64
        L.orc_bf16.restype = C.c_float
        L.orc_bf16.argtypes = [C.c_uint16]
        L.orc_f16.restype = C.c_float
        L.orc_f16.argtypes = [C.c_uint16]
        L.orc_e2m1.restype = C.c_float
        L.orc_e2m1.argtypes = [C.c_uint]
        L.orc_e8m0.restype = C.c_double
        L.orc_e8m0.argtypes = [C.c_uint]
        L.orc_e4m3.restype = C.c_float
        L.orc_e4m3.argtypes = [C.c_uint]
        L.orc_to_e4m3.restype = C.c_uint8
        L.orc_to_e4m3.argtypes = [C.c_double]
        L.orc_splitmix64.restype = C.c_uint64
        L.orc_splitmix64.argtypes = [C.c_uint64]
        L.orc_dequant.restype = i32
        L.orc_dequant.argtypes = [C.POINTER(Proj), i32, i64, i64, vp]
        L.orc_router_logits.argtypes = [i32, i32, i32, vp, vp, vp]
        L.orc_select_topk.argtypes = [i32, i32, i32, vp, vp, vp]
        L.orc_select_hash.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.orc_route.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.orc_dispatch.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_expert_ffn.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp]
        L.orc_shared_ffn.argtypes = [C.POINTER(Layer), i32, vp, vp]
        L.orc_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, C.c_float, vp]
        L.orc_forward.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp, vp, vp]
        L.orc_forward_a8.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp, vp, vp]
        L.orc_dense_masked.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp]
        L.orc_mxfp8_quant.argtypes = [i32, i32, vp, vp, vp]
        L.orc_a8_swiglu_codes.argtypes = [C.POINTER(Layer), i32, vp, vp, vp, vp, vp]
        L.orc_a8_down.argtypes = [C.POINTER(Layer), vp, vp, vp, vp]
        L.orc_threads.restype = i32
        L.orc_set_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# scalar decodes
# --------------------------------------------------------------------------

def bf16(b):
    return lib().orc_bf16(int(b))


def f16(h):
    return lib().orc_f16(int(h))


def e2m1(n):
    return lib().orc_e2m1(int(n))


def e8m0(e):
    return lib().orc_e8m0(int(e))


def e4m3(c):
    return lib().orc_e4m3(int(c))


def to_e4m3(v):
    return int(lib().orc_to_e4m3(float(v)))


def splitmix64(x):
    return int(lib().orc_splitmix64(int(x) & 0xFFFFFFFFFFFFFFFF))


def threads():
    return int(lib().orc_threads())


def set_threads(n):
    """Threads of the oracle's parallel loops (results do not depend on it)."""
    lib().orc_set_threads(int(n))


# --------------------------------------------------------------------------
# weights
# --------------------------------------------------------------------------

def _proj(p, keep):
    """orc_proj for a synth.Proj (keeps the contiguous arrays alive in keep)."""
    data = _c(p.data, p.data.dtype)
    keep.append(data)
    sc = cb = None
    if p.scales is not None:
        sc = _c(p.scales, p.scales.dtype)
        keep.append(sc)
    if p.codebook is not None:
        cb = _c(p.codebook, np.int8)
        keep.append(cb)
    return Proj(p.fmt, p.E, p.N, p.K, _p(data), _p(sc), _p(cb))


def dequant(p, expert=0, n0=0, count=None):
    """fp32 weights [n0, n0+count) of one expert's row-major flattened matrix."""
    keep = []
    cp = _proj(p, keep)
    if count is None:
        count = p.N * p.K - n0
    out = np.empty(count, np.float32)
    rc = lib().orc_dequant(C.byref(cp), expert, n0, count, out.ctypes.data)
    if rc:
        raise ValueError("orc_dequant rejected its arguments")
    return out


def dequant_matrix(p, expert=0):
    return dequant(p, expert).reshape(p.N, p.K)


# --------------------------------------------------------------------------
# layer
# --------------------------------------------------------------------------

class LayerRef:
    """Binds a synth.Layer for the oracle calls."""

    def __init__(self, layer, route_mode=0, steer_dir=None, steer_alpha=0.0):
        s = layer.spec
        self.layer = layer
        self.keep = []
        wr = _c(layer.w_router, np.uint16)
        self.keep.append(wr)
        sh = []
        for a in (layer.shared_gate, layer.shared_up, layer.shared_down):
            if a is None:
                sh.append(None)
            else:
                a = _c(a, np.uint16)
                self.keep.append(a)
                sh.append(_p(a))
        sd = None
        if steer_dir is not None:
            sd = _c(steer_dir, np.float32)
            self.keep.append(sd)
        self.c = Layer(s.H, s.I, s.E, s.k, s.I_shared if layer.shared_gate is not None else 0,
                       route_mode, _p(wr), _proj(layer.gate, self.keep),
                       _proj(layer.up, self.keep), _proj(layer.down, self.keep), *sh, _p(sd),
                       float(steer_alpha))
        self.H, self.I, self.E, self.k = s.H, s.I, s.E, s.k

    def route(self, x, logits_in=None, token_ids=None, mode=None):
        mode = self.c.route_mode if mode is None else mode
        x = _c(x, np.uint16)
        T = x.shape[0]
        idx = np.empty((T, self.k), np.int32)
        w = np.empty((T, self.k), np.float32)
        lo = np.empty((T, self.E), np.float32)
        li = None if logits_in is None else _c(logits_in, np.float32)
        ti = None if token_ids is None else _c(token_ids, np.int64)
        rc = lib().orc_route(mode, T, self.H, self.E, self.k, _p(x), self.c.w_router, _p(li),
                             _p(ti), _p(idx), _p(w), _p(lo))
        if rc:
            raise ValueError("orc_route rejected its arguments")
        return idx, w, lo

    def expert_ffn(self, x, offsets, sorted_token):
        x = _c(x, np.uint16)
        offsets = _c(offsets, np.int32)
        st = _c(sorted_token, np.int32)
        y = np.empty((int(offsets[-1]), self.H), np.float32)
        rc = lib().orc_expert_ffn(C.byref(self.c), x.shape[0], _p(x), _p(offsets), _p(st), _p(y))
        if rc:
            raise ValueError("orc_expert_ffn failed")
        return y

    def shared_ffn(self, x):
        x = _c(x, np.uint16)
        y = np.empty((x.shape[0], self.H), np.float32)
        lib().orc_shared_ffn(C.byref(self.c), x.shape[0], _p(x), _p(y))
        return y

    def forward(self, x, logits_in=None, token_ids=None, a8=False):
        x = _c(x, np.uint16)
        T = x.shape[0]
        out = np.empty((T, self.H), np.float32)
        idx = np.empty((T, self.k), np.int32)
        w = np.empty((T, self.k), np.float32)
        li = None if logits_in is None else _c(logits_in, np.float32)
        ti = None if token_ids is None else _c(token_ids, np.int64)
        f = lib().orc_forward_a8 if a8 else lib().orc_forward
        rc = f(C.byref(self.c), T, _p(x), _p(li), _p(ti), _p(out), _p(idx), _p(w))
        if rc:
            raise ValueError("orc_forward failed")
        return out, idx, w

    def a8_swiglu_codes(self, x, offsets, sorted_token):
        """MX-FP8 codes [n_rows, I] and E8M0 scales [n_rows, I/32] of each bucket
        row's SwiGLU output in the A8 variant (x quantized first)."""
        x = _c(x, np.uint16)
        offsets = _c(offsets, np.int32)
        st = _c(sorted_token, np.int32)
        n = int(offsets[-1])
        codes = np.empty((n, self.I), np.uint8)
        scales = np.empty((n, self.I // 32), np.uint8)
        rc = lib().orc_a8_swiglu_codes(C.byref(self.c), x.shape[0], _p(x), _p(offsets), _p(st),
                                       _p(codes), _p(scales))
        if rc:
            raise ValueError("orc_a8_swiglu_codes failed")
        return codes, scales

    def a8_down(self, offsets, codes, scales):
        """y_rows [n_rows, H]: each bucket row's down projection of the given
        MX-FP8 codes and scales."""
        offsets = _c(offsets, np.int32)
        codes = _c(codes, np.uint8)
        scales = _c(scales, np.uint8)
        y = np.empty((int(offsets[-1]), self.H), np.float32)
        rc = lib().orc_a8_down(C.byref(self.c), _p(offsets), _p(codes), _p(scales), _p(y))
        if rc:
            raise ValueError("orc_a8_down failed")
        return y

    def dense_masked(self, x, idx, w):
        x = _c(x, np.uint16)
        idx = _c(idx, np.int32)
        w = _c(w, np.float32)
        out = np.empty((x.shape[0], self.H), np.float32)
        rc = lib().orc_dense_masked(C.byref(self.c), x.shape[0], _p(x), _p(idx), _p(w), _p(out))
        if rc:
            raise ValueError("orc_dense_masked failed")
        return out


def router_logits(x, w_router):
    x = _c(x, np.uint16)
    wr = _c(w_router, np.uint16)
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float32)
    lib().orc_router_logits(T, H, E, _p(x), _p(wr), _p(out))
    return out


def select_topk(logits, k):
    lg = _c(logits, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().orc_select_topk(T, E, k, _p(lg), _p(idx), _p(w))
    return idx, w


def select_hash(token_ids, logits, k):
    lg = _c(logits, np.float32)
    ti = _c(token_ids, np.int64)
    T, E = lg.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().orc_select_hash(T, E, k, _p(ti), _p(lg), _p(idx), _p(w))
    return idx, w


def dispatch(idx, E):
    idx = _c(idx, np.int32)
    T, k = idx.shape
    off = np.empty(E + 1, np.int32)
    st = np.empty(T * k, np.int32)
    ss = np.empty(T * k, np.int32)
    sp = np.empty(T * k, np.int32)
    lib().orc_dispatch(T, E, k, _p(idx), _p(off), _p(st), _p(ss), _p(sp))
    return off, st, ss, sp


def combine(y_rows, slot_pos, w, shared_y=None, steer_dir=None, steer_alpha=0.0):
    y = _c(y_rows, np.float32)
    sp = _c(slot_pos, np.int32)
    w = _c(w, np.float32)
    T, k = w.shape
    H = y.shape[1]
    sy = None if shared_y is None else _c(shared_y, np.float32)
    sd = None if steer_dir is None else _c(steer_dir, np.float32)
    out = np.empty((T, H), np.float32)
    lib().orc_combine(T, H, k, _p(y), _p(sp), _p(w), _p(sy), _p(sd), float(steer_alpha), _p(out))
    return out


def mxfp8_quant(a):
    a = _c(a, np.float32)
    rows, K = a.shape
    codes = np.empty((rows, K), np.uint8)
    scales = np.empty((rows, (K + 31) // 32), np.uint8)
    lib().orc_mxfp8_quant(rows, K, _p(a), _p(codes), _p(scales))
    return codes, scales

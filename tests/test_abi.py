"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe.h declares, and rejects bad arguments on the host before any HIP
call (so these run in a container with no GPU)."""
import ctypes as C
import glob
import os
import re

import pytest

import routed_expert_ffn_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # an aligned, never dereferenced "device pointer"


def _lib():
    if not os.path.exists(moe.LIB_PATH):
        pytest.skip("libmoe.so not built")
    return moe.lib()


def declared_functions():
    """Every function declared by the headers under include/."""
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(moe_\w+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["moe_route", "moe_dispatch", "moe_expert_ffn", "moe_combine", "moe_forward",
              "moe_dequantize", "moe_last_error", "moe_abi_version", "moe_route_workspace",
              "moe_dispatch_workspace", "moe_expert_ffn_workspace", "moe_forward_workspace",
              "moe_mxfp8_quantize", "moe_expert_ffn_a8_layout", "moe_probe_hbm_read",
              "moe_probe_mfma", "moe_probe_read_blocks"]:
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = _lib()
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_abi_version():
    assert moe.abi_version() == 5


def test_library_creates_no_hip_objects():
    """No stream, event, graph or memory of the library's own: every HIP
    object it touches is the caller's."""
    csrc = os.path.join(ROOT, "routed_expert_ffn_router_amd", "csrc")
    banned = re.compile(r"\b(hip(Stream|Event|Graph)Create\w*|hipMalloc\w*|hipFree\w*|"
                        r"hipHostMalloc|thread_local\s+\w*Stream)")
    for f in sorted(os.listdir(csrc)):
        src = open(os.path.join(csrc, f)).read()
        src = re.sub(r"//[^\n]*", "", src)
        assert not banned.search(src), (f, banned.search(src).group(0))


def _w(fmt=moe.FMT_VQ2, E=8, N=2048, K=4096, data=FAKE, scales=FAKE, cb=FAKE):
    return moe.Weights(fmt, E, N, K, data, scales, cb)


def _err():
    return moe.lib().moe_last_error().decode()


def test_route_rejects_bad_arguments():
    lib = _lib()
    ok_args = dict(mode=0, T=4, H=256, E=8, k=2, x=FAKE, wr=FAKE, li=None, tid=None, idx=FAKE,
                   w=FAKE, lo=FAKE, ws=None, wsb=0, s=None)

    def call(**kw):
        a = dict(ok_args, **kw)
        return lib.moe_route(a["mode"], a["T"], a["H"], a["E"], a["k"], a["x"], a["wr"], a["li"],
                             a["tid"], a["idx"], a["w"], a["lo"], a["ws"], a["wsb"], a["s"])

    assert call(k=0) == moe.EINVAL and "k = 0" in _err()
    assert call(k=9) == moe.EINVAL
    assert call(k=17, E=32) == moe.EINVAL
    assert call(E=0) == moe.EINVAL
    assert call(E=2000) == moe.EINVAL
    assert call(mode=7) == moe.EINVAL
    assert call(T=-1) == moe.EINVAL
    assert call(mode=1) == moe.EINVAL and "token_ids" in _err()
    assert call(idx=None) == moe.EINVAL
    assert call(x=None) == moe.EINVAL
    assert call(H=100) == moe.EINVAL
    assert call(x=FAKE + 2) == moe.EINVAL and "misaligned" in _err()
    assert call(lo=None) == moe.ENOSPC
    assert call(lo=None, ws=FAKE, wsb=lib.moe_route_workspace(4, 8) - 1) == moe.ENOSPC
    assert call(T=0) == moe.OK  # no tokens: nothing to do, nothing enqueued


def test_dispatch_rejects_bad_arguments():
    lib = _lib()
    f = lib.moe_dispatch
    ws = lib.moe_dispatch_workspace(16, 8, 2)
    assert ws > 0
    assert f(16, 8, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == moe.EINVAL
    assert f(16, 8, 2, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None) == moe.EINVAL
    assert f(16, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, None) == moe.ENOSPC
    assert f(16, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == moe.ENOSPC
    assert f(0, 8, 2, None, None, None, None, None, None, 0, None) == moe.OK


def test_expert_ffn_rejects_bad_arguments():
    lib = _lib()
    g, u, d = _w(), _w(), _w(moe.FMT_Q2K, 8, 4096, 2048, FAKE, None, None)
    f = lib.moe_expert_ffn
    ws = lib.moe_expert_ffn_workspace(1, 8, 8, 4096, 2048, moe.FMT_VQ2, moe.FMT_Q2K, 0)

    def call(g=g, u=u, d=d, H=4096, I=2048, off=FAKE, st=FAKE, n=8, ws_=ws, act=0):
        return f(1, H, I, FAKE, C.byref(g), C.byref(u), C.byref(d), act, off, st, n, FAKE, FAKE,
                 ws_, None)

    assert call(H=2048) == moe.EINVAL and "shape" in _err()
    assert call(u=_w(moe.FMT_MXFP4)) == moe.EUNSUPPORTED
    assert call(u=_w(cb=FAKE + 1024)) == moe.EUNSUPPORTED and "codebook" in _err()
    assert call(g=_w(scales=None), u=_w(scales=None)) == moe.EINVAL
    assert call(g=_w(data=FAKE + 8), u=_w(data=FAKE + 8)) == moe.EINVAL
    bad = _w(moe.FMT_VQ2, 8, 2048, 4000)
    assert call(g=bad, u=bad, H=4000) == moe.EINVAL
    odd = _w(moe.FMT_BF16, 8, 2048, 3072, FAKE, None, None)
    dd = _w(moe.FMT_BF16, 8, 3072, 2048, FAKE, None, None)
    assert call(g=odd, u=odd, d=dd, H=3072) == moe.EUNSUPPORTED
    assert call(st=None) == moe.EINVAL
    assert call(ws_=ws - 1) == moe.ENOSPC
    assert call(off=None, n=5) == moe.EINVAL and "n_rows == T" in _err()
    assert call(n=0) == moe.OK
    # MX-FP8 activations: MXFP4 weights only, H and I multiples of 512
    assert call(act=moe.ACT_MXFP8) == moe.EUNSUPPORTED and "MX-FP8" in _err()
    assert call(act=7) == moe.EINVAL
    mg = _w(moe.FMT_MXFP4, 8, 2048, 4096, FAKE, FAKE, None)
    md = _w(moe.FMT_MXFP4, 8, 4096, 2048, FAKE, FAKE, None)
    ws8 = lib.moe_expert_ffn_workspace(1, 8, 8, 4096, 2048, moe.FMT_MXFP4, moe.FMT_MXFP4,
                                       moe.ACT_MXFP8)
    assert ws8 > lib.moe_expert_ffn_workspace(1, 8, 8, 4096, 2048, moe.FMT_MXFP4,
                                              moe.FMT_MXFP4, 0)
    assert call(g=mg, u=mg, d=md, act=moe.ACT_MXFP8, ws_=ws8 - 1) == moe.ENOSPC
    assert call(g=mg, u=mg, d=md, act=moe.ACT_MXFP8, n=0) == moe.OK
    q = lib.moe_mxfp8_quantize
    assert q(4, 100, FAKE, FAKE, FAKE, None) == moe.EINVAL
    assert q(4, 128, None, FAKE, FAKE, None) == moe.EINVAL
    assert q(0, 128, None, None, None, None) == moe.OK


def test_combine_and_dequantize_reject_bad_arguments():
    lib = _lib()
    c = lib.moe_combine
    assert c(4, 4096, 0, FAKE, FAKE, FAKE, None, None, 0.0, FAKE, None, None) == moe.EINVAL
    assert c(4, 4094, 8, FAKE, FAKE, FAKE, None, None, 0.0, FAKE, None, None) == moe.EINVAL
    assert c(4, 4096, 8, None, FAKE, FAKE, None, None, 0.0, FAKE, None, None) == moe.EINVAL
    assert c(4, 4096, 8, FAKE, FAKE, FAKE, None, FAKE + 4, 1.0, FAKE, None, None) == moe.EINVAL
    assert "misaligned" in _err()
    assert c(0, 4096, 8, None, None, None, None, None, 0.0, None, None, None) == moe.OK
    w = _w(moe.FMT_Q2K, 2, 64, 256, FAKE, None, None)
    dq = lib.moe_dequantize
    assert dq(C.byref(w), 2, 0, 10, FAKE, None) == moe.EINVAL
    assert dq(C.byref(w), 0, 64 * 256 - 5, 10, FAKE, None) == moe.EINVAL
    assert dq(C.byref(w), 0, 0, 0, FAKE, None) == moe.OK
    bad = _w(moe.FMT_Q2K, 1, 3, 100, FAKE, None, None)
    assert dq(C.byref(bad), 0, 0, 10, FAKE, None) == moe.EINVAL
    assert dq(C.byref(_w(fmt=9)), 0, 0, 10, FAKE, None) == moe.EUNSUPPORTED


def test_forward_validation_and_workspace_sizes():
    lib = _lib()
    g, u = _w(E=256), _w(E=256)
    d = _w(moe.FMT_Q2K, 256, 4096, 2048, FAKE, None, None)
    L = moe.Layer(4096, 2048, 256, 8, 2048, 0, FAKE, g, u, d, FAKE, FAKE, FAKE)
    ws1 = lib.moe_forward_workspace(C.byref(L), 1)
    ws2048 = lib.moe_forward_workspace(C.byref(L), 2048)
    assert 0 < ws1 < ws2048
    f = lib.moe_forward

    def call(L=L, T=1, ws=ws1, side=None):
        return f(C.byref(L), T, FAKE, None, None, FAKE, None, None, None, FAKE, ws,
                 None if side is None else C.byref(side), FAKE + 256)

    assert call(ws=ws1 - 1) == moe.ENOSPC
    assert f(C.byref(L), 0, None, None, None, None, None, None, None, None, 0, None, None) == moe.OK
    Lh = moe.Layer(4096, 2048, 256, 8, 2048, 1, FAKE, g, u, d, FAKE, FAKE, FAKE)
    assert call(Lh) == moe.EINVAL
    Lk = moe.Layer(4096, 2048, 256, 0, 2048, 0, FAKE, g, u, d, FAKE, FAKE, FAKE)
    assert call(Lk) == moe.EINVAL
    # the caller's second stream: all three handles, and not the call's own stream
    assert call(side=moe.SideStream(FAKE, FAKE, None)) == moe.EINVAL and "side" in _err()
    assert call(side=moe.SideStream(FAKE + 256, FAKE, FAKE)) == moe.EINVAL
    # the fp32 trace is for moe_expert_ffn only
    mg = _w(moe.FMT_MXFP4, 256, 2048, 4096, FAKE, FAKE, None)
    md = _w(moe.FMT_MXFP4, 256, 4096, 2048, FAKE, FAKE, None)
    La = moe.Layer(4096, 2048, 256, 8, 2048, 0, FAKE, mg, mg, md, FAKE, FAKE, FAKE,
                   moe.ACT_MXFP8 | moe.ACT_TRACE, None, 0.0)
    assert call(La, ws=lib.moe_forward_workspace(C.byref(La), 1)) == moe.EINVAL
        # a steering direction must be 16-byte aligned
    Ls = moe.Layer(4096, 2048, 256, 8, 2048, 0, FAKE, g, u, d, FAKE, FAKE, FAKE, 0, FAKE + 8, 1.0)
    assert call(Ls) == moe.EINVAL and "steer" in _err()


def test_a8_layout_inside_the_workspace():
    lib = _lib()
    for T, n, E, H, I in [(1, 8, 256, 4096, 2048), (4096, 32768, 256, 4096, 2048),
                          (3, 6, 8, 512, 512)]:
        co, so, fo = C.c_size_t(0), C.c_size_t(0), C.c_size_t(0)
        assert lib.moe_expert_ffn_a8_layout(T, n, E, H, I, C.byref(co), C.byref(so),
                                            C.byref(fo)) == moe.OK
        ws = lib.moe_expert_ffn_workspace(T, n, E, H, I, moe.FMT_MXFP4, moe.FMT_MXFP4,
                                          moe.ACT_MXFP8)
        assert ws == lib.moe_expert_ffn_workspace(T, n, E, H, I, moe.FMT_MXFP4, moe.FMT_MXFP4,
                                                  moe.ACT_MXFP8 | moe.ACT_TRACE)
        assert co.value % 256 == 0 and so.value % 256 == 0 and fo.value % 256 == 0
        assert co.value + n * I <= so.value and so.value + n * I // 32 <= ws
        # the fp32 trace lies before the MX-FP8 region, clear of it
        assert fo.value + 4 * n * I <= co.value
    co = C.c_size_t(0)
    assert lib.moe_expert_ffn_a8_layout(1, 8, 8, 512, 100, C.byref(co), C.byref(co),
                                        C.byref(co)) == moe.EINVAL
    assert lib.moe_expert_ffn_a8_layout(1, 8, 8, 512, 512, None, C.byref(co),
                                        C.byref(co)) == moe.EINVAL


def test_binding_refuses_host_tensors():
    import torch
    _lib()
    with pytest.raises(TypeError):
        moe.dispatch(torch.zeros((4, 2), dtype=torch.int32), 8)


def test_check_buckets():
    """moe_check_buckets (host only) accepts the oracle's dispatch of random
    and edge-case choices and names the first fault of each planted error."""
    _lib()
    import numpy as np

    import oracle

    rng = np.random.default_rng(3)
    for T, E, k in [(1, 8, 2), (37, 16, 4), (300, 256, 8), (5, 1024, 16)]:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        if T > 1:
            idx[0] = np.arange(k) % E  # distinct choices of token 0; repeats elsewhere
        off, st, _, sp = oracle.dispatch(idx, E)
        moe.check_buckets(T, E, k, T * k, off, st, sp)
        moe.check_buckets(T, E, k, T * k, off)  # offsets alone
    T, E, k = 37, 16, 4
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    off, st, _, sp = oracle.dispatch(idx, E)
    n = T * k

    def bad(msg, o=off, s=st, p=sp, nr=n):
        with pytest.raises(moe.MoeError) as ei:
            moe.check_buckets(T, E, k, nr, o, s, p)
        assert ei.value.code == moe.EINVAL and msg in str(ei.value), str(ei.value)

    o = off.copy(); o[0] = 1
    bad("expert_offsets[0] = 1", o=o)
    o = off.copy(); e = int(np.argmax(np.diff(off) > 0)); o[e + 1] = o[e] - 1
    bad(f"expert_offsets decreases at {e}", o=o)
    bad(f"expert_offsets[E] = {n}, not n_rows = {n + 1}", nr=n + 1, s=np.append(st, 0), p=None)
    s = st.copy(); s[5] = T
    bad(f"sorted_token[5] = {T} outside", s=s)
    s = st.copy(); s[9] = -1
    bad("sorted_token[9] = -1 outside", s=s)
    p = sp.copy(); p[7] = n
    bad(f"slot_pos[7] = {n} outside", p=p)
    p = sp.copy(); p[11] = p[3]
    bad("slot_pos[11]", p=p)
    bad("slot_pos needs T * k = n_rows", nr=n - 1, o=np.minimum(off, n - 1), s=st[:-1])

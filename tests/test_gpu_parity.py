"""GPU parity: libmoe's HIP kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs.

Bit-exact: dequantized weights, router logits, selected experts, bucket
arrays.  Floating point (routing weights, FFN rows, layer outputs): the
normwise relative error max|y - y_ref| / max|y_ref| must stay within 2e-3;
the weights within 1e-6 relative.
"""
import numpy as np
import pytest
import torch

import oracle
import routed_expert_ffn_router_amd as moe
import synth

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="session")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def tiny():
    return synth.gen_layer(synth.TINY, 0)


@pytest.fixture(scope="session")
def q2():
    return synth.gen_layer(synth.Q2, 0)


@pytest.fixture(scope="session")
def mx():
    return synth.gen_layer(synth.MX, 0)


@pytest.fixture(scope="session")
def dq2(q2, dev):
    return moe.DeviceLayer.upload(q2, device=dev)


@pytest.fixture(scope="session")
def dmx(mx, dev):
    return moe.DeviceLayer.upload(mx, device=dev)


def t16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)


def tnp(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def normwise(y, ref):
    ref = ref.astype(np.float64)
    return np.abs(y.astype(np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30)


def bits_equal(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32),
                          np.asarray(b, np.float32).view(np.uint32))


# --------------------------------------------------------------------------
# dequantization: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,N,K", [
    (synth.FMT_Q2K, 64, 1024), (synth.FMT_Q2K, 4, 128), (synth.FMT_Q2K, 7, 256),
    (synth.FMT_VQ2, 64, 1024), (synth.FMT_VQ2, 3, 256),
    (synth.FMT_MXFP4, 64, 1024), (synth.FMT_MXFP4, 5, 96),
    (synth.FMT_BF16, 16, 512),
])
def test_dequant_stress_bit_exact(dev, fmt, N, K):
    p = synth.gen_stress_proj(fmt, N, K, seed=N + K)
    got = tnp(moe.dequantize(moe.DeviceProj.upload(p, dev)))
    assert bits_equal(got, oracle.dequant(p))


@pytest.mark.parametrize("which,expert,w0,count", [
    ("gate", 0, 0, None), ("up", 255, 0, None), ("down", 7, 0, None),
    ("down", 100, 12345, 70001), ("gate", 31, 4096 * 7 + 3, 9999),
])
def test_dequant_layer_bit_exact(dev, q2, mx, which, expert, w0, count):
    for layer in (q2, mx):
        p = getattr(layer, which)
        dp = moe.DeviceProj.upload(p, dev)
        got = tnp(moe.dequantize(dp, expert, w0, count))
        assert bits_equal(got, oracle.dequant(p, expert, w0, count))


# --------------------------------------------------------------------------
# routing: logits and indices bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 4, 9, 37, 300, 2048])
def test_router_softmax_topk(dev, q2, T):
    x = synth.gen_x(4096, T, seed=100 + T)
    idx, w, lo = moe.route(t16(x, dev), t16(q2.w_router, dev), 8)
    ref_lo = oracle.router_logits(x, q2.w_router)
    assert bits_equal(tnp(lo), ref_lo)
    ref_idx, ref_w = oracle.select_topk(ref_lo, 8)
    assert np.array_equal(tnp(idx), ref_idx)
    np.testing.assert_allclose(tnp(w), ref_w, rtol=1e-6, atol=1e-7)


def test_router_tiny(dev, tiny):
    x = synth.gen_x(256, 4, seed=0)
    idx, w, lo = moe.route(t16(x, dev), t16(tiny.w_router, dev), 2)
    ref_idx, ref_w, ref_lo = oracle.LayerRef(tiny).route(x)
    assert bits_equal(tnp(lo), ref_lo)
    assert np.array_equal(tnp(idx), ref_idx)
    np.testing.assert_allclose(tnp(w), ref_w, rtol=1e-6)


@pytest.mark.parametrize("T", [1, 16, 4096])
def test_router_hash(dev, q2, T):
    x = synth.gen_x(4096, T, seed=7)
    tids = synth.gen_token_ids(T, seed=T)
    tids[0] = 0
    if T > 1:
        tids[1] = 129279
    idx, w, lo = moe.route(t16(x, dev), t16(q2.w_router, dev), 8, mode=moe.ROUTE_HASH,
                           token_ids=torch.from_numpy(tids).to(dev))
    ref_idx, ref_w = oracle.select_hash(tids, tnp(lo), 8)
    assert np.array_equal(tnp(idx), ref_idx)
    assert list(ref_idx[0]) == list(range(175, 183))
    np.testing.assert_allclose(tnp(w), ref_w, rtol=1e-6, atol=1e-7)


def test_router_logits_in_zipf_and_ties(dev):
    lg = synth.gen_zipf_logits(256, 16, 1.1, seed=0)
    lg[3, :] = 0.5  # a token whose logits all tie: experts 0..7
    lg[5, 10:20] = lg[5].max() + 1  # ten equal maxima
    lt = torch.from_numpy(lg).to(dev)
    idx, w, lo = moe.route(None, None, 8, logits_in=lt)
    ref_idx, ref_w = oracle.select_topk(lg, 8)
    assert np.array_equal(tnp(idx), ref_idx)
    assert list(ref_idx[3]) == list(range(8)) and list(ref_idx[5]) == list(range(10, 18))
    np.testing.assert_allclose(tnp(w), ref_w, rtol=1e-6)
    assert bits_equal(tnp(lo), lg)


# --------------------------------------------------------------------------
# dispatch: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (16, 256, 8), (37, 8, 2), (2048, 256, 8),
                                   (4096, 256, 8), (1000, 1024, 16), (300, 3, 3)])
def test_dispatch_bit_exact(dev, T, E, k):
    rng = np.random.default_rng(T * 31 + E)
    p = (np.arange(1, E + 1) ** -1.1)
    p /= p.sum()
    idx = np.array([rng.choice(E, k, replace=False, p=p) for _ in range(T)], np.int32)
    got = [tnp(a) for a in moe.dispatch(torch.from_numpy(idx).to(dev), E)]
    ref = oracle.dispatch(idx, E)
    for g, r, name in zip(got, ref, ["offsets", "sorted_token", "sorted_slot", "slot_pos"]):
        assert np.array_equal(g, r), name


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,H", [(1, 8, 4096), (16, 8, 4096), (300, 8, 256), (5, 2, 64)])
def test_combine(dev, T, k, H):
    rng = np.random.default_rng(T + k)
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    sp = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    out, ob = moe.combine(torch.from_numpy(y).to(dev), torch.from_numpy(sp).to(dev),
                          torch.from_numpy(w).to(dev), torch.from_numpy(sh).to(dev),
                          want_bf16=True)
    ref = oracle.combine(y, sp, w.reshape(T, k), sh)
    assert normwise(tnp(out), ref) < 1e-6
    rb = torch.from_numpy(tnp(out)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(tnp(ob), rb)


# --------------------------------------------------------------------------
# expert FFN (bucketed and dense)
# --------------------------------------------------------------------------

def _bucketed_ffn_case(layer, dl, dev, T, seed):
    R = oracle.LayerRef(layer)
    x = synth.gen_x(layer.spec.H, T, seed=seed)
    idx, w, _ = R.route(x)
    off, st, ss, sp = oracle.dispatch(idx, layer.spec.E)
    y = moe.expert_ffn(t16(x, dev), dl.gate, dl.up, dl.down, torch.from_numpy(off).to(dev),
                       torch.from_numpy(st).to(dev))
    return tnp(y), R.expert_ffn(x, off, st)


def test_expert_ffn_tiny(dev, tiny):
    dl = moe.DeviceLayer.upload(tiny, device=dev)
    y, ref = _bucketed_ffn_case(tiny, dl, dev, 4, 0)
    assert normwise(y, ref) < TOL


@pytest.mark.parametrize("T", [1, 3, 16])
def test_expert_ffn_q2(dev, q2, dq2, T):
    y, ref = _bucketed_ffn_case(q2, dq2, dev, T, 50 + T)
    assert normwise(y, ref) < TOL


@pytest.mark.parametrize("T", [1, 5])
def test_expert_ffn_mxfp4(dev, mx, dmx, T):
    y, ref = _bucketed_ffn_case(mx, dmx, dev, T, 60 + T)
    assert normwise(y, ref) < TOL


@pytest.mark.parametrize("T", [1, 4, 7])
def test_expert_ffn_dense_shared(dev, q2, dq2, T):
    x = synth.gen_x(4096, T, seed=T)
    sg = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, dq2.shared_gate)
    su = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, dq2.shared_up)
    sd = moe.DeviceProj(moe.FMT_BF16, 1, 4096, 2048, dq2.shared_down)
    y = tnp(moe.expert_ffn(t16(x, dev), sg, su, sd))
    ref = oracle.LayerRef(q2).shared_ffn(x)
    assert normwise(y, ref) < TOL


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------

def _forward_case(layer, dl, dev, T, seed, route=moe.ROUTE_SOFTMAX_TOPK, zipf=False, a8=False):
    x = synth.gen_x(layer.spec.H, T, seed=seed)
    lg = synth.gen_zipf_logits(layer.spec.E, T, 1.1, seed=seed) if zipf else None
    tids = synth.gen_token_ids(T, seed=seed) if route == moe.ROUTE_HASH else None
    ref, ref_idx, ref_w = oracle.LayerRef(layer, route_mode=route).forward(x, lg, tids, a8=a8)
    L = dl.with_route_mode(route)
    out, idx, w = moe.forward(L, t16(x, dev), None if lg is None else torch.from_numpy(lg).to(dev),
                              None if tids is None else torch.from_numpy(tids).to(dev))
    out, idx, w = tnp(out), tnp(idx), tnp(w)
    assert np.array_equal(idx, ref_idx)
    np.testing.assert_allclose(w, ref_w, rtol=1e-6, atol=1e-7)
    if a8:
        _assert_a8_close(layer, x, ref_idx, ref_w, out, ref)
    else:
        err = normwise(out, ref)
        assert err < TOL, err
    return out


def test_forward_tiny(dev, tiny):
    dl = moe.DeviceLayer.upload(tiny, device=dev)
    for T in (1, 4, 13):
        _forward_case(tiny, dl, dev, T, seed=T)


def test_forward_decode_b1(dev, q2, dq2):
    for seed in range(3):
        _forward_case(q2, dq2, dev, 1, seed)


# one-token layers of other shapes: H 2048, I 4096, no shared expert, a wide
# shared expert whose rows take several rounds of p2's waves, MXFP4 with hash
# routing, few experts and odd k
_DECODE_SHAPES = [
    ("h2048_k1_shared4096", 2048, 2048, 8, 1, "vq2", "vq2", "q2k", 4096),
    ("h2048_i4096_noshared", 2048, 4096, 16, 4, "vq2", "vq2", "q2k", 0),
    ("h2048_e16_k6", 2048, 2048, 16, 6, "vq2", "vq2", "q2k", 2048),
    ("h2048_mxfp4", 2048, 2048, 12, 3, "mxfp4", "mxfp4", "mxfp4", 2048),
    ("h4096_bf16_down", 4096, 2048, 8, 2, "vq2", "vq2", "bf16", 2048),
    # the other gate/up formats of the selection-and-gate/up launch, and VQ2 down
    ("h2048_q2k_gateup", 2048, 2048, 8, 2, "q2k", "q2k", "q2k", 2048),
    ("h2048_bf16_gateup_vq2_down", 2048, 2048, 8, 2, "bf16", "bf16", "vq2", 2048),
]
_FMT = {"bf16": synth.FMT_BF16, "q2k": synth.FMT_Q2K, "vq2": synth.FMT_VQ2,
        "mxfp4": synth.FMT_MXFP4}


@pytest.mark.parametrize("shape", _DECODE_SHAPES, ids=[c[0] for c in _DECODE_SHAPES])
def test_forward_decode_shapes(dev, shape):
    name, H, I, E, k, fg, fu, fd, Is = shape
    spec = synth.LayerSpec(name, H, I, E, k, _FMT[fg], _FMT[fu], _FMT[fd], Is)
    layer = synth.gen_layer(spec, seed=11)
    dl = moe.DeviceLayer.upload(layer, device=dev)
    for seed in range(2):
        _forward_case(layer, dl, dev, 1, 500 + seed)
    if fg == "mxfp4":
        _forward_case(layer, dl, dev, 1, 510, route=moe.ROUTE_HASH)


def test_forward_decode_b16_zipf(dev, q2, dq2):
    _forward_case(q2, dq2, dev, 16, 0, zipf=True)


@pytest.mark.parametrize("T", [2, 64, 200])
def test_forward_q2_batches(dev, q2, dq2, T):
    _forward_case(q2, dq2, dev, T, 1000 + T)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_mxfp4_decode(dev, mx, dmx, route):
    _forward_case(mx, dmx, dev, 1, 3, route=route)
    _forward_case(mx, dmx, dev, 9, 4, route=route)


def _decode_select_cases(E):
    """Logit rows for one-token selection edge cases (E >= 32)."""
    rng = np.random.default_rng(77)
    rows = []
    rows.append(np.full(E, 0.5, np.float32))                 # all tie: 0..7
    r = rng.standard_normal(E).astype(np.float32)
    r[10:20] = r.max() + 1                                   # ten equal maxima
    rows.append(r)
    r = rng.standard_normal(E).astype(np.float32)
    r[::3] = np.nan                                          # NaN ranks as -inf
    rows.append(r)
    r = np.full(E, -np.inf, np.float32)
    r[[E - 1, 7, 130 % E, 64 % E, 3]] = [2.0, 1.0, 1.0, -0.0, 0.0]  # 5 finite, -0 ties +0
    r[[11, 12]] = np.nan
    rows.append(r)
    r = rng.standard_normal(E).astype(np.float32)
    r[[5, 69 % E, 133 % E, 197 % E]] = 9.0                   # one tie per lane slot
    rows.append(r)
    rows.append(-np.abs(rng.standard_normal(E)).astype(np.float32))
    return rows


def test_forward_decode_b1_selection_edges(dev, q2, dq2):
    """One-token forward with given logits: the choices and weights equal the
    oracle's selection and the batched moe_route's bit for bit, on ties,
    NaNs, -inf, signed zeros and ties across lane slots."""
    E = 256
    x = t16(synth.gen_x(4096, 1, seed=9), dev)
    for n, row in enumerate(_decode_select_cases(E)):
        lg = row[None, :].copy()
        lt = torch.from_numpy(lg).to(dev)
        _, idx, w = moe.forward(dq2, x, logits_in=lt)
        ref_idx, ref_w = oracle.select_topk(lg, 8)
        assert np.array_equal(tnp(idx).reshape(1, 8), ref_idx), (n, tnp(idx), ref_idx)
        np.testing.assert_allclose(tnp(w).reshape(1, 8), ref_w, rtol=1e-6, err_msg=str(n))
        idx2, w2, _ = moe.route(None, None, 8, logits_in=lt)
        assert np.array_equal(tnp(idx).reshape(1, 8), tnp(idx2)), n
        assert bits_equal(tnp(w).reshape(1, 8), tnp(w2)), n


def _graph_replays(f, xs, tids=None):
    """Capture one forward in a HIP graph, replay it once per input with
    eager work and synchronisations between the replays; every replay must
    equal the eager run of the same input bit for bit."""
    refs = []
    for i, x in enumerate(xs):
        f(x, None, None if tids is None else tids[i])
        torch.cuda.synchronize()
        refs.append((f.out.clone(), f.idx.clone(), f.w.clone()))
    xb = xs[0].clone()
    tb = None if tids is None else tids[0].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f(xb, None, tb)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f(xb, None, tb)
    for rep in range(2):
        for i, x in enumerate(xs):
            xb.copy_(x)
            if tb is not None:
                tb.copy_(tids[i])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(f.out, refs[i][0]), (rep, i)
            assert torch.equal(f.idx, refs[i][1]) and torch.equal(f.w, refs[i][2]), (rep, i)
            f(xs[(i + 1) % len(xs)], None, None if tids is None else tids[(i + 1) % len(xs)])
            torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 16, 300])
def test_forward_graph_replay(dev, q2, dq2, T):
    f = moe.Forward(dq2, T, dev)
    xs = [t16(synth.gen_x(4096, T, seed=300 + 7 * T + i), dev) for i in range(3)]
    _graph_replays(f, xs)


def test_forward_graph_replay_mxfp4_hash_a8(dev, mx, dmx):
    """Hash routing with MX-FP8 activations (quantization pass + FP4 MFMA)."""
    layer = dmx.with_route_mode(moe.ROUTE_HASH).with_act(moe.ACT_MXFP8)
    T = 40
    f = moe.Forward(layer, T, dev)
    xs = [t16(synth.gen_x(4096, T, seed=400 + i), dev) for i in range(3)]
    tids = [torch.from_numpy(synth.gen_token_ids(T, 0, i)).to(dev) for i in range(3)]
    _graph_replays(f, xs, tids)


def test_forward_deterministic(dev, q2, dq2):
    x = t16(synth.gen_x(4096, 16, seed=5), dev)
    a, _, _ = moe.forward(dq2, x)
    b, _, _ = moe.forward(dq2, x)
    assert np.array_equal(tnp(a).view(np.uint32), tnp(b).view(np.uint32))


def test_forward_equals_composed_calls(dev, q2, dq2):
    """moe_forward vs moe_route -> moe_dispatch -> moe_expert_ffn x2 -> moe_combine."""
    T = 24
    x = t16(synth.gen_x(4096, T, seed=8), dev)
    out, idx, w = moe.forward(dq2, x)
    idx2, w2, _ = moe.route(x, dq2.w_router, 8)
    off, st, ss, sp = moe.dispatch(idx2, 256)
    y = moe.expert_ffn(x, dq2.gate, dq2.up, dq2.down, off, st)
    sg = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, dq2.shared_gate)
    su = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, dq2.shared_up)
    sd = moe.DeviceProj(moe.FMT_BF16, 1, 4096, 2048, dq2.shared_down)
    sh = moe.expert_ffn(x, sg, su, sd)
    out2, _ = moe.combine(y, sp, w2, sh)
    assert np.array_equal(tnp(idx), tnp(idx2))
    assert normwise(tnp(out2), tnp(out).astype(np.float64)) < 1e-5


# --------------------------------------------------------------------------
# prefill: the grouped-GEMM path (buckets of several rows per expert).
# The oracle runs on sampled rows/tokens: a row of the expert FFN depends only
# on its token and expert, a token's output only on its own input.
# --------------------------------------------------------------------------

def _sub_buckets(off, st, rows):
    """The bucket arrays restricted to `rows` (bucket positions), in bucket order."""
    rows = np.unique(np.asarray(rows))
    e_of = np.searchsorted(off, rows, side="right") - 1
    cnt = np.bincount(e_of, minlength=len(off) - 1)
    sub_off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    return rows, sub_off, st[rows].astype(np.int32)


def _gemm_rows_case(layer, dl, dev, x, off, st, n_sample, seed):
    """expert_ffn over (off, st) on the GPU; sampled rows against the oracle."""
    n = int(off[-1])
    y = tnp(moe.expert_ffn(t16(x, dev), dl.gate, dl.up, dl.down, torch.from_numpy(off).to(dev),
                           torch.from_numpy(st).to(dev)))
    assert y.shape == (n, layer.spec.H) and np.isfinite(y).all()
    rng = np.random.default_rng(seed)
    # both ends of every tile boundary region, plus random rows
    ends = np.concatenate([off[:-1][np.diff(off) > 0], off[1:][np.diff(off) > 0] - 1])
    rows = np.concatenate([rng.choice(ends, min(len(ends), n_sample // 2), replace=False),
                           rng.choice(n, n_sample // 2, replace=False), [0, n - 1]])
    rows, sub_off, sub_st = _sub_buckets(off, st, rows)
    ref = oracle.LayerRef(layer).expert_ffn(x, sub_off, sub_st)
    return normwise(y[rows], ref)


@pytest.mark.parametrize("T", [4, 16, 128, 161, 3072])
def test_expert_ffn_gemm_q2(dev, q2, dq2, T):
    x = synth.gen_x(4096, T, seed=70 + T)
    idx, _, _ = oracle.LayerRef(q2).route(x)
    off, st, _, _ = oracle.dispatch(idx, 256)
    assert _gemm_rows_case(q2, dq2, dev, x, off, st, 48, T) < TOL


@pytest.mark.parametrize("T", [40, 300, 1100])
def test_expert_ffn_gemm_q2k_gateup(dev, T):
    """Q2K gate, up and down on the GEMM path (16- and 64-row tiles, up to
    four tiles per expert)."""
    spec = synth.LayerSpec("q2k_gemm", 512, 256, 8, 2, synth.FMT_Q2K, synth.FMT_Q2K,
                           synth.FMT_Q2K, 256)
    layer = synth.gen_layer(spec, seed=7)
    dl = moe.DeviceLayer.upload(layer, device=dev)
    y, ref = _bucketed_ffn_case(layer, dl, dev, T, 100 + T)
    assert normwise(y, ref) < TOL


def test_expert_ffn_gemm_mxfp4(dev, mx, dmx):
    T = 150
    x = synth.gen_x(4096, T, seed=80)
    idx, _, _ = oracle.LayerRef(mx).route(x)
    off, st, _, _ = oracle.dispatch(idx, 256)
    assert _gemm_rows_case(mx, dmx, dev, x, off, st, 48, 81) < TOL


def test_expert_ffn_gemm_ragged_buckets(dev, q2, dq2):
    """Hand-made bucket sizes around the 64-row tile: 0, 1, 63, 64, 65, 127, 128, 129, ..."""
    sizes = np.array([0, 1, 63, 64, 65, 127, 128, 129, 2, 0, 31, 3] * 22)[:256]
    assert sizes.sum() >= 4 * 256
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = 97
    st = np.random.default_rng(5).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.gen_x(4096, T, seed=90)
    assert _gemm_rows_case(q2, dq2, dev, x, off, st, 64, 91) < TOL


def test_expert_ffn_gemm_ragged_buckets_128(dev, q2, dq2):
    """Bucket sizes around 128 rows (up to three 64-row tiles per expert)."""
    sizes = np.array([0, 1, 127, 128, 129, 255, 256, 257, 95, 96, 97, 300] * 22)[:256]
    assert sizes.sum() >= 96 * 256
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = 97
    st = np.random.default_rng(6).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.gen_x(4096, T, seed=92)
    assert _gemm_rows_case(q2, dq2, dev, x, off, st, 64, 93) < TOL


@pytest.mark.parametrize("T", [2, 16, 33, 64, 97, 1100])
def test_expert_ffn_dense_shared_gemm(dev, q2, dq2, T):
    x = synth.gen_x(4096, T, seed=T)
    sg = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, dq2.shared_gate)
    su = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, dq2.shared_up)
    sd = moe.DeviceProj(moe.FMT_BF16, 1, 4096, 2048, dq2.shared_down)
    y = tnp(moe.expert_ffn(t16(x, dev), sg, su, sd))
    ref = oracle.LayerRef(q2).shared_ffn(x)
    assert normwise(y, ref) < TOL


def _forward_sampled(layer, dl, dev, T, seed, n_sample, route=moe.ROUTE_SOFTMAX_TOPK,
                     zipf=False, a8=False):
    """Full-size forward on the GPU; routing of every token bit-exact against the
    oracle, outputs of sampled tokens within the tolerance."""
    x = synth.gen_x(layer.spec.H, T, seed=seed)
    lg = synth.gen_zipf_logits(layer.spec.E, T, 1.1, seed=seed) if zipf else None
    tids = synth.gen_token_ids(T, seed=seed) if route == moe.ROUTE_HASH else None
    L = dl.with_route_mode(route)
    out, idx, w = moe.forward(L, t16(x, dev), None if lg is None else torch.from_numpy(lg).to(dev),
                              None if tids is None else torch.from_numpy(tids).to(dev))
    out, idx, w = tnp(out), tnp(idx), tnp(w)
    assert np.isfinite(out).all()
    R = oracle.LayerRef(layer, route_mode=route)
    ridx, rw, _ = R.route(x, lg, tids)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(w, rw, rtol=1e-6, atol=1e-7)
    rng = np.random.default_rng(seed + 1)
    sel = np.unique(np.concatenate([[0, T - 1], rng.choice(T, n_sample - 2, replace=False)]))
    ref, _, _ = R.forward(x[sel], None if lg is None else lg[sel],
                          None if tids is None else tids[sel], a8=a8)
    if a8:
        _assert_a8_close(layer, x[sel], idx[sel], w[sel], out[sel], ref)
    else:
        err = normwise(out[sel], ref)
        assert err < TOL, err


def test_forward_prefill_2048(dev, q2, dq2):
    _forward_sampled(q2, dq2, dev, 2048, 2048, 8)


def test_forward_q2_zipf_gemm(dev, q2, dq2):
    _forward_sampled(q2, dq2, dev, 256, 77, 8, zipf=True)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_mxfp4_prefill_4096(dev, mx, dmx, route):
    _forward_sampled(mx, dmx, dev, 4096, 4096 + route, 6, route=route)


# --------------------------------------------------------------------------
# MX-FP8 activations on the FP4 matrix instructions (the A8 variant)
#
# The tokens' quantization is compared bit-exact (same inputs on both sides).
# The SwiGLU output is quantized from values the GPU accumulates in fp32 and
# the oracle in fp64 (where every product and sum is exact), so an element
# lying within fp32 error of an E4M3 rounding midpoint may take either
# neighbouring code on the GPU -- both are correct A8 results.  The layer
# output is therefore compared elementwise within TOL * max|ref| plus the
# most those ambiguous decisions can move it: for each ambiguous element,
# one E4M3 step times |W_down| times the routing weight (a group whose
# largest magnitude is that close to a power of two may also take the
# neighbouring scale).  Everything else must agree to TOL.
# --------------------------------------------------------------------------

_E4M3 = None


def _e4m3_values():
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([oracle.e4m3(c) for c in range(256)], np.float64)
    return _E4M3


def _chunked_error(X, W, chunk=32):
    """Rounding-error bound of a product X W^T accumulated in fp32 with a
    rounding at most every 32 products (one E8M0 scale block; each FP4
    matrix instruction sums 4 of them): every chunk's sum rounded once and
    added to the running fp32 sum with one more rounding:
    2^-24 (sum_c |chunk sum_c| + sum_c |running sum_c|)."""
    K = X.shape[1]
    run = np.zeros((X.shape[0], W.shape[0]))
    bound = np.zeros_like(run)
    for c in range(0, K, chunk):
        part = X[:, c:c + chunk] @ W[:, c:c + chunk].T
        run += part
        bound += np.abs(part) + np.abs(run)
    return 2.0 ** -24 * bound


def _a8_ambiguity(layer, x, idx, w):
    """[T][H] bound on the output change from ambiguous MX-FP8 decisions on
    the SwiGLU output (see above).  The GPU's gate/up sums may differ from
    the exact ones by twice the accumulation bound of _chunked_error; the
    SwiGLU in fp32 adds 2^-20 relative."""
    spec = layer.spec
    H, I = spec.H, spec.I
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    codes, sc = oracle.mxfp8_quant(xv)
    xq = _e4m3_values()[codes] * np.exp2(np.repeat(sc.astype(np.float64) - 127.0, 32, axis=1))
    T = x.shape[0]
    B = np.zeros((T, H))
    pairs = {}
    for t in range(T):
        for j in range(idx.shape[1]):
            pairs.setdefault(int(idx[t, j]), []).append((t, j))
    n_amb = 0
    for e, tj in pairs.items():
        G = oracle.dequant_matrix(layer.gate, e).astype(np.float64)
        U = oracle.dequant_matrix(layer.up, e).astype(np.float64)
        D = np.abs(oracle.dequant_matrix(layer.down, e).astype(np.float64))
        X = xq[[t for t, _ in tj]]
        g, u = X @ G.T, X @ U.T
        eg, eu = 2 * _chunked_error(X, G), 2 * _chunked_error(X, U)
        sig = 1.0 / (1.0 + np.exp(-g))
        silu = g * sig
        a = silu * u
        da = (np.abs(sig * (1 + g * (1 - sig))) * eg * np.abs(u) + np.abs(silu) * eu
              + 2.0 ** -20 * np.abs(a))
        n = len(tj)
        ag, dg = np.abs(a).reshape(n, I // 32, 32), da.reshape(n, I // 32, 32)
        amax = ag.max(axis=2)
        safe = np.where(amax > 0, amax, 1.0)
        Xs = np.exp2(np.clip(np.floor(np.log2(safe)) - 8, -127, 127))[:, :, None]
        y = ag / Xs
        step = np.exp2(np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3)
        dist = np.abs(y / step - np.floor(y / step) - 0.5) * step * Xs
        delta = np.where((dist <= dg) & (y < 448), step * Xs, 0.0)
        p2 = np.exp2(np.round(np.log2(safe)))
        damax = np.take_along_axis(dg, ag.argmax(axis=2)[:, :, None], 2)[:, :, 0]
        samb = (amax > 0) & (np.abs(amax - p2) <= damax)
        delta = np.where(samb[:, :, None], 0.25 * ag + 2 * step * Xs, delta)
        n_amb += int((delta > 0).sum())
        contrib = delta.reshape(n, I) @ D.T
        for r, (t, j) in enumerate(tj):
            B[t] += float(w[t, j]) * contrib[r]
    return B, n_amb


def _assert_a8_close(layer, x, idx, w, out, ref):
    B, n_amb = _a8_ambiguity(layer, x, idx, w)
    base = TOL * np.abs(ref).max()
    excess = np.abs(out.astype(np.float64) - ref) - (base + B)
    assert (excess <= 0).all(), (float(excess.max()), normwise(out, ref), n_amb)
    # the ambiguous decisions are a small minority of the SwiGLU elements
    assert n_amb <= 0.01 * x.shape[0] * idx.shape[1] * layer.spec.I, n_amb

def _bf16_round(v):
    """fp32 -> bf16 bit patterns, round to nearest even (no NaNs here)."""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_mxfp8_quantize_bit_exact(dev):
    """Codes and scales of the device quantizer equal the oracle's, on wide
    magnitude ranges and hand-made groups: all zeros, saturation (scaled
    values in [448, 512)), ties between E4M3 neighbours (normal and
    subnormal), signed values, bf16 subnormals."""
    rng = np.random.default_rng(7)
    rows, K = 96, 1024
    v = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-30, 30, (rows, 1)))).astype(np.float32)
    v[0, :32] = 0.0
    v[1, :32] = 496.0 * (1 - 2 * (np.arange(32) % 2))       # amax 496: X = 1, all saturate
    v[2, :32] = 1.0                                          # X = 2^-8
    g = np.zeros(32, np.float32)                             # X = 1 (amax 256): exact ties
    g[:8] = [256.0, 1.0625, 1.1875, -1.0625, 3 * 2.0 ** -10, 5 * 2.0 ** -10, 2.0 ** -9, 15.5]
    v[3, :32] = g
    v[4, :32] = np.float32(2.0 ** -130) * (1 + np.arange(32) % 3)   # bf16 subnormals
    v[5, :] = -np.abs(v[5, :])
    bits = _bf16_round(v)
    q, sc = moe.mxfp8_quantize(t16(bits, dev))
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    rq, rs = oracle.mxfp8_quant(vals)
    assert np.array_equal(tnp(sc), rs)
    assert np.array_equal(tnp(q), rq)


@pytest.mark.parametrize("T", [1, 3, 40, 300])
def test_forward_mxfp4_a8(dev, mx, dmx, T):
    _forward_case(mx, dmx.with_act(moe.ACT_MXFP8), dev, T, 500 + T, a8=True)


def test_forward_mxfp4_a8_hash(dev, mx, dmx):
    _forward_case(mx, dmx.with_act(moe.ACT_MXFP8), dev, 100, 601, route=moe.ROUTE_HASH, a8=True)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_mxfp4_a8_prefill_4096(dev, mx, dmx, route):
    _forward_sampled(mx, dmx.with_act(moe.ACT_MXFP8), dev, 4096, 7000 + route, 6, route=route,
                     a8=True)


def test_forward_a8_equals_composed_calls(dev, mx, dmx):
    """moe_forward with MX-FP8 activations vs the four calls with act_fmt set."""
    T = 70
    L = dmx.with_act(moe.ACT_MXFP8)
    x = t16(synth.gen_x(4096, T, seed=9), dev)
    out, idx, w = moe.forward(L, x)
    idx2, w2, _ = moe.route(x, L.w_router, 8)
    off, st, ss, sp = moe.dispatch(idx2, 256)
    y = moe.expert_ffn(x, L.gate, L.up, L.down, off, st, act=moe.ACT_MXFP8)
    sg = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, L.shared_gate)
    su = moe.DeviceProj(moe.FMT_BF16, 1, 2048, 4096, L.shared_up)
    sd = moe.DeviceProj(moe.FMT_BF16, 1, 4096, 2048, L.shared_down)
    sh = moe.expert_ffn(x, sg, su, sd)
    out2, _ = moe.combine(y, sp, w2, sh)
    assert np.array_equal(tnp(idx), tnp(idx2))
    assert normwise(tnp(out2), tnp(out).astype(np.float64)) < 1e-5

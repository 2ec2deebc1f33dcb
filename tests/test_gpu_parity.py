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


@pytest.mark.parametrize("mode", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_router_screened_no_logits(dev, q2, mode):
    """moe_route without a logits output at 2048 tokens takes the screened
    router: the same indices and weights as the oracle's exact logits."""
    T = 2048
    x = synth.gen_x(4096, T, seed=111)
    tids = synth.gen_token_ids(T, seed=112) if mode == moe.ROUTE_HASH else None
    idx, w, lo = moe.route(t16(x, dev), t16(q2.w_router, dev), 8, mode=mode,
                           token_ids=None if tids is None else torch.from_numpy(tids).to(dev),
                           want_logits=False)
    assert lo is None
    ref_lo = oracle.router_logits(x, q2.w_router)
    if mode == moe.ROUTE_HASH:
        ref_idx, ref_w = oracle.select_hash(tids, ref_lo, 8)
    else:
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
    # the host-side bucket check accepts the device's bucketing
    moe.check_buckets(T, E, k, T * k, got[0], got[1], got[3])


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,H", [(1, 8, 4096), (16, 8, 4096), (300, 8, 256), (5, 2, 64)])
@pytest.mark.parametrize("shared,steer", [(True, False), (False, False), (True, True),
                                          (False, True)])
def test_combine(dev, T, k, H, shared, steer):
    """Bit-equal to the oracle's combine: both sum in fp64 in the same order
    (shared, then j, then the steering term), every product exact."""
    rng = np.random.default_rng(T + k)
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    sp = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32) if shared else None
    d = rng.standard_normal(H).astype(np.float32) if steer else None
    alpha = -1.75 if steer else 0.0
    out, ob = moe.combine(torch.from_numpy(y).to(dev), torch.from_numpy(sp).to(dev),
                          torch.from_numpy(w).to(dev),
                          None if sh is None else torch.from_numpy(sh).to(dev), want_bf16=True,
                          steer_dir=None if d is None else torch.from_numpy(d).to(dev),
                          steer_alpha=alpha)
    ref = oracle.combine(y, sp, w.reshape(T, k), sh, d, alpha)
    assert bits_equal(tnp(out), ref)
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
    R = oracle.LayerRef(layer, route_mode=route)
    if a8:  # the A8 check runs the oracle's layer itself, where it applies
        ref_idx, ref_w, _ = R.route(x, lg, tids)
    else:
        ref, ref_idx, ref_w = R.forward(x, lg, tids)
    L = dl.with_route_mode(route)
    out, idx, w = moe.forward(L, t16(x, dev), None if lg is None else torch.from_numpy(lg).to(dev),
                              None if tids is None else torch.from_numpy(tids).to(dev))
    out, idx, w = tnp(out), tnp(idx), tnp(w)
    assert np.array_equal(idx, ref_idx)
    np.testing.assert_allclose(w, ref_w, rtol=1e-6, atol=1e-7)
    if a8:
        _assert_a8_forward(layer, L, dev, x, ref_idx, ref_w, out, route, lg, tids)
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


@pytest.mark.parametrize("fmt", ["q2", "mx"])
def test_expert_ffn_gemm_ragged_buckets_64(dev, q2, dq2, mx, dmx, fmt):
    """Bucket sizes around the 64-row tile, 33..48 rows per active expert on
    average (VQ2 / Q2K: the register-staged tiles; MXFP4: the direct-load
    ones)."""
    layer, dl = (q2, dq2) if fmt == "q2" else (mx, dmx)
    sizes = np.array([0, 1, 31, 32, 33, 40, 47, 48, 49, 63, 64, 65] * 22)[:256]
    active = (sizes > 0).sum()
    assert 32 * active <= sizes.sum() <= 48 * active
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = 97
    st = np.random.default_rng(9).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.gen_x(4096, T, seed=98)
    assert _gemm_rows_case(layer, dl, dev, x, off, st, 64, 99) < TOL


def test_expert_ffn_gemm_ragged_buckets_96(dev, q2, dq2):
    """Bucket sizes around the 96- and 128-row tiles, 49..96 rows per active
    expert on average: one, two or three tiles per expert, each with one to
    three live 32-row blocks."""
    sizes = np.array([0, 1, 31, 32, 33, 64, 95, 96, 97, 128, 160, 193] * 22)[:256]
    active = (sizes > 0).sum()
    assert 48 * active < sizes.sum() <= 96 * active
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = 97
    st = np.random.default_rng(7).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.gen_x(4096, T, seed=94)
    assert _gemm_rows_case(q2, dq2, dev, x, off, st, 64, 95) < TOL


def test_expert_ffn_gemm_ragged_buckets_128_tiles(dev, q2, dq2):
    """Bucket sizes around the 128-row tile, more than 96 rows per active
    expert on average: one to three tiles per expert, one to four live
    32-row blocks each."""
    sizes = np.array([1, 32, 96, 97, 127, 128, 129, 160, 200, 255, 256, 257] * 22)[:256]
    assert sizes.sum() > 96 * (sizes > 0).sum()
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = 97
    st = np.random.default_rng(8).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.gen_x(4096, T, seed=96)
    assert _gemm_rows_case(q2, dq2, dev, x, off, st, 64, 97) < TOL


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
    # the first and last row of a few experts' buckets (tile edges), then random tokens
    off, st, _, _ = oracle.dispatch(idx, layer.spec.E)
    edges = []
    for e in rng.choice(layer.spec.E, 8, replace=False):
        if off[e + 1] > off[e]:
            edges += [st[off[e]], st[off[e + 1] - 1]]
    sel = np.unique(np.concatenate([[0, T - 1], edges,
                                    rng.choice(T, max(n_sample - 2 - len(edges), 1),
                                               replace=False)]))
    sub = (x[sel], None if lg is None else lg[sel], None if tids is None else tids[sel])
    if a8:
        _assert_a8_forward(layer, L, dev, x, idx, rw, out, route, lg, tids, sel=sel)
    else:
        ref, _, _ = R.forward(*sub)
        err = normwise(out[sel], ref)
        assert err < TOL, err


def test_forward_prefill_2048(dev, q2, dq2):
    _forward_sampled(q2, dq2, dev, 2048, 2048, 64)


def test_forward_q2_zipf_gemm(dev, q2, dq2):
    _forward_sampled(q2, dq2, dev, 256, 77, 8, zipf=True)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_mxfp4_prefill_4096(dev, mx, dmx, route):
    _forward_sampled(mx, dmx, dev, 4096, 4096 + route, 6, route=route)


# --------------------------------------------------------------------------
# MX-FP8 activations on the FP4 matrix instructions (the A8 variant)
#
# The tokens' quantization is compared bit-exact (same inputs on both sides).
# The SwiGLU output is quantized from values the GPU accumulates on the
# matrix cores in fp32 and the oracle in fp64, so an element near an E4M3
# rounding midpoint may take the neighbouring code on the GPU.  The check is
# made on the quantized SwiGLU output itself: with MOE_ACT_TRACE the GPU also
# leaves the fp32 values it quantized, and its codes and scales must equal
# the oracle quantizer's codes of those very values bit for bit; the values
# themselves must match the exact A8 SwiGLU output within the tolerance; the
# codes differing from those of the exact values must stay a small minority;
# and the layer's outputs must match, at the plain tolerance with no slack,
# the oracle's down projection and combine run on the GPU's own codes.
# --------------------------------------------------------------------------

_E4M3 = None


def _e4m3_values():
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([oracle.e4m3(c) for c in range(256)], np.float64)
    return _E4M3


def _a8_exact_rows(layer, x, off, st):
    """For every bucket row: the SwiGLU output a of its expert on the MX-FP8
    tokens in fp64 (exact products and sums)."""
    I = layer.spec.I
    xv = (x.astype(np.uint32) << 16).view(np.float32)
    codes, sc = oracle.mxfp8_quant(xv)
    xq = _e4m3_values()[codes] * np.exp2(np.repeat(sc.astype(np.float64) - 127.0, 32, axis=1))
    A = np.zeros((int(off[-1]), I))
    for e in range(len(off) - 1):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r0 == r1:
            continue
        G = oracle.dequant_matrix(layer.gate, e).astype(np.float64)
        U = oracle.dequant_matrix(layer.up, e).astype(np.float64)
        X = xq[st[r0:r1]]
        g, u = X @ G.T, X @ U.T
        A[r0:r1] = g / (1.0 + np.exp(-g)) * u
    return A


def _check_a8_codes(layer, x, off, st, gcodes, gscales, gvals):
    """The GPU's MX-FP8 SwiGLU output (codes, scales) must be exactly the
    oracle quantizer's codes of the fp32 values the GPU quantized (gvals,
    kept by MOE_ACT_TRACE) -- bit for bit -- and those values must equal the
    exact A8 SwiGLU output (fp64, same MX-FP8 tokens) within TOL normwise per
    row.  Returns the number of codes that differ from the codes of the exact
    values (decisions near an E4M3 rounding midpoint, an fp32 effect)."""
    rc, rs = oracle.mxfp8_quant(gvals)
    assert np.array_equal(gscales, rs), np.argwhere(gscales != rs)[:5]
    assert np.array_equal(gcodes, rc), np.argwhere(gcodes != rc)[:5]
    A = _a8_exact_rows(layer, x, off, st)
    err = np.abs(gvals.astype(np.float64) - A).max(1) / np.maximum(np.abs(A).max(1), 1e-30)
    assert err.max() < TOL, (err.max(), err.argmax())
    ec, es = oracle.LayerRef(layer).a8_swiglu_codes(x, off, st)
    vals = _e4m3_values()
    dv = (vals[gcodes] * np.exp2(np.repeat(gscales.astype(np.float64) - 127, 32, 1))
          != vals[ec] * np.exp2(np.repeat(es.astype(np.float64) - 127, 32, 1)))
    n_diff = int(dv.sum())
    assert n_diff <= 0.01 * gcodes.size, n_diff
    return n_diff


def _assert_a8_forward(layer, dl, dev, x, idx, w, out, route=moe.ROUTE_SOFTMAX_TOPK, lg=None,
                       tids=None, sel=None):
    """The A8 layer output of tokens `sel` (all when None) against the oracle.
    moe_expert_ffn with MX-FP8 activations runs on the whole batch's buckets
    (the same kernels and inputs as the layer's own call, plus the fp32
    trace of the SwiGLU output); the quantized SwiGLU rows of the selected
    tokens are checked by _check_a8_codes, their y_rows against the oracle's
    down projection of the GPU's codes, and the output against the oracle's
    combine of those rows plus the shared expert -- both at TOL with no slack
    -- and against the oracle's own A8 forward when no code differs."""
    spec = layer.spec
    T, k = idx.shape
    sel = np.arange(T) if sel is None else np.asarray(sel)
    off, st, _, sp = oracle.dispatch(idx, spec.E)
    n = int(off[-1])
    y, ws = moe.expert_ffn(t16(x, dev), dl.gate, dl.up, dl.down, torch.from_numpy(off).to(dev),
                           torch.from_numpy(st).to(dev), act=moe.ACT_MXFP8 | moe.ACT_TRACE,
                           keep_ws=True)
    gc, gs, gv = moe.a8_intermediate(ws, T, n, spec.E, spec.H, spec.I)
    gc, gs, gv, y = tnp(gc), tnp(gs), tnp(gv), tnp(y)
    # the layer's own call (no trace) leaves the same codes: same kernels, same inputs
    y2 = tnp(moe.expert_ffn(t16(x, dev), dl.gate, dl.up, dl.down, torch.from_numpy(off).to(dev),
                            torch.from_numpy(st).to(dev), act=moe.ACT_MXFP8))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    rows, sub_off, sub_st = _sub_buckets(off, st, sp.reshape(T, k)[sel].reshape(-1))
    n_diff = _check_a8_codes(layer, x, sub_off, sub_st, gc[rows], gs[rows], gv[rows])
    R = oracle.LayerRef(layer, route_mode=route)
    y_ref = R.a8_down(sub_off, gc[rows], gs[rows])
    err = normwise(y[rows], y_ref)
    assert err < TOL, err
    sp_sub = np.searchsorted(rows, sp.reshape(T, k)[sel]).astype(np.int32)
    xs = x[sel]
    ref = oracle.combine(y_ref, sp_sub.reshape(-1), w[sel], R.shared_ffn(xs))
    err = normwise(out[sel], ref)
    assert err < TOL, (err, n_diff)
    if n_diff == 0:
        ref2, _, _ = R.forward(xs, None if lg is None else lg[sel],
                               None if tids is None else tids[sel], a8=True)
        assert normwise(out[sel], ref2) < TOL


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


def _a8_rows_case(layer, dl, dev, x, off, st, rows):
    """moe_expert_ffn with MX-FP8 activations over the buckets (off, st); the
    bucket rows `rows`: their quantized SwiGLU output (_check_a8_codes) and
    their y rows against the oracle's down projection of the GPU's codes."""
    spec = layer.spec
    T, n = x.shape[0], int(off[-1])
    y, ws = moe.expert_ffn(t16(x, dev), dl.gate, dl.up, dl.down, torch.from_numpy(off).to(dev),
                           torch.from_numpy(st).to(dev), act=moe.ACT_MXFP8 | moe.ACT_TRACE,
                           keep_ws=True)
    gc, gs, gv = moe.a8_intermediate(ws, T, n, spec.E, spec.H, spec.I)
    gc, gs, gv, y = tnp(gc), tnp(gs), tnp(gv), tnp(y)
    y2 = tnp(moe.expert_ffn(t16(x, dev), dl.gate, dl.up, dl.down, torch.from_numpy(off).to(dev),
                            torch.from_numpy(st).to(dev), act=moe.ACT_MXFP8))
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    assert np.isfinite(y).all()
    rows, sub_off, sub_st = _sub_buckets(off, st, rows)
    _check_a8_codes(layer, x, sub_off, sub_st, gc[rows], gs[rows], gv[rows])
    y_ref = oracle.LayerRef(layer).a8_down(sub_off, gc[rows], gs[rows])
    return normwise(y[rows], y_ref)


@pytest.mark.parametrize("tile", [128, 192])
def test_expert_ffn_a8_ragged_buckets(dev, mx, dmx, tile):
    """MX-FP8 GEMMs on bucket sizes around their tiles: more than 112 rows per
    active expert on average (192-row tiles: one or two per expert, a wave
    half of 96 rows with zero to six live 16-row blocks), or 96..112 (128-row
    tiles).  Checked rows: the first and last of each bucket and those at the
    wave-half and tile boundaries (64, 96, 128, 192 rows in)."""
    if tile == 192:
        sizes = np.array([1, 97, 112, 128, 129, 150, 176, 191, 192, 193, 200, 0] * 22)[:256]
        assert sizes.sum() >= 112 * 256  # the host's test: rows per min(E, rows)
    else:
        sizes = np.array([1, 64, 96, 97, 100, 120, 127, 128, 129, 140, 0, 160] * 22)[:256]
        assert 96 * 256 <= sizes.sum() < 112 * 256
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = 211
    st = np.random.default_rng(tile).integers(0, T, int(off[-1])).astype(np.int32)
    x = synth.gen_x(4096, T, seed=tile + 1)
    rows = []
    for e in range(12):
        r0, r1 = int(off[e]), int(off[e + 1])
        rows += [r for r in (r0, r0 + 63, r0 + 64, r0 + 95, r0 + 96, r0 + 127, r0 + 128,
                             r0 + 191, r0 + 192, r1 - 1) if r0 <= r < r1]
    assert _a8_rows_case(mx, dmx, dev, x, off, st, rows) < TOL


@pytest.mark.parametrize("T", [1, 3, 40, 300])
def test_forward_mxfp4_a8(dev, mx, dmx, T):
    _forward_case(mx, dmx.with_act(moe.ACT_MXFP8), dev, T, 500 + T, a8=True)


def test_forward_mxfp4_a8_hash(dev, mx, dmx):
    _forward_case(mx, dmx.with_act(moe.ACT_MXFP8), dev, 100, 601, route=moe.ROUTE_HASH, a8=True)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_mxfp4_a8_prefill_4096(dev, mx, dmx, route):
    _forward_sampled(mx, dmx.with_act(moe.ACT_MXFP8), dev, 4096, 7000 + route, 24, route=route,
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


# --------------------------------------------------------------------------
# selection with more than 256 experts (the general branch of the one-wave
# selection: ballot, readlane, minimum-index ties, NaN from the owner lane),
# and k = 16
# --------------------------------------------------------------------------

def _big_e_logits(E, T, seed):
    lg = np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)
    rows = _decode_select_cases(E)
    lg[:len(rows)] = np.stack(rows)[:T]
    if T > 8:
        lg[7, E - 20:] = lg[7].max() + 3  # maxima in the last lanes' slots
    return lg


@pytest.mark.parametrize("E", [512, 1024])
@pytest.mark.parametrize("k", [8, 16])
@pytest.mark.parametrize("T", [1, 300])
def test_route_large_e(dev, E, k, T):
    lg = _big_e_logits(E, T, E + k + T)
    lt = torch.from_numpy(lg).to(dev)
    idx, w, _ = moe.route(None, None, k, logits_in=lt)
    ref_idx, ref_w = oracle.select_topk(lg, k)
    assert np.array_equal(tnp(idx), ref_idx)
    np.testing.assert_allclose(tnp(w), ref_w, rtol=1e-6, atol=1e-7)
    tids = synth.gen_token_ids(T, seed=E + T)
    tids[0] = 129279
    idx, w, _ = moe.route(None, None, k, mode=moe.ROUTE_HASH, logits_in=lt,
                          token_ids=torch.from_numpy(tids).to(dev))
    ref_idx, ref_w = oracle.select_hash(tids, lg, k)
    assert np.array_equal(tnp(idx), ref_idx)
    np.testing.assert_allclose(tnp(w), ref_w, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("E", [512, 1024])
def test_router_logits_large_e(dev, E):
    H, T = 2048, 37
    wr = synth.gen_bf16(np.random.default_rng(E), (E, H), 1 / np.sqrt(H))
    x = synth.gen_x(H, T, seed=E)
    idx, w, lo = moe.route(t16(x, dev), t16(wr, dev), 16)
    ref_lo = oracle.router_logits(x, wr)
    assert bits_equal(tnp(lo), ref_lo)
    ref_idx, ref_w = oracle.select_topk(ref_lo, 16)
    assert np.array_equal(tnp(idx), ref_idx)


@pytest.fixture(scope="module")
def e512():
    spec = synth.LayerSpec("e512", 2048, 2048, 512, 8, synth.FMT_VQ2, synth.FMT_VQ2,
                           synth.FMT_Q2K, 2048)
    return synth.gen_layer(spec, seed=21)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_large_e_decode(dev, e512, route):
    """One token through the three decode launches with 512 experts, whose
    selection takes the general branch; edge-case logit rows too."""
    dl = moe.DeviceLayer.upload(e512, device=dev)
    _forward_case(e512, dl, dev, 1, 40, route=route)
    _forward_case(e512, dl, dev, 1, 41, route=route)
    if route == moe.ROUTE_SOFTMAX_TOPK:
        x = t16(synth.gen_x(2048, 1, seed=9), dev)
        for n, row in enumerate(_decode_select_cases(512)):
            lg = row[None, :].copy()
            _, idx, w = moe.forward(dl, x, logits_in=torch.from_numpy(lg).to(dev))
            ref_idx, ref_w = oracle.select_topk(lg, 8)
            assert np.array_equal(tnp(idx).reshape(1, 8), ref_idx), n
            np.testing.assert_allclose(tnp(w).reshape(1, 8), ref_w, rtol=1e-6, err_msg=str(n))


@pytest.mark.parametrize("T", [9, 300])
def test_forward_large_e_batches(dev, e512, T):
    """512 experts on the one-block selection-and-bucketing path (T = 9) and
    the selection + dispatch + grouped GEMM path (T = 300, sampled tokens)."""
    dl = moe.DeviceLayer.upload(e512, device=dev)
    if T == 9:
        _forward_case(e512, dl, dev, T, 42)
        _forward_case(e512, dl, dev, T, 43, route=moe.ROUTE_HASH)
    else:
        _forward_sampled(e512, dl, dev, T, 44, 8)
        _forward_sampled(e512, dl, dev, T, 45, 8, route=moe.ROUTE_HASH)


def test_forward_e1024(dev):
    """1024 experts (the largest E): one token through the decode launches,
    and 300 tokens through selection, dispatch and the grouped GEMM."""
    spec = synth.LayerSpec("e1024d", 2048, 2048, 1024, 16, synth.FMT_Q2K, synth.FMT_Q2K,
                           synth.FMT_Q2K, 0)
    layer = synth.gen_layer(spec, seed=31)
    dl = moe.DeviceLayer.upload(layer, device=dev)
    _forward_case(layer, dl, dev, 1, 50)
    _forward_case(layer, dl, dev, 1, 51, route=moe.ROUTE_HASH)
    del dl
    spec = synth.LayerSpec("e1024g", 512, 256, 1024, 8, synth.FMT_VQ2, synth.FMT_VQ2,
                           synth.FMT_Q2K, 256)
    layer = synth.gen_layer(spec, seed=32)
    dl = moe.DeviceLayer.upload(layer, device=dev)
    _forward_case(layer, dl, dev, 300, 52)
    _forward_case(layer, dl, dev, 300, 53, route=moe.ROUTE_HASH)


@pytest.mark.parametrize("T", [1, 9, 100])
def test_forward_k16(dev, T):
    spec = synth.LayerSpec("k16", 2048, 2048, 64, 16, synth.FMT_VQ2, synth.FMT_VQ2,
                           synth.FMT_Q2K, 2048)
    layer = synth.gen_layer(spec, seed=60)
    dl = moe.DeviceLayer.upload(layer, device=dev)
    if T == 100:
        _forward_sampled(layer, dl, dev, T, 61, 8)
    else:
        _forward_case(layer, dl, dev, T, 61 + T)


# --------------------------------------------------------------------------
# activation steering: out += alpha * dir on every forward path
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,alpha", [(1, 2.0), (1, -1.0), (9, -1.0), (300, 2.0)])
def test_forward_steering(dev, q2, dq2, T, alpha):
    d = np.random.default_rng(70).standard_normal(4096)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    dd = torch.from_numpy(d).to(dev)
    L = dq2.with_steering(dd, alpha)
    x = synth.gen_x(4096, T, seed=71 + T)
    xt = t16(x, dev)
    out, idx, w = moe.forward(L, xt)
    plain, _, _ = moe.forward(dq2, xt)
    out, plain = tnp(out), tnp(plain)
    R = oracle.LayerRef(q2, steer_dir=d, steer_alpha=alpha)
    if T <= 9:
        ref, ref_idx, _ = R.forward(x)
        assert np.array_equal(tnp(idx), ref_idx)
        assert normwise(out, ref) < TOL
    else:
        sel = np.array([0, 17, 150, 299])
        ref, _, _ = R.forward(x[sel])
        assert normwise(out[sel], ref) < TOL
    # the steering term itself: within fp32 rounding of the output
    delta = out.astype(np.float64) - plain - alpha * d.astype(np.float64)[None, :]
    assert np.abs(delta).max() <= 4 * 2.0 ** -24 * np.abs(out).max()


# --------------------------------------------------------------------------
# the caller's second stream: the shared expert beside the routed work gives
# the same bits as one stream
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [16, 300])
def test_forward_side_stream_equals_one_stream(dev, q2, dq2, T):
    x = t16(synth.gen_x(4096, T, seed=80 + T), dev)
    f1 = moe.Forward(dq2, T, dev, side_stream=True)
    f2 = moe.Forward(dq2, T, dev, side_stream=False)
    a = f1(x).clone()
    b = f2(x).clone()
    assert np.array_equal(tnp(a).view(np.uint32), tnp(b).view(np.uint32))
    assert torch.equal(f1.idx, f2.idx)


# --------------------------------------------------------------------------
# inputs at the edge of the binary16 domain of the matrix-core and one-token
# down paths: outlier token channels, and Q2K down blocks whose d * scale
# and dequantized weights come near 65504
# --------------------------------------------------------------------------

def _outlier_x(H, T, seed):
    """N(0, 1) tokens with four outlier channels of magnitude 2000, 1000, 800
    and 500 (random signs): g and u reach a few hundred, the SwiGLU output a
    few times 10^4, inside binary16's range."""
    x = (synth.gen_x(H, T, seed=seed).astype(np.uint32) << 16).view(np.float32).copy()
    rng = np.random.default_rng(seed)
    ch = rng.choice(H, 4, replace=False)
    x[:, ch] = rng.choice([-1.0, 1.0], (T, 4)) * np.array([2000.0, 1000.0, 800.0, 500.0])
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("T", [1, 64])
def test_forward_outlier_tokens(dev, q2, dq2, T):
    x = _outlier_x(4096, T, 90 + T)
    ref, ref_idx, _ = oracle.LayerRef(q2).forward(x)
    out, idx, _ = moe.forward(dq2, t16(x, dev))
    out = tnp(out)
    assert np.isfinite(out).all()
    assert np.array_equal(tnp(idx), ref_idx)
    assert normwise(out, ref) < TOL


@pytest.mark.parametrize("T", [1, 64])
def test_forward_q2k_down_large_scales(dev, T):
    spec = synth.LayerSpec("bigd", 2048, 2048, 16, 4, synth.FMT_VQ2, synth.FMT_VQ2,
                           synth.FMT_Q2K, 2048)
    layer = synth.gen_layer(spec, seed=95)
    blk = layer.down.data.reshape(-1, 84)
    rng = np.random.default_rng(96)
    n = blk.shape[0]
    # d * 15 * 3 and dmin * 15 stay below 65504: d, dmin in [600, 1400]
    blk[:, 80:82] = synth.f32_to_f16_bits(rng.uniform(600, 1400, n)).view(np.uint8).reshape(-1, 2)
    blk[:, 82:84] = synth.f32_to_f16_bits(rng.uniform(600, 1400, n)).view(np.uint8).reshape(-1, 2)
    w = oracle.dequant(layer.down, 3, 0, 2048 * 64)
    assert np.abs(w).max() > 30000
    dl = moe.DeviceLayer.upload(layer, device=dev)
    _forward_case(layer, dl, dev, T, 97 + T)


# --------------------------------------------------------------------------
# router logits at the edge of the exactness domain
# --------------------------------------------------------------------------

def test_router_exactness_domain(dev):
    """Inside the stated domain (nonzero |x|, |w| >= 2^-14, sum |x w| < 2^11)
    the logits are bit-exact for every kernel's summation order (the one-
    token wave, the GEMV, the fp64 MFMA tiles); far outside it (elements
    down to 2^-100) they stay within one fp32 ulp."""
    H, E = 4096, 256
    rng = np.random.default_rng(99)

    def bf(mag):
        return synth.f32_to_bf16_bits((mag * rng.choice([-1, 1], mag.shape)).astype(np.float32))

    wr = bf(np.exp2(rng.uniform(-14, -4, (E, H))))
    for T in (1, 5, 64):
        x = bf(np.exp2(rng.uniform(-14, 1, (T, H))))
        xv = (x.astype(np.uint32) << 16).view(np.float32)
        wv = (wr.astype(np.uint32) << 16).view(np.float32)
        assert np.abs(xv).min() >= 2.0 ** -14 and np.abs(wv).min() >= 2.0 ** -14
        assert (np.abs(xv.astype(np.float64)) @ np.abs(wv.astype(np.float64)).T).max() < 2 ** 11
        _, _, lo = moe.route(t16(x, dev), t16(wr, dev), 8)
        assert bits_equal(tnp(lo), oracle.router_logits(x, wr)), T
        x2 = xv.copy()
        x2[:, ::7] *= np.float32(2.0 ** -100)
        x2 = synth.f32_to_bf16_bits(x2)
        _, _, lo2 = moe.route(t16(x2, dev), t16(wr, dev), 8)
        ref2 = oracle.router_logits(x2, wr)
        ulp = np.abs(tnp(lo2).view(np.int32).astype(np.int64) - ref2.view(np.int32).astype(np.int64))
        assert ulp.max() <= 1, T


# --------------------------------------------------------------------------
# the screened router of many-token forwards: exact and near ties among the
# experts near the top, and tokens whose approximate logits are useless
# (non-finite, zero, subnormal, near the end of the fp32 range)
# --------------------------------------------------------------------------

def _tie_router(wr):
    """Rows 1 = row 0; rows 10..19 one row times 2 (a ten-way exact tie, most
    often in the top 8); rows 30..37 one row times 1.5, each with one element
    moved by one bf16 ulp (ties broken only in the last bits)."""
    wr = wr.copy()
    f = (wr.astype(np.uint32) << 16).view(np.float32)
    wr[1] = wr[0]
    wr[10:20] = synth.f32_to_bf16_bits(f[10] * 2)
    near = synth.f32_to_bf16_bits(f[30] * 1.5)
    for j in range(8):
        row = near.copy()
        row[7 * j + 3] += 1
        wr[30 + j] = row
    return wr


def _odd_tokens(x, wr):
    """Token rows 5..12 replaced by inputs outside the screen's comfort zone;
    row 9 is router row 50 times 2.5 * 2^127, whose logit overflows fp32."""
    f = (x.astype(np.uint32) << 16).view(np.float32).copy()
    f[5, 17] = np.inf
    f[6] *= np.float32(2.0 ** -120)
    f[7] = 0
    f[8] *= np.float32(2.0 ** 100)
    f[9] = ((wr[50].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            * (2.5 * 2.0 ** 127)).astype(np.float32)
    f[11] = f[10]
    f[12, 3] = np.nan
    return synth.f32_to_bf16_bits(f)


@pytest.mark.parametrize("route", [moe.ROUTE_SOFTMAX_TOPK, moe.ROUTE_HASH])
def test_forward_screened_router_edges(dev, q2, dq2, route):
    import dataclasses
    T = 2048
    wr = _tie_router(q2.w_router)
    layer = dataclasses.replace(q2, w_router=wr)
    dl = moe.DeviceLayer(dq2.H, dq2.I, dq2.E, dq2.k, route, t16(wr, dev), dq2.gate, dq2.up,
                         dq2.down, dq2.shared_gate, dq2.shared_up, dq2.shared_down)
    x = _odd_tokens(synth.gen_x(4096, T, seed=123), wr)
    tids = synth.gen_token_ids(T, seed=124) if route == moe.ROUTE_HASH else None
    out, idx, w = moe.forward(dl, t16(x, dev), None,
                              None if tids is None else torch.from_numpy(tids).to(dev))
    out, idx, w = tnp(out), tnp(idx), tnp(w)
    R = oracle.LayerRef(layer, route_mode=route)
    ridx, rw, rlo = R.route(x, None, tids)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(w, rw, rtol=1e-6, atol=1e-7, equal_nan=True)
    if route == moe.ROUTE_SOFTMAX_TOPK:
        # the ties did reach the top 8: exact ties decided by the index
        tie = np.isin(ridx, np.arange(10, 20)).sum(1)
        assert (tie == 8).sum() > 50 and list(ridx[7]) == list(range(8))
        assert (np.isin(ridx, np.arange(30, 38)).sum(1) >= 2).sum() > 50
    sel = np.array([0, 1, 2, 3, 4, 13, 1000, T - 1])
    ref, _, _ = R.forward(x[sel], None, None if tids is None else tids[sel])
    assert normwise(out[sel], ref) < TOL


# --------------------------------------------------------------------------
# speculative-decode verification batches: 1 + 5 tokens per session, one
# session (T = 6) or 16 (T = 96), router or Zipf logits
# --------------------------------------------------------------------------

@pytest.mark.parametrize("wname", ["verify_t6", "verify_t6_zipf", "verify_t96",
                                   "verify_t96_zipf"])
def test_forward_verify_batch(dev, q2, dq2, wname):
    w = synth.WORKLOADS[wname]
    zipf = w.logits == "zipf"
    if w.T <= 6:
        _forward_case(q2, dq2, dev, w.T, 110, zipf=zipf)
        _forward_case(q2, dq2, dev, w.T, 111, zipf=zipf)
    else:
        _forward_sampled(q2, dq2, dev, w.T, 112, 16, zipf=zipf)


@pytest.mark.parametrize("T", [6, 96])
def test_forward_verify_graph_replay(dev, q2, dq2, T):
    f = moe.Forward(dq2, T, dev)
    xs = [t16(synth.gen_x(4096, T, seed=120 + T + i), dev) for i in range(3)]
    _graph_replays(f, xs)


# --------------------------------------------------------------------------
# the routed-expert residency cache: experts in pinned host memory, a pool of
# slots in HBM, decided and filled on the device
# --------------------------------------------------------------------------

def _logits_for(E, chosen, rng):
    """Logits whose top-len(chosen) are `chosen`, in that order."""
    lg = rng.standard_normal(E).astype(np.float32) - 10.0
    lg[chosen] = 10.0 - np.arange(len(chosen), dtype=np.float32)
    return lg[None, :]


def _pick(rng, resident, E, k, n_hit):
    res = np.flatnonzero(resident >= 0)
    non = np.flatnonzero(resident < 0)
    return np.concatenate([rng.choice(res, n_hit, replace=False),
                           rng.choice(non, k - n_hit, replace=False)])


@pytest.fixture(scope="module")
def cached_q2(q2, dev):
    return moe.CachedLayer(q2, 32, dev)


@pytest.mark.parametrize("hit", [0.0, 0.5, 1.0])
def test_forward_cached_hit_rates(dev, q2, dq2, cached_q2, hit):
    """Steps at a controlled hit rate (the chosen experts picked from the
    resident ones and the others): every step's output, choices and weights
    equal moe_forward's bit for bit, the counters record exactly the planned
    hits and misses, and a step matches the oracle."""
    cl = cached_q2
    cl.reset()
    rng = np.random.default_rng(int(hit * 10) + 3)
    E, k = 256, 8
    # warm: fill the 32 slots with 4 steps of misses
    for s in range(4):
        chosen = _pick(rng, cl.resident(), E, k, 0)
        x = t16(synth.gen_x(4096, 1, seed=200 + s), dev)
        cl(x, torch.from_numpy(_logits_for(E, chosen, rng)).to(dev))
    assert (cl.resident() >= 0).sum() == 32
    n_hit = int(round(hit * k))
    for s in range(6):
        h0, m0 = cl.counts()
        chosen = _pick(rng, cl.resident(), E, k, n_hit)
        lg = _logits_for(E, chosen, rng)
        x = synth.gen_x(4096, 1, seed=300 + s)
        lt, xt = torch.from_numpy(lg).to(dev), t16(x, dev)
        out = tnp(cl(xt, lt)).copy()
        idx, w = tnp(cl.idx).copy(), tnp(cl.w).copy()
        ref, ridx, rw = moe.forward(dq2, xt, lt)
        assert np.array_equal(out.view(np.uint32), tnp(ref).view(np.uint32)), s
        assert np.array_equal(idx, tnp(ridx)) and np.array_equal(w, tnp(rw))
        assert list(idx.reshape(-1)) == list(chosen)
        h1, m1 = cl.counts()
        assert (h1 - h0, m1 - m0) == (n_hit, k - n_hit), (s, h1 - h0, m1 - m0)
        res = cl.resident()
        assert (res[chosen] >= 0).all() and len(set(res[chosen])) == k
    oref, oidx, _ = oracle.LayerRef(q2).forward(x, lg)
    assert np.array_equal(idx, oidx)
    assert normwise(out, oref) < TOL


def test_forward_cached_router_hash_and_graph(dev, q2, dq2, cached_q2):
    """Router logits (computed by the layer's own p1) and hash routing through
    the cache; a captured step replayed with eager steps between the replays
    equals the eager result every time (hits or misses)."""
    cl = cached_q2
    cl.reset()
    for s in range(5):
        xt = t16(synth.gen_x(4096, 1, seed=400 + s), dev)
        out = tnp(cl(xt)).copy()
        ref, _, _ = moe.forward(dq2, xt)
        assert np.array_equal(out.view(np.uint32), tnp(ref).view(np.uint32)), s
    hl = moe.CachedLayer.__new__(moe.CachedLayer)
    hl.__dict__.update(cl.__dict__)
    hl.layer = cl.layer.with_route_mode(moe.ROUTE_HASH)
    hl.f = moe.Forward(hl.layer, 1, dev, side_stream=False)
    dh = dq2.with_route_mode(moe.ROUTE_HASH)
    for s in range(3):
        xt = t16(synth.gen_x(4096, 1, seed=500 + s), dev)
        tid = torch.from_numpy(synth.gen_token_ids(1, seed=s)).to(dev)
        out = tnp(hl(xt, None, tid)).copy()
        ref, _, _ = moe.forward(dh, xt, None, tid)
        assert np.array_equal(out.view(np.uint32), tnp(ref).view(np.uint32)), s
    xs = [t16(synth.gen_x(4096, 1, seed=600 + i), dev) for i in range(3)]
    refs = [tnp(moe.forward(dq2, x)[0]).copy() for x in xs]
    xb = xs[0].clone()
    cl(xb)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        cl(xb)
    torch.cuda.current_stream().wait_stream(s_)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        cl(xb)
    for rep in range(2):
        for i, x in enumerate(xs):
            xb.copy_(x)
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(tnp(cl.f.out).view(np.uint32), refs[i].view(np.uint32)), (rep, i)
            cl(xs[(i + 1) % 3])
            torch.cuda.synchronize()

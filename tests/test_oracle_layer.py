"""Whole-layer pins of the CPU oracle.

* one expert, k = 1, weight 1: the layer is the textbook SwiGLU FFN plus the
  shared expert, checked against torch fp64 CPU ops on the decoded weights;
* the bucketed path (route -> dispatch -> FFN -> combine) equals a
  brute-force dense masked evaluation with no dispatch;
* special cases: zero routed weights leave only the shared expert; the
  combine is linear in the routing weights; permuting experts together with
  their router rows leaves the output unchanged;
* MX-FP8 activation quantization follows the OCP MX scale rule.
"""
import dataclasses

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import synth


def _spec(H=256, I=128, E=8, k=2, fg=synth.FMT_Q2K, fu=synth.FMT_Q2K, fd=synth.FMT_Q2K, Is=128):
    return synth.LayerSpec("t", H, I, E, k, fg, fu, fd, Is)


def _f64(m):
    return torch.from_numpy(m.astype(np.float64))


def _x64(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).double()


def _swiglu_torch(x, wg, wu, wd):
    return (torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)) @ wd.T


@pytest.mark.parametrize("fmts", [
    (synth.FMT_Q2K, synth.FMT_Q2K, synth.FMT_Q2K),
    (synth.FMT_VQ2, synth.FMT_VQ2, synth.FMT_Q2K),
    (synth.FMT_MXFP4, synth.FMT_MXFP4, synth.FMT_MXFP4),
    (synth.FMT_BF16, synth.FMT_BF16, synth.FMT_BF16),
])
def test_single_expert_is_textbook_swiglu(fmts):
    spec = _spec(H=512, I=256, E=1, k=1, fg=fmts[0], fu=fmts[1], fd=fmts[2], Is=256)
    L = synth.gen_layer(spec, seed=11)
    R = oracle.LayerRef(L)
    x = synth.gen_x(spec.H, 3, seed=12)
    out, idx, w = R.forward(x)
    assert np.all(idx == 0) and np.all(w == 1.0)
    xt = _x64(x)
    wg, wu, wd = (_f64(oracle.dequant_matrix(p)) for p in (L.gate, L.up, L.down))
    sg, su, sd = (_x64(a) for a in (L.shared_gate, L.shared_up, L.shared_down))
    ref = _swiglu_torch(xt, wg, wu, wd) + _swiglu_torch(xt, sg, su, sd)
    np.testing.assert_allclose(out, ref.numpy().astype(np.float32), rtol=2e-6, atol=1e-9)


def _normwise(a, b):
    return np.abs(a.astype(np.float64) - b).max() / max(np.abs(b).max(), 1e-30)


@pytest.mark.parametrize("seed", [0, 1])
def test_dense_masked_equals_bucketed_tiny(seed):
    L = synth.gen_layer(synth.TINY, seed)
    R = oracle.LayerRef(L)
    x = synth.gen_x(256, 4, seed)
    out, idx, w = R.forward(x)
    dm = R.dense_masked(x, idx, w)
    assert _normwise(out, dm) <= 1e-6


@settings(max_examples=25, deadline=None)
@given(
    H=st.sampled_from([256, 512]), I=st.sampled_from([128, 256]), E=st.integers(1, 8),
    kk=st.integers(1, 4), T=st.integers(1, 5), seed=st.integers(0, 2**31 - 1),
    fmts=st.sampled_from([(1, 1, 1), (2, 2, 1), (3, 3, 3), (0, 0, 0), (2, 3, 1)]),
    hash_route=st.booleans(), shared=st.booleans())
def test_dense_masked_equals_bucketed_fuzz(H, I, E, kk, T, seed, fmts, hash_route, shared):
    k = min(kk, E)
    spec = _spec(H, I, E, k, *fmts, Is=I if shared else 0)
    L = synth.gen_layer(spec, seed % 1000)
    R = oracle.LayerRef(L, route_mode=1 if hash_route else 0)
    x = synth.gen_x(H, T, seed)
    tids = synth.gen_token_ids(T, seed) if hash_route else None
    out, idx, w = R.forward(x, token_ids=tids)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) < 1e-6)
    dm = R.dense_masked(x, idx, w)
    assert _normwise(out, dm) <= 1e-6


def test_bucketed_pieces_compose_to_forward():
    L = synth.gen_layer(synth.TINY, 3)
    R = oracle.LayerRef(L)
    x = synth.gen_x(256, 6, 3)
    out, idx, w = R.forward(x)
    idx2, w2, _ = R.route(x)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    off, st_, ss, sp = oracle.dispatch(idx, L.spec.E)
    y = R.expert_ffn(x, off, st_)
    sh = R.shared_ffn(x)
    comb = oracle.combine(y, sp, w, sh)
    assert _normwise(comb, out.astype(np.float64)) <= 1e-6


def test_zero_routed_weights_leave_shared_expert():
    L = synth.gen_layer(synth.TINY, 4)
    L.down.data[:] = 0  # d = dmin = 0 in every block: every routed down weight is 0
    R = oracle.LayerRef(L)
    x = synth.gen_x(256, 4, 4)
    out, _, _ = R.forward(x)
    assert np.array_equal(out, R.shared_ffn(x))


def test_combine_linear_in_weights():
    rng = np.random.default_rng(0)
    T, k, H = 5, 3, 64
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    sp = rng.permutation(T * k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    base = oracle.combine(y, sp, w)
    twice = oracle.combine(y, sp, (2 * w).astype(np.float32))
    np.testing.assert_allclose(twice, 2 * base, rtol=1e-6)
    # gather form: out[t] = sum_j w[t,j] * y[sp[t*k+j]]
    ref = np.einsum("tk,tkh->th", w.astype(np.float64), y[sp].reshape(T, k, H).astype(np.float64))
    np.testing.assert_allclose(twice / 2, ref, rtol=1e-6)


def test_expert_permutation_invariance():
    spec = _spec(E=8, k=2)
    L = synth.gen_layer(spec, 5)
    x = synth.gen_x(256, 4, 5)
    out, idx, w = oracle.LayerRef(L).forward(x)
    perm = np.random.default_rng(1).permutation(8)
    P = dataclasses.replace(L)
    P.w_router = L.w_router[perm]
    P.gate = dataclasses.replace(L.gate, data=L.gate.data[perm])
    P.up = dataclasses.replace(L.up, data=L.up.data[perm])
    P.down = dataclasses.replace(L.down, data=L.down.data[perm])
    out2, idx2, w2 = oracle.LayerRef(P).forward(x)
    assert np.array_equal(perm[idx2], idx)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-7)


# --------------------------------------------------------------------------
# MX-FP8 activations (the A8 variant for FP4 matrix instructions)
# --------------------------------------------------------------------------

def test_mxfp8_scale_rule_examples():
    # amax = 1 -> floor(log2 1) - 8 = -8 -> byte 119; amax = 448 -> 0 -> 127;
    # amax = 3 -> 1 - 8 = -7 -> 120; all zero -> byte 0
    a = np.zeros((4, 32), np.float32)
    a[0, 5] = 1.0
    a[1, 0] = -448.0
    a[2, 31] = 3.0
    codes, scales = oracle.mxfp8_quant(a)
    assert list(scales[:, 0]) == [119, 127, 120, 0]
    assert codes[0, 5] == 0x78  # 1/2^-8 = 256 = 1.0 * 2^8 -> exponent 15, mantissa 0
    assert codes[1, 0] == 0xFE  # -448
    assert codes[2, 31] == oracle.to_e4m3(3.0 * 2**7)
    assert not codes[3].any()


def test_mxfp8_codes_match_torch_conversion():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal((16, 128)) * np.exp2(rng.integers(-20, 20, (16, 1)))).astype(np.float32)
    codes, scales = oracle.mxfp8_quant(a)
    g = a.reshape(16, 4, 32).astype(np.float64)
    amax = np.abs(g).max(2)
    s = np.floor(np.log2(amax)) - 8
    assert np.array_equal(scales, (s + 127).astype(np.uint8))
    scaled = (g / np.exp2(s)[..., None]).reshape(16, 128)
    ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch's cast gives NaN above 448; the MX rule saturates there
    inside = np.abs(scaled) <= 448
    assert np.array_equal(codes[inside], ref[inside])
    assert (~inside).any()
    assert np.all(codes[~inside] == np.where(scaled[~inside] > 0, 0x7E, 0xFE))


def test_a8_forward_close_to_plain_forward():
    spec = _spec(H=512, I=256, E=4, k=2, fg=3, fu=3, fd=3, Is=256)
    L = synth.gen_layer(spec, 9)
    R = oracle.LayerRef(L)
    x = synth.gen_x(512, 4, 9)
    out, idx, w = R.forward(x)
    out8, idx8, w8 = R.forward(x, a8=True)
    assert np.array_equal(idx, idx8)
    err = _normwise(out8, out.astype(np.float64))
    assert 1e-4 < err < 0.1


# --------------------------------------------------------------------------
# the A8 variant's two quantization points, pinned against hand-derived
# values: torch's E4M3 conversion and the OCP MX scale rule written out here
# --------------------------------------------------------------------------

_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mx8_torch(v):
    """OCP MX-FP8 of fp64 values per 32 along the last axis, by hand: scale
    2^(floor(log2 amax) - 8), elements through torch's float8_e4m3fn cast
    (ties to even) after clamping to +-448 (the MX rule saturates)."""
    g = v.reshape(*v.shape[:-1], -1, 32)
    amax = np.abs(g).max(-1, keepdims=True)
    s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    y = np.clip(g / np.exp2(s), -448, 448)
    q = torch.from_numpy(y).to(torch.float8_e4m3fn).double().numpy()
    return (q * np.exp2(s)).reshape(v.shape)


def _mxfp4_matrix(vals):
    """An MXFP4 projection [1, N, K] holding exactly `vals` (each entry an
    E2M1 value times the power of two of its group of 32, zeros elsewhere)."""
    N, K = vals.shape
    nib = np.zeros((N, K), np.uint8)
    sc = np.full((N, K // 32), 127, np.uint8)
    for n in range(N):
        for g in range(K // 32):
            grp = vals[n, 32 * g:32 * g + 32]
            nz = grp[grp != 0]
            e = 0 if nz.size == 0 else int(np.floor(np.log2(np.abs(nz).max() / 6.0)) + 1)
            sc[n, g] = 127 + e
            for i, v in enumerate(grp):
                m = abs(v) / 2.0 ** e
                c = _E2M1.index(m)
                nib[n, 32 * g + i] = c | (8 if v < 0 else 0)
    data = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return synth.Proj(synth.FMT_MXFP4, 1, N, K, data.reshape(1, N, K // 2), sc.reshape(1, N, K // 32))


def _one_hot_a8_layer():
    """E = 1, k = 1, H = I = 64, MXFP4 weights, no shared expert: the token
    e_0 picks column 0 of gate and up, so g_i = G[i], u_i = U[i] exactly, and
    the down projection is the identity, so the layer's output is the
    SwiGLU output after its MX-FP8 rounding."""
    H = I = 64
    rng = np.random.default_rng(21)
    Gv = np.array([_E2M1[1 + i % 7] * (-1) ** (i // 7) * 2.0 ** (i % 5 - 2) for i in range(I)])
    Uv = np.array([_E2M1[1 + (3 * i) % 7] * (-1) ** i * 2.0 ** ((i // 32) * 3 - 1) for i in range(I)])
    G = np.zeros((I, H))
    U = np.zeros((I, H))
    G[:, 0], U[:, 0] = Gv, Uv
    spec = synth.LayerSpec("onehot", H, I, 1, 1, synth.FMT_MXFP4, synth.FMT_MXFP4,
                           synth.FMT_MXFP4, 0)
    L = synth.Layer(spec, synth.gen_bf16(rng, (1, H), 0.1), _mxfp4_matrix(G), _mxfp4_matrix(U),
                    _mxfp4_matrix(np.eye(H)), None, None, None, None)
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80  # 1.0: its MX-FP8 projection is itself
    return L, x, Gv, Uv


def test_a8_swiglu_output_quantized_one_hot():
    L, x, g, u = _one_hot_a8_layer()
    R = oracle.LayerRef(L)
    assert np.array_equal(oracle.dequant_matrix(L.gate)[:, 0], g)
    assert np.array_equal(oracle.dequant_matrix(L.down), np.eye(64))
    a = g / (1.0 + np.exp(-g)) * u
    want = _mx8_torch(a)
    out, idx, w = R.forward(x, a8=True)
    assert idx[0, 0] == 0 and w[0, 0] == 1.0
    assert np.array_equal(out[0].astype(np.float64), want)
    # the rounding is visible: without it the output would be fp32(a)
    assert (out[0] != a.astype(np.float32)).sum() > 32
    # the plain layer keeps a
    plain, _, _ = R.forward(x)
    np.testing.assert_allclose(plain[0], a, rtol=1e-6)
    # the first stage alone gives the same codes
    off, st, _, _ = oracle.dispatch(idx, 1)
    codes, scales = R.a8_swiglu_codes(x, off, st)
    dec = np.array([oracle.e4m3(c) for c in codes[0]]) * np.repeat(
        [oracle.e8m0(s) for s in scales[0]], 32)
    assert np.array_equal(dec, want)


def test_a8_forward_invariant_under_token_requantization():
    """The tokens enter gate/up through their MX-FP8 projection: replacing x
    by that projection (computed here with torch) changes nothing in the A8
    layer, while the plain layer sees the difference."""
    spec = _spec(H=512, I=256, E=4, k=2, fg=3, fu=3, fd=3, Is=0)
    L = synth.gen_layer(spec, 13)
    R = oracle.LayerRef(L)
    x = synth.gen_x(512, 5, 14)
    xv = _x64(x).numpy()
    xq = _mx8_torch(xv)
    xq_bits = synth.f32_to_bf16_bits(xq.astype(np.float32))
    assert np.array_equal(_x64(xq_bits).numpy(), xq)  # exact in bf16
    assert not np.array_equal(xq, xv)
    lg = np.random.default_rng(15).standard_normal((5, 4)).astype(np.float32)
    a, ia, wa = R.forward(x, logits_in=lg, a8=True)
    b, ib, wb = R.forward(xq_bits, logits_in=lg, a8=True)
    assert np.array_equal(ia, ib) and np.array_equal(wa, wb)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    p, _, _ = R.forward(x, logits_in=lg)
    q, _, _ = R.forward(xq_bits, logits_in=lg)
    assert _normwise(p, q.astype(np.float64)) > 1e-3


def test_a8_stages_compose_to_forward():
    """codes -> down -> combine equals the A8 forward (the fp32 rounding of the
    rows is the only difference)."""
    spec = _spec(H=512, I=256, E=4, k=2, fg=3, fu=3, fd=3, Is=256)
    L = synth.gen_layer(spec, 16)
    R = oracle.LayerRef(L)
    x = synth.gen_x(512, 6, 17)
    out, idx, w = R.forward(x, a8=True)
    off, st, _, sp = oracle.dispatch(idx, 4)
    codes, scales = R.a8_swiglu_codes(x, off, st)
    y = R.a8_down(off, codes, scales)
    ref = oracle.combine(y, sp, w, R.shared_ffn(x))
    assert _normwise(ref, out.astype(np.float64)) < 1e-6
    # and differs from the plain layer's rows by the MX-FP8 effect
    assert _normwise(y, R.expert_ffn(x, off, st).astype(np.float64)) > 1e-3


# --------------------------------------------------------------------------
# activation steering: out += alpha * dir, added after the routed sum
# --------------------------------------------------------------------------

def _unit_dir(H, seed):
    d = np.random.default_rng(seed).standard_normal(H)
    return (d / np.linalg.norm(d)).astype(np.float32)


def test_steering_alone_is_alpha_dir():
    """With every routed weight zero and no shared expert the layer's output
    is the steering term alone: fp32(alpha * dir), one rounding of the exact
    product."""
    spec = _spec(Is=0)
    L = synth.gen_layer(spec, 5)
    L.down.data[:] = 0
    d = _unit_dir(256, 6)
    for alpha in (2.0, -1.0, 0.3):
        out, _, _ = oracle.LayerRef(L, steer_dir=d, steer_alpha=alpha).forward(synth.gen_x(256, 3, 7))
        want = (np.float64(np.float32(alpha)) * d.astype(np.float64)).astype(np.float32)
        assert np.array_equal(out, np.tile(want, (3, 1)))


def test_steering_shifts_the_layer_by_alpha_dir():
    """Steered minus plain output is alpha * dir, within the fp32 rounding of
    the two outputs; strength 0 changes nothing."""
    L = synth.gen_layer(synth.TINY, 8)
    x = synth.gen_x(256, 5, 9)
    d = _unit_dir(256, 10)
    plain, idx, w = oracle.LayerRef(L).forward(x)
    for alpha in (2.0, -1.0):
        out, idx2, w2 = oracle.LayerRef(L, steer_dir=d, steer_alpha=alpha).forward(x)
        assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
        delta = out.astype(np.float64) - plain - alpha * d.astype(np.float64)
        assert np.abs(delta).max() <= 2 * 2.0 ** -24 * np.abs(out).max()
    zero, _, _ = oracle.LayerRef(L, steer_dir=d, steer_alpha=0.0).forward(x)
    assert np.array_equal(zero, plain)


def test_steering_dense_masked_equals_bucketed():
    L = synth.gen_layer(synth.TINY, 11)
    x = synth.gen_x(256, 6, 12)
    d = _unit_dir(256, 13)
    R = oracle.LayerRef(L, steer_dir=d, steer_alpha=-1.5)
    out, idx, w = R.forward(x)
    dense = R.dense_masked(x, idx, w)
    np.testing.assert_allclose(out, dense, rtol=0, atol=1e-6 * np.abs(dense).max())
    # and the steered combine of the bucketed pieces
    off, st, _, sp = oracle.dispatch(idx, L.spec.E)
    y = R.expert_ffn(x, off, st)
    ref = oracle.combine(y, sp, w, R.shared_ffn(x), d, -1.5)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-6 * np.abs(ref).max())

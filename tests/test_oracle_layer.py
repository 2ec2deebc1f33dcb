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

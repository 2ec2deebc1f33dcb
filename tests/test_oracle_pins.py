"""Pins of the CPU oracle against things other than itself.

Scalar decoders are checked exhaustively against library conversions
(numpy float16, torch bfloat16 / float8_e4m3fn / float8_e8m0fnu); the block
formats against hand-built blocks whose values were worked out by hand
(tests/golden); routing against brute-force sorts and library softmax;
dispatch against a library stable sort; SplitMix64 against its published
reference stream.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.golden import fixtures


# --------------------------------------------------------------------------
# scalars
# --------------------------------------------------------------------------

def test_f16_all_patterns_match_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16(b) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_all_patterns_match_torch():
    bits = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16(b) for b in range(1 << 16)], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e2m1_table():
    # OCP MX v1.0 FP4 E2M1 value table
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1(c)
        want = -mags[c & 7] if c & 8 else mags[c & 7]
        assert v == want and math.copysign(1, v) == math.copysign(1, want)


def test_e8m0_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()
    for e in range(256):
        v = oracle.e8m0(e)
        if e == 255:
            assert math.isnan(v)
        else:
            assert v == math.ldexp(1.0, e - 127) == ref[e]


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3(c) for c in range(256)], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(5)
    # random magnitudes over the whole range, every code value and every midpoint
    vals = list(rng.uniform(-448, 448, 4000)) + list(np.exp2(rng.uniform(-12, 8.8, 4000)))
    finite = [oracle.e4m3(c) for c in range(0x7F)]
    vals += finite + [-v for v in finite]
    vals += [(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])]
    t = torch.tensor(vals, dtype=torch.float64)
    ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.to_e4m3(v) for v in vals], np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    assert oracle.to_e4m3(1e6) == 0x7E
    assert oracle.to_e4m3(-500.0) == 0xFE
    assert oracle.to_e4m3(0.0) == 0x00


def test_splitmix64_reference_stream():
    for x, want in fixtures.splitmix64_vectors():
        assert oracle.splitmix64(x) == want


# --------------------------------------------------------------------------
# weight formats: hand-built blocks
# --------------------------------------------------------------------------

def _one(fmt, N, K, data, scales=None, cb=None):
    return synth.Proj(fmt, 1, N, K, data, scales, cb)


@pytest.mark.parametrize("name", ["A", "B", "Z"])
def test_q2k_hand_blocks(name):
    blk, exp = fixtures.q2k_blocks()[name]
    w = oracle.dequant(_one(synth.FMT_Q2K, 1, 256, blk.reshape(1, 84)))
    for i, v in exp.items():
        assert w[i] == v, (name, i, w[i], v)


def test_q2k_position_coded_block():
    """Pack chosen (scale, min, code) fields by the layout and decode them."""
    rng = np.random.default_rng(1)
    sc = rng.integers(0, 16, 16)
    mn = rng.integers(0, 16, 16)
    q = rng.integers(0, 4, 256)
    blk = np.zeros(84, np.uint8)
    blk[:16] = sc | (mn << 4)
    for i in range(256):
        blk[16 + i // 4] |= q[i] << (2 * (i % 4))
    blk[80:82] = np.array([0x3555], np.uint16).view(np.uint8)  # 0.333...
    blk[82:84] = np.array([0x2E66], np.uint16).view(np.uint8)  # 0.1
    d = float(np.uint16(0x3555).view(np.float16))
    dmin = float(np.uint16(0x2E66).view(np.float16))
    w = oracle.dequant(_one(synth.FMT_Q2K, 1, 256, blk.reshape(1, 84)))
    s = np.arange(256) // 16
    want = (np.float32(d) * sc[s].astype(np.float32)) * q.astype(np.float32) - np.float32(dmin) * mn[s].astype(np.float32)
    assert np.array_equal(w, want.astype(np.float32))


def test_q2k_blocks_span_rows():
    """[N, K] with K = 128: block b covers rows 2b and 2b+1 (row-major flattening)."""
    blk, exp = fixtures.q2k_blocks()["B"]
    z = np.zeros(84, np.uint8)
    data = np.concatenate([z, blk]).reshape(1, 168)
    w = oracle.dequant(_one(synth.FMT_Q2K, 4, 128, data)).reshape(4, 128)
    assert not w[:2].any()
    for i, v in exp.items():
        assert w[2 + i // 128, i % 128] == v


def test_vq2_hand_row():
    cb, d, idx, exp = fixtures.vq2_row()
    p = _one(synth.FMT_VQ2, 1, 512, idx.reshape(1, 1, 128), d.reshape(1, 1, 2), cb)
    w = oracle.dequant(p)
    for i, v in exp.items():
        assert w[i] == v and math.copysign(1, w[i]) == math.copysign(1, v), (i, w[i], v)
    assert np.array_equal(w[:256].reshape(64, 4), np.tile([0.5, -1, 1.5, -2], (64, 1)))


def test_vq2_second_row_uses_its_own_planes():
    cb, d, idx, exp = fixtures.vq2_row()
    idx2 = np.stack([np.zeros(128, np.uint8), idx]).reshape(1, 2, 128)
    d2 = np.stack([np.array([0x3C00, 0x3C00], np.uint16), d]).reshape(1, 2, 2)
    w = oracle.dequant(_one(synth.FMT_VQ2, 2, 512, idx2, d2, cb)).reshape(2, 512)
    assert not w[0].any()
    for i, v in exp.items():
        assert w[1, i] == v


def test_mxfp4_hand_row():
    vals, scales, exp = fixtures.mxfp4_row()
    w = oracle.dequant(_one(synth.FMT_MXFP4, 1, 64, vals.reshape(1, 1, 32), scales.reshape(1, 1, 2)))
    for i, v in exp.items():
        assert w[i] == v and math.copysign(1, w[i]) == math.copysign(1, v), (i, w[i], v)


def test_mxfp4_scale_examples():
    # nibble 0x7 with e = 128 -> 12.0; 0xF with e = 127 -> -6.0; 0x8 -> -0.0
    vals = np.full((1, 1, 16), 0x87, np.uint8)
    vals[0, 0, 8:] = 0xF7
    for e, lo, hi in [(128, 12.0, -0.0), (127, 6.0, -0.0)]:
        w = oracle.dequant(_one(synth.FMT_MXFP4, 1, 32, vals, np.full((1, 1, 1), e, np.uint8)))
        assert w[0] == lo and w[1] == hi and math.copysign(1, w[1]) < 0
        assert w[17] == (-6.0 if e == 127 else -12.0)


def test_bf16_projection_is_identity_decode():
    p = synth.gen_stress_proj(synth.FMT_BF16, 8, 64, seed=3)
    w = oracle.dequant(p)
    ref = torch.from_numpy(p.data.reshape(-1).view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------

def _bf16_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_router_logits_match_fp64_matmul():
    H, E, T = 512, 32, 9
    wr = synth.gen_bf16(np.random.default_rng(2), (E, H), 1 / np.sqrt(H))
    x = synth.gen_x(H, T, seed=4)
    got = oracle.router_logits(x, wr)
    ref = (_bf16_to_f64(x) @ _bf16_to_f64(wr).T).astype(np.float32)
    ulp = np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1 and (ulp == 0).mean() > 0.99


@pytest.mark.parametrize("E,k", [(8, 2), (256, 8), (5, 5), (16, 1)])
def test_topk_matches_stable_sort(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[::7, : E // 2] = 0.25  # ties: lower index first
    idx, w = oracle.select_topk(logits, k)
    ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref)
    sel = np.take_along_axis(logits, ref, 1).astype(np.float64)
    full = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    renorm = np.take_along_axis(full, ref, 1)
    renorm /= renorm.sum(1, keepdims=True)
    np.testing.assert_allclose(w, renorm, rtol=1e-6, atol=0)
    np.testing.assert_allclose(w, torch.softmax(torch.from_numpy(sel), 1).numpy(), rtol=1e-6)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1) <= 4 * 2.0 ** -23)


def test_topk_all_equal_picks_lowest_indices():
    idx, w = oracle.select_topk(np.zeros((3, 10), np.float32), 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1)))
    assert np.all(w == np.float32(0.25))


def test_hash_routing_closed_form():
    E, k = 256, 8
    tids = np.array([0, 129279, 1, 77777], np.int64)
    logits = np.random.default_rng(0).standard_normal((4, E)).astype(np.float32)
    idx, w = oracle.select_hash(tids, logits, k)
    # splitmix64(0) = 0xE220A8397B1DCDAF, whose low byte is 0xAF = 175
    assert list(idx[0]) == list(range(175, 183))
    for t, tid in enumerate(tids):
        z = oracle.splitmix64(int(tid))
        assert list(idx[t]) == [(z + j) % E for j in range(k)]
        assert len(set(idx[t])) == k
        sel = logits[t, idx[t]].astype(np.float64)
        np.testing.assert_allclose(w[t], torch.softmax(torch.from_numpy(sel), 0).numpy(), rtol=1e-6)


def test_hash_routing_wraps_mod_E():
    # worked out by hand from the definition: splitmix64(129279) =
    # 0x269DD7175F5319FF, low byte 0xFF = 255, so the k = 8 consecutive
    # experts wrap past E - 1 to 0
    E, k = 256, 8
    idx, _ = oracle.select_hash(np.array([129279], np.int64), np.zeros((1, E), np.float32), k)
    assert list(idx[0]) == [255, 0, 1, 2, 3, 4, 5, 6]
    assert oracle.splitmix64(129279) == 0x269DD7175F5319FF


def test_topk_nan_ranks_as_minus_inf():
    """NaN ranks as -inf: never ahead of a finite logit, tied with -inf (the
    lower index first), and its weight is exp(-inf) = 0."""
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    logits = np.array([[nan, 1.0, nan, 0.0],
                       [nan, -inf, 2.0, nan],
                       [-inf, nan, nan, nan]], np.float32)
    idx, w = oracle.select_topk(logits, 3)
    assert list(idx[0]) == [1, 3, 0]
    assert list(idx[1]) == [2, 0, 1]
    assert list(idx[2]) == [0, 1, 2]
    e = math.e
    np.testing.assert_allclose(w[0], [e / (e + 1), 1 / (e + 1), 0.0], rtol=1e-7, atol=0)
    assert list(w[1]) == [1.0, 0.0, 0.0]
    # brute force: a stable descending sort with NaN replaced by -inf
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((40, 16)).astype(np.float32)
    lg[rng.random((40, 16)) < 0.3] = np.nan
    lg[rng.random((40, 16)) < 0.1] = -np.inf
    idx, w = oracle.select_topk(lg, 6)
    ref = np.argsort(-np.where(np.isnan(lg), -np.inf, lg), axis=1, kind="stable")[:, :6]
    assert np.array_equal(idx, ref)
    assert not np.isnan(w).any()


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (4, 8, 2), (37, 16, 3), (200, 256, 8), (0, 4, 2)])
def test_dispatch_brute_force(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = np.array([rng.choice(E, k, replace=False) for _ in range(T)], np.int32).reshape(T, k)
    off, st, ss, sp = oracle.dispatch(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
    assert off[0] == 0 and off[-1] == T * k
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(ss, order)
    assert np.array_equal(st, order // k)
    assert np.array_equal(sp[ss], np.arange(T * k))
    for e in range(E):
        b = ss[off[e]:off[e + 1]]
        assert np.all(flat[b] == e) and np.all(np.diff(b) > 0)

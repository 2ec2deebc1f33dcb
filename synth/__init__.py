"""Seeded synthetic inputs for the routed-expert MoE FFN layer.

This module is the only code shared by the CPU oracle (``oracle/``) and the
GPU library's tests and benchmark.  It draws random bytes and random numbers
and nothing else: it decodes no weight format, computes no routing, no
dispatch and no FFN.  Quantized expert weights are produced by drawing the
fields of each block directly (random 2-bit codes, random 4-bit scale/min
nibbles, random codebook indices, random FP4 nibbles, fp16 or E8M0 scales
drawn from a range), sized so that the weights they encode have an rms near
0.02; no quantizer runs here.

Layer shapes follow the DeepSeek-V4-Flash-class routed MoE FFN of the ds4
pages (hidden 4096, 256 routed experts + 1 shared, expert intermediate 2048,
top-8) and a tiny 256/128/8-expert/top-2 layer for fast checks.

Storage of each projection (``N`` output rows, ``K`` input columns, ``E``
experts, expert-major):

* ``FMT_BF16``  -- ``uint16 [E, N, K]`` bf16 bit patterns.
* ``FMT_Q2K``   -- ``uint8 [E, N*K/256*84]``: the row-major flattened matrix
  cut into 256-weight super-blocks of 84 bytes each:
  ``uint8 sc[16]`` (low nibble = 4-bit scale, high nibble = 4-bit min of
  sub-block s), ``uint8 qs[64]`` (weight i of the block is
  ``(qs[i/4] >> 2*(i%4)) & 3``), ``fp16 d``, ``fp16 dmin``.
* ``FMT_VQ2``   -- codes plane ``uint8 [E, N, K/4]`` (one codebook index per
  4 consecutive weights), scale plane ``uint16 [E, N, K/256]`` (fp16 per 256
  weights), and one ``int8 [256, 4]`` codebook shared by the layer.
* ``FMT_MXFP4`` -- values plane ``uint8 [E, N, K/2]`` (E2M1 nibbles, even k in
  the low nibble) and scale plane ``uint8 [E, N, K/32]`` (E8M0 per 32).
"""
from __future__ import annotations

import dataclasses
import zlib

import numpy as np

FMT_BF16, FMT_Q2K, FMT_VQ2, FMT_MXFP4 = 0, 1, 2, 3
FMT_NAMES = {FMT_BF16: "bf16", FMT_Q2K: "q2k", FMT_VQ2: "vq2", FMT_MXFP4: "mxfp4"}
ROUTE_SOFTMAX_TOPK, ROUTE_HASH = 0, 1

Q2K_BLOCK_BYTES = 84
QK = 256  # weights per Q2K super-block / VQ2 scale group
MX_GROUP = 32  # weights per E8M0 scale
HASH_VOCAB = 129280  # token ids for hash routing are uniform in [0, HASH_VOCAB)

WEIGHT_RMS = 0.02


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    H: int  # hidden size
    I: int  # routed expert intermediate size
    E: int  # routed experts
    k: int  # experts per token
    fmt_gate: int
    fmt_up: int
    fmt_down: int
    I_shared: int  # shared-expert intermediate size (0 = no shared expert)


TINY = LayerSpec("tiny", 256, 128, 8, 2, FMT_Q2K, FMT_Q2K, FMT_Q2K, 128)
Q2 = LayerSpec("q2", 4096, 2048, 256, 8, FMT_VQ2, FMT_VQ2, FMT_Q2K, 2048)
MX = LayerSpec("mxfp4", 4096, 2048, 256, 8, FMT_MXFP4, FMT_MXFP4, FMT_MXFP4, 2048)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layer: LayerSpec
    T: int
    route: int = ROUTE_SOFTMAX_TOPK
    logits: str = "router"  # "router": computed from x and the router; "zipf": drawn
    act: int = 0  # activations of the routed experts: 0 bf16, 1 MX-FP8 (the A8 variant)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_t4", TINY, 4),
        Workload("decode_b1", Q2, 1),
        Workload("decode_b16_zipf", Q2, 16, logits="zipf"),
        # speculative-decode verification: each session checks its next token
        # plus 5 drafted ones in one step (1 + 5 = 6 tokens); one session, or
        # 16 sessions batched (96 tokens).  Tokens are drawn independently:
        # consecutive positions of one sequence would share experts more often.
        Workload("verify_t6", Q2, 6),
        Workload("verify_t6_zipf", Q2, 6, logits="zipf"),
        Workload("verify_t96", Q2, 96),
        Workload("verify_t96_zipf", Q2, 96, logits="zipf"),
        Workload("prefill_2048", Q2, 2048),
        Workload("prefill_4096", Q2, 4096),
        Workload("mxfp4_decode_b1", MX, 1),
        Workload("mxfp4_hash_decode_b1", MX, 1, route=ROUTE_HASH),
        Workload("mxfp4_prefill_2048", MX, 2048),
        Workload("mxfp4_prefill_4096", MX, 4096),
        Workload("mxfp4_hash_prefill_4096", MX, 4096, route=ROUTE_HASH),
        Workload("mxfp4_a8_prefill_4096", MX, 4096, act=1),
        Workload("mxfp4_hash_a8_prefill_4096", MX, 4096, route=ROUTE_HASH, act=1),
    ]
}


def _rng(seed: int, tag: str, *extra: int) -> np.random.Generator:
    """Independent stream per (seed, tensor tag, extra ids)."""
    return np.random.default_rng([seed & 0xFFFFFFFF, zlib.crc32(tag.encode()), *extra])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------

def gen_bf16(rng, shape, std):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


def gen_q2k(rng, E, N, K):
    """Q2K super-blocks with uniformly random codes and nibbles.

    The rms of d*(sc*q - 1.5*m) over uniform sc, m in 0..15 and q in 0..3 is
    about 13.9*d, so d is drawn around 0.02/13.9 and dmin around 1.5*d.
    """
    assert (N * K) % QK == 0
    nblk = N * K // QK
    raw = np.frombuffer(rng.bytes(E * nblk * Q2K_BLOCK_BYTES), dtype=np.uint8).copy()
    blk = raw.reshape(E * nblk, Q2K_BLOCK_BYTES)
    base = WEIGHT_RMS / 13.9
    u = rng.random((E * nblk, 2), dtype=np.float32)
    d = f32_to_f16_bits(base * (0.5 + u[:, 0]))
    dmin = f32_to_f16_bits(1.5 * base * (0.5 + u[:, 1]))
    blk[:, 80:82] = d.view(np.uint8).reshape(-1, 2)
    blk[:, 82:84] = dmin.view(np.uint8).reshape(-1, 2)
    return raw.reshape(E, nblk * Q2K_BLOCK_BYTES)


def gen_vq2_codebook(rng):
    return rng.integers(-127, 128, size=(256, 4), dtype=np.int8)


def gen_vq2(rng, E, N, K):
    """VQ2 planes: uniform codebook indices and an fp16 scale per 256 weights.

    Codebook entries are uniform in [-127, 127] (rms ~73.3), so d is drawn
    around 0.02/73.3.
    """
    assert K % QK == 0
    idx = np.frombuffer(rng.bytes(E * N * K // 4), dtype=np.uint8).reshape(E, N, K // 4).copy()
    base = WEIGHT_RMS / 73.3
    d = f32_to_f16_bits(base * (0.5 + rng.random((E, N, K // QK), dtype=np.float32)))
    return idx, d


def gen_mxfp4(rng, E, N, K):
    """MXFP4 planes: uniform E2M1 nibbles, E8M0 exponents uniform in [117, 121]."""
    assert K % MX_GROUP == 0
    vals = np.frombuffer(rng.bytes(E * N * K // 2), dtype=np.uint8).reshape(E, N, K // 2).copy()
    scales = rng.integers(117, 122, size=(E, N, K // MX_GROUP), dtype=np.uint8)
    return vals, scales


@dataclasses.dataclass
class Proj:
    """One projection of all experts: [E, N, K] in format ``fmt``."""
    fmt: int
    E: int
    N: int
    K: int
    data: np.ndarray  # bf16 bits | Q2K blocks | VQ2 codes | MXFP4 nibbles
    scales: np.ndarray | None = None  # VQ2 fp16 bits | MXFP4 E8M0
    codebook: np.ndarray | None = None  # VQ2 int8 [256, 4]

    def nbytes_per_expert(self) -> int:
        n = self.data.nbytes // self.E
        if self.scales is not None:
            n += self.scales.nbytes // self.E
        return n


def gen_proj(rng, fmt, E, N, K, codebook=None) -> Proj:
    if fmt == FMT_BF16:
        return Proj(fmt, E, N, K, gen_bf16(rng, (E, N, K), WEIGHT_RMS))
    if fmt == FMT_Q2K:
        return Proj(fmt, E, N, K, gen_q2k(rng, E, N, K))
    if fmt == FMT_VQ2:
        idx, d = gen_vq2(rng, E, N, K)
        return Proj(fmt, E, N, K, idx, d, codebook)
    if fmt == FMT_MXFP4:
        v, s = gen_mxfp4(rng, E, N, K)
        return Proj(fmt, E, N, K, v, s)
    raise ValueError(fmt)


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    w_router: np.ndarray  # uint16 [E, H] bf16
    gate: Proj  # [E, I, H]
    up: Proj  # [E, I, H]
    down: Proj  # [E, H, I]
    shared_gate: np.ndarray | None  # uint16 [I_s, H]
    shared_up: np.ndarray | None  # uint16 [I_s, H]
    shared_down: np.ndarray | None  # uint16 [H, I_s]
    codebook: np.ndarray | None  # int8 [256, 4] when a projection is VQ2

    def routed_bytes_per_expert(self) -> int:
        return sum(p.nbytes_per_expert() for p in (self.gate, self.up, self.down))

    def shared_bytes(self) -> int:
        if self.shared_gate is None:
            return 0
        return self.shared_gate.nbytes + self.shared_up.nbytes + self.shared_down.nbytes


def gen_layer(spec: LayerSpec, seed: int = 0) -> Layer:
    """All weights of one layer.  Router ~ N(0, 1/H) bf16, shared expert
    ~ N(0, 0.02^2) bf16, routed experts in their formats."""
    H, I, E = spec.H, spec.I, spec.E
    need_cb = FMT_VQ2 in (spec.fmt_gate, spec.fmt_up, spec.fmt_down)
    cb = gen_vq2_codebook(_rng(seed, "codebook")) if need_cb else None
    w_router = gen_bf16(_rng(seed, "router"), (E, H), 1.0 / np.sqrt(H))
    gate = gen_proj(_rng(seed, "gate"), spec.fmt_gate, E, I, H, cb)
    up = gen_proj(_rng(seed, "up"), spec.fmt_up, E, I, H, cb)
    down = gen_proj(_rng(seed, "down"), spec.fmt_down, E, H, I, cb)
    if spec.I_shared:
        Is = spec.I_shared
        sg = gen_bf16(_rng(seed, "shared_gate"), (Is, H), WEIGHT_RMS)
        su = gen_bf16(_rng(seed, "shared_up"), (Is, H), WEIGHT_RMS)
        sd = gen_bf16(_rng(seed, "shared_down"), (H, Is), WEIGHT_RMS)
    else:
        sg = su = sd = None
    return Layer(spec, w_router, gate, up, down, sg, su, sd, cb)


# ----------------------------------------------------------------------------
# per-step inputs
# ----------------------------------------------------------------------------

def gen_x(H: int, T: int, seed: int = 0, step: int = 0) -> np.ndarray:
    """Token activations ~ N(0, 1) rounded to bf16: uint16 [T, H]."""
    return gen_bf16(_rng(seed, "x", step), (T, H), 1.0)


def gen_zipf_logits(E: int, T: int, s: float = 1.1, seed: int = 0, step: int = 0) -> np.ndarray:
    """Router logits whose top-k picks follow a Zipf(s) expert popularity.

    logits[t, e] = ln p_e + G[t, e] with p_e proportional to (e+1)^-s and G
    i.i.d. standard Gumbel: the k largest of Gumbel-perturbed log
    probabilities are k draws without replacement in proportion to p.
    """
    rng = _rng(seed, "zipf", step)
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    g = rng.gumbel(size=(T, E))
    return (np.log(p)[None, :] + g).astype(np.float32)


def gen_token_ids(T: int, seed: int = 0, step: int = 0) -> np.ndarray:
    return _rng(seed, "token_ids", step).integers(0, HASH_VOCAB, size=T, dtype=np.int64)


def gen_step_inputs(w: Workload, seed: int = 0, step: int = 0):
    """(x, logits_in or None, token_ids or None) for one step of workload w."""
    x = gen_x(w.layer.H, w.T, seed, step)
    logits = gen_zipf_logits(w.layer.E, w.T, 1.1, seed, step) if w.logits == "zipf" else None
    tids = gen_token_ids(w.T, seed, step) if w.route == ROUTE_HASH else None
    return x, logits, tids


# ----------------------------------------------------------------------------
# stress tensors for bit-exact decode checks: every field drawn over its full
# bit range (fp16 scales over all finite patterns, subnormals included;
# E8M0 over 0..254).
# ----------------------------------------------------------------------------

def _finite_f16_bits(rng, n):
    b = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    inf_nan = (b & 0x7C00) == 0x7C00
    b[inf_nan] &= 0xBBFF  # clear one exponent bit: finite
    return b


def gen_stress_proj(fmt: int, N: int, K: int, seed: int = 0) -> Proj:
    rng = _rng(seed, "stress", fmt)
    if fmt == FMT_BF16:
        b = rng.integers(0, 1 << 16, size=(1, N, K), dtype=np.uint32).astype(np.uint16)
        b[(b & 0x7F80) == 0x7F80] &= 0xBF7F
        return Proj(fmt, 1, N, K, b)
    if fmt == FMT_Q2K:
        nblk = N * K // QK
        raw = np.frombuffer(rng.bytes(nblk * Q2K_BLOCK_BYTES), dtype=np.uint8).copy()
        blk = raw.reshape(nblk, Q2K_BLOCK_BYTES)
        blk[:, 80:82] = _finite_f16_bits(rng, nblk).view(np.uint8).reshape(-1, 2)
        blk[:, 82:84] = _finite_f16_bits(rng, nblk).view(np.uint8).reshape(-1, 2)
        return Proj(fmt, 1, N, K, raw.reshape(1, -1))
    if fmt == FMT_VQ2:
        idx = np.frombuffer(rng.bytes(N * K // 4), dtype=np.uint8).reshape(1, N, K // 4).copy()
        d = _finite_f16_bits(rng, N * K // QK).reshape(1, N, K // QK)
        cb = rng.integers(-128, 128, size=(256, 4), dtype=np.int8)
        return Proj(fmt, 1, N, K, idx, d, cb)
    if fmt == FMT_MXFP4:
        v = np.frombuffer(rng.bytes(N * K // 2), dtype=np.uint8).reshape(1, N, K // 2).copy()
        s = rng.integers(0, 255, size=(1, N, K // MX_GROUP), dtype=np.uint8)
        return Proj(fmt, 1, N, K, v, s)
    raise ValueError(fmt)

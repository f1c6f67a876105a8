"""Seeded synthetic inputs for the MoE layer (tests and bench both use them).

This module only draws random numbers and packs already-chosen integer fields
into the byte layouts that include/moe.h documents.  It holds none of the
layer's arithmetic: no dequantisation, no router, no FFN.  Random numbers
the method itself would draw do not exist here (the layer is deterministic).

Workloads (the pages print no test vectors; every workload is synthetic):

* ``tiny``      E=8, k=2, d=256, f=512, T=4, fp32 x.  Its weights are
                N(0, 0.02) floats (``gaussian``) encoded by the data-generation
                quantizers at the end of this module (``quantize_q2k`` and
                friends: offline encoders the layer never runs).
* ``decode``    E=384, k=6, d=4096, f=2048, T=1, fp32 x; gate/up IQ2XXS_L,
                down Q2K_L, shared expert Q8_0_L, all random valid codes.
                DeepSeek V4.1 Flash has 384 experts per layer and routes 6
                (YoungAi -- DeepSeek V4.1 Flash on one DGX Spark, section
                2.2); d = 4096 matches the 16 KB fp32 gate vectors mentioned
                for V4 Flash on the RTX 5080 / ds4 page (two-Mac tensor
                parallel section).
* ``prefill``   the decode layer, T=1024 bf16 x (the RTX 5080 fork uses a
                1,024-token prefill chunk), routes from the real router.
* ``small_batch`` the decode layer, T=16 = 4 sessions x 4 consecutive tokens
                with expert reuse between consecutive tokens of a session.
* ``long_prefill`` 8 layers of the decode shape, T=4096 bf16, Zipf(1.1)
                expert popularity.

Seeds: every tensor has its own ``numpy.random.SeedSequence`` keyed by
(seed, workload, layer, expert, tensor name), so any single expert can be
regenerated on the host without building the whole layer.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

FMT_NONE, FMT_IQ2, FMT_Q2K, FMT_Q8, FMT_Q4K, FMT_MX4, FMT_VQ12, FMT_VQ13 = 0, 1, 2, 3, 4, 5, 6, 7
BLOCK_WEIGHTS = {FMT_IQ2: 256, FMT_Q2K: 256, FMT_Q8: 32, FMT_Q4K: 256, FMT_MX4: 32}
BLOCK_BYTES = {FMT_IQ2: 66, FMT_Q2K: 84, FMT_Q8: 34, FMT_Q4K: 144, FMT_MX4: 17}
VQ_FORMATS = (FMT_VQ12, FMT_VQ13)
VQ_CODES = {FMT_VQ12: 4096, FMT_VQ13: 8192}

F32, BF16 = 0, 1


# --------------------------------------------------------------------------
# seeding
# --------------------------------------------------------------------------
def _key_int(part) -> int:
    if isinstance(part, (int, np.integer)):
        return int(part) & 0xFFFFFFFF
    return zlib.crc32(str(part).encode())


def rng_for(seed: int, *key) -> np.random.Generator:
    """A PCG64 generator for (seed, *key); key parts are ints or strings."""
    ss = np.random.SeedSequence(entropy=int(seed), spawn_key=tuple(_key_int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------
# bit-level helpers (no arithmetic of the layer)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (round to nearest even); uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _u32_le_bytes(v: np.ndarray) -> np.ndarray:
    """uint32 [..., n] -> uint8 [..., 4n], little-endian."""
    return np.ascontiguousarray(v.astype("<u4")).view(np.uint8)


# --------------------------------------------------------------------------
# packers: integer fields -> canonical bytes (layouts of include/moe.h)
# --------------------------------------------------------------------------
def pack_iq2(d: np.ndarray, grid_row: np.ndarray, signs7: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """IQ2XXS_L blocks.

    d        float16 [nb]           superblock scale
    grid_row uint8   [nb, 32]       grid row of each 8-weight group
    signs7   uint8   [nb, 32]       7 stored sign bits of each group (0..127)
    scale    uint8   [nb, 8]        4-bit sub-block scales (0..15)
    returns  uint8   [nb, 66]
    """
    nb = d.shape[0]
    out = np.empty((nb, 66), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(nb, 2)
    g = grid_row.reshape(nb, 8, 4).astype(np.uint8)
    s7 = signs7.reshape(nb, 8, 4).astype(np.uint32)
    b = (s7[:, :, 0] | (s7[:, :, 1] << 7) | (s7[:, :, 2] << 14) | (s7[:, :, 3] << 21)
         | (scale.astype(np.uint32) << 28))
    pairs = np.empty((nb, 8, 8), dtype=np.uint8)
    pairs[:, :, 0:4] = g
    pairs[:, :, 4:8] = _u32_le_bytes(b).reshape(nb, 8, 4)
    out[:, 2:66] = pairs.reshape(nb, 64)
    return out


def pack_q2k(d: np.ndarray, dmin: np.ndarray, sc: np.ndarray, m: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Q2K_L blocks.

    d, dmin float16 [nb]; sc, m uint8 [nb, 16] (0..15); q uint8 [nb, 256] (0..3)
    returns uint8 [nb, 84]
    """
    nb = d.shape[0]
    out = np.empty((nb, 84), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = np.ascontiguousarray(dmin.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 4:20] = (sc.astype(np.uint8) & 15) | ((m.astype(np.uint8) & 15) << 4)
    qq = q.reshape(nb, 64, 4).astype(np.uint8) & 3
    out[:, 20:84] = qq[:, :, 0] | (qq[:, :, 1] << 2) | (qq[:, :, 2] << 4) | (qq[:, :, 3] << 6)
    return out


def pack_q4k(d: np.ndarray, dmin: np.ndarray, sc: np.ndarray, m: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Q4K_L blocks.

    d, dmin float16 [nb]; sc, m uint8 [nb, 8] (0..63); q uint8 [nb, 256] (0..15)
    returns uint8 [nb, 144]
    """
    nb = d.shape[0]
    sc = sc.astype(np.uint8) & 63
    m = m.astype(np.uint8) & 63
    out = np.empty((nb, 144), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = np.ascontiguousarray(dmin.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 4:12] = (sc & 15) | ((m & 15) << 4)
    top = (sc >> 4) | ((m >> 4) << 2)  # 4 bits per sub-block
    out[:, 12:16] = top[:, 0::2] | (top[:, 1::2] << 4)
    qq = q.reshape(nb, 128, 2).astype(np.uint8) & 15
    out[:, 16:144] = qq[:, :, 0] | (qq[:, :, 1] << 4)
    return out


def pack_mx4(e: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """MXFP4_L blocks.  e uint8 [nb] (E8M0 scale exponents, 0..254); codes
    uint8 [nb, 32] (E2M1 codes 0..15); returns uint8 [nb, 17]."""
    nb = e.shape[0]
    out = np.empty((nb, 17), dtype=np.uint8)
    out[:, 0] = e.astype(np.uint8)
    c = codes.reshape(nb, 16, 2).astype(np.uint8) & 15
    out[:, 1:17] = c[:, :, 0] | (c[:, :, 1] << 4)
    return out


def pack_vq(gain: np.ndarray, idx: np.ndarray, bits: int) -> np.ndarray:
    """VQ12_L / VQ13_L rows.  gain float16 [R]; idx integers [R, K/8] below
    2^bits (bits 12 or 13); returns uint8 [R, 2 + 3K/16 (+ K/64 for 13)]:
    the fp16 gain, the low 12 bits of every index as one little-endian bit
    stream (index j at stream bits 12j..12j+11), then for 13 bits a plane
    holding bit 12 of index j at bit j."""
    idx = np.asarray(idx, dtype=np.int64)
    R, n = idx.shape
    assert n % (8 if bits == 13 else 2) == 0 and bits in (12, 13) and idx.min(initial=0) >= 0 and idx.max(initial=0) < (1 << bits)
    lo = idx & 0xFFF
    pairs = lo.reshape(R, n // 2, 2)  # two 12-bit indices = three bytes
    v = pairs[:, :, 0] | (pairs[:, :, 1] << 12)
    stream = np.stack([v & 255, (v >> 8) & 255, (v >> 16) & 255], axis=2).reshape(R, 3 * n // 2)
    parts = [np.ascontiguousarray(gain.astype("<f2")).view(np.uint8).reshape(R, 2), stream.astype(np.uint8)]
    if bits == 13:
        hi = ((idx >> 12) & 1).reshape(R, n // 8, 8)
        parts.append((hi << np.arange(8)).sum(axis=2).astype(np.uint8))
    return np.concatenate(parts, axis=1)


def pack_q8(d: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Q8_0_L blocks.  d float16 [nb]; q int8 [nb, 32]; returns uint8 [nb, 34]."""
    nb = d.shape[0]
    out = np.empty((nb, 34), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d.astype("<f2")).view(np.uint8).reshape(nb, 2)
    out[:, 2:34] = q.astype(np.int8).view(np.uint8)
    return out


# --------------------------------------------------------------------------
# random valid codes
# --------------------------------------------------------------------------
# Scale magnitudes give dequantised weights a standard deviation near 0.02
# (the spread the tiny workload states for its float weights):
#   IQ2: |k| = (2s+1)*mag with s ~ U{0..15}, mag ~ U{1,3,5,7}:
#        E[k^2] = 341 * 21  ->  std 84.6  ->  d ~ 2.36e-4
#   Q2K: sc, m ~ U{0..15}, q ~ U{0..3}; dmin = 1.5 d centres the weights;
#        std ~ 14.9 d  ->  d ~ 1.35e-3
#   Q8 : q ~ U{-128..127}, std ~ 73.9  ->  d ~ 2.7e-4
#   Q4K: sc, m ~ U{0..63}, q ~ U{0..15}; dmin = 7.5 d centres the weights;
#        var = var(sc q) + 7.5^2 var(m) = 47532 + 19195 -> std 258 d -> d ~ 7.74e-5
#   MX4: E2M1 codes ~ U{0..15}: E[v^2] = 8.5625 -> std 2.93; the E8M0
#        exponent drawn from {119, 120} (scale 2^-8 or 2^-7): std ~ 0.018
#   VQ : codewords from make_codebook have an RMS near 1.5, so a row gain
#        near 0.0137 gives std ~ 0.02
IQ2_D, Q2K_D, Q8_D, Q4K_D = 2.36e-4, 1.35e-3, 2.7e-4, 7.74e-5
MX4_E = 120
VQ_G = 0.0137


def _rand_scale(rng, nb, base):
    # vary the per-block scale by up to a factor sqrt(2) either way so that
    # using the wrong block's scale changes the result
    return (base * np.exp2(rng.uniform(-0.5, 0.5, size=nb))).astype(np.float16)


def _random_blocks(rng, nb, nbytes):
    # every bit pattern of the quant fields (grid rows, signs, sub-block
    # scales and mins, 2-bit and 8-bit quants) is a valid code, so a block of
    # random codes is random bytes with its fp16 scale fields set afterwards
    return np.frombuffer(rng.bytes(nb * nbytes), dtype=np.uint8).reshape(nb, nbytes).copy()


def _put_f16(blocks, offset, values):
    blocks[:, offset:offset + 2] = np.ascontiguousarray(values.astype("<f2")).view(np.uint8).reshape(-1, 2)


def random_iq2(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Random IQ2XXS_L blocks: uniform grid rows, signs and sub-block scales."""
    out = _random_blocks(rng, nb, 66)
    _put_f16(out, 0, _rand_scale(rng, nb, IQ2_D))
    return out


def random_q2k(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Random Q2K_L blocks: uniform sub-block scales, mins and 2-bit quants;
    dmin = 1.5 d centres the weights on zero."""
    out = _random_blocks(rng, nb, 84)
    d = _rand_scale(rng, nb, Q2K_D)
    _put_f16(out, 0, d)
    _put_f16(out, 2, (d.astype(np.float32) * 1.5).astype(np.float16))
    return out


def random_q4k(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Random Q4K_L blocks: uniform 6-bit sub-block scales and mins, 4-bit
    quants; dmin = 7.5 d centres the weights on zero."""
    out = _random_blocks(rng, nb, 144)
    d = _rand_scale(rng, nb, Q4K_D)
    _put_f16(out, 0, d)
    _put_f16(out, 2, (d.astype(np.float32) * 7.5).astype(np.float16))
    return out


def random_q8(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Random Q8_0_L blocks: uniform int8 quants in -128..127."""
    out = _random_blocks(rng, nb, 34)
    _put_f16(out, 0, _rand_scale(rng, nb, Q8_D))
    return out


def random_mx4(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Random MXFP4_L blocks: uniform E2M1 codes, scale exponent MX4_E - 1
    or MX4_E."""
    out = _random_blocks(rng, nb, 17)
    out[:, 0] = (MX4_E + rng.integers(-1, 1, size=nb)).astype(np.uint8)
    return out


def random_vq(rng: np.random.Generator, rows: int, K: int, bits: int) -> np.ndarray:
    """Random VQ rows: uniform indices below 2^bits, gains near VQ_G."""
    gain = _rand_scale(rng, rows, VQ_G)
    idx = rng.integers(0, 1 << bits, size=(rows, K // 8))
    return pack_vq(gain, idx, bits)


RANDOM_CODES = {FMT_IQ2: random_iq2, FMT_Q2K: random_q2k, FMT_Q8: random_q8, FMT_Q4K: random_q4k,
                FMT_MX4: random_mx4}


def row_bytes(fmt: int, K: int) -> int:
    """Bytes of one canonical row of K weights."""
    if fmt in VQ_FORMATS:
        return 2 + 3 * K // 16 + (K // 64 if fmt == FMT_VQ13 else 0)
    return (K // BLOCK_WEIGHTS[fmt]) * BLOCK_BYTES[fmt]


def matrix_bytes(fmt: int, n_experts: int, rows: int, K: int) -> int:
    return n_experts * rows * row_bytes(fmt, K)


def random_matrix(seed, tag, fmt: int, rows: int, K: int) -> np.ndarray:
    """One expert's matrix of random valid codes: uint8 [rows * row_bytes]."""
    rng = rng_for(seed, *tag)
    if fmt in VQ_FORMATS:
        return random_vq(rng, rows, K, 12 if fmt == FMT_VQ12 else 13).reshape(-1)
    nb = rows * (K // BLOCK_WEIGHTS[fmt])
    return RANDOM_CODES[fmt](rng, nb).reshape(-1)


E4M3_NAN = (0x7F, 0xFF)


def make_codebook(seed: int, n: int, tag=(), every_code: bool = False) -> np.ndarray:
    """A per-layer codebook of n codewords of 8 E4M3 bytes: uint8 [n, 8].

    The first codewords hold, in increasing byte order, every code whose
    exponent field is at most 9 (magnitudes up to 7.5: both zeros, every
    subnormal, the small normals; 160 codes = 20 codewords), or with
    every_code all 256 byte values (32 codewords, the two not-a-number codes
    replaced by +0 and -0, so up to the largest magnitude 448).  The others
    take a random sign, a random 3-bit mantissa and an exponent field in
    4..8 (magnitudes 0.125 .. 3.75, RMS near 1.5, like codewords trained on
    rows normalised to unit RMS)."""
    rng = rng_for(seed, "vq-codebook", n, *tag)
    codes = np.arange(256, dtype=np.int64)
    if every_code:
        codes[0x7F], codes[0xFF] = 0x00, 0x80
    else:
        codes = codes[((codes >> 3) & 15) <= 9]
    first = codes.reshape(-1, 8)
    cb = np.empty((n, 8), dtype=np.uint8)
    cb[:len(first)] = first
    m = n - len(first)
    sign = rng.integers(0, 2, size=(m, 8)) << 7
    expo = rng.integers(4, 9, size=(m, 8)) << 3
    mant = rng.integers(0, 8, size=(m, 8))
    cb[len(first):] = (sign | expo | mant).astype(np.uint8)
    return cb


def make_grid(seed: int) -> np.ndarray:
    """A 256 x 8 grid of magnitudes in {1,3,5,7} with distinct rows."""
    rng = rng_for(seed, "iq2-grid")
    grid = (2 * rng.integers(0, 4, size=(256, 8)) + 1).astype(np.uint8)
    while True:
        _, first = np.unique(grid, axis=0, return_index=True)
        dup = np.setdiff1d(np.arange(256), first)
        if dup.size == 0:
            return grid
        grid[dup] = (2 * rng.integers(0, 4, size=(dup.size, 8)) + 1).astype(np.uint8)


def gaussian(seed, tag, shape, std=0.02) -> np.ndarray:
    return (rng_for(seed, *tag).standard_normal(size=shape) * std).astype(np.float32)


def activations(seed, tag, T: int, d: int, dtype: int) -> np.ndarray:
    """x ~ N(0, 1); fp32 array, or bf16 bits (uint16) when dtype == BF16."""
    x = rng_for(seed, *tag).standard_normal(size=(T, d)).astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == BF16 else x


def router_weights(seed, tag, E: int, d: int) -> np.ndarray:
    return gaussian(seed, tag, (E, d), 0.02)


# --------------------------------------------------------------------------
# caller-supplied routes (small_batch and long_prefill)
# --------------------------------------------------------------------------
def _mixing_weights(rng, T, k):
    # caller-supplied mixing weights: positive, best first, summing to one
    # (Dirichlet draws sorted in decreasing order)
    w = -np.sort(-rng.dirichlet(np.full(k, 2.0), size=T), axis=1)
    return w.astype(np.float32)


def session_routes(seed, E=384, k=6, sessions=4, steps=4, keep_p=1.0 / 3.0, tag="small_batch"):
    """Routes for `sessions` interleaved sessions of `steps` consecutive tokens.

    Token t = steps_index * sessions + session.  The first token of a session
    draws k distinct experts; each later token keeps r ~ Binomial(k, keep_p)
    of its predecessor's experts and draws k - r fresh ones that are not in
    its set yet.  With keep_p = 1/3 the mean number of distinct experts over
    1..5 consecutive tokens is close to the 6 / 10.0 / 13.3 / 17.4 / 21.7
    the YoungAi page (section 2.2) reports for DeepSeek V4.1 Flash routing.
    Returns (idx int32 [T, k], wt fp32 [T, k]).
    """
    rng = rng_for(seed, tag, "routes")
    T = sessions * steps
    idx = np.empty((T, k), dtype=np.int32)
    for s in range(sessions):
        prev = None
        for p in range(steps):
            if prev is None:
                cur = rng.choice(E, size=k, replace=False)
            else:
                r = rng.binomial(k, keep_p)
                kept = rng.choice(prev, size=r, replace=False)
                pool = np.setdiff1d(np.arange(E), kept)
                fresh = rng.choice(pool, size=k - r, replace=False)
                cur = np.concatenate([kept, fresh])
                rng.shuffle(cur)
            idx[p * sessions + s] = cur
            prev = cur
    return idx, _mixing_weights(rng, T, k)


def zipf_routes(seed, T, E=384, k=6, s=1.1, layer=0, tag="long_prefill"):
    """Zipf(s)-skewed routes: expert popularity p_r ~ r^-s over ranks 1..E,
    a seeded per-layer permutation maps rank to expert id, and each token
    takes k distinct experts by Gumbel-top-k on log p (sampling without
    replacement).  Returns (idx int32 [T, k], wt fp32 [T, k])."""
    rng = rng_for(seed, tag, "routes", layer)
    perm = rng.permutation(E)
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    g = logp[None, :] + rng.gumbel(size=(T, E))
    ranks = np.argsort(-g, axis=1, kind="stable")[:, :k]
    idx = perm[ranks].astype(np.int32)
    return idx, _mixing_weights(rng, T, k)


# --------------------------------------------------------------------------
# layers
# --------------------------------------------------------------------------
@dataclass
class LayerSpec:
    E: int
    k: int
    d: int
    f: int
    fmt_gate_up: int
    fmt_down: int
    has_shared: bool
    fmt_shared: int = FMT_Q8


@dataclass
class Layer:
    """Canonical bytes of one layer (host numpy arrays)."""
    spec: LayerSpec
    w_gate: np.ndarray    # uint8, matrix_bytes(fmt_gate_up, E, f, d)
    w_up: np.ndarray
    w_down: np.ndarray    # uint8, matrix_bytes(fmt_down, E, d, f)
    grid: np.ndarray      # uint8 [256, 8]
    w_router: np.ndarray  # float32 [E, d]
    s_gate: np.ndarray | None = None
    s_up: np.ndarray | None = None
    s_down: np.ndarray | None = None
    router_bias: np.ndarray | None = None  # float32 [E]: selection-only bias (None: select on the logits)
    down_gain: np.ndarray | None = None    # float32 [E, d]: per-channel down gains (None: ones)
    vq_codebook: np.ndarray | None = None  # uint8 [4096 or 8192, 8] E4M3 codewords (VQ routed formats)
    meta: dict = field(default_factory=dict)


DECODE_SPEC = LayerSpec(E=384, k=6, d=4096, f=2048, fmt_gate_up=FMT_IQ2, fmt_down=FMT_Q2K,
                        has_shared=True, fmt_shared=FMT_Q8)
TINY_SPEC = LayerSpec(E=8, k=2, d=256, f=512, fmt_gate_up=FMT_Q2K, fmt_down=FMT_Q2K, has_shared=False)


def random_layer(spec: LayerSpec, seed: int = 0, workload: str = "decode", layer: int = 0,
                 experts: list[int] | None = None) -> Layer:
    """A layer of random valid codes.

    experts: generate only these experts (others left zero) -- lets a host
    check regenerate exactly the experts it needs; the bytes of each
    generated expert do not depend on which others are generated.
    """
    E, d, f = spec.E, spec.d, spec.f
    gu = matrix_bytes(spec.fmt_gate_up, 1, f, d)
    dn = matrix_bytes(spec.fmt_down, 1, d, f)
    w_gate = np.zeros(E * gu, dtype=np.uint8)
    w_up = np.zeros(E * gu, dtype=np.uint8)
    w_down = np.zeros(E * dn, dtype=np.uint8)
    for e in (range(E) if experts is None else experts):
        w_gate[e * gu:(e + 1) * gu] = random_matrix(seed, (workload, layer, e, "gate"), spec.fmt_gate_up, f, d)
        w_up[e * gu:(e + 1) * gu] = random_matrix(seed, (workload, layer, e, "up"), spec.fmt_gate_up, f, d)
        w_down[e * dn:(e + 1) * dn] = random_matrix(seed, (workload, layer, e, "down"), spec.fmt_down, d, f)
    L = Layer(spec=spec, w_gate=w_gate, w_up=w_up, w_down=w_down, grid=make_grid(seed),
              w_router=router_weights(seed, (workload, layer, "router"), E, d))
    n_codes = codebook_size(spec)
    if n_codes:
        L.vq_codebook = make_codebook(seed, n_codes, (workload, layer))
    if spec.has_shared:
        L.s_gate = random_matrix(seed, (workload, layer, "shared", "gate"), spec.fmt_shared, f, d)
        L.s_up = random_matrix(seed, (workload, layer, "shared", "up"), spec.fmt_shared, f, d)
        L.s_down = random_matrix(seed, (workload, layer, "shared", "down"), spec.fmt_shared, d, f)
    return L


def codebook_size(spec: LayerSpec) -> int:
    """Codewords a layer's codebook needs (0: no VQ routed format)."""
    return max([VQ_CODES.get(spec.fmt_gate_up, 0), VQ_CODES.get(spec.fmt_down, 0)])


def scaled_spec(E, k, d, f, fmt_gate_up=FMT_IQ2, fmt_down=FMT_Q2K, has_shared=True, fmt_shared=FMT_Q8):
    return LayerSpec(E=E, k=k, d=d, f=f, fmt_gate_up=fmt_gate_up, fmt_down=fmt_down,
                     has_shared=has_shared, fmt_shared=fmt_shared)


WORKLOADS = {
    # name: (spec, T, x dtype, route source)
    "tiny": (TINY_SPEC, 4, F32, "router"),
    "decode": (DECODE_SPEC, 1, F32, "router"),
    "prefill": (DECODE_SPEC, 1024, BF16, "router"),
    "small_batch": (DECODE_SPEC, 16, F32, "sessions"),
    "long_prefill": (DECODE_SPEC, 4096, BF16, "zipf"),
}
LONG_PREFILL_LAYERS = 8


# --------------------------------------------------------------------------
# encoders for float weights (offline tooling: the layer never quantizes;
# these only turn the tiny workload's N(0, 0.02) floats into codes)
# --------------------------------------------------------------------------
def _safe_div(a, b):
    out = np.zeros(np.broadcast(a, b).shape, dtype=np.float64)
    np.divide(a, b, out=out, where=(b != 0))
    return out


def quantize_q2k(w: np.ndarray) -> np.ndarray:
    """Float weights [nb * 256] -> Q2K_L blocks [nb, 84].

    Per 16-weight sub-block: lo = min(0, min w), hi = max w, step a = (hi - lo)/3,
    offset b = -lo.  The superblock scales are d = fp16(max a / 15) and
    dmin = fp16(max b / 15); sub-block scale and min are rint(a / d) and
    rint(b / dmin) clamped to 0..15, computed with the fp16-rounded d and
    dmin; q = rint((w + dmin m) / (d sc)) clamped to 0..3 (q = 0 when the
    sub-block scale is 0).  Choosing codes with the scales already rounded to
    their stored precision follows the YoungAi page, section 4.1 (the final
    assignment uses the stored-precision codebook and gains).
    """
    w = np.asarray(w, dtype=np.float64).reshape(-1, 16, 16)
    nb = w.shape[0]
    lo = np.minimum(0.0, w.min(axis=2))
    hi = w.max(axis=2)
    a = (hi - lo) / 3.0
    b = -lo
    d = (a.max(axis=1) / 15.0).astype(np.float16)
    dmin = (b.max(axis=1) / 15.0).astype(np.float16)
    df = d.astype(np.float64)[:, None]
    dmf = dmin.astype(np.float64)[:, None]
    sc = np.clip(np.rint(_safe_div(a, df)), 0, 15)
    m = np.clip(np.rint(_safe_div(b, dmf)), 0, 15)
    step = (df * sc)[:, :, None]
    q = np.clip(np.rint(_safe_div(w + (dmf * m)[:, :, None], step)), 0, 3)
    q = np.where(step > 0, q, 0)
    return pack_q2k(d, dmin, sc.astype(np.uint8), m.astype(np.uint8), q.reshape(nb, 256).astype(np.uint8))


def quantize_q8(w: np.ndarray) -> np.ndarray:
    """Float weights [nb * 32] -> Q8_0_L blocks [nb, 34]:
    d = fp16(max |w| / 127), q = rint(w / d) clamped to -127..127."""
    w = np.asarray(w, dtype=np.float64).reshape(-1, 32)
    d = (np.abs(w).max(axis=1) / 127.0).astype(np.float16)
    q = np.clip(np.rint(_safe_div(w, d.astype(np.float64)[:, None])), -127, 127).astype(np.int8)
    return pack_q8(d, q)


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # magnitudes of codes 0..7 (OCP MX)


def quantize_mx4(w: np.ndarray) -> np.ndarray:
    """Float weights [nb * 32] -> MXFP4_L blocks [nb, 17]: the scale is the
    smallest power of two 2^k with max|w| / 2^k <= 6 (k clamped to the E8M0
    range), each weight takes the nearest E2M1 magnitude of |w| / 2^k (ties
    to the even code) and the sign of w (zero keeps code 0)."""
    w = np.asarray(w, dtype=np.float64).reshape(-1, 32)
    nb = w.shape[0]
    amax = np.abs(w).max(axis=1)
    k = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / 6.0)), 0).astype(np.int64)
    k = np.clip(k, -127, 127)
    v = np.abs(w) / np.exp2(k)[:, None]
    dist = np.abs(v[:, :, None] - E2M1_GRID[None, None, :])
    best = np.argmin(dist + 1e-12 * (np.arange(8) % 2)[None, None, :], axis=2)  # ties: even code
    codes = best.astype(np.uint8) | np.where((w < 0) & (best > 0), 8, 0).astype(np.uint8)
    return pack_mx4((k + 127).astype(np.uint8), codes)


def quantize_iq2(w: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Float weights [nb * 256] -> IQ2XXS_L blocks [nb, 66] by exhaustive search.

    d = fp16(max |w| / 217) (217 = 31 * 7 is the largest code magnitude); per
    sub-block every scale s in 0..15 is tried; per 8-weight group the signs
    are those of w (if their count of negatives is odd, the smallest |w| in
    the group takes the other sign) and the grid row minimises the squared
    error.  Slow; meant for a handful of blocks.
    """
    w = np.asarray(w, dtype=np.float64).reshape(-1, 8, 4, 8)
    nb = w.shape[0]
    g = grid.astype(np.float64)
    d = (np.abs(w).reshape(nb, -1).max(axis=1) / 217.0).astype(np.float16)
    rows = np.zeros((nb, 8, 4), dtype=np.uint8)
    signs = np.zeros((nb, 8, 4), dtype=np.uint8)
    scales = np.zeros((nb, 8), dtype=np.uint8)
    for b in range(nb):
        db = float(d[b])
        for j in range(8):
            best = None
            for s in range(16):
                step = db * (2 * s + 1)
                err_total, pick = 0.0, []
                for i in range(4):
                    v = w[b, j, i]
                    neg = v < 0
                    if neg.sum() % 2:
                        neg = neg.copy()
                        p = int(np.argmin(np.abs(v)))
                        neg[p] = not neg[p]
                    sgn = np.where(neg, -1.0, 1.0)
                    err = ((v[None, :] - step * g * sgn[None, :]) ** 2).sum(axis=1)
                    r = int(np.argmin(err))
                    err_total += float(err[r])
                    bits = int(sum(1 << p for p in range(7) if neg[p]))
                    pick.append((r, bits))
                if best is None or err_total < best[0]:
                    best = (err_total, s, pick)
            _, s, pick = best
            scales[b, j] = s
            for i, (r, bits) in enumerate(pick):
                rows[b, j, i] = r
                signs[b, j, i] = bits
    return pack_iq2(d, rows.reshape(nb, 32), signs.reshape(nb, 32), scales)


def tiny_layer(seed: int = 0, spec: LayerSpec = TINY_SPEC, workload: str = "tiny") -> Layer:
    """The tiny workload: N(0, 0.02) weights quantized per `spec` formats."""
    enc = {FMT_Q2K: quantize_q2k, FMT_Q8: quantize_q8}
    E, d, f = spec.E, spec.d, spec.f

    def mat(tag, fmt, rows, K):
        return enc[fmt](gaussian(seed, (workload,) + tag, (rows, K))).reshape(-1)

    w_gate = np.concatenate([mat((e, "gate"), spec.fmt_gate_up, f, d) for e in range(E)])
    w_up = np.concatenate([mat((e, "up"), spec.fmt_gate_up, f, d) for e in range(E)])
    w_down = np.concatenate([mat((e, "down"), spec.fmt_down, d, f) for e in range(E)])
    L = Layer(spec=spec, w_gate=w_gate, w_up=w_up, w_down=w_down, grid=make_grid(seed),
              w_router=router_weights(seed, (workload, "router"), E, d))
    if spec.has_shared:
        L.s_gate = mat(("shared", "gate"), spec.fmt_shared, f, d)
        L.s_up = mat(("shared", "up"), spec.fmt_shared, f, d)
        L.s_down = mat(("shared", "down"), spec.fmt_shared, d, f)
    return L

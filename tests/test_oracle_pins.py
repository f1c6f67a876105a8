"""Pins of the CPU oracle to things other than itself.

Each test ties one oracle function to a closed form, a hand-worked value, a
textbook/library routine it does not use, an invariant, or brute force, so
that a plausible slip (a dropped term, a wrong sign or index, a transposed
operand, a different summation order) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from quantized_moe_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_worked_values.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _bytes(h):
    return np.frombuffer(bytes.fromhex(h.replace(" ", "")), dtype=np.uint8)


# ---------------------------------------------------------------- fp16 ----
def test_half_matches_numpy_float16_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


# ------------------------------------------------------- formats: worked ----
def _golden_grid(g):
    grid = np.ones((256, 8), dtype=np.uint8)
    for r, vals in g["iq2_grid_rows"].items():
        grid[int(r)] = vals
    return grid


def test_iq2_worked_blocks():
    g = _golden()
    grid = _golden_grid(g)
    base = {b["name"]: b for b in g["iq2_blocks"]}
    for b in g["iq2_blocks"]:
        groups = base[b.get("same_groups_as", b["name"])]["groups"]
        want = np.array(groups, dtype=np.float64).reshape(-1) * b["scale"]
        got = oracle.dequant(oracle.IQ2, _bytes(b["hex"]), grid)
        assert np.array_equal(got, want), b["name"]


def test_iq2_packer_reproduces_hand_bytes():
    b = _golden()["iq2_blocks"][0]
    f = b["fields"]
    packed = synth.pack_iq2(np.array([1.0], np.float16), np.array([f["rows"]], np.uint8),
                            np.array([f["signs7"]], np.uint8), np.array([f["scales"]], np.uint8))
    assert np.array_equal(packed.reshape(-1), _bytes(b["hex"]))


def test_q2k_worked_block_and_packer():
    b = _golden()["q2k_blocks"][0]
    want = np.array(b["subblocks"], dtype=np.float64).reshape(-1)
    assert np.array_equal(oracle.dequant(oracle.Q2K, _bytes(b["hex"])), want)
    f = b["fields"]
    q = np.tile([0, 1, 2, 3], 64).reshape(16, 16).astype(np.uint8)
    q[1] = 3
    q[2] = 2
    packed = synth.pack_q2k(np.array([0.5], np.float16), np.array([0.25], np.float16),
                            np.array([f["sc"]], np.uint8), np.array([f["m"]], np.uint8), q.reshape(1, 256))
    assert np.array_equal(packed.reshape(-1), _bytes(b["hex"]))


def test_q4k_worked_block_and_packer():
    b = _golden()["q4k_blocks"][0]
    want = np.array(b["subblocks"], dtype=np.float64).reshape(-1)
    assert np.array_equal(oracle.dequant(oracle.Q4K, _bytes(b["hex"])), want)
    f = b["fields"]
    q = np.tile(np.arange(16), 16).reshape(8, 32).astype(np.uint8)
    q[1], q[2], q[3] = 15, 7, 1
    packed = synth.pack_q4k(np.array([0.5], np.float16), np.array([0.25], np.float16),
                            np.array([f["sc"]], np.uint8), np.array([f["m"]], np.uint8), q.reshape(1, 256))
    assert np.array_equal(packed.reshape(-1), _bytes(b["hex"]))


def test_q4k_agrees_with_q2k_where_both_can_hold_the_block():
    # A Q4K block whose 6-bit scales and mins fit 4 bits and whose quants fit
    # 2 bits holds the same weights as the Q2K block with those fields (each
    # 32-weight sub-block as two 16-weight ones): two decoders of different
    # byte layouts must agree exactly.
    rng = np.random.default_rng(5)
    nb = 32
    d = (rng.uniform(0.5, 2.0, nb) * 1e-3).astype(np.float16)
    dmin = (rng.uniform(0.5, 2.0, nb) * 1e-3).astype(np.float16)
    sc = rng.integers(0, 16, (nb, 8)).astype(np.uint8)
    m = rng.integers(0, 16, (nb, 8)).astype(np.uint8)
    q = rng.integers(0, 4, (nb, 256)).astype(np.uint8)
    w4 = oracle.dequant(oracle.Q4K, synth.pack_q4k(d, dmin, sc, m, q))
    w2 = oracle.dequant(oracle.Q2K, synth.pack_q2k(d, dmin, np.repeat(sc, 2, axis=1), np.repeat(m, 2, axis=1), q))
    assert np.array_equal(w4, w2)
    # the top bits: sc + 16 t adds 16 t d q to every weight of the sub-block,
    # m + 16 t subtracts 16 t dmin
    for j in range(8):
        for field in ("sc", "m"):
            sc2, m2 = sc.copy(), m.copy()
            (sc2 if field == "sc" else m2)[:, j] += 48
            w = oracle.dequant(oracle.Q4K, synth.pack_q4k(d, dmin, sc2, m2, q)).reshape(nb, 8, 32)
            delta = w - w4.reshape(nb, 8, 32)
            others = [i for i in range(8) if i != j]
            assert np.all(delta[:, others] == 0)
            if field == "sc":
                expect = 48 * d.astype(np.float64)[:, None] * q.reshape(nb, 8, 32)[:, j]
            else:
                expect = -48 * np.broadcast_to(dmin.astype(np.float64)[:, None], (nb, 32))
            assert np.allclose(delta[:, j], expect, rtol=1e-12, atol=0)


def test_q4k_random_codes_are_centred_with_the_stated_spread():
    blocks = synth.random_q4k(np.random.default_rng(6), 4096)
    w = oracle.dequant(oracle.Q4K, blocks)
    assert abs(w.mean()) < 2e-4 and 0.017 < w.std() < 0.023


def test_q8_worked_blocks():
    g = _golden()["q8_blocks"]
    a = np.array(g[0]["weights"], dtype=np.float64)
    assert np.array_equal(oracle.dequant(oracle.Q8, _bytes(g[0]["hex"])), a)
    assert np.array_equal(oracle.dequant(oracle.Q8, _bytes(g[1]["hex"])), a * g[1]["scale_vs_q8_a"])
    q = np.array([-128, 127] + list(range(-14, 16)), dtype=np.int8)
    assert np.array_equal(synth.pack_q8(np.array([0.5], np.float16), q[None]).reshape(-1), _bytes(g[0]["hex"]))


def test_mx4_worked_blocks_and_packer():
    """MXFP4 blocks worked by hand from the OCP MX definition of E2M1 (the
    magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) and E8M0 (2^(s - 127)), including
    both ends of the scale range."""
    g = {b["name"]: b for b in _golden()["mx4_blocks"]}
    for name in ("mx4_a", "mx4_b"):
        w = oracle.dequant(oracle.MX4, _bytes(g[name]["hex"]))
        assert np.array_equal(w, np.array(g[name]["weights"]))
    a = oracle.dequant(oracle.MX4, _bytes(g["mx4_a"]["hex"]))
    assert np.array_equal(np.signbit(a[:16]), np.arange(16) >= 8)  # code 8 is -0
    assert np.all(oracle.dequant(oracle.MX4, _bytes(g["mx4_c"]["hex"])) == 2.0 ** g["mx4_c"]["weights_log2"])
    assert np.all(oracle.dequant(oracle.MX4, _bytes(g["mx4_d"]["hex"])) == g["mx4_d"]["weights_times_2_pow_minus_127"] * 2.0 ** 127)
    codes = np.tile(np.arange(16, dtype=np.uint8), 2)[None]
    assert np.array_equal(synth.pack_mx4(np.array([127], np.uint8), codes).reshape(-1), _bytes(g["mx4_a"]["hex"]))


def _torch_e4m3(codes):
    """E4M3 bytes decoded by torch's float8_e4m3fn (a library routine the
    oracle does not use), as float64."""
    torch = pytest.importorskip("torch")
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_every_code_matches_torch_float8():
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3(codes)
    got = np.array([oracle.e4m3(int(c)) for c in codes])
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.isnan(got).sum() == 2
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_hand_values():
    for c in _golden()["e4m3_values"]:
        v = oracle.e4m3(int(c["code"], 16))
        if c["value"] is None:
            assert math.isnan(v), c
        else:
            assert v == c["value"] and math.copysign(1, v) == math.copysign(1, c["value"]), c


def _vq_codebook(entry):
    cb = np.zeros((entry["n_codes"], 8), np.uint8)
    for i, h in entry["codewords"].items():
        cb[int(i)] = _bytes(h)
    return cb


def test_vq_worked_rows_and_packer():
    g = {r["name"]: r for r in _golden()["vq_rows"]}
    a, b = g["vq12_a"], g["vq13_b"]
    w = oracle.dequant_rows(oracle.VQ12, _bytes(a["hex"]), a["K"], codebook=_vq_codebook(a))
    assert np.array_equal(w.reshape(-1), a["weights"])
    assert np.array_equal(np.signbit(w.reshape(-1)), np.signbit(a["weights"]))
    w = oracle.dequant_rows(oracle.VQ13, _bytes(b["hex"]), b["K"], codebook=_vq_codebook(b))
    assert np.array_equal(w.reshape(-1), np.repeat(b["weights_per_group"], 8))
    # the packer reproduces the hand bytes
    assert np.array_equal(synth.pack_vq(np.array([1.0], np.float16), np.array([a["indices"]]), 12).reshape(-1),
                          _bytes(a["hex"]))
    assert np.array_equal(synth.pack_vq(np.array([-0.5], np.float16), np.array([b["indices"]]), 13).reshape(-1),
                          _bytes(b["hex"]))
    # a VQ row needs its codebook
    with pytest.raises(ValueError):
        oracle.dequant_rows(oracle.VQ12, _bytes(a["hex"]), a["K"])


def _vq_dense_by_bits(rows, K, fmt, codebook):
    """VQ rows decoded a second way: indices read with numpy's unpackbits
    (little bit order) from the documented layout, codewords through torch's
    float8_e4m3fn.  Returns float64 [R, K]."""
    n = K // 8
    rb = 2 + 3 * K // 16 + (K // 64 if fmt == synth.FMT_VQ13 else 0)
    rows = np.asarray(rows, np.uint8).reshape(-1, rb)
    gain = rows[:, 0:2].copy().view("<f2").astype(np.float64).reshape(-1)
    bits = np.unpackbits(rows[:, 2:2 + 3 * K // 16], axis=1, bitorder="little").reshape(-1, n, 12)
    idx = (bits.astype(np.int64) << np.arange(12)).sum(axis=2)
    if fmt == synth.FMT_VQ13:
        plane = np.unpackbits(rows[:, 2 + 3 * K // 16:], axis=1, bitorder="little")[:, :n]
        idx += plane.astype(np.int64) << 12
    cw = _torch_e4m3(codebook)
    return gain[:, None] * cw[idx].reshape(-1, K)


@pytest.mark.parametrize("fmt", [synth.FMT_VQ12, synth.FMT_VQ13])
def test_vq_random_rows_against_bit_unpacking(fmt):
    """Many rows of random indices (so every index bit and every row's own
    plane matters), several row lengths, against the second decoder."""
    bits = 12 if fmt == synth.FMT_VQ12 else 13
    cb = synth.make_codebook(5, synth.VQ_CODES[fmt])
    for K in (64, 256, 2048):
        rows = synth.random_vq(np.random.default_rng(K + bits), 17, K, bits)
        got = oracle.dequant_rows(fmt, rows, K, codebook=cb)
        ref = _vq_dense_by_bits(rows, K, fmt, cb)
        assert np.array_equal(got, ref)
        assert np.all(np.isfinite(got))


def test_vq_codebook_spread_and_special_codes():
    cb = synth.make_codebook(0, 4096)
    v = _torch_e4m3(cb)
    assert np.all(np.isfinite(v)) and np.abs(v).max() == 7.5
    assert set(np.unique(cb[:20])) == {c for c in range(256) if (c >> 3) & 15 <= 9}
    rms = np.sqrt(np.mean(v[20:] ** 2))
    assert 1.3 < rms < 1.7
    every = synth.make_codebook(0, 4096, every_code=True)
    assert set(np.unique(every[:32])) == set(range(256)) - {0x7F, 0xFF}
    assert np.all(np.isfinite(_torch_e4m3(every))) and np.abs(_torch_e4m3(every)).max() == 448
    rows = synth.random_vq(np.random.default_rng(3), 512, 256, 12)
    w = oracle.dequant_rows(oracle.VQ12, rows, 256, codebook=cb)
    assert 0.015 < w.std() < 0.03


def test_mx4_round_trip_and_error_bound():
    """Blocks whose weights lie on the E2M1 grid times a power of two survive
    quantize -> dequantize exactly; Gaussian blocks round to the nearest grid
    point: error at most half the grid gap around the value (0.25, 0.5 or 1
    times the block scale)."""
    rng = np.random.default_rng(11)
    nb = 64
    k = rng.integers(-20, 5, nb)
    codes = rng.integers(0, 16, (nb, 32))
    vals = synth.E2M1_GRID[codes & 7] * np.where(codes >= 8, -1.0, 1.0)
    w = (vals * np.exp2(k)[:, None]).reshape(-1)
    assert np.array_equal(oracle.dequant(oracle.MX4, synth.quantize_mx4(w)), w)
    g = rng.normal(0, 0.02, 32 * 256)
    blocks = synth.quantize_mx4(g)
    back = oracle.dequant(oracle.MX4, blocks).reshape(-1, 32)
    scale = np.exp2(blocks[:, 0].astype(np.float64) - 127)[:, None]
    v = np.abs(g.reshape(-1, 32)) / scale
    assert np.all(v <= 6.0 + 1e-12)
    gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    assert np.all(np.abs(back - g.reshape(-1, 32)) <= gap * scale * (1 + 1e-12))


def test_mx4_random_codes_spread():
    w = oracle.dequant(oracle.MX4, synth.random_mx4(np.random.default_rng(12), 8192))
    assert abs(w.mean()) < 3e-4 and 0.015 < w.std() < 0.022


# ---------------------------------------------------- formats: round trip ----
def test_q2k_round_trip_exact_on_representable_blocks():
    rng = np.random.default_rng(1)
    nb = 64
    d = (rng.uniform(0.5, 2.0, nb) * 1e-3).astype(np.float16)
    dmin = (rng.uniform(0.5, 2.0, nb) * 1e-3).astype(np.float16)
    sc = rng.integers(1, 16, (nb, 16)).astype(np.uint8)
    m = rng.integers(0, 16, (nb, 16)).astype(np.uint8)
    sc[:, 3] = 15  # makes max step / 15 equal d exactly
    m[:, 5] = 15   # makes max offset / 15 equal dmin exactly
    q = rng.integers(0, 4, (nb, 16, 16)).astype(np.uint8)
    q[:, :, 0] = 0  # every sub-block spans its full range [-dmin m, 3 d sc - dmin m]
    q[:, :, 1] = 3
    w = oracle.dequant(oracle.Q2K, synth.pack_q2k(d, dmin, sc, m, q.reshape(nb, 256)))
    assert np.array_equal(oracle.dequant(oracle.Q2K, synth.quantize_q2k(w)), w)


def test_q2k_error_bound_on_gaussian_blocks():
    # |w - dq(q(w))| <= step/2 inside the range, plus the scale-rounding slack:
    # |err| <= 0.5 d sc_j + 1.6 d + 0.6 dmin  (derivation in quantize_q2k's notes)
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, (200, 256))
    blocks = synth.quantize_q2k(w)
    back = oracle.dequant(oracle.Q2K, blocks).reshape(200, 16, 16)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64)
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float64)
    sc = (blocks[:, 4:20] & 15).astype(np.float64)
    bound = 0.5 * d * sc + 1.6 * d + 0.6 * dmin
    assert np.all(np.abs(back - w.reshape(200, 16, 16)) <= bound[:, :, None] + 1e-12)
    # and it is a real quantizer, not a constant (which would give 1.0): four
    # levels over a 16-sample Gaussian range leave an RMS error near 0.34 sigma
    assert np.sqrt(np.mean((back.reshape(200, 256) - w) ** 2)) / 0.02 < 0.45


def test_q8_round_trip_and_error_bound():
    rng = np.random.default_rng(3)
    nb = 64
    d = (rng.uniform(0.5, 2.0, nb) * 1e-3).astype(np.float16)
    q = rng.integers(-127, 128, (nb, 32)).astype(np.int8)
    q[:, 7] = 127 * np.where(rng.integers(0, 2, nb) > 0, 1, -1)
    w = oracle.dequant(oracle.Q8, synth.pack_q8(d, q))
    assert np.array_equal(oracle.dequant(oracle.Q8, synth.quantize_q8(w)), w)
    g = rng.normal(0, 0.02, (100, 32))
    blk = synth.quantize_q8(g)
    dd = blk[:, 0:2].copy().view("<f2").astype(np.float64)
    back = oracle.dequant(oracle.Q8, blk).reshape(100, 32)
    assert np.all(np.abs(back - g) <= 0.57 * dd + 1e-12)


def test_iq2_round_trip_exact_on_representable_blocks():
    grid = synth.make_grid(0)
    rng = np.random.default_rng(4)
    nb = 3
    d = (rng.uniform(0.5, 2.0, nb) * 1e-4).astype(np.float16)
    rows = rng.integers(0, 256, (nb, 32)).astype(np.uint8)
    signs = rng.integers(0, 128, (nb, 32)).astype(np.uint8)
    scales = rng.integers(0, 16, (nb, 8)).astype(np.uint8)
    scales[:, 2] = 15
    rows[:, 8] = int(np.nonzero(grid[:, 0] == 7)[0][0])  # one weight has |code| = 31 * 7
    w = oracle.dequant(oracle.IQ2, synth.pack_iq2(d, rows, signs, scales), grid)
    again = oracle.dequant(oracle.IQ2, synth.quantize_iq2(w, grid), grid)
    assert np.array_equal(again, w)


def test_iq2_parity_sign_makes_negatives_even():
    grid = synth.make_grid(0)
    blk = synth.random_iq2(np.random.default_rng(5), 50)
    w = oracle.dequant(oracle.IQ2, blk, grid).reshape(-1, 8)
    assert np.all((w < 0).sum(axis=1) % 2 == 0)
    assert np.all(w != 0)


def test_grid_rows_distinct_and_odd():
    grid = synth.make_grid(0)
    assert grid.shape == (256, 8)
    assert set(np.unique(grid)) <= {1, 3, 5, 7}
    assert np.unique(grid, axis=0).shape[0] == 256


# ----------------------------------------------------------------- router ----
def _logit(xv, wv):
    x = np.asarray(xv, np.float32)[None]
    W = np.asarray(wv, np.float32)[None]
    return float(oracle.router_logits(x, oracle.F32, W)[0, 0])


def test_router_fold_order_hand_computed():
    # products 2^24 at i=0 (partial 0), 1 at i=4 (partial 1), -2^24 at i=128
    # (partial 32).  Folding s=32 first cancels the big terms exactly, then
    # the 1 survives: z = 1.  A left-to-right sum gives 2^24 + 1 -> 2^24 and
    # then 0; folding adjacent pairs first also loses the 1.
    d = 256
    x = np.zeros(d)
    w = np.ones(d)
    x[0], x[4], x[128] = 2.0 ** 24, 1.0, -(2.0 ** 24)
    assert _logit(x, w) == 1.0


def test_router_partial_assignment_hand_computed():
    # elements 0..3 belong to the same partial and are consumed in order:
    # 2^24, +1 (rounds back to 2^24), +1 (again), -2^24 -> z = 0.  With a
    # strided assignment (i mod 64) the same products would give z = 1.
    d = 256
    x = np.zeros(d)
    w = np.ones(d)
    x[0:4] = [2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]
    assert _logit(x, w) == 0.0


def test_router_fma_single_rounding():
    # partial 0 takes -1 * 1 first (p = -1), then a * a with a = 1 + 2^-12:
    # a fused multiply-add keeps a^2 - 1 = 2^-11 + 2^-24 exactly, while a
    # separate multiply would round a^2 to 1 + 2^-11 first and give 2^-11.
    a = np.float32(1.0 + 2.0 ** -12)
    x = np.zeros(256, np.float32)
    w = np.zeros(256, np.float32)
    x[0], w[0] = -1.0, 1.0
    x[1], w[1] = a, a
    assert _logit(x, w) == 2.0 ** -11 + 2.0 ** -24


def test_router_basis_vectors_read_one_weight():
    rng = np.random.default_rng(6)
    W = rng.normal(0, 0.02, (8, 512)).astype(np.float32)
    for i in [0, 3, 4, 255, 256, 511]:
        x = np.zeros((1, 512), np.float32)
        x[0, i] = 1.0
        assert np.array_equal(oracle.router_logits(x, oracle.F32, W)[0], W[:, i])


def test_router_error_bound_against_fp64():
    rng = np.random.default_rng(7)
    d, E = 4096, 64
    x = rng.normal(0, 1, (4, d)).astype(np.float32)
    W = rng.normal(0, 0.02, (E, d)).astype(np.float32)
    z = oracle.router_logits(x, oracle.F32, W).astype(np.float64)
    exact = x.astype(np.float64) @ W.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(W.astype(np.float64)).T
    n = d // 64 + 6  # longest chain of roundings: one partial, then the folds
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(z - exact) <= gamma * mag)


def test_router_bf16_input_is_widened_exactly():
    rng = np.random.default_rng(8)
    xb = synth.f32_to_bf16_bits(rng.normal(0, 1, (3, 256)).astype(np.float32))
    W = rng.normal(0, 0.02, (5, 256)).astype(np.float32)
    zf = oracle.router_logits(synth.bf16_bits_to_f32(xb), oracle.F32, W)
    zb = oracle.router_logits(xb, oracle.BF16, W)
    assert np.array_equal(zf, zb)


# ------------------------------------------------------------------ top-k ----
def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(9)
    for E, k in [(8, 2), (384, 6), (37, 16), (5, 5)]:
        z = rng.integers(-3, 4, (20, E)).astype(np.float32)  # many exact ties
        idx = oracle.topk(z, k)
        for t in range(20):
            want = sorted(range(E), key=lambda e: (-z[t, e], e))[:k]
            assert list(idx[t]) == want


def test_topk_special_cases():
    z = np.zeros((1, 10), np.float32)
    assert list(oracle.topk(z, 4)[0]) == [0, 1, 2, 3]          # all equal -> lowest indices
    z = np.array([[0.5, 0.0, 0.5, -0.0, 0.25]], np.float32)
    assert list(oracle.topk(z, 4)[0]) == [0, 2, 4, 1]         # -0 == +0 -> lower index 1
    z = np.array([[-0.0, 0.0, -1.0]], np.float32)
    assert list(oracle.topk(z, 3)[0]) == [0, 1, 2]
    rng = np.random.default_rng(10)
    z = rng.normal(size=(3, 12)).astype(np.float32)
    for t in range(3):                                        # k = E: a full permutation
        assert sorted(oracle.topk(z, 12)[t]) == list(range(12))
    # duplicated router rows give equal logits: the lower expert wins
    W = rng.normal(0, 0.02, (6, 256)).astype(np.float32)
    W[4] = W[1]
    x = rng.normal(0, 1, (5, 256)).astype(np.float32)
    _, idx, _ = oracle.route(x, oracle.F32, W, 6)
    for t in range(5):
        assert list(idx[t]).index(1) == list(idx[t]).index(4) - 1


# ---------------------------------------------------------------- weights ----
def test_weights_closed_forms():
    z = np.array([[0.0, math.log(3.0), -5.0]], np.float32)
    wt = oracle.route_weights(z, np.array([[1, 0]], np.int32))
    # sigmoid(log 3) = 3/4, sigmoid(0) = 1/2 -> 0.75/1.25, 0.5/1.25
    assert abs(wt[0, 0] - 0.6) < 1e-7 and abs(wt[0, 1] - 0.4) < 1e-7
    assert oracle.route_weights(z, np.array([[2]], np.int32))[0, 0] == 1.0
    zz = np.full((1, 6), 0.3, np.float32)
    assert np.allclose(oracle.route_weights(zz, np.arange(6, dtype=np.int32)[None]), 1 / 6, atol=1e-7)


def test_weights_sum_to_one_and_positive():
    rng = np.random.default_rng(11)
    z = rng.normal(0, 3, (50, 384)).astype(np.float32)
    idx = oracle.topk(z, 6)
    wt = oracle.route_weights(z, idx)
    assert np.all(wt > 0)
    assert np.all(np.abs(wt.astype(np.float64).sum(axis=1) - 1) < 1e-6)
    assert np.all(np.diff(wt, axis=1) <= 0)  # rank order -> non-increasing weights


# ------------------------------------------------ selection bias, gains ----
def test_sigmoid32_against_fp64_and_shape():
    zs = np.concatenate([np.linspace(-90, 90, 20001), [0.0, 1e-30, -1e-30, 80.0, -80.0, 1e4, -1e4]]).astype(np.float32)
    got = np.array([oracle.sigmoid32(float(z)) for z in zs], np.float64)
    zc = np.clip(zs.astype(np.float64), -80, 80)
    exact = 1.0 / (1.0 + np.exp(-zc))
    assert np.all(np.abs(got - exact) <= 4e-7 * exact)            # a few fp32 ulp everywhere
    assert oracle.sigmoid32(0.0) == 0.5                             # e = 1 exactly
    order = np.argsort(zs, kind="stable")
    assert np.all(np.diff(got[order]) >= 0)                         # non-decreasing
    for z in [0.5, 3.0, 17.25, 60.0]:                               # sigma(z) + sigma(-z) = 1
        assert abs(oracle.sigmoid32(z) + oracle.sigmoid32(-z) - 1.0) <= 2e-7
    assert oracle.sigmoid32(100.0) == oracle.sigmoid32(80.0) == 1.0   # clamp
    assert oracle.sigmoid32(-100.0) == oracle.sigmoid32(-80.0) > 0.0


def test_bias_selection_against_brute_force_and_invariants():
    rng = np.random.default_rng(21)
    E, k, T = 40, 6, 25
    z = rng.normal(0, 2, (T, E)).astype(np.float32)
    b = rng.normal(0, 0.05, E).astype(np.float32)
    key = oracle.bias_keys(z, b)
    s32 = np.array([[oracle.sigmoid32(float(v)) for v in row] for row in z], np.float32)
    assert np.array_equal(key, (s32 + b).astype(np.float32))        # one fp32 addition per key
    # brute force on the keys, ties to the lower index
    idx = oracle.topk(key, k)
    for t in range(T):
        assert list(idx[t]) == sorted(range(E), key=lambda e: (-key[t, e], e))[:k]
    # zero bias selects as the logits do (sigmoid is increasing; distinct logits here)
    assert np.array_equal(oracle.topk(oracle.bias_keys(z, np.zeros(E, np.float32)), k), oracle.topk(z, k))
    # a large bias on a chosen set forces exactly that set, best logit first
    forced = np.array([3, 11, 17, 22, 30, 39])
    bb = np.zeros(E, np.float32)
    bb[forced] = 4.0
    sel = oracle.topk(oracle.bias_keys(z, bb), k)
    for t in range(T):
        assert sorted(sel[t]) == sorted(forced)
        assert list(sel[t]) == sorted(forced, key=lambda e: (-z[t, e], e))
    # equal keys: lower index first
    zt = np.zeros((1, 8), np.float32)
    assert list(oracle.topk(oracle.bias_keys(zt, np.full(8, 0.25, np.float32)), 3)[0]) == [0, 1, 2]
    # the bias moves the selection, not the weights: weights = normalised sigmoid(z) of the chosen set
    W = rng.normal(0, 0.02, (E, 256)).astype(np.float32)
    xs = rng.normal(0, 1, (T, 256)).astype(np.float32)
    zz, idx_b, wt_b = oracle.route(xs, oracle.F32, W, k, bias=bb)
    for t in range(T):
        s = 1.0 / (1.0 + np.exp(-zz[t, idx_b[t]].astype(np.float64)))
        assert np.allclose(wt_b[t], s / s.sum(), rtol=0, atol=2e-7)
        assert sorted(idx_b[t]) == sorted(forced)


def test_down_gains_scale_each_expert_channel():
    spec = synth.scaled_spec(E=6, k=3, d=256, f=256)
    L = synth.random_layer(spec, seed=22, workload="gain")
    x = synth.activations(22, ("gain", "x"), 4, spec.d, synth.F32)
    _, idx, wt = oracle.route(x, oracle.F32, L.w_router, spec.k)
    y0 = oracle.ffn(L, x, oracle.F32, idx, wt)
    Lg = synth.Layer(**{**L.__dict__, "down_gain": np.ones((spec.E, spec.d), np.float32)})
    assert np.array_equal(oracle.ffn(Lg, x, oracle.F32, idx, wt), y0)        # unit gains change nothing
    # routed part alone (no shared expert): gains c_e scale expert e's contribution, per channel
    spec_ns = synth.scaled_spec(E=6, k=3, d=256, f=256, has_shared=False)
    Ln = synth.random_layer(spec_ns, seed=22, workload="gain")
    ones = np.ones((1, 1), np.float32)
    g = np.random.default_rng(23).uniform(0.5, 1.5, (6, 256)).astype(np.float32)
    g[:, 7] = 0.0                                                           # a muted channel
    Lng = synth.Layer(**{**Ln.__dict__, "down_gain": g})
    for t in range(4):
        e = int(idx[t, 0])
        one = np.array([[e]], np.int32)
        solo = oracle.ffn(Ln, x[t:t + 1], oracle.F32, one, ones)[0].astype(np.float64)
        solo_g = oracle.ffn(Lng, x[t:t + 1], oracle.F32, one, ones)[0].astype(np.float64)
        assert np.allclose(solo_g, g[e] * solo, rtol=1e-6, atol=1e-12)
        assert solo_g[7] == 0.0
    yng = oracle.ffn(Lng, x, oracle.F32, idx, wt)
    assert np.all(yng[:, 7] == 0.0)


# ---------------------------------------------------------------- buckets ----
def test_bucket_matches_stable_argsort():
    rng = np.random.default_rng(12)
    for T, k, E in [(1, 6, 384), (1024, 6, 384), (7, 2, 8), (0, 6, 384), (33, 16, 20)]:
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        counts, offsets, perm, pos = oracle.bucket(idx, E)
        flat = idx.reshape(-1)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * k
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(pos[perm], np.arange(T * k))


def test_bucket_refuses_keys_out_of_range():
    for bad in (8, -1):
        idx = np.array([[0, 3], [bad, 1]], np.int32)
        with pytest.raises(ValueError):
            oracle.bucket(idx, 8)


def test_bucket_mean_load_matches_closed_form():
    # T*k/E routed rows per expert on average: 8,192 tokens x 6 / 384 = 128,
    # the ~128 rows per expert the YoungAi page (section 4.2) quotes.
    rng = np.random.default_rng(13)
    idx = np.stack([rng.choice(384, 6, replace=False) for _ in range(8192)]).astype(np.int32)
    counts, *_ = oracle.bucket(idx, 384)
    assert counts.mean() == 128.0


# -------------------------------------------------------------------- FFN ----
def _q8_identity_layer(E, d, f, gate_col, up_col, has_shared):
    """Q8 layer with d = 1: gate row n reads x[gate_col], up row n reads
    x[up_col], down row r reads h[r] (r < f) -- so y has a closed form."""
    def mat(rows, K, col_of_row):
        q = np.zeros((rows, K), np.int8)
        for r in range(rows):
            c = col_of_row(r)
            if c is not None:
                q[r, c] = 1
        return synth.pack_q8(np.ones(rows * K // 32, np.float16), q.reshape(-1, 32)).reshape(-1)

    spec = synth.LayerSpec(E=E, k=1, d=d, f=f, fmt_gate_up=synth.FMT_Q8, fmt_down=synth.FMT_Q8,
                           has_shared=has_shared, fmt_shared=synth.FMT_Q8)
    g = mat(f, d, lambda r: gate_col)
    u = mat(f, d, lambda r: up_col)
    dn = mat(d, f, lambda r: r if r < f else None)
    L = synth.Layer(spec=spec, w_gate=np.tile(g, E), w_up=np.tile(u, E), w_down=np.tile(dn, E),
                    grid=synth.make_grid(0), w_router=np.zeros((E, d), np.float32))
    if has_shared:
        L.s_gate, L.s_up, L.s_down = g, u, dn
    return L


def test_ffn_closed_form_swiglu():
    d, f = 64, 32
    L = _q8_identity_layer(E=2, d=d, f=f, gate_col=0, up_col=1, has_shared=True)
    x = np.zeros((1, d), np.float32)
    x[0, 0], x[0, 1] = 1.0, 2.0
    # g = 1, u = 2 -> h = silu(1) * 2 = 2 / (1 + e^-1); y[r] = wt * h + h for r < f
    h = 2.0 / (1.0 + math.exp(-1.0))
    y = oracle.ffn(L, x, oracle.F32, np.array([[1]], np.int32), np.array([[0.25]], np.float32))
    want = np.zeros(d)
    want[:f] = 1.25 * h
    assert np.allclose(y[0], want, rtol=1e-7, atol=0)
    x[0, 0] = -3.0  # silu(-3) = -3 / (1 + e^3)
    y = oracle.ffn(L, x, oracle.F32, np.array([[0]], np.int32), np.array([[1.0]], np.float32))
    assert np.allclose(y[0, :f], 2 * (-3.0 / (1 + math.exp(3.0))) * 2.0, rtol=1e-7)


def _dense(L, fmt, blob, e, rows, K):
    per = blob.size // (L.spec.E if e is not None else 1)
    b = blob if e is None else blob[e * per:(e + 1) * per]
    if fmt in synth.VQ_FORMATS:
        return _vq_dense_by_bits(b, K, fmt, L.vq_codebook)
    return oracle.dequant(fmt, b, L.grid).reshape(rows, K)


def _numpy_ffn(L, x, idx, wt):
    s = L.spec
    y = np.zeros((x.shape[0], s.d))
    for t in range(x.shape[0]):
        xv = x[t].astype(np.float64)
        for j in range(s.k):
            e = idx[t, j]
            g = _dense(L, s.fmt_gate_up, L.w_gate, e, s.f, s.d) @ xv
            u = _dense(L, s.fmt_gate_up, L.w_up, e, s.f, s.d) @ xv
            h = g / (1 + np.exp(-g)) * u
            y[t] += float(wt[t, j]) * (_dense(L, s.fmt_down, L.w_down, e, s.d, s.f) @ h)
        if s.has_shared:
            g = _dense(L, s.fmt_shared, L.s_gate, None, s.f, s.d) @ xv
            u = _dense(L, s.fmt_shared, L.s_up, None, s.f, s.d) @ xv
            y[t] += _dense(L, s.fmt_shared, L.s_down, None, s.d, s.f) @ (g / (1 + np.exp(-g)) * u)
    return y


@pytest.mark.parametrize("spec", [
    synth.TINY_SPEC,
    synth.scaled_spec(E=6, k=3, d=512, f=256),                       # IQ2 gate/up, Q2K down, Q8 shared
    synth.scaled_spec(E=5, k=2, d=256, f=512, fmt_gate_up=synth.FMT_Q8, fmt_down=synth.FMT_IQ2,
                      fmt_shared=synth.FMT_Q2K),
    synth.scaled_spec(E=5, k=2, d=512, f=256, fmt_gate_up=synth.FMT_Q4K, fmt_down=synth.FMT_Q4K),
    synth.scaled_spec(E=5, k=2, d=256, f=512, fmt_gate_up=synth.FMT_MX4, fmt_down=synth.FMT_MX4),
    synth.scaled_spec(E=5, k=2, d=256, f=512, fmt_gate_up=synth.FMT_VQ12, fmt_down=synth.FMT_VQ12),
    synth.scaled_spec(E=5, k=3, d=512, f=256, fmt_gate_up=synth.FMT_VQ13, fmt_down=synth.FMT_VQ13),
])
def test_ffn_matches_numpy_dense_matmul(spec):
    L = synth.random_layer(spec, seed=3, workload="pin")
    x = synth.activations(3, ("pin", "x"), 5, spec.d, synth.F32)
    _, idx, wt = oracle.route(x, oracle.F32, L.w_router, spec.k)
    y = oracle.ffn(L, x, oracle.F32, idx, wt)
    ref = _numpy_ffn(L, x, idx, wt)
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())


@pytest.mark.parametrize("spec,gains", [
    (synth.scaled_spec(E=6, k=3, d=512, f=256), False),
    (synth.scaled_spec(E=5, k=2, d=256, f=512, fmt_gate_up=synth.FMT_Q8, fmt_down=synth.FMT_IQ2,
                       fmt_shared=synth.FMT_Q2K), True),
    (synth.scaled_spec(E=7, k=4, d=256, f=256, fmt_gate_up=synth.FMT_Q4K, fmt_down=synth.FMT_Q2K,
                       has_shared=False), True),
    (synth.scaled_spec(E=6, k=3, d=512, f=256, fmt_gate_up=synth.FMT_MX4, fmt_down=synth.FMT_MX4), False),
    (synth.scaled_spec(E=6, k=3, d=256, f=512, fmt_gate_up=synth.FMT_VQ13, fmt_down=synth.FMT_VQ12), True),
])
def test_grouped_ffn_is_bitwise_the_token_loop(spec, gains):
    """The expert-grouped evaluation (each expert dequantised once) performs
    the same fp64 operations per output as the token-by-token loop: equal bit
    for bit, on all tokens, on a token subset with repeats, and with gains;
    and it agrees with numpy dense matmul like the plain loop does."""
    L = synth.random_layer(spec, seed=6, workload="grouped")
    if gains:
        rng = np.random.default_rng(6)
        L = synth.Layer(**{**L.__dict__, "down_gain": rng.uniform(0.5, 1.5, (spec.E, spec.d)).astype(np.float32)})
    x = synth.activations(6, ("grouped", "x"), 9, spec.d, synth.F32)
    _, idx, wt = oracle.route(x, oracle.F32, L.w_router, spec.k)
    y = oracle.ffn(L, x, oracle.F32, idx, wt)
    assert np.array_equal(oracle.ffn(L, x, oracle.F32, idx, wt, grouped=True), y)
    tok = [8, 0, 3, 3]
    assert np.array_equal(oracle.ffn(L, x, oracle.F32, idx, wt, tokens=tok, grouped=True), y[tok])
    if not gains:
        ref = _numpy_ffn(L, x, idx, wt)
        yg = oracle.ffn(L, x, oracle.F32, idx, wt, grouped=True)
        assert np.allclose(yg, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())
    with pytest.raises(ValueError):
        bad = idx.copy()
        bad[2, 1] = spec.E
        oracle.ffn(L, x, oracle.F32, bad, wt, grouped=True)


def test_ffn_invariants():
    spec = synth.scaled_spec(E=6, k=3, d=256, f=256, has_shared=False)
    L = synth.random_layer(spec, seed=4, workload="inv")
    x = synth.activations(4, ("inv", "x"), 3, spec.d, synth.F32)
    _, idx, wt = oracle.route(x, oracle.F32, L.w_router, spec.k)
    y = oracle.ffn(L, x, oracle.F32, idx, wt)
    # relabelling experts (weights and routes together) changes nothing
    perm = np.array([3, 5, 0, 1, 4, 2])
    inv = np.argsort(perm)

    def relabel(blob):
        per = blob.size // spec.E
        return np.concatenate([blob[perm[e] * per:(perm[e] + 1) * per] for e in range(spec.E)])
    L2 = synth.Layer(spec=spec, w_gate=relabel(L.w_gate), w_up=relabel(L.w_up), w_down=relabel(L.w_down),
                     grid=L.grid, w_router=L.w_router[perm])
    assert np.array_equal(oracle.ffn(L2, x, oracle.F32, inv[idx].astype(np.int32), wt), y)
    # doubling every down-projection scale doubles the (routed-only) output exactly
    dn = L.w_down.reshape(-1, 84).copy()
    for off in (0, 2):
        v = dn[:, off:off + 2].copy().view("<f2").astype(np.float32) * 2
        dn[:, off:off + 2] = v.astype("<f2").view(np.uint8).reshape(-1, 2)
    L3 = synth.Layer(spec=spec, w_gate=L.w_gate, w_up=L.w_up, w_down=dn.reshape(-1), grid=L.grid,
                     w_router=L.w_router)
    assert np.array_equal(oracle.ffn(L3, x, oracle.F32, idx, wt), 2 * y)
    # one-hot routing weights pick one expert's output
    one = np.zeros_like(wt)
    one[:, 1] = 1.0
    y1 = oracle.ffn(L, x, oracle.F32, idx, one)
    for t in range(3):
        solo = oracle.ffn(L, x[t:t + 1], oracle.F32, idx[t:t + 1, 1:2].copy(), np.ones((1, 1), np.float32))
        assert np.array_equal(y1[t], solo[0])
    # a token subset gives the same rows as the full call
    assert np.array_equal(oracle.ffn(L, x, oracle.F32, idx, wt, tokens=[2, 0]), y[[2, 0]])


def test_tiny_workload_layer_forward_against_dense():
    L = synth.tiny_layer(0)
    x = synth.activations(0, ("tiny", "x"), 4, 256, synth.F32)
    y, idx, wt = oracle.layer_forward(L, x, oracle.F32)
    ref = _numpy_ffn(L, x, idx, wt)
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-7 * np.abs(ref).max())
    assert np.all(np.abs(wt.sum(axis=1) - 1) < 1e-6)


def test_session_routes_distinct_expert_curve():
    # the reuse generator follows the pages' distinct-expert curve over 1..5
    # consecutive tokens: 6, 10.0, 13.3, 17.4, 21.7 (YoungAi page, section 2.2).
    # The printed increments (4.0, 3.3, 4.1, 4.3) dip at the third token, which
    # no memoryless reuse model reproduces; the model sits ~0.55 above 13.3 and
    # within ~0.35 of the other points, hence the 0.7 band.
    idx, wt = synth.session_routes(0, sessions=2000, steps=5, tag="curve")
    per = idx.reshape(5, 2000, 6)
    means = [np.mean([len(set(per[:n, s].reshape(-1))) for s in range(2000)]) for n in range(1, 6)]
    for got, want in zip(means, [6, 10.0, 13.3, 17.4, 21.7]):
        assert abs(got - want) < 0.7, means
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])  # distinct per token
    assert np.all(np.abs(wt.sum(axis=1) - 1) < 1e-6)


def test_zipf_routes_are_skewed_and_distinct():
    idx, _ = synth.zipf_routes(0, 4096)
    counts = np.bincount(idx.reshape(-1), minlength=384)
    assert counts.sum() == 4096 * 6 and counts.max() > 20 * max(1, np.median(counts))
    assert np.all(np.sort(idx, axis=1)[:, 1:] != np.sort(idx, axis=1)[:, :-1])

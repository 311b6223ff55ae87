"""Pins of the CPU oracle to things other than itself (CPU only, no GPU).

Each test ties one oracle function to an independent fact: IEEE binary16 as
implemented by numpy, hand-worked fixtures under tests/golden/, closed forms,
encoders written here as the inverse of the block-layout reading, structural
bit-flip properties, or fp64 brute force through numpy's matmul.  A dropped
term, a wrong sign, index or shift, or a transposed operand in the oracle
fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle as orc
from quant_mat_vec_amd import synth
from tests.q8_fixtures import near_tie_blocks, numpy_q8_1, s_tie_blocks

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def h2b(x):
    return int(x, 16)


# ---------------------------------------------------------------- fp16
def test_fp16_decode_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp16_encode_vs_numpy_ties_and_random():
    fin = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)            # exact in fp32
    vals = np.concatenate([
        fin.astype(np.float32), mids,
        np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
        np.float32([65504, 65519.99, 65520, 65536, 1e9, 1e-30, 0.0]),
    ])
    g = synth.rng(1234)
    rnd = (g.standard_normal(20000) * np.exp2(g.integers(-30, 17, 20000))).astype(np.float32)
    vals = np.concatenate([vals, -vals, rnd])
    ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([orc.float_to_half(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_fp16_golden():
    gd = gold("fp16_values.json")
    for bits, val, _why in gd["decode"]:
        got = orc.half_to_double(h2b(bits))
        assert got == val and np.signbit(got) == np.signbit(val), (bits, got, val)
    for val, bits, _why in gd["encode"]:
        assert orc.float_to_half(val) == h2b(bits), (val, hex(orc.float_to_half(val)), bits)


# ---------------------------------------------------------------- Q6_K
def q6k_from_golden(gd):
    blk = np.zeros(210, np.uint8)
    for k, v in gd["bytes"]["ql"].items():
        blk[int(k)] = h2b(v)
    for k, v in gd["bytes"]["qh"].items():
        blk[128 + int(k)] = h2b(v)
    for k, v in gd["bytes"]["scales"].items():
        blk[192 + int(k)] = np.int8(v).view(np.uint8)
    d = h2b(gd["bytes"]["d_bits"])
    blk[208], blk[209] = d & 0xFF, d >> 8
    return blk


def test_q6k_golden_handworked():
    gd = gold("q6k_block_handworked.json")
    blk = q6k_from_golden(gd)
    q, sc, d = orc.q6k_decode(blk)
    assert d == 0.5
    exp_q = np.full(256, gd["expected_q"]["default"], np.int64)
    for k, v in gd["expected_q"].items():
        if k != "default":
            exp_q[int(k)] = v
    assert np.array_equal(q.astype(np.int64), exp_q)
    w = orc.dequant("q6k", blk, 1, 256)[0]
    exp_w = np.repeat(np.array(gd["expected_w_default_per_scale_group"]), 16)
    for k, v in gd["expected_w"].items():
        exp_w[int(k)] = v
    assert np.array_equal(w, exp_w)


def encode_q6k(q6, sc, d_bits):
    """Inverse of the Q6_K layout reading, written independently of the
    oracle: q6 (256 values in [0,63]) -> ql/qh bytes."""
    blk = np.zeros(210, np.uint8)
    for h in range(2):
        for l in range(32):
            for c in range(4):
                v = int(q6[128 * h + 32 * c + l])
                blk[64 * h + 32 * (c & 1) + l] |= (v & 15) << (4 * (c >> 1))
                blk[128 + 32 * h + l] |= (v >> 4) << (2 * c)
    blk[192:208] = np.asarray(sc, np.int8).view(np.uint8)
    blk[208], blk[209] = d_bits & 0xFF, d_bits >> 8
    return blk


def test_q6k_encode_decode_roundtrip():
    g = synth.rng(7)
    for _ in range(50):
        q6 = g.integers(0, 64, 256)
        sc = g.integers(-128, 128, 16)
        blk = encode_q6k(q6, sc, 0x1234)
        q, s, d = orc.q6k_decode(blk)
        assert np.array_equal(q.astype(np.int64), q6 - 32)
        assert np.array_equal(s.astype(np.int64), sc)
        assert d == orc.half_to_double(0x1234)


def test_q6k_bitflip_structure():
    """Every ql bit moves exactly one weight by 1, 2, 4 or 8 and every qh bit
    exactly one weight by 16 or 32; each weight owns 4 ql bits and 2 qh bits."""
    blk = synth.q6k_blocks(synth.rng(3), 1, 256)
    q0, _, _ = orc.q6k_decode(blk)
    owners_l = np.zeros(256, int)
    owners_h = np.zeros(256, int)
    for byte in range(192):
        for bit in range(8):
            b2 = blk.copy()
            b2[byte] ^= 1 << bit
            q1, _, _ = orc.q6k_decode(b2)
            diff = q1.astype(int) - q0.astype(int)
            nz = np.nonzero(diff)[0]
            assert nz.size == 1, (byte, bit)
            step = abs(int(diff[nz[0]]))
            if byte < 128:
                assert step == 1 << (bit % 4)
                owners_l[nz[0]] += 1
            else:
                assert step == 16 << (bit % 2)
                owners_h[nz[0]] += 1
    assert np.all(owners_l == 4) and np.all(owners_h == 2)


def test_q6k_scale_group_placement():
    sc = np.arange(16) * 7 - 60
    blk = encode_q6k(np.full(256, 17), sc, 0x3C00)            # q = -15, d = 1
    w = orc.dequant("q6k", blk, 1, 256)[0]
    assert np.array_equal(w, -15.0 * np.repeat(sc, 16))


# ---------------------------------------------------------- Q4_K / Q5_K
def encode_scales(sc, m):
    """Inverse of the 6-bit scale/min packing reading (12 bytes)."""
    s = np.zeros(12, np.uint8)
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return s


def q45_from_golden(gd, five):
    n = 176 if five else 144
    blk = np.zeros(n, np.uint8)
    d, dm = h2b(gd["header"]["d_bits"]), h2b(gd["header"]["dmin_bits"])
    blk[0], blk[1], blk[2], blk[3] = d & 0xFF, d >> 8, dm & 0xFF, dm >> 8
    blk[4:16] = [h2b(x) for x in gd["scales"]]
    qs_off = 48 if five else 16
    for k, v in gd["qs"].items():
        blk[qs_off + int(k)] = h2b(v)
    if five:
        for k, v in gd["qh_q5k"].items():
            blk[16 + int(k)] = h2b(v)
    return blk


@pytest.mark.parametrize("five", [False, True])
def test_q45_golden_handworked(five):
    gd = gold("q4k_block_handworked.json")
    blk = q45_from_golden(gd, five)
    dec = orc.q5k_decode if five else orc.q4k_decode
    q, sc, m, d, dmin = dec(blk)
    assert (d, dmin) == (1.0, 0.5)
    assert list(sc) == gd["expected_sc"] and list(m) == gd["expected_m"]
    key = "q5k" if five else "q4k"
    exp_q = np.full(256, gd[f"{key}_expected_q"]["default"])
    for k, v in gd[f"{key}_expected_q"].items():
        if k != "default":
            exp_q[int(k)] = v
    assert np.array_equal(q.astype(int), exp_q)
    w = orc.dequant(key, blk, 1, 256)[0]
    exp_w = np.repeat(np.array(gd["expected_w_default_per_subblock"]), 32)
    for k, v in gd[f"{key}_expected_w"].items():
        exp_w[int(k)] = v
    # weights whose q is nonzero but whose scale and min are 0 stay 0
    assert np.array_equal(w, exp_w)


def test_q45_scale_roundtrip_and_bitflips():
    g = synth.rng(11)
    edge = [0, 1, 15, 16, 62, 63]
    cases = [(np.full(8, a), np.full(8, b)) for a in edge for b in edge]
    cases += [(g.integers(0, 64, 8), g.integers(0, 64, 8)) for _ in range(200)]
    for sc, m in cases:
        blk = np.zeros(144, np.uint8)
        blk[4:16] = encode_scales(sc, m)
        _, s2, m2, _, _ = orc.q4k_decode(blk)
        assert np.array_equal(s2.astype(int), sc) and np.array_equal(m2.astype(int), m)
    # each of the 96 scale bits moves exactly one 6-bit field by a power of two
    blk = synth.q4k_blocks(g, 1, 256)
    _, s0, m0, _, _ = orc.q4k_decode(blk)
    hits = np.zeros(16, int)
    for byte in range(4, 16):
        for bit in range(8):
            b2 = blk.copy()
            b2[byte] ^= 1 << bit
            _, s1, m1, _, _ = orc.q4k_decode(b2)
            diff = np.concatenate([s1.astype(int) - s0, m1.astype(int) - m0])
            nz = np.nonzero(diff)[0]
            assert nz.size == 1
            assert abs(diff[nz[0]]) in (1, 2, 4, 8, 16, 32)
            hits[nz[0]] += 1
    assert np.all(hits == 6)


@pytest.mark.parametrize("five", [False, True])
def test_q45_quant_bitflip_structure(five):
    kind = "q5k" if five else "q4k"
    blk = synth.blocks(kind, synth.rng(5), 1, 256)
    dec = orc.q5k_decode if five else orc.q4k_decode
    q0 = dec(blk)[0].astype(int)
    qs_off = 48 if five else 16
    owners = np.zeros(256, int)
    for byte in range(16, len(blk)):
        for bit in range(8):
            b2 = blk.copy()
            b2[byte] ^= 1 << bit
            diff = dec(b2)[0].astype(int) - q0
            nz = np.nonzero(diff)[0]
            assert nz.size == 1
            step = abs(diff[nz[0]])
            assert step == (1 << (bit % 4) if byte >= qs_off else 16)
            owners[nz[0]] += 1
    assert np.all(owners == (5 if five else 4))


# ---------------------------------------------------------------- Q8_1
def test_q8_1_golden_handworked():
    gd = gold("q8_1_handworked.json")
    x = np.array([b["x"] for b in gd["blocks"]], np.float32).reshape(1, -1)
    xq = orc.quantize_q8_1(x).reshape(-1, 36)
    for i, b in enumerate(gd["blocks"]):
        assert int(xq[i, 0]) | int(xq[i, 1]) << 8 == h2b(b["d_bits"])
        assert int(xq[i, 2]) | int(xq[i, 3]) << 8 == h2b(b["s_bits"])
        assert list(xq[i, 4:].view(np.int8)) == b["q"]
    deq = orc.dequant_q8_1(xq.reshape(1, -1), 96)[0]
    assert np.array_equal(deq[:32], np.array(gd["blocks"][0]["q"], np.float64))
    assert np.array_equal(deq[64:], 2.0 * np.array(gd["blocks"][2]["q"], np.float64))


def test_q8_1_invariants():
    g = synth.rng(21)
    x = synth.activations(g, 4, 2560) * np.float32(3.0)
    x[0, :32] = 0.0                                      # an all-zero block
    x[1, 32:64] = np.float32(1e-30)                      # a tiny constant block
    xq = orc.quantize_q8_1(x).reshape(4, -1, 36)
    d = xq[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    s = xq[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    q = xq[..., 4:].view(np.int8).astype(np.int64)
    xb = x.reshape(4, -1, 32).astype(np.float64)
    amax = np.abs(xb).max(-1)
    d32 = (amax.astype(np.float32) / np.float32(127)).astype(np.float64)
    assert np.all(np.abs(q) <= 127)
    assert np.all(np.abs(q).max(-1)[amax > 0] == 127)
    assert np.all(q[amax == 0] == 0) and np.all(d[amax == 0] == 0) and np.all(s[amax == 0] == 0)
    nz = amax > 0
    # q is the nearest integer to x/d (ties away): |x/d - q| <= 1/2 (+ fp32 rounding)
    r = np.abs(xb[nz] / d32[nz][:, None] - q[nz])
    assert r.max() <= 0.5 + 1e-5
    # stored d is the fp16 rounding of d32 (relative half-ulp, or the
    # subnormal absolute half-ulp)
    assert np.all(np.abs(d - d32) <= np.maximum(np.abs(d32) * 2.0 ** -11, 2.0 ** -25))
    # stored s equals d * sum(q) up to fp16 rounding of that product
    dsum = d32 * q.sum(-1)
    assert np.all(np.abs(s - dsum) <= np.abs(dsum) * 2.0 ** -11 * (1 + 1e-6) + 2.0 ** -25)


def test_q8_1_scale_and_sign_symmetry():
    g = synth.rng(22)
    x = synth.activations(g, 2, 512)
    a = orc.quantize_q8_1(x).reshape(2, -1, 36)
    b = orc.quantize_q8_1(np.float32(8.0) * x).reshape(2, -1, 36)
    c = orc.quantize_q8_1(-x).reshape(2, -1, 36)
    assert np.array_equal(a[..., 4:], b[..., 4:])                   # power-of-two scaling
    da = a[..., 0:2].copy().view(np.float16).astype(np.float64)
    db = b[..., 0:2].copy().view(np.float16).astype(np.float64)
    assert np.array_equal(8.0 * da, db)
    assert np.array_equal(a[..., 4:].view(np.int8), -c[..., 4:].view(np.int8))
    assert np.array_equal(a[..., 0:2], c[..., 0:2])


# ------------------------------------------ Q8_1 vs an independent numpy quantizer
def test_q8_1_vs_independent_numpy_random():
    g = synth.rng(41)
    x = synth.activations(g, 6, 2560)
    x[1] *= np.float32(1e-6)                       # small d (still normal)
    x[2] *= np.float32(1e-39 / 3)                  # subnormal x and d
    x[3, :64] = 0.0                                # all-zero blocks
    x[4] = np.float32(7.25)                        # constant blocks
    x[5] *= np.float32(2.0 ** 12)                  # large values (d and s still finite in fp16)
    assert np.array_equal(orc.quantize_q8_1(x), numpy_q8_1(x))


def test_q8_1_near_ties_decide_the_division_reading():
    x = near_tie_blocks()
    ref = numpy_q8_1(x)
    assert np.array_equal(orc.quantize_q8_1(x), ref)
    # the fixture separates the reading from each plausible other one, so an
    # oracle that multiplied by the reciprocal, divided in fp64 or rounded
    # ties to even would fail the line above
    for mode in ("recip", "div64", "even"):
        other = numpy_q8_1(x, mode)
        assert not np.array_equal(other, ref), mode
        nq = np.count_nonzero(other.reshape(-1, 36)[:, 4:] != ref.reshape(-1, 36)[:, 4:])
        assert nq >= 50, (mode, nq)


def test_q8_1_sum_field_rounds_the_fp32_product():
    """s = fp16(fp32(d * sum)): on blocks where the fp32 product is an fp16
    midpoint but the exact product is not, the two roundings differ; the
    oracle must take the fp32 product (a fused multiply-convert would fail)."""
    x = s_tie_blocks()
    ref = numpy_q8_1(x)
    assert np.array_equal(orc.quantize_q8_1(x), ref)
    fused = numpy_q8_1(x, "fused_s").reshape(-1, 36)
    r = ref.reshape(-1, 36)
    assert np.array_equal(fused[:, 4:], r[:, 4:]) and np.array_equal(fused[:, :2], r[:, :2])
    assert np.count_nonzero((fused[:, 2:4] != r[:, 2:4]).any(-1)) == len(r)   # every block's s differs


# ------------------------------------------ exhaustive decoders vs numpy
def numpy_q6k_codes(blocks):
    """q6 in [0, 63] per weight of [nb][210] GGUF Q6_K blocks, from the layout
    reading (h = i/128, c = (i%128)/32, l = i%32)."""
    i = np.arange(256)
    h, c, l = i // 128, (i % 128) // 32, i % 32
    low = (blocks[:, 64 * h + 32 * (c % 2) + l] >> (4 * (c // 2))) & 15
    high = (blocks[:, 128 + 32 * h + l] >> (2 * c)) & 3
    return low.astype(np.int64) | (high.astype(np.int64) << 4)


def numpy_q45_codes(blocks, five):
    i = np.arange(256)
    j, l = i // 32, i % 32
    qs0 = 48 if five else 16
    q = (blocks[:, qs0 + 32 * (j // 2) + l] >> (4 * (j % 2))) & 15
    q = q.astype(np.int64)
    if five:
        q |= ((blocks[:, 16 + l] >> j) & 1).astype(np.int64) << 4
    return q


def numpy_q45_scales(blocks):
    """(sc, m) [nb][8] from the 12 packed bytes at offset 4."""
    s = blocks[:, 4:16].astype(np.int64)
    sc = np.zeros((len(blocks), 8), np.int64)
    m = np.zeros((len(blocks), 8), np.int64)
    for j in range(8):
        if j < 4:
            sc[:, j] = s[:, j] & 63
            m[:, j] = s[:, j + 4] & 63
        else:
            sc[:, j] = (s[:, j + 4] & 15) | ((s[:, j - 4] >> 6) << 4)
            m[:, j] = (s[:, j + 4] >> 4) | ((s[:, j] >> 6) << 4)
    return sc, m


def _all_pairs():
    t = np.arange(65536)
    return (t >> 8).astype(np.uint8), (t & 255).astype(np.uint8)


def test_q6k_decoder_exhaustive_byte_pairs_vs_numpy():
    """Every (ql byte, qh byte) pair at every weight position: block t holds
    ql bytes t>>8 and qh bytes t&255 throughout, d = 1 and unit scales, so
    the dequantized weight is q6 - 32; and random blocks (distinct bytes per
    position) for the byte indexing."""
    a, b = _all_pairs()
    blk = np.zeros((65536, 210), np.uint8)
    blk[:, :128] = a[:, None]
    blk[:, 128:192] = b[:, None]
    blk[:, 192:208] = 1
    blk[:, 208], blk[:, 209] = 0x00, 0x3C                       # fp16 1.0
    w = orc.dequant("q6k", blk.reshape(-1), 65536, 256)
    assert np.array_equal(w, (numpy_q6k_codes(blk) - 32).astype(np.float64))
    rnd = synth.q6k_blocks(synth.rng(51), 4096, 256).reshape(4096, 210).copy()
    rnd[:, 192:208] = 1
    rnd[:, 208], rnd[:, 209] = 0x00, 0x3C
    w = orc.dequant("q6k", rnd.reshape(-1), 4096, 256)
    assert np.array_equal(w, (numpy_q6k_codes(rnd) - 32).astype(np.float64))


@pytest.mark.parametrize("five", [False, True])
def test_q45_decoder_exhaustive_vs_numpy(five):
    """Q4_K/Q5_K: every (qs byte, qh byte) pair at every position (unit
    scales, zero mins, d = 1, dmin = 0, so w = q), and every pair of the
    bytes each 6-bit scale and min is built from (w = sc with q = 1, and
    w = -m with d = 0, dmin = 1)."""
    kind, nbytes = ("q5k", 176) if five else ("q4k", 144)
    qs0 = 48 if five else 16
    a, b = _all_pairs()
    ones = encode_scales(np.ones(8, int), np.zeros(8, int))
    blk = np.zeros((65536, nbytes), np.uint8)
    blk[:, 0], blk[:, 1] = 0x00, 0x3C                           # d = 1, dmin = 0
    blk[:, 4:16] = ones
    blk[:, qs0:qs0 + 128] = a[:, None]
    if five:
        blk[:, 16:48] = b[:, None]
    w = orc.dequant(kind, blk.reshape(-1), 65536, 256)
    assert np.array_equal(w, numpy_q45_codes(blk, five).astype(np.float64))
    g = synth.rng(52)
    # sub-blocks 4..7 take sc from bytes 8..11 and 0..3, m from bytes 8..11
    # and 4..7 (sub-blocks 0..3 one byte each): sweep both pairs of groups,
    # the third group random
    for other in ((0, 4), (4, 8)):
        sb = np.zeros((65536, nbytes), np.uint8)
        sb[:, 4:16] = g.integers(0, 256, (65536, 12), dtype=np.uint8)
        sb[:, 12:16] = a[:, None]
        sb[:, 4 + other[0]:4 + other[1]] = b[:, None]
        sc, m = numpy_q45_scales(sb)
        one = sb.copy()
        one[:, 0], one[:, 1] = 0x00, 0x3C                   # d = 1, dmin = 0
        one[:, qs0:qs0 + 128] = 0x11
        if five:
            one[:, 16:48] = 0
        w = orc.dequant(kind, one.reshape(-1), 65536, 256)
        assert np.array_equal(w, np.repeat(sc, 32, axis=1).astype(np.float64))
        mn = sb.copy()
        mn[:, 2], mn[:, 3] = 0x00, 0x3C                     # d = 0, dmin = 1
        w = orc.dequant(kind, mn.reshape(-1), 65536, 256)
        assert np.array_equal(w, -np.repeat(m, 32, axis=1).astype(np.float64))


# --------------------------------------------------------- integer sums
def unpack_matrix(kind, w, rows, K):
    """Per-weight integer codes and per-weight integer scales from the
    (pinned) block decoders."""
    nb = K // 256
    bpb = synth.BLOCK_BYTES[kind]
    Q = np.zeros((rows, K), np.int64)
    SC = np.zeros((rows, K), np.int64)
    M = np.zeros((rows, K), np.int64)
    for r in range(rows):
        for s in range(nb):
            blk = w[(r * nb + s) * bpb:(r * nb + s + 1) * bpb]
            if kind == "q6k":
                q, sc, _ = orc.q6k_decode(blk)
                SC[r, s * 256:(s + 1) * 256] = np.repeat(sc.astype(np.int64), 16)
            else:
                q, sc, m, _, _ = (orc.q5k_decode if kind == "q5k" else orc.q4k_decode)(blk)
                SC[r, s * 256:(s + 1) * 256] = np.repeat(sc.astype(np.int64), 32)
                M[r, s * 256:(s + 1) * 256] = np.repeat(m.astype(np.int64), 32)
            Q[r, s * 256:(s + 1) * 256] = q.astype(np.int64)
    return Q, SC, M


@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
def test_integer_sums_vs_numpy(kind):
    rows, K, ncols = 12, 768, 3
    g = synth.rng(31)
    w = synth.blocks(kind, g, rows, K)
    xq = orc.quantize_q8_1(synth.activations(g, ncols, K))
    q8 = xq.reshape(ncols, K // 32, 36)[..., 4:].view(np.int8).astype(np.int64)
    Q, SC, _ = unpack_matrix(kind, w, rows, K)
    A = (Q * SC if kind == "q6k" else Q).reshape(rows, K // 32, 32)
    ref = np.einsum("rbi,nbi->nrb", A, q8)
    got = orc.q6k_isums(w, xq, rows, K) if kind == "q6k" else orc.q45_dots(kind, w, xq, rows, K)
    assert np.array_equal(got.astype(np.int64), ref)


# ---------------------------------------------------------------- MMVQ
@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
@pytest.mark.parametrize("rows,K,ncols", [(16, 512, 1), (9, 1024, 3), (5, 256, 8)])
def test_mmvq_vs_fp64_bruteforce(kind, rows, K, ncols):
    g = synth.rng(41 + rows + K + ncols)
    w = synth.blocks(kind, g, rows, K)
    xq = orc.quantize_q8_1(synth.activations(g, ncols, K))
    W = orc.dequant(kind, w, rows, K)
    X = orc.dequant_q8_1(xq, K)
    ref = X @ W.T                                     # [ncols][rows]
    out, ab = orc.mmvq(kind, w, xq, rows, K)
    assert np.all(np.abs(out - ref.T.T) <= 1e-12 * ab + 1e-300)
    # row-window form gives the same numbers
    out2, _ = orc.mmvq(kind, w, xq, rows, K, row0=rows // 2, nrows=rows - rows // 2)
    assert np.array_equal(out2, out[:, rows // 2:])


def test_q6k_integer_matvec_special_case():
    """d = 1 and every scale 1: the product is d_a times a plain integer
    matrix-vector product of (q6 - 32) with the Q8_1 quants."""
    g = synth.rng(51)
    rows, K = 6, 512
    M = g.integers(0, 64, (rows, K))
    w = np.concatenate([encode_q6k(M[r, s * 256:(s + 1) * 256], np.ones(16, int), 0x3C00)
                        for r in range(rows) for s in range(K // 256)])
    xq = synth.exact_q8_1(g, 2, K, qmax=127)
    q8 = xq.reshape(2, K // 32, 36)[..., 4:].view(np.int8).astype(np.int64).reshape(2, K)
    ref = 0.25 * ((M - 32) @ q8.T).T
    out, _ = orc.mmvq("q6k", w, xq, rows, K)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
def test_exact_arithmetic_configuration(kind):
    g = synth.rng(61)
    rows, K, ncols = 7, 2560, 4
    if kind == "q6k":
        w = synth.exact_q6k_blocks(g, rows, K)
    else:
        w = synth.exact_q45_blocks(g, rows, K, kind == "q5k")
    xq = synth.exact_q8_1(g, ncols, K)
    out, _ = orc.mmvq(kind, w, xq, rows, K)
    ref = orc.dequant_q8_1(xq, K) @ orc.dequant(kind, w, rows, K).T
    assert np.array_equal(out, ref)
    assert np.array_equal(out.astype(np.float32).astype(np.float64), out)


# ---------------------------------------------------------- planar Q6_K
def test_planar_layout_pins():
    g = synth.rng(71)
    rows, K = 3, 512
    w = synth.q6k_blocks(g, rows, K)
    P = orc.q6k_to_planar(w, rows, K)
    NB = rows * K // 256
    assert P.size == w.size
    blk = w.reshape(NB, 210)
    assert np.array_equal(P[192 * NB:208 * NB].reshape(NB, 16), blk[:, 192:208])
    assert np.array_equal(P[208 * NB:].reshape(NB, 2), blk[:, 208:210])
    # dword-level unpack (shift/mask form) gives 4*(q6-32) as int8 per weight
    A = P[:128 * NB].reshape(NB, 8, 4, 4).view("<u4")[..., 0].astype(np.uint64)    # [NB][8][4]
    B = P[128 * NB:192 * NB].reshape(NB, 8, 2, 4).view("<u4")[..., 0].astype(np.uint64)
    m3, mfc = 0x03030303, 0xFCFCFCFC
    O = [A[..., 0] & mfc, A[..., 1] & mfc, A[..., 2] & mfc, A[..., 3] & mfc,
         B[..., 0] & mfc, B[..., 1] & mfc,
         ((A[..., 2] & m3) << 6) | ((A[..., 1] & m3) << 4) | ((A[..., 0] & m3) << 2),
         ((B[..., 1] & m3) << 6) | ((B[..., 0] & m3) << 4) | ((A[..., 3] & m3) << 2)]
    O = np.stack(O, -1).astype(np.uint32)                    # [NB][8][8 dwords]
    v = O.view(np.uint8).reshape(NB, 256).view(np.int8).astype(np.int64)
    q = np.stack([orc.q6k_decode(blk[t])[0] for t in range(NB)]).astype(np.int64)
    assert np.array_equal(v, 4 * q)
    # the conversion is a bit permutation (up to a constant): one flipped
    # source bit of ql/qh flips exactly one planar bit
    for byte, bit in [(0, 0), (5, 7), (100, 3), (130, 1), (191, 6)]:
        w2 = w.copy()
        w2[byte] ^= 1 << bit
        P2 = orc.q6k_to_planar(w2, rows, K)
        flips = np.unpackbits(P2 ^ P).sum()
        assert flips == 1


def test_q8_1_planar_pins():
    """Column-planar Q8_1 (the layout text of the library header): a tiny
    case enumerated by hand, and on real activations the planar quants and d
    dequantize to the same values as the blocks."""
    K, ncols = 64, 2                       # two blocks per column
    src = np.arange(144, dtype=np.uint8)
    got = orc.q8_1_to_planar(src, K)
    want = []
    for c in (0, 72):                      # column base in both forms
        want += list(range(c + 4, c + 36))     # block 0 quants
        want += list(range(c + 40, c + 72))    # block 1 quants
        want += [c + 0, c + 1, c + 36, c + 37]  # d of blocks 0, 1
        want += [c + 2, c + 3, c + 38, c + 39]  # s of blocks 0, 1
    assert got.tolist() == want
    # semantics on quantized data: q (int8) * d (fp16) per block
    g = synth.rng(77)
    K, ncols = 512, 3
    x = synth.activations(g, ncols, K)
    xq = orc.quantize_q8_1(x)
    pl = orc.q8_1_to_planar(xq, K).reshape(ncols, K // 32 * 36)
    deq = orc.dequant_q8_1(xq, K)
    q = pl[:, :K].view(np.int8).astype(np.float64)
    d = pl[:, K:K + 2 * (K // 32)].copy().view(np.float16).astype(np.float64)
    assert np.array_equal(q * np.repeat(d, 32, axis=1), deq)
    s16 = pl[:, K + 2 * (K // 32):].copy().view(np.float16)
    blk = xq.reshape(ncols, K // 32, 36)
    assert np.array_equal(s16.view(np.uint16), blk[:, :, 2:4].copy().view(np.uint16)[:, :, 0])


def test_tiled_layout_pins():
    """The tiled layout is the (pinned) planar one with the entries of every
    16-row group interleaved: for one row it is the planar layout itself,
    and for any row count each plane is the planar plane with [row][position]
    turned into [position][row] inside every tile (a numpy transpose, the
    last tile R = rows % 16 rows high)."""
    for rows, K in [(1, 512), (16, 256), (37, 768)]:
        w = synth.q6k_blocks(synth.rng(72 + rows), rows, K)
        P = orc.q6k_to_planar(w, rows, K)
        T = orc.q6k_to_tiled(w, rows, K)
        assert T.size == P.size
        if rows == 1:
            assert np.array_equal(T, P)
        NB, nsb, nb = rows * K // 256, K // 32, K // 256
        for lo, hi, esz, npos in [(0, 128 * NB, 16, nsb), (128 * NB, 192 * NB, 8, nsb),
                                  (192 * NB, 208 * NB, 8, nsb // 4), (208 * NB, 210 * NB, 2, nb)]:
            p = P[lo:hi].reshape(rows, npos, esz)
            t = T[lo:hi]
            off = 0
            for r0 in range(0, rows, 16):
                part = p[r0:r0 + 16].transpose(1, 0, 2).reshape(-1)
                assert np.array_equal(t[off:off + part.size], part), (rows, K, lo, r0)
                off += part.size
            assert off == hi - lo


def test_gather_pins():
    """Row gather: on GGUF it is numpy block indexing (zero rows for bad
    ids); gathering every row in order is the conversion itself; on the
    planar layout each plane of the output is the numpy row selection of the
    full conversion's plane; the tiled output is the per-tile transpose of
    the planar one (the pinned relation between the two layouts)."""
    rows, K = 37, 768
    nb, nsb = K // 256, K // 32
    w = synth.q6k_blocks(synth.rng(73), rows, K)
    ids = np.array([3, 36, 0, 3, -1, 40, 20, 16, 17, 5, 6, 7, 8, 9, 10, 11, 12, 30], np.int32)
    nout = ids.size
    ok = (ids >= 0) & (ids < rows)
    rb = nb * 210
    exp = np.concatenate([w[i * rb:(i + 1) * rb] if 0 <= i < rows else np.zeros(rb, np.uint8) for i in ids])
    assert np.array_equal(orc.q6k_gather(w, 0, rows, K, ids), exp)
    every = np.arange(rows, dtype=np.int32)
    assert np.array_equal(orc.q6k_gather(w, 1, rows, K, every), orc.q6k_to_planar(w, rows, K))
    assert np.array_equal(orc.q6k_gather(w, 2, rows, K, every), orc.q6k_to_tiled(w, rows, K))
    full = orc.q6k_to_planar(w, rows, K)
    gp = orc.q6k_gather(w, 1, rows, K, ids)
    gt = orc.q6k_gather(w, 2, rows, K, ids)
    NBs, NBd = rows * nb, nout * nb
    for (lo, hi, esz, npos) in [(0, 128, 16, nsb), (128, 192, 8, nsb), (192, 208, 8, nsb // 4), (208, 210, 2, nb)]:
        fs = full[lo * NBs:hi * NBs].reshape(rows, npos, esz)
        pd = gp[lo * NBd:hi * NBd].reshape(nout, npos, esz)
        assert np.array_equal(pd[ok], fs[ids[ok]])
        assert not pd[~ok].any()
        td = gt[lo * NBd:hi * NBd]
        off = 0
        for r0 in range(0, nout, 16):
            part = pd[r0:r0 + 16].transpose(1, 0, 2).reshape(-1)
            assert np.array_equal(td[off:off + part.size], part)
            off += part.size


# ----------------------------------------------------------------- MoE
def test_moe_chain_vs_fp64_bruteforce():
    g = synth.rng(81)
    E, T, topk, dm, dff = 4, 3, 2, 512, 256
    gate, up, down = synth.moe_weights(g, E, dm, dff)
    ids, rw = synth.routing(g, T, E, topk)
    xq = orc.quantize_q8_1(synth.activations(g, T, dm))
    res = orc.grouped_expert(gate, up, down, xq, ids, rw, E, T, topk, dm, dff)
    X = orc.dequant_q8_1(xq, dm)
    gb, db = dff * (dm // 256) * 144, dm * (dff // 256) * 210
    out = np.zeros((T, dm))
    for t in range(T):
        for k in range(topk):
            e, slot = ids[t, k], t * topk + k
            Wg = orc.dequant("q4k", gate[e * gb:(e + 1) * gb], dff, dm)
            Wu = orc.dequant("q4k", up[e * gb:(e + 1) * gb], dff, dm)
            Wd = orc.dequant("q6k", down[e * db:(e + 1) * db], dm, dff)
            gg, uu = Wg @ X[t], Wu @ X[t]
            assert np.allclose(res["g"][slot], gg, rtol=0, atol=1e-12 * np.abs(gg).max())
            assert np.allclose(res["u"][slot], uu, rtol=0, atol=1e-12 * np.abs(uu).max())
            h = (gg / (1 + np.exp(-gg)) * uu).astype(np.float32)
            # the fp32 rounding of h may differ only where fp64 sums differ
            assert np.all(np.abs(res["h"][slot] - h) <= np.abs(h) * 2.0 ** -23)
            hq = orc.quantize_q8_1(res["h"][slot][None])[0]
            assert np.array_equal(res["hq"][slot], hq)
            y = Wd @ orc.dequant_q8_1(hq[None], dff)[0]
            assert np.allclose(res["y"][slot], y, rtol=0, atol=1e-12 * res["y_absum"][slot].max())
            out[t] += float(rw[t, k]) * y
    assert np.allclose(res["out"], out, rtol=0, atol=1e-12 * res["out_absum"].max())
    # the staged form (down product fed an externally supplied hidden-state
    # Q8_1, slot-major) reproduces the chain when fed the chain's own hq
    res2 = orc.grouped_expert(gate, up, down, xq, ids, rw, E, T, topk, dm, dff, hq_in=res["hq"])
    assert np.array_equal(res2["out"], res["out"]) and np.array_equal(res2["y"], res["y"])
    # and a perturbed hq for one slot changes exactly that slot's y
    hq_bad = res["hq"].copy()
    hq_bad[1, 4] ^= 1
    res3 = orc.grouped_expert(gate, up, down, xq, ids, rw, E, T, topk, dm, dff, hq_in=hq_bad)
    changed = [s for s in range(T * topk) if not np.array_equal(res3["y"][s], res["y"][s])]
    assert changed == [1]


def test_moe_single_slot_reduces_to_dense_chain():
    g = synth.rng(82)
    E, dm, dff = 3, 256, 256
    gate, up, down = synth.moe_weights(g, E, dm, dff)
    xq = orc.quantize_q8_1(synth.activations(g, 1, dm))
    ids, rw = np.array([[2]], np.int32), np.array([[1.0]], np.float32)
    res = orc.grouped_expert(gate, up, down, xq, ids, rw, E, 1, 1, dm, dff)
    gb, db = dff * (dm // 256) * 144, dm * (dff // 256) * 210
    gg, _ = orc.mmvq("q4k", gate[2 * gb:3 * gb], xq, dff, dm)
    uu, _ = orc.mmvq("q4k", up[2 * gb:3 * gb], xq, dff, dm)
    h = (gg / (1 + np.exp(-gg)) * uu).astype(np.float32)
    y, _ = orc.mmvq("q6k", down[2 * db:3 * db], orc.quantize_q8_1(h), dm, dff)
    assert np.array_equal(res["out"], y)


def test_moe_rejects_bad_ids():
    g = synth.rng(83)
    gate, up, down = synth.moe_weights(g, 2, 256, 256)
    xq = orc.quantize_q8_1(synth.activations(g, 1, 256))
    with pytest.raises(ValueError):
        orc.grouped_expert(gate, up, down, xq, np.array([[2]], np.int32),
                           np.array([[1.0]], np.float32), 2, 1, 1, 256, 256)


def test_rmsnorm_pins():
    """RMSNorm oracle (the norm ahead of the fused quantizer): a hand-worked
    block, exact invariances of the definition, unit RMS, the eps limit."""
    # x = 2 everywhere: mean x^2 = 4, r = 1/2, y = 1 -> every code 127
    K = 32
    x = np.full((1, K), 2.0, np.float32)
    g = np.ones(K, np.float32)
    assert np.array_equal(orc.rmsnorm(x, g, 0.0), np.ones((1, K), np.float32))
    q = orc.rmsnorm_quantize_q8_1(x, g, 0.0)[0]
    assert np.all(q[4:].view(np.int8) == 127)
    assert q[0:2].view(np.float16)[0] == np.float16(np.float32(1.0) / np.float32(127.0))
    # random columns
    r = synth.rng(4242)
    K, n = 2560, 3
    x = (r.standard_normal((n, K)) * 3.0).astype(np.float32)
    g = (0.5 + r.random(K)).astype(np.float32)
    y = orc.rmsnorm(x, g, 0.0)
    # invariant under x -> 4x with eps = 0 (every step scales exactly)
    assert np.array_equal(orc.rmsnorm(x * np.float32(4.0), g, 0.0), y)
    # linear in gamma: 2*gamma doubles y exactly; the codes stay, d doubles
    y2 = orc.rmsnorm(x, g * np.float32(2.0), 0.0)
    assert np.array_equal(y2, 2 * y)
    qa = orc.quantize_q8_1(y).reshape(n, -1, 36)
    qb = orc.quantize_q8_1(y2).reshape(n, -1, 36)
    assert np.array_equal(qa[:, :, 4:], qb[:, :, 4:])
    assert np.array_equal(qa[:, :, 0:2].copy().view(np.float16).astype(np.float64) * 2,
                          qb[:, :, 0:2].copy().view(np.float16).astype(np.float64))
    # unit root-mean-square of y / gamma when eps = 0
    rms = np.sqrt(np.mean((y.astype(np.float64) / g) ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-6)
    # eps far above mean(x^2): y -> x * gamma / sqrt(eps)
    xs = (x * np.float32(1e-4)).astype(np.float32)
    ye = orc.rmsnorm(xs, g, 1.0e4)
    want = xs.astype(np.float64) * g / 100.0
    assert np.all(np.abs(ye - want) <= 1e-6 * np.abs(want) + 1e-12)
    # the fused form is the quantizer of y, block for block
    assert np.array_equal(orc.rmsnorm_quantize_q8_1(x, g, 1e-6), orc.quantize_q8_1(orc.rmsnorm(x, g, 1e-6)))

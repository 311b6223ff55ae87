"""Q8_1 quantizer fixtures shared by the CPU pins and the GPU tests.

numpy_q8_1 is a Q8_1 quantizer written here, independently of the oracle and
of the HIP library, from the reading of the quantizer: amax = max|x|,
d = amax/127 and x/d as fp32 divisions, round half away from zero, clamp to
+-127, d and s = d * sum q (an fp32 product) stored as fp16 rounded to
nearest even.  The block generators search seeded random inputs (numpy's
IEEE fp32 arithmetic) for the places where plausible other readings give
other bytes: quotients x/d at or next to half-integers, and sums whose fp32
product d * sum lands exactly on an fp16 midpoint while the exact product
does not (there a single rounding of the exact product to fp16, as a fused
multiply-convert does, goes the other way).
"""
import numpy as np

from quant_mat_vec_amd import synth


def numpy_q8_1(x, mode="div32"):
    """Q8_1 written here from the quantizer reading, with numpy's IEEE fp32
    arithmetic: amax = max|x|, d = amax/127 (fp32 division), q =
    round-half-away-from-zero(x/d) with x/d an fp32 division, clamped to
    +-127 (all zero when d == 0), stored d = fp16(d), s = fp16(d * sum q)
    (fp32 product), both rounded to nearest even by numpy's cast.  `mode`
    selects a deliberately wrong variant to show that the fixtures below tell
    them apart: "recip" (x times the fp32 reciprocal of d), "div64" (x/d in
    fp64), "even" (ties to even) and "fused_s" (s as the exact product d *
    sum rounded to fp16 once)."""
    x = np.ascontiguousarray(x, np.float32)
    ncols, K = x.shape
    xb = x.reshape(ncols, K // 32, 32)
    amax = np.abs(xb).max(-1)
    d = amax / np.float32(127)
    assert d.dtype == np.float32
    dz = np.where(d > 0, d, np.float32(1))[..., None]
    if mode == "recip":
        v = (xb * (np.float32(1) / dz)).astype(np.float64)
    elif mode == "div64":
        v = xb.astype(np.float64) / dz.astype(np.float64)
    else:
        v = (xb / dz).astype(np.float64)
    if mode == "even":
        q = np.rint(v)
    else:
        q = np.sign(v) * np.floor(np.abs(v) + 0.5)       # exact in fp64
    q = np.clip(q, -127, 127)
    q[d == 0] = 0
    q = q.astype(np.int8)
    s = d * q.astype(np.int32).sum(-1).astype(np.float32)
    assert s.dtype == np.float32
    if mode == "fused_s":
        s = d.astype(np.float64) * q.astype(np.int64).sum(-1)      # exact, rounded once below
    out = np.zeros((ncols, K // 32, 36), np.uint8)
    out[..., 0:2] = d.astype(np.float16).view(np.uint8).reshape(ncols, K // 32, 2)
    out[..., 2:4] = s.astype(np.float16).view(np.uint8).reshape(ncols, K // 32, 2)
    out[..., 4:] = q.view(np.uint8)
    return out.reshape(ncols, -1)


def near_tie_blocks(seed=31, nblocks=512):
    """fp32 activations whose quotient x/d lies at or within a few ulps of a
    half-integer k + 1/2, chosen where an fp32 division, a multiply by the
    fp32 reciprocal and an fp64 division round to different codes, plus exact
    ties for the tie rule.  Each block holds its amax first (so d is fixed)
    and 31 such values."""
    g = synth.rng(seed)
    picked = []
    while len(picked) < nblocks:
        amax = np.float32(np.exp2(g.uniform(-8, 8)) * (1 + g.random()))
        d = amax / np.float32(127)
        r = np.float32(1) / d
        vals = []
        for k in g.integers(0, 126, 64):
            x0 = np.float32((k + 0.5) * float(d))
            for j in range(-3, 4):
                x = x0
                for _ in range(abs(j)):
                    x = np.nextafter(x, np.float32(np.inf if j > 0 else -np.inf))
                q32 = float(x / d)
                a = np.floor(abs(q32) + 0.5)
                b = np.floor(abs(float(x * r)) + 0.5)
                c = np.floor(abs(float(x) / float(d)) + 0.5)
                e = np.rint(abs(q32))
                if a != b or a != c or a != e:
                    vals.append(x if g.random() < 0.5 else -x)
        if len(vals) >= 31:
            blk = np.zeros(32, np.float32)
            blk[0] = amax if g.random() < 0.5 else -amax
            blk[1:] = np.asarray(vals[:31], np.float32)
            picked.append(blk)
    return np.concatenate(picked).reshape(1, -1)




def s_tie_blocks(seed=32, nblocks=48):
    """fp32 [1][32 * nblocks]: blocks whose fp32 product d * sum is the
    midpoint of two consecutive normal fp16 values while the exact product
    lies on the side that the tie rule does not pick, so that rounding the
    fp32 product and rounding the exact product give different fp16 s."""
    g = synth.rng(seed)
    found = []
    while sum(len(f) for f in found) < nblocks:
        x = (g.standard_normal((1 << 16, 32)) * np.exp2(g.integers(-6, 7, (1 << 16, 1)))).astype(np.float32)
        amax = np.abs(x).max(-1)
        d = amax / np.float32(127)
        v = (x / d[:, None]).astype(np.float64)
        q = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127).astype(np.int64)
        sm = q.sum(-1)
        p = d * sm.astype(np.float32)
        bits = p.view(np.uint32)
        mag = np.abs(p)
        mid = ((bits & 0x1FFF) == 0x1000) & (mag >= 2.0 ** -14) & (mag < 65504)
        exact = d.astype(np.float64) * sm
        with np.errstate(over="ignore"):
            apart = exact.astype(np.float16) != p.astype(np.float16)     # the two roundings differ
        found.append(x[mid & apart])
    return np.concatenate(found)[:nblocks].reshape(1, -1)

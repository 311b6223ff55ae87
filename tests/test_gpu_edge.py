"""GPU parity on edge-case inputs, through the C ABI, against the CPU oracle.

The routed-expert validation of PR #2746 ("sycl: use packed word expansion
for Q2_0 expert down on Battlemage", section "B70 validation") runs its
kernels over several activation patterns and token windows; here every
product layout meets the oracle on inputs at the edges of the formats:

* the int32 bound of a Q6_K sub-block sum: scales -128 and 127, codes 0 and
  63 (q6 - 32 = -32 and 31) against quants +-127, so that |isum| reaches
  2 * 128 * 16 * 32 * 127 = 16,646,144; the Q4_K/Q5_K counterpart with 6-bit
  scales and mins of 63 and codes 15 / 31;
* activation blocks with d = 0 (all-zero quants), with subnormal fp16 d, and
  weights with negative fp16 d (and dmin);
* five activation patterns through the quantizer (the reading of the
  unnamed "activation patterns": N(0,1), an all-zero block, constant
  blocks, one-hot sparse columns, alternating +-large values);
* Q4_K and Q5_K at six and seven columns on long rows (K = 4096 .. 10240),
  the column counts of a verify window.

Bars: integer sums bit for bit; fp32 outputs within 1e-5 of the oracle
relative to the sum of absolute terms (tests/gpu_util.py), on every row.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import assert_close, dev, isums, mmvq, note, planar, quantize, tiled, DEV

pytestmark = pytest.mark.gpu

GG, PL, TL = qmv.LAYOUT_GGUF, qmv.LAYOUT_PLANAR, qmv.LAYOUT_TILED
XT = TL | qmv.ACT_PLANAR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def f16(v) -> np.ndarray:
    return np.asarray(v, np.float16).reshape(-1).view(np.uint8)


def q8_1_bytes(d_bits: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Q8_1 blocks [ncols][nb] from fp16 d bit patterns and int8 quants
    [ncols][nb][32]; s = fp16(d * sum q) rounded by numpy."""
    ncols, nb = d_bits.shape
    blk = np.zeros((ncols, nb, 36), np.uint8)
    blk[..., 0:2] = d_bits.astype(np.uint16).view(np.uint8).reshape(ncols, nb, 2)
    d = d_bits.astype(np.uint16).view(np.float16).astype(np.float32)
    s = (d * q.astype(np.int32).sum(-1).astype(np.float32)).astype(np.float16)
    blk[..., 2:4] = s.view(np.uint8).reshape(ncols, nb, 2)
    blk[..., 4:] = q.astype(np.int8).view(np.uint8)
    return blk.reshape(ncols, -1)


def col_planar(xq_np: np.ndarray, K: int) -> np.ndarray:
    """The column-planar arrangement of Q8_1 blocks [ncols][K/32*36]: per
    column the quants, then the fp16 d, then the fp16 s."""
    nb = K // 32
    b = xq_np.reshape(-1, nb, 36)
    return np.concatenate([b[..., 4:].reshape(len(b), -1), b[..., 0:2].reshape(len(b), -1),
                           b[..., 2:4].reshape(len(b), -1)], axis=1)


def check_every_layout(kind, w, xq_np, rows, K, what):
    """isums bit for bit and outputs within tolerance, every row, for every
    layout the format has (Q6_K: GGUF, planar, tiled with Q8_1 blocks and
    with column-planar activations)."""
    ncols = xq_np.shape[0]
    xq = dev(xq_np.reshape(-1))
    ref, ab = orc.mmvq(kind, w, xq_np, rows, K)
    wd = dev(w)
    if kind == "q6k":
        ref_i = orc.q6k_isums(w, xq_np, rows, K)
        xp = dev(col_planar(xq_np, K).reshape(-1))
        for lay, wl, a in ((GG, wd, xq), (PL, planar(wd, rows, K), xq), (TL, tiled(wd, rows, K), xq),
                           (XT, tiled(wd, rows, K), xp)):
            note(f"{what}: q6k layout={lay} {rows}x{K} N={ncols}")
            assert np.array_equal(isums(kind, wl, a, rows, K, ncols, lay), ref_i), f"{what} isums layout {lay}"
            assert_close(mmvq(kind, wl, a, rows, K, ncols, lay), ref, ab, f"{what} layout {lay}")
    else:
        note(f"{what}: {kind} {rows}x{K} N={ncols}")
        assert np.array_equal(isums(kind, wd, xq, rows, K, ncols), orc.q45_dots(kind, w, xq_np, rows, K)), what
        assert_close(mmvq(kind, wd, xq, rows, K, ncols), ref, ab, what)
    return ref


# ------------------------------------------------- the int32 sum bound
def q6k_extreme(g, rows, K):
    """Q6_K blocks whose every scale is -128 or 127 and every code 0 or 63;
    row r takes (scale, code) pattern r % 4 with random flips elsewhere."""
    nb = rows * (K // 256)
    blk = np.zeros((rows, K // 256, 210), np.uint8)
    pat = np.arange(rows) % 4
    sc = np.where((pat == 0) | (pat == 2), -128, 127).astype(np.int8)
    code0 = (pat <= 1)                                         # all codes 0, else all 63
    for r in range(rows):
        q6 = np.full(256, 0 if code0[r] else 63, np.int64)
        if pat[r] >= 2:
            flip = g.random((K // 256, 256)) < 0.5
        else:
            flip = np.zeros((K // 256, 256), bool)
        for s in range(K // 256):
            v = np.where(flip[s], 63 - q6, q6)
            for h in range(2):
                for l in range(32):
                    for c in range(4):
                        x = int(v[128 * h + 32 * c + l])
                        blk[r, s, 64 * h + 32 * (c & 1) + l] |= (x & 15) << (4 * (c >> 1))
                        blk[r, s, 128 + 32 * h + l] |= (x >> 4) << (2 * c)
            blk[r, s, 192:208] = np.full(16, sc[r], np.int8).view(np.uint8)
            blk[r, s, 208:210] = f16(2.0 ** -12)
    return blk.reshape(-1), nb


@pytest.mark.parametrize("rows,K,ncols", [(37, 2560, 8), (20, 768, 3), (17, 10240, 1)])
def test_q6k_int32_bound(rows, K, ncols):
    g = synth.rng(1700 + rows)
    w, _ = q6k_extreme(g, rows, K)
    nb = K // 32
    # quants +-127: column 0 all +127 (rows with code 0 and scale -128 reach
    # +16,646,144), column 1 all -127, the rest random signs
    q = np.where(g.random((ncols, nb, 32)) < 0.5, 127, -127).astype(np.int8)
    q[0] = 127
    if ncols > 1:
        q[1] = -127
    xq_np = q8_1_bytes(np.full((ncols, nb), 0x2C00, np.uint16), q)     # d = 2^-4
    check_every_layout("q6k", w, xq_np, rows, K, "Q6_K int32 bound")
    i = orc.q6k_isums(w, xq_np, rows, K)
    assert i.max() == 16646144          # the bound is reached (scale -128, code 0, quants 127)


@pytest.mark.parametrize("kind", ["q4k", "q5k"])
def test_q45_extreme_scales(kind):
    rows, K, ncols = 33, 2560, 4
    g = synth.rng(1710)
    nbytes = 176 if kind == "q5k" else 144
    blk = synth.blocks(kind, g, rows, K).reshape(-1, nbytes).copy()
    blk[:, 4:16] = 0xFF                                       # every 6-bit scale and min = 63
    qs0 = 48 if kind == "q5k" else 16
    blk[::2, qs0:] = 0xFF                                     # codes 15 (31 with qh)
    if kind == "q5k":
        blk[::2, 16:48] = 0xFF
    blk[1::2, 0:2] = f16(-(2.0 ** -10))                       # negative d on odd blocks
    blk[:, 2:4] = f16(2.0 ** -11)
    q = np.where(g.random((ncols, K // 32, 32)) < 0.5, 127, -127).astype(np.int8)
    q[0] = 127
    xq_np = q8_1_bytes(np.full((ncols, K // 32), 0x3000, np.uint16), q)    # d = 2^-3
    check_every_layout(kind, blk.reshape(-1), xq_np, rows, K, f"{kind} extreme scales")


# ------------------------------------ zero, subnormal and negative scales
@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
def test_zero_and_subnormal_activation_blocks_negative_d(kind):
    rows, K, ncols = 45, 2560, 5
    g = synth.rng(1720)
    w = synth.blocks(kind, g, rows, K)
    bpb = {"q6k": 210, "q4k": 144, "q5k": 176}[kind]
    wb = w.reshape(-1, bpb)
    neg = g.random(len(wb)) < 0.5
    if kind == "q6k":
        wb[neg, 209] |= 0x80                                  # negative d
    else:
        wb[neg, 1] |= 0x80                                    # negative d
        wb[g.random(len(wb)) < 0.3, 3] |= 0x80                # negative dmin
    nb = K // 32
    q = g.integers(-127, 128, (ncols, nb, 32)).astype(np.int8)
    d = (np.abs(g.standard_normal((ncols, nb))) * 2e-2).astype(np.float16).view(np.uint16)
    zero = g.random((ncols, nb)) < 0.2                        # blocks of a zero activation
    d[zero] = 0
    q[zero] = 0
    sub = (~zero) & (g.random((ncols, nb)) < 0.3)             # subnormal fp16 d
    d[sub] = g.integers(1, 1024, int(sub.sum())).astype(np.uint16)
    d[0, :] = 0                                               # one all-zero column
    q[0] = 0
    xq_np = q8_1_bytes(d, q)
    ref = check_every_layout(kind, wb.reshape(-1), xq_np, rows, K, f"{kind} zero/subnormal d_a, negative d")
    assert np.all(ref[0] == 0)


# ------------------------------------------- five activation patterns
def patterns(g, K):
    """fp32 [5][K]: N(0,1); N(0,1) with an all-zero block; constant blocks
    (a different constant per block); one-hot sparse (one nonzero value per
    block, the rest zero); alternating +-large values."""
    nb = K // 32
    x = np.zeros((5, K), np.float32)
    x[0] = g.standard_normal(K)
    x[1] = g.standard_normal(K)
    x[1, 64:96] = 0.0
    x[2] = np.repeat(g.standard_normal(nb).astype(np.float32) * 3, 32)
    x[3, np.arange(nb) * 32 + g.integers(0, 32, nb)] = g.standard_normal(nb).astype(np.float32) * 10
    x[4] = np.float32(3.0e4) * np.where(np.arange(K) % 2 == 0, 1, -1) * (1 + g.random(K).astype(np.float32))
    return x


@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
@pytest.mark.parametrize("rows,K", [(37, 2560), (50, 768)])
def test_five_activation_patterns(kind, rows, K):
    g = synth.rng(1730 + K)
    w = synth.blocks(kind, g, rows, K)
    x = patterns(g, K)
    xq, xq_np = quantize(x)                               # the GPU quantizer ...
    assert np.array_equal(xq_np, orc.quantize_q8_1(x))    # ... bit for bit
    check_every_layout(kind, w, xq_np, rows, K, f"{kind} activation patterns")
    # each pattern alone (one column) gives the bits of its column in the
    # five-column call
    if kind != "q6k":
        full = mmvq(kind, dev(w), xq, rows, K, 5)
        nbq = K // 32 * 36
        for c in range(5):
            one = mmvq(kind, dev(w), xq[c * nbq:(c + 1) * nbq], rows, K, 1)
            assert np.array_equal(one[0].view(np.uint32), full[c].view(np.uint32))


# --------------------------------- Q4_K / Q5_K, verify-window widths, long rows
@pytest.mark.parametrize("K", [4096, 6144, 8192, 10240])
@pytest.mark.parametrize("ncols", [6, 7])
@pytest.mark.parametrize("kind", ["q4k", "q5k"])
def test_q45_six_seven_columns_long_rows(kind, ncols, K):
    rows = 70
    g = synth.rng(1740 + K + ncols)
    w = synth.blocks(kind, g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    check_every_layout(kind, w, xq_np, rows, K, f"{kind} N={ncols} K={K}")


@pytest.mark.parametrize("ncols", [6, 7])
@pytest.mark.parametrize("kind", ["q4k", "q5k"])
def test_q45_six_seven_columns_full_size(kind, ncols):
    """The 2560 x 6144 decode matrix (rows x cols) at six and seven columns,
    every row."""
    from tests.gpu_util import check_all_rows
    rows, K = 2560, 6144
    g = synth.rng(synth.seed_for(3, 7, ncols))
    w = synth.blocks(kind, g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    note(f"{kind} {rows}x{K} N={ncols} all rows")
    check_all_rows(kind, w, xq_np, mmvq(kind, dev(w), xq, rows, K, ncols), rows, K)

"""Grouped MoE expert chain in exact arithmetic, through the C ABI, against
the CPU oracle bit for bit.

The routed-expert kernels of issue #2801 ("[Feature]: SYCL: cheaper IQ weight
decodes in the grouped expert kernels") are held to the same bits as a
reference (its "exactly the same bits"; PR #2746 "B70 validation" checks
byte-exact outputs).  The chain's float stages (silu, the product with up,
the requantization, the routed sum) would blur an integer mistake into fp32
rounding, so these inputs make every float step exact:

* the gate output is at least 128 for every row, so exp(-g) underflows and
  silu(g) = g exactly in fp32 and fp64;
* weights and activations take power-of-two d, dmin and small quants, so
  every partial sum of the gate, up and down products is an exact multiple
  of one unit below 2^24 units (exact in fp32 in any order);
* one factor of h = g * u has a single significant bit, so h is exact.

Three configurations, each isolating one integer path with random full
weights while the others are held to known values:
  gate: random positive gate rows (every sub-block), up = +-2^j per row;
  up:   gate = 128 or 256 per row, random up rows (every sub-block, min
        term included);
  down: gate = 128, up = integers U in [-127, 127] with a 127 in every
        32-row group, so h = 128 U quantizes to d = 128, q = U exactly;
        random down rows (q6 - 32 in [-4, 3], scales -1..1, d in {1/2, 1})
        and route weights in {1/2, 1}: y and out are exact.
h (gate, up) and h, hq, y and out (down) must equal the oracle bit for bit,
with both down layouts and both the one-token (fused down + routed sum) and
the multi-token (three-launch) paths.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import DEV, canaries_intact, dev, guarded, host, note, planar

pytestmark = pytest.mark.gpu

E, DM, DFF, TOPK = 16, 2560, 768, 8
GG, PL = qmv.LAYOUT_GGUF, qmv.LAYOUT_PLANAR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def f16(v, n):
    return np.broadcast_to(np.asarray(v, np.float16), (n,)).copy().view(np.uint8).reshape(n, 2)


def enc_q4k(q4, sc, m, d, dmin):
    """Q4_K blocks [n][144] from codes [n][256] in 0..15, 6-bit scales and
    mins [n][8], fp16 d and dmin [n] (the GGUF layout written out)."""
    n = len(q4)
    q4, sc, m = q4.astype(np.int64), sc.astype(np.int64), m.astype(np.int64)
    blk = np.zeros((n, 144), np.uint8)
    blk[:, 0:2], blk[:, 2:4] = f16(d, n), f16(dmin, n)
    for j in range(4):
        blk[:, 4 + j] = (sc[:, j] & 63) | ((sc[:, j + 4] >> 4) << 6)
        blk[:, 8 + j] = (m[:, j] & 63) | ((m[:, j + 4] >> 4) << 6)
        blk[:, 12 + j] = (sc[:, j + 4] & 15) | ((m[:, j + 4] & 15) << 4)
    l = np.arange(32)
    for j in range(8):
        blk[:, 16 + 32 * (j // 2) + l] |= ((q4[:, 32 * j + l] & 15) << (4 * (j % 2))).astype(np.uint8)
    return blk


def enc_q6k(q6, sc, d):
    """Q6_K blocks [n][210] from codes [n][256] in 0..63, int8 scales [n][16]
    and fp16 d [n]."""
    n = len(q6)
    q6 = q6.astype(np.int64)
    blk = np.zeros((n, 210), np.uint8)
    l = np.arange(32)
    for h in range(2):
        for c in range(4):
            v = q6[:, 128 * h + 32 * c + l]
            blk[:, 64 * h + 32 * (c & 1) + l] |= ((v & 15) << (4 * (c >> 1))).astype(np.uint8)
            blk[:, 128 + 32 * h + l] |= ((v >> 4) << (2 * c)).astype(np.uint8)
    blk[:, 192:208] = sc.astype(np.int8).view(np.uint8)
    blk[:, 208:210] = f16(d, n)
    return blk


def activation(g, T, nonneg):
    """Q8_1 [T][DM/32 * 36]: block 0 has d = 1 and every quant 1; the other
    blocks d = 1/4 and quants in [0, 2] (nonneg) or [-2, 2]."""
    nb = DM // 32
    q = g.integers(0 if nonneg else -2, 3, (T, nb, 32))
    q[:, 0, :] = 1
    d = np.full((T, nb), 0.25)
    d[:, 0] = 1.0
    blk = np.zeros((T, nb, 36), np.uint8)
    blk[..., 0:2] = d.astype(np.float16).view(np.uint8).reshape(T, nb, 2)
    blk[..., 2:4] = (d * q.sum(-1)).astype(np.float16).view(np.uint8).reshape(T, nb, 2)
    blk[..., 4:] = q.astype(np.int8).view(np.uint8)
    return blk.reshape(T, -1)


def one_hot_rows(n, first_q4, sc0, m0, d, dmin):
    """Q4_K rows of DM/256 blocks whose only non-zero codes are in sub-block
    0 of block 0 (first_q4 [n][32]), with scale sc0 and min m0 there and all
    other scales and mins zero; the other blocks are all zero."""
    nb = DM // 256
    q4 = np.zeros((n, nb, 256), np.int64)
    q4[:, 0, :32] = first_q4
    sc = np.zeros((n, nb, 8), np.int64)
    m = np.zeros((n, nb, 8), np.int64)
    sc[:, 0, 0], m[:, 0, 0] = sc0, m0
    dd = np.zeros((n, nb))
    dm = np.zeros((n, nb))
    dd[:, 0], dm[:, 0] = d, dmin
    return enc_q4k(q4.reshape(-1, 256), sc.reshape(-1, 8), m.reshape(-1, 8), dd.reshape(-1),
                   dm.reshape(-1)).reshape(-1)


def gate_const(g, n, values):
    """Gate rows whose output is values[r] (128 or 256): d = 8, code 1 at
    position 0 of block 0 (quant 1, d_a = 1), scale 16 or 32."""
    q = np.zeros((n, 32), np.int64)
    q[:, 0] = 1
    return one_hot_rows(n, q, values // 128 * 16, 0, 8.0, 0.0)


def up_pow2(g, n):
    """Up rows whose output is +-2^j, j in -3..3: +2^j from d = 2^j and one
    code 1 (scale 1); -2^j from the min term (min 1, dmin = 2^(j-5), block
    sum 32)."""
    j = g.integers(-3, 4, n)
    neg = g.random(n) < 0.5
    q = np.zeros((n, 32), np.int64)
    q[:, 0] = np.where(neg, 0, 1)
    vals = np.where(neg, -1.0, 1.0) * np.exp2(j)
    return one_hot_rows(n, q, np.where(neg, 0, 1), np.where(neg, 1, 0), np.where(neg, 0.0, np.exp2(j)),
                        np.where(neg, np.exp2(j - 5.0), 0.0)), vals


def up_int(g, n):
    """Up rows whose output is an integer U in [-127, 127], every 32-row
    group holding a +-127: d = dmin = 1, scale 1, min mm = ceil(-U/32) for
    U < 0, and codes of sub-block 0 summing to U + 32 mm (block sum 32)."""
    U = g.integers(-127, 128, n)
    for r0 in range(0, n, 32):
        U[r0 + g.integers(0, 32)] = 127 if g.random() < 0.5 else -127
    mm = np.where(U < 0, -(U // 32), 0)
    k = U + 32 * mm
    q = np.zeros((n, 32), np.int64)
    for r in range(n):
        left = int(k[r])
        for i in g.permutation(32):
            t = min(15, left)
            q[r, i] = t
            left -= t
        assert left == 0
    return one_hot_rows(n, q, 1, mm, 1.0, 1.0), U


def gate_random_positive(g, n):
    """Random gate rows with positive output >= 128: codes 0..15 (1..15 in
    sub-block 0 of block 0), scales 4..63, no min term, d in {1/2, 1}."""
    nb = DM // 256
    q4 = g.integers(0, 16, (n, nb, 256))
    q4[:, 0, :32] = g.integers(1, 16, (n, 32))
    sc = g.integers(4, 64, (n, nb, 8))
    d = np.where(g.random((n, nb)) < 0.5, 0.5, 1.0)
    return enc_q4k(q4.reshape(-1, 256), sc.reshape(-1, 8), np.zeros((n * nb, 8), np.int64), d.reshape(-1),
                   np.zeros(n * nb)).reshape(-1)


def up_random(g, n):
    """Random up rows: codes 0..15, scales and mins 0..63, d and dmin in
    {1/2, 1}."""
    nb = DM // 256
    q4 = g.integers(0, 16, (n * nb, 256))
    sc = g.integers(0, 64, (n * nb, 8))
    m = g.integers(0, 64, (n * nb, 8))
    d = np.where(g.random(n * nb) < 0.5, 0.5, 1.0)
    dmin = np.where(g.random(n * nb) < 0.5, 0.5, 1.0)
    return enc_q4k(q4, sc, m, d, dmin).reshape(-1)


def down_small(g, n):
    """Q6_K down rows: q6 - 32 in [-4, 3], scales in {-1, 0, 1}, d in {1/2, 1}."""
    nb = DFF // 256
    q6 = g.integers(28, 36, (n * nb, 256))
    sc = g.integers(-1, 2, (n * nb, 16))
    d = np.where(g.random(n * nb) < 0.5, 0.5, 1.0)
    return enc_q6k(q6, sc, d).reshape(-1)


def run(gate, up, down, xq_np, ids, rw, T, layout):
    S = T * TOPK
    wsb = qmv.grouped_expert_mmvq_workspace(E, T, TOPK, DM, DFF)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out, buf = guarded(T * DM)
    dd = dev(down)
    wdn = planar(dd, E * DM, DFF) if layout == PL else dd
    qmv.grouped_expert_mmvq(dev(gate), dev(up), wdn, layout, dev(xq_np.reshape(-1)), dev(ids), dev(rw), out,
                            E, T, TOPK, DM, DFF, ws, wsb)
    assert canaries_intact(buf, T * DM)
    wsh = host(ws)
    L = qmv.moe_workspace_layout(T, TOPK, DM, DFF)
    h = wsh[L["h"]:L["h"] + 4 * S * DFF].view(np.float32).reshape(S, DFF)
    hq = wsh[L["hq"]:L["hq"] + 36 * S * DFF // 32].reshape(S, -1)
    y = wsh[L["y"]:L["y"] + 4 * S * DM].view(np.float32).reshape(S, DM)
    return host(out).reshape(T, DM), h, hq, y


def routing(g, T):
    ids = np.stack([g.choice(E, size=TOPK, replace=False) for _ in range(T)]).astype(np.int32)
    return ids


@pytest.mark.parametrize("T", [1, 3])
@pytest.mark.parametrize("which", ["gate", "up"])
def test_moe_exact_gate_up_paths(which, T):
    note(f"MoE exact arithmetic, {which} path, T={T}")
    g = synth.rng(1800 + 10 * T + (which == "up"))
    n = E * DFF
    if which == "gate":
        gate = gate_random_positive(g, n)
        up, _ = up_pow2(g, n)
        xq_np = activation(g, T, nonneg=True)
    else:
        gate = gate_const(g, n, np.where(g.random(n) < 0.5, 128, 256))
        up = up_random(g, n)
        xq_np = activation(g, T, nonneg=False)
    down = synth.q6k_blocks(g, E * DM, DFF)
    ids = routing(g, T)
    rw = np.full((T, TOPK), 0.125, np.float32)
    res = orc.grouped_expert(gate, up, down, xq_np, ids, rw, E, T, TOPK, DM, DFF)
    assert np.all(res["g"] >= 128)                      # silu(g) = g exactly
    for layout in (PL, GG):
        _, h, hq, _ = run(gate, up, down, xq_np, ids, rw, T, layout)
        assert np.array_equal(h.view(np.uint32), res["h"].view(np.uint32)), f"h, layout {layout}"
        assert np.array_equal(hq, res["hq"]), f"hq, layout {layout}"


@pytest.mark.parametrize("T", [1, 2, 3])
def test_moe_exact_down_and_routed_sum(T):
    """The down product and the routed sum bit for bit: T = 1 (eight slots)
    takes the fused down + sum launch with planar down weights and the
    three-launch chain with GGUF ones; T = 2, 3 the chain with both."""
    note(f"MoE exact arithmetic, down path, T={T}")
    g = synth.rng(1830 + T)
    n = E * DFF
    gate = gate_const(g, n, np.full(n, 128))
    up, U = up_int(g, n)
    down = down_small(g, E * DM)
    xq_np = activation(g, T, nonneg=False)
    ids = routing(g, T)
    rw = np.where(g.random((T, TOPK)) < 0.5, 0.5, 1.0).astype(np.float32)
    res = orc.grouped_expert(gate, up, down, xq_np, ids, rw, E, T, TOPK, DM, DFF)
    # the construction: h = 128 U, quantized to d = 128 and q = U
    for s in range(T * TOPK):
        e = ids.reshape(-1)[s]
        assert np.array_equal(res["h"][s], 128.0 * U[e * DFF:(e + 1) * DFF])
    hq_d = res["hq"].reshape(-1, DFF // 32, 36)[..., 0:2].copy().view(np.float16)
    assert np.all(hq_d == 128.0)
    for layout in (PL, GG):
        out, h, hq, y = run(gate, up, down, xq_np, ids, rw, T, layout)
        assert np.array_equal(h.view(np.uint32), res["h"].view(np.uint32)), f"h, layout {layout}"
        assert np.array_equal(hq, res["hq"]), f"hq, layout {layout}"
        assert np.array_equal(y.astype(np.float64), res["y"]), f"y, layout {layout}"
        assert np.array_equal(out.astype(np.float64), res["out"]), f"out, layout {layout}"

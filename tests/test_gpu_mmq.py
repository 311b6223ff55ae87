"""GPU parity of the many-column Q6_K product (mmq_q6k, tiled weights),
through the C ABI, against the CPU oracle and against the decode product.

Bars: fp32 outputs within 1e-5 of the oracle relative to the sum of
absolute terms (every row and column, small and full sizes); every
column bit-for-bit equal to the decode product (mmvq_q6k, at most eight
columns) of the same column; column-planar activations bit-for-bit equal to
Q8_1 blocks.  The shapes take every batch width and launch shape (16
columns with 1, 2, 4 and 8 waves along K, 12 columns with 16 waves, one and
two chunks per row; the weights-stationary launch with full and partial
groups of batches) with ragged rests of 1 to 13 columns after the batches.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import (DEV, assert_close, canaries_intact, check_all_rows, dev, guarded, host, mmvq, note,
                            quantize, tiled)

pytestmark = pytest.mark.gpu

TL, XT = qmv.LAYOUT_TILED, qmv.LAYOUT_TILED | qmv.ACT_PLANAR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def mmq(w, xq, rows, K, ncols, layout=TL):
    out, buf = guarded(ncols * rows)
    qmv.mmq_q6k(w, layout, xq, out, rows, K, ncols)
    assert canaries_intact(buf, ncols * rows), "output guard words overwritten"
    return host(out).reshape(ncols, rows)


def quantize_planar(x):
    ncols, K = x.shape
    xp = torch.empty(ncols * (K // 32) * 36, dtype=torch.uint8, device=DEV)
    qmv.quantize_q8_1_planar(dev(np.ascontiguousarray(x, dtype=np.float32)), xp, K, ncols)
    return xp


def decode_columns(w, xq, rows, K, ncols):
    """The decode product, eight columns at a time."""
    nb = K // 32 * 36
    parts = [mmvq("q6k", w, xq[c * nb:(c + min(8, ncols - c)) * nb], rows, K, min(8, ncols - c), TL)
             for c in range(0, ncols, 8)]
    return np.concatenate(parts)


# (rows, K, ncols): K = 512 one wave along K (two batches + 1), 768 two
# waves (1 + 3), 2560 four (2 + 8, 3 + 0), 5120 eight (1 + 0, 1 + 11),
# 10240 sixteen at twelve columns (2 + 5), 20480 two chunks (2 + 1); from
# 128 columns on, K = 2560 and 5120 take the launch that holds the weights
# across eight batches of eight columns per workgroup: 17 batches + 5
# (groups of 8, 8, 1), 18 + 6 (8, 8, 2), 25 + 0 (8, 8, 8, 1); K = 10240
# (sixteen waves) 16 + 2 (8, 8)
SMALL = [(70, 512, 33), (37, 768, 19), (19, 2560, 40), (130, 2560, 48), (40, 5120, 16), (23, 5120, 27),
         (9, 10240, 29), (17, 20480, 25), (19, 2560, 141), (21, 2560, 150), (40, 5120, 200), (9, 10240, 130)]


@pytest.mark.parametrize("rows,K,ncols", SMALL)
def test_mmq_vs_oracle_and_decode(rows, K, ncols):
    note(f"mmq_q6k rows={rows} K={K} ncols={ncols}")
    g = synth.rng(1300 + rows + K + ncols)
    w = synth.q6k_blocks(g, rows, K)
    x = synth.activations(g, ncols, K)
    xq, xq_np = quantize(x)
    wt = tiled(dev(w), rows, K)
    got = mmq(wt, xq, rows, K, ncols)
    ref, ab = orc.mmvq("q6k", w, xq_np, rows, K)
    assert_close(got, ref, ab, f"mmq {rows}x{K} N={ncols}")
    assert np.array_equal(got.view(np.uint32), decode_columns(wt, xq, rows, K, ncols).view(np.uint32))
    gp = mmq(wt, quantize_planar(x), rows, K, ncols, XT)
    assert np.array_equal(gp.view(np.uint32), got.view(np.uint32))


# edge cases: one column (no batch), exactly one batch, a one-row matrix,
# and the most columns the entry point takes (4095 batches + 15 columns)
EDGE = [(300, 2560, 1), (5, 512, 16), (1, 256, 17), (16, 256, 65535)]


@pytest.mark.parametrize("rows,K,ncols", EDGE)
def test_mmq_edge_cases(rows, K, ncols):
    note(f"mmq_q6k edge rows={rows} K={K} ncols={ncols}")
    g = synth.rng(1330 + rows + ncols)
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    wt = tiled(dev(w), rows, K)
    got = mmq(wt, xq, rows, K, ncols)
    ref, ab = orc.mmvq("q6k", w, xq_np, rows, K)
    assert_close(got, ref, ab, f"mmq {rows}x{K} N={ncols}")
    cs = sorted(set(g.choice(ncols, size=min(24, ncols), replace=False).tolist()) | {0, ncols - 1})
    nb = K // 32 * 36
    for c in cs:
        one = mmvq("q6k", wt, xq[c * nb:(c + 1) * nb], rows, K, 1, TL)
        assert np.array_equal(one[0].view(np.uint32), got[c].view(np.uint32)), c


def test_mmq_exact_arithmetic_bitexact():
    """Inputs whose every fp32 product and partial sum is exact: the
    batched product must return the oracle's value exactly."""
    note("exact-arithmetic mmq_q6k")
    g = synth.rng(1310)
    rows, K, ncols = 45, 2560, 37
    w = synth.exact_q6k_blocks(g, rows, K)
    xq_np = synth.exact_q8_1(g, ncols, K)
    ref, _ = orc.mmvq("q6k", w, xq_np, rows, K)
    got = mmq(tiled(dev(w), rows, K), dev(xq_np), rows, K, ncols)
    assert np.array_equal(got.astype(np.float64), ref)


# full sizes: the decode matrices at prompt widths, the LM head, and
# partial last row tiles / row workgroups (32805 x 256, 4100 x 1280)
FULL = [(10240, 2560, 512), (10240, 2560, 70), (2560, 10240, 100), (151936, 2560, 20), (32805, 256, 45),
        (4100, 1280, 17), (3000, 5120, 40), (3000, 5120, 130), (2560, 10240, 136), (8200, 20480, 13)]


@pytest.mark.parametrize("rows,K,ncols", FULL)
def test_mmq_full_size_all_rows(rows, K, ncols):
    note(f"mmq_q6k full size {rows}x{K} N={ncols}")
    g = synth.rng(synth.seed_for(13, rows % 101, ncols))
    w = synth.q6k_blocks(g, rows, K)
    wt = tiled(dev(w), rows, K)
    x = synth.activations(g, ncols, K)
    xq, xq_np = quantize(x)
    got = mmq(wt, xq, rows, K, ncols)
    check_all_rows("q6k", w, xq_np, got, rows, K, f"mmq {rows}x{K} N={ncols} all rows and columns")
    assert np.array_equal(got.view(np.uint32), decode_columns(wt, xq, rows, K, ncols).view(np.uint32))
    gp = mmq(wt, quantize_planar(x), rows, K, ncols, XT)
    assert np.array_equal(gp.view(np.uint32), got.view(np.uint32))


def test_mmq_graph_replay_matches_eager():
    note("graph capture of quantize_q8_1_planar + mmq_q6k")
    rows, K, ncols = 2048, 2560, 137
    g = synth.rng(1320)
    w = tiled(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    x = dev(synth.activations(g, ncols, K))
    xq = torch.empty(ncols * K // 32 * 36, dtype=torch.uint8, device=DEV)
    out = torch.empty(ncols * rows, dtype=torch.float32, device=DEV)
    qmv.quantize_q8_1_planar(x, xq, K, ncols)
    qmv.mmq_q6k(w, XT, xq, out, rows, K, ncols)
    eager = host(out).copy()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qmv.quantize_q8_1_planar(x, xq, K, ncols, stream=s)
            qmv.mmq_q6k(w, XT, xq, out, rows, K, ncols, stream=s)
    for i in range(5):
        out.fill_(float("nan"))
        xq.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), eager.view(np.uint32)), f"replay {i}"
        _ = (x * 2).sum().item()               # eager work between replays

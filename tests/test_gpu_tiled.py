"""GPU parity of the tiled Q6_K layout and its matrix-core kernel, through
the C ABI, against the CPU oracle.

Bars: bit-exact for the conversion (against the oracle's tiled layout and
back to GGUF), the per-sub-block int32 sums and the column-count identities;
fp32 outputs within 1e-5 of the oracle relative to the sum of absolute terms.
The sizes cover every workgroup shape the kernel picks by row length (1, 2,
4, 8 and 16 waves along K), partial last tiles and workgroups, ragged and
multi-chunk rows, each against the oracle on every row at full size.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import (DEV, assert_close, check_all_rows, dev, host, isums, mmvq, note, oracle_all_rows,
                            oracle_isums_all_rows, planar, quantize, tiled)

pytestmark = pytest.mark.gpu

TL, PL, GG = qmv.LAYOUT_TILED, qmv.LAYOUT_PLANAR, qmv.LAYOUT_GGUF


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


# ------------------------------------------------------------ conversion
@pytest.mark.parametrize("rows,K", [(1, 256), (7, 768), (16, 512), (33, 2560), (50, 10240)])
def test_tiled_repack_bytes_and_roundtrip(rows, K):
    note(f"repack_q6k_tiled rows={rows} K={K}")
    w = synth.q6k_blocks(synth.rng(900 + rows), rows, K)
    wd = dev(w)
    t = tiled(wd, rows, K)
    assert np.array_equal(host(t), orc.q6k_to_tiled(w, rows, K))
    back = torch.empty_like(wd)
    qmv.unpack_q6k_tiled(t, back, rows, K)
    assert np.array_equal(host(back), w)


# ------------------------------------------------------- small, all rows
SMALL = [(1, 256, 1), (37, 768, 3), (19, 2560, 8), (9, 10240, 2), (70, 512, 5), (5, 1280, 8),
         (40, 3584, 5), (130, 2560, 4), (17, 20480, 6), (21, 12800, 7)]


@pytest.mark.parametrize("rows,K,ncols", SMALL)
def test_tiled_isums_bitexact(rows, K, ncols):
    note(f"mmvq_q6k_isums tiled rows={rows} K={K} ncols={ncols}")
    g = synth.rng(910 + rows + K + ncols)
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    got = isums("q6k", tiled(dev(w), rows, K), xq, rows, K, ncols, TL)
    assert np.array_equal(got, orc.q6k_isums(w, xq_np, rows, K))


@pytest.mark.parametrize("rows,K,ncols", SMALL)
def test_tiled_outputs_vs_oracle(rows, K, ncols):
    note(f"mmvq_q6k tiled rows={rows} K={K} ncols={ncols}")
    g = synth.rng(920 + rows + K + ncols)
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    ref, ab = orc.mmvq("q6k", w, xq_np, rows, K)
    got = mmvq("q6k", tiled(dev(w), rows, K), xq, rows, K, ncols, TL)
    assert_close(got, ref, ab, f"tiled {rows}x{K} N={ncols}")


def test_tiled_exact_arithmetic_configuration_bitexact():
    """Weights and activations whose every fp32 product and partial sum is
    exact: the tiled kernel must then return the oracle's value exactly."""
    note("exact-arithmetic q6k tiled")
    g = synth.rng(500)
    rows, K, ncols = 45, 2560, 8
    w = synth.exact_q6k_blocks(g, rows, K)
    xq_np = synth.exact_q8_1(g, ncols, K)
    ref, _ = orc.mmvq("q6k", w, xq_np, rows, K)
    got = mmvq("q6k", tiled(dev(w), rows, K), dev(xq_np), rows, K, ncols, TL)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("rows,K", [(64, 768), (64, 2560), (64, 10240), (8200, 2560)])
def test_tiled_column_count_invariance(rows, K):
    """Column c of an N-column call has the bits of a 1-column call on c."""
    note(f"column invariance tiled {rows}x{K}")
    g = synth.rng(930 + K)
    w = tiled(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    xq, _ = quantize(synth.activations(g, 8, K))
    full = mmvq("q6k", w, xq, rows, K, 8, TL)
    for n in (2, 3, 5, 7):
        part = mmvq("q6k", w, xq, rows, K, n, TL)
        assert np.array_equal(part.view(np.uint32), full[:n].view(np.uint32)), n
    nb = K // 32 * 36
    for c in (0, 3, 4, 7):
        one = mmvq("q6k", w, xq[c * nb:(c + 1) * nb], rows, K, 1, TL)
        assert np.array_equal(one[0].view(np.uint32), full[c].view(np.uint32)), c


# ------------------------------------------ full sizes, every launch shape
# The kernel takes ceil(K/640) waves along K (rounded up to 1, 2, 4, 8, 16):
# K = 256, 512 -> one wave, four tiles per workgroup (32805 rows: a partial
# tile and a workgroup with an empty tile slot); K = 768, 1280 -> two waves,
# two tiles (4100 x 1280: a ragged chunk); K = 2560 -> four waves (10240 x
# 2560, the LM head, 2560 x 2560); K = 5120 -> eight; K = 10240 -> sixteen
# (2560 x 10240); K = 20480 -> sixteen with two chunks per row (8200 rows: a
# half tile).
FULL = [(32805, 256, (8, 1)), (16405, 512, (5, 2)), (4100, 1280, (3, 8)), (10240, 2560, (8, 6, 4, 2, 1)),
        (151936, 2560, (4, 1)), (2560, 2560, (1, 7)), (3000, 5120, (8, 2)), (2560, 10240, (8, 4, 1)),
        (8200, 20480, (8, 3))]


@pytest.mark.parametrize("rows,K,cols", FULL)
def test_tiled_full_size_all_rows(rows, K, cols):
    note(f"tiled full size {rows}x{K} N={cols}")
    g = synth.rng(synth.seed_for(4, rows % 101, 8))
    w = synth.q6k_blocks(g, rows, K)
    wt = tiled(dev(w), rows, K)
    xq, xq_np = quantize(synth.activations(g, 8, K))
    ref, ab = oracle_all_rows("q6k", w, xq_np[:max(cols)].reshape(-1), rows, K)
    nb = K // 32 * 36
    first = None
    for n in cols:
        got = mmvq("q6k", wt, xq[:n * nb], rows, K, n, TL)
        assert_close(got, ref[:n], ab[:n], f"tiled {rows}x{K} N={n} all rows")
        if first is None:
            first = got
        else:
            m = min(n, first.shape[0])
            assert np.array_equal(got[:m].view(np.uint32), first[:m].view(np.uint32))


@pytest.mark.parametrize("rows,K,ncols", [(10240, 2560, 8), (2560, 10240, 4), (32805, 256, 3)])
def test_tiled_isums_full_size_all_rows(rows, K, ncols):
    note(f"tiled isums full size {rows}x{K} N={ncols}")
    g = synth.rng(synth.seed_for(5, rows % 101, ncols))
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    got = isums("q6k", tiled(dev(w), rows, K), xq, rows, K, ncols, TL)
    assert np.array_equal(got, oracle_isums_all_rows("q6k", w, xq_np, rows, K))


def test_tiled_agrees_with_planar():
    """Same matrix in both planar layouts: outputs within fp32 rounding of
    each other (different summation orders), integer sums identical."""
    rows, K, ncols = 3000, 2560, 8
    note(f"tiled vs planar {rows}x{K} N={ncols}")
    g = synth.rng(940)
    w = synth.q6k_blocks(g, rows, K)
    wd = dev(w)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    pt, pp = tiled(wd, rows, K), planar(wd, rows, K)
    assert np.array_equal(isums("q6k", pt, xq, rows, K, ncols, TL), isums("q6k", pp, xq, rows, K, ncols, PL))
    a, b = mmvq("q6k", pt, xq, rows, K, ncols, TL), mmvq("q6k", pp, xq, rows, K, ncols, PL)
    check_all_rows("q6k", w, xq_np, a, rows, K, "tiled")
    assert np.all(np.abs(a.astype(np.float64) - b) <= 3e-5 * np.abs(b).max(axis=-1, keepdims=True))


@pytest.mark.parametrize("act_planar", [False, True])
def test_tiled_graph_replay_matches_eager(act_planar):
    note(f"graph capture of quantize + tiled mmvq_q6k (column-planar activations: {act_planar})")
    rows, K, ncols = 2048, 2560, 4
    g = synth.rng(950)
    w = tiled(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    x = dev(synth.activations(g, ncols, K))
    xq = torch.empty(ncols * K // 32 * 36, dtype=torch.uint8, device=DEV)
    out = torch.empty(ncols * rows, dtype=torch.float32, device=DEV)
    quant = qmv.quantize_q8_1_planar if act_planar else qmv.quantize_q8_1
    lay = TL | qmv.ACT_PLANAR if act_planar else TL
    quant(x, xq, K, ncols)
    qmv.mmvq_q6k(w, lay, xq, out, rows, K, ncols)
    eager = host(out).copy()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            quant(x, xq, K, ncols, stream=s)
            qmv.mmvq_q6k(w, lay, xq, out, rows, K, ncols, stream=s)
    for i in range(5):
        out.fill_(float("nan"))
        xq.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), eager.view(np.uint32)), f"replay {i}"
        _ = (x * 2).sum().item()               # eager work between replays


# ------------------------------------------------------------- row gather
@pytest.mark.parametrize("layout", [GG, PL, TL])
def test_gather_rows_bytes_and_products(layout):
    """A draft-head-like row subset (repeats, an out-of-range id, a partial
    last tile) gathered on the GPU in each layout: bytes equal the oracle's,
    and the product on the gathered matrix matches the oracle on the
    gathered GGUF rows."""
    rows, K, ncols = 5000, 2560, 4
    note(f"gather_q6k_rows layout={layout} {rows}x{K}")
    g = synth.rng(960 + layout)
    w = synth.q6k_blocks(g, rows, K)
    ids = g.choice(rows, size=1000, replace=True).astype(np.int32)
    ids[[7, 500]] = [-3, rows]
    wd = dev(w)
    src = wd if layout == GG else (planar(wd, rows, K) if layout == PL else tiled(wd, rows, K))
    nout = ids.size
    dst = torch.empty(nout * (K // 256) * 210, dtype=torch.uint8, device=DEV)
    qmv.gather_q6k_rows(src, layout, rows, K, dev(ids), nout, dst)
    assert np.array_equal(host(dst), orc.q6k_gather(w, layout, rows, K, ids))
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    got = mmvq("q6k", dst, xq, nout, K, ncols, layout)
    wg = orc.q6k_gather(w, GG, rows, K, ids)
    ref, ab = orc.mmvq("q6k", wg, xq_np, nout, K)
    ok = (ids >= 0) & (ids < rows)
    assert_close(got[:, ok], ref[:, ok], ab[:, ok], f"gathered layout={layout}")
    assert not np.any(got[:, ~ok])       # all-zero rows (d = 0) give exact zeros


# ---------------------------------------------------------- greedy argmax
@pytest.mark.parametrize("rows,K,ncols", [(151936, 2560, 4), (151936, 2560, 1), (10240, 2560, 8),
                                          (5003, 768, 5), (32805, 256, 3), (2560, 10240, 2), (7, 512, 2)])
def test_argmax_matches_own_outputs_and_oracle(rows, K, ncols):
    """idx/val equal numpy's first-occurrence argmax of the same kernel's fp32
    outputs (bits of the value included); the chosen row is a maximum of the
    oracle's outputs within the fp32 tolerance; a copy of the winning row
    planted at a lower index then wins the tie."""
    note(f"mmvq_q6k_argmax {rows}x{K} N={ncols}")
    g = synth.rng(synth.seed_for(6, rows % 101, ncols))
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    wb = w.reshape(rows, -1)

    def run(wmat):
        wt = tiled(dev(wmat.reshape(-1)), rows, K)
        out = mmvq("q6k", wt, xq, rows, K, ncols, TL)
        nws = qmv.mmvq_q6k_argmax_workspace(rows, ncols)
        ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
        idx = torch.empty(ncols, dtype=torch.int32, device=DEV)
        val = torch.empty(ncols, dtype=torch.float32, device=DEV)
        qmv.mmvq_q6k_argmax(wt, TL, xq, rows, K, ncols, idx, val, ws, nws)
        return out, host(idx), host(val)

    out, idx, val = run(wb)
    assert np.array_equal(idx, np.argmax(out, axis=1))
    assert np.array_equal(val.view(np.uint32), out[np.arange(ncols), idx].view(np.uint32))
    # against the oracle on every row: the outputs within tolerance, and the
    # chosen row's exact value within tolerance of the exact maximum
    ref, ab = oracle_all_rows("q6k", w, xq_np, rows, K)
    assert_close(out, ref, ab, f"argmax product {rows}x{K} N={ncols}")
    best = ref.max(axis=1)
    chosen = ref[np.arange(ncols), idx]
    assert np.all(chosen >= best - 2e-5 * ab.max(axis=1))
    if rows > 1 and idx[0] > 0:
        w2 = wb.copy()
        lo = int(idx[0]) // 2
        w2[lo] = wb[idx[0]]
        out2, idx2, val2 = run(w2)
        assert idx2[0] == lo and np.array_equal(val2[:1].view(np.uint32), val[:1].view(np.uint32))
        assert np.array_equal(idx2, np.argmax(out2, axis=1))


# --------------------------------------------- column-planar activations
XT = TL | qmv.ACT_PLANAR


def quantize_planar(x: np.ndarray) -> torch.Tensor:
    x = np.ascontiguousarray(x, dtype=np.float32)
    ncols, K = x.shape
    xp = torch.empty(ncols * (K // 32) * 36, dtype=torch.uint8, device=DEV)
    qmv.quantize_q8_1_planar(dev(x), xp, K, ncols)
    return xp


@pytest.mark.parametrize("K,ncols", [(32, 1), (256, 3), (2560, 13), (10240, 8), (992, 5)])
def test_planar_quantizer_bytes(K, ncols):
    """quantize_q8_1_planar writes the oracle's Q8_1 blocks, rearranged by the
    oracle's column-planar permutation, byte for byte."""
    note(f"quantize_q8_1_planar K={K} ncols={ncols}")
    x = synth.activations(synth.rng(960 + K + ncols), ncols, K)
    want = orc.q8_1_to_planar(orc.quantize_q8_1(x), K)
    assert np.array_equal(host(quantize_planar(x)), want)


@pytest.mark.parametrize("rows,K,ncols", SMALL + [(300, 1280, 8), (2100, 2560, 5)])
def test_planar_activations_match_blocks_bitexact(rows, K, ncols):
    """The tiled product and its integer sums from column-planar activations
    have the bits of those from the same values in Q8_1 blocks, and the
    isums equal the oracle's."""
    note(f"mmvq_q6k tiled|act_planar rows={rows} K={K} ncols={ncols}")
    g = synth.rng(970 + rows + K + ncols)
    w = synth.q6k_blocks(g, rows, K)
    x = synth.activations(g, ncols, K)
    xq, xq_np = quantize(x)
    xp = quantize_planar(x)
    wt = tiled(dev(w), rows, K)
    a = mmvq("q6k", wt, xq, rows, K, ncols, TL)
    b = mmvq("q6k", wt, xp, rows, K, ncols, XT)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    ib = isums("q6k", wt, xp, rows, K, ncols, XT)
    assert np.array_equal(ib, orc.q6k_isums(w, xq_np, rows, K))


@pytest.mark.parametrize("rows,K,cols", [(10240, 2560, (8, 4, 1)), (2560, 10240, (8, 3)), (16405, 512, (6,)),
                                         (8200, 20480, (2,))])
def test_planar_activations_full_size(rows, K, cols):
    """Full sizes (every launch shape): bits equal to the Q8_1-block path,
    every row within the oracle tolerance."""
    g = synth.rng(980 + rows)
    w = synth.q6k_blocks(g, rows, K)
    wt = tiled(dev(w), rows, K)
    x = synth.activations(g, 8, K)
    xq, xq_np = quantize(x)
    xp = quantize_planar(x)
    for n in cols:
        note(f"mmvq_q6k tiled|act_planar full {rows}x{K} N={n}")
        a = mmvq("q6k", wt, xq, rows, K, n, TL)
        b = mmvq("q6k", wt, xp, rows, K, n, XT)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
        check_all_rows("q6k", w, xq_np[:n].reshape(-1), b, rows, K, f"act_planar {rows}x{K} N={n}")


@pytest.mark.parametrize("rows,K,ncols", [(151936, 2560, 4), (1000, 2560, 1), (37, 768, 8)])
def test_planar_activations_argmax(rows, K, ncols):
    """The fused argmax from column-planar activations gives the same index
    and value bits as from Q8_1 blocks."""
    note(f"mmvq_q6k_argmax tiled|act_planar {rows}x{K} N={ncols}")
    g = synth.rng(990 + rows)
    wt = tiled(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    x = synth.activations(g, ncols, K)
    xq, _ = quantize(x)
    xp = quantize_planar(x)
    nws = qmv.mmvq_q6k_argmax_workspace(rows, ncols)
    res = []
    for lay, a in ((TL, xq), (XT, xp)):
        ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
        idx = torch.empty(ncols, dtype=torch.int32, device=DEV)
        val = torch.empty(ncols, dtype=torch.float32, device=DEV)
        qmv.mmvq_q6k_argmax(wt, lay, a, rows, K, ncols, idx, val, ws, nws)
        res.append((host(idx), host(val).view(np.uint32)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


def test_argmax_graph_replay_poisoned_workspace():
    """The fused argmax captured in a HIP graph: with the workspace poisoned
    before every replay (the per-column reduction state included) each
    replay gives the eager index and value bits."""
    note("mmvq_q6k_argmax graph replay")
    rows, K, ncols = 40000, 2560, 4
    g = synth.rng(1500)
    wt = tiled(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    xq, _ = quantize(synth.activations(g, ncols, K))
    nws = qmv.mmvq_q6k_argmax_workspace(rows, ncols)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    idx = torch.empty(ncols, dtype=torch.int32, device=DEV)
    val = torch.empty(ncols, dtype=torch.float32, device=DEV)
    qmv.mmvq_q6k_argmax(wt, TL, xq, rows, K, ncols, idx, val, ws, nws)
    e_idx, e_val = host(idx).copy(), host(val).view(np.uint32).copy()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qmv.mmvq_q6k_argmax(wt, TL, xq, rows, K, ncols, idx, val, ws, nws, stream=s)
    for i in range(4):
        ws.fill_(0xFF)
        idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), e_idx) and np.array_equal(host(val).view(np.uint32), e_val), f"replay {i}"

"""GPU parity of mmvq_q6k_topk (the k largest outputs per column), through
the C ABI: indices and value bits equal to the stable descending order of the
same kernel's fp32 outputs (lower row first among equal values); the chosen
values within the oracle tolerance of the oracle's exact top-k values (the
i-th largest of two sets of numbers that differ elementwise by at most e
differ by at most e); a planted copy of the best row at a lower index comes
first; every layout; chunk edges (rows = 4096 + 1), k = rows, k = 64 over the
LM head; graph replay with the workspace poisoned."""
import numpy as np
import pytest
import torch

from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import DEV, dev, host, mmvq, note, oracle_all_rows, planar, quantize, tiled

pytestmark = pytest.mark.gpu

GG, PL, TL = qmv.LAYOUT_GGUF, qmv.LAYOUT_PLANAR, qmv.LAYOUT_TILED
XT = TL | qmv.ACT_PLANAR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def quantize_planar(x):
    ncols, K = x.shape
    xp = torch.empty(ncols * (K // 32) * 36, dtype=torch.uint8, device=DEV)
    qmv.quantize_q8_1_planar(dev(np.ascontiguousarray(x, dtype=np.float32)), xp, K, ncols)
    return xp


def layout_weights(wd, rows, K, lay):
    base = lay & ~qmv.ACT_PLANAR
    if base == PL:
        return planar(wd, rows, K)
    if base == TL:
        return tiled(wd, rows, K)
    return wd


def topk(w, lay, xq, rows, K, n, k):
    nws = qmv.mmvq_q6k_topk_workspace(rows, n, k)
    ws = torch.full((nws,), 0x5A, dtype=torch.uint8, device=DEV)
    idx = torch.empty(n * k, dtype=torch.int32, device=DEV)
    val = torch.empty(n * k, dtype=torch.float32, device=DEV)
    qmv.mmvq_q6k_topk(w, lay, xq, rows, K, n, k, idx, val, ws, nws)
    return host(idx).reshape(n, k), host(val).reshape(n, k)


CASES = [(151936, 2560, 4, 16, XT), (151936, 2560, 1, 64, TL), (5003, 768, 5, 7, PL), (700, 2560, 3, 10, GG),
         (20, 512, 2, 20, TL), (4097, 256, 8, 64, TL), (40000, 10240, 2, 33, XT)]


@pytest.mark.parametrize("rows,K,ncols,k,lay", CASES)
def test_topk_matches_own_outputs_and_oracle(rows, K, ncols, k, lay):
    note(f"mmvq_q6k_topk {rows}x{K} N={ncols} k={k} layout={lay}")
    g = synth.rng(2100 + rows % 997 + k)
    w = synth.q6k_blocks(g, rows, K)
    x = synth.activations(g, ncols, K)
    xq, xq_np = quantize(x)
    act = quantize_planar(x) if lay & qmv.ACT_PLANAR else xq
    wl = layout_weights(dev(w), rows, K, lay)
    out = mmvq("q6k", wl, act, rows, K, ncols, lay)
    idx, val = topk(wl, lay, act, rows, K, ncols, k)
    order = np.argsort(-out, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, order)
    assert np.array_equal(val.view(np.uint32), np.take_along_axis(out, order, axis=1).view(np.uint32))
    ref, ab = oracle_all_rows("q6k", w, xq_np, rows, K)
    best = -np.sort(-ref, axis=1)[:, :k]
    tol = 1e-5 * ab.max(axis=1, keepdims=True)
    assert np.all(np.abs(val.astype(np.float64) - best) <= tol)


def test_topk_ties_lower_row_first():
    rows, K, n, k = 3000, 2560, 2, 12
    note("mmvq_q6k_topk planted tie")
    g = synth.rng(2150)
    w = synth.q6k_blocks(g, rows, K).reshape(rows, -1)
    xq, _ = quantize(synth.activations(g, n, K))
    wt = tiled(dev(w.reshape(-1)), rows, K)
    idx, _ = topk(wt, TL, xq, rows, K, n, k)
    top = int(idx[0, 0])
    lo = top // 3
    w2 = w.copy()
    w2[lo] = w[top]
    idx2, val2 = topk(tiled(dev(w2.reshape(-1)), rows, K), TL, xq, rows, K, n, k)
    first = [int(i) for i in idx2[0, :2]]
    assert first == [lo, top] and val2[0, 0] == val2[0, 1]


def test_topk_graph_replay_poisoned_workspace():
    rows, K, n, k = 20000, 2560, 4, 20
    note("mmvq_q6k_topk graph replay")
    g = synth.rng(2160)
    wt = tiled(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    xq, _ = quantize(synth.activations(g, n, K))
    nws = qmv.mmvq_q6k_topk_workspace(rows, n, k)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    idx = torch.empty(n * k, dtype=torch.int32, device=DEV)
    val = torch.empty(n * k, dtype=torch.float32, device=DEV)
    qmv.mmvq_q6k_topk(wt, TL, xq, rows, K, n, k, idx, val, ws, nws)
    e_idx, e_val = host(idx).copy(), host(val).copy()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qmv.mmvq_q6k_topk(wt, TL, xq, rows, K, n, k, idx, val, ws, nws, stream=s)
    for i in range(4):
        ws.fill_(0xC3)
        idx.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(idx), e_idx) and np.array_equal(host(val).view(np.uint32), e_val.view(np.uint32))
        _ = (val * 2).sum().item()

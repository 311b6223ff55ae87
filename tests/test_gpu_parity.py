"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bars: bit-exact for the Q8_1 quantizer, the per-sub-block int32 sums, the
planar conversion and every layout/column-count identity; fp32 outputs within
1e-5 of the oracle relative to the sum of absolute terms (tests/gpu_util.py).
Sizes: small ragged cases the oracle checks element by element, and the
workloads' full sizes checked on every row (the oracle spread over host threads).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import (DEV, assert_close, check_all_rows, dev, guarded, canaries_intact, host, isums, mmvq,
                            note, planar, quantize)

pytestmark = pytest.mark.gpu

GG, PL = qmv.LAYOUT_GGUF, qmv.LAYOUT_PLANAR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


# ------------------------------------------------------------ quantizer
@pytest.mark.parametrize("K,ncols", [(2560, 1), (2560, 8), (10240, 4), (768, 3), (96, 5)])
def test_quantize_q8_1_bitexact(K, ncols):
    note(f"quantize_q8_1 K={K} ncols={ncols}")
    g = synth.rng(100 + K + ncols)
    x = synth.activations(g, ncols, K) * np.float32(g.uniform(0.01, 50))
    x[0, :32] = 0.0
    x[-1, 32:64] = np.float32(3e-8)            # d falls in the fp16 subnormal range
    _, got = quantize(x)
    assert np.array_equal(got, orc.quantize_q8_1(x))


@pytest.mark.parametrize("planar_out", [False, True])
def test_quantize_q8_1_ties(planar_out):
    """Blocks whose quotients x/d sit at or next to half-integers, and blocks
    whose fp32 product d * sum is an fp16 midpoint (the sum field must round
    the fp32 product, not the exact one): bytes equal to the oracle's."""
    from tests.q8_fixtures import near_tie_blocks, s_tie_blocks
    for x in (near_tie_blocks(), s_tie_blocks()):
        K = x.shape[1]
        note(f"quantize_q8_1 ties K={K} planar={planar_out}")
        ref = orc.quantize_q8_1(x)
        xd = dev(x)
        xq = torch.empty(K // 32 * 36, dtype=torch.uint8, device=DEV)
        if planar_out:
            qmv.quantize_q8_1_planar(xd, xq, K, 1)
            ref = orc.q8_1_to_planar(ref, K)
        else:
            qmv.quantize_q8_1(xd, xq, K, 1)
        assert np.array_equal(host(xq).reshape(ref.shape), ref)


def test_quantize_q8_1_ties_golden():
    import json, os
    gd = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "q8_1_handworked.json")))
    x = np.array([b["x"] for b in gd["blocks"]], np.float32).reshape(1, -1)
    _, got = quantize(x)
    assert np.array_equal(got, orc.quantize_q8_1(x))


# ---------------------------------------------------------- integer sums
SMALL = [(1, 256, 1), (37, 768, 3), (19, 2560, 8), (9, 10240, 2), (70, 512, 5), (5, 1280, 8)]


@pytest.mark.parametrize("rows,K,ncols", SMALL + [(40, 3584, 5)])
@pytest.mark.parametrize("layout", [PL, GG])
def test_q6k_isums_bitexact(rows, K, ncols, layout):
    note(f"mmvq_q6k_isums rows={rows} K={K} ncols={ncols} layout={layout}")
    g = synth.rng(200 + rows + K + ncols)
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    wd = dev(w)
    if layout == PL:
        wd = planar(wd, rows, K)
    assert np.array_equal(isums("q6k", wd, xq, rows, K, ncols, layout), orc.q6k_isums(w, xq_np, rows, K))


@pytest.mark.parametrize("rows,K,ncols", SMALL + [(33, 6144, 4), (24, 7168, 8), (33, 6144, 8)])
@pytest.mark.parametrize("kind", ["q4k", "q5k"])
def test_q45_isums_bitexact(rows, K, ncols, kind):
    note(f"mmvq_{kind}_isums rows={rows} K={K} ncols={ncols}")
    g = synth.rng(300 + rows + K + ncols)
    w = synth.blocks(kind, g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    assert np.array_equal(isums(kind, dev(w), xq, rows, K, ncols), orc.q45_dots(kind, w, xq_np, rows, K))


# --------------------------------------------------------------- outputs
# (40, 3584): a full register chunk then a ragged one in every row (Q6_K: 16
# lanes x 7 units, depth 5); (24, 7168, 8): the same for Q4_K/Q5_K; (33,
# 6144, 8): Q4_K/Q5_K with the activation tile in two LDS sub-tiles.
@pytest.mark.parametrize("rows,K,ncols", SMALL + [(130, 2560, 4), (40, 3584, 5), (24, 7168, 8), (33, 6144, 8)])
@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
def test_mmvq_outputs_vs_oracle(rows, K, ncols, kind):
    note(f"mmvq_{kind} rows={rows} K={K} ncols={ncols}")
    g = synth.rng(400 + rows + K + ncols)
    w = synth.blocks(kind, g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    ref, ab = orc.mmvq(kind, w, xq_np, rows, K)
    wd = dev(w)
    got = mmvq(kind, wd, xq, rows, K, ncols)
    assert_close(got, ref, ab, f"{kind} {rows}x{K} N={ncols}")
    if kind == "q6k":
        got_p = mmvq(kind, planar(wd, rows, K), xq, rows, K, ncols, PL)
        assert np.array_equal(got_p.view(np.uint32), got.view(np.uint32)), "planar != GGUF bits"


@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
def test_exact_arithmetic_configuration_bitexact(kind):
    note(f"exact-arithmetic {kind}")
    g = synth.rng(500)
    rows, K, ncols = 45, 2560, 8
    w = (synth.exact_q6k_blocks(g, rows, K) if kind == "q6k"
         else synth.exact_q45_blocks(g, rows, K, kind == "q5k"))
    xq_np = synth.exact_q8_1(g, ncols, K)
    ref, _ = orc.mmvq(kind, w, xq_np, rows, K)
    got = mmvq(kind, dev(w), dev(xq_np), rows, K, ncols)
    assert np.array_equal(got.astype(np.float64), ref)


@pytest.mark.parametrize("K", [768, 2560, 10240])
@pytest.mark.parametrize("kind,layout", [("q6k", PL), ("q6k", GG), ("q4k", GG), ("q5k", GG)])
def test_column_count_invariance(K, kind, layout):
    """Column c of an N-column call has the bits of a 1-column call on c."""
    note(f"column invariance {kind} layout={layout} K={K}")
    g = synth.rng(600 + K)
    rows = 64
    w = synth.blocks(kind, g, rows, K)
    x = synth.activations(g, 8, K)
    xq, _ = quantize(x)
    wd = dev(w)
    if layout == PL:
        wd = planar(wd, rows, K)
    full = mmvq(kind, wd, xq, rows, K, 8, layout)
    for n in (2, 5):
        part = mmvq(kind, wd, xq, rows, K, n, layout)
        assert np.array_equal(part.view(np.uint32), full[:n].view(np.uint32))
    nb = K // 32 * 36
    for c in (0, 3, 7):
        one = mmvq(kind, wd, xq[c * nb:(c + 1) * nb], rows, K, 1, layout)
        assert np.array_equal(one[0].view(np.uint32), full[c].view(np.uint32))


@pytest.mark.parametrize("ncols", range(1, 9))
@pytest.mark.parametrize("kind", ["q6k", "q4k", "q5k"])
def test_every_column_count(kind, ncols):
    """Each of the eight column-count instantiations against the oracle."""
    note(f"mmvq_{kind} every column count: N={ncols}")
    rows, K = 96, 2560
    g = synth.rng(700 + ncols)
    w = synth.blocks(kind, g, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    ref, ab = orc.mmvq(kind, w, xq_np, rows, K)
    wd = dev(w)
    if kind == "q6k":
        got = mmvq(kind, planar(wd, rows, K), xq, rows, K, ncols, PL)
        got_g = mmvq(kind, wd, xq, rows, K, ncols, GG)
        assert np.array_equal(got_g.view(np.uint32), got.view(np.uint32)), "planar != GGUF bits"
    else:
        got = mmvq(kind, wd, xq, rows, K, ncols)
    assert_close(got, ref, ab, f"{kind} {rows}x{K} N={ncols}")


def test_ten_wave_launch_two_chunks():
    """Long rows in one-workgroup-per-CU launches: 64 lanes per row, two full
    register chunks and several LDS sub-tiles per row (K = 20480)."""
    note("Q6_K 2240x20480 N=8 (ten-wave workgroups, two chunks, LDS sub-tiles), all rows")
    rows, K = 2240, 20480
    g = synth.rng(720)
    w = synth.q6k_blocks(g, rows, K)
    xq, xq_np = quantize(synth.activations(g, 8, K))
    wd = dev(w)
    got = mmvq("q6k", planar(wd, rows, K), xq, rows, K, 8, PL)
    check_all_rows("q6k", w, xq_np, got, rows, K)
    got_g = mmvq("q6k", wd, xq, rows, K, 8, GG)
    assert np.array_equal(got_g.view(np.uint32), got.view(np.uint32)), "planar != GGUF bits"


# ------------------------------------------------------ planar conversion
@pytest.mark.parametrize("rows,K", [(1, 256), (7, 768), (33, 2560)])
def test_repack_bytes_and_roundtrip(rows, K):
    note(f"repack_q6k_planar rows={rows} K={K}")
    w = synth.q6k_blocks(synth.rng(700 + rows), rows, K)
    wd = dev(w)
    p = planar(wd, rows, K)
    assert np.array_equal(host(p), orc.q6k_to_planar(w, rows, K))
    back = torch.empty_like(wd)
    qmv.unpack_q6k_planar(p, back, rows, K)
    assert np.array_equal(host(back), w)


# ----------------------------------------------- full sizes, every row
@pytest.mark.parametrize("rows,K", [(10240, 2560), (2560, 10240), (2560, 2560)])
def test_q6k_full_size_all_rows(rows, K):
    note(f"full-size Q6_K {rows}x{K}")
    g = synth.rng(synth.seed_for(1, 0 if rows == 2560 and K == 10240 else 1, 8))
    w = synth.q6k_blocks(g, rows, K)
    wd = dev(w)
    pd = planar(wd, rows, K)
    x = synth.activations(g, 8, K)
    xq, xq_np = quantize(x)
    nb = K // 32 * 36
    full = None
    for n in (8, 6, 4, 2, 1):
        got = mmvq("q6k", pd, xq[:n * nb], rows, K, n, PL)
        if full is None:
            full = got
            check_all_rows("q6k", w, xq_np, got, rows, K)
            got_g = mmvq("q6k", wd, xq, rows, K, 8, GG)
            assert np.array_equal(got_g.view(np.uint32), got.view(np.uint32))
        else:
            assert np.array_equal(got.view(np.uint32), full[:n].view(np.uint32))


@pytest.mark.parametrize("ncols", [1, 4])
def test_lm_head_planar_equals_interleaved(ncols):
    rows, K = 151936, 2560
    note(f"LM head {rows}x{K} ncols={ncols}")
    g = synth.rng(synth.seed_for(2, 0, ncols))
    w = synth.q6k_blocks(g, rows, K)
    wd = dev(w)
    pd = planar(wd, rows, K)
    xq, xq_np = quantize(synth.activations(g, ncols, K))
    got_p = mmvq("q6k", pd, xq, rows, K, ncols, PL)
    got_g = mmvq("q6k", wd, xq, rows, K, ncols, GG)
    assert np.array_equal(got_p.view(np.uint32), got_g.view(np.uint32))
    check_all_rows("q6k", w, xq_np, got_p, rows, K)


@pytest.mark.parametrize("rows,K", [(12288, 2560), (6144, 2560), (2560, 6144), (512, 2560)])
@pytest.mark.parametrize("kind", ["q4k", "q5k"])
def test_q45_full_size_all_rows(rows, K, kind):
    note(f"full-size {kind} {rows}x{K}")
    g = synth.rng(synth.seed_for(3, rows % 97, 4))
    w = synth.blocks(kind, g, rows, K)
    wd = dev(w)
    xq, xq_np = quantize(synth.activations(g, 4, K))
    got4 = mmvq(kind, wd, xq, rows, K, 4)
    check_all_rows(kind, w, xq_np, got4, rows, K)
    got1 = mmvq(kind, wd, xq, rows, K, 1)
    assert np.array_equal(got1[0].view(np.uint32), got4[0].view(np.uint32))


# ------------------------------------------------------------ graph replay
def test_graph_replay_matches_eager():
    note("graph capture of quantize + mmvq_q6k")
    rows, K, ncols = 2048, 2560, 4
    g = synth.rng(800)
    w = planar(dev(synth.q6k_blocks(g, rows, K)), rows, K)
    x = dev(synth.activations(g, ncols, K))
    xq = torch.empty(ncols * K // 32 * 36, dtype=torch.uint8, device=DEV)
    out = torch.empty(ncols * rows, dtype=torch.float32, device=DEV)
    qmv.quantize_q8_1(x, xq, K, ncols)
    qmv.mmvq_q6k(w, PL, xq, out, rows, K, ncols)
    eager = host(out).copy()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qmv.quantize_q8_1(x, xq, K, ncols, stream=s)
            qmv.mmvq_q6k(w, PL, xq, out, rows, K, ncols, stream=s)
    for i in range(5):
        out.fill_(float("nan"))
        xq.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), eager.view(np.uint32)), f"replay {i}"
        _ = (x * 2).sum().item()               # eager work between replays


# ------------------------------------------------------------------- MoE
E, DM, DFF, TOPK = 128, 2560, 768, 8


@pytest.fixture(scope="module")
def moe():
    note("MoE weights (E=128, d_model=2560, d_ff=768)")
    g = synth.rng(synth.seed_for(4, 0, 0))
    gate, up, down = synth.moe_weights(g, E, DM, DFF)
    return dict(gate=gate, up=up, down=down, gd=dev(gate), ud=dev(up), dd=dev(down),
                dp=planar(dev(down), E * DM, DFF))


def run_moe(m, xq, ids, rw, T, layout=PL, wg=None, wu=None, wdn=None):
    ws_bytes = qmv.grouped_expert_mmvq_workspace(E, T, TOPK, DM, DFF)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    out, buf = guarded(T * DM)
    wdn = wdn if wdn is not None else (m["dp"] if layout == PL else m["dd"])
    qmv.grouped_expert_mmvq(wg if wg is not None else m["gd"], wu if wu is not None else m["ud"], wdn,
                            layout, xq, dev(ids), dev(rw), out, E, T, TOPK, DM, DFF, ws, ws_bytes)
    assert canaries_intact(buf, T * DM)
    return host(out).reshape(T, DM), host(ws)


@pytest.mark.parametrize("T", range(1, 9))
def test_moe_staged_parity(moe, T):
    note(f"grouped_expert_mmvq T={T}")
    g = synth.rng(synth.seed_for(4, 1, T))
    ids, rw = synth.routing(g, T, E, TOPK)
    xq, xq_np = quantize(synth.activations(g, T, DM))
    out, ws = run_moe(moe, xq, ids, rw, T)
    L = qmv.moe_workspace_layout(T, TOPK, DM, DFF)
    S = T * TOPK
    wsi = ws[:L["h"]].view(np.int32)
    # routing tables (index work: exact)
    hit = sorted(set(ids.reshape(-1).tolist()))
    assert wsi[0] == len(hit) and wsi[1] == 0
    exp_list = [s for e in hit for s in range(S) if ids.reshape(-1)[s] == e]
    assert list(wsi[64:64 + len(hit)]) == hit
    assert list(wsi[64 + 3 * S:64 + 4 * S]) == exp_list
    cnts = [int((ids.reshape(-1) == e).sum()) for e in hit]
    assert list(wsi[64 + S:64 + S + len(hit)]) == cnts
    assert list(wsi[64 + 2 * S:64 + 2 * S + len(hit)]) == [int(v) for v in np.cumsum([0] + cnts[:-1])]
    h = ws[L["h"]:L["h"] + 4 * S * DFF].view(np.float32).reshape(S, DFF)
    hq = ws[L["hq"]:L["hq"] + 36 * S * DFF // 32].reshape(S, -1)
    y = ws[L["y"]:L["y"] + 4 * S * DM].view(np.float32).reshape(S, DM)
    res = orc.grouped_expert(moe["gate"], moe["up"], moe["down"], xq_np, ids, rw, E, T, TOPK, DM, DFF,
                             hq_in=hq)
    gb = DFF * (DM // 256) * 144
    for s in range(S):
        t, e = s // TOPK, ids.reshape(-1)[s]
        # (ii) h within tolerance of the oracle's fp64 chain from the same xq
        gref, ga = orc.mmvq("q4k", moe["gate"][e * gb:(e + 1) * gb], xq_np[t], DFF, DM)
        uref, ua = orc.mmvq("q4k", moe["up"][e * gb:(e + 1) * gb], xq_np[t], DFF, DM)
        gref, ga, uref, ua = gref[0], ga[0], uref[0], ua[0]
        sig = 1 / (1 + np.exp(-gref))
        href = gref * sig * uref
        bound = 1e-5 * (ga * np.abs(uref) * 1.1 + np.abs(gref * sig) * ua) + 4 * np.spacing(np.abs(href).astype(np.float32))
        assert np.all(np.abs(h[s] - href) <= bound), f"h slot {s}"
        # (iii) requantization of the GPU's own h is bit-exact
        assert np.array_equal(hq[s], orc.quantize_q8_1(h[s][None])[0]), f"hq slot {s}"
        # (iv)/(v) down product from the GPU's hq within tolerance
        assert_close(y[s][None], res["y"][s][None], res["y_absum"][s][None], f"y slot {s}")
    assert_close(out, res["out"], res["out_absum"], "out")
    # (vi) fully independent chain: report the requantization flips
    ind = orc.grouped_expert(moe["gate"], moe["up"], moe["down"], xq_np, ids, rw, E, T, TOPK, DM, DFF)
    flips = int((ind["hq"] != hq).sum())
    rel = np.abs(out - ind["out"]).max() / np.abs(ind["out"]).max()
    note(f"T={T}: independent chain: {flips} differing hq bytes, max rel err {rel:.2e}")
    assert rel < 1e-2


@pytest.mark.parametrize("T", [1, 3])
def test_moe_graph_replay_matches_eager(moe, T):
    """The routed chain captured in a HIP graph: every replay (workspace and
    output poisoned before it, eager work between replays) gives the eager
    output and routing tables bit for bit (T = 1: the short-window launch
    pair; T = 3: the three-launch chain)."""
    note(f"MoE graph replay T={T}")
    g = synth.rng(synth.seed_for(4, 5, T))
    ids, rw = synth.routing(g, T, E, TOPK)
    xq, _ = quantize(synth.activations(g, T, DM))
    wsb = qmv.grouped_expert_mmvq_workspace(E, T, TOPK, DM, DFF)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out = torch.empty(T * DM, dtype=torch.float32, device=DEV)
    idd, rwd = dev(ids), dev(rw)
    L = qmv.moe_workspace_layout(T, TOPK, DM, DFF)

    def call(stream=None):
        qmv.grouped_expert_mmvq(moe["gd"], moe["ud"], moe["dp"], PL, xq, idd, rwd, out, E, T, TOPK, DM, DFF,
                                ws, wsb, stream=stream)
    S = T * TOPK
    nhit = len(set(ids.reshape(-1).tolist()))

    def written(wsh):                 # the table entries a call writes
        wi = wsh[:L["h"]].view(np.int32)
        return np.concatenate([wi[0:2], wi[64:64 + nhit], wi[64 + S:64 + S + nhit],
                               wi[64 + 2 * S:64 + 2 * S + nhit], wi[64 + 3 * S:64 + 4 * S]])
    call()
    eager, tables = host(out).copy(), written(host(ws))
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            call(stream=s)
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), eager.view(np.uint32)), f"replay {i}"
        assert np.array_equal(written(host(ws)), tables), f"tables, replay {i}"
        _ = (out * 2).sum().item()             # eager work between replays


def test_moe_unrouted_experts_unread(moe):
    """NaN scales in every expert no token is routed to leave out unchanged."""
    note("MoE poisoned unrouted experts")
    T = 4
    g = synth.rng(synth.seed_for(4, 2, T))
    ids, rw = synth.routing(g, T, E, TOPK)
    xq, _ = quantize(synth.activations(g, T, DM))
    base, _ = run_moe(moe, xq, ids, rw, T)
    hit = set(ids.reshape(-1).tolist())
    gate, up, down = moe["gate"].copy(), moe["up"].copy(), moe["down"].copy()
    gbk, dbk = DFF * (DM // 256), DM * (DFF // 256)
    for e in range(E):
        if e in hit:
            continue
        gv = gate.reshape(E * gbk, 144)[e * gbk:(e + 1) * gbk]
        uv = up.reshape(E * gbk, 144)[e * gbk:(e + 1) * gbk]
        dv = down.reshape(E * dbk, 210)[e * dbk:(e + 1) * dbk]
        gv[:, 0:4] = uv[:, 0:4] = np.array([0x00, 0x7E, 0x00, 0x7E], np.uint8)   # fp16 NaN d, dmin
        dv[:, 208:210] = np.array([0x00, 0x7E], np.uint8)
    dd = dev(down)
    for layout, wdn in ((PL, planar(dd, E * DM, DFF)), (GG, dd)):
        got, _ = run_moe(moe, xq, ids, rw, T, layout, wg=dev(gate), wu=dev(up), wdn=wdn)
        assert np.array_equal(got.view(np.uint32), base.view(np.uint32)), f"layout {layout}"


def test_moe_out_of_range_id_is_skipped(moe):
    note("MoE out-of-range id")
    T = 2
    g = synth.rng(synth.seed_for(4, 3, T))
    ids, rw = synth.routing(g, T, E, TOPK)
    xq, xq_np = quantize(synth.activations(g, T, DM))
    bad = ids.copy()
    bad[1, 3] = E + 5
    out, ws = run_moe(moe, xq, bad, rw, T)
    assert ws[:8].view(np.int32)[1] == 1
    # the oracle chained on the GPU's requantized h, the bad slot given
    # weight 0 and an all-zero hq (so it adds exactly 0): out within the
    # tolerance rule, like the staged parity
    L = qmv.moe_workspace_layout(T, TOPK, DM, DFF)
    S = T * TOPK
    hq = ws[L["hq"]:L["hq"] + 36 * S * DFF // 32].reshape(S, -1).copy()
    hq[1 * TOPK + 3] = 0
    rw0 = rw.copy()
    rw0[1, 3] = 0.0
    res = orc.grouped_expert(moe["gate"], moe["up"], moe["down"], xq_np, ids, rw0, E, T, TOPK, DM, DFF,
                             hq_in=hq)
    assert_close(out, res["out"], res["out_absum"], "out with an out-of-range id")
    # the other slots' requantized h are still those of the GPU's own h
    h = ws[L["h"]:L["h"] + 4 * S * DFF].view(np.float32).reshape(S, DFF)
    for s in range(S):
        if s != 1 * TOPK + 3:
            assert np.array_equal(hq[s], orc.quantize_q8_1(h[s][None])[0]), f"hq slot {s}"


@pytest.mark.parametrize("T", [2, 3])
def test_moe_small_ragged_topk4(T):
    """Rows that are not whole register chunks (the ragged kernels) and a
    routing width of 4: E = 6, d_model = 512, d_ff = 256, T = 2 (eight
    slots: the short-window down+combine launch) and T = 3."""
    note(f"grouped_expert_mmvq small: E=6 d_model=512 d_ff=256 T={T} topk=4")
    e_, dm, dff, tk = 6, 512, 256, 4
    g = synth.rng(730)
    gate, up, down = synth.moe_weights(g, e_, dm, dff)
    ids, rw = synth.routing(g, T, e_, tk)
    xq, xq_np = quantize(synth.activations(g, T, dm))
    wsb = qmv.grouped_expert_mmvq_workspace(e_, T, tk, dm, dff)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    L = qmv.moe_workspace_layout(T, tk, dm, dff)
    for layout in (PL, GG):
        dd = dev(down)
        wdn = planar(dd, e_ * dm, dff) if layout == PL else dd
        out, buf = guarded(T * dm)
        qmv.grouped_expert_mmvq(dev(gate), dev(up), wdn, layout, xq, dev(ids), dev(rw), out, e_, T, tk, dm, dff,
                                ws, wsb)
        assert canaries_intact(buf, T * dm)
        got, wsh = host(out).reshape(T, dm), host(ws)
        S = T * tk
        h = wsh[L["h"]:L["h"] + 4 * S * dff].view(np.float32).reshape(S, dff)
        hq = wsh[L["hq"]:L["hq"] + 36 * S * dff // 32].reshape(S, -1)
        y = wsh[L["y"]:L["y"] + 4 * S * dm].view(np.float32).reshape(S, dm)
        res = orc.grouped_expert(gate, up, down, xq_np, ids, rw, e_, T, tk, dm, dff, hq_in=hq)
        for s in range(S):
            assert np.array_equal(hq[s], orc.quantize_q8_1(h[s][None])[0]), f"hq slot {s}"
            assert_close(y[s][None], res["y"][s][None], res["y_absum"][s][None], f"y slot {s}")
        assert_close(got, res["out"], res["out_absum"], f"out layout {layout}")

"""GPU parity of mmvq_q6k_batch (several tiled Q6_K products of one K in one
launch), through the C ABI: every job's output bit for bit what mmvq_q6k
gives for it alone, and within the oracle's tolerance on every row, at every
workgroup shape the tiled kernel takes by row length (1, 2, 4, 8 and 16
waves along K, two chunks per row), with ragged row counts, every column
count, Q8_1 blocks and column-planar activations; the decode step of three
10240 x 2560 products at 8, 4 and 1 columns at full size; graph replay."""
import numpy as np
import pytest
import torch

from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import (DEV, assert_close, canaries_intact, check_all_rows, dev, guarded, host, mmvq, note,
                            oracle_all_rows, quantize, tiled)

pytestmark = pytest.mark.gpu

TL, XT = qmv.LAYOUT_TILED, qmv.LAYOUT_TILED | qmv.ACT_PLANAR


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def quantize_planar(x):
    ncols, K = x.shape
    xp = torch.empty(ncols * (K // 32) * 36, dtype=torch.uint8, device=DEV)
    qmv.quantize_q8_1_planar(dev(np.ascontiguousarray(x, dtype=np.float32)), xp, K, ncols)
    return xp


def make_jobs(seed, K, shapes, planar_act):
    g = synth.rng(seed)
    jobs = []
    for rows, n in shapes:
        w = synth.q6k_blocks(g, rows, K)
        x = synth.activations(g, n, K)
        xq, xq_np = quantize(x)
        jobs.append(dict(w=w, wt=tiled(dev(w), rows, K), x=quantize_planar(x) if planar_act else xq, xq_np=xq_np,
                         rows=rows, n=n))
    return jobs


def run_batch(jobs, K, layout):
    outs = [guarded(j["n"] * j["rows"]) for j in jobs]
    qmv.mmvq_q6k_batch([(j["wt"], j["x"], o[0], j["rows"], j["n"]) for j, o in zip(jobs, outs)], layout, K)
    res = []
    for j, (o, buf) in zip(jobs, outs):
        assert canaries_intact(buf, j["n"] * j["rows"]), "output guard words overwritten"
        res.append(host(o).reshape(j["n"], j["rows"]))
    return res


# (K, [(rows, ncols), ...]): K = 512 one wave along K with four row tiles per
# workgroup, 768 two waves and two tiles, 2560 four waves, 5120 eight,
# 10240 sixteen, 20480 sixteen with two chunks per row; ragged row counts
SHAPES = [(512, [(37, 3), (100, 8), (1, 1)]), (768, [(19, 5), (64, 2), (33, 7)]),
          (2560, [(130, 8), (37, 4), (16, 1), (50, 6)]), (5120, [(40, 8), (23, 3)]),
          (10240, [(9, 8), (40, 2), (17, 5)]), (20480, [(17, 6), (8, 1)])]


@pytest.mark.parametrize("planar_act", [False, True])
@pytest.mark.parametrize("K,shapes", SHAPES)
def test_batch_equals_single_products_and_oracle(K, shapes, planar_act):
    note(f"mmvq_q6k_batch K={K} jobs={shapes} column-planar={planar_act}")
    jobs = make_jobs(1950 + K, K, shapes, planar_act)
    lay = XT if planar_act else TL
    got = run_batch(jobs, K, lay)
    for j, o in zip(jobs, got):
        alone = mmvq("q6k", j["wt"], j["x"], j["rows"], K, j["n"], lay)
        assert np.array_equal(o.view(np.uint32), alone.view(np.uint32)), f"job {j['rows']}x{K} N={j['n']}"
        ref, ab = oracle_all_rows("q6k", j["w"], j["xq_np"], j["rows"], K)
        assert_close(o, ref, ab, f"job {j['rows']}x{K} N={j['n']}")


def test_batch_every_column_count_and_eight_jobs():
    K = 2560
    shapes = [(48 + 7 * n, n) for n in range(1, 9)]
    note(f"mmvq_q6k_batch eight jobs N=1..8 K={K}")
    jobs = make_jobs(1960, K, shapes, True)
    for order in (jobs, jobs[::-1]):
        got = run_batch(order, K, XT)
        for j, o in zip(order, got):
            alone = mmvq("q6k", j["wt"], j["x"], j["rows"], K, j["n"], XT)
            assert np.array_equal(o.view(np.uint32), alone.view(np.uint32))


def test_batch_decode_step_full_size():
    """The benchmark's step: 10240 x 2560 at 8, 4 and 1 columns, each on its
    own weights and columns, in one launch; every row against the oracle."""
    K, rows = 2560, 10240
    note("mmvq_q6k_batch 3 x 10240x2560 (N = 8, 4, 1)")
    jobs = make_jobs(1970, K, [(rows, 8), (rows, 4), (rows, 1)], True)
    got = run_batch(jobs, K, XT)
    for j, o in zip(jobs, got):
        alone = mmvq("q6k", j["wt"], j["x"], rows, K, j["n"], XT)
        assert np.array_equal(o.view(np.uint32), alone.view(np.uint32))
        check_all_rows("q6k", j["w"], j["xq_np"], o, rows, K, f"batch job N={j['n']}")


@pytest.mark.parametrize("K,shapes", [(2560, [(100, 8), (17, 1), (300, 4), (64, 7), (5, 2), (1000, 3)]),
                                      (5120, [(3000, 8), (3000, 4), (3000, 1)]),
                                      (5120, [(90, 8), (17, 1), (300, 4), (64, 7), (5, 2), (777, 3)])])
def test_batch_streamed_form(K, shapes):
    """Column-planar jobs at K = 2560 and 5120 take the streamed form (one
    wave per row tile over all of K; four-entry job table up to four jobs,
    eight beyond): every job bit for bit its single product and within s6 of
    the oracle on every row."""
    note(f"mmvq_q6k_batch streamed K={K} jobs={shapes}")
    jobs = make_jobs(2010 + K // 256 + len(shapes), K, shapes, True)
    got = run_batch(jobs, K, XT)
    for j, o in zip(jobs, got):
        alone = mmvq("q6k", j["wt"], j["x"], j["rows"], K, j["n"], XT)
        assert np.array_equal(o.view(np.uint32), alone.view(np.uint32)), f"job {j['rows']}x{K} N={j['n']}"
        ref, ab = oracle_all_rows("q6k", j["w"], j["xq_np"], j["rows"], K)
        assert_close(o, ref, ab, f"job {j['rows']}x{K} N={j['n']}")


@pytest.mark.parametrize("case", range(6))
def test_batch_random_batches(case):
    """Seeded random batches: K a multiple of 256 up to 20480 (every number
    of waves along K), 1-8 jobs of 1-3000 rows and 1-8 columns each, Q8_1
    blocks or column-planar activations; every job bit for bit its single
    launch and within tolerance of the oracle on every row."""
    g = synth.rng(1995 + case)
    K = 256 * int(g.integers(1, 81))
    shapes = [(int(g.integers(1, 3001)), int(g.integers(1, 9))) for _ in range(int(g.integers(1, 9)))]
    planar_act = bool(case % 2)
    note(f"mmvq_q6k_batch random K={K} jobs={shapes} column-planar={planar_act}")
    jobs = make_jobs(2000 + case, K, shapes, planar_act)
    lay = XT if planar_act else TL
    got = run_batch(jobs, K, lay)
    for j, o in zip(jobs, got):
        alone = mmvq("q6k", j["wt"], j["x"], j["rows"], K, j["n"], lay)
        assert np.array_equal(o.view(np.uint32), alone.view(np.uint32)), f"job {j['rows']}x{K} N={j['n']}"
        ref, ab = oracle_all_rows("q6k", j["w"], j["xq_np"], j["rows"], K)
        assert_close(o, ref, ab, f"job {j['rows']}x{K} N={j['n']}")


def test_batch_single_job_and_shared_weights():
    """One job alone; and two jobs on the same weights with different
    columns (a matrix applied to two windows)."""
    K, rows = 2560, 300
    jobs = make_jobs(1980, K, [(rows, 8), (rows, 3)], False)
    jobs[1]["wt"], jobs[1]["w"] = jobs[0]["wt"], jobs[0]["w"]
    for sel in ([jobs[0]], jobs):
        got = run_batch(sel, K, TL)
        for j, o in zip(sel, got):
            alone = mmvq("q6k", j["wt"], j["x"], rows, K, j["n"], TL)
            assert np.array_equal(o.view(np.uint32), alone.view(np.uint32))


def test_batch_graph_replay():
    K = 2560
    jobs = make_jobs(1990, K, [(3000, 8), (1000, 4), (2000, 1)], True)
    outs = [torch.empty(j["n"] * j["rows"], dtype=torch.float32, device=DEV) for j in jobs]
    desc = [(j["wt"], j["x"], o, j["rows"], j["n"]) for j, o in zip(jobs, outs)]
    qmv.mmvq_q6k_batch(desc, XT, K)
    eager = [host(o).copy() for o in outs]
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qmv.mmvq_q6k_batch(desc, XT, K, stream=s)
    for i in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(host(o).view(np.uint32), e.view(np.uint32)), f"replay {i}"
        _ = (outs[0] * 2).sum().item()

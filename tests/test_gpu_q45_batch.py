"""GPU parity of mmvq_q4k_batch / mmvq_q5k_batch (several Q4_K or Q5_K
products of one K in one call), through the C ABI: every job's output bit
for bit what mmvq_q4k / mmvq_q5k gives for it alone, and within the
oracle's tolerance on every row.  The shapes take every lanes-per-row class
(8, 16, 32, 64) and both register depths (three units, and five with a
ragged and a whole last chunk), batches that mix classes in one call (one
launch for up to four jobs of the two widths one K can take, one launch
per width beyond), every column count 1-8 in one batch, the long-row
matrices whose single products take ten-wave workgroups, the dense
benchmark's 12288 / 6144 / 512 x 2560 decode step at full size, exact
arithmetic, and graph replay."""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import (DEV, assert_close, canaries_intact, check_all_rows, dev, guarded, host, mmvq, note,
                            oracle_all_rows, quantize)

pytestmark = pytest.mark.gpu

KINDS = ["q4k", "q5k"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def blocks(kind, g, rows, K):
    return synth.q4k_blocks(g, rows, K) if kind == "q4k" else synth.q5k_blocks(g, rows, K)


def make_jobs(kind, seed, K, shapes):
    g = synth.rng(seed)
    jobs = []
    for rows, n in shapes:
        w = blocks(kind, g, rows, K)
        xq, xq_np = quantize(synth.activations(g, n, K))
        jobs.append(dict(w=w, wd=dev(w), x=xq, xq_np=xq_np, rows=rows, n=n))
    return jobs


def run_batch(kind, jobs, K):
    outs = [guarded(j["n"] * j["rows"]) for j in jobs]
    fn = qmv.mmvq_q4k_batch if kind == "q4k" else qmv.mmvq_q5k_batch
    fn([(j["wd"], j["x"], o[0], j["rows"], j["n"]) for j, o in zip(jobs, outs)], K)
    res = []
    for j, (o, buf) in zip(jobs, outs):
        assert canaries_intact(buf, j["n"] * j["rows"]), "output guard words overwritten"
        res.append(host(o).reshape(j["n"], j["rows"]))
    return res


def same_bits_as_alone(kind, jobs, got, K):
    for j, o in zip(jobs, got):
        alone = mmvq(kind, j["wd"], j["x"], j["rows"], K, j["n"])
        assert np.array_equal(o.view(np.uint32), alone.view(np.uint32)), f"job {j['rows']}x{K} N={j['n']}"


# (K, [(rows, ncols), ...]) -> lanes per row (depth): K = 256 and 512 8 (3);
# 1024: 16 below 2048 rows, 8 from there (3); 2560: 32 below 1024 rows, 16
# from there (3); 3584: 32 (3) below 1024 rows, 16 (5) from there; 5120: 64
# below 512 rows, 32 from there (3); 14336: 64 (5, ragged last chunk);
# 20480: 64 (5, one whole chunk); ragged row counts.  Up to four jobs of
# two widths run in one launch; the five-job batch of two widths runs one
# launch per width.
SHAPES = [(256, [(37, 3), (100, 8), (1, 1)]), (512, [(19, 5), (64, 2), (33, 7)]),
          (1024, [(300, 4), (2100, 1), (50, 6)]), (2560, [(130, 8), (1100, 4), (16, 1), (1030, 7)]),
          (2560, [(300, 1), (2000, 2), (310, 3), (1500, 4), (320, 5)]),
          (3584, [(1200, 2), (200, 5), (1100, 8)]),
          (5120, [(40, 8), (600, 3), (23, 6)]), (14336, [(9, 8), (40, 2), (17, 5)]),
          (20480, [(17, 6), (8, 1)])]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("K,shapes", SHAPES)
def test_q45_batch_equals_single_products_and_oracle(kind, K, shapes):
    note(f"mmvq_{kind}_batch K={K} jobs={shapes}")
    jobs = make_jobs(kind, 2050 + K + len(shapes), K, shapes)
    got = run_batch(kind, jobs, K)
    same_bits_as_alone(kind, jobs, got, K)
    for j, o in zip(jobs, got):
        ref, ab = oracle_all_rows(kind, j["w"], j["xq_np"], j["rows"], K)
        assert_close(o, ref, ab, f"job {j['rows']}x{K} N={j['n']}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rows", [700, 1500])
def test_q45_batch_every_column_count_and_eight_jobs(kind, rows):
    """Eight jobs at 1..8 columns (32 and 16 lanes per row at K = 2560),
    in both orders."""
    K = 2560
    shapes = [(rows + 7 * n, n) for n in range(1, 9)]
    note(f"mmvq_{kind}_batch eight jobs N=1..8 K={K} rows~{rows}")
    jobs = make_jobs(kind, 2060 + rows, K, shapes)
    for order in (jobs, jobs[::-1]):
        same_bits_as_alone(kind, order, run_batch(kind, order, K), K)


@pytest.mark.parametrize("kind", KINDS)
def test_q45_batch_long_rows(kind):
    """Matrices whose single Q4_K products take ten-wave workgroups (64 lanes
    per row, 2300 rows) beside a short one, at depths three and five."""
    for K in (10240, 20480):
        note(f"mmvq_{kind}_batch long rows K={K}")
        jobs = make_jobs(kind, 2070 + K // 256, K, [(2300, 4), (2300, 1), (90, 8)])
        got = run_batch(kind, jobs, K)
        same_bits_as_alone(kind, jobs, got, K)
        check_all_rows(kind, jobs[2]["w"], jobs[2]["xq_np"], got[2], 90, K)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n", [1, 4])
def test_q45_batch_decode_step_full_size(kind, n):
    """The dense benchmark's K = 2560 matrices (12288, 6144 and 512 rows) in
    one call at n columns; every row against the oracle."""
    K = 2560
    note(f"mmvq_{kind}_batch 12288/6144/512 x 2560 N={n}")
    jobs = make_jobs(kind, 2080 + n, K, [(12288, n), (6144, n), (512, n)])
    got = run_batch(kind, jobs, K)
    same_bits_as_alone(kind, jobs, got, K)
    for j, o in zip(jobs, got):
        check_all_rows(kind, j["w"], j["xq_np"], o, j["rows"], K, f"batch job {j['rows']}x{K} N={n}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("case", range(6))
def test_q45_batch_random_batches(kind, case):
    """Seeded random batches: K a multiple of 256 up to 8192, 1-8 jobs of
    1-3000 rows and 1-8 columns each (one or two widths, four or more
    jobs); every job bit for bit its single launch and within tolerance of
    the oracle on every row."""
    g = synth.rng(2120 + case)
    K = 256 * int(g.integers(1, 33))
    shapes = [(int(g.integers(1, 3001)), int(g.integers(1, 9))) for _ in range(int(g.integers(1, 9)))]
    note(f"mmvq_{kind}_batch random K={K} jobs={shapes}")
    jobs = make_jobs(kind, 2130 + case, K, shapes)
    got = run_batch(kind, jobs, K)
    same_bits_as_alone(kind, jobs, got, K)
    for j, o in zip(jobs, got):
        ref, ab = oracle_all_rows(kind, j["w"], j["xq_np"], j["rows"], K)
        assert_close(o, ref, ab, f"job {j['rows']}x{K} N={j['n']}")


@pytest.mark.parametrize("kind", KINDS)
def test_q45_batch_exact_arithmetic_bitexact(kind):
    """Inputs whose every fp32 product and partial sum is exact: each job
    returns the oracle's value exactly."""
    g = synth.rng(2090)
    K = 2560
    outs, refs = [], []
    desc = []
    for rows, n in ((45, 3), (1200, 8), (7, 1)):
        w = synth.exact_q45_blocks(g, rows, K, kind == "q5k")
        xq_np = synth.exact_q8_1(g, n, K)
        refs.append(orc.mmvq(kind, w, xq_np, rows, K)[0])
        o = torch.empty(n * rows, dtype=torch.float32, device=DEV)
        outs.append((o, rows, n))
        desc.append((dev(w), dev(xq_np), o, rows, n))
    (qmv.mmvq_q4k_batch if kind == "q4k" else qmv.mmvq_q5k_batch)(desc, K)
    for (o, rows, n), ref in zip(outs, refs):
        assert np.array_equal(host(o).reshape(n, rows).astype(np.float64), ref)


@pytest.mark.parametrize("kind", KINDS)
def test_q45_batch_shared_weights_and_single_job(kind):
    """One job alone; and two jobs on the same weights with different
    columns."""
    K, rows = 2560, 300
    jobs = make_jobs(kind, 2100, K, [(rows, 8), (rows, 3)])
    jobs[1]["wd"], jobs[1]["w"] = jobs[0]["wd"], jobs[0]["w"]
    for sel in ([jobs[0]], jobs):
        same_bits_as_alone(kind, sel, run_batch(kind, sel, K), K)


def test_q45_batch_graph_replay():
    K = 2560
    jobs = make_jobs("q4k", 2110, K, [(12288, 4), (6144, 1), (512, 4)])
    outs = [torch.empty(j["n"] * j["rows"], dtype=torch.float32, device=DEV) for j in jobs]
    desc = [(j["wd"], j["x"], o, j["rows"], j["n"]) for j, o in zip(jobs, outs)]
    qmv.mmvq_q4k_batch(desc, K)
    eager = [host(o).copy() for o in outs]
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            qmv.mmvq_q4k_batch(desc, K, stream=s)
    for i in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(host(o).view(np.uint32), e.view(np.uint32)), f"replay {i}"
        _ = (outs[0] * 2).sum().item()

"""Helpers of the GPU parity tests: device upload, calls through the C ABI,
and the comparison rules.

Tolerance rule for fp32 outputs (the GPU sums in fp32 in an order of its own;
the oracle sums exact terms in fp64): for every output, |gpu - oracle| <=
1e-5 * A, where A is the sum of the absolute values of the terms the oracle
added (the scale of any reordering error); and per column,
max|gpu - oracle| <= 1e-5 * max|oracle|.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch

import oracle as orc
from quant_mat_vec_amd import qmv

DEV = "cuda:0"
TOL = 1e-5
CANARY = 0x7FC0DEAD          # a NaN pattern no kernel writes


def note(msg: str) -> None:
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def guarded(n: int, dtype=torch.float32, pad: int = 64):
    """(view of n elements, whole buffer) with `pad` canary words each side."""
    buf = torch.full((n + 2 * pad,), CANARY, dtype=torch.int32, device=DEV)
    view = buf[pad:pad + n]
    if dtype == torch.float32:
        view = view.view(torch.float32)
    return view, buf


def canaries_intact(buf: torch.Tensor, n: int, pad: int = 64) -> bool:
    b = host(buf)
    return bool(np.all(b[:pad] == CANARY) and np.all(b[pad + n:] == CANARY))


def quantize(x: np.ndarray) -> tuple[torch.Tensor, np.ndarray]:
    x = np.ascontiguousarray(x, dtype=np.float32)
    ncols, K = x.shape
    xd = dev(x)
    xq = torch.empty(ncols * (K // 32) * 36, dtype=torch.uint8, device=DEV)
    qmv.quantize_q8_1(xd, xq, K, ncols)
    return xq, host(xq).reshape(ncols, -1)


def mmvq(kind: str, w: torch.Tensor, xq: torch.Tensor, rows: int, K: int, ncols: int,
         layout: int = qmv.LAYOUT_GGUF) -> np.ndarray:
    out, buf = guarded(ncols * rows)
    if kind == "q6k":
        qmv.mmvq_q6k(w, layout, xq, out, rows, K, ncols)
    elif kind == "q4k":
        qmv.mmvq_q4k(w, xq, out, rows, K, ncols)
    else:
        qmv.mmvq_q5k(w, xq, out, rows, K, ncols)
    assert canaries_intact(buf, ncols * rows), "output guard words overwritten"
    return host(out).reshape(ncols, rows)


def isums(kind: str, w: torch.Tensor, xq: torch.Tensor, rows: int, K: int, ncols: int,
          layout: int = qmv.LAYOUT_GGUF) -> np.ndarray:
    n = ncols * rows * (K // 32)
    out, buf = guarded(n, dtype=torch.int32)
    if kind == "q6k":
        qmv.mmvq_q6k_isums(w, layout, xq, out, rows, K, ncols)
    elif kind == "q4k":
        qmv.mmvq_q4k_isums(w, xq, out, rows, K, ncols)
    else:
        qmv.mmvq_q5k_isums(w, xq, out, rows, K, ncols)
    assert canaries_intact(buf, n), "isum guard words overwritten"
    return host(out).reshape(ncols, rows, K // 32)


def planar(w: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    p = torch.empty_like(w)
    qmv.repack_q6k_planar(w, p, rows, K)
    return p


def tiled(w: torch.Tensor, rows: int, K: int) -> torch.Tensor:
    t = torch.empty_like(w)
    qmv.repack_q6k_tiled(w, t, rows, K)
    return t


def assert_close(got: np.ndarray, ref: np.ndarray, absum: np.ndarray, what: str = "") -> None:
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    bad = err > TOL * absum
    assert not np.any(bad), (f"{what}: {int(bad.sum())} outputs beyond 1e-5*A; worst rel-to-A "
                             f"{float((err / np.maximum(absum, 1e-300)).max()):.3e}")
    colmax = np.abs(ref).max(axis=-1)
    assert np.all(err.max(axis=-1) <= TOL * colmax), f"{what}: column max error beyond 1e-5*max|ref|"


# ------------------------------------------------ the oracle on every row
_POOL = None


def _pool() -> cf.ThreadPoolExecutor:
    """Host threads for the oracle (its calls release the GIL)."""
    global _POOL
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(max(1, min(len(os.sched_getaffinity(0)), 16)))
    return _POOL


def _row_chunks(rows: int):
    n = _pool()._max_workers
    step = max(1, -(-rows // (4 * n)))
    return [(r0, min(step, rows - r0)) for r0 in range(0, rows, step)]


def oracle_all_rows(kind: str, w: np.ndarray, xq_np: np.ndarray, rows: int, K: int):
    """(out, absum) of the oracle for every row, fp64 [ncols][rows], the
    rows split over host threads."""
    futs = [_pool().submit(orc.mmvq, kind, w, xq_np, rows, K, r0, n) for r0, n in _row_chunks(rows)]
    parts = [f.result() for f in futs]
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def oracle_isums_all_rows(kind: str, w: np.ndarray, xq_np: np.ndarray, rows: int, K: int) -> np.ndarray:
    """The oracle's per-sub-block integer sums for every row, int32
    [ncols][rows][K/32] (Q6_K isums, Q4_K/Q5_K dots), rows split over host
    threads."""
    bpb = {"q6k": 210, "q4k": 144, "q5k": 176}[kind] * (K // 256)

    def part(r0, n):
        sub = w[r0 * bpb:(r0 + n) * bpb]
        return orc.q6k_isums(sub, xq_np, n, K) if kind == "q6k" else orc.q45_dots(kind, sub, xq_np, n, K)
    futs = [_pool().submit(part, r0, n) for r0, n in _row_chunks(rows)]
    return np.concatenate([f.result() for f in futs], axis=1)


def check_all_rows(kind: str, w: np.ndarray, xq_np: np.ndarray, got: np.ndarray, rows: int, K: int,
                   what: str = "") -> None:
    """Every output of a full-size product against the oracle (tolerance
    rule above)."""
    ref, ab = oracle_all_rows(kind, w, xq_np, rows, K)
    assert_close(got, ref, ab, what or f"{kind} {rows}x{K} all rows")

"""CPU oracle for the quantized matrix-vector product -- TEST INFRASTRUCTURE.

Plain scalar C (``qmv_oracle.c``, built into ``liboracle.so`` with gcc) behind
a thin numpy/ctypes wrapper.  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the GPU library
(``quant_mat_vec_amd``) never does, and this package never imports it.

Every function restates what the pages define; the C file's header lists the
pages and the readings taken where they are silent.  Parity pins (tests marked
``not gpu``) tie each function to something other than itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q6K_BYTES, Q4K_BYTES, Q5K_BYTES, Q81_BYTES = 210, 144, 176, 36


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
             "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_half_to_double.restype = D
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_float_to_half.restype = ctypes.c_uint16
        for name in ("orc_q6k_decode",):
            getattr(L, name).argtypes = [P, P, P, P]
        for name in ("orc_q4k_decode", "orc_q5k_decode"):
            getattr(L, name).argtypes = [P, P, P, P, P, P]
        for name in ("orc_dequant_q6k", "orc_dequant_q4k", "orc_dequant_q5k",
                     "orc_q6k_to_planar", "orc_q6k_to_tiled"):
            getattr(L, name).argtypes = [P, P, I64, I64]
        L.orc_q6k_gather.argtypes = [P, I, I64, I64, P, I64, P]
        L.orc_quantize_q8_1.argtypes = [P, P, I64, I]
        L.orc_q8_1_to_planar.argtypes = [P, P, I64, I]
        L.orc_rmsnorm.argtypes = [P, P, D, P, I64, I]
        L.orc_dequant_q8_1.argtypes = [P, P, I64, I]
        for name in ("orc_q6k_isums", "orc_q4k_dots", "orc_q5k_dots"):
            getattr(L, name).argtypes = [P, P, P, I64, I64, I]
        for name in ("orc_mmvq_q6k", "orc_mmvq_q4k", "orc_mmvq_q5k"):
            getattr(L, name).argtypes = [P, P, P, P, I64, I64, I, I64, I64]
        L.orc_grouped_expert.argtypes = [P, P, P, P, P, P, I, I, I, I64, I64, P,
                                         P, P, P, P, P, P, P, P]
        L.orc_grouped_expert.restype = I
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint8
    return a


# ------------------------------------------------------------------ fp16
def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(int(bits))


def float_to_half(x: float) -> int:
    return int(lib().orc_float_to_half(float(np.float32(x))))


# --------------------------------------------------------------- decoders
def q6k_decode(blk):
    blk = _u8(blk)
    q = np.zeros(256, np.int8)
    sc = np.zeros(16, np.int8)
    d = np.zeros(1, np.float64)
    lib().orc_q6k_decode(_p(blk), _p(q), _p(sc), _p(d))
    return q, sc, float(d[0])


def _q45_decode(blk, five):
    blk = _u8(blk)
    q = np.zeros(256, np.uint8)
    sc = np.zeros(8, np.uint8)
    m = np.zeros(8, np.uint8)
    d = np.zeros(1, np.float64)
    dm = np.zeros(1, np.float64)
    fn = lib().orc_q5k_decode if five else lib().orc_q4k_decode
    fn(_p(blk), _p(q), _p(sc), _p(m), _p(d), _p(dm))
    return q, sc, m, float(d[0]), float(dm[0])


def q4k_decode(blk):
    return _q45_decode(blk, False)


def q5k_decode(blk):
    return _q45_decode(blk, True)


def dequant(kind: str, w, rows: int, K: int):
    """Weights as fp64 [rows][K]."""
    w = _u8(w)
    out = np.zeros((rows, K), np.float64)
    getattr(lib(), f"orc_dequant_{kind}")(_p(w), _p(out), rows, K)
    return out


# ------------------------------------------------------------------ Q8_1
def quantize_q8_1(x):
    """x: fp32 [ncols][K] -> Q8_1 bytes [ncols][K/32*36]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    ncols, K = x.shape
    assert K % 32 == 0
    xq = np.zeros((ncols, K // 32 * Q81_BYTES), np.uint8)
    lib().orc_quantize_q8_1(_p(x), _p(xq), K, ncols)
    return xq


def rmsnorm(x, gamma, eps: float):
    """RMSNorm per column in fp64, rounded to fp32: [ncols][K]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None]
    ncols, K = x.shape
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    assert gamma.shape == (K,)
    y = np.zeros((ncols, K), np.float32)
    lib().orc_rmsnorm(_p(x), _p(gamma), float(eps), _p(y), K, ncols)
    return y


def rmsnorm_quantize_q8_1(x, gamma, eps: float):
    """The fused norm + quantizer: quantize_q8_1 of rmsnorm(x)."""
    return quantize_q8_1(rmsnorm(x, gamma, eps))


def q8_1_to_planar(xq, K: int):
    """Q8_1 blocks [ncols][K/32] -> the column-planar layout (same bytes)."""
    xq = _u8(xq)
    ncols = xq.size // (K // 32 * Q81_BYTES)
    dst = np.zeros(xq.size, np.uint8)
    lib().orc_q8_1_to_planar(_p(xq), _p(dst), K, ncols)
    return dst


def dequant_q8_1(xq, K: int):
    xq = _u8(xq)
    ncols = xq.size // (K // 32 * Q81_BYTES)
    out = np.zeros((ncols, K), np.float64)
    lib().orc_dequant_q8_1(_p(xq), _p(out), K, ncols)
    return out


# ----------------------------------------------------------- integer sums
def q6k_isums(w, xq, rows: int, K: int):
    """int32 [ncols][rows][K/32]."""
    w, xq = _u8(w), _u8(xq)
    ncols = xq.size // (K // 32 * Q81_BYTES)
    out = np.zeros((ncols, rows, K // 32), np.int32)
    lib().orc_q6k_isums(_p(w), _p(xq), _p(out), rows, K, ncols)
    return out


def q45_dots(kind: str, w, xq, rows: int, K: int):
    w, xq = _u8(w), _u8(xq)
    ncols = xq.size // (K // 32 * Q81_BYTES)
    out = np.zeros((ncols, rows, K // 32), np.int32)
    getattr(lib(), f"orc_{kind}_dots")(_p(w), _p(xq), _p(out), rows, K, ncols)
    return out


# ------------------------------------------------------------------ MMVQ
def mmvq(kind: str, w, xq, rows: int, K: int, row0: int = 0, nrows: int | None = None):
    """(out, absum), both fp64 [ncols][nrows], for rows [row0, row0+nrows)."""
    w, xq = _u8(w), _u8(xq)
    if nrows is None:
        nrows = rows - row0
    ncols = xq.size // (K // 32 * Q81_BYTES)
    out = np.zeros((ncols, nrows), np.float64)
    ab = np.zeros((ncols, nrows), np.float64)
    getattr(lib(), f"orc_mmvq_{kind}")(_p(w), _p(xq), _p(out), _p(ab), rows, K, ncols,
                                       row0, nrows)
    return out, ab


def q6k_to_planar(w, rows: int, K: int):
    w = _u8(w)
    dst = np.zeros(w.size, np.uint8)
    lib().orc_q6k_to_planar(_p(w), _p(dst), rows, K)
    return dst


def q6k_to_tiled(w, rows: int, K: int):
    w = _u8(w)
    dst = np.zeros(w.size, np.uint8)
    lib().orc_q6k_to_tiled(_p(w), _p(dst), rows, K)
    return dst


def q6k_gather(w, layout: int, rows: int, K: int, ids):
    """Rows ids of the GGUF matrix w, in `layout` (0 GGUF, 1 planar, 2 tiled);
    ids outside [0, rows) give all-zero rows."""
    w = _u8(w)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    dst = np.zeros(ids.size * (K // 256) * Q6K_BYTES, np.uint8)
    lib().orc_q6k_gather(_p(w), layout, rows, K, _p(ids), ids.size, _p(dst))
    return dst


# ------------------------------------------------------------- MoE chain
def grouped_expert(w_gate, w_up, w_down, xq, ids, route_w, E, T, topk, d_model, d_ff,
                   hq_in=None):
    """Full routed-expert chain; returns a dict of every intermediate."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    route_w = np.ascontiguousarray(route_w, dtype=np.float32)
    S = T * topk
    g = np.zeros((S, d_ff), np.float64)
    u = np.zeros((S, d_ff), np.float64)
    h = np.zeros((S, d_ff), np.float32)
    hq = np.zeros((S, d_ff // 32 * Q81_BYTES), np.uint8)
    y = np.zeros((S, d_model), np.float64)
    ya = np.zeros((S, d_model), np.float64)
    out = np.zeros((T, d_model), np.float64)
    oa = np.zeros((T, d_model), np.float64)
    hq_in_a = None if hq_in is None else _u8(hq_in)
    rc = lib().orc_grouped_expert(
        _p(_u8(w_gate)), _p(_u8(w_up)), _p(_u8(w_down)), _p(_u8(xq)), _p(ids), _p(route_w),
        E, T, topk, d_model, d_ff, _p(hq_in_a),
        _p(g), _p(u), _p(h), _p(hq), _p(y), _p(ya), _p(out), _p(oa))
    if rc != 0:
        raise ValueError("expert id out of range")
    return dict(g=g, u=u, h=h, hq=hq, y=y, y_absum=ya, out=out, out_absum=oa)

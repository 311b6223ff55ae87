"""Thin ctypes binding of libqmv's C ABI (declared in include/qmv.h).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the library entry point of the same name and raises
QmvError on a non-zero status.  Tensors are torch tensors on the GPU (torch is
used for device memory and streams only).  The library is opened on first
use; if it is missing the call raises at once -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqmv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "qmv.h")

QMV_OK, QMV_ERR_INVALID_ARG, QMV_ERR_UNSUPPORTED = 0, -1, -2
QMV_ERR_ALIGNMENT, QMV_ERR_WORKSPACE, QMV_ERR_HIP = -3, -4, -5
LAYOUT_GGUF, LAYOUT_PLANAR, LAYOUT_TILED = 0, 1, 2
ACT_PLANAR = 16   # OR-ed into the layout with LAYOUT_TILED: column-planar activations

_lib = None


class Q6kJob(ctypes.Structure):
    """qmv_q6k_job of include/qmv.h."""
    _fields_ = [("w", ctypes.c_void_p), ("xq", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("ncols", ctypes.c_int)]


class QmvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {strerror(code)} ({code})"
                         + (f", hipError {last_hip_error()}" if code == QMV_ERR_HIP else ""))


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libqmv is not built ({LIB_PATH} missing); "
                               "run python -m quant_mat_vec_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sig = {
            "quantize_q8_1": [P, P, I64, I, P],
            "quantize_q8_1_planar": [P, P, I64, I, P],
            "rmsnorm_quantize_q8_1": [P, P, ctypes.c_float, P, I64, I, I, P],
            "mmvq_q6k": [P, I, P, P, I64, I64, I, P],
            "mmq_q6k": [P, I, P, P, I64, I64, I, P],
            "mmvq_q4k": [P, P, P, I64, I64, I, P],
            "mmvq_q5k": [P, P, P, I64, I64, I, P],
            "repack_q6k_planar": [P, P, I64, I64, P],
            "unpack_q6k_planar": [P, P, I64, I64, P],
            "repack_q6k_tiled": [P, P, I64, I64, P],
            "unpack_q6k_tiled": [P, P, I64, I64, P],
            "gather_q6k_rows": [P, I, I64, I64, P, I64, P, P],
            "mmvq_q6k_argmax": [P, I, P, I64, I64, I, P, P, P, SZ, P],
            "mmvq_q6k_topk": [P, I, P, I64, I64, I, I, P, P, P, SZ, P],
            "mmvq_q6k_isums": [P, I, P, P, I64, I64, I, P],
            "mmvq_q4k_isums": [P, P, P, I64, I64, I, P],
            "mmvq_q5k_isums": [P, P, P, I64, I64, I, P],
            "grouped_expert_mmvq": [P, P, P, I, P, P, P, P, I, I, I, I64, I64, P, SZ, P],
            "grouped_expert_mmvq_noalloc": [P, P, P, I, P, P, P, P, I, I, I, I64, I64, P],
            "qmv_stream_read": [P, I64, P, I, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I
        L.mmvq_q6k_batch.argtypes = [ctypes.POINTER(Q6kJob), I, I, I64, P]
        L.mmvq_q6k_batch.restype = I
        for name in ("mmvq_q4k_batch", "mmvq_q5k_batch"):
            getattr(L, name).argtypes = [ctypes.POINTER(Q6kJob), I, I64, P]
            getattr(L, name).restype = I
        L.grouped_expert_mmvq_workspace.argtypes = [I, I, I, I64, I64]
        L.mmvq_q6k_topk_workspace.restype = SZ
        L.mmvq_q6k_topk_workspace.argtypes = [I64, I, I]
        L.mmvq_q6k_argmax_workspace.restype = SZ
        L.mmvq_q6k_argmax_workspace.argtypes = [I64, I]
        L.grouped_expert_mmvq_workspace.restype = SZ
        L.qmv_strerror.argtypes = [I]
        L.qmv_strerror.restype = ctypes.c_char_p
        L.qmv_last_hip_error.argtypes = []
        L.qmv_last_hip_error.restype = I
        _lib = L
    return _lib


def declared_symbols() -> list[str]:
    """Names of the functions include/qmv.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)


def strerror(code: int) -> str:
    return lib().qmv_strerror(int(code)).decode()


def last_hip_error() -> int:
    return lib().qmv_last_hip_error()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != QMV_OK:
        raise QmvError(rc, what)


# ------------------------------------------------------------ entry points
def quantize_q8_1(x, xq, K: int, ncols: int, stream=None) -> None:
    _check(lib().quantize_q8_1(_ptr(x), _ptr(xq), K, ncols, _stream(stream)), "quantize_q8_1")


def quantize_q8_1_planar(x, xq, K: int, ncols: int, stream=None) -> None:
    _check(lib().quantize_q8_1_planar(_ptr(x), _ptr(xq), K, ncols, _stream(stream)), "quantize_q8_1_planar")


def rmsnorm_quantize_q8_1(x, gamma, eps: float, xq, K: int, ncols: int, act_layout: int = 0,
                          stream=None) -> None:
    _check(lib().rmsnorm_quantize_q8_1(_ptr(x), _ptr(gamma), float(eps), _ptr(xq), K, ncols, act_layout,
                                       _stream(stream)), "rmsnorm_quantize_q8_1")


def mmvq_q6k(w, layout: int, xq, out, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmvq_q6k(_ptr(w), layout, _ptr(xq), _ptr(out), rows, K, ncols, _stream(stream)),
           "mmvq_q6k")


def mmq_q6k(w, layout: int, xq, out, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmq_q6k(_ptr(w), layout, _ptr(xq), _ptr(out), rows, K, ncols, _stream(stream)), "mmq_q6k")


def mmvq_q4k(w, xq, out, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmvq_q4k(_ptr(w), _ptr(xq), _ptr(out), rows, K, ncols, _stream(stream)), "mmvq_q4k")


def mmvq_q5k(w, xq, out, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmvq_q5k(_ptr(w), _ptr(xq), _ptr(out), rows, K, ncols, _stream(stream)), "mmvq_q5k")


def repack_q6k_planar(src, dst, rows: int, K: int, stream=None) -> None:
    _check(lib().repack_q6k_planar(_ptr(src), _ptr(dst), rows, K, _stream(stream)), "repack_q6k_planar")


def unpack_q6k_planar(src, dst, rows: int, K: int, stream=None) -> None:
    _check(lib().unpack_q6k_planar(_ptr(src), _ptr(dst), rows, K, _stream(stream)), "unpack_q6k_planar")


def repack_q6k_tiled(src, dst, rows: int, K: int, stream=None) -> None:
    _check(lib().repack_q6k_tiled(_ptr(src), _ptr(dst), rows, K, _stream(stream)), "repack_q6k_tiled")


def unpack_q6k_tiled(src, dst, rows: int, K: int, stream=None) -> None:
    _check(lib().unpack_q6k_tiled(_ptr(src), _ptr(dst), rows, K, _stream(stream)), "unpack_q6k_tiled")


def gather_q6k_rows(src, layout: int, rows: int, K: int, ids, nout: int, dst, stream=None) -> None:
    _check(lib().gather_q6k_rows(_ptr(src), layout, rows, K, _ptr(ids), nout, _ptr(dst), _stream(stream)),
           "gather_q6k_rows")


def mmvq_q6k_argmax_workspace(rows: int, ncols: int) -> int:
    return int(lib().mmvq_q6k_argmax_workspace(rows, ncols))


def mmvq_q6k_argmax(w, layout: int, xq, rows: int, K: int, ncols: int, idx, val, ws, ws_bytes: int,
                    stream=None) -> None:
    _check(lib().mmvq_q6k_argmax(_ptr(w), layout, _ptr(xq), rows, K, ncols, _ptr(idx), _ptr(val), _ptr(ws),
                                 ws_bytes, _stream(stream)), "mmvq_q6k_argmax")


def mmvq_q6k_topk_workspace(rows: int, ncols: int, k: int) -> int:
    return int(lib().mmvq_q6k_topk_workspace(rows, ncols, k))


def mmvq_q6k_topk(w, layout: int, xq, rows: int, K: int, ncols: int, k: int, idx, val, ws, ws_bytes: int,
                  stream=None) -> None:
    _check(lib().mmvq_q6k_topk(_ptr(w), layout, _ptr(xq), rows, K, ncols, k, _ptr(idx), _ptr(val), _ptr(ws),
                               ws_bytes, _stream(stream)), "mmvq_q6k_topk")


def mmvq_q6k_isums(w, layout: int, xq, isums, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmvq_q6k_isums(_ptr(w), layout, _ptr(xq), _ptr(isums), rows, K, ncols, _stream(stream)),
           "mmvq_q6k_isums")


def mmvq_q4k_isums(w, xq, isums, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmvq_q4k_isums(_ptr(w), _ptr(xq), _ptr(isums), rows, K, ncols, _stream(stream)),
           "mmvq_q4k_isums")


def mmvq_q5k_isums(w, xq, isums, rows: int, K: int, ncols: int, stream=None) -> None:
    _check(lib().mmvq_q5k_isums(_ptr(w), _ptr(xq), _ptr(isums), rows, K, ncols, _stream(stream)),
           "mmvq_q5k_isums")


def mmvq_q6k_batch(jobs, layout: int, K: int, stream=None) -> None:
    """jobs: sequence of (w, xq, out, rows, ncols) -- one launch for all."""
    _check(lib().mmvq_q6k_batch(_jobs(jobs), len(jobs), layout, K, _stream(stream)), "mmvq_q6k_batch")


def _jobs(jobs):
    return (Q6kJob * max(1, len(jobs)))(*[Q6kJob(_ptr(w), _ptr(x), _ptr(o), rows, n) for w, x, o, rows, n in jobs])


def mmvq_q4k_batch(jobs, K: int, stream=None) -> None:
    """jobs: sequence of (w, xq, out, rows, ncols) of Q4_K products."""
    _check(lib().mmvq_q4k_batch(_jobs(jobs), len(jobs), K, _stream(stream)), "mmvq_q4k_batch")


def mmvq_q5k_batch(jobs, K: int, stream=None) -> None:
    """jobs: sequence of (w, xq, out, rows, ncols) of Q5_K products."""
    _check(lib().mmvq_q5k_batch(_jobs(jobs), len(jobs), K, _stream(stream)), "mmvq_q5k_batch")


def grouped_expert_mmvq_workspace(E: int, T: int, topk: int, d_model: int, d_ff: int) -> int:
    return int(lib().grouped_expert_mmvq_workspace(E, T, topk, d_model, d_ff))


def grouped_expert_mmvq(w_gate, w_up, w_down, down_layout: int, xq, ids, route_w, out, E: int, T: int,
                        topk: int, d_model: int, d_ff: int, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().grouped_expert_mmvq(_ptr(w_gate), _ptr(w_up), _ptr(w_down), down_layout, _ptr(xq), _ptr(ids),
                                     _ptr(route_w), _ptr(out), E, T, topk, d_model, d_ff, _ptr(ws), ws_bytes,
                                     _stream(stream)), "grouped_expert_mmvq")


def grouped_expert_mmvq_noalloc(w_gate, w_up, w_down, down_layout: int, xq, ids, route_w, out, E: int, T: int,
                                topk: int, d_model: int, d_ff: int, stream=None) -> None:
    _check(lib().grouped_expert_mmvq_noalloc(_ptr(w_gate), _ptr(w_up), _ptr(w_down), down_layout, _ptr(xq),
                                             _ptr(ids), _ptr(route_w), _ptr(out), E, T, topk, d_model, d_ff,
                                             _stream(stream)), "grouped_expert_mmvq_noalloc")


def qmv_stream_read(src, nbytes: int, sink, blocks: int, stream=None) -> None:
    _check(lib().qmv_stream_read(_ptr(src), nbytes, _ptr(sink), blocks, _stream(stream)), "qmv_stream_read")


def moe_workspace_layout(T: int, topk: int, d_model: int, d_ff: int) -> dict:
    """Byte offsets of the workspace regions, as include/qmv.h documents."""
    S = T * topk
    a = lambda x: (x + 255) & ~255  # noqa: E731
    h = a(256 + 16 * S)
    hq = a(h + 4 * S * d_ff)
    y = a(hq + 36 * S * (d_ff // 32))
    return {"S": S, "expert": 256, "count": 256 + 4 * S, "first": 256 + 8 * S, "slot_list": 256 + 12 * S,
            "h": h, "hq": hq, "y": y, "total": a(y + 4 * S * d_model)}

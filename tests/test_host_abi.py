"""C-ABI library checks that need no GPU: the library loads, exports every
symbol include/qmv.h declares, and rejects every invalid argument on the host
(the checks run before any HIP call, so fake pointer values are safe here)."""
import ctypes
import os

import pytest

from quant_mat_vec_amd import qmv

E_INV, E_UNS, E_ALN, E_WS = (qmv.QMV_ERR_INVALID_ARG, qmv.QMV_ERR_UNSUPPORTED,
                             qmv.QMV_ERR_ALIGNMENT, qmv.QMV_ERR_WORKSPACE)
P = 0x7F0000000000          # a fake, 256-byte aligned "device address"; never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qmv.LIB_PATH):
        from quant_mat_vec_amd import build
        build.build(verbose=False)
    return qmv.lib()


def test_exports_every_declared_symbol(L):
    names = qmv.declared_symbols()
    expected = {"quantize_q8_1", "quantize_q8_1_planar", "rmsnorm_quantize_q8_1", "mmvq_q6k", "mmq_q6k", "mmvq_q4k", "mmvq_q5k", "repack_q6k_planar",
                "unpack_q6k_planar", "repack_q6k_tiled", "unpack_q6k_tiled", "gather_q6k_rows", "mmvq_q6k_argmax", "mmvq_q6k_argmax_workspace",
                "mmvq_q6k_isums",
                "mmvq_q4k_isums", "mmvq_q5k_isums",
                "grouped_expert_mmvq", "grouped_expert_mmvq_workspace", "grouped_expert_mmvq_noalloc",
                "mmvq_q6k_batch", "mmvq_q4k_batch", "mmvq_q5k_batch", "mmvq_q6k_topk", "mmvq_q6k_topk_workspace", "qmv_strerror",
                "qmv_last_hip_error", "qmv_stream_read"}
    assert expected <= set(names), set(names) ^ expected
    for n in names:
        assert hasattr(L, n), n


def test_strerror_names_every_code(L):
    for c in (0, -1, -2, -3, -4, -5):
        assert qmv.strerror(c) and "unknown" not in qmv.strerror(c)
    assert "unknown" in qmv.strerror(-99)
    assert L.qmv_last_hip_error() == 0


@pytest.mark.parametrize("name", ["quantize_q8_1", "quantize_q8_1_planar"])
def test_quantize_rejects(L, name):
    q = getattr(L, name)
    assert q(None, P, 256, 1, None) == E_INV
    assert q(P, None, 256, 1, None) == E_INV
    assert q(P, P, 0, 1, None) == E_INV
    assert q(P, P, 256, 0, None) == E_INV
    assert q(P, P, 100, 1, None) == E_UNS
    assert q(P, P, (1 << 20) + 32, 1, None) == E_UNS
    assert q(P, P, 256, 65536, None) == E_UNS
    assert q(P + 2, P, 256, 1, None) == E_ALN
    assert q(P, P + 1, 256, 1, None) == E_ALN


def test_rmsnorm_quantize_rejects(L):
    f = L.rmsnorm_quantize_q8_1

    def call(x=P, g=P, eps=1e-6, xq=P, K=256, n=1, lay=0):
        return f(x, g, eps, xq, K, n, lay, None)

    assert call(x=None) == E_INV and call(g=None) == E_INV and call(xq=None) == E_INV
    assert call(K=0) == E_INV and call(n=0) == E_INV
    assert call(eps=-1.0) == E_INV and call(eps=float("nan")) == E_INV and call(eps=float("inf")) == E_INV
    assert call(K=100) == E_UNS and call(K=(1 << 20) + 32) == E_UNS and call(n=65536) == E_UNS
    assert call(lay=1) == E_UNS and call(lay=qmv.LAYOUT_TILED | qmv.ACT_PLANAR) == E_UNS
    assert call(x=P + 4) == E_ALN and call(g=P + 8) == E_ALN and call(xq=P + 2) == E_ALN


def test_mmq_rejects(L):
    T, XT = qmv.LAYOUT_TILED, qmv.LAYOUT_TILED | qmv.ACT_PLANAR

    def call(w=P, xq=P, out=P, rows=16, K=512, ncols=1, layout=T):
        return L.mmq_q6k(w, layout, xq, out, rows, K, ncols, None)

    assert call(w=None) == E_INV and call(xq=None) == E_INV and call(out=None) == E_INV
    assert call(rows=0) == E_INV and call(K=0) == E_INV
    assert call(K=300) == E_UNS and call(K=1 << 21) == E_UNS and call(rows=1 << 31) == E_UNS
    assert call(ncols=0) == E_UNS and call(ncols=65536) == E_UNS
    # tiled weights only
    for lay in (qmv.LAYOUT_GGUF, qmv.LAYOUT_PLANAR, qmv.LAYOUT_PLANAR | qmv.ACT_PLANAR, 3, -1):
        assert call(layout=lay) == E_UNS, lay
    # the grid bound: (ceil(rows/16) + 32) * ceil(ncols/12) < 2^22
    assert call(rows=16 * ((1 << 22) // 12 - 32), ncols=12 * 13) == E_UNS
    assert call(w=P + 8) == E_ALN and call(xq=P + 2) == E_ALN and call(out=P + 2) == E_ALN
    assert call(layout=XT, xq=P + 4) == E_ALN and call(layout=XT, xq=P + 8) == E_ALN


@pytest.mark.parametrize("name", ["mmvq_q6k", "mmvq_q4k", "mmvq_q5k",
                                  "mmvq_q6k_isums", "mmvq_q4k_isums", "mmvq_q5k_isums"])
def test_mmvq_rejects(L, name):
    fn = getattr(L, name)
    q6 = "q6k" in name

    def call(w=P, xq=P, out=P, rows=16, K=512, ncols=1, layout=qmv.LAYOUT_PLANAR):
        if q6:
            return fn(w, layout, xq, out, rows, K, ncols, None)
        return fn(w, xq, out, rows, K, ncols, None)

    assert call(w=None) == E_INV
    assert call(xq=None) == E_INV
    assert call(out=None) == E_INV
    assert call(rows=0) == E_INV
    assert call(rows=-3) == E_INV
    assert call(K=0) == E_INV
    assert call(K=300) == E_UNS
    assert call(K=1 << 21) == E_UNS
    assert call(rows=1 << 31) == E_UNS
    assert call(ncols=0) == E_UNS
    assert call(ncols=9) == E_UNS
    assert call(xq=P + 2) == E_ALN
    assert call(out=P + 2) == E_ALN
    if q6:
        assert call(layout=3) == E_UNS
        assert call(layout=-1) == E_UNS
        assert call(w=P + 8, layout=qmv.LAYOUT_PLANAR) == E_ALN
        assert call(w=P + 8, layout=qmv.LAYOUT_TILED) == E_ALN
        assert call(K=300, layout=qmv.LAYOUT_TILED) == E_UNS
        assert call(ncols=9, layout=qmv.LAYOUT_TILED) == E_UNS
        assert call(w=P + 2, layout=qmv.LAYOUT_GGUF) == E_ALN
        # column-planar activations: only with the tiled layout, xq 16-byte aligned
        XT = qmv.LAYOUT_TILED | qmv.ACT_PLANAR
        assert call(layout=qmv.LAYOUT_PLANAR | qmv.ACT_PLANAR) == E_UNS
        assert call(layout=qmv.LAYOUT_GGUF | qmv.ACT_PLANAR) == E_UNS
        assert call(layout=3 | qmv.ACT_PLANAR) == E_UNS
        assert call(layout=XT, xq=P + 4) == E_ALN
        assert call(layout=XT, xq=P + 8) == E_ALN
        assert call(layout=XT, w=P + 8) == E_ALN
        assert call(layout=XT, xq=None) == E_INV
        assert call(layout=XT, ncols=9) == E_UNS
    else:
        assert call(w=P + 8) == E_ALN


def test_repack_rejects(L):
    for fn, a_src, a_dst in ((L.repack_q6k_planar, 2, 16), (L.unpack_q6k_planar, 16, 2),
                             (L.repack_q6k_tiled, 2, 16), (L.unpack_q6k_tiled, 16, 2)):
        assert fn(None, P, 4, 256, None) == E_INV
        assert fn(P, None, 4, 256, None) == E_INV
        assert fn(P, P + 4096, 0, 256, None) == E_INV
        assert fn(P, P + 4096, 4, 100, None) == E_UNS
        assert fn(P, P + 832, 4, 256, None) == E_INV            # overlapping buffers
        if a_src > 1:
            assert fn(P + a_src // 2, P + 4096, 4, 256, None) == E_ALN
        assert fn(P, P + 4096 + a_dst // 2, 4, 256, None) == E_ALN


def test_gather_rejects(L):
    f = L.gather_q6k_rows
    assert f(None, 1, 4, 256, P, 2, P + 8192, None) == E_INV
    assert f(P, 1, 4, 256, None, 2, P + 8192, None) == E_INV
    assert f(P, 1, 4, 256, P, 2, None, None) == E_INV
    assert f(P, 1, 0, 256, P, 2, P + 8192, None) == E_INV
    assert f(P, 1, 4, 256, P, 0, P + 8192, None) == E_INV
    assert f(P, 3, 4, 256, P, 2, P + 8192, None) == E_UNS
    assert f(P, 1, 4, 300, P, 2, P + 8192, None) == E_UNS
    assert f(P + 8, 1, 4, 256, P, 2, P + 8192, None) == E_ALN
    assert f(P, 2, 4, 256, P, 2, P + 8200, None) == E_ALN
    assert f(P, 1, 4, 256, P + 2, 2, P + 8192, None) == E_ALN
    assert f(P, 1, 4, 256, P, 2, P + 416, None) == E_INV      # overlapping buffers


def test_argmax_rejects(L):
    f = L.mmvq_q6k_argmax
    TL = qmv.LAYOUT_TILED
    nws = L.mmvq_q6k_argmax_workspace(100, 4)
    assert nws == (7 * 4 * 8 + 255) // 256 * 256 + 256
    assert L.mmvq_q6k_argmax_workspace(0, 4) == 0 and L.mmvq_q6k_argmax_workspace(100, 9) == 0

    def call(w=P, lay=TL, xq=P, rows=100, K=512, n=4, idx=P, val=P, ws=P, wsb=nws):
        return f(w, lay, xq, rows, K, n, idx, val, ws, wsb, None)

    assert call(idx=None) == E_INV
    assert call(val=None) == E_INV
    assert call(ws=None) == E_INV
    assert call(w=None) == E_INV
    assert call(lay=qmv.LAYOUT_PLANAR) == E_UNS
    assert call(lay=qmv.LAYOUT_GGUF) == E_UNS
    assert call(K=300) == E_UNS
    assert call(n=9) == E_UNS
    assert call(w=P + 8) == E_ALN
    assert call(val=P + 2) == E_ALN
    assert call(ws=P + 4) == E_ALN
    assert call(wsb=nws - 1) == E_WS
    XT = TL | qmv.ACT_PLANAR
    assert call(lay=qmv.LAYOUT_PLANAR | qmv.ACT_PLANAR) == E_UNS
    assert call(lay=XT, xq=P + 4) == E_ALN
    assert call(lay=XT, wsb=nws - 1) == E_WS


def test_topk_rejects_and_workspace(L):
    f = L.mmvq_q6k_topk
    TL = qmv.LAYOUT_TILED
    nws = L.mmvq_q6k_topk_workspace(100, 4, 8)
    assert nws == (4 * 100 * 4 + 255) // 256 * 256 + 8 * 1 * 8 * 4
    assert L.mmvq_q6k_topk_workspace(100, 4, 0) == 0 and L.mmvq_q6k_topk_workspace(100, 4, 65) == 0
    assert L.mmvq_q6k_topk_workspace(5, 4, 6) == 0 and L.mmvq_q6k_topk_workspace(100, 9, 4) == 0
    assert L.mmvq_q6k_topk_workspace(4096 * 65, 1, 64) == 0          # 65 chunks x 64 candidates > 4096

    def call(w=P, lay=TL, xq=P, rows=100, K=512, n=4, k=8, idx=P, val=P, ws=P, wsb=nws):
        return f(w, lay, xq, rows, K, n, k, idx, val, ws, wsb, None)

    assert call(idx=None) == E_INV and call(val=None) == E_INV and call(ws=None) == E_INV
    assert call(w=None) == E_INV and call(k=0) == E_INV and call(rows=0) == E_INV
    assert call(k=65) == E_UNS and call(k=101) == E_UNS and call(n=9) == E_UNS and call(K=300) == E_UNS
    assert call(lay=7) == E_UNS and call(lay=qmv.LAYOUT_PLANAR | qmv.ACT_PLANAR) == E_UNS
    assert call(rows=4096 * 65, k=64) == E_UNS
    assert call(w=P + 8) == E_ALN and call(idx=P + 2) == E_ALN and call(ws=P + 64) == E_ALN
    assert call(wsb=nws - 1) == E_WS


def test_moe_rejects_and_workspace(L):
    ws_size = L.grouped_expert_mmvq_workspace(128, 8, 8, 2560, 768)
    lay = qmv.moe_workspace_layout(8, 8, 2560, 768)
    assert ws_size == lay["total"] and ws_size % 256 == 0
    assert lay["h"] >= lay["slot_list"] + 4 * 64
    assert L.grouped_expert_mmvq_workspace(128, 9, 8, 2560, 768) == 0
    assert L.grouped_expert_mmvq_workspace(128, 8, 8, 2500, 768) == 0

    def call(**kw):
        a = dict(wg=P, wu=P, wd=P, lay=1, xq=P, ids=P, rw=P, out=P, E=128, T=8, topk=8, dm=2560,
                 dff=768, ws=P, wsb=ws_size)
        a.update(kw)
        return L.grouped_expert_mmvq(a["wg"], a["wu"], a["wd"], a["lay"], a["xq"], a["ids"], a["rw"],
                                     a["out"], a["E"], a["T"], a["topk"], a["dm"], a["dff"], a["ws"],
                                     a["wsb"], None)

    assert call(wg=None) == E_INV
    assert call(ids=None) == E_INV
    assert call(E=0) == E_INV
    assert call(T=0) == E_INV
    assert call(T=9) == E_UNS
    assert call(topk=9) == E_UNS
    assert call(dm=2500) == E_UNS
    assert call(dff=700) == E_UNS
    assert call(lay=5) == E_UNS
    assert call(lay=qmv.LAYOUT_TILED) == E_UNS     # the expert path takes GGUF or planar
    assert call(ws=None) == E_WS
    assert call(wsb=ws_size - 1) == E_WS
    assert call(ws=P + 64) == E_ALN
    assert call(wg=P + 8) == E_ALN
    assert call(wd=P + 2, lay=0) == E_ALN
    assert call(wd=P + 8, lay=1) == E_ALN


def test_moe_noalloc_rejects(L):
    """The allocation-free MoE entry point: the same argument checks as the
    workspace form, and windows whose workspace exceeds its 4 MiB array."""
    f = L.grouped_expert_mmvq_noalloc

    def call(**kw):
        a = dict(wg=P, wu=P, wd=P, lay=1, xq=P, ids=P, rw=P, out=P, E=128, T=8, topk=8, dm=2560, dff=768)
        a.update(kw)
        return f(a["wg"], a["wu"], a["wd"], a["lay"], a["xq"], a["ids"], a["rw"], a["out"], a["E"], a["T"],
                 a["topk"], a["dm"], a["dff"], None)

    assert call(wg=None) == E_INV and call(out=None) == E_INV and call(E=0) == E_INV
    assert call(T=9) == E_UNS and call(dff=700) == E_UNS and call(lay=qmv.LAYOUT_TILED) == E_UNS
    assert call(wd=P + 8, lay=1) == E_ALN
    assert L.grouped_expert_mmvq_workspace(128, 8, 8, 2560, 16384) > 4 << 20
    assert call(dff=16384) == E_UNS


def test_batch_rejects(L):
    T, XT = qmv.LAYOUT_TILED, qmv.LAYOUT_TILED | qmv.ACT_PLANAR

    def call(jobs, layout=T, K=512, n=None):
        arr = (qmv.Q6kJob * max(1, len(jobs)))(*[qmv.Q6kJob(*j) for j in jobs])
        return L.mmvq_q6k_batch(arr, len(jobs) if n is None else n, layout, K, None)

    ok = (P, P, P, 16, 2)
    assert L.mmvq_q6k_batch(None, 1, T, 512, None) == E_INV
    assert call([ok], n=0) == E_INV
    assert call([ok] * 9) == E_UNS
    assert call([ok], layout=qmv.LAYOUT_PLANAR) == E_UNS and call([ok], layout=qmv.LAYOUT_GGUF) == E_UNS
    assert call([ok], K=300) == E_UNS and call([ok], K=1 << 21) == E_UNS
    assert call([ok, (P, P, P, 16, 9)]) == E_UNS and call([ok, (P, P, P, 16, 0)]) == E_UNS
    assert call([ok, (P, P, P, 0, 2)]) == E_INV and call([ok, (None, P, P, 16, 2)]) == E_INV
    assert call([ok, (P + 8, P, P, 16, 2)]) == E_ALN and call([ok, (P, P, P + 2, 16, 2)]) == E_ALN
    assert call([ok, (P, P + 4, P, 16, 2)], layout=XT) == E_ALN
    half = (1 << 25)
    assert call([(P, P, P, half, 1), (P, P, P, half, 1)]) == E_UNS      # rows summed past the product limit


@pytest.mark.parametrize("name", ["mmvq_q4k_batch", "mmvq_q5k_batch"])
def test_q45_batch_rejects(L, name):
    f = getattr(L, name)

    def call(jobs, K=512, n=None):
        arr = (qmv.Q6kJob * max(1, len(jobs)))(*[qmv.Q6kJob(*j) for j in jobs])
        return f(arr, len(jobs) if n is None else n, K, None)

    ok = (P, P, P, 16, 2)
    assert f(None, 1, 512, None) == E_INV
    assert call([ok], n=0) == E_INV and call([ok], n=-1) == E_INV
    assert call([ok] * 9) == E_UNS
    assert call([ok], K=300) == E_UNS and call([ok], K=1 << 21) == E_UNS and call([ok], K=0) == E_INV
    assert call([ok, (P, P, P, 16, 9)]) == E_UNS and call([ok, (P, P, P, 16, 0)]) == E_UNS
    assert call([ok, (P, P, P, 0, 2)]) == E_INV and call([ok, (None, P, P, 16, 2)]) == E_INV
    assert call([ok, (P, None, P, 16, 2)]) == E_INV and call([ok, (P, P, None, 16, 2)]) == E_INV
    assert call([ok, (P + 8, P, P, 16, 2)]) == E_ALN            # weights 16-byte aligned
    assert call([ok, (P, P + 2, P, 16, 2)]) == E_ALN and call([ok, (P, P, P + 2, 16, 2)]) == E_ALN
    half = (1 << 25)
    assert call([(P, P, P, half, 1), (P, P, P, half, 1)]) == E_UNS      # rows summed past the product limit


def test_stream_read_rejects(L):
    f = L.qmv_stream_read
    assert f(None, 4096, P, 8, None) == E_INV
    assert f(P, 0, P, 8, None) == E_INV
    assert f(P, 4096, P, -1, None) == E_INV
    assert f(P, 4100, P, 8, None) == E_UNS
    assert f(P + 4, 4096, P, 8, None) == E_ALN


def test_binding_raises_on_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(qmv, "LIB_PATH", str(tmp_path / "nope.so"))
    monkeypatch.setattr(qmv, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        qmv.lib()


def test_binding_raises_qmv_error(L):
    with pytest.raises(qmv.QmvError) as ei:
        qmv.mmvq_q6k(P, 1, P, P, 16, 300, 1, stream=0)
    assert ei.value.code == E_UNS


def test_launch_size_limits_rejected_on_host(L):
    """Calls whose launches would exceed 2^32 work-items along x or 65535
    workgroups along y are rejected as unsupported before any HIP call."""
    K20 = 1 << 20
    for q in (L.quantize_q8_1, L.quantize_q8_1_planar):
        # ncols * K / 4 work-items: 16385 columns of 2^20 exceed 2^32
        assert q(P, P, K20, 16385, None) == E_UNS
        assert q(P, P, K20 // 2, 32769, None) == E_UNS
    big = (1 << 26) - 1024 + 1                     # one row past the product limit
    for lay in (qmv.LAYOUT_GGUF, qmv.LAYOUT_PLANAR, qmv.LAYOUT_TILED, qmv.LAYOUT_TILED | qmv.ACT_PLANAR):
        assert L.mmvq_q6k(P, lay, P, P, big, 256, 1, None) == E_UNS
        assert L.mmvq_q6k_isums(P, lay, P, P, big, 256, 1, None) == E_UNS
    assert L.mmvq_q4k(P, P, P, big, 256, 1, None) == E_UNS
    assert L.mmvq_q5k(P, P, P, big, 256, 1, None) == E_UNS
    assert L.mmvq_q4k_isums(P, P, P, big, 256, 8, None) == E_UNS
    assert L.mmq_q6k(P, qmv.LAYOUT_TILED, P, P, big, 256, 1, None) == E_UNS
    assert L.mmvq_q6k_argmax_workspace(big, 1) == 0
    assert L.mmvq_q6k_argmax(P, qmv.LAYOUT_TILED, P, big, 256, 1, P, P, P, 1 << 40, None) == E_UNS
    # conversions: eight work-items per block (2^32 blocks here)
    for fn in (L.repack_q6k_planar, L.repack_q6k_tiled, L.unpack_q6k_planar, L.unpack_q6k_tiled):
        assert fn(P, P + (1 << 41), 1 << 20, K20, None) == E_UNS
    assert L.gather_q6k_rows(P, 1, 4, K20, P, 1 << 20, P + (1 << 41), None) == E_UNS
    # grouped MoE: d_ff = 6144 runs 64 lanes per down row, four rows per
    # workgroup, so d_model = 2^20 needs 262144 workgroups along y
    ws = L.grouped_expert_mmvq_workspace(1, 1, 1, K20, 6144)
    assert ws > 0
    assert L.grouped_expert_mmvq(P, P, P, 1, P, P, P, P, 1, 1, 1, K20, 6144, P, ws, None) == E_UNS
    # streaming read with one step per thread: bytes / 64 work-items
    assert L.qmv_stream_read(P, 1 << 39, P, 0, None) == E_UNS

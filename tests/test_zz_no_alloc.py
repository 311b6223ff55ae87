"""The allocation-free grouped MoE entry point (grouped_expert_mmvq_noalloc),
through the C ABI: its outputs equal grouped_expert_mmvq's (workspace
passed by the caller) bit for bit, on two calls in a row with the second on
a smaller window and smaller matrices (the scratch array keeps the first
call's contents), with planar and GGUF down weights; and the size limit."""
import numpy as np
import pytest
import torch

from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import DEV, canaries_intact, dev, guarded, host, note, planar, quantize

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()                      # fails loudly if the HIP library is missing


def case(seed, E, T, topk, dm, dff):
    g = synth.rng(seed)
    gate, up, down = synth.moe_weights(g, E, dm, dff)
    ids, rw = synth.routing(g, T, E, topk)
    xq, _ = quantize(synth.activations(g, T, dm))
    return dict(E=E, T=T, topk=topk, dm=dm, dff=dff, gd=dev(gate), ud=dev(up), dd=dev(down),
                dp=planar(dev(down), E * dm, dff), ids=dev(ids), rw=dev(rw), xq=xq)


def with_workspace(c, layout):
    wsb = qmv.grouped_expert_mmvq_workspace(c["E"], c["T"], c["topk"], c["dm"], c["dff"])
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device=DEV)
    out = torch.empty(c["T"] * c["dm"], dtype=torch.float32, device=DEV)
    qmv.grouped_expert_mmvq(c["gd"], c["ud"], c["dp"] if layout == qmv.LAYOUT_PLANAR else c["dd"], layout, c["xq"],
                            c["ids"], c["rw"], out, c["E"], c["T"], c["topk"], c["dm"], c["dff"], ws, wsb)
    return host(out)


def without_workspace(c, layout):
    out, buf = guarded(c["T"] * c["dm"])
    qmv.grouped_expert_mmvq_noalloc(c["gd"], c["ud"], c["dp"] if layout == qmv.LAYOUT_PLANAR else c["dd"], layout,
                                    c["xq"], c["ids"], c["rw"], out, c["E"], c["T"], c["topk"], c["dm"], c["dff"])
    assert canaries_intact(buf, c["T"] * c["dm"]), "output guard words overwritten"
    return host(out)


def test_noalloc_equals_workspace_entry_point_two_calls():
    big = case(1900, 128, 8, 8, 2560, 768)        # 64 slots: the three-launch chain
    small = case(1901, 6, 1, 4, 512, 256)         # 4 slots, smaller matrices: fused down + sum (planar)
    for layout in (qmv.LAYOUT_PLANAR, qmv.LAYOUT_GGUF):
        for c in (big, small):
            note(f"grouped_expert_mmvq_noalloc E={c['E']} T={c['T']} topk={c['topk']} "
                 f"d_model={c['dm']} d_ff={c['dff']} layout={layout}")
            got = without_workspace(c, layout)
            ref = with_workspace(c, layout)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"layout {layout}, T={c['T']}"


def test_noalloc_rejects_windows_beyond_its_scratch():
    # d_ff = 16384 at 64 slots needs about 6 MB of workspace: more than the 4 MiB array
    assert qmv.grouped_expert_mmvq_workspace(128, 8, 8, 2560, 16384) > 4 << 20
    assert qmv.grouped_expert_mmvq_workspace(128, 8, 8, 2560, 8192) <= 4 << 20
    L = qmv.lib()
    P = 0x7F0000000000
    rc = L.grouped_expert_mmvq_noalloc(P, P, P, 1, P, P, P, P, 128, 8, 8, 2560, 16384, None)
    assert rc == qmv.QMV_ERR_UNSUPPORTED

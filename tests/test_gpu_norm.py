"""GPU parity of the fused RMSNorm -> Q8_1 quantizer, through the C ABI,
against the CPU oracle (RMSNorm in fp64 rounded to fp32 once, then the
oracle quantizer).

The kernel forms y in fp32 (its sum of squares in a fixed order), so a
code can differ from the oracle's where y/d lies within rounding of a
half-integer.  Bars: every code within one step of the oracle's and at most
one in a thousand different; fp16 d equal or adjacent; s consistent with the
kernel's own codes and d; the column-planar output byte for byte the
permuted block output; exactly representable cases bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from quant_mat_vec_amd import qmv, synth
from tests.gpu_util import DEV, dev, host, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    qmv.lib()


def fused(x, g, eps, act_layout=0):
    ncols, K = x.shape
    xq = torch.empty(ncols * (K // 32) * 36, dtype=torch.uint8, device=DEV)
    qmv.rmsnorm_quantize_q8_1(dev(x), dev(g), eps, xq, K, ncols, act_layout)
    return host(xq).reshape(ncols, K // 32, 36)


def inputs(seed, ncols, K):
    r = synth.rng(seed)
    scale = np.exp(r.uniform(-4, 4, size=(ncols, 1)))          # columns of very different size
    x = (r.standard_normal((ncols, K)) * scale).astype(np.float32)
    g = r.uniform(0.5, 1.5, size=K).astype(np.float32)
    return x, g


@pytest.mark.parametrize("K,ncols", [(2560, 13), (10240, 8), (768, 5), (32, 1), (4096, 64), (992, 3)])
def test_fused_norm_quantize_vs_oracle(K, ncols):
    note(f"rmsnorm_quantize_q8_1 K={K} ncols={ncols}")
    x, g = inputs(1300 + K + ncols, ncols, K)
    eps = float(np.float32(1e-6))
    got = fused(x, g, eps)
    want = orc.rmsnorm_quantize_q8_1(x, g, eps).reshape(ncols, K // 32, 36)
    qg, qw = got[:, :, 4:].view(np.int8).astype(int), want[:, :, 4:].view(np.int8).astype(int)
    diff = np.abs(qg - qw)
    assert diff.max() <= 1, "a code more than one step from the oracle's"
    assert (diff > 0).mean() <= 1e-3, f"{int((diff > 0).sum())} differing codes"
    dg = got[:, :, 0:2].copy().view(np.uint16)[:, :, 0].astype(int)
    dw = want[:, :, 0:2].copy().view(np.uint16)[:, :, 0].astype(int)
    assert np.abs(dg - dw).max() <= 1, "fp16 d more than one unit apart"
    # s = fp16(d32 * sum q): within half an fp16 ulp of s plus the fp16 rounding of d
    d16 = got[:, :, 0:2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    s16 = got[:, :, 2:4].copy().view(np.float16)[:, :, 0].astype(np.float64)
    sq = qg.sum(axis=2)
    ulp = lambda v: np.spacing(np.abs(v).astype(np.float16)).astype(np.float64)  # noqa: E731
    assert np.all(np.abs(s16 - d16 * sq) <= 0.5 * ulp(s16) + 0.5 * np.abs(sq) * ulp(d16) + 1e-30)
    note(f"  {int((diff > 0).sum())} of {diff.size} codes differ by one step")


@pytest.mark.parametrize("K,ncols", [(2560, 13), (768, 4)])
def test_fused_norm_planar_is_permuted_blocks(K, ncols):
    note(f"rmsnorm_quantize_q8_1 column-planar K={K} ncols={ncols}")
    x, g = inputs(1400 + K, ncols, K)
    blocks = fused(x, g, 1e-5).reshape(-1)
    planar = fused(x, g, 1e-5, qmv.ACT_PLANAR).reshape(-1)
    assert np.array_equal(planar, orc.q8_1_to_planar(blocks, K))


def test_fused_norm_exact_cases():
    """Columns whose fp32 arithmetic is exact give the oracle's bytes: a
    constant column (y = 1) and a constant negative column (y = -1) with
    eps = 0, and a column of zeros with eps > 0 (all codes 0, d = s = 0)."""
    note("rmsnorm_quantize_q8_1 exact cases")
    K = 512
    x = np.zeros((2, K), np.float32)
    x[0] = 2.0
    x[1] = -0.125
    g = np.ones(K, np.float32)
    got = fused(x, g, 0.0)
    assert np.array_equal(got, orc.rmsnorm_quantize_q8_1(x, g, 0.0).reshape(2, K // 32, 36))
    assert np.all(got[0, :, 4:].view(np.int8) == 127) and np.all(got[1, :, 4:].view(np.int8) == -127)
    z = np.zeros((1, K), np.float32)
    gz = fused(z, g, 1e-6)
    assert np.array_equal(gz, orc.rmsnorm_quantize_q8_1(z, g, 1e-6).reshape(1, K // 32, 36))
    assert np.all(gz == 0)

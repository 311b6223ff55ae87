"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it draws random block bytes,
fp32 activations and routing tables, nothing more.  Quantizing, decoding and
multiplying are done separately by the GPU library and by the CPU oracle.

Distributions (the workloads' own, with seeded numpy PCG64 streams):
* Q6_K: ql and qh uniform random bytes, the 16 int8 scales uniform in
  [-64, 63], fp16 d = |N(0,1)| * 2e-3 (numpy's round-to-nearest-even cast).
* Q4_K / Q5_K: fp16 d and dmin = |N(0,1)| * 2e-3, the 12 packed scale bytes
  uniform random (so every 6-bit scale and min is uniform in [0, 63]), qs and
  qh uniform random bytes.
* Activations: independent N(0,1) fp32 per column.
* MoE routing: per token, topk distinct expert ids drawn uniformly without
  replacement; route weights = fp32 softmax of topk i.i.d. N(0,1) logits.
"""
from __future__ import annotations

import numpy as np

Q6K_BYTES, Q4K_BYTES, Q5K_BYTES, Q81_BYTES = 210, 144, 176, 36
BLOCK_BYTES = {"q6k": Q6K_BYTES, "q4k": Q4K_BYTES, "q5k": Q5K_BYTES}


def seed_for(config: int, shape: int, ncols: int) -> int:
    """Seed of workload `config`, shape index `shape`, column count `ncols`."""
    return 0x51A00000 + 256 * config + 16 * shape + ncols


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _fp16_scale(g: np.random.Generator, n: int) -> np.ndarray:
    d = (np.abs(g.standard_normal(n)) * 2e-3).astype(np.float16)
    return d.view(np.uint8).reshape(n, 2)


def q6k_blocks(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """GGUF-layout Q6_K matrix, rows x K, as a flat uint8 array."""
    assert K % 256 == 0
    nb = rows * (K // 256)
    blk = np.empty((nb, Q6K_BYTES), np.uint8)
    blk[:, :192] = g.integers(0, 256, size=(nb, 192), dtype=np.uint8)
    blk[:, 192:208] = g.integers(-64, 64, size=(nb, 16), dtype=np.int8).view(np.uint8)
    blk[:, 208:210] = _fp16_scale(g, nb)
    return blk.reshape(-1)


def _q45_blocks(g, rows, K, five):
    assert K % 256 == 0
    nb = rows * (K // 256)
    nbytes = Q5K_BYTES if five else Q4K_BYTES
    blk = np.empty((nb, nbytes), np.uint8)
    blk[:, 0:2] = _fp16_scale(g, nb)
    blk[:, 2:4] = _fp16_scale(g, nb)
    blk[:, 4:] = g.integers(0, 256, size=(nb, nbytes - 4), dtype=np.uint8)
    return blk.reshape(-1)


def q4k_blocks(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    return _q45_blocks(g, rows, K, False)


def q5k_blocks(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    return _q45_blocks(g, rows, K, True)


def blocks(kind: str, g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    return {"q6k": q6k_blocks, "q4k": q4k_blocks, "q5k": q5k_blocks}[kind](g, rows, K)


def activations(g: np.random.Generator, ncols: int, K: int) -> np.ndarray:
    """fp32 [ncols][K], N(0,1)."""
    return g.standard_normal((ncols, K), dtype=np.float32)


def routing(g: np.random.Generator, T: int, E: int, topk: int):
    """(ids int32 [T][topk], weights fp32 [T][topk])."""
    ids = np.stack([g.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    logits = g.standard_normal((T, topk)).astype(np.float32)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.reshape(T, topk), w


def moe_weights(g: np.random.Generator, E: int, d_model: int, d_ff: int):
    """(gate Q4_K [E][d_ff][d_model/256], up likewise, down Q6_K
    [E][d_model][d_ff/256]) as flat uint8 arrays."""
    gate = q4k_blocks(g, E * d_ff, d_model)
    up = q4k_blocks(g, E * d_ff, d_model)
    down = q6k_blocks(g, E * d_model, d_ff)
    return gate, up, down


# --------------------------------------------------------------------------
# Exact-arithmetic inputs: built so that every partial sum of the product is
# exactly representable in fp32, whatever the summation order.
def exact_q6k_blocks(g: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """Q6_K blocks with d in {2^-3, 2^-2, 2^-1, 1} and scales in {-1, 0, 1};
    ql/qh uniform random."""
    assert K % 256 == 0
    nb = rows * (K // 256)
    blk = np.empty((nb, Q6K_BYTES), np.uint8)
    blk[:, :192] = g.integers(0, 256, size=(nb, 192), dtype=np.uint8)
    blk[:, 192:208] = g.integers(-1, 2, size=(nb, 16), dtype=np.int8).view(np.uint8)
    d = np.ldexp(1.0, -g.integers(0, 4, size=nb)).astype(np.float16)
    blk[:, 208:210] = d.view(np.uint8).reshape(nb, 2)
    return blk.reshape(-1)


def exact_q45_blocks(g: np.random.Generator, rows: int, K: int, five: bool) -> np.ndarray:
    """Q4_K/Q5_K blocks with d, dmin in {2^-3 .. 1} and 6-bit scales and mins
    in {0, 1}: the scale bytes are drawn bit by bit so that every decoded 6-bit
    field is 0 or 1 (only bit 0 of each field may be set)."""
    assert K % 256 == 0
    nb = rows * (K // 256)
    nbytes = Q5K_BYTES if five else Q4K_BYTES
    blk = np.empty((nb, nbytes), np.uint8)
    for off in (0, 2):
        d = np.ldexp(1.0, -g.integers(0, 4, size=nb)).astype(np.float16)
        blk[:, off:off + 2] = d.view(np.uint8).reshape(nb, 2)
    # bytes 0..7 of the scale field: bit 0 is the low bit of a j<4 scale/min,
    # bits 6-7 are high bits of j>=4 fields (kept 0); bytes 8..11: the two
    # nibbles are the low bits of j>=4 scale (low nibble) and min (high).
    s = np.zeros((nb, 12), np.uint8)
    s[:, 0:8] = g.integers(0, 2, size=(nb, 8), dtype=np.uint8)
    s[:, 8:12] = (g.integers(0, 2, size=(nb, 4), dtype=np.uint8)
                  | (g.integers(0, 2, size=(nb, 4), dtype=np.uint8) << 4))
    blk[:, 4:16] = s
    blk[:, 16:] = g.integers(0, 256, size=(nb, nbytes - 16), dtype=np.uint8)
    return blk.reshape(-1)


def exact_q8_1(g: np.random.Generator, ncols: int, K: int, qmax: int = 4) -> np.ndarray:
    """Q8_1 blocks built directly: d = 2^-2 (fp16 0x3400), quants uniform in
    [-qmax, qmax], s = fp16 of d * sum (exact here: |sum| <= 128)."""
    nb = K // 32
    q = g.integers(-qmax, qmax + 1, size=(ncols, nb, 32), dtype=np.int8)
    blk = np.empty((ncols, nb, Q81_BYTES), np.uint8)
    blk[..., 0:2] = np.array([0x00, 0x34], np.uint8)
    s = (0.25 * q.astype(np.int32).sum(axis=2)).astype(np.float16)
    blk[..., 2:4] = s.view(np.uint8).reshape(ncols, nb, 2)
    blk[..., 4:] = q.view(np.uint8)
    return blk.reshape(ncols, -1)

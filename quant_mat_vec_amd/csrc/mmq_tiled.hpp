// mmq_tiled.hpp -- the many-column Q6_K product with the weights held in
// registers across column batches (tiled weights, Q8_1 activations as
// blocks or column-planar, rows whose K is exactly one chunk of the tiled
// kernel).
//
// k_mmvq_q6_tiled at N = 16 spends about half of each wave's VALU issue on
// the weight side (plane addresses and loads, code unpack, scale words, the
// K-split sum), which a batch of 16 columns repeats for every batch.  Here
// a workgroup (one 16-row tile, KS waves along K, IT steps each) loads and
// unpacks its weights once and then runs a loop over BPW batches of B
// columns: stage the batch's activation tile in LDS, the matrix-core steps,
// the K-split sum, the stores.  Per column the arithmetic is that of
// tiled_chunk (same products, same order: the fma chain over a step's four
// blocks, then d_w, steps in order, the KS partial sums in wave order), so
// every output is bit-for-bit that of k_mmvq_q6_tiled for the column.
#pragma once

#include "mmvq_tiled.hpp"

namespace qmv {

// Columns per batch, batches per workgroup and the fewest batches for which
// this launch is taken (128 columns; below that the one-batch-per-workgroup
// launch is as fast or faster: 16 columns 9.6 against 10.6 us).  Measured
// at 512 columns, 10240x2560 / 3000x5120: 8 x 8 116 / 76 us, 8 x 4 121 /
// 78 us, 16 x 4 119 / 92 us, 16 x 8 123 us, 16 x 2 145 us, 8 x 16 115 /
// 76 us but slower from 128 to 256 columns and on 2560x10240 (169 against
// 151 us: too few workgroups); the same bits whatever the split.  Eight-column batches halve the LDS tile and the
// staging registers (121 VGPRs: four waves per SIMD).
#ifndef QMV_MMQ_B
#define QMV_MMQ_B 8
#endif
#ifndef QMV_MMQ_BPW
#define QMV_MMQ_BPW 8
#endif
constexpr int kMmqB = QMV_MMQ_B;
constexpr int kMmqBatchesPerWg = QMV_MMQ_BPW, kMmqMinBatches = 128 / QMV_MMQ_B;

template <int B, int KS, int IT, bool XP>
struct MmqCfg {
    static constexpr int NTHR = KS * kWave;
    static constexpr int NCG = B / 4;
    static constexpr int TNB = 4 * KS * IT;            // blocks per column (the whole row)
    static constexpr int QU = 2 * TNB;                 // uint4 of quants per column
    static constexpr int DU = TNB / 4;                 // uint2 of d per column
    static constexpr int QSL = (B * QU + NTHR - 1) / NTHR;
    static constexpr int DSL = (B * DU + NTHR - 1) / NTHR;
    static constexpr int SI = (B * TNB + NTHR - 1) / NTHR;   // Q8_1 blocks per thread
    static constexpr int ZW = 4 * (IT - 1) + 1;        // zero entries (masked lanes)
    static constexpr int XE = B * TNB + ZW;
    // column-planar: entries of 32 B (quants), then fp16 d per block; Q8_1
    // blocks: x0 | x1 (16 B entries each), then d/4 per block (fp32)
    static constexpr size_t TILE = (size_t)XE * 32 + (size_t)B * TNB * (XP ? 2 : 4);
    static constexpr size_t RED = KS > 1 ? (size_t)KS * NCG * kWave * 4 : 0;
    static constexpr size_t LDS = TILE + RED;
};

// grid: 8 * ceil(tiles / 8) * ngrp workgroups; workgroup b takes group
// (b/8) % ngrp of tile 8*((b/8)/ngrp) + b%8 (a tile's groups on one XCD,
// together in time).  Group g covers batches BPW*g .. BPW*g + BPW - 1 of
// nbat.  Requires K == 128 * KS * IT.
template <int B, int KS, int IT, bool XP>
__global__ __launch_bounds__(KS * kWave) void k_mmq_q6_tiled(const void *__restrict__ w, const uint8_t *__restrict__ xq,
                                                             float *__restrict__ out, int64_t rows, int64_t K,
                                                             int nbat) {
    using C = MmqCfg<B, KS, IT, XP>;
    constexpr int TNB = C::TNB, NCG = C::NCG, NTHR = C::NTHR;
    constexpr int XS = XP ? 2 : 1;                     // uint4 per entry in x0 indexing
    extern __shared__ __align__(16) uint8_t lds[];
    Q6Tiled f;
    f.init(w, rows, K);
    const int tid = threadIdx.x, l = tid & (kWave - 1), kg = l >> 4;
    const int ks = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t ntiles = (rows + 15) / 16;
    const int ngrp = (nbat + kMmqBatchesPerWg - 1) / kMmqBatchesPerWg;
    const int64_t j = blockIdx.x >> 3;
    const int grp = (int)(j % ngrp);
    const int64_t tile = (j / ngrp) * 8 + (blockIdx.x & 7);
    if (tile >= ntiles) return;                          // the whole workgroup
    const int R = (int)min((int64_t)16, rows - 16 * tile);
    const int r = l & 15, rr = min(r, R - 1);
    const int64_t row = 16 * tile + r;
    const bool rok = r < R;

    // ---- weight side, once: codes, scale words and d of the wave's steps
    const __amdgpu_buffer_rsrc_t pa = plane_rsrc(f.A + 16 * tile * f.nsb, 16 * R * f.nsb);
    const __amdgpu_buffer_rsrc_t pb = plane_rsrc(f.B + 16 * tile * f.nsb, 8 * R * f.nsb);
    const __amdgpu_buffer_rsrc_t psc = plane_rsrc(f.SC + 16 * tile * (f.nsb / 4), 8 * R * (f.nsb / 4));
    const __amdgpu_buffer_rsrc_t pd = plane_rsrc(f.D + 16 * tile * f.nb, 2 * R * f.nb);
    const uint32_t oa = 16u * (uint32_t)(kg * R + rr), ob = 8u * (uint32_t)(kg * R + rr);
    const uint32_t osc = 8u * (uint32_t)rr, od = 2u * (uint32_t)rr;
    v4i32 W0[IT], W1[IT];
    uint2 sct[IT];
    float dw[IT];
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int z = ks * IT + it, zr = z * R;            // wave-uniform
        const v4u32 va = __builtin_amdgcn_raw_buffer_load_b128(pa, oa, 64 * zr, kNonTemporal);
        const v2u32 vb = __builtin_amdgcn_raw_buffer_load_b64(pb, ob, 32 * zr, kNonTemporal);
        const v2u32 sc = __builtin_amdgcn_raw_buffer_load_b64(psc, osc, 8 * zr, 0);
        const uint32_t dt = __builtin_amdgcn_raw_buffer_load_b16(pd, od, 2 * ((z >> 1) * R), 0);
        Q6Planar::Raw rw;
        rw.a = make_uint4(va.x, va.y, va.z, va.w);
        rw.b = make_uint2(vb.x, vb.y);
        int v[8];
        Q6Planar::codes(rw, v);
        W0[it] = (v4i32){v[0], v[1], v[2], v[3]};
        W1[it] = (v4i32){v[4], v[5], v[6], v[7]};
        sct[it] = make_uint2(sc.x, sc.y);
        // (the 1/4 of the codes 4*(q6-32): on d_w for column-planar
        // activations, on d_a for Q8_1 blocks, as in tiled_chunk)
        dw[it] = XP ? half_to_float(dt) * 0.25f : half_to_float(dt);
    }

    // LDS: quant entries of 32 B (B*TNB, then the zero entries), d per block
    // (fp16, four to a uint2), then the K-split partial sums
    uint4 *x0 = reinterpret_cast<uint4 *>(lds);
    uint4 *x1 = x0 + (XP ? 1 : C::XE);
    uint2 *dh = reinterpret_cast<uint2 *>(x0 + 2 * C::XE);
    float *fd = reinterpret_cast<float *>(x0 + 2 * C::XE);
    float *red = reinterpret_cast<float *>(lds + C::TILE);
    if (tid < C::ZW) {
        x0[XS * (B * TNB + tid)] = make_uint4(0, 0, 0, 0);
        x1[XS * (B * TNB + tid)] = make_uint4(0, 0, 0, 0);
    }
    int xb[NCG];
    {
        const bool am = (l & 3) == kg;
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) xb[cg] = am ? (4 * cg + ((l & 15) >> 2)) * TNB + 4 * ks * IT + kg : B * TNB;
    }
    const uint32_t cstride = (uint32_t)(36 * (K / 32));
    const int b0 = grp * kMmqBatchesPerWg, b1 = min(nbat, b0 + kMmqBatchesPerWg);
#pragma unroll 1
    for (int cb = b0; cb < b1; cb++) {
        // stage the batch's B columns (consecutive in xq).  (Loading the
        // next batch while this one is computed measured slower: 195
        // VGPRs, two waves per SIMD.)
        if constexpr (XP) {
            const __amdgpu_buffer_rsrc_t xr = plane_rsrc(xq + (int64_t)cb * B * cstride, (int64_t)B * cstride);
            v4u32 xv[C::QSL];
            v2u32 dv[C::DSL];
#pragma unroll
            for (int s = 0; s < C::QSL; s++) {
                const int i = min(tid + s * NTHR, B * C::QU - 1), n = i / C::QU, jq = i - n * C::QU;
                xv[s] = __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)n * cstride + 16u * (uint32_t)jq, 0, 0);
            }
#pragma unroll
            for (int s = 0; s < C::DSL; s++) {
                const int i = min(tid + s * NTHR, B * C::DU - 1), n = i / C::DU, k = i - n * C::DU;
                dv[s] = __builtin_amdgcn_raw_buffer_load_b64(xr, (uint32_t)n * cstride + (uint32_t)K + 8u * (uint32_t)k,
                                                             0, 0);
            }
#pragma unroll
            for (int s = 0; s < C::QSL; s++) {
                const int i = tid + s * NTHR;
                if (i < B * C::QU) {
                    const int n = i / C::QU, jq = i - n * C::QU;
                    reinterpret_cast<v4u32 *>(x0)[2 * n * TNB + jq] = xv[s];
                }
            }
#pragma unroll
            for (int s = 0; s < C::DSL; s++) {
                const int i = tid + s * NTHR;
                if (i < B * C::DU) {
                    const int n = i / C::DU, k = i - n * C::DU;
                    reinterpret_cast<v2u32 *>(dh)[n * (TNB / 4) + k] = dv[s];
                }
            }
        } else {
            // Q8_1 blocks: block b of column n is block n*K/32 + b of the batch
            const uint8_t *xb8 = xq + (int64_t)cb * B * cstride;
            ActRaw ar[C::SI];
#pragma unroll
            for (int s = 0; s < C::SI; s++) {
                const int i = min(tid + s * NTHR, B * TNB - 1), n = i / TNB, b = i - n * TNB;
                act_load(ar[s], xb8, (int64_t)n * (K / 32) + b);
            }
#pragma unroll
            for (int s = 0; s < C::SI; s++) {
                const int i = tid + s * NTHR;
                if (i < B * TNB) {
                    x0[i] = make_uint4(ar[s].w[1], ar[s].w[2], ar[s].w[3], ar[s].w[4]);
                    x1[i] = make_uint4(ar[s].w[5], ar[s].w[6], ar[s].w[7], ar[s].w[8]);
                    fd[i] = half_to_float(ar[s].w[0]) * 0.25f;    // the codes are 4 * (q6 - 32)
                }
            }
        }
        lds_barrier();

        float acc[NCG];
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) acc[cg] = 0.0f;
#pragma unroll
        for (int it = 0; it < IT; it++) {
            const int zt = 4 * (ks * IT + it);
            int sl[4], sh[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t word = i < 2 ? sct[it].x : sct[it].y;
                sl[i] = sext8(word, 2 * (i & 1));
                sh[i] = sext8(word, 2 * (i & 1) + 1);
            }
#pragma unroll
            for (int cg = 0; cg < NCG; cg++) {
                const int idx = xb[cg] + 4 * it;
                const uint4 X0 = x0[XS * idx], X1 = x1[XS * idx];
                const v4i32 A0 = {(int)X0.x, (int)X0.y, (int)X0.z, (int)X0.w};
                const v4i32 A1 = {(int)X1.x, (int)X1.y, (int)X1.z, (int)X1.w};
                const v4i32 Z = {0, 0, 0, 0};
                const v4i32 D0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, W0[it], Z, 0, 0, 0);
                const v4i32 D1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, W1[it], Z, 0, 0, 0);
                const int no = 4 * cg + kg;
                float dxa[4];
                if constexpr (XP) {
                    const uint2 h = dh[(no * TNB + zt) / 4];
                    dxa[0] = half_to_float(h.x);
                    dxa[1] = half_to_float(h.x >> 16);
                    dxa[2] = half_to_float(h.y);
                    dxa[3] = half_to_float(h.y >> 16);
                } else {
                    const float4 dx = *reinterpret_cast<const float4 *>(fd + no * TNB + zt);
                    dxa[0] = dx.x;
                    dxa[1] = dx.y;
                    dxa[2] = dx.z;
                    dxa[3] = dx.w;
                }
                int I[4];
#pragma unroll
                for (int i = 0; i < 4; i++) I[i] = __mul24(sl[i], D0[i]) + __mul24(sh[i], D1[i]);
                float t = __builtin_fmaf(dxa[0], (float)I[0], 0.0f);
#pragma unroll
                for (int i = 1; i < 4; i++) t = __builtin_fmaf(dxa[i], (float)I[i], t);
                acc[cg] = __builtin_fmaf(dw[it], t, acc[cg]);
            }
        }
        float *ob_ = out + (int64_t)cb * B * rows;
        if constexpr (KS > 1) {
#pragma unroll
            for (int cg = 0; cg < NCG; cg++) red[(ks * NCG + cg) * kWave + l] = acc[cg];
        }
        // (also: every wave is past its reads of this batch's tile, so the
        // next batch may be staged)
        lds_barrier();
        if (ks == 0) {
#pragma unroll
            for (int cg = 0; cg < NCG; cg++) {
                float s = acc[cg];
                if constexpr (KS > 1) {
                    s = red[cg * kWave + l];
#pragma unroll
                    for (int k = 1; k < KS; k++) s += red[(k * NCG + cg) * kWave + l];
                }
                if (rok) ob_[(int64_t)(4 * cg + kg) * rows + row] = s;
            }
        }
    }
}

template <int B, int KS, int IT, bool XP>
hipError_t launch_mmq_ws_cfg(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int nbat,
                             hipStream_t s) {
    using C = MmqCfg<B, KS, IT, XP>;
    const int64_t ntiles = (rows + 15) / 16;
    const int64_t ngrp = (nbat + kMmqBatchesPerWg - 1) / kMmqBatchesPerWg;
    const int64_t grid = 8 * ((ntiles + 7) / 8) * ngrp;
    if (grid * C::NTHR > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    const hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_mmq_q6_tiled<B, KS, IT, XP>), C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_mmq_q6_tiled<B, KS, IT, XP>), dim3((unsigned)grid), dim3(C::NTHR), C::LDS, s, w,
                       reinterpret_cast<const uint8_t *>(xq), out, rows, K, nbat);
    return hipGetLastError();
}

// The batch width of the weights-stationary launch for K, ncols and the
// activation layout (0: K is not one whole chunk of four, eight or sixteen
// waves, or too few columns; use the batched tiled launch).  The same waves
// along K as launch_tiled_n, so the same sums.  (Sixteen waves with Q8_1
// blocks would spill at 128 VGPRs: column-planar only there.)
inline int mmq_ws_batch_cols(int64_t K, int64_t ncols, bool xp) {
    const bool one_chunk = K == 128 * 4 * 5 || K == 128 * 8 * 5 || (xp && K == 128 * 16 * 5);
    return one_chunk && ncols / kMmqB >= kMmqMinBatches ? kMmqB : 0;
}

template <bool XP>
hipError_t launch_mmq_ws(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int nbat,
                         hipStream_t s) {
    if (K == 128 * 4 * 5) return launch_mmq_ws_cfg<kMmqB, 4, 5, XP>(w, xq, out, rows, K, nbat, s);
    if (K == 128 * 8 * 5) return launch_mmq_ws_cfg<kMmqB, 8, 5, XP>(w, xq, out, rows, K, nbat, s);
    if constexpr (XP) return launch_mmq_ws_cfg<kMmqB, 16, 5, XP>(w, xq, out, rows, K, nbat, s);
    return hipErrorInvalidValue;                       // (not chosen: see mmq_ws_batch_cols)
}

}  // namespace qmv

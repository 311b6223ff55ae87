// mmvq_tiled.hpp -- Q6_K MMVQ on the int8 matrix cores, tiled weight layout.
//
// The integer part of the Q6_K x Q8_1 dot product (per 16-weight scale
// group, the sum of code x quant) comes from v_mfma_i32_16x16x64_i8; the
// scales are then applied on the vector ALU per sub-block, as in the dot4
// kernels, so every integer partial sum is the same number.
//
// Mapping (one wave, one 16-row tile, one step z of four sub-blocks 4z..4z+3):
//   B operand (weights): lane l holds row l%16 of the tile, sub-block
//     4z + l/16, half h (16 codes); with the tiled layout the 64 lanes of a
//     load instruction read one contiguous kilobyte.
//   A operand (activations): row r' = l%16 of A is the pair (column
//     n = 4cg + r'/4, sub-block 4z + r'%4); lane l holds the 16 quants of its
//     k-group (sub-block 4z + l/16, half h) when that sub-block is r'%4 and
//     reads a zero entry otherwise, so output (r', row) sums only its own
//     scale group.  (The 16x16x64 operands share one k order for A and B:
//     lane l carries k-group l/16 in both.)
//   Result: lane l gets, for tile row l%16 and column 4cg + l/16, the four
//     half-sub-block sums of sub-blocks 4z..4z+3 in its four registers.
// The two halves (codes 0-15, 16-31) take one MFMA each per group of four
// columns.  A workgroup holds RTW row tiles x KS waves along K; the KS
// partial sums of a row are added through LDS in wave order at the end.
#pragma once

#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace qmv {

typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

// Cache-policy bit of a buffer load: non-temporal.  The code planes are read
// once per product, so they are streamed past the caches (measured ~0.1 us
// faster per launch at eight columns than the default policy); the scales
// and d keep the default.  (The batched product in its chunked form
// measured the same with the default policy; in the streamed form, three
// 10240x2560 products, the default policy took 13.46-13.69 against
// 12.23-12.56 us per launch.)
constexpr int kNonTemporal = 2;

// Buffer resource for `bytes` bytes at `base` (raw, unformatted dword
// access; reads past the end return zero).  Loads through it take a lane
// offset in a vector register and a wave-uniform offset in a scalar one, so
// a step's address costs no vector instruction.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Weight planes of the tiled layout (see repack_q6k_tiled): per 16-row tile
// (the last one R rows high) entries are ordered [position][row of tile].
struct Q6Tiled {
    const uint4 *A;        // 16 B per (row, sub-block)
    const uint2 *B;        // 8 B per (row, sub-block)
    const uint2 *SC;       // 8 B per (row, four sub-blocks): their scale pairs
    const uint16_t *D;     // 2 B per (row, block)
    int64_t nsb, nb;       // sub-blocks and blocks per row

    __device__ __forceinline__ void init(const void *w, int64_t rows, int64_t K) {
        const uint8_t *base = reinterpret_cast<const uint8_t *>(w);
        nb = K / 256;
        nsb = K / 32;
        const int64_t NB = rows * nb;
        A = reinterpret_cast<const uint4 *>(base);
        B = reinterpret_cast<const uint2 *>(base + 128 * NB);
        SC = reinterpret_cast<const uint2 *>(base + 192 * NB);
        D = reinterpret_cast<const uint16_t *>(base + 208 * NB);
    }
};

// Weight steps whose code-plane loads are issued before the activation tile
// is stored (the rest follow it): measured best at two, and at three with
// eight or more waves along K (of 1, 2, 3 and all five; 2560x10240:
// 0.05-0.1 us faster than two).  Re-measured in the batched launch of three
// 10240x2560 products (8, 4, 1 columns): 1, 3 and all five steps, and
// per-wave staging with four waves along K, all within -0.1..+0.6 us of two.
constexpr int kTiledPre = 2, kTiledPreLong = 3;


template <int N, int KS, int RTW, int IT, bool XP = false>
struct TiledCfg {
    static constexpr int W = KS * RTW;                 // waves per workgroup
    static constexpr int NTHR = W * kWave;
    static constexpr int NCG = (N + 3) / 4;            // column groups of four
    static constexpr int CZ = KS * IT;                 // steps per chunk
    static constexpr int TNB = 4 * CZ;                 // tile blocks per column
    static constexpr int SI = (N * TNB + NTHR - 1) / NTHR;
    // Wave tiles: with one row tile per workgroup the KS waves read disjoint
    // steps, so each wave can stage only its own 4*IT blocks per column and
    // skip the workgroup barrier (a wave's LDS accesses execute in order).
    // Measured (graph replays, rotated weights): 0.1-0.3 us faster with 16
    // waves along K (2560x10240), 0.1-0.2 us slower with four (10240x2560
    // at N = 4, 8), so only from eight waves on.
    static constexpr bool WT = RTW == 1 && KS >= 8;
    static constexpr int WB = 4 * IT;                  // blocks per column of one wave
    static constexpr int SL = WT ? (N * WB + kWave - 1) / kWave : SI;   // load slots per lane
    // Shared scale loads: the scales and d of a wave's steps in three loads
    // instead of two per step -- lane (row r, k-group kg) loads the entry of
    // step z0 + kg (a second load: z0 + 4 + kg) and of block z0/2 + kg, and
    // each step takes its row's entry from lane r + 16*j with a lane shuffle.
    // Measured (graph replays): 0.17-0.24 us faster with 16 waves along K
    // (2560x10240), within +-0.03 us at N = 1, 8 but 0.14 us slower at N = 4
    // with four (10240x2560), so only from eight waves on.
    static constexpr bool SCS = KS >= 8;
    // d alone shared the same way (one load instead of five): with four
    // waves along K 0.11 us faster at N = 8 and 0.1 us slower at N = 1, 4
    // (10240x2560).  The values, and so every output bit, are the same
    // either way.
    static constexpr bool DS = SCS || N >= 8;
    // XP: per column, 2 uint4 of quants and a quarter uint2 of d per block
    static constexpr int SLOTW = WT ? kWave : NTHR;    // threads sharing the staging
    static constexpr int QU = 2 * (WT ? WB : TNB);     // quant uint4 per column staged by them
    static constexpr int DU = (WT ? WB : TNB) / 4;     // uint2 of d per column
    static constexpr int QSL = (N * QU + SLOTW - 1) / SLOTW;
    static constexpr int DSL = (N * DU + SLOTW - 1) / SLOTW;
    // zero entries after each quant array: a masked lane reads entry
    // N*TNB + 4*it at step it, so its LDS offset follows the step like the
    // others' and the step's part of every address is an immediate
    static constexpr int ZW = 4 * (IT - 1) + 1;
    static constexpr int XE = N * TNB + ZW;            // entries per quant array
    // Q8_1 blocks: x0 | zeros | x1 | zeros (uint4) and d/4 per block
    // (float).  Column-planar activations (XP): quant entries of 32 B (both
    // halves) with the zero entries after them, then d per block (fp16).
    static constexpr size_t TILE = XP ? (size_t)XE * 32 + (size_t)N * TNB * 2
                                      : (size_t)XE * 32 + (size_t)N * TNB * 4;
    static constexpr size_t RED = KS > 1 ? (size_t)W * NCG * kWave * 4 : 0;
    static constexpr size_t LDS = TILE > RED ? TILE : RED;
    static constexpr int PRE = (KS >= 8 ? kTiledPreLong : kTiledPre) < IT ? (KS >= 8 ? kTiledPreLong : kTiledPre) : IT;
};

// Position of a lane in the tiled planes: one buffer resource per plane over
// the wave's tile (wave-uniform, in scalar registers), the tile height R and
// fixed 32-bit lane offsets; a step adds only a scalar offset.  xb[cg]: the
// lane's LDS entry for step 0 of column group cg (the zero entries for a
// masked lane); step it reads entry xb[cg] + 4*it.
template <int NCG>
struct TiledLane {
    __amdgpu_buffer_rsrc_t a, b, sc, d;   // planes A, B, SC, D of the tile
    int R;                                // rows of the tile: entry stride between positions
    uint32_t oa, ob, osc, od;             // lane byte offsets: (row, k-group) in A/B, row in SC/D
    int xb[NCG];
};

// The arithmetic of one step of four sub-blocks for one wave: the codes of
// its plane pieces (wa, wb), the four sub-blocks' scale bytes (sct) and the
// block's d (dt), against the activation tile in LDS (lane entry xb[cg] +
// 4*it; zt = the step's first tile block) -- two matrix-core products per
// column group, then per sub-block the scales, d_a and d_w on the vector
// ALU.  Accumulates into acc (DUMP: writes the per-sub-block sums of step
// z instead).  Every product path of the tiled layout runs its steps through
// this function, so a column's sum is the same sequence of operations in
// each.
template <int N, int NCG, int TNB, int IT, bool DUMP, bool XP>
__device__ __forceinline__ void tiled_step(uint4 wa, uint2 wb, uint2 sct, uint32_t dt, const int (&xb)[NCG], int it,
                                           int zt, uint8_t *lds, int kg, const MmvqArgs &a, int64_t row, bool rok,
                                           int z, float (&acc)[NCG]) {
    constexpr int XE = N * TNB + 4 * (IT - 1) + 1;  // entries per quant array (the zero entries included)
    const uint4 *x0 = reinterpret_cast<const uint4 *>(lds);
    const uint4 *x1 = x0 + (XP ? 1 : XE);
    constexpr int XS = XP ? 2 : 1;                     // uint4 per entry in x0/x1 indexing
    const float *fd = reinterpret_cast<const float *>(x0 + 2 * XE);
    const uint2 *dh = reinterpret_cast<const uint2 *>(x0 + 2 * XE);
    Q6Planar::Raw r;
    r.a = wa;
    r.b = wb;
    int v[8];
    Q6Planar::codes(r, v);
    const v4i32 W0 = {v[0], v[1], v[2], v[3]}, W1 = {v[4], v[5], v[6], v[7]};
    int sl[4], sh[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t word = i < 2 ? sct.x : sct.y;
        sl[i] = sext8(word, 2 * (i & 1));
        sh[i] = sext8(word, 2 * (i & 1) + 1);
    }
    // (XP: the 1/4 of the codes 4*(q6-32) is taken on d_w instead of d_a,
    // a power of two, so every product and sum is the same number)
    const float dw = XP ? half_to_float(dt) * 0.25f : half_to_float(dt);
    v4i32 D0[NCG], D1[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; cg++) {
        const int idx = xb[cg] + 4 * it;
        const uint4 X0 = x0[XS * idx], X1 = x1[XS * idx];
        const v4i32 A0 = {(int)X0.x, (int)X0.y, (int)X0.z, (int)X0.w};
        const v4i32 A1 = {(int)X1.x, (int)X1.y, (int)X1.z, (int)X1.w};
        const v4i32 Z = {0, 0, 0, 0};
        D0[cg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, W0, Z, 0, 0, 0);
        D1[cg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, W1, Z, 0, 0, 0);
    }
#pragma unroll
    for (int cg = 0; cg < NCG; cg++) {
        const int no = 4 * cg + kg;            // this lane's output column
        float dxa[4];
        if constexpr (XP) {
            const uint2 h = dh[(min(no, N - 1) * TNB + zt) / 4];
            dxa[0] = half_to_float(h.x);
            dxa[1] = half_to_float(h.x >> 16);
            dxa[2] = half_to_float(h.y);
            dxa[3] = half_to_float(h.y >> 16);
        } else {
            const float4 dx = *reinterpret_cast<const float4 *>(fd + min(no, N - 1) * TNB + zt);
            dxa[0] = dx.x;
            dxa[1] = dx.y;
            dxa[2] = dx.z;
            dxa[3] = dx.w;
        }
        int I[4];
#pragma unroll
        for (int i = 0; i < 4; i++) I[i] = __mul24(sl[i], D0[cg][i]) + __mul24(sh[i], D1[cg][i]);   // 4 * isum
        if constexpr (DUMP) {
            if (rok && no < N) {
                const int64_t nsb = a.K / 32;
                int32_t *dp = a.dump + ((int64_t)no * a.rows + row) * nsb + 4 * (int64_t)z;
#pragma unroll
                for (int i = 0; i < 4; i++) dp[i] = I[i] >> 2;
            }
        } else {
            // (an fma with +0 is the product: d_a >= 0, so no -0 arises;
            // the fp16 d_a of column-planar tiles then feeds the fma
            // without a conversion)
            float t = __builtin_fmaf(dxa[0], (float)I[0], 0.0f);
#pragma unroll
            for (int i = 1; i < 4; i++) t = __builtin_fmaf(dxa[i], (float)I[i], t);
            acc[cg] = __builtin_fmaf(dw, t, acc[cg]);
        }
    }
}

// One chunk of CZ steps starting at step zc0: wave ks of the row tile takes
// steps zc0 + ks*IT + it.  FULL: all steps exist (no clamping).
template <bool FULL, int N, int KS, int RTW, int IT, bool DUMP, bool XP>
__device__ __forceinline__ void tiled_chunk(const Q6Tiled &f, const TiledLane<TiledCfg<N, KS, RTW, IT>::NCG> &tl,
                                            const MmvqArgs &a, uint8_t *lds,
                                            int zc0, int ZS, int64_t row, bool rok,
                                            float (&acc)[TiledCfg<N, KS, RTW, IT>::NCG]) {
    using C = TiledCfg<N, KS, RTW, IT, XP>;
    constexpr int TNB = C::TNB, NTHR = C::NTHR;
    const int tid = threadIdx.x, l = tid & (kWave - 1), kg = l >> 4;
    const int ks = __builtin_amdgcn_readfirstlane(tid / kWave) % KS;    // wave-uniform
    const int64_t nsb = f.nsb;
    const int nblk = FULL ? TNB : min(TNB, (int)(nsb - 4 * (int64_t)zc0));

    // activation loads first (loads retire in order: the tile can be stored
    // while the weight loads behind it are still in flight).  Slot s of the
    // lane is block b of column n; own_slot gives both and whether the slot
    // exists.
    auto own_slot = [&](int s, int &n, int &b) -> bool {
        int i, lim;
        if constexpr (C::WT) {
            i = l + s * kWave;
            lim = N * C::WB;
            n = min(i, lim - 1) / C::WB;
            b = 4 * ks * IT + (min(i, lim - 1) - n * C::WB);
        } else {
            i = tid + s * NTHR;
            lim = N * TNB;
            n = min(i, lim - 1) / TNB;
            b = min(i, lim - 1) - n * TNB;
        }
        return i < lim && (FULL || b < nblk);
    };
    // column-planar activations: column n's quants are K bytes at
    // 36*xcol_of(n), its d values (fp16) follow them.  Quant slot s of the
    // lane is uint4 j of column n's run for this chunk (two per block), d
    // slot s is uint2 k (four blocks).
    const int st = C::WT ? l : tid;
    auto quant_slot = [&](int s, int &n, int &j) -> bool {
        const int i = st + s * C::SLOTW, lim = N * C::QU, ic = min(i, lim - 1);
        n = ic / C::QU;
        j = ic - n * C::QU + (C::WT ? 8 * ks * IT : 0);
        return i < lim && (FULL || j < 2 * nblk);
    };
    auto d_slot = [&](int s, int &n, int &k) -> bool {
        const int i = st + s * C::SLOTW, lim = N * C::DU, ic = min(i, lim - 1);
        n = ic / C::DU;
        k = ic - n * C::DU + (C::WT ? ks * IT : 0);
        return i < lim && (FULL || 4 * k < nblk);
    };
    ActRaw ar[XP ? 1 : C::SL];
    v4u32 xv[XP ? C::QSL : 1];
    v2u32 dv[XP ? C::DSL : 1];
    if constexpr (XP) {
        // the N columns are consecutive (the tiled launch passes them in
        // order): one buffer over them, lane offsets within it, the chunk's
        // offset in a scalar register
        const uint32_t cstride = (uint32_t)(36 * (a.K / 32));
        const __amdgpu_buffer_rsrc_t xr = plane_rsrc(a.xq, (int64_t)N * cstride);
#pragma unroll
        for (int s = 0; s < C::QSL; s++) {
            int n, j;
            quant_slot(s, n, j);
            const uint32_t off = (uint32_t)n * cstride + 16u * (uint32_t)(FULL ? j : min(j, 2 * nblk - 1));
            xv[s] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 128 * zc0, 0);
        }
#pragma unroll
        for (int s = 0; s < C::DSL; s++) {
            int n, k;
            d_slot(s, n, k);
            const uint32_t off = (uint32_t)n * cstride + (uint32_t)a.K + 8u * (uint32_t)(FULL ? k : min(k, nblk / 4 - 1));
            dv[s] = __builtin_amdgcn_raw_buffer_load_b64(xr, off, 8 * zc0, 0);
        }
    } else {
#pragma unroll
        for (int s = 0; s < C::SL; s++) {
            int n, b;
            own_slot(s, n, b);
            act_load(ar[s], a.xq, xcol_of<N>(a, n) + 4 * (int64_t)zc0 + (FULL ? b : min(b, nblk - 1)));
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // weight loads: scales and d of every step, then the code planes of the
    // first PRE steps; the rest after the tile is stored
    uint4 wa[IT];
    uint2 wb[IT], wsc[C::SCS ? 1 : IT];
    uint32_t wd[C::DS ? 1 : IT];
    int zs[IT];
#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int z = zc0 + ks * IT + it;
        zs[it] = FULL ? z : min(z, ZS - 1);
    }
    static_assert(!C::SCS || IT <= 7, "shared scale loads cover seven steps");
    const int z0 = zs[0], rr = min(l & 15, tl.R - 1);
    v2u32 scA = {0u, 0u}, scB = {0u, 0u};
    uint32_t dsh = 0;
    // (entries past the tile's planes read as zero and are never used)
    if constexpr (C::DS) dsh = __builtin_amdgcn_raw_buffer_load_b16(tl.d, tl.ob >> 2, 2 * ((z0 >> 1) * tl.R), 0);
    if constexpr (C::SCS) {
        scA = __builtin_amdgcn_raw_buffer_load_b64(tl.sc, tl.ob, 8 * z0 * tl.R, 0);
        if constexpr (IT > 4) scB = __builtin_amdgcn_raw_buffer_load_b64(tl.sc, tl.ob, 8 * (z0 + 4) * tl.R, 0);
    } else {
#pragma unroll
        for (int it = 0; it < IT; it++) {
            const int zr = zs[it] * tl.R;                          // wave-uniform
            const v2u32 sc = __builtin_amdgcn_raw_buffer_load_b64(tl.sc, tl.osc, 8 * zr, 0);
            wsc[it] = make_uint2(sc.x, sc.y);
            if constexpr (!C::DS)
                wd[it] = __builtin_amdgcn_raw_buffer_load_b16(tl.d, tl.od, 2 * ((zs[it] >> 1) * tl.R), 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    auto load_ab = [&](auto lo_c, auto hi_c) {
        constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
#pragma unroll
        for (int it = LO; it < HI; it++) {
            const int zr = zs[it] * tl.R;                          // wave-uniform
            const v4u32 va = __builtin_amdgcn_raw_buffer_load_b128(tl.a, tl.oa, 64 * zr, kNonTemporal);
            const v2u32 vb = __builtin_amdgcn_raw_buffer_load_b64(tl.b, tl.ob, 32 * zr, kNonTemporal);
            wa[it] = make_uint4(va.x, va.y, va.z, va.w);
            wb[it] = make_uint2(vb.x, vb.y);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    load_ab(std::integral_constant<int, 0>{}, std::integral_constant<int, C::PRE>{});

    // stage the tile.  Q8_1 blocks: x0 (N*TNB entries + ZW zero entries), x1
    // (the same), fd.  XP: q (entry e = uint4 2e, 2e+1; N*TNB entries + ZW
    // zero entries), then dh (fp16 d per block, four to a uint2).
    uint4 *x0 = reinterpret_cast<uint4 *>(lds);
    uint4 *x1 = x0 + (XP ? 1 : C::XE);
    constexpr int XS = XP ? 2 : 1;                     // uint4 per entry in x0/x1 indexing
    float *fd = reinterpret_cast<float *>(x0 + 2 * C::XE);
    uint2 *dh = reinterpret_cast<uint2 *>(x0 + 2 * C::XE);
    // (with wave tiles every wave writes the zero entries itself: the same
    // values, and then its own reads follow its own writes)
    if (st < C::ZW) {
        x0[XS * (N * TNB + st)] = make_uint4(0, 0, 0, 0);
        x1[XS * (N * TNB + st)] = make_uint4(0, 0, 0, 0);
    }
    if constexpr (XP) {
#pragma unroll
        for (int s = 0; s < C::QSL; s++) {
            int n, j;
            if (quant_slot(s, n, j)) reinterpret_cast<v4u32 *>(x0)[2 * n * TNB + j] = xv[s];
        }
#pragma unroll
        for (int s = 0; s < C::DSL; s++) {
            int n, k;
            if (d_slot(s, n, k)) reinterpret_cast<v2u32 *>(dh)[n * (TNB / 4) + k] = dv[s];
        }
    } else {
#pragma unroll
        for (int s = 0; s < C::SL; s++) {
            int n, b;
            if (own_slot(s, n, b)) {
                const int i = n * TNB + b;
                x0[i] = make_uint4(ar[s].w[1], ar[s].w[2], ar[s].w[3], ar[s].w[4]);
                x1[i] = make_uint4(ar[s].w[5], ar[s].w[6], ar[s].w[7], ar[s].w[8]);
                fd[i] = half_to_float(ar[s].w[0]) * 0.25f;    // the codes are 4 * (q6 - 32)
            }
        }
    }
    if constexpr (C::WT) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {
        lds_barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    load_ab(std::integral_constant<int, C::PRE>{}, std::integral_constant<int, IT>{});

#pragma unroll
    for (int it = 0; it < IT; it++) {
        const int z = zc0 + ks * IT + it;
        if (!FULL && z >= ZS) break;
        uint2 sct;
        uint32_t dt;
        if constexpr (C::SCS) {
            const int dz = zs[it] - z0;                            // wave-uniform, 0..IT-1
            const v2u32 src = dz < 4 ? scA : scB;
            const int from = rr + 16 * (dz & 3);
            sct = make_uint2((uint32_t)__shfl((int)src.x, from), (uint32_t)__shfl((int)src.y, from));
        } else {
            sct = wsc[it];
        }
        if constexpr (C::DS)
            dt = (uint32_t)__shfl((int)dsh, rr + 16 * ((zs[it] >> 1) - (z0 >> 1)));
        else
            dt = wd[it];
        tiled_step<N, C::NCG, TNB, IT, DUMP, XP>(wa[it], wb[it], sct, dt, tl.xb, it, 4 * (z - zc0), lds, kg, a, row,
                                                 rok, z, acc);
    }
}

// Greedy-argmax key of an output: the float's bits made order-preserving as
// an unsigned integer (-0 taken as +0) above the complement of the row, so
// the largest key is the largest value and, among equal values, the lowest
// row.
__device__ __forceinline__ uint64_t argmax_key(float v, int64_t row) {
    uint32_t b = __float_as_uint(v + 0.0f);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)row);
}

// AMAX: instead of the outputs, each row tile writes, per column n, the
// largest argmax_key over its rows to keys[n * ntiles + tile] (out is then
// a uint64 array of N * ceil(rows/16) keys).
//
// More than eight columns (N = 12 or 16): the batched product.  The grid
// covers every row workgroup once per batch of N consecutive columns, and
// workgroup b takes batch (b/8) % nbat of row workgroup 8*((b/8)/nbat) +
// b%8: workgroups are handed to the eight XCDs in turn, so the batches of
// one row workgroup run on one XCD close together in time and read its
// weights from that XCD's L2 after the first.  Every column goes through the
// same arithmetic as in a product of eight or fewer columns.
// One workgroup of the tiled product: row workgroup wg (RTW tiles of 16
// rows, KS waves along K each), the N columns at a.xq; outputs to out (or
// keys, or integer sums to a.dump).
template <int N, int KS, int RTW, int IT, bool DUMP, bool AMAX, bool XP>
__device__ __forceinline__ void tiled_workgroup(const void *__restrict__ w, const MmvqArgs &a,
                                                float *__restrict__ out, int64_t wg, uint8_t *lds) {
    using C = TiledCfg<N, KS, RTW, IT, XP>;
    Q6Tiled f;
    f.init(w, a.rows, a.K);
    const int tid = threadIdx.x, l = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int ks = wave % KS, rt = wave / KS;
    // the wave's tile and the lane's row; lanes past the last row load from a
    // row that exists and store nothing
    const int64_t ntiles = (a.rows + 15) / 16;
    const int64_t tile = wg * RTW + rt, tc = min(tile, ntiles - 1);
    const int R = (int)min((int64_t)16, a.rows - 16 * tc);
    const int r = l & 15, rr = min(r, R - 1), kg = l >> 4;
    const int64_t row = 16 * tile + r;
    const bool rok = tile < ntiles && r < R;
    TiledLane<C::NCG> tl;
    tl.R = R;
    tl.a = plane_rsrc(f.A + 16 * tc * f.nsb, 16 * R * f.nsb);
    tl.b = plane_rsrc(f.B + 16 * tc * f.nsb, 8 * R * f.nsb);
    tl.sc = plane_rsrc(f.SC + 16 * tc * (f.nsb / 4), 8 * R * (f.nsb / 4));
    tl.d = plane_rsrc(f.D + 16 * tc * f.nb, 2 * R * f.nb);
    tl.oa = 16u * (uint32_t)(kg * R + rr);
    tl.ob = 8u * (uint32_t)(kg * R + rr);
    tl.osc = 8u * (uint32_t)rr;
    tl.od = 2u * (uint32_t)rr;
    {
        // A row l%16 is (column 4cg + (l%16)/4, sub-block (l%16)%4); the lane
        // carries data only where that sub-block is its k-group
        const bool am = (l & 3) == kg;
        constexpr int TNB = C::TNB;
#pragma unroll
        for (int cg = 0; cg < C::NCG; cg++) {
            const int na = min(4 * cg + ((l & 15) >> 2), N - 1);
            tl.xb[cg] = am ? na * TNB + 4 * ks * IT + kg : N * TNB;
        }
    }
    const int ZS = (int)(a.K / 128);
    float acc[C::NCG];
#pragma unroll
    for (int cg = 0; cg < C::NCG; cg++) acc[cg] = 0.0f;
    const int nfull = ZS / C::CZ;
    for (int c = 0; c < nfull; c++) {
        if (!C::WT && c > 0) lds_barrier();
        tiled_chunk<true, N, KS, RTW, IT, DUMP, XP>(f, tl, a, lds, c * C::CZ, ZS, row, rok, acc);
    }
    if (nfull * C::CZ < ZS) {
        if (!C::WT && nfull > 0) lds_barrier();
        tiled_chunk<false, N, KS, RTW, IT, DUMP, XP>(f, tl, a, lds, nfull * C::CZ, ZS, row, rok, acc);
    }
    if constexpr (!DUMP) {
        if constexpr (KS > 1) {
            // partial sums of the KS waves of each row tile, added in wave order
            float *red = reinterpret_cast<float *>(lds);
            lds_barrier();
#pragma unroll
            for (int cg = 0; cg < C::NCG; cg++) red[(wave * C::NCG + cg) * kWave + l] = acc[cg];
            lds_barrier();
            if (ks == 0) {
#pragma unroll
                for (int cg = 0; cg < C::NCG; cg++) {
                    float s = red[((rt * KS) * C::NCG + cg) * kWave + l];
#pragma unroll
                    for (int k = 1; k < KS; k++) s += red[((rt * KS + k) * C::NCG + cg) * kWave + l];
                    acc[cg] = s;
                }
            }
        }
        if (ks == 0) {
#pragma unroll
            for (int cg = 0; cg < C::NCG; cg++) {
                const int no = 4 * cg + (l >> 4);
                if constexpr (AMAX) {
                    // largest key over the 16 lanes (rows) of this column
                    uint64_t key = argmax_key(rok ? acc[cg] : -__builtin_inff(), row);
#pragma unroll
                    for (int m = 1; m < 16; m <<= 1) {
                        const uint32_t lo = __shfl_xor((uint32_t)key, m), hi = __shfl_xor((uint32_t)(key >> 32), m);
                        const uint64_t o = ((uint64_t)hi << 32) | lo;
                        key = o > key ? o : key;
                    }
                    if ((l & 15) == 0 && no < N && tile < ntiles)
                        reinterpret_cast<uint64_t *>(out)[no * ntiles + tile] = key;
                } else {
                    if (rok && no < N) out[(int64_t)no * a.rows + row] = acc[cg];
                }
            }
        }
    }
}

template <int N, int KS, int RTW, int IT, bool DUMP, bool AMAX = false, bool XP = false>
__global__ __launch_bounds__(KS * RTW * kWave) void k_mmvq_q6_tiled(const void *__restrict__ w, MmvqArgs a,
                                                                    float *__restrict__ out) {
    static_assert(N <= 8 || (!DUMP && !AMAX), "batched products write outputs only");
    extern __shared__ __align__(16) uint8_t lds[];
    const int64_t ntiles = (a.rows + 15) / 16;
    int64_t wg = blockIdx.x;
    if constexpr (N > 8) {
        const int64_t nrw = (ntiles + RTW - 1) / RTW, g8 = (nrw + 7) / 8;
        const int64_t nbat = gridDim.x / (8 * g8), j = blockIdx.x >> 3;
        const int64_t cb = j % nbat;
        wg = (j / nbat) * 8 + (blockIdx.x & 7);
        if (wg >= nrw) return;                              // the whole workgroup
        a.xq += cb * N * 36 * (a.K / 32);
        out += cb * N * a.rows;
    }
    if constexpr (AMAX) {
        // clear the reduction's running maxima and counts (k_argmax_reduce)
        if (blockIdx.x == 0 && threadIdx.x < N) {
            uint8_t *tail = reinterpret_cast<uint8_t *>(out) + argmax_tail(ntiles, N);
            reinterpret_cast<uint64_t *>(tail)[threadIdx.x] = 0;
            reinterpret_cast<uint32_t *>(tail + 64)[threadIdx.x] = 0;
        }
    }
    tiled_workgroup<N, KS, RTW, IT, DUMP, AMAX, XP>(w, a, out, wg, lds);
}

// Streamed form of a workgroup of column-planar products whose K is one
// chunk of VKS waves of IT steps (K = 128 * VKS * IT): one wave per 16-row
// tile takes all VKS * IT steps, with RG steps' weight loads in flight (a
// ring: step s + RG's loads go out once step s is computed), against one
// activation tile of the whole K staged once for the workgroup's RTW tiles.
// The VKS partial sums -- one per IT consecutive steps, what the VKS waves
// of the chunked form each add up -- are kept apart and added in wave
// order, so every output is the chunked form's bits.  No cross-wave sum, a
// quarter of the activation reads per weight byte at RTW = 4, and a batch's
// waves (one per row tile) all resident at once rather than in two rounds.
template <int N, int RTW, int VKS, int IT, int RG>
__device__ __forceinline__ void tiled_stream_workgroup(const void *__restrict__ w, const MmvqArgs &a,
                                                       float *__restrict__ out, int64_t wg, uint8_t *lds) {
    constexpr int ST = VKS * IT;                       // steps of K
    static_assert(RG >= 1 && RG <= ST, "ring of at most the steps of K");
    using C = TiledCfg<N, 1, RTW, ST, true>;           // staging geometry: one tile of the whole K
    constexpr int TNB = C::TNB, NCG = C::NCG;
    static_assert(!C::WT && !C::SCS && TNB == 4 * ST, "one shared tile of the whole K");
    Q6Tiled f;
    f.init(w, a.rows, a.K);
    const int tid = threadIdx.x, l = tid & (kWave - 1);
    const int rt = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int64_t ntiles = (a.rows + 15) / 16;
    const int64_t tile = wg * RTW + rt, tc = min(tile, ntiles - 1);
    const int R = (int)min((int64_t)16, a.rows - 16 * tc);
    const int r = l & 15, rr = min(r, R - 1), kg = l >> 4;
    const int64_t row = 16 * tile + r;
    const bool rok = tile < ntiles && r < R;
    TiledLane<NCG> tl;
    tl.R = R;
    tl.a = plane_rsrc(f.A + 16 * tc * f.nsb, 16 * R * f.nsb);
    tl.b = plane_rsrc(f.B + 16 * tc * f.nsb, 8 * R * f.nsb);
    tl.sc = plane_rsrc(f.SC + 16 * tc * (f.nsb / 4), 8 * R * (f.nsb / 4));
    tl.d = plane_rsrc(f.D + 16 * tc * f.nb, 2 * R * f.nb);
    tl.oa = 16u * (uint32_t)(kg * R + rr);
    tl.ob = 8u * (uint32_t)(kg * R + rr);
    tl.osc = 8u * (uint32_t)rr;
    tl.od = 2u * (uint32_t)rr;
    {
        const bool am = (l & 3) == kg;
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) {
            const int na = min(4 * cg + ((l & 15) >> 2), N - 1);
            tl.xb[cg] = am ? na * TNB + kg : N * TNB;
        }
    }

    // activation loads first: the whole K of the N columns (consecutive),
    // shared by the workgroup's threads
    const uint32_t cstride = (uint32_t)(36 * (a.K / 32));
    const __amdgpu_buffer_rsrc_t xr = plane_rsrc(a.xq, (int64_t)N * cstride);
    v4u32 xv[C::QSL];
    v2u32 dv[C::DSL];
#pragma unroll
    for (int s = 0; s < C::QSL; s++) {
        const int i = tid + s * C::SLOTW, ic = min(i, N * C::QU - 1), n = ic / C::QU, j = ic - n * C::QU;
        xv[s] = __builtin_amdgcn_raw_buffer_load_b128(xr, (uint32_t)n * cstride + 16u * (uint32_t)j, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < C::DSL; s++) {
        const int i = tid + s * C::SLOTW, ic = min(i, N * C::DU - 1), n = ic / C::DU, k = ic - n * C::DU;
        dv[s] = __builtin_amdgcn_raw_buffer_load_b64(xr, (uint32_t)n * cstride + (uint32_t)a.K + 8u * (uint32_t)k,
                                                     0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);

    // the first RG steps' weights (the ring)
    uint4 wa[RG];
    uint2 wb[RG], wsc[RG];
    uint32_t wd[RG];
    auto load_step = [&](int z, int slot) {
        const int zr = z * tl.R;                                   // wave-uniform
        const v2u32 sc = __builtin_amdgcn_raw_buffer_load_b64(tl.sc, tl.osc, 8 * zr, 0);
        wd[slot] = __builtin_amdgcn_raw_buffer_load_b16(tl.d, tl.od, 2 * ((z >> 1) * tl.R), 0);
        const v4u32 va = __builtin_amdgcn_raw_buffer_load_b128(tl.a, tl.oa, 64 * zr, kNonTemporal);
        const v2u32 vb = __builtin_amdgcn_raw_buffer_load_b64(tl.b, tl.ob, 32 * zr, kNonTemporal);
        wsc[slot] = make_uint2(sc.x, sc.y);
        wa[slot] = make_uint4(va.x, va.y, va.z, va.w);
        wb[slot] = make_uint2(vb.x, vb.y);
    };
#pragma unroll
    for (int z = 0; z < RG; z++) {
        load_step(z, z);
        __builtin_amdgcn_sched_barrier(0);
    }

    // stage the tile: quant entries (32 B), the zero entries, then d
    uint4 *x0 = reinterpret_cast<uint4 *>(lds);
    uint2 *dh = reinterpret_cast<uint2 *>(x0 + 2 * C::XE);
    if (tid < C::ZW) {
        x0[2 * (N * TNB + tid)] = make_uint4(0, 0, 0, 0);
        x0[2 * (N * TNB + tid) + 1] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < C::QSL; s++) {
        const int i = tid + s * C::SLOTW, n = i / C::QU, j = i - n * C::QU;
        if (i < N * C::QU) reinterpret_cast<v4u32 *>(x0)[2 * n * TNB + j] = xv[s];
    }
#pragma unroll
    for (int s = 0; s < C::DSL; s++) {
        const int i = tid + s * C::SLOTW, n = i / C::DU, k = i - n * C::DU;
        if (i < N * C::DU) reinterpret_cast<v2u32 *>(dh)[n * (TNB / 4) + k] = dv[s];
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // The steps in order, unrolled (ring slot z % RG).  Quarter q (the IT
    // steps one wave of the chunked form takes) has its sum formed alone,
    // then added to those before it in order.  Two empty asm statements
    // per step keep the code in step order: the step index reaches the LDS
    // addresses through one (so no later step's activation operands are
    // fetched ahead), and the quarter's sum passes through the other once
    // the step is added (so its scale arithmetic is not deferred, holding
    // every step's matrix-core results).  Unrolled without them the kernel
    // took 256 VGPRs.  (A rolled loop over quarters with a ring of one
    // quarter, five steps, measured 0.6-0.8 us slower per batched launch.)
    float acc[NCG], accq[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; cg++) acc[cg] = 0.0f;
#pragma unroll
    for (int z = 0; z < ST; z++) {
        if (z % IT == 0) {
#pragma unroll
            for (int cg = 0; cg < NCG; cg++) accq[cg] = 0.0f;
        }
        const int slot = z % RG;
        int zs = z;
        asm volatile("" : "+s"(zs));
        tiled_step<N, NCG, TNB, ST, false, true>(wa[slot], wb[slot], wsc[slot], wd[slot], tl.xb, zs, 4 * zs, lds, kg,
                                                 a, row, rok, z, accq);
#pragma unroll
        for (int cg = 0; cg < NCG; cg++) asm volatile("" : "+v"(accq[cg]));
        __builtin_amdgcn_sched_barrier(0);
        if (z + RG < ST) load_step(z + RG, slot);
        __builtin_amdgcn_sched_barrier(0);
        if (z % IT == IT - 1) {
#pragma unroll
            for (int cg = 0; cg < NCG; cg++) acc[cg] = z < IT ? accq[cg] : acc[cg] + accq[cg];
        }
    }
#pragma unroll
    for (int cg = 0; cg < NCG; cg++) {
        const int no = 4 * cg + (l >> 4);
        if (rok && no < N) out[(int64_t)no * a.rows + row] = acc[cg];
    }
}

// Several independent products of the same K in one launch (the matrices of
// a layer, each with its own activation columns): job j takes workgroups
// wg0[j] .. wg0[j+1]-1, each one row workgroup of that job's product, with
// the same waves along K and so the same bits as the job launched alone.
// One launch ramps up and drains once for all of them.
// Every wave reads the job table from the kernel arguments before its first
// weight load, so the table is kept small: MJ (4 or 8) entries, the count
// and K first.  Three 10240x2560 products (8, 4, 1 columns) measured 13.09
// us per launch with eight entries followed by the count and K, 12.89 with
// the count and K first, 12.75 with four entries.  (Loading every entry at
// once and selecting by value, one round of argument loads instead of two,
// measured 12.87.)
constexpr int kMaxTiledJobs = 8;
struct TiledJob {
    const void *w;
    const uint8_t *xq;
    float *out;
    int64_t rows;
    int32_t ncols, wg0;
};
template <int MJ>
struct TiledJobs {
    int64_t K;
    int32_t njobs;
    TiledJob job[MJ];
};

template <int KS, int RTW, int IT, bool XP, int MJ>
__global__ __launch_bounds__(KS * RTW * kWave) void k_mmvq_q6_tiled_jobs(const TiledJobs<MJ> js) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int b = blockIdx.x;
    // this workgroup's job, and its fields, by selects over the (scalar)
    // kernel arguments rather than an indexed access.  (The jobs' workgroups
    // handed out interleaved, round by round, measured 0.2-0.4 us slower on
    // three 10240x2560 products than each job's in one consecutive range.)
    int j = 0;
#pragma unroll
    for (int i = 1; i < MJ; i++) j = (i < js.njobs && b >= js.job[i].wg0) ? i : j;
    TiledJob jb = js.job[0];
#pragma unroll
    for (int i = 1; i < MJ; i++)
        if (j == i) jb = js.job[i];
    MmvqArgs a;
    a.xq = jb.xq;
    a.dump = nullptr;
    a.rows = jb.rows;
    a.K = js.K;
    a.colpack = 0x0706050403020100ull;
    a.xstride = js.K / 32;
    a.its = IT;
    a.nout = jb.ncols;
    const int64_t wg = b - jb.wg0;
    switch (jb.ncols) {
    case 1: tiled_workgroup<1, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    case 2: tiled_workgroup<2, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    case 3: tiled_workgroup<3, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    case 4: tiled_workgroup<4, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    case 5: tiled_workgroup<5, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    case 6: tiled_workgroup<6, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    case 7: tiled_workgroup<7, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    default: tiled_workgroup<8, KS, RTW, IT, false, false, XP>(jb.w, a, jb.out, wg, lds); break;
    }
}

// Steps in flight per wave of the streamed form (its ring).  Three
// 10240x2560 products (8, 4, 1 columns), per batched launch in one run:
// 12.80 / 12.71 us at a ring of two, 12.33 / 12.46 at three, 12.23 / 12.26
// at four, 12.58 / 12.28 at five, 12.55 / 12.62 at six, 12.72 / 12.78 at
// seven; a deeper ring (ten) and whole quarters refilled at once were slower
// still.  Three 5120x5120 products: 13.10 -> 12.76 us against the rolled
// ring of five.
constexpr int kStreamRing = 4;

// The jobs kernel in the streamed form (column-planar activations, K one
// chunk of VKS waves of IT steps): workgroup b takes RTW row tiles of its
// job, one wave each.
template <int RTW, int VKS, int IT, int MJ>
__global__ __launch_bounds__(RTW * kWave) void k_mmvq_q6_tiled_jobs_stream(const TiledJobs<MJ> js) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int b = blockIdx.x;
    int j = 0;
#pragma unroll
    for (int i = 1; i < MJ; i++) j = (i < js.njobs && b >= js.job[i].wg0) ? i : j;
    TiledJob jb = js.job[0];
#pragma unroll
    for (int i = 1; i < MJ; i++)
        if (j == i) jb = js.job[i];
    MmvqArgs a;
    a.xq = jb.xq;
    a.dump = nullptr;
    a.rows = jb.rows;
    a.K = js.K;
    a.colpack = 0x0706050403020100ull;
    a.xstride = js.K / 32;
    a.its = IT;
    a.nout = jb.ncols;
    const int64_t wg = b - jb.wg0;
    switch (jb.ncols) {
    case 1: tiled_stream_workgroup<1, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    case 2: tiled_stream_workgroup<2, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    case 3: tiled_stream_workgroup<3, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    case 4: tiled_stream_workgroup<4, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    case 5: tiled_stream_workgroup<5, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    case 6: tiled_stream_workgroup<6, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    case 7: tiled_stream_workgroup<7, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    default: tiled_stream_workgroup<8, RTW, VKS, IT, kStreamRing>(jb.w, a, jb.out, wg, lds); break;
    }
}

// Per column n, workgroup g: the largest of keys 1024g .. 1024g + 1023
// (four per thread, all loads at once), merged into the column's maximum
// with a 64-bit atomic max (order-free: the maximum is unique); the
// workgroup that completes the column's count (acquire-release, one thread
// per workgroup) decodes it into the row and its value.  Several
// workgroups per column spread the key reads over CUs (one workgroup per
// column took ~5.9 us for the 9,496 tiles of a 151,936-row head).
constexpr int kArgmaxThreads = 256, kArgmaxLoads = 4, kArgmaxSpan = kArgmaxThreads * kArgmaxLoads;
__global__ __launch_bounds__(kArgmaxThreads) void k_argmax_reduce(uint64_t *__restrict__ keys, int64_t ntiles,
                                                                  int ncols, int32_t *__restrict__ idx,
                                                                  float *__restrict__ val) {
    __shared__ uint64_t red[kArgmaxThreads / kWave];
    const int n = blockIdx.x, t = threadIdx.x;
    const uint64_t *kc = keys + (int64_t)n * ntiles;
    const int64_t base = (int64_t)blockIdx.y * kArgmaxSpan;
    // unconditional loads from indices clamped to the last key, all in
    // flight at once (a conditional load each waited for the one before; a
    // repeated key does not change the maximum)
    uint64_t v[kArgmaxLoads];
#pragma unroll
    for (int u = 0; u < kArgmaxLoads; u++) {
        const int64_t i = base + (int64_t)u * kArgmaxThreads + t;
        v[u] = kc[i < ntiles ? i : ntiles - 1];
    }
    uint64_t k = 0;
#pragma unroll
    for (int u = 0; u < kArgmaxLoads; u++) k = v[u] > k ? v[u] : k;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)k, m), hi = __shfl_xor((uint32_t)(k >> 32), m);
        const uint64_t o = ((uint64_t)hi << 32) | lo;
        k = o > k ? o : k;
    }
    if ((t & (kWave - 1)) == 0) red[t / kWave] = k;
    __syncthreads();
    if (t == 0) {
        uint64_t best = red[0];
        for (int i = 1; i < kArgmaxThreads / kWave; i++) best = red[i] > best ? red[i] : best;
        uint8_t *tail = reinterpret_cast<uint8_t *>(keys) + argmax_tail(ntiles, ncols);
        unsigned long long *fin = reinterpret_cast<unsigned long long *>(tail);
        uint32_t *cnt = reinterpret_cast<uint32_t *>(tail + 64);
        atomicMax(fin + n, (unsigned long long)best);
        const uint32_t done = __hip_atomic_fetch_add(cnt + n, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.y - 1) {
            const uint64_t b64 = __hip_atomic_load(fin + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t b = (uint32_t)(b64 >> 32);
            idx[n] = (int32_t)(0xFFFFFFFFu - (uint32_t)b64);
            val[n] = __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
        }
    }
}

// nbat: batches of N columns (N > 8 only)
template <int N, int KS, int RTW, int IT, bool DUMP, bool AMAX = false, bool XP = false>
hipError_t launch_tiled_cfg(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                            hipStream_t s, int64_t nbat = 1) {
    using C = TiledCfg<N, KS, RTW, IT, XP>;
    MmvqArgs a;
    a.xq = reinterpret_cast<const uint8_t *>(xq);
    a.dump = dump;
    a.rows = rows;
    a.K = K;
    a.colpack = 0x0706050403020100ull;
    a.xstride = K / 32;
    a.its = IT;
    a.nout = N;
    const int64_t tiles = (rows + 15) / 16;
    int64_t grid = (tiles + RTW - 1) / RTW;
    if constexpr (N > 8) grid = 8 * ((grid + 7) / 8) * nbat;
    if (grid * C::NTHR > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_mmvq_q6_tiled<N, KS, RTW, IT, DUMP, AMAX, XP>), C::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_mmvq_q6_tiled<N, KS, RTW, IT, DUMP, AMAX, XP>), dim3((unsigned)grid), dim3(C::NTHR), C::LDS,
                       s, w, a, out);
    return hipGetLastError();
}

// Waves along K per row tile: enough waves of five steps to cover a row in
// one chunk (at most sixteen), and workgroups of at least four waves.  A
// function of K only, so every column count sums a row in the same order.
template <int N, bool DUMP, bool AMAX = false, bool XP = false>
hipError_t launch_tiled_n(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                          hipStream_t s) {
    const int64_t need = (K / 128 + 4) / 5;
    if (need <= 1) return launch_tiled_cfg<N, 1, 4, 5, DUMP, AMAX, XP>(w, xq, out, dump, rows, K, s);
    if (need <= 2) return launch_tiled_cfg<N, 2, 2, 5, DUMP, AMAX, XP>(w, xq, out, dump, rows, K, s);
    if (need <= 4) return launch_tiled_cfg<N, 4, 1, 5, DUMP, AMAX, XP>(w, xq, out, dump, rows, K, s);
    if (need <= 8) return launch_tiled_cfg<N, 8, 1, 5, DUMP, AMAX, XP>(w, xq, out, dump, rows, K, s);
    return launch_tiled_cfg<N, 16, 1, 5, DUMP, AMAX, XP>(w, xq, out, dump, rows, K, s);
}

// LDS of the jobs kernel: the largest any column count needs.
template <int KS, int RTW, int IT, bool XP>
constexpr size_t tiled_jobs_lds() {
    size_t m = 0;
    const size_t v[8] = {TiledCfg<1, KS, RTW, IT, XP>::LDS, TiledCfg<2, KS, RTW, IT, XP>::LDS,
                         TiledCfg<3, KS, RTW, IT, XP>::LDS, TiledCfg<4, KS, RTW, IT, XP>::LDS,
                         TiledCfg<5, KS, RTW, IT, XP>::LDS, TiledCfg<6, KS, RTW, IT, XP>::LDS,
                         TiledCfg<7, KS, RTW, IT, XP>::LDS, TiledCfg<8, KS, RTW, IT, XP>::LDS};
    for (size_t x : v) m = x > m ? x : m;
    return m;
}

// Jobs (at most MJ, same K) in one launch; the caller has checked every job.
// Workgroup ranges in the given job order.
template <int KS, int RTW, int IT, bool XP, int MJ>
hipError_t launch_tiled_jobs_mj(const TiledJobs<kMaxTiledJobs> &all, hipStream_t s) {
    constexpr int NTHR = KS * RTW * kWave;
    TiledJobs<MJ> js;
    js.K = all.K;
    js.njobs = all.njobs;
    int64_t wg = 0;
    for (int j = 0; j < js.njobs; j++) {
        js.job[j] = all.job[j];
        js.job[j].wg0 = (int32_t)wg;
        wg += ((js.job[j].rows + 15) / 16 + RTW - 1) / RTW;
    }
    for (int j = js.njobs; j < MJ; j++) js.job[j] = js.job[0];
    if (wg * NTHR > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    constexpr size_t lds = tiled_jobs_lds<KS, RTW, IT, XP>();
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_mmvq_q6_tiled_jobs<KS, RTW, IT, XP, MJ>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_mmvq_q6_tiled_jobs<KS, RTW, IT, XP, MJ>), dim3((unsigned)wg), dim3(NTHR), lds, s, js);
    return hipGetLastError();
}

template <int KS, int RTW, int IT, bool XP>
hipError_t launch_tiled_jobs_cfg(const TiledJobs<kMaxTiledJobs> &js, hipStream_t s) {
    if (js.njobs <= 4) return launch_tiled_jobs_mj<KS, RTW, IT, XP, 4>(js, s);
    return launch_tiled_jobs_mj<KS, RTW, IT, XP, kMaxTiledJobs>(js, s);
}

// Row tiles (waves) per workgroup of the streamed form.  Three 10240x2560
// products (8, 4, 1 columns), per launch: with a rolled ring of five steps
// 12.30 us at four tiles, 13.43 at two, 12.52 at eight; with the unrolled
// ring of four (graph replays of 27 launches, two runs) 12.23-12.56 at
// four, 14.07-14.14 at two, 12.72-13.17 at eight.
constexpr int kStreamRtw = 4;

template <int VKS, int IT, int MJ>
hipError_t launch_tiled_jobs_stream_mj(const TiledJobs<kMaxTiledJobs> &all, hipStream_t s) {
    constexpr int NTHR = kStreamRtw * kWave;
    TiledJobs<MJ> js;
    js.K = all.K;
    js.njobs = all.njobs;
    int64_t wg = 0;
    for (int j = 0; j < js.njobs; j++) {
        js.job[j] = all.job[j];
        js.job[j].wg0 = (int32_t)wg;
        wg += ((js.job[j].rows + 15) / 16 + kStreamRtw - 1) / kStreamRtw;
    }
    for (int j = js.njobs; j < MJ; j++) js.job[j] = js.job[0];
    if (wg * NTHR > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    size_t lds = 0;
    const size_t v[8] = {TiledCfg<1, 1, kStreamRtw, VKS * IT, true>::LDS, TiledCfg<2, 1, kStreamRtw, VKS * IT, true>::LDS,
                         TiledCfg<3, 1, kStreamRtw, VKS * IT, true>::LDS, TiledCfg<4, 1, kStreamRtw, VKS * IT, true>::LDS,
                         TiledCfg<5, 1, kStreamRtw, VKS * IT, true>::LDS, TiledCfg<6, 1, kStreamRtw, VKS * IT, true>::LDS,
                         TiledCfg<7, 1, kStreamRtw, VKS * IT, true>::LDS, TiledCfg<8, 1, kStreamRtw, VKS * IT, true>::LDS};
    for (size_t x : v) lds = x > lds ? x : lds;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_mmvq_q6_tiled_jobs_stream<kStreamRtw, VKS, IT, MJ>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_mmvq_q6_tiled_jobs_stream<kStreamRtw, VKS, IT, MJ>), dim3((unsigned)wg), dim3(NTHR), lds, s,
                       js);
    return hipGetLastError();
}

template <bool XP>
hipError_t launch_tiled_jobs(const TiledJobs<kMaxTiledJobs> &js, hipStream_t s) {
    const int64_t need = (js.K / 128 + 4) / 5;
    // column-planar jobs whose K is exactly one chunk of four or eight waves
    // of five steps (K = 2560, 5120): the streamed form, the same bits.
    // Three products of 8, 4 and 1 columns, per launch (its first, rolled
    // ring of five): 10240x2560 12.75 -> 12.30 us, 5120x5120 13.34 -> 12.95
    // us; at K = 1280 (two waves) the streamed form was slower (10240 rows:
    // 7.65 -> 7.90 us), so not there.
    if constexpr (XP) {
        if (js.K == 4 * 5 * 128)
            return js.njobs <= 4 ? launch_tiled_jobs_stream_mj<4, 5, 4>(js, s)
                                 : launch_tiled_jobs_stream_mj<4, 5, kMaxTiledJobs>(js, s);
        if (js.K == 8 * 5 * 128)
            return js.njobs <= 4 ? launch_tiled_jobs_stream_mj<8, 5, 4>(js, s)
                                 : launch_tiled_jobs_stream_mj<8, 5, kMaxTiledJobs>(js, s);
    }
    if (need <= 1) return launch_tiled_jobs_cfg<1, 4, 5, XP>(js, s);
    if (need <= 2) return launch_tiled_jobs_cfg<2, 2, 5, XP>(js, s);
    if (need <= 4) return launch_tiled_jobs_cfg<4, 1, 5, XP>(js, s);
    if (need <= 8) return launch_tiled_jobs_cfg<8, 1, 5, XP>(js, s);
    return launch_tiled_jobs_cfg<16, 1, 5, XP>(js, s);
}

// Columns per batch of the batched product: sixteen, twelve with sixteen
// waves along K (sixteen columns of that chunk do not fit the 160 KB of LDS).
inline int tiled_batch_cols(int64_t K) { return (K / 128 + 4) / 5 > 8 ? 12 : 16; }

// nbat batches of tiled_batch_cols(K) columns, with the waves along K that
// launch_tiled_n takes for the same K (so the same sums in the same order).
// (Twice the row tiles per workgroup, staging each activation tile for
// twice the rows, measured within +-10 % either way.)
template <bool XP>
hipError_t launch_tiled_batched(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int64_t nbat,
                                hipStream_t s) {
    const int64_t need = (K / 128 + 4) / 5;
    if (need <= 1) return launch_tiled_cfg<16, 1, 4, 5, false, false, XP>(w, xq, out, nullptr, rows, K, s, nbat);
    if (need <= 2) return launch_tiled_cfg<16, 2, 2, 5, false, false, XP>(w, xq, out, nullptr, rows, K, s, nbat);
    if (need <= 4) return launch_tiled_cfg<16, 4, 1, 5, false, false, XP>(w, xq, out, nullptr, rows, K, s, nbat);
    if (need <= 8) return launch_tiled_cfg<16, 8, 1, 5, false, false, XP>(w, xq, out, nullptr, rows, K, s, nbat);
    return launch_tiled_cfg<12, 16, 1, 5, false, false, XP>(w, xq, out, nullptr, rows, K, s, nbat);
}

}  // namespace qmv

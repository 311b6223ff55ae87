// device.hpp -- gfx950 device building blocks of libqmv: integer dot
// products, fp16 decode, wave64 DPP reductions, the K-quant block loaders and
// the MMVQ kernel template shared by the dense and grouped products.
//
// Work mapping (a design for CDNA4 wave64, not the 32-lane sub-group
// mapping of the SYCL kernels on the pages):
//   * a "unit" is the piece of a weight row one lane handles per step:
//     one 32-weight sub-block for Q6_K, a pair of sub-blocks (one 32-byte
//     qs chunk) for Q4_K/Q5_K;
//   * U lanes (8, 16, 32 or 64; a function of K only) share a row; lane u
//     of the group takes units u, u+U, u+2U, ...; a wave holds 64/U rows;
//   * a lane keeps N fp32 accumulators (one per activation column), so the
//     weights are read once for all N columns;
//   * the Q8_1 activation tile is staged once per workgroup in LDS and read
//     by every row of the workgroup;
//   * the U partial sums of a row are combined by a fixed DPP butterfly, so
//     results do not depend on N, on the weight layout or on the launch
//     shape, only on K.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace qmv {

constexpr int kWave = 64;
constexpr int kQ6Bytes = 210, kQ4Bytes = 144, kQ5Bytes = 176, kQ81Bytes = 36;

// Lanes sharing a row: the largest of 64, 32, 16 (not above cap) that
// divides the row's units with at least three units per lane, else 8.  A
// function of the row length only, so every launch of a given K sums a row
// in the same order.
__host__ __device__ constexpr int choose_u(int units, int cap = 64) {
    for (int U = 64; U >= 16; U /= 2)
        if (U <= cap && units % U == 0 && units / U >= 3) return U;
    return 8;
}

// The largest of 64, 32, 16 lanes per row that gives every lane at least two
// units (not necessarily the same number), else 8.
__host__ __device__ constexpr int choose_u_min2(int units) {
    for (int U = 64; U >= 16; U /= 2)
        if (units >= 2 * U) return U;
    return 8;
}

// Activation tile limits: bytes of LDS per workgroup (the device allows
// 160 KB) and Q8_1 blocks each thread loads ahead of the weights.
constexpr int kMaxTileBytes = 120 * 1024;
constexpr int kMaxStageItems = 5;
constexpr int kActBytesPerBlock = 40;

// Register steps staged per LDS sub-tile: as many as fit both limits
// (ideally all IT steps, so a register chunk needs one staging pass).  Large
// workgroups keep to three staged blocks per thread: they run three waves per
// SIMD, and the staging registers would not fit beside the weights.
__host__ __device__ constexpr int its_for(int IT, int N, int U, int SBPU, int nthr) {
    const int max_items = nthr > 256 ? 3 : kMaxStageItems;
    int its = IT;
    while (its > 1 && (N * its * U * SBPU > max_items * nthr ||
                       N * its * U * SBPU * kActBytesPerBlock > kMaxTileBytes))
        its--;
    return its;
}

// Register depth: three steps when a lane has at most three units of a row
// (no clamped duplicate loads), else the format's own depth.
__host__ __device__ constexpr int depth_for(int units, int U, int IT) {
    return (units + U - 1) / U <= 3 ? 3 : IT;
}

// ---------------------------------------------------------------- basics
__device__ __forceinline__ int sdot4(int a, int b, int c) {
    return __builtin_amdgcn_sdot4(a, b, c, false);
}

#ifndef QMV_DOT_HEAD_ASM
#define QMV_DOT_HEAD_ASM 1
#endif
// First dot of a chain (accumulator 0).  The compiler emits v_mov 0 +
// v_dot4c for sdot4(a, b, 0); the three-operand form takes the 0 inline.
__device__ __forceinline__ int sdot4_head(int a, int b) {
#if QMV_DOT_HEAD_ASM
    int d;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
#else
    return __builtin_amdgcn_sdot4(a, b, 0, false);
#endif
}

__device__ __forceinline__ float half_to_float(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ int sext8(uint32_t v, int byte) {
    return __builtin_amdgcn_sbfe((int)v, 8 * byte, 8);
}

__device__ __forceinline__ uint32_t ubyte(uint32_t v, int byte) {
    return __builtin_amdgcn_ubfe(v, 8 * byte, 8);
}

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum of v over each aligned group of U lanes; every lane of a group ends
// with the same bits (each step adds a lane's value to its partner's, and
// fp32 addition is commutative).  All 64 lanes must be active.
template <int U>
__device__ __forceinline__ float group_sum(float v) {
    v = dpp_add<0xB1>(v);                       // quad_perm [1,0,3,2]: lane ^ 1
    v = dpp_add<0x4E>(v);                       // quad_perm [2,3,0,1]: lane ^ 2
    v = dpp_add<0x141>(v);                      // row_half_mirror: i <-> 7-i
    if constexpr (U >= 16) v = dpp_add<0x140>(v);   // row_mirror: i <-> 15-i
    if constexpr (U >= 32) v += __shfl_xor(v, 16);
    if constexpr (U >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Workgroup barrier that orders LDS only: weight loads still in flight are
// not waited for.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// --------------------------------------------------------- LDS act tile
// One staged Q8_1 block of one column: quants 0-15 and 16-31 in two
// 16-byte arrays (conflict-free ds_read_b128 for consecutive blocks) and a
// float pair: (d * dscale, d * sum(q)) where dscale is 1/4 for the Q6_K
// 4x codes.
// nb (blocks per column) is the tile's compile-time column stride, so every
// read of column n is a constant offset from one per-lane address.
template <int NB>
struct ActTile {
    static constexpr int nb = NB;
    uint4 *x0;
    uint4 *x1;
    float2 *f;
};

template <int NB>
__device__ __forceinline__ ActTile<NB> act_tile(void *lds, int ncols) {
    ActTile<NB> t;
    t.x0 = reinterpret_cast<uint4 *>(lds);
    t.x1 = t.x0 + ncols * NB;
    t.f = reinterpret_cast<float2 *>(t.x1 + ncols * NB);
    return t;
}

struct ActRaw {
    uint32_t w[9];
};

__device__ __forceinline__ void act_load(ActRaw &r, const uint8_t *xq, int64_t blk) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(xq + blk * kQ81Bytes);
#pragma unroll
    for (int i = 0; i < 9; i++) r.w[i] = p[i];
}

// Stores one Q8_1 block into the tile; the exact quant sum (times d) is only
// formed for the formats whose min term needs it.
template <bool NEED_SUM, int NB>
__device__ __forceinline__ void act_store(const ActTile<NB> &t, int idx, const ActRaw &r, float dscale) {
    uint4 a = make_uint4(r.w[1], r.w[2], r.w[3], r.w[4]);
    uint4 b = make_uint4(r.w[5], r.w[6], r.w[7], r.w[8]);
    float d = half_to_float(r.w[0]);
    float ds = 0.0f;
    if constexpr (NEED_SUM) {
        int s = 0;
#pragma unroll
        for (int i = 1; i < 9; i++) s = sdot4((int)r.w[i], 0x01010101, s);
        ds = d * (float)s;
    }
    t.x0[idx] = a;
    t.x1[idx] = b;
    t.f[idx] = make_float2(d * dscale, ds);
}

// ------------------------------------------------------- format policies
// Each policy defines:
//   SBPU     sub-blocks per unit;   IT  units held in registers per lane
//   Raw      registers of one unit; load(); dot<N>() accumulating into acc[N]
//   DSCALE   scale applied to d_a when staged;  NEED_SUM  stage d_a * sum(q8).

// Q6_K, planar layout (see qmv.h).  Codes are 4*(q6-32) as int8.
#ifndef QMV_Q6P_IT
#define QMV_Q6P_IT 5
#endif
struct Q6Planar {
    static constexpr int SBPU = 1, IT = QMV_Q6P_IT;
    static constexpr float DSCALE = 0.25f;
    static constexpr bool NEED_SUM = false;
    struct Raw {
        uint4 a;
        uint2 b;
        uint32_t sc, d;
    };
    const uint4 *A;
    const uint2 *B;
    const uint16_t *SC;
    const uint16_t *D;
    int64_t nsb;   // sub-blocks per row

    __device__ __forceinline__ void init(const void *w, int64_t rows, int64_t K) {
        const uint8_t *base = reinterpret_cast<const uint8_t *>(w);
        int64_t NB = rows * (K / 256);
        A = reinterpret_cast<const uint4 *>(base);
        B = reinterpret_cast<const uint2 *>(base + 128 * NB);
        SC = reinterpret_cast<const uint16_t *>(base + 192 * NB);
        D = reinterpret_cast<const uint16_t *>(base + 208 * NB);
        nsb = K / 32;
    }
    __device__ __forceinline__ void load(Raw &r, int64_t row, int unit) const {
        int64_t i = row * nsb + unit;
        r.a = A[i];
        r.b = B[i];
        r.sc = SC[i];
        r.d = D[i >> 3];
    }
    // units unit0 + U*it (it < IT) of one row, all in range
    // units unit0 + U*it, it in [B0, B1), of one row, all in range; SCD: also
    // the scale and d loads of all IT units (issued first)
    template <int U, int IT, int P, int B0, int B1, bool SCD>
    __device__ __forceinline__ void load_chunk(Raw (&r)[IT][P], int p, int64_t row, int unit0) const {
        static_assert(U % 8 == 0, "d index shift");
        const int64_t i0 = row * nsb + unit0;
        const uint4 *pa = A + i0;
        const uint2 *pb = B + i0;
        const uint16_t *ps = SC + i0;
        const uint16_t *pd = D + (i0 >> 3);
        // the small scale and d loads first, then the code planes unit by
        // unit, so unit it waits only for the loads of units 0..it
        if constexpr (SCD) {
#pragma unroll
            for (int it = 0; it < IT; it++) {
                r[it][p].sc = ps[U * it];
                r[it][p].d = pd[(U / 8) * it];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int it = B0; it < B1; it++) {
            r[it][p].a = pa[U * it];
            r[it][p].b = pb[U * it];
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __device__ __forceinline__ static void codes(const Raw &r, int v[8]) {
        const uint32_t m3 = 0x03030303u, mfc = 0xFCFCFCFCu;
        v[0] = (int)(r.a.x & mfc);
        v[1] = (int)(r.a.y & mfc);
        v[2] = (int)(r.a.z & mfc);
        v[3] = (int)(r.a.w & mfc);
        v[4] = (int)(r.b.x & mfc);
        v[5] = (int)(r.b.y & mfc);
        v[6] = (int)(((r.a.z & m3) << 6) | ((r.a.y & m3) << 4) | ((r.a.x & m3) << 2));
        v[7] = (int)(((r.b.y & m3) << 6) | ((r.b.x & m3) << 4) | ((r.a.w & m3) << 2));
    }
};

// Q6_K, GGUF layout: 210-byte blocks, only 2-byte aligned; read as aligned
// dwords and realigned with alignbit, then turned into the same 4x codes.
struct Q6Gguf {
    static constexpr int SBPU = 1, IT = 3;
    static constexpr float DSCALE = 0.25f;
    static constexpr bool NEED_SUM = false;
    struct Raw {
        uint32_t l[9], h[9];
        uint32_t sc, d, shift;   // shift: bit 0-4 realign shift, 8-9: c
    };
    const uint8_t *W;
    int64_t nbk;   // blocks per row

    __device__ __forceinline__ void init(const void *w, int64_t, int64_t K) {
        W = reinterpret_cast<const uint8_t *>(w);
        nbk = K / 256;
    }
    __device__ __forceinline__ void load(Raw &r, int64_t row, int unit) const {
        int j = unit & 7, h = j >> 2, c = j & 3;
        const uint8_t *blk = W + (row * nbk + (unit >> 3)) * kQ6Bytes;
        uintptr_t pl = reinterpret_cast<uintptr_t>(blk) + 64 * h + 32 * (c & 1);
        uintptr_t ph = reinterpret_cast<uintptr_t>(blk) + 128 + 32 * h;
        const uint32_t *al = reinterpret_cast<const uint32_t *>(pl & ~uintptr_t(3));
        const uint32_t *ah = reinterpret_cast<const uint32_t *>(ph & ~uintptr_t(3));
#pragma unroll
        for (int i = 0; i < 9; i++) {
            r.l[i] = al[i];
            r.h[i] = ah[i];
        }
        r.sc = *reinterpret_cast<const uint16_t *>(blk + 192 + 2 * j);
        r.d = *reinterpret_cast<const uint16_t *>(blk + 208);
        r.shift = (uint32_t)((pl & 3) * 8) | ((uint32_t)c << 8);
    }
    __device__ __forceinline__ static void codes(const Raw &r, int v[8]) {
        uint32_t sh = r.shift & 31, c = r.shift >> 8;
        uint32_t nsh = 4 * (c >> 1), hsh = 2 * c;
#pragma unroll
        for (int m = 0; m < 8; m++) {
            uint32_t L = __builtin_amdgcn_alignbit(r.l[m + 1], r.l[m], sh);
            uint32_t H = __builtin_amdgcn_alignbit(r.h[m + 1], r.h[m], sh);
            uint32_t q6 = ((L >> nsh) & 0x0F0F0F0Fu) | (((H >> hsh) & 0x03030303u) << 4);
            v[m] = (int)((q6 ^ 0x20202020u) << 2);
        }
    }
};

// Q6_K dot products of one unit for P rows and N columns; the activation of
// all N columns is read from LDS in one burst (one LDS latency per unit, not
// per column), and each read serves all P rows.  Shared by the two Q6_K
// layouts.
template <class F, int N, int P, bool DUMP, int NB>
__device__ __forceinline__ void q6_dot(const typename F::Raw (&r)[P], const ActTile<NB> &t, int tb,
                                       float (&acc)[P][N], int32_t *const (&dump)[P], const bool (&rok)[P],
                                       int64_t dstride) {
    int v[P][8], sc0[P], sc1[P];
    float dw[P];
#pragma unroll
    for (int p = 0; p < P; p++) {
        F::codes(r[p], v[p]);
        sc0[p] = sext8(r[p].sc, 0);
        sc1[p] = sext8(r[p].sc, 1);
        dw[p] = half_to_float(r[p].d);
    }
    // all columns' activation for this unit in one burst of LDS reads
    uint4 ax0[N], ax1[N];
    float ada[N];
#pragma unroll
    for (int n = 0; n < N; n++) {
        ax0[n] = t.x0[n * NB + tb];
        ax1[n] = t.x1[n * NB + tb];
        ada[n] = DUMP ? 0.0f : t.f[n * NB + tb].x;
    }
#pragma unroll
    for (int n = 0; n < N; n++) {
        const uint4 x0 = ax0[n], x1 = ax1[n];
        const float da = ada[n];
#pragma unroll
        for (int p = 0; p < P; p++) {
            int d0 = sdot4_head(v[p][0], (int)x0.x);
            d0 = sdot4(v[p][1], (int)x0.y, d0);
            d0 = sdot4(v[p][2], (int)x0.z, d0);
            d0 = sdot4(v[p][3], (int)x0.w, d0);
            int d1 = sdot4_head(v[p][4], (int)x1.x);
            d1 = sdot4(v[p][5], (int)x1.y, d1);
            d1 = sdot4(v[p][6], (int)x1.z, d1);
            d1 = sdot4(v[p][7], (int)x1.w, d1);
            // 4 * isum, exact (|operands| < 2^23)
            const int isum4 = __mul24(sc0[p], d0) + __mul24(sc1[p], d1);
            if constexpr (DUMP) {
                if (rok[p]) dump[p][n * dstride] = isum4 >> 2;
            } else {
                acc[p][n] = __builtin_fmaf(dw[p] * da, (float)isum4, acc[p][n]);
            }
        }
    }
}

// Q4_K / Q5_K (GGUF blocks, 16-byte aligned).  Unit = pair p of sub-blocks
// (2p', 2p'+1) of superblock p/4, p' = p%4, i.e. the 32-byte qs chunk whose
// low nibbles are sub-block 2p' and high nibbles sub-block 2p'+1.
template <bool FIVE>
struct Q45 {
    static constexpr int SBPU = 2, IT = 5;
    static constexpr float DSCALE = 1.0f;
    static constexpr bool NEED_SUM = true;
    static constexpr int BYTES = FIVE ? kQ5Bytes : kQ4Bytes;
    struct Raw {
        uint4 hdr, q0, q1;
        uint4 h0, h1;   // Q5_K only
    };
    const uint8_t *W;
    int64_t nbk;

    __device__ __forceinline__ void init(const void *w, int64_t, int64_t K) {
        W = reinterpret_cast<const uint8_t *>(w);
        nbk = K / 256;
    }
    __device__ __forceinline__ void load(Raw &r, int64_t row, int unit) const {
        const uint8_t *blk = W + (row * nbk + (unit >> 2)) * BYTES;
        int pp = unit & 3;
        r.hdr = *reinterpret_cast<const uint4 *>(blk);
        const uint8_t *qs = blk + (FIVE ? 48 : 16) + 32 * pp;
        r.q0 = *reinterpret_cast<const uint4 *>(qs);
        r.q1 = *reinterpret_cast<const uint4 *>(qs + 16);
        if constexpr (FIVE) {
            r.h0 = *reinterpret_cast<const uint4 *>(blk + 16);
            r.h1 = *reinterpret_cast<const uint4 *>(blk + 32);
        }
    }
};

// 6-bit scale and min of sub-block j (0..7) from the 12 packed bytes held in
// hdr.y (bytes 0-3), hdr.z (4-7), hdr.w (8-11).
__device__ __forceinline__ void q45_scale_min(const uint4 &hdr, int j, int &sc, int &m) {
    int jj = j & 3;
    uint32_t Y = ubyte(hdr.y, jj), Z = ubyte(hdr.z, jj), Wb = ubyte(hdr.w, jj);
    int sl = (int)(Y & 63), ml = (int)(Z & 63);
    int sh = (int)((Wb & 15) | ((Y >> 6) << 4)), mh = (int)((Wb >> 4) | ((Z >> 6) << 4));
    sc = j < 4 ? sl : sh;
    m = j < 4 ? ml : mh;
}

template <bool FIVE, int N, int P, bool DUMP, int NB>
__device__ __forceinline__ void q45_dot(const typename Q45<FIVE>::Raw (&r)[P], int unit, const ActTile<NB> &t,
                                        int tb, float (&acc)[P][N], int32_t *const (&dump)[P],
                                        const bool (&rok)[P], int64_t dstride) {
    const int pp = unit & 3, j0 = 2 * pp, j1 = 2 * pp + 1;
    int lo[P][8], hi[P][8], sc0[P], sc1[P];
    float d[P], dmin[P], m0f[P], m1f[P];
#pragma unroll
    for (int p = 0; p < P; p++) {
        const uint32_t q[8] = {r[p].q0.x, r[p].q0.y, r[p].q0.z, r[p].q0.w,
                               r[p].q1.x, r[p].q1.y, r[p].q1.z, r[p].q1.w};
        if constexpr (FIVE) {
            const uint32_t h[8] = {r[p].h0.x, r[p].h0.y, r[p].h0.z, r[p].h0.w,
                                   r[p].h1.x, r[p].h1.y, r[p].h1.z, r[p].h1.w};
#pragma unroll
            for (int m = 0; m < 8; m++) {
                lo[p][m] = (int)((q[m] & 0x0F0F0F0Fu) | (((h[m] >> j0) & 0x01010101u) << 4));
                hi[p][m] = (int)(((q[m] >> 4) & 0x0F0F0F0Fu) | (((h[m] >> j1) & 0x01010101u) << 4));
            }
        } else {
#pragma unroll
            for (int m = 0; m < 8; m++) {
                lo[p][m] = (int)(q[m] & 0x0F0F0F0Fu);
                hi[p][m] = (int)((q[m] >> 4) & 0x0F0F0F0Fu);
            }
        }
        int m0, m1;
        q45_scale_min(r[p].hdr, j0, sc0[p], m0);
        q45_scale_min(r[p].hdr, j1, sc1[p], m1);
        d[p] = half_to_float(r[p].hdr.x);
        dmin[p] = half_to_float(r[p].hdr.x >> 16);
        m0f[p] = (float)m0;
        m1f[p] = (float)m1;
    }
    uint4 na0 = t.x0[tb], na1 = t.x1[tb], nb0 = t.x0[tb + 1], nb1 = t.x1[tb + 1];
    float2 nfa = make_float2(0.0f, 0.0f), nfb = nfa;
    if constexpr (!DUMP) {
        nfa = t.f[tb];
        nfb = t.f[tb + 1];
    }
#pragma unroll
    for (int n = 0; n < N; n++) {
        const uint4 a0 = na0, a1 = na1, b0 = nb0, b1 = nb1;
        const float2 fa = nfa, fb = nfb;
        if (n + 1 < N) {                          // read column n+1 while computing n
            const int o = (n + 1) * NB + tb;
            na0 = t.x0[o];
            na1 = t.x1[o];
            nb0 = t.x0[o + 1];
            nb1 = t.x1[o + 1];
            if constexpr (!DUMP) {
                nfa = t.f[o];
                nfb = t.f[o + 1];
            }
        }
#pragma unroll
        for (int p = 0; p < P; p++) {
            int da = sdot4_head(lo[p][0], (int)a0.x);
            da = sdot4(lo[p][1], (int)a0.y, da);
            da = sdot4(lo[p][2], (int)a0.z, da);
            da = sdot4(lo[p][3], (int)a0.w, da);
            da = sdot4(lo[p][4], (int)a1.x, da);
            da = sdot4(lo[p][5], (int)a1.y, da);
            da = sdot4(lo[p][6], (int)a1.z, da);
            da = sdot4(lo[p][7], (int)a1.w, da);
            int db = sdot4_head(hi[p][0], (int)b0.x);
            db = sdot4(hi[p][1], (int)b0.y, db);
            db = sdot4(hi[p][2], (int)b0.z, db);
            db = sdot4(hi[p][3], (int)b0.w, db);
            db = sdot4(hi[p][4], (int)b1.x, db);
            db = sdot4(hi[p][5], (int)b1.y, db);
            db = sdot4(hi[p][6], (int)b1.z, db);
            db = sdot4(hi[p][7], (int)b1.w, db);
            if constexpr (DUMP) {
                if (rok[p]) {
                    dump[p][n * dstride] = da;
                    dump[p][n * dstride + 1] = db;
                }
            } else {
                float s2 = fa.x * (float)__mul24(sc0[p], da);
                s2 = __builtin_fmaf(fb.x, (float)__mul24(sc1[p], db), s2);
                float mm = m0f[p] * fa.y;
                mm = __builtin_fmaf(m1f[p], fb.y, mm);
                acc[p][n] = __builtin_fmaf(d[p], s2, acc[p][n]);
                acc[p][n] = __builtin_fmaf(-dmin[p], mm, acc[p][n]);
            }
        }
    }
}

template <class F>
struct Dot;
template <>
struct Dot<Q6Planar> {
    template <int N, int P, bool DUMP, int NB>
    __device__ __forceinline__ static void run(const Q6Planar::Raw (&r)[P], int, const ActTile<NB> &t, int tb,
                                               float (&acc)[P][N], int32_t *const (&dp)[P],
                                               const bool (&rok)[P], int64_t ds) {
        q6_dot<Q6Planar, N, P, DUMP, NB>(r, t, tb, acc, dp, rok, ds);
    }
};
template <>
struct Dot<Q6Gguf> {
    template <int N, int P, bool DUMP, int NB>
    __device__ __forceinline__ static void run(const Q6Gguf::Raw (&r)[P], int, const ActTile<NB> &t, int tb,
                                               float (&acc)[P][N], int32_t *const (&dp)[P],
                                               const bool (&rok)[P], int64_t ds) {
        q6_dot<Q6Gguf, N, P, DUMP, NB>(r, t, tb, acc, dp, rok, ds);
    }
};
template <bool FIVE>
struct Dot<Q45<FIVE>> {
    template <int N, int P, bool DUMP, int NB>
    __device__ __forceinline__ static void run(const typename Q45<FIVE>::Raw (&r)[P], int unit,
                                               const ActTile<NB> &t, int tb, float (&acc)[P][N],
                                               int32_t *const (&dp)[P], const bool (&rok)[P], int64_t ds) {
        q45_dot<FIVE, N, P, DUMP, NB>(r, unit, t, tb, acc, dp, rok, ds);
    }
};

// Gate and up matrices of one expert read as one matrix of interleaved
// virtual rows: virtual row 2r is gate row r, 2r+1 is up row r.  A wave then
// holds gate and up of the same rows side by side.
struct Q4GateUp {
    static constexpr int SBPU = Q45<false>::SBPU, IT = Q45<false>::IT;
    static constexpr float DSCALE = 1.0f;
    static constexpr bool NEED_SUM = true;
    using Raw = Q45<false>::Raw;
    Q45<false> g, u;
    int64_t base_row;   // first row of the expert in both tensors

    __device__ __forceinline__ void load(Raw &r, int64_t vrow, int unit) const {
        // select the base pointer, not the policy object (a runtime choice
        // between two objects would put them in scratch memory)
        const uintptr_t wg = reinterpret_cast<uintptr_t>(g.W), wu = reinterpret_cast<uintptr_t>(u.W);
        Q45<false> m;
        m.W = reinterpret_cast<const uint8_t *>(wg ^ ((wg ^ wu) & (uintptr_t)0 - (uintptr_t)(vrow & 1)));
        m.nbk = g.nbk;
        m.load(r, base_row + (vrow >> 1), unit);
    }
};
template <>
struct Dot<Q4GateUp> {
    template <int N, int P, bool DUMP, int NB>
    __device__ __forceinline__ static void run(const Q4GateUp::Raw (&r)[P], int unit, const ActTile<NB> &t,
                                               int tb, float (&acc)[P][N], int32_t *const (&dp)[P],
                                               const bool (&rok)[P], int64_t ds) {
        q45_dot<false, N, P, DUMP, NB>(r, unit, t, tb, acc, dp, rok, ds);
    }
};

// ------------------------------------------------------- Q8_1 quantizer
// Quantizes one block of 32 values held one per lane by an aligned group of
// 32 lanes (all 32 lanes active).  Returns the lane's int8 quant; the block's
// fp16 d and s bits are returned in every lane.  d = amax/127 and x/d are
// IEEE fp32 divisions, rounding is half away from zero, the fp16 stores
// round to nearest even.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true)));
}
template <int CTRL>
__device__ __forceinline__ int dpp_iadd(int v) {
    return v + __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// fp16 bits of the Q8_1 sum field: the fp32 product d * sum, rounded to
// fp32, then to fp16 (both to nearest even).  The compiler would otherwise
// fuse the multiply and the conversion into one mixed-precision fma, which
// rounds the exact product to fp16 once -- a different result where the
// fp32 product lands on an fp16 midpoint.  The empty register-only asm
// makes the fp32 product a value the conversion must start from.
__device__ __forceinline__ uint32_t q8_1_sum_bits(float d, int sum) {
    float p = d * (float)sum;
    asm volatile("" : "+v"(p));
    return __builtin_bit_cast(uint16_t, (_Float16)p);
}

__device__ __forceinline__ int q8_1_quantize32(float x, uint32_t &dbits, uint32_t &sbits) {
    // max and sum over the 32 lanes: DPP inside each 16-lane row, then one
    // exchange between the two rows (both orders give the same result)
    float a = fabsf(x);
    a = dpp_max<0xB1>(a);
    a = dpp_max<0x4E>(a);
    a = dpp_max<0x141>(a);
    a = dpp_max<0x140>(a);
    a = fmaxf(a, __shfl_xor(a, 16, 32));
    float d = a / 127.0f;
    int q = 0;
    if (d != 0.0f) {
        float r = roundf(x / d);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q = (int)r;
    }
    int s = q;
    s = dpp_iadd<0xB1>(s);
    s = dpp_iadd<0x4E>(s);
    s = dpp_iadd<0x141>(s);
    s = dpp_iadd<0x140>(s);
    s += __shfl_xor(s, 16, 32);
    dbits = __builtin_bit_cast(uint16_t, (_Float16)d);
    sbits = q8_1_sum_bits(d, s);
    return q;
}

// Stores the quant of lane i (0..31) of a 32-lane group as one Q8_1 block at
// blk (4-byte aligned): lanes 0, 4, .. write a dword of four quants each,
// lane 0 also the (d, s) header.  All 32 lanes must be active; `store`
// masks the writes.
__device__ __forceinline__ void q8_1_store32(uint8_t *blk, int i, int q, uint32_t dbits, uint32_t sbits,
                                             bool store) {
    uint32_t b = (uint32_t)q & 0xFFu;
    uint32_t b1 = __shfl_down(b, 1, 32), b2 = __shfl_down(b, 2, 32), b3 = __shfl_down(b, 3, 32);
    if (store) {
        uint32_t *p = reinterpret_cast<uint32_t *>(blk);
        if ((i & 3) == 0) p[1 + (i >> 2)] = b | (b1 << 8) | (b2 << 16) | (b3 << 24);
        if (i == 0) p[0] = dbits | (sbits << 16);
    }
}

// Loads of one register chunk of one row: the policy's own chunk loader
// where it has one (constant offsets from per-plane bases), unit by unit
// otherwise.
template <class F, int U, int IT, int P, int B0 = 0, int B1 = IT, bool SCD = true>
__device__ __forceinline__ void load_chunk(const F &fmt, typename F::Raw (&r)[IT][P], int p, int64_t row,
                                           int unit0) {
    if constexpr (std::is_same<F, Q6Planar>::value) {
        fmt.template load_chunk<U, IT, P, B0, B1, SCD>(r, p, row, unit0);
    } else {
#pragma unroll
        for (int it = B0; it < B1; it++) fmt.load(r[it][p], row, unit0 + U * it);
    }
}

// ------------------------------------------------------------- the core
// Parameters of one MMVQ call as the kernel sees them.  Column n of the
// activation starts at Q8_1 block ((colpack >> 8n) & 255) * xstride of xq
// (a packed index rather than an array: a runtime-indexed array would be
// read from memory); dumps go to dump[n * rows * K/32 + row * K/32 + b].
struct MmvqArgs {
    const uint8_t *xq;
    int32_t *dump;
    int64_t rows, K;
    uint64_t colpack;
    int64_t xstride;
    int its;              // register steps staged per LDS sub-tile
    int nout;             // columns the dense kernel stores (its N, or fewer)
};

// First Q8_1 block of column n.
// (more than eight columns: only the batched tiled product, whose columns
// are consecutive)
template <int N>
__device__ __forceinline__ int64_t xcol_of(const MmvqArgs &a, int n) {
    if constexpr (N > 8) return (int64_t)n * a.xstride;
    return (int64_t)((a.colpack >> (8 * n)) & 255u) * a.xstride;
}

// p-th row of the calling lane in a workgroup that starts at row0: a wave
// holds P groups of 64/U consecutive rows, lane l takes row l/U of each.
template <int U, int P>
__device__ __forceinline__ int64_t lane_row(int64_t row0, int p) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    return row0 + ((int64_t)wave * P + p) * (kWave / U) + lane / U;
}

template <int U, int P>
constexpr int kRowsPerWave = P * (kWave / U);


// Register units whose weight loads are issued before the activation tile
// is stored (see mmvq_chunk); two measured best on the 10240 x 2560 and
// 8192 x 2560 Q6_K products (zero, one, three, four and all were slower).
constexpr int kPreUnits = 2;

// One register chunk of a call: units c0 + u + U*it (it < IT) of each of the
// lane's rows.  FULL: the chunk lies wholly inside the row, so every address
// is a constant offset from a per-lane base and no bound is checked.
template <bool FULL, class F, int N, int U, int P, int NTHR, bool DUMP, int IT, int PRE>
__device__ __forceinline__ void mmvq_chunk(const F &fmt, const MmvqArgs &a, void *lds, int c0, int units,
                                           const int64_t (&row)[P], const bool (&rok)[P], float (&acc)[P][N]) {
    constexpr int SBPU = F::SBPU;
    constexpr int ITS = its_for(IT, N, U, SBPU, NTHR);   // register steps per LDS sub-tile
    constexpr int TNB = ITS * U * SBPU;                  // tile column stride (blocks)
    // activation blocks per thread loaded ahead of the weights; item i is
    // block i % TNB of column i / TNB (a constant divisor)
    constexpr int SI = (N * TNB + NTHR - 1) / NTHR;
    const int tid = threadIdx.x;
    const int u = (tid & (kWave - 1)) % U;
    const int64_t nsb = a.K / 32;
    typename F::Raw r[IT][P];
    bool ok[IT];
    int sub_sb0 = c0 * SBPU;
    int sub_nsb = FULL ? TNB : min(TNB, (int)nsb - sub_sb0);
    // activation loads go first: loads retire in order, so waiting for them
    // does not wait for the weight loads behind them.  Unconditional (clamped
    // index), so the order survives scheduling.
    ActRaw ar[SI];
#pragma unroll
    for (int s = 0; s < SI; s++) {
        const int i = min(tid + s * NTHR, N * TNB - 1), n = i / TNB;
        const int b = FULL ? i - n * TNB : min(i - n * TNB, sub_nsb - 1);
        act_load(ar[s], a.xq, xcol_of<N>(a, n) + sub_sb0 + b);
    }
    __builtin_amdgcn_sched_barrier(0);
    const ActTile<TNB> t = act_tile<TNB>(lds, N);
    // Weight loads of the first PRE units go out with the activation loads;
    // then the tile is stored (waiting for the activation only) and the
    // remaining units' loads follow.  The tile thus arrives behind only a
    // fraction of the weight stream and the dot products start while most
    // weights are still in flight.  PRE = 0 stages the whole tile first.
    static_assert(PRE >= 0 && PRE <= IT, "pre-issued units");
    auto stage = [&]() {
#pragma unroll
        for (int s = 0; s < SI; s++) {
            const int i = tid + s * NTHR, n = i / TNB, b = i - n * TNB;
            if (i < N * TNB && (FULL || b < sub_nsb)) act_store<F::NEED_SUM>(t, i, ar[s], F::DSCALE);
        }
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // weight loads, unconditional (lanes past the end read a clamped, valid
    // address and ignore it): branches here would make the wait counts
    // conservative and serialize the stream behind the tile
    int64_t lrow[P];
#pragma unroll
    for (int p = 0; p < P; p++) lrow[p] = rok[p] ? row[p] : a.rows - 1;
    if constexpr (FULL) {
#pragma unroll
        for (int it = 0; it < IT; it++) ok[it] = true;
        if constexpr (PRE > 0) {
#pragma unroll
            for (int p = 0; p < P; p++) load_chunk<F, U, IT, P, 0, PRE, true>(fmt, r, p, lrow[p], c0 + u);
        }
        stage();
        if constexpr (PRE < IT) {
#pragma unroll
            for (int p = 0; p < P; p++) load_chunk<F, U, IT, P, PRE, IT, PRE == 0>(fmt, r, p, lrow[p], c0 + u);
        }
    } else {
        if constexpr (PRE == 0) stage();
#pragma unroll
        for (int it = 0; it < IT; it++) {
            const int unit = c0 + u + U * it;
            ok[it] = unit < units;
#pragma unroll
            for (int p = 0; p < P; p++) fmt.load(r[it][p], lrow[p], min(unit, units - 1));
        }
        if constexpr (PRE > 0) stage();
    }

#pragma unroll
    for (int st = 0; st < IT; st += ITS) {
        if (st > 0) {                                       // next LDS sub-tile
            if (!FULL && c0 + st * U >= units) break;
            lds_barrier();
            sub_sb0 = (c0 + st * U) * SBPU;
            sub_nsb = FULL ? TNB : min(TNB, (int)nsb - sub_sb0);
            for (int i = tid; i < N * TNB; i += NTHR) {
                const int n = i / TNB, b = i - n * TNB;
                if (FULL || b < sub_nsb) {
                    ActRaw x;
                    act_load(x, a.xq, xcol_of<N>(a, n) + sub_sb0 + b);
                    act_store<F::NEED_SUM>(t, i, x, F::DSCALE);
                }
            }
            lds_barrier();
        }
#pragma unroll
        for (int it = st; it < st + ITS && it < IT; it++) {
            if (FULL || ok[it]) {
                const int unit = c0 + u + U * it;
                const int tb = (u + U * (it - st)) * SBPU;
                int32_t *dp[P];
#pragma unroll
                for (int p = 0; p < P; p++)
                    dp[p] = DUMP ? a.dump + row[p] * nsb + (int64_t)unit * SBPU : nullptr;
                Dot<F>::template run<N, P, DUMP, TNB>(r[it], unit, t, tb, acc, dp, rok, a.rows * nsb);
            }
        }
    }
}

// Computes N dot products for P rows per lane of one workgroup (rows
// lane_row<U, P>(row0, p)) and leaves in acc[p][n] the full sum of (row p,
// column n), identical in every lane of the row's group.  Rows at or past
// a.rows compute on clamped data and must not be stored.  NTHR is the
// workgroup size, IT the register depth (units per lane held at once); lds
// holds at least N * its_for(IT, N, U, F::SBPU, NTHR) * U * F::SBPU *
// kActBytesPerBlock bytes.  Every thread of the workgroup must call it (it
// has barriers); it starts with no barrier, so a caller that reuses lds must
// place one before.  RAGGED = false: the caller guarantees that the row
// length is a whole number of register chunks (K/32/SBPU % (U*IT) == 0), and
// the ragged-chunk code is not compiled.
// Default pre-issued units: the dense one-workgroup-per-CU launches (long
// rows, more than 256 threads) stage the whole tile first, which measured
// better there; other launches issue kPreUnits units first.
__host__ __device__ constexpr int default_pre(int nthr, int it) {
    return nthr > 256 ? 0 : (kPreUnits < it ? kPreUnits : it);
}

template <class F, int N, int U, int P, int NTHR, bool DUMP, int IT = F::IT, bool RAGGED = true,
          int PRE = default_pre(NTHR, IT)>
__device__ __forceinline__ void mmvq_rows(const F &fmt, const MmvqArgs &a, int64_t row0, void *lds,
                                          float (&acc)[P][N]) {
    int64_t row[P];
    bool rok[P];
#pragma unroll
    for (int p = 0; p < P; p++) {
        row[p] = lane_row<U, P>(row0, p);
        rok[p] = row[p] < a.rows;
    }
    const int units = (int)(a.K / 32 / F::SBPU);
#pragma unroll
    for (int p = 0; p < P; p++)
#pragma unroll
        for (int n = 0; n < N; n++) acc[p][n] = 0.0f;

    constexpr int CH = U * IT;                              // units per register chunk
    const int nfull = units / CH;
    for (int c = 0; c < nfull; c++) {
        if (c > 0) lds_barrier();
        mmvq_chunk<true, F, N, U, P, NTHR, DUMP, IT, PRE>(fmt, a, lds, c * CH, units, row, rok, acc);
    }
    if constexpr (RAGGED) {                                 // ragged last chunk
        if (nfull * CH < units) {
            if (nfull > 0) lds_barrier();
            mmvq_chunk<false, F, N, U, P, NTHR, DUMP, IT, PRE>(fmt, a, lds, nfull * CH, units, row, rok, acc);
        }
    }
#pragma unroll
    for (int p = 0; p < P; p++)
#pragma unroll
        for (int n = 0; n < N; n++) acc[p][n] = group_sum<U>(acc[p][n]);
}

}  // namespace qmv

// misc.hip -- Q8_1 activation quantizer and the load-time Q6_K planar
// conversion (and its inverse).
#include "device.hpp"
#include "launch.hpp"

namespace qmv {

// Eight lanes per Q8_1 block, four consecutive values per lane: the max and
// the quant sum reduce inside each lane and then over the eight lanes with
// DPP (no cross-row exchange), and every lane writes its own dword of four
// quants.  x is [ncols][K], xq [ncols][K/32].  The arithmetic (max, d =
// max / 127, round(x / d), sum) is that of q8_1_quantize32.  PLANAR: the
// same bytes in the column-planar layout (per column of nb = K/32 blocks:
// the K quants, then nb fp16 d, then nb fp16 s).
template <bool PLANAR>
__global__ __launch_bounds__(256) void k_quantize_q8_1(const float *__restrict__ x, uint8_t *__restrict__ xq,
                                                       int64_t K, int64_t nblocks) {
    const int64_t g = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3;
    const int i = threadIdx.x & 7;
    const bool ok = g < nblocks;
    const int64_t nb = K / 32;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
        const int64_t col = g / nb, b = g - col * nb;
        const float *p = x + col * K + b * 32 + 4 * i;
#pragma unroll
        for (int k = 0; k < 4; k++) v[k] = p[k];
    }
    float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    a = dpp_max<0xB1>(a);     // lane ^ 1
    a = dpp_max<0x4E>(a);     // lane ^ 2
    a = dpp_max<0x141>(a);    // mirror within eight lanes
    const float d = a / 127.0f;
    int q[4] = {0, 0, 0, 0};
    if (d != 0.0f) {
#pragma unroll
        for (int k = 0; k < 4; k++) q[k] = (int)fminf(fmaxf(roundf(v[k] / d), -127.0f), 127.0f);
    }
    int s = q[0] + q[1] + q[2] + q[3];
    s = dpp_iadd<0xB1>(s);
    s = dpp_iadd<0x4E>(s);
    s = dpp_iadd<0x141>(s);
    if (ok) {
        const uint32_t qw = ((uint32_t)q[0] & 0xFFu) | (((uint32_t)q[1] & 0xFFu) << 8) |
                            (((uint32_t)q[2] & 0xFFu) << 16) | ((uint32_t)q[3] << 24);
        const uint32_t dbits = __builtin_bit_cast(uint16_t, (_Float16)d);
        const uint32_t sbits = q8_1_sum_bits(d, s);
        if constexpr (PLANAR) {
            const int64_t col = g / nb, b = g - col * nb;
            uint8_t *c = xq + col * nb * kQ81Bytes;
            reinterpret_cast<uint32_t *>(c + 32 * b)[i] = qw;
            if (i == 0) {
                reinterpret_cast<uint16_t *>(c + K)[b] = (uint16_t)dbits;
                reinterpret_cast<uint16_t *>(c + K + 2 * nb)[b] = (uint16_t)sbits;
            }
        } else {
            uint32_t *blk = reinterpret_cast<uint32_t *>(xq + g * kQ81Bytes);
            blk[1 + i] = qw;
            if (i == 0) blk[0] = dbits | (sbits << 16);
        }
    }
}

hipError_t launch_quantize(const float *x, uint8_t *xq, int64_t K, int ncols, bool planar, hipStream_t s) {
    const int64_t nblocks = (int64_t)ncols * (K / 32);
    const int64_t threads = nblocks * 8;
    const int64_t grid = (threads + 255) / 256;
    if (planar)
        hipLaunchKernelGGL(k_quantize_q8_1<true>, dim3((unsigned)grid), dim3(256), 0, s, x, xq, K, nblocks);
    else
        hipLaunchKernelGGL(k_quantize_q8_1<false>, dim3((unsigned)grid), dim3(256), 0, s, x, xq, K, nblocks);
    return hipGetLastError();
}

// Fused RMSNorm -> Q8_1: one 1024-thread workgroup per column.  Pass 1
// sums x^2 (fp32, fixed order: each thread's float4s in sequence, a 64-lane
// butterfly, the sixteen waves in order, so every thread holds the same
// sum); r = 1/sqrt(sum/K + eps) (IEEE division and square root); pass 2
// forms y = (x*r)*gamma and quantizes it with the arithmetic of
// k_quantize_q8_1 (eight lanes per block), in the Q8_1 blocks or the
// column-planar layout.  Up to K = 4096 thread t's one float4 of pass 1 is
// the one it quantizes in pass 2 (float4 8b + i is lane i of block b), so
// x is read once and each pass is one step; longer columns loop and read x
// again (from L2) for the codes.  (256 threads, three steps per pass at
// K = 2560: 3.6 us per launch of 13 columns; this form 2.9 us.)  No
// intermediate y in memory and one launch instead of a norm pass plus a
// quantize pass.
constexpr int kNormThreads = 1024;

template <bool PLANAR>
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm_q8_1(const float *__restrict__ x,
                                                               const float *__restrict__ gamma, float eps,
                                                               uint8_t *__restrict__ xq, int64_t K) {
    __shared__ float part[kNormThreads / kWave];
    const int64_t col = blockIdx.x, nb = K / 32, n4 = K / 4;
    const float *xc = x + col * K;
    const int tid = threadIdx.x, lane = tid & 63;
    const bool held = n4 <= kNormThreads;
    float4 xh = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float ss = 0.0f;
    if (held) {
        if (tid < n4) {
            xh = reinterpret_cast<const float4 *>(xc)[tid];
            ss = __builtin_fmaf(xh.x, xh.x, ss);
            ss = __builtin_fmaf(xh.y, xh.y, ss);
            ss = __builtin_fmaf(xh.z, xh.z, ss);
            ss = __builtin_fmaf(xh.w, xh.w, ss);
        }
    } else {
        for (int64_t i = tid; i < n4; i += kNormThreads) {
            const float4 v = reinterpret_cast<const float4 *>(xc)[i];
            ss = __builtin_fmaf(v.x, v.x, ss);
            ss = __builtin_fmaf(v.y, v.y, ss);
            ss = __builtin_fmaf(v.z, v.z, ss);
            ss = __builtin_fmaf(v.w, v.w, ss);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if (lane == 0) part[tid >> 6] = ss;
    __syncthreads();
    ss = part[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / kWave; w++) ss += part[w];
    const float r = 1.0f / sqrtf(ss / (float)K + eps);
    uint8_t *c = xq + col * nb * kQ81Bytes;
    const int i = tid & 7;
    for (int64_t b0 = 0; b0 < nb; b0 += kNormThreads / 8) {
        const int64_t b = b0 + (tid >> 3);
        const bool ok = b < nb;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (ok) {
            const float4 xv = held ? xh : reinterpret_cast<const float4 *>(xc + 32 * b)[i];
            const float4 gv = reinterpret_cast<const float4 *>(gamma + 32 * b)[i];
            v[0] = (xv.x * r) * gv.x;
            v[1] = (xv.y * r) * gv.y;
            v[2] = (xv.z * r) * gv.z;
            v[3] = (xv.w * r) * gv.w;
        }
        float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
        a = dpp_max<0xB1>(a);
        a = dpp_max<0x4E>(a);
        a = dpp_max<0x141>(a);
        const float d = a / 127.0f;
        int q[4] = {0, 0, 0, 0};
        if (d != 0.0f) {
#pragma unroll
            for (int k = 0; k < 4; k++) q[k] = (int)fminf(fmaxf(roundf(v[k] / d), -127.0f), 127.0f);
        }
        int s = q[0] + q[1] + q[2] + q[3];
        s = dpp_iadd<0xB1>(s);
        s = dpp_iadd<0x4E>(s);
        s = dpp_iadd<0x141>(s);
        if (ok) {
            const uint32_t qw = ((uint32_t)q[0] & 0xFFu) | (((uint32_t)q[1] & 0xFFu) << 8) |
                                (((uint32_t)q[2] & 0xFFu) << 16) | ((uint32_t)q[3] << 24);
            const uint32_t dbits = __builtin_bit_cast(uint16_t, (_Float16)d);
            const uint32_t sbits = q8_1_sum_bits(d, s);
            if constexpr (PLANAR) {
                reinterpret_cast<uint32_t *>(c + 32 * b)[i] = qw;
                if (i == 0) {
                    reinterpret_cast<uint16_t *>(c + K)[b] = (uint16_t)dbits;
                    reinterpret_cast<uint16_t *>(c + K + 2 * nb)[b] = (uint16_t)sbits;
                }
            } else {
                uint32_t *blk = reinterpret_cast<uint32_t *>(c + b * kQ81Bytes);
                blk[1 + i] = qw;
                if (i == 0) blk[0] = dbits | (sbits << 16);
            }
        }
    }
}

hipError_t launch_rmsnorm_quantize(const float *x, const float *gamma, float eps, uint8_t *xq, int64_t K, int ncols,
                                   bool planar, hipStream_t s) {
    if (planar)
        hipLaunchKernelGGL(k_rmsnorm_q8_1<true>, dim3((unsigned)ncols), dim3(kNormThreads), 0, s, x, gamma, eps, xq,
                           K);
    else
        hipLaunchKernelGGL(k_rmsnorm_q8_1<false>, dim3((unsigned)ncols), dim3(kNormThreads), 0, s, x, gamma, eps, xq,
                           K);
    return hipGetLastError();
}

// Where the parts of GGUF block t (row t / nb, block t % nb of the row) go
// in the planar layouts, in units of the part's size: 16-byte A and 8-byte B
// pieces of sub-block j, the two 8-byte halves of the scales, the 2-byte d.
//   planar: row-major, pieces t*8 + j, halves 2t + h, d t;
//   tiled:  16-row tiles (the last one R = rows - 16*tile rows high), row r
//           of the tile, sub-block s = 8*(t % nb) + j of the row:
//           pieces 16*tile*nsb + s*R + r, halves 16*tile*(nsb/4) + (2*(t%nb)
//           + h)*R + r, d 16*tile*nb + (t%nb)*R + r.
template <bool TILED>
struct PlaneIndex {
    int64_t rows, nb;
    __device__ __forceinline__ void at(int64_t t, int64_t &p0, int64_t &pstride, int64_t &h0, int64_t &hstride,
                                       int64_t &d) const {
        if constexpr (!TILED) {
            p0 = t * 8, pstride = 1, h0 = 2 * t, hstride = 1, d = t;
        } else {
            const int64_t row = t / nb, b = t - row * nb, tile = row >> 4, r = row & 15;
            const int64_t R = min((int64_t)16, rows - 16 * tile), nsb = 8 * nb;
            p0 = 16 * tile * nsb + 8 * b * R + r, pstride = R;
            h0 = 16 * tile * (nsb / 4) + 2 * b * R + r, hstride = R;
            d = 16 * tile * nb + b * R + r;
        }
    }
};

// GGUF Q6_K -> planar or tiled.  One thread per (block, sub-block j): it
// decodes the 32 six-bit values of sub-block j, writes its 16-byte plane-A
// and 8-byte plane-B pieces, and sub-block 0's thread copies the scales and d.
template <bool TILED>
__global__ __launch_bounds__(256) void k_repack_q6k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                    int64_t NB, PlaneIndex<TILED> ix) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= NB * 8) return;
    const int64_t t = gid >> 3;
    const int j = (int)(gid & 7), h = j >> 2, c = j & 3;
    const uint8_t *blk = src + t * kQ6Bytes;
    uint32_t v[32];
#pragma unroll
    for (int l = 0; l < 32; l++) {
        uint32_t lo = (blk[64 * h + 32 * (c & 1) + l] >> (4 * (c >> 1))) & 15u;
        uint32_t hi = (blk[128 + 32 * h + l] >> (2 * c)) & 3u;
        v[l] = (lo | (hi << 4)) ^ 32u;                 // (q6 - 32) mod 64
    }
    uint32_t A[4], B[2];
#pragma unroll
    for (int m = 0; m < 4; m++)
        A[m] = (v[4 * m] << 2) | (v[4 * m + 1] << 10) | (v[4 * m + 2] << 18) | (v[4 * m + 3] << 26);
#pragma unroll
    for (int m = 0; m < 2; m++)
        B[m] = (v[16 + 4 * m] << 2) | (v[17 + 4 * m] << 10) | (v[18 + 4 * m] << 18) | (v[19 + 4 * m] << 26);
    // spare bit pairs: weight 24+k -> bits 0-1 of A0, A1, A2 byte k (its
    // bits 0-1, 2-3, 4-5); weight 28+k -> A3, B0, B1 byte k
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t w24 = v[24 + k], w28 = v[28 + k];
        A[0] |= (w24 & 3u) << (8 * k);
        A[1] |= ((w24 >> 2) & 3u) << (8 * k);
        A[2] |= ((w24 >> 4) & 3u) << (8 * k);
        A[3] |= (w28 & 3u) << (8 * k);
        B[0] |= ((w28 >> 2) & 3u) << (8 * k);
        B[1] |= ((w28 >> 4) & 3u) << (8 * k);
    }
    int64_t p0, ps, h0, hs, di;
    ix.at(t, p0, ps, h0, hs, di);
    reinterpret_cast<uint4 *>(dst)[p0 + j * ps] = make_uint4(A[0], A[1], A[2], A[3]);
    reinterpret_cast<uint2 *>(dst + 128 * NB)[p0 + j * ps] = make_uint2(B[0], B[1]);
    if (j == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            uint8_t *sc = dst + 192 * NB + 8 * (h0 + hh * hs);
#pragma unroll
            for (int k = 0; k < 8; k++) sc[k] = blk[192 + 8 * hh + k];
        }
        dst[208 * NB + 2 * di] = blk[208];
        dst[208 * NB + 2 * di + 1] = blk[209];
    }
}

// planar or tiled -> GGUF Q6_K.  Eight threads per block, one per
// sub-block j: each decodes its 32 six-bit values from its plane-A and
// plane-B pieces into LDS; then thread k of the block assembles GGUF bytes
// 24k .. 24k+23 of ql/qh from the eight sub-blocks' values, and thread 0 also
// copies the scales and d.  (One thread per whole block held 192 bytes of
// ql/qh in registers: 256 VGPRs plus accumulation registers.)
constexpr int kUnpackThreads = 256, kUnpackBlocks = kUnpackThreads / 8;
template <bool TILED>
__global__ __launch_bounds__(kUnpackThreads) void k_unpack_q6k(const uint8_t *__restrict__ src,
                                                               uint8_t *__restrict__ dst, int64_t NB,
                                                               PlaneIndex<TILED> ix) {
    __shared__ uint8_t vals[kUnpackBlocks][8][32];          // (q6 - 32) mod 64 per sub-block position
    const int bl = threadIdx.x >> 3, j = threadIdx.x & 7;
    const int64_t t = (int64_t)blockIdx.x * kUnpackBlocks + bl;
    const bool live = t < NB;
    int64_t p0 = 0, ps = 0, h0 = 0, hs = 0, di = 0;
    if (live) {
        ix.at(t, p0, ps, h0, hs, di);
        const uint4 a = reinterpret_cast<const uint4 *>(src)[p0 + j * ps];
        const uint2 b = reinterpret_cast<const uint2 *>(src + 128 * NB)[p0 + j * ps];
        const uint32_t A[4] = {a.x, a.y, a.z, a.w}, B[2] = {b.x, b.y};
#pragma unroll
        for (int k = 0; k < 16; k++) vals[bl][j][k] = (uint8_t)((A[k >> 2] >> (8 * (k & 3) + 2)) & 63u);
#pragma unroll
        for (int k = 0; k < 8; k++) vals[bl][j][16 + k] = (uint8_t)((B[k >> 2] >> (8 * (k & 3) + 2)) & 63u);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int sh = 8 * k;
            vals[bl][j][24 + k] =
                (uint8_t)(((A[0] >> sh) & 3u) | (((A[1] >> sh) & 3u) << 2) | (((A[2] >> sh) & 3u) << 4));
            vals[bl][j][28 + k] =
                (uint8_t)(((A[3] >> sh) & 3u) | (((B[0] >> sh) & 3u) << 2) | (((B[1] >> sh) & 3u) << 4));
        }
    }
    __syncthreads();
    if (!live) return;
    uint8_t *blk = dst + t * kQ6Bytes;
    for (int i = 24 * j; i < 24 * j + 24; i++) {
        uint32_t byte;
        if (i < 128) {
            // ql byte 64h + 32(c%2) + l: the low nibble from c = c%2, the
            // high one from c = c%2 + 2 (sub-blocks 4h + c)
            const int h = i >> 6, c1 = (i >> 5) & 1, l = i & 31;
            const uint32_t lo = (vals[bl][4 * h + c1][l] ^ 32u) & 15u;
            const uint32_t hi = (vals[bl][4 * h + c1 + 2][l] ^ 32u) & 15u;
            byte = lo | (hi << 4);
        } else {
            // qh byte 32h + l: bits 2c from sub-block 4h + c
            const int h = (i - 128) >> 5, l = (i - 128) & 31;
            byte = 0;
#pragma unroll
            for (int c = 0; c < 4; c++) byte |= (((vals[bl][4 * h + c][l] ^ 32u) >> 4) & 3u) << (2 * c);
        }
        blk[i] = (uint8_t)byte;
    }
    if (j == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            const uint8_t *sc = src + 192 * NB + 8 * (h0 + hh * hs);
#pragma unroll
            for (int k = 0; k < 8; k++) blk[192 + 8 * hh + k] = sc[k];
        }
        blk[208] = src[208 * NB + 2 * di];
        blk[209] = src[208 * NB + 2 * di + 1];
    }
}

// Streaming-read calibration: the fastest plain read of a buffer found on
// this GPU.  Every thread issues four independent 16-byte non-temporal loads
// per step (a grid-stride loop; with the default grid each thread takes one
// step), folds them with XOR and stores only if the fold hits a fixed
// value, so the loads stay live without write traffic.
__global__ __launch_bounds__(256) void k_stream_read(const uint4 *__restrict__ src, int64_t n16,
                                                     uint32_t *__restrict__ sink) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 *p = reinterpret_cast<const u32x4 *>(src);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x * 4 + threadIdx.x; i < n16; i += stride) {
        u32x4 v[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int64_t j = min(i + (int64_t)k * blockDim.x, n16 - 1);
            v[k] = __builtin_nontemporal_load(p + j);
        }
#pragma unroll
        for (int k = 0; k < 4; k++) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
    }
    if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int blocks, hipStream_t s) {
    const int64_t n16 = bytes / 16;
    const int64_t grid = blocks > 0 ? blocks : (n16 + 1023) / 1024;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, s, reinterpret_cast<const uint4 *>(src),
                       n16, sink);
    return hipGetLastError();
}

// Row gather in one layout: output row j is source row ids[j] (a draft head
// taken from the planar LM head).  One thread per (output row, block): the
// block's eight A and B pieces, its two scale halves and d.  GGUF layout
// (LAYOUT 0): the 210-byte block is copied as it is.  An id outside
// [0, rows) gives an all-zero output row.
template <int LAYOUT>
__global__ __launch_bounds__(256) void k_gather_q6k(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                    const int32_t *__restrict__ ids, int64_t rows, int64_t nout,
                                                    int64_t nb) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= nout * nb) return;
    const int64_t j = gid / nb, b = gid - j * nb;
    const int32_t id = ids[j];
    const bool ok = id >= 0 && id < rows;
    const int64_t ts = (ok ? id : 0) * nb + b, td = j * nb + b;   // source and output block
    if constexpr (LAYOUT == 0) {
        const uint8_t *ps = src + ts * kQ6Bytes;
        uint8_t *pd = dst + td * kQ6Bytes;
        for (int k = 0; k < kQ6Bytes; k++) pd[k] = ok ? ps[k] : 0;
    } else {
        constexpr bool TILED = LAYOUT == 2;
        const int64_t NBs = rows * nb, NBd = nout * nb;
        int64_t sp, sps, sh, shs, sd, dp, dps, dh, dhs, dd;
        PlaneIndex<TILED>{rows, nb}.at(ts, sp, sps, sh, shs, sd);
        PlaneIndex<TILED>{nout, nb}.at(td, dp, dps, dh, dhs, dd);
#pragma unroll
        for (int k = 0; k < 8; k++) {
            uint4 a = make_uint4(0, 0, 0, 0);
            uint2 bb = make_uint2(0, 0);
            if (ok) {
                a = reinterpret_cast<const uint4 *>(src)[sp + k * sps];
                bb = reinterpret_cast<const uint2 *>(src + 128 * NBs)[sp + k * sps];
            }
            reinterpret_cast<uint4 *>(dst)[dp + k * dps] = a;
            reinterpret_cast<uint2 *>(dst + 128 * NBd)[dp + k * dps] = bb;
        }
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint2 sc = make_uint2(0, 0);
            if (ok) sc = reinterpret_cast<const uint2 *>(src + 192 * NBs)[sh + h * shs];
            reinterpret_cast<uint2 *>(dst + 192 * NBd)[dh + h * dhs] = sc;
        }
        uint16_t dv = 0;
        if (ok) dv = reinterpret_cast<const uint16_t *>(src + 208 * NBs)[sd];
        reinterpret_cast<uint16_t *>(dst + 208 * NBd)[dd] = dv;
    }
}

hipError_t launch_gather(const uint8_t *src, uint8_t *dst, const int32_t *ids, int64_t rows, int64_t nout,
                         int64_t K, int layout, hipStream_t s) {
    const int64_t nb = K / 256;
    const dim3 grid((unsigned)((nout * nb + 255) / 256));
    if (layout == 2)
        hipLaunchKernelGGL(k_gather_q6k<2>, grid, dim3(256), 0, s, src, dst, ids, rows, nout, nb);
    else if (layout == 1)
        hipLaunchKernelGGL(k_gather_q6k<1>, grid, dim3(256), 0, s, src, dst, ids, rows, nout, nb);
    else
        hipLaunchKernelGGL(k_gather_q6k<0>, grid, dim3(256), 0, s, src, dst, ids, rows, nout, nb);
    return hipGetLastError();
}

hipError_t launch_repack(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K, bool tiled, hipStream_t s) {
    const int64_t nb = K / 256, NB = rows * nb;
    const dim3 grid((unsigned)((NB * 8 + 255) / 256));
    if (tiled)
        hipLaunchKernelGGL(k_repack_q6k<true>, grid, dim3(256), 0, s, src, dst, NB, PlaneIndex<true>{rows, nb});
    else
        hipLaunchKernelGGL(k_repack_q6k<false>, grid, dim3(256), 0, s, src, dst, NB, PlaneIndex<false>{rows, nb});
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K, bool tiled, hipStream_t s) {
    const int64_t nb = K / 256, NB = rows * nb;
    const dim3 grid((unsigned)((NB + kUnpackBlocks - 1) / kUnpackBlocks));
    if (tiled)
        hipLaunchKernelGGL(k_unpack_q6k<true>, grid, dim3(kUnpackThreads), 0, s, src, dst, NB,
                           PlaneIndex<true>{rows, nb});
    else
        hipLaunchKernelGGL(k_unpack_q6k<false>, grid, dim3(kUnpackThreads), 0, s, src, dst, NB,
                           PlaneIndex<false>{rows, nb});
    return hipGetLastError();
}

}  // namespace qmv

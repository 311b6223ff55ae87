// topk.hip -- the k largest rows of each column of a product (the verify
// window's candidate tokens over an LM head).
//
// Keys: an output's float bits made order-preserving as an unsigned
// integer (-0 as +0) above the complement of its row, so that keys are
// unique and nonzero, a larger key is a larger value and, among equal
// values, the lower row.  Key 0 marks an empty slot.  Two launches after the
// product (whose fp32 outputs sit in the workspace):
//   k_topk_chunks  one workgroup per (chunk of kTopkChunk rows, column): the
//                  chunk's keys in LDS, the k-th largest found by a radix
//                  select over 8-bit digits (an LDS histogram per digit, a
//                  wave suffix scan to find the digit holding the k-th key,
//                  stop as soon as every key sharing the decided prefix is
//                  in), the k largest keys written unordered as candidates;
//   k_topk_final   one workgroup per column: the same select over the
//                  column's candidates, then each winner's place found by
//                  counting the winners above it (k <= 64), decoded.
// Both read and write plain global memory and LDS only; every loop is
// bounded by kTopkChunk or the digit count.
#include "launch.hpp"

namespace qmv {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kTopkPer = kTopkChunk / kTopkThreads;     // keys per thread of a full chunk
static_assert(kTopkChunk % kTopkThreads == 0, "whole loads per thread");

__device__ __forceinline__ uint64_t topk_key(float v, uint32_t row) {
    uint32_t b = __float_as_uint(v + 0.0f);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint64_t)(0xFFFFFFFFu - row);
}

struct SelectLds {
    uint64_t key[kTopkChunk];
    uint64_t sel[kTopkMax];
    int hist[256];
    int digit, above, at, nsel;
};

// Marks in s.sel the `need` largest nonzero keys of s.key[0..m) (there are
// at least `need`), in no particular order.  Every thread of the workgroup
// calls it.
__device__ void select_largest(SelectLds &s, int m, int need) {
    const int t = threadIdx.x;
    uint64_t prefix = 0, mask = 0;
    for (int shift = 56; shift >= 0; shift -= 8) {
        s.hist[t] = 0;                                    // kTopkThreads == 256 bins
        __syncthreads();
        // every LDS read of the pass issued before the first count (the
        // array holds kTopkChunk keys; entries from m on are not counted)
        uint64_t kv[kTopkPer];
#pragma unroll
        for (int j = 0; j < kTopkPer; j++) kv[j] = s.key[t + j * kTopkThreads];
#pragma unroll
        for (int j = 0; j < kTopkPer; j++) {
            const uint64_t key = kv[j];
            if (t + j * kTopkThreads < m && key != 0 && (key & mask) == prefix)
                atomicAdd(&s.hist[(int)(key >> shift) & 255], 1);
        }
        __syncthreads();
        if (t < 64) {                                     // wave 0: bins 4t .. 4t+3, suffix sums over lanes
            const int h0 = s.hist[4 * t], h1 = s.hist[4 * t + 1], h2 = s.hist[4 * t + 2], h3 = s.hist[4 * t + 3];
            const int own = h0 + h1 + h2 + h3;
            int suf = own;
            for (int off = 1; off < 64; off <<= 1) {
                const int v = __shfl_down(suf, off, 64);
                if (t + off < 64) suf += v;
            }
            const int higher = suf - own;                 // keys in bins above this lane's four
            if (higher < need && suf >= need) {           // exactly one lane
                int acc = higher, d = 4 * t + 3, hd = h3;
                if (acc + h3 < need) {
                    acc += h3; d = 4 * t + 2; hd = h2;
                    if (acc + h2 < need) {
                        acc += h2; d = 4 * t + 1; hd = h1;
                        if (acc + h1 < need) { acc += h1; d = 4 * t; hd = h0; }
                    }
                }
                s.digit = d;
                s.above = acc;
                s.at = hd;
            }
        }
        __syncthreads();
        const int d = s.digit, above = s.above, at = s.at;
        prefix |= (uint64_t)d << shift;
        mask |= (uint64_t)255 << shift;
        need -= above;
        if (at == need) break;                            // every key with this prefix is in (always at shift 0)
        __syncthreads();                                  // the next pass clears hist
    }
    if (t == 0) s.nsel = 0;
    __syncthreads();
    uint64_t kv[kTopkPer];
#pragma unroll
    for (int j = 0; j < kTopkPer; j++) kv[j] = s.key[t + j * kTopkThreads];
#pragma unroll
    for (int j = 0; j < kTopkPer; j++) {
        const uint64_t key = kv[j];
        if (t + j * kTopkThreads < m && key != 0 && (key & mask) >= prefix) s.sel[atomicAdd(&s.nsel, 1)] = key;
    }
    __syncthreads();
}

// Chunk c of column n: rows c*kTopkChunk ..; its min(k, rows in the chunk)
// largest keys to cand[(n * nchunks + c) * k ..], the rest of the k slots 0.
__global__ __launch_bounds__(kTopkThreads) void k_topk_chunks(const float *__restrict__ out, int64_t rows, int k,
                                                              int nchunks, uint64_t *__restrict__ cand) {
    __shared__ SelectLds s;
    const int n = blockIdx.y, c = blockIdx.x;
    const float *o = out + (int64_t)n * rows;
    const int64_t r0 = (int64_t)c * kTopkChunk;
    const int m = (int)(rows - r0 < kTopkChunk ? rows - r0 : kTopkChunk);
    // every load of the thread in flight before the first key is stored:
    // unconditional loads from indices clamped into the chunk (a load per
    // key stored as it arrived, or a branch around each load, waited for
    // each in turn: ~13 us for the 38 chunks of a 151,936-row column)
    float v[kTopkPer];
#pragma unroll
    for (int j = 0; j < kTopkPer; j++) v[j] = o[r0 + min((int)threadIdx.x + j * kTopkThreads, m - 1)];
#pragma unroll
    for (int j = 0; j < kTopkPer; j++) {
        const int i = threadIdx.x + j * kTopkThreads;
        if (i < m) s.key[i] = topk_key(v[j], (uint32_t)(r0 + i));
    }
    __syncthreads();
    const int need = m < k ? m : k;
    select_largest(s, m, need);
    uint64_t *dst = cand + ((int64_t)n * nchunks + c) * k;
    for (int i = threadIdx.x; i < k; i += kTopkThreads) dst[i] = i < need ? s.sel[i] : 0;
}

// Column n: the k largest of its nchunks * k candidates (at most
// kTopkChunk), placed in descending order and decoded.
__global__ __launch_bounds__(kTopkThreads) void k_topk_final(const uint64_t *__restrict__ cand, int k, int nchunks,
                                                             int32_t *__restrict__ idx, float *__restrict__ val) {
    __shared__ SelectLds s;
    const int n = blockIdx.x, m = nchunks * k;          // 1 <= m <= kTopkChunk (checked by the caller)
    uint64_t v[kTopkPer];
#pragma unroll
    for (int j = 0; j < kTopkPer; j++) v[j] = cand[(int64_t)n * m + min((int)threadIdx.x + j * kTopkThreads, m - 1)];
#pragma unroll
    for (int j = 0; j < kTopkPer; j++) {
        const int i = threadIdx.x + j * kTopkThreads;
        if (i < m) s.key[i] = v[j];
    }
    __syncthreads();
    select_largest(s, m, k);
    const int t = threadIdx.x;
    if (t < k) {
        const uint64_t kk = s.sel[t];
        int place = 0;
        for (int j = 0; j < k; ++j) place += s.sel[j] > kk;
        const uint32_t b = (uint32_t)(kk >> 32);
        idx[n * k + place] = (int32_t)(0xFFFFFFFFu - (uint32_t)kk);
        val[n * k + place] = __uint_as_float((b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
    }
}

}  // namespace

hipError_t launch_topk(const float *out, int64_t rows, int ncols, int k, uint64_t *cand, int32_t *idx, float *val,
                       hipStream_t s) {
    const int nchunks = (int)((rows + kTopkChunk - 1) / kTopkChunk);
    hipLaunchKernelGGL(k_topk_chunks, dim3((unsigned)nchunks, (unsigned)ncols), dim3(kTopkThreads), 0, s, out, rows,
                       k, nchunks, cand);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_topk_final, dim3((unsigned)ncols), dim3(kTopkThreads), 0, s, cand, k, nchunks, idx, val);
    return hipGetLastError();
}

}  // namespace qmv

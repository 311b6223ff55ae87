// mmvq_q6_tiled.hip -- instantiations of the tiled-layout Q6_K MMVQ.
#include "mmq_tiled.hpp"
#include "mmvq_tiled.hpp"

namespace qmv {
template <bool DUMP, bool XP>
static hipError_t tiled_cols(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                             int ncols, hipStream_t s) {
    switch (ncols) {
    case 1: return launch_tiled_n<1, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 2: return launch_tiled_n<2, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 3: return launch_tiled_n<3, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 4: return launch_tiled_n<4, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 5: return launch_tiled_n<5, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 6: return launch_tiled_n<6, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 7: return launch_tiled_n<7, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    case 8: return launch_tiled_n<8, DUMP, false, XP>(w, xq, out, dump, rows, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mmvq_q6_tiled(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                                int ncols, bool xp, hipStream_t s) {
    if (xp)
        return dump ? tiled_cols<true, true>(w, xq, out, dump, rows, K, ncols, s)
                    : tiled_cols<false, true>(w, xq, out, dump, rows, K, ncols, s);
    return dump ? tiled_cols<true, false>(w, xq, out, dump, rows, K, ncols, s)
                : tiled_cols<false, false>(w, xq, out, dump, rows, K, ncols, s);
}

hipError_t launch_mmvq_q6_tiled_jobs(const TiledJobDesc *jobs, int njobs, int64_t K, bool xp, hipStream_t s) {
    if (njobs < 1 || njobs > kMaxTiledJobs) return hipErrorInvalidValue;
    TiledJobs<kMaxTiledJobs> js;
    js.njobs = njobs;
    js.K = K;
    for (int j = 0; j < njobs; j++) {
        js.job[j].w = jobs[j].w;
        js.job[j].xq = reinterpret_cast<const uint8_t *>(jobs[j].xq);
        js.job[j].out = jobs[j].out;
        js.job[j].rows = jobs[j].rows;
        js.job[j].ncols = jobs[j].ncols;
        js.job[j].wg0 = 0;
    }
    return xp ? launch_tiled_jobs<true>(js, s) : launch_tiled_jobs<false>(js, s);
}

// Batched product of any number of columns: full batches in one launch,
// the rest (fewer than a batch) as products of at most eight columns.
hipError_t launch_mmq_q6_tiled(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int ncols,
                               bool xp, hipStream_t s) {
    // weights held across batches where K is one whole chunk and there are
    // enough columns; else one workgroup per (row tiles, batch)
    const int BW = mmq_ws_batch_cols(K, ncols, xp);
    const int B = BW ? BW : tiled_batch_cols(K);
    const int64_t nbat = ncols / B, cstride = 36 * (K / 32);
    if (nbat > 0) {
        const hipError_t e = BW ? (xp ? launch_mmq_ws<true>(w, xq, out, rows, K, (int)nbat, s)
                                      : launch_mmq_ws<false>(w, xq, out, rows, K, (int)nbat, s))
                             : xp ? launch_tiled_batched<true>(w, xq, out, rows, K, nbat, s)
                                  : launch_tiled_batched<false>(w, xq, out, rows, K, nbat, s);
        if (e != hipSuccess) return e;
    }
    for (int n0 = (int)nbat * B; n0 < ncols; n0 += 8) {
        const int n = ncols - n0 < 8 ? ncols - n0 : 8;
        const void *x = static_cast<const uint8_t *>(xq) + n0 * cstride;
        float *o = out + n0 * rows;
        const hipError_t e = xp ? tiled_cols<false, true>(w, x, o, nullptr, rows, K, n, s)
                                : tiled_cols<false, false>(w, x, o, nullptr, rows, K, n, s);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Fused greedy argmax: the product's per-tile column maxima into keys, then
// one reduction launch.
template <bool XP>
static hipError_t tiled_argmax_cols(const void *w, const void *xq, float *k, int64_t rows, int64_t K, int ncols,
                                    hipStream_t s) {
    switch (ncols) {
    case 1: return launch_tiled_n<1, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 2: return launch_tiled_n<2, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 3: return launch_tiled_n<3, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 4: return launch_tiled_n<4, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 5: return launch_tiled_n<5, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 6: return launch_tiled_n<6, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 7: return launch_tiled_n<7, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    case 8: return launch_tiled_n<8, false, true, XP>(w, xq, k, nullptr, rows, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mmvq_q6_tiled_argmax(const void *w, const void *xq, uint64_t *keys, int64_t rows, int64_t K,
                                       int ncols, int32_t *idx, float *val, bool xp, hipStream_t s) {
    float *k = reinterpret_cast<float *>(keys);
    const hipError_t e = xp ? tiled_argmax_cols<true>(w, xq, k, rows, K, ncols, s)
                            : tiled_argmax_cols<false>(w, xq, k, rows, K, ncols, s);
    if (e != hipSuccess) return e;
    const int64_t ntiles = (rows + 15) / 16;
    hipLaunchKernelGGL(k_argmax_reduce, dim3(ncols, (unsigned)((ntiles + kArgmaxSpan - 1) / kArgmaxSpan)),
                       dim3(kArgmaxThreads), 0, s, keys, ntiles, ncols, idx, val);
    return hipGetLastError();
}
}  // namespace qmv

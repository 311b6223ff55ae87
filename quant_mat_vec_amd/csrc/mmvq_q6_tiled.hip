// mmvq_q6_tiled.hip -- instantiations of the tiled-layout Q6_K MMVQ.
#include "mmvq_tiled.hpp"

namespace qmv {
template <bool DUMP>
static hipError_t tiled_cols(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                             int ncols, hipStream_t s) {
    switch (ncols) {
    case 1: return launch_tiled_n<1, DUMP>(w, xq, out, dump, rows, K, s);
    case 2: return launch_tiled_n<2, DUMP>(w, xq, out, dump, rows, K, s);
    case 3: return launch_tiled_n<3, DUMP>(w, xq, out, dump, rows, K, s);
    case 4: return launch_tiled_n<4, DUMP>(w, xq, out, dump, rows, K, s);
    case 5: return launch_tiled_n<5, DUMP>(w, xq, out, dump, rows, K, s);
    case 6: return launch_tiled_n<6, DUMP>(w, xq, out, dump, rows, K, s);
    case 7: return launch_tiled_n<7, DUMP>(w, xq, out, dump, rows, K, s);
    case 8: return launch_tiled_n<8, DUMP>(w, xq, out, dump, rows, K, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mmvq_q6_tiled(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                                int ncols, hipStream_t s) {
    return dump ? tiled_cols<true>(w, xq, out, dump, rows, K, ncols, s)
                : tiled_cols<false>(w, xq, out, dump, rows, K, ncols, s);
}

// Fused greedy argmax: the product's per-tile column maxima into keys, then
// one reduction launch.
hipError_t launch_mmvq_q6_tiled_argmax(const void *w, const void *xq, uint64_t *keys, int64_t rows, int64_t K,
                                       int ncols, int32_t *idx, float *val, hipStream_t s) {
    float *k = reinterpret_cast<float *>(keys);
    hipError_t e;
    switch (ncols) {
    case 1: e = launch_tiled_n<1, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 2: e = launch_tiled_n<2, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 3: e = launch_tiled_n<3, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 4: e = launch_tiled_n<4, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 5: e = launch_tiled_n<5, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 6: e = launch_tiled_n<6, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 7: e = launch_tiled_n<7, false, true>(w, xq, k, nullptr, rows, K, s); break;
    case 8: e = launch_tiled_n<8, false, true>(w, xq, k, nullptr, rows, K, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_reduce, dim3(ncols), dim3(kArgmaxThreads), 0, s, keys, (rows + 15) / 16, idx, val);
    return hipGetLastError();
}
}  // namespace qmv

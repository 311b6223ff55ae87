// mmvq_q4.hip -- dense MMVQ instantiations for one weight format.
#include "mmvq_dense.hpp"

namespace qmv {
hipError_t launch_mmvq_q4(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows,
                            int64_t K, int ncols, hipStream_t s) {
    return launch_dense_any<Q45<false>>(w, xq, out, dump, rows, K, ncols, s);
}
}  // namespace qmv

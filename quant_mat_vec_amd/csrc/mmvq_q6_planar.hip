// mmvq_q6_planar.hip -- dense MMVQ instantiations for one weight format.
#include "mmvq_dense.hpp"

namespace qmv {
hipError_t launch_mmvq_q6_planar(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows,
                            int64_t K, int ncols, hipStream_t s) {
    return launch_dense_any<Q6Planar>(w, xq, out, dump, rows, K, ncols, s);
}
}  // namespace qmv

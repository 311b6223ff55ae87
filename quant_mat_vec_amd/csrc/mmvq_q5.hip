// mmvq_q5.hip -- dense MMVQ instantiations for one weight format.
#include "mmvq_dense.hpp"

namespace qmv {
hipError_t launch_mmvq_q5(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows,
                            int64_t K, int ncols, hipStream_t s) {
    return launch_dense_any<Q45<true>>(w, xq, out, dump, rows, K, ncols, s);
}
hipError_t launch_mmvq_q5_jobs(const TiledJobDesc *jobs, int njobs, int64_t K, hipStream_t s) {
    DenseJob d[kMaxDenseJobs];
    for (int j = 0; j < njobs; j++)
        d[j] = {jobs[j].w, reinterpret_cast<const uint8_t *>(jobs[j].xq), jobs[j].out, (int32_t)jobs[j].rows,
                jobs[j].ncols, 0, 0};
    return launch_dense_jobs<Q45<true>>(d, njobs, K, s);
}
}  // namespace qmv

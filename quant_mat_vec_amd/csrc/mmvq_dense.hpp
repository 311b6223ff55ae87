// mmvq_dense.hpp -- the dense MMVQ kernel and its compile-time dispatch on
// (lanes per row U, columns N, dump flag).  Included by one source file per
// weight format so the instantiations compile in parallel.
#pragma once

#include "device.hpp"
#include "launch.hpp"

namespace qmv {

#ifndef QMV_DENSE_WAVES
#define QMV_DENSE_WAVES 4
#endif
constexpr int kDenseWaves = QMV_DENSE_WAVES;

// Rows per lane group: one.  (The core takes P rows per lane; two rows, which
// halve the activation reads from LDS, measured no faster at 1-8 columns.)
template <int N>
constexpr int kDenseP = 1;

// W waves per workgroup; the kernel is compiled for up to kMaxDenseWaves.
constexpr int kMaxDenseWaves = 10;

template <class F, int N, int U, int W, int IT, bool DUMP>
__global__ __launch_bounds__(W * kWave) void k_mmvq_dense(const void *__restrict__ w, MmvqArgs a,
                                                        float *__restrict__ out) {
    constexpr int P = kDenseP<N>;
    extern __shared__ __align__(16) uint8_t lds[];
    F fmt;
    fmt.init(w, a.rows, a.K);
    const int64_t row0 = (int64_t)blockIdx.x * W * kRowsPerWave<U, P>;
    float acc[P][N];
    mmvq_rows<F, N, U, P, W * kWave, DUMP, IT>(fmt, a, row0, lds, acc);
    if constexpr (!DUMP) {
        // every lane of a row holds all N sums; lane u < N of the row stores
        // column u (U >= 8 >= N)
        static_assert(U >= N, "one lane per column");
        const int u = (threadIdx.x & (kWave - 1)) % U;
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int64_t row = lane_row<U, P>(row0, p);
            float v = acc[p][0];
#pragma unroll
            for (int n = 1; n < N; n++) v = u == n ? acc[p][n] : v;
            if (row < a.rows && u < N && u < a.nout) out[(int64_t)u * a.rows + row] = v;
        }
    }
}

// ncols <= N real columns: columns ncols .. N-1 of the kernel read the last
// real column again and are not stored.
template <class F, int N, int U, int W, int IT, bool DUMP>
hipError_t launch_dense_nuw(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                            hipStream_t s, int ncols = N) {
    constexpr int threads = W * kWave;
    constexpr int its = its_for(IT, N, U, F::SBPU, threads);
    MmvqArgs a;
    a.xq = reinterpret_cast<const uint8_t *>(xq);
    a.dump = dump;
    a.rows = rows;
    a.K = K;
    a.colpack = 0;
    for (int n = 0; n < 8; n++) a.colpack |= (uint64_t)(n < ncols ? n : ncols - 1) << (8 * n);
    a.nout = ncols;
    a.xstride = K / 32;
    a.its = its;
    const size_t lds = (size_t)N * its * U * F::SBPU * kActBytesPerBlock;
    const int64_t rpb = W * kRowsPerWave<U, kDenseP<N>>;
    const int64_t grid = (rows + rpb - 1) / rpb;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_mmvq_dense<F, N, U, W, IT, DUMP>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_mmvq_dense<F, N, U, W, IT, DUMP>), dim3((unsigned)grid), dim3(threads), lds, s, w, a,
                       out);
    return hipGetLastError();
}

// Ten-wave workgroups for long rows (a wave holds at most two rows) when that
// still gives about one workgroup per CU or more: the activation tile is then
// staged once per CU rather than once per four waves.  Four-wave workgroups
// otherwise.
#ifndef QMV_DENSE_BIG_GRID
#define QMV_DENSE_BIG_GRID 224
#endif
template <class F, int N, int U, int IT, bool DUMP>
hipError_t launch_dense_nui(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                            hipStream_t s, int ncols) {
    // (not for Q5_K: its registers do not fit three waves per SIMD)
    if constexpr (!DUMP && kRowsPerWave<U, kDenseP<N>> <= 2 && sizeof(typename F::Raw) <= 64) {
        constexpr int64_t rpb10 = kMaxDenseWaves * kRowsPerWave<U, kDenseP<N>>;
        if ((rows + rpb10 - 1) / rpb10 >= QMV_DENSE_BIG_GRID)
            // (seven columns at depth five do not fit 168 registers)
            return launch_dense_nuw<F, N, U, kMaxDenseWaves, (N == 7 ? 3 : IT), DUMP>(w, xq, out, dump, rows, K, s,
                                                                                      ncols);
    }
    return launch_dense_nuw<F, N, U, kDenseWaves, IT, DUMP>(w, xq, out, dump, rows, K, s, ncols);
}

template <class F, int N, int U, bool DUMP>
hipError_t launch_dense_nu(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                           hipStream_t s, int ncols = N) {
    const int units = (int)(K / 32 / F::SBPU);
    if constexpr (F::IT > 3) {
        if (depth_for(units, U, F::IT) == 3)
            return launch_dense_nui<F, N, U, 3, DUMP>(w, xq, out, dump, rows, K, s, ncols);
    }
    return launch_dense_nui<F, N, U, F::IT, DUMP>(w, xq, out, dump, rows, K, s, ncols);
}

// Q4_K/Q5_K at six or seven columns with 32 or 64 lanes per row: the
// compiler puts those instantiations at 256 VGPRs plus accumulation
// registers (one wave per SIMD) while eight columns fit in 140-187.  The
// products run on the eight-column kernel with the last real column read
// again for the missing ones and only the real columns stored; the
// per-sub-block sums (a test dump) run as four columns, then the rest.
// Every column's arithmetic is the same at any column count, so the bits
// do not change.
template <class F, int U>
constexpr bool kDenseWide67 = F::SBPU == 2 && U >= 32;

template <class F, int U, bool DUMP>
hipError_t launch_dense_u(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                          int ncols, hipStream_t s) {
    if constexpr (kDenseWide67<F, U>) {
        if (ncols == 6 || ncols == 7) {
            if constexpr (DUMP) {
                const hipError_t e = launch_dense_nu<F, 4, U, DUMP>(w, xq, out, dump, rows, K, s);
                if (e != hipSuccess) return e;
                const uint8_t *x4 = static_cast<const uint8_t *>(xq) + 4 * (K / 32) * kQ81Bytes;
                int32_t *d4 = dump + 4 * rows * (K / 32);
                return ncols == 6 ? launch_dense_nu<F, 2, U, DUMP>(w, x4, out, d4, rows, K, s)
                                  : launch_dense_nu<F, 3, U, DUMP>(w, x4, out, d4, rows, K, s);
            } else {
                return launch_dense_nu<F, 8, U, DUMP>(w, xq, out, dump, rows, K, s, ncols);
            }
        }
    }
    switch (ncols) {
    case 1: return launch_dense_nu<F, 1, U, DUMP>(w, xq, out, dump, rows, K, s);
    case 2: return launch_dense_nu<F, 2, U, DUMP>(w, xq, out, dump, rows, K, s);
    case 3: return launch_dense_nu<F, 3, U, DUMP>(w, xq, out, dump, rows, K, s);
    case 4: return launch_dense_nu<F, 4, U, DUMP>(w, xq, out, dump, rows, K, s);
    case 5: return launch_dense_nu<F, 5, U, DUMP>(w, xq, out, dump, rows, K, s);
    case 6:
        if constexpr (!kDenseWide67<F, U>) return launch_dense_nu<F, 6, U, DUMP>(w, xq, out, dump, rows, K, s);
        return hipErrorInvalidValue;
    case 7:
        if constexpr (!kDenseWide67<F, U>) return launch_dense_nu<F, 7, U, DUMP>(w, xq, out, dump, rows, K, s);
        return hipErrorInvalidValue;
    case 8: return launch_dense_nu<F, 8, U, DUMP>(w, xq, out, dump, rows, K, s);
    default: return hipErrorInvalidValue;
    }
}

constexpr int64_t kDenseFillWaves = 256;

// Lanes per row of the dense kernel for a rows x K matrix.
template <class F>
int dense_lanes(int64_t rows, int64_t K) {
    const int units = (int)(K / 32 / F::SBPU);
    // Q4_K/Q5_K (a unit is a 32-byte pair of sub-blocks): the most lanes per
    // row that leave each lane at least two units, the last chunk ragged if
    // need be -- at K = 2560, 16 lanes and 2.5 units measured 7-15 % faster
    // than 8 lanes and 5 units (twice the waves; 6144 and 12288 rows, N = 1
    // and 4).  Q6_K keeps choose_u (a function of K only, so planar and GGUF
    // outputs are the same bits).
    int u = F::SBPU == 2 ? choose_u_min2(units) : choose_u(units);
    // Q4_K/Q5_K matrices too short to give every CU a wave take more lanes
    // per row while each lane keeps a unit: 512 x 2560 (128 waves at 16
    // lanes) at 32 lanes, N = 1 / 4: Q4_K 2.49 / 3.47 -> 2.39 / 3.30 us, Q5_K
    // 2.84 / 3.90 -> 2.67 / 3.61 us.  At 2560 x 2560 (640 waves) 32 lanes
    // were slower (Q4_K 2.99 -> 3.27 us).  Not a function of the column
    // count, so every column's sum is the same at any N.
    if (F::SBPU == 2)
        while (u < 64 && rows * u / kWave < kDenseFillWaves && units >= 2 * u) u *= 2;
    return u;
}

template <class F, bool DUMP>
hipError_t launch_dense(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                        int ncols, hipStream_t s) {
    switch (dense_lanes<F>(rows, K)) {
    case 8: return launch_dense_u<F, 8, DUMP>(w, xq, out, dump, rows, K, ncols, s);
    case 16: return launch_dense_u<F, 16, DUMP>(w, xq, out, dump, rows, K, ncols, s);
    case 32: return launch_dense_u<F, 32, DUMP>(w, xq, out, dump, rows, K, ncols, s);
    case 64: return launch_dense_u<F, 64, DUMP>(w, xq, out, dump, rows, K, ncols, s);
    default: return hipErrorInvalidValue;
    }
}

// ------------------------------------------------- several products, one launch
// Jobs of one K (at most kMaxDenseJobs), each with its own weights,
// activation columns, outputs and 1-8 columns.  Every job runs with the
// lanes per row and register depth of its single launch, and a row's sum
// depends on nothing else -- not on the waves per workgroup nor on the
// column count -- so every job's outputs are the bits of its own product.
// Within one K the lanes per row take at most two values, the base width and
// twice it for matrices too short to fill the chip (dense_lanes: doubling
// needs at least twice as many units as lanes, which the base width already
// rules out for a second doubling); a launch serves one width (U2 = 0) or
// both (U2 = 2U, the "wide" jobs), so a batch of up to four jobs is one
// launch whatever its matrices' heights.  A second launch for a short matrix
// cost about as much as that matrix alone (12288, 6144 and 512 x 2560 Q4_K at
// one column: 7.4 us for the first two in one launch, 10.3 with the third in
// a launch of its own).  Workgroups of kDenseWaves waves; workgroup b belongs
// to the last job whose first workgroup is at or before b.
constexpr int kMaxDenseJobs = 8;
struct DenseJob {
    const void *w;
    const uint8_t *xq;
    float *out;
    int32_t rows, ncols, wg0, wide;
};
// (MJ entries, the count and K first: the table's size, which every wave
// reads, is kept small, as for the tiled Q6_K batches)
template <int MJ>
struct DenseJobs {
    int64_t K;
    int32_t njobs;
    DenseJob job[MJ];
};

template <class F, int N, int U, int IT>
__device__ __forceinline__ void dense_job_rows(const F &fmt, const MmvqArgs &a, int64_t row0, void *lds,
                                               float *out) {
    float acc[1][N];
    mmvq_rows<F, N, U, 1, kDenseWaves * kWave, false, IT>(fmt, a, row0, lds, acc);
    const int u = (threadIdx.x & (kWave - 1)) % U;
    const int64_t row = lane_row<U, 1>(row0, 0);
    float v = acc[0][0];
#pragma unroll
    for (int n = 1; n < N; n++) v = u == n ? acc[0][n] : v;
    if (row < a.rows && u < N && u < a.nout) out[(int64_t)u * a.rows + row] = v;
}

// Workgroup b's rows of job jb at U lanes per row and depth IT.
template <class F, int U, int IT, int NMAX>
__device__ __forceinline__ void dense_job(const DenseJob &jb, int64_t K, int b, void *lds) {
    F fmt;
    fmt.init(jb.w, jb.rows, K);
    MmvqArgs a;
    a.xq = jb.xq;
    a.dump = nullptr;
    a.rows = jb.rows;
    a.K = K;
    a.colpack = 0;
#pragma unroll
    for (int n = 0; n < 8; n++) a.colpack |= (uint64_t)(n < jb.ncols ? n : jb.ncols - 1) << (8 * n);
    a.nout = jb.ncols;
    a.xstride = K / 32;
    a.its = IT;
    const int64_t row0 = (int64_t)(b - jb.wg0) * kDenseWaves * kRowsPerWave<U, 1>;
    // six and seven columns run as eight (the missing columns read the last
    // real one again and are not stored), as their single launches do
    switch (jb.ncols) {
    case 1: dense_job_rows<F, 1, U, IT>(fmt, a, row0, lds, jb.out); break;
    case 2: if constexpr (NMAX >= 2) dense_job_rows<F, 2, U, IT>(fmt, a, row0, lds, jb.out); break;
    case 3: if constexpr (NMAX >= 4) dense_job_rows<F, 3, U, IT>(fmt, a, row0, lds, jb.out); break;
    case 4: if constexpr (NMAX >= 4) dense_job_rows<F, 4, U, IT>(fmt, a, row0, lds, jb.out); break;
    case 5: if constexpr (NMAX >= 8) dense_job_rows<F, 5, U, IT>(fmt, a, row0, lds, jb.out); break;
    default: if constexpr (NMAX >= 8) dense_job_rows<F, 8, U, IT>(fmt, a, row0, lds, jb.out); break;
    }
}

template <class F, int U, int IT, int U2, int IT2, int NMAX, int MJ>
__global__ __launch_bounds__(kDenseWaves *kWave) void k_mmvq_dense_jobs(const DenseJobs<MJ> js) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int b = blockIdx.x;
    // the job and its fields by selects over the (scalar) kernel arguments
    int j = 0;
#pragma unroll
    for (int i = 1; i < MJ; i++) j = (i < js.njobs && b >= js.job[i].wg0) ? i : j;
    DenseJob jb = js.job[0];
#pragma unroll
    for (int i = 1; i < MJ; i++)
        if (j == i) jb = js.job[i];
    if constexpr (U2 > 0) {
        if (jb.wide) {
            dense_job<F, U2, IT2, NMAX>(jb, js.K, b, lds);
            return;
        }
    }
    dense_job<F, U, IT, NMAX>(jb, js.K, b, lds);
}

template <class F, int U, int IT, int NMAX>
constexpr size_t dense_jobs_lds() {
    size_t m = 0;
    for (int n = 1; n <= NMAX; n++) {
        const size_t b = (size_t)n * its_for(IT, n, U, F::SBPU, kDenseWaves * kWave) * U * F::SBPU *
                         kActBytesPerBlock;
        m = b > m ? b : m;
    }
    return m;
}

template <class F, int U, int IT, int U2, int IT2, int NMAX, int MJ>
hipError_t launch_dense_jobs_mj(const DenseJobs<kMaxDenseJobs> &all, hipStream_t s) {
    DenseJobs<MJ> js;
    js.K = all.K;
    js.njobs = all.njobs;
    int64_t wg = 0;
    for (int j = 0; j < js.njobs; j++) {
        js.job[j] = all.job[j];
        js.job[j].wg0 = (int32_t)wg;
        const int64_t rpw = kDenseWaves * (js.job[j].wide ? kWave / U2 : kWave / U);
        wg += (js.job[j].rows + rpw - 1) / rpw;
    }
    for (int j = js.njobs; j < MJ; j++) js.job[j] = js.job[0];
    if (wg * kDenseWaves * kWave > 0xFFFFFFFFLL) return hipErrorInvalidConfiguration;
    constexpr size_t l1 = dense_jobs_lds<F, U, IT, NMAX>();
    constexpr size_t l2 = U2 > 0 ? dense_jobs_lds<F, (U2 > 0 ? U2 : U), IT2, NMAX>() : 0;
    constexpr size_t lds = l1 > l2 ? l1 : l2;
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_mmvq_dense_jobs<F, U, IT, U2, IT2, NMAX, MJ>), lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_mmvq_dense_jobs<F, U, IT, U2, IT2, NMAX, MJ>), dim3((unsigned)wg),
                       dim3(kDenseWaves * kWave), lds, s, js);
    return hipGetLastError();
}

// Table size: four entries for up to four jobs, else eight (one width only).
template <class F, int U, int IT, int U2, int IT2, int NMAX>
hipError_t launch_dense_jobs_cfg(const DenseJobs<kMaxDenseJobs> &js, hipStream_t s) {
    if (js.njobs <= 4) return launch_dense_jobs_mj<F, U, IT, U2, IT2, NMAX, 4>(js, s);
    if constexpr (U2 == 0) return launch_dense_jobs_mj<F, U, IT, 0, 3, NMAX, kMaxDenseJobs>(js, s);
    return hipErrorInvalidValue;
}

template <class F, int U, int IT, int U2, int IT2>
hipError_t launch_dense_jobs_it(const DenseJobs<kMaxDenseJobs> &js, int maxcols, hipStream_t s) {
    if (maxcols <= 1) return launch_dense_jobs_cfg<F, U, IT, U2, IT2, 1>(js, s);
    if (maxcols <= 2) return launch_dense_jobs_cfg<F, U, IT, U2, IT2, 2>(js, s);
    if (maxcols <= 4) return launch_dense_jobs_cfg<F, U, IT, U2, IT2, 4>(js, s);
    return launch_dense_jobs_cfg<F, U, IT, U2, IT2, 8>(js, s);
}

// One width (wide = false): it = the depth of the U-lane jobs.  Two widths
// (wide = true): the U-lane jobs at depth it and the 2U-lane jobs at depth
// three (they have at most two units per lane).
template <class F, int U>
hipError_t launch_dense_jobs_u(const DenseJobs<kMaxDenseJobs> &js, int it, bool wide, int maxcols, hipStream_t s) {
    if (wide) {
        if constexpr (2 * U <= 64) {
            if constexpr (F::IT > 3) {
                if (it == 3) return launch_dense_jobs_it<F, U, 3, 2 * U, 3>(js, maxcols, s);
            }
            return launch_dense_jobs_it<F, U, F::IT, 2 * U, 3>(js, maxcols, s);
        }
        return hipErrorInvalidValue;
    }
    if constexpr (F::IT > 3) {
        if (it == 3) return launch_dense_jobs_it<F, U, 3, 0, 3>(js, maxcols, s);
    }
    return launch_dense_jobs_it<F, U, F::IT, 0, 3>(js, maxcols, s);
}

// The jobs (the caller has checked each).  Up to four jobs of one or two
// widths: one launch.  Otherwise one launch per width, the jobs of each in
// their given order.
template <class F>
hipError_t launch_dense_jobs(const DenseJob *jobs, int njobs, int64_t K, hipStream_t s) {
    if (njobs < 1 || njobs > kMaxDenseJobs) return hipErrorInvalidValue;
    const int units = (int)(K / 32 / F::SBPU);
    auto depth = [&](int u) { return F::IT > 3 && depth_for(units, u, F::IT) == 3 ? 3 : F::IT; };
    int lanes[kMaxDenseJobs], umin = 64, umax = 0;
    for (int j = 0; j < njobs; j++) {
        lanes[j] = dense_lanes<F>(jobs[j].rows, K);
        umin = lanes[j] < umin ? lanes[j] : umin;
        umax = lanes[j] > umax ? lanes[j] : umax;
    }
    auto launch = [&](const DenseJobs<kMaxDenseJobs> &js, int u, bool wide, int maxcols) {
        switch (u) {
        case 8: return launch_dense_jobs_u<F, 8>(js, depth(u), wide, maxcols, s);
        case 16: return launch_dense_jobs_u<F, 16>(js, depth(u), wide, maxcols, s);
        case 32: return launch_dense_jobs_u<F, 32>(js, depth(u), wide, maxcols, s);
        default: return launch_dense_jobs_u<F, 64>(js, depth(u), wide, maxcols, s);
        }
    };
    if (umax == 2 * umin && njobs <= 4 && depth(umax) == 3) {
        DenseJobs<kMaxDenseJobs> js;
        js.njobs = njobs;
        js.K = K;
        int maxcols = 1;
        for (int j = 0; j < njobs; j++) {
            js.job[j] = jobs[j];
            js.job[j].wide = lanes[j] == umax;
            maxcols = jobs[j].ncols > maxcols ? jobs[j].ncols : maxcols;
        }
        return launch(js, umin, true, maxcols);
    }
    bool done[kMaxDenseJobs] = {};
    for (int j0 = 0; j0 < njobs; j0++) {
        if (done[j0]) continue;
        DenseJobs<kMaxDenseJobs> js;
        js.njobs = 0;
        js.K = K;
        int maxcols = 1;
        for (int j = j0; j < njobs; j++) {
            if (done[j] || lanes[j] != lanes[j0]) continue;
            done[j] = true;
            js.job[js.njobs] = jobs[j];
            js.job[js.njobs++].wide = 0;
            maxcols = jobs[j].ncols > maxcols ? jobs[j].ncols : maxcols;
        }
        const hipError_t e = launch(js, lanes[j0], false, maxcols);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class F>
hipError_t launch_dense_any(const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                            int ncols, hipStream_t s) {
    return dump ? launch_dense<F, true>(w, xq, out, dump, rows, K, ncols, s)
                : launch_dense<F, false>(w, xq, out, dump, rows, K, ncols, s);
}

}  // namespace qmv

// launch.hpp -- internal host-side launchers of libqmv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace qmv {

enum Fmt { FMT_Q6_PLANAR = 0, FMT_Q6_GGUF = 1, FMT_Q4 = 2, FMT_Q5 = 3 };

// Lets a kernel use more than 64 KB of dynamic LDS (gfx950 allows 160 KB per
// workgroup); a no-op below that.
inline hipError_t allow_lds(const void *kernel, size_t bytes) {
    if (bytes <= 65536) return hipSuccess;
    return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_quantize(const float *x, uint8_t *xq, int64_t K, int ncols, bool planar, hipStream_t s);
hipError_t launch_rmsnorm_quantize(const float *x, const float *gamma, float eps, uint8_t *xq, int64_t K, int ncols,
                                   bool planar, hipStream_t s);
// Q6_K GGUF <-> planar (tiled = false: row-major planes; true: 16-row tiles)
hipError_t launch_repack(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K, bool tiled, hipStream_t s);
hipError_t launch_stream_read(const void *src, int64_t bytes, uint32_t *sink, int blocks, hipStream_t s);
hipError_t launch_unpack(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t K, bool tiled, hipStream_t s);
// Q6_K row gather within one layout (0 GGUF, 1 planar, 2 tiled)
hipError_t launch_gather(const uint8_t *src, uint8_t *dst, const int32_t *ids, int64_t rows, int64_t nout,
                         int64_t K, int layout, hipStream_t s);

hipError_t launch_mmvq_q6_planar(const void *w, const void *xq, float *out, int32_t *dump,
                                 int64_t rows, int64_t K, int ncols, hipStream_t s);
// xp: activations in the column-planar Q8_1 layout
hipError_t launch_mmvq_q6_tiled(const void *w, const void *xq, float *out, int32_t *dump,
                                int64_t rows, int64_t K, int ncols, bool xp, hipStream_t s);
// independent products of the same K in one launch (checked by the caller);
// also the Q4_K/Q5_K batches (GGUF weights, at most kMaxDenseJobs jobs)
struct TiledJobDesc {
    const void *w;
    const void *xq;
    float *out;
    int64_t rows;
    int ncols;
};
hipError_t launch_mmvq_q6_tiled_jobs(const TiledJobDesc *jobs, int njobs, int64_t K, bool xp, hipStream_t s);
// any number of columns (batches of twelve or sixteen, then at most eight)
hipError_t launch_mmq_q6_tiled(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int ncols,
                               bool xp, hipStream_t s);
// The argmax workspace: the keys, keys[n * ntiles + tile], then (256-byte
// aligned) per column the running maximum key (8 bytes, at most 8 columns)
// and, 64 bytes further, the count of reduction workgroups done (4 bytes).
// Both are cleared by the product launch, which runs first.
__host__ __device__ inline int64_t argmax_tail(int64_t ntiles, int ncols) {
    return (ntiles * ncols * 8 + 255) & ~(int64_t)255;
}
hipError_t launch_mmvq_q6_tiled_argmax(const void *w, const void *xq, uint64_t *keys, int64_t rows, int64_t K,
                                       int ncols, int32_t *idx, float *val, bool xp, hipStream_t s);
// Top-k rows per column of fp32 outputs [ncols][rows] (k <= kTopkMax,
// ceil(rows / kTopkChunk) * k <= kTopkChunk); cand: ncols * ceil(rows /
// kTopkChunk) * k keys of scratch; idx/val [ncols][k], descending.
constexpr int kTopkChunk = 4096, kTopkMax = 64;
hipError_t launch_topk(const float *out, int64_t rows, int ncols, int k, uint64_t *cand, int32_t *idx, float *val,
                       hipStream_t s);
hipError_t launch_mmvq_q6_gguf(const void *w, const void *xq, float *out, int32_t *dump,
                               int64_t rows, int64_t K, int ncols, hipStream_t s);
hipError_t launch_mmvq_q4(const void *w, const void *xq, float *out, int32_t *dump,
                          int64_t rows, int64_t K, int ncols, hipStream_t s);
hipError_t launch_mmvq_q5(const void *w, const void *xq, float *out, int32_t *dump,
                          int64_t rows, int64_t K, int ncols, hipStream_t s);
hipError_t launch_mmvq_q4_jobs(const TiledJobDesc *jobs, int njobs, int64_t K, hipStream_t s);
hipError_t launch_mmvq_q5_jobs(const TiledJobDesc *jobs, int njobs, int64_t K, hipStream_t s);

struct MoeArgs {
    const uint8_t *w_gate, *w_up, *w_down;
    const uint8_t *xq;
    const int32_t *ids;
    const float *route_w;
    float *out;
    uint8_t *ws;
    int E, T, topk, S;
    int64_t d_model, d_ff;
    int64_t off_h, off_hq, off_y;   // byte offsets of h, hq, y in ws
};

// Byte offsets of the workspace regions (see qmv.h) and its total size.
struct MoeLayout {
    int64_t off_h, off_hq, off_y, total;
};
MoeLayout moe_layout(int T, int topk, int64_t d_model, int64_t d_ff);

hipError_t launch_moe(const MoeArgs &m, int down_layout, hipStream_t s);

// Bytes of the per-device scratch array of grouped_expert_mmvq_noalloc, and
// its device address on `device` (the calling thread's current device),
// looked up on the first call for that device.
constexpr int64_t kMoeScratchBytes = 4LL << 20;
hipError_t moe_scratch(int device, void **ptr);
// Whether every launch of launch_moe for S slots stays within max_grid_y
// workgroups along y (host arithmetic only).
bool moe_grid_fits(int S, int64_t d_model, int64_t d_ff, int64_t max_grid_y);

}  // namespace qmv

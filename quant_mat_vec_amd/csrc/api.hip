// api.hip -- the C ABI of libqmv (declared in include/qmv.h): argument
// checks on the host, then the launches.  No entry point allocates, frees or
// synchronizes; every check runs before the first HIP call.
#include <stdint.h>

#include "../../include/qmv.h"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxRows = 2147483647LL;
constexpr int64_t kMaxK = 1LL << 20;
constexpr int64_t kMaxBytes = 1LL << 40;
// Launch limits: work-items along x of one launch below 2^32, workgroups
// along y at most 65535.  The products launch at most 64 work-items per row
// (sixteen waves per 16-row tile, or one wave per row) plus one workgroup,
// so rows up to kMaxProductRows always fit.
constexpr int64_t kMaxItems = 0xFFFFFFFFLL;
constexpr int64_t kMaxGridY = 65535;
constexpr int64_t kMaxProductRows = (1LL << 26) - 1024;

// work-items of a launch of ceil(items / 256) workgroups of 256
bool items_fit(int64_t items) { return items <= kMaxItems - 255; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int from_hip(hipError_t e) {
    if (e == hipSuccess) return QMV_OK;
    g_last_hip_error = (int)e;
    return QMV_ERR_HIP;
}

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Checks shared by the MMVQ entry points.
int check_mmvq(const void *w, const void *xq, const void *out, int64_t rows, int64_t K, int ncols,
               int64_t block_bytes, uintptr_t w_align, int max_cols = 8) {
    if (!w || !xq || !out) return QMV_ERR_INVALID_ARG;
    if (rows <= 0 || K <= 0) return QMV_ERR_INVALID_ARG;
    if (K % 256 != 0 || K > kMaxK || rows > kMaxProductRows) return QMV_ERR_UNSUPPORTED;
    if (ncols < 1 || ncols > max_cols) return QMV_ERR_UNSUPPORTED;
    if (rows * (K / 256) * block_bytes >= kMaxBytes || rows * ncols * 4 >= kMaxBytes) return QMV_ERR_UNSUPPORTED;
    if (!aligned(w, w_align) || !aligned(xq, 4) || !aligned(out, 4)) return QMV_ERR_ALIGNMENT;
    return QMV_OK;
}

// The checks of a Q6_K product's weights, activations and shape (layout
// with the activation flag), outputs aside.
int q6_check(const void *w, int layout_arg, const void *xq, int64_t rows, int64_t K, int ncols) {
    const bool xp = (layout_arg & QMV_ACT_PLANAR) != 0;
    const int layout = layout_arg & ~QMV_ACT_PLANAR;
    if ((layout != QMV_LAYOUT_GGUF && layout != QMV_LAYOUT_PLANAR && layout != QMV_LAYOUT_TILED) ||
        (xp && layout != QMV_LAYOUT_TILED)) {
        if (!w || !xq) return QMV_ERR_INVALID_ARG;
        return QMV_ERR_UNSUPPORTED;
    }
    // (a 4-byte aligned stand-in for the output: only its alignment is checked)
    int rc = check_mmvq(w, xq, xq, rows, K, ncols, 210, layout == QMV_LAYOUT_GGUF ? 4 : 16);
    if (rc) return rc;
    if (xp && !aligned(xq, 16)) return QMV_ERR_ALIGNMENT;
    return QMV_OK;
}

int q6_dispatch(const void *w, int layout_arg, const void *xq, float *out, int32_t *dump, int64_t rows,
                int64_t K, int ncols, void *stream) {
    const bool xp = (layout_arg & QMV_ACT_PLANAR) != 0;
    const int layout = layout_arg & ~QMV_ACT_PLANAR;
    if ((layout != QMV_LAYOUT_GGUF && layout != QMV_LAYOUT_PLANAR && layout != QMV_LAYOUT_TILED) ||
        (xp && layout != QMV_LAYOUT_TILED)) {
        if (!w || !xq || !(out || dump)) return QMV_ERR_INVALID_ARG;
        return QMV_ERR_UNSUPPORTED;
    }
    const void *o = out ? static_cast<const void *>(out) : static_cast<const void *>(dump);
    int rc = check_mmvq(w, xq, o, rows, K, ncols, 210, layout == QMV_LAYOUT_GGUF ? 4 : 16);
    if (rc) return rc;
    if (xp && !aligned(xq, 16)) return QMV_ERR_ALIGNMENT;
    hipError_t e;
    if (layout == QMV_LAYOUT_TILED)
        e = qmv::launch_mmvq_q6_tiled(w, xq, out, dump, rows, K, ncols, xp, as_stream(stream));
    else if (layout == QMV_LAYOUT_PLANAR)
        e = qmv::launch_mmvq_q6_planar(w, xq, out, dump, rows, K, ncols, as_stream(stream));
    else
        e = qmv::launch_mmvq_q6_gguf(w, xq, out, dump, rows, K, ncols, as_stream(stream));
    return from_hip(e);
}

int q45_dispatch(bool five, const void *w, const void *xq, float *out, int32_t *dump, int64_t rows, int64_t K,
                 int ncols, void *stream) {
    const void *o = out ? static_cast<const void *>(out) : static_cast<const void *>(dump);
    int rc = check_mmvq(w, xq, o, rows, K, ncols, five ? 176 : 144, 16);
    if (rc) return rc;
    hipError_t e = five ? qmv::launch_mmvq_q5(w, xq, out, dump, rows, K, ncols, as_stream(stream))
                        : qmv::launch_mmvq_q4(w, xq, out, dump, rows, K, ncols, as_stream(stream));
    return from_hip(e);
}

int check_repack(const void *src, const void *dst, int64_t rows, int64_t K, uintptr_t src_align,
                 uintptr_t dst_align) {
    if (!src || !dst) return QMV_ERR_INVALID_ARG;
    if (rows <= 0 || K <= 0) return QMV_ERR_INVALID_ARG;
    if (K % 256 != 0 || K > kMaxK || rows > kMaxRows) return QMV_ERR_UNSUPPORTED;
    const int64_t bytes = rows * (K / 256) * 210;
    if (bytes >= kMaxBytes || !items_fit(rows * (K / 256) * 8)) return QMV_ERR_UNSUPPORTED;   // 8 per block
    if (!aligned(src, src_align) || !aligned(dst, dst_align)) return QMV_ERR_ALIGNMENT;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + (uintptr_t)bytes && d < s + (uintptr_t)bytes) return QMV_ERR_INVALID_ARG;   // overlap
    return QMV_OK;
}

// Checks shared by the grouped MoE entry points (all but the workspace).
int check_moe(const void *w_gate, const void *w_up, const void *w_down, int down_layout, const void *xq,
              const int32_t *ids, const float *route_w, const float *out, int E, int T, int topk, int64_t d_model,
              int64_t d_ff) {
    if (!w_gate || !w_up || !w_down || !xq || !ids || !route_w || !out) return QMV_ERR_INVALID_ARG;
    if (E < 1 || T < 1 || topk < 1 || d_model <= 0 || d_ff <= 0) return QMV_ERR_INVALID_ARG;
    if (T > 8 || topk > 8 || d_model % 256 || d_ff % 256 || d_model > kMaxK || d_ff > kMaxK)
        return QMV_ERR_UNSUPPORTED;
    if (down_layout != QMV_LAYOUT_GGUF && down_layout != QMV_LAYOUT_PLANAR) return QMV_ERR_UNSUPPORTED;
    const int64_t gu_bytes = (int64_t)E * d_ff * (d_model / 256) * 144;
    const int64_t dn_bytes = (int64_t)E * d_model * (d_ff / 256) * 210;
    if (gu_bytes >= kMaxBytes || dn_bytes >= kMaxBytes || (int64_t)E * d_model > kMaxRows)
        return QMV_ERR_UNSUPPORTED;
    if (!qmv::moe_grid_fits(T * topk, d_model, d_ff, kMaxGridY)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, down_layout == QMV_LAYOUT_PLANAR ? 16 : 4) ||
        !aligned(xq, 4) || !aligned(ids, 4) || !aligned(route_w, 4) || !aligned(out, 4))
        return QMV_ERR_ALIGNMENT;
    return QMV_OK;
}

int run_moe(const void *w_gate, const void *w_up, const void *w_down, int down_layout, const void *xq,
            const int32_t *ids, const float *route_w, float *out, int E, int T, int topk, int64_t d_model,
            int64_t d_ff, void *ws, const qmv::MoeLayout &L, void *stream) {
    qmv::MoeArgs m;
    m.w_gate = reinterpret_cast<const uint8_t *>(w_gate);
    m.w_up = reinterpret_cast<const uint8_t *>(w_up);
    m.w_down = reinterpret_cast<const uint8_t *>(w_down);
    m.xq = reinterpret_cast<const uint8_t *>(xq);
    m.ids = ids;
    m.route_w = route_w;
    m.out = out;
    m.ws = reinterpret_cast<uint8_t *>(ws);
    m.E = E;
    m.T = T;
    m.topk = topk;
    m.S = T * topk;
    m.d_model = d_model;
    m.d_ff = d_ff;
    m.off_h = L.off_h;
    m.off_hq = L.off_hq;
    m.off_y = L.off_y;
    return from_hip(qmv::launch_moe(m, down_layout, as_stream(stream)));
}

int q45_batch(bool five, const qmv_q6k_job *jobs, int njobs, int64_t K, void *stream) {
    if (!jobs || njobs < 1) return QMV_ERR_INVALID_ARG;
    if (njobs > 8) return QMV_ERR_UNSUPPORTED;
    qmv::TiledJobDesc d[8];
    int64_t total_rows = 0;
    for (int j = 0; j < njobs; j++) {
        const qmv_q6k_job &jb = jobs[j];
        const int rc = check_mmvq(jb.w, jb.xq, jb.out, jb.rows, K, jb.ncols, five ? 176 : 144, 16);
        if (rc) return rc;
        total_rows += jb.rows;
        d[j] = {jb.w, jb.xq, jb.out, jb.rows, jb.ncols};
    }
    if (total_rows > kMaxProductRows) return QMV_ERR_UNSUPPORTED;
    hipError_t e = five ? qmv::launch_mmvq_q5_jobs(d, njobs, K, as_stream(stream))
                        : qmv::launch_mmvq_q4_jobs(d, njobs, K, as_stream(stream));
    return from_hip(e);
}
}  // namespace

extern "C" {

int quantize_q8_1(const float *x, void *xq, int64_t K, int ncols, void *stream) {
    if (!x || !xq) return QMV_ERR_INVALID_ARG;
    if (K <= 0 || ncols <= 0) return QMV_ERR_INVALID_ARG;
    if (K % 32 != 0 || K > kMaxK || ncols > 65535) return QMV_ERR_UNSUPPORTED;
    if (!items_fit((int64_t)ncols * (K / 32) * 8)) return QMV_ERR_UNSUPPORTED;    // eight per block
    if (!aligned(x, 4) || !aligned(xq, 4)) return QMV_ERR_ALIGNMENT;
    return from_hip(qmv::launch_quantize(x, reinterpret_cast<uint8_t *>(xq), K, ncols, false, as_stream(stream)));
}

int quantize_q8_1_planar(const float *x, void *xq, int64_t K, int ncols, void *stream) {
    if (!x || !xq) return QMV_ERR_INVALID_ARG;
    if (K <= 0 || ncols <= 0) return QMV_ERR_INVALID_ARG;
    if (K % 32 != 0 || K > kMaxK || ncols > 65535) return QMV_ERR_UNSUPPORTED;
    if (!items_fit((int64_t)ncols * (K / 32) * 8)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(x, 4) || !aligned(xq, 4)) return QMV_ERR_ALIGNMENT;
    return from_hip(qmv::launch_quantize(x, reinterpret_cast<uint8_t *>(xq), K, ncols, true, as_stream(stream)));
}

int rmsnorm_quantize_q8_1(const float *x, const float *gamma, float eps, void *xq, int64_t K, int ncols,
                          int act_layout, void *stream) {
    if (!x || !gamma || !xq) return QMV_ERR_INVALID_ARG;
    if (K <= 0 || ncols <= 0) return QMV_ERR_INVALID_ARG;
    if (K % 32 != 0 || K > kMaxK || ncols > 65535 || (act_layout != 0 && act_layout != QMV_ACT_PLANAR))
        return QMV_ERR_UNSUPPORTED;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return QMV_ERR_INVALID_ARG;   // also rejects NaN
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(xq, 4)) return QMV_ERR_ALIGNMENT;
    return from_hip(qmv::launch_rmsnorm_quantize(x, gamma, eps, reinterpret_cast<uint8_t *>(xq), K, ncols,
                                                 act_layout == QMV_ACT_PLANAR, as_stream(stream)));
}

int mmvq_q6k(const void *w, int layout, const void *xq, float *out, int64_t rows, int64_t K, int ncols,
             void *stream) {
    if (!out) return QMV_ERR_INVALID_ARG;
    return q6_dispatch(w, layout, xq, out, nullptr, rows, K, ncols, stream);
}

int mmq_q6k(const void *w, int layout, const void *xq, float *out, int64_t rows, int64_t K, int ncols,
            void *stream) {
    if (!out) return QMV_ERR_INVALID_ARG;
    const bool xp = (layout & QMV_ACT_PLANAR) != 0;
    if ((layout & ~QMV_ACT_PLANAR) != QMV_LAYOUT_TILED) {
        if (!w || !xq) return QMV_ERR_INVALID_ARG;
        return QMV_ERR_UNSUPPORTED;
    }
    int rc = check_mmvq(w, xq, out, rows, K, ncols, 210, 16, 65535);
    if (rc) return rc;
    // the batched launch's grid stays under 2^32 threads
    if (((rows + 15) / 16 + 32) * ((ncols + 11) / 12) >= (1LL << 22)) return QMV_ERR_UNSUPPORTED;
    if (xp && !aligned(xq, 16)) return QMV_ERR_ALIGNMENT;
    return from_hip(qmv::launch_mmq_q6_tiled(w, xq, out, rows, K, ncols, xp, as_stream(stream)));
}

int mmvq_q6k_batch(const qmv_q6k_job *jobs, int njobs, int layout, int64_t K, void *stream) {
    if (!jobs || njobs < 1) return QMV_ERR_INVALID_ARG;
    if (njobs > 8) return QMV_ERR_UNSUPPORTED;
    const bool xp = (layout & QMV_ACT_PLANAR) != 0;
    if ((layout & ~QMV_ACT_PLANAR) != QMV_LAYOUT_TILED) return QMV_ERR_UNSUPPORTED;
    qmv::TiledJobDesc d[8];
    int64_t total_rows = 0;
    for (int j = 0; j < njobs; j++) {
        const qmv_q6k_job &jb = jobs[j];
        const int rc = check_mmvq(jb.w, jb.xq, jb.out, jb.rows, K, jb.ncols, 210, 16);
        if (rc) return rc;
        if (xp && !aligned(jb.xq, 16)) return QMV_ERR_ALIGNMENT;
        total_rows += jb.rows;
        d[j] = {jb.w, jb.xq, jb.out, jb.rows, jb.ncols};
    }
    if (total_rows > kMaxProductRows) return QMV_ERR_UNSUPPORTED;
    return from_hip(qmv::launch_mmvq_q6_tiled_jobs(d, njobs, K, xp, as_stream(stream)));
}

int mmvq_q4k(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int ncols, void *stream) {
    if (!out) return QMV_ERR_INVALID_ARG;
    return q45_dispatch(false, w, xq, out, nullptr, rows, K, ncols, stream);
}

int mmvq_q5k(const void *w, const void *xq, float *out, int64_t rows, int64_t K, int ncols, void *stream) {
    if (!out) return QMV_ERR_INVALID_ARG;
    return q45_dispatch(true, w, xq, out, nullptr, rows, K, ncols, stream);
}

int mmvq_q4k_batch(const qmv_q6k_job *jobs, int njobs, int64_t K, void *stream) {
    return q45_batch(false, jobs, njobs, K, stream);
}

int mmvq_q5k_batch(const qmv_q6k_job *jobs, int njobs, int64_t K, void *stream) {
    return q45_batch(true, jobs, njobs, K, stream);
}

int mmvq_q6k_isums(const void *w, int layout, const void *xq, int32_t *isums, int64_t rows, int64_t K,
                   int ncols, void *stream) {
    if (!isums) return QMV_ERR_INVALID_ARG;
    return q6_dispatch(w, layout, xq, nullptr, isums, rows, K, ncols, stream);
}

int mmvq_q4k_isums(const void *w, const void *xq, int32_t *isums, int64_t rows, int64_t K, int ncols,
                   void *stream) {
    if (!isums) return QMV_ERR_INVALID_ARG;
    return q45_dispatch(false, w, xq, nullptr, isums, rows, K, ncols, stream);
}

int mmvq_q5k_isums(const void *w, const void *xq, int32_t *isums, int64_t rows, int64_t K, int ncols,
                   void *stream) {
    if (!isums) return QMV_ERR_INVALID_ARG;
    return q45_dispatch(true, w, xq, nullptr, isums, rows, K, ncols, stream);
}

int repack_q6k_planar(const void *src, void *dst, int64_t rows, int64_t K, void *stream) {
    int rc = check_repack(src, dst, rows, K, 2, 16);
    if (rc) return rc;
    return from_hip(qmv::launch_repack(reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst),
                                       rows, K, false, as_stream(stream)));
}

int unpack_q6k_planar(const void *src, void *dst, int64_t rows, int64_t K, void *stream) {
    int rc = check_repack(src, dst, rows, K, 16, 2);
    if (rc) return rc;
    return from_hip(qmv::launch_unpack(reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst),
                                       rows, K, false, as_stream(stream)));
}

int repack_q6k_tiled(const void *src, void *dst, int64_t rows, int64_t K, void *stream) {
    int rc = check_repack(src, dst, rows, K, 2, 16);
    if (rc) return rc;
    return from_hip(qmv::launch_repack(reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst),
                                       rows, K, true, as_stream(stream)));
}

int unpack_q6k_tiled(const void *src, void *dst, int64_t rows, int64_t K, void *stream) {
    int rc = check_repack(src, dst, rows, K, 16, 2);
    if (rc) return rc;
    return from_hip(qmv::launch_unpack(reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst),
                                       rows, K, true, as_stream(stream)));
}

int gather_q6k_rows(const void *src, int layout, int64_t rows, int64_t K, const int32_t *ids, int64_t nout,
                    void *dst, void *stream) {
    if (!src || !dst || !ids) return QMV_ERR_INVALID_ARG;
    if (rows <= 0 || K <= 0 || nout <= 0) return QMV_ERR_INVALID_ARG;
    if (layout != QMV_LAYOUT_GGUF && layout != QMV_LAYOUT_PLANAR && layout != QMV_LAYOUT_TILED)
        return QMV_ERR_UNSUPPORTED;
    if (K % 256 != 0 || K > kMaxK || rows > kMaxRows || nout > kMaxRows) return QMV_ERR_UNSUPPORTED;
    const int64_t sb = rows * (K / 256) * 210, db = nout * (K / 256) * 210;
    if (sb >= kMaxBytes || db >= kMaxBytes || !items_fit(nout * (K / 256))) return QMV_ERR_UNSUPPORTED;
    const uintptr_t al = layout == QMV_LAYOUT_GGUF ? 1 : 16;
    if (!aligned(src, al) || !aligned(dst, al) || !aligned(ids, 4)) return QMV_ERR_ALIGNMENT;
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + (uintptr_t)db && d < s + (uintptr_t)sb) return QMV_ERR_INVALID_ARG;   // overlap
    return from_hip(qmv::launch_gather(reinterpret_cast<const uint8_t *>(src), reinterpret_cast<uint8_t *>(dst), ids,
                                       rows, nout, K, layout, as_stream(stream)));
}

size_t mmvq_q6k_argmax_workspace(int64_t rows, int ncols) {
    if (rows <= 0 || rows > kMaxProductRows || ncols < 1 || ncols > 8) return 0;
    return (size_t)(qmv::argmax_tail((rows + 15) / 16, ncols) + 256);
}

int mmvq_q6k_argmax(const void *w, int layout, const void *xq, int64_t rows, int64_t K, int ncols, int32_t *idx,
                    float *val, void *ws, size_t ws_bytes, void *stream) {
    if (!idx || !val || !ws) return QMV_ERR_INVALID_ARG;
    const bool xp = (layout & QMV_ACT_PLANAR) != 0;
    if ((layout & ~QMV_ACT_PLANAR) != QMV_LAYOUT_TILED) {
        if (!w || !xq) return QMV_ERR_INVALID_ARG;
        return QMV_ERR_UNSUPPORTED;
    }
    int rc = check_mmvq(w, xq, idx, rows, K, ncols, 210, 16);
    if (rc) return rc;
    if (!aligned(val, 4) || !aligned(ws, 8) || (xp && !aligned(xq, 16))) return QMV_ERR_ALIGNMENT;
    if (ws_bytes < mmvq_q6k_argmax_workspace(rows, ncols)) return QMV_ERR_WORKSPACE;
    return from_hip(qmv::launch_mmvq_q6_tiled_argmax(w, xq, reinterpret_cast<uint64_t *>(ws), rows, K, ncols, idx,
                                                     val, xp, as_stream(stream)));
}

size_t mmvq_q6k_topk_workspace(int64_t rows, int ncols, int k) {
    if (rows <= 0 || rows > kMaxProductRows || ncols < 1 || ncols > 8 || k < 1 || k > qmv::kTopkMax || k > rows)
        return 0;
    const int64_t nchunks = (rows + qmv::kTopkChunk - 1) / qmv::kTopkChunk;
    if (nchunks * k > qmv::kTopkChunk) return 0;
    const int64_t outs = (4 * rows * ncols + 255) & ~(int64_t)255;
    return (size_t)(outs + 8 * nchunks * k * ncols);
}

int mmvq_q6k_topk(const void *w, int layout, const void *xq, int64_t rows, int64_t K, int ncols, int k,
                  int32_t *idx, float *val, void *ws, size_t ws_bytes, void *stream) {
    if (!idx || !val || !ws || !w || !xq || k < 1) return QMV_ERR_INVALID_ARG;
    const int rc = q6_check(w, layout, xq, rows, K, ncols);
    if (rc) return rc;
    if (k > qmv::kTopkMax || k > rows || ((rows + qmv::kTopkChunk - 1) / qmv::kTopkChunk) * k > qmv::kTopkChunk)
        return QMV_ERR_UNSUPPORTED;
    if (!aligned(idx, 4) || !aligned(val, 4) || !aligned(ws, 256)) return QMV_ERR_ALIGNMENT;
    if (ws_bytes < mmvq_q6k_topk_workspace(rows, ncols, k)) return QMV_ERR_WORKSPACE;
    float *out = reinterpret_cast<float *>(ws);
    const int64_t outs = (4 * rows * ncols + 255) & ~(int64_t)255;
    uint64_t *cand = reinterpret_cast<uint64_t *>(static_cast<uint8_t *>(ws) + outs);
    const int e = q6_dispatch(w, layout, xq, out, nullptr, rows, K, ncols, stream);
    if (e) return e;
    return from_hip(qmv::launch_topk(out, rows, ncols, k, cand, idx, val, as_stream(stream)));
}

size_t grouped_expert_mmvq_workspace(int E, int T, int topk, int64_t d_model, int64_t d_ff) {
    if (E < 1 || T < 1 || T > 8 || topk < 1 || topk > 8 || d_model < 256 || d_ff < 256 || d_model % 256 ||
        d_ff % 256 || d_model > kMaxK || d_ff > kMaxK)
        return 0;
    return (size_t)qmv::moe_layout(T, topk, d_model, d_ff).total;
}

int grouped_expert_mmvq(const void *w_gate, const void *w_up, const void *w_down, int down_layout,
                        const void *xq, const int32_t *ids, const float *route_w, float *out, int E, int T,
                        int topk, int64_t d_model, int64_t d_ff, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_moe(w_gate, w_up, w_down, down_layout, xq, ids, route_w, out, E, T, topk, d_model, d_ff);
    if (rc) return rc;
    const qmv::MoeLayout L = qmv::moe_layout(T, topk, d_model, d_ff);
    if (!ws || ws_bytes < (size_t)L.total) return QMV_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return QMV_ERR_ALIGNMENT;
    return run_moe(w_gate, w_up, w_down, down_layout, xq, ids, route_w, out, E, T, topk, d_model, d_ff, ws, L,
                   stream);
}

int grouped_expert_mmvq_noalloc(const void *w_gate, const void *w_up, const void *w_down, int down_layout,
                                const void *xq, const int32_t *ids, const float *route_w, float *out, int E,
                                int T, int topk, int64_t d_model, int64_t d_ff, void *stream) {
    int rc = check_moe(w_gate, w_up, w_down, down_layout, xq, ids, route_w, out, E, T, topk, d_model, d_ff);
    if (rc) return rc;
    const qmv::MoeLayout L = qmv::moe_layout(T, topk, d_model, d_ff);
    if (L.total > qmv::kMoeScratchBytes) return QMV_ERR_UNSUPPORTED;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return from_hip(e);
    void *ws = nullptr;
    e = qmv::moe_scratch(device, &ws);
    if (e != hipSuccess) return from_hip(e);
    return run_moe(w_gate, w_up, w_down, down_layout, xq, ids, route_w, out, E, T, topk, d_model, d_ff, ws, L,
                   stream);
}

int qmv_stream_read(const void *src, int64_t bytes, uint32_t *sink, int blocks, void *stream) {
    if (!src || !sink || bytes <= 0 || blocks < 0) return QMV_ERR_INVALID_ARG;
    if (bytes % 16 != 0 || bytes >= kMaxBytes || blocks > 65535) return QMV_ERR_UNSUPPORTED;
    if (blocks == 0 && !items_fit((bytes / 16 + 1023) / 1024 * 256)) return QMV_ERR_UNSUPPORTED;
    if (!aligned(src, 16) || !aligned(sink, 4)) return QMV_ERR_ALIGNMENT;
    return from_hip(qmv::launch_stream_read(src, bytes, sink, blocks, as_stream(stream)));
}

const char *qmv_strerror(int code) {
    switch (code) {
    case QMV_OK: return "ok";
    case QMV_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size or overlapping buffers)";
    case QMV_ERR_UNSUPPORTED: return "unsupported shape or option (K % 256, ncols 1..8, T/topk 1..8, layout, size)";
    case QMV_ERR_ALIGNMENT: return "pointer below its required alignment";
    case QMV_ERR_WORKSPACE: return "workspace missing or too small";
    case QMV_ERR_HIP: return "HIP launch failed (see qmv_last_hip_error)";
    default: return "unknown error code";
    }
}

int qmv_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"

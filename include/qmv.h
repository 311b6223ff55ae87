/*
 * qmv.h -- C ABI of libqmv: quantized matrix-vector products (MMVQ) for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Weights are K-quant blocks (Q6_K, Q4_K, Q5_K), the
 * activations are Q8_1 blocks, and for every activation column n and weight
 * row r
 *     out[n][r] = sum over 32-weight sub-blocks b of
 *                 d_w * scale * d_a(n, b) * (integer dot of the unpacked
 *                 weight quants of sub-block b with the Q8_1 quants)
 * (minus the Q4_K/Q5_K min term), the per-sub-block value of PR #1774
 * ("sycl opt-in: STRATA_IQ3S_WIDE=1, a wide mmvq kernel for the dense IQ3_S
 * matrices", section "What changed"), for 1 to 8 activation columns with the
 * weights read once for all columns (PR #2207, "Issue: #1545, #1606 (Arc
 * A-series decode)", section "Summary").  Integer dots are exact int32; the
 * scaling and accumulation are fp32, so results agree with the exact value to
 * within fp32 rounding of a sum whose order differs from any other
 * implementation's (PR #1774, "What changed", notes the same for its kernel).
 *
 * Block formats (little-endian; the pages name the GGUF-layout blocks, PR
 * #2340 "sycl mmvq: Q6_K decode kernels no longer ALU-bound; Q6_K output
 * heads as aligned planes; int4 activation loads", section "What it
 * changes"; the bit layout is the GGUF K-quant convention):
 *   Q6_K, 210 B per 256 weights: ql[128] @0, qh[64] @128, int8 scales[16]
 *     @192, fp16 d @208.  Weight i: h = i/128, c = (i%128)/32, l = i%32,
 *     q6 = ((ql[64h+32(c%2)+l] >> 4(c/2)) & 15) | ((qh[32h+l] >> 2c) & 3) << 4,
 *     w = d * scales[i/16] * (q6 - 32).
 *   Q4_K, 144 B: fp16 d @0, fp16 dmin @2, scales[12] @4, qs[128] @16.
 *     Sub-block j = i/32: q4 = (qs[32(j/2)+i%32] >> 4(j%2)) & 15,
 *     w = d*sc_j*q4 - dmin*m_j with 6-bit sc_j, m_j packed in scales[12]
 *     (j<4: low six bits of bytes j and j+4; j>=4: the nibbles of byte j+4
 *     joined with the top two bits of bytes j-4 and j).
 *   Q5_K, 176 B: as Q4_K with qh[32] @16 and qs[128] @48;
 *     q5 = q4 | ((qh[i%32] >> j) & 1) << 4.
 *   Q8_1, 36 B per 32 values: fp16 d @0, fp16 s @2, int8 q[32] @4.
 *   A matrix of R rows and K columns is R*K/256 blocks, row-major (row r
 *   holds blocks r*K/256 .. (r+1)*K/256-1).  A Q8_1 activation of ncols
 *   columns is [ncols][K/32] blocks.  Outputs are fp32 [ncols][R].
 *
 * Planar Q6_K layout (QMV_LAYOUT_PLANAR), produced by repack_q6k_planar: the
 * same number of bytes as the GGUF matrix, split into planes whose every
 * lane-load is an aligned 16-byte load (the load-time conversion of PR #2340,
 * "What it changes").  With NB = R*K/256 blocks, block t = r*(K/256) + s,
 * v_i = (q6_i - 32) mod 64 for weight i of the block:
 *   plane A at byte 0, 128 B per block, 16 B per sub-block j (0..7):
 *     byte k (0..15) = v[32j+k] << 2 | spare_A(k);
 *   plane B at byte 128*NB, 64 B per block, 8 B per sub-block:
 *     byte k (0..7) = v[32j+16+k] << 2 | spare_B(k);
 *   the two spare bits of every byte hold weights 32j+24 .. 32j+31: for
 *     k = 0..3, weight 32j+24+k keeps bits 0-1 of v in spare_A(k), bits 2-3
 *     in spare_A(4+k), bits 4-5 in spare_A(8+k); weight 32j+28+k keeps bits
 *     0-1 in spare_A(12+k), bits 2-3 in spare_B(k), bits 4-5 in spare_B(4+k);
 *   plane SC at byte 192*NB, 16 B per block: the int8 scales, unchanged;
 *   plane D at byte 208*NB, 2 B per block: fp16 d, unchanged.
 * Read as int8, a plane byte with its spare bits cleared is 4*(q6-32), so the
 * six-bit offset costs no instruction.  Planar and GGUF inputs give
 * bit-identical outputs.
 *
 * Tiled Q6_K layout (QMV_LAYOUT_TILED), produced by repack_q6k_tiled: the
 * planes of the planar layout (same sizes and offsets, same 16-byte A and
 * 8-byte B pieces, same scale and d bytes), with the entries of each group
 * of 16 consecutive rows interleaved so that the entries of one position in
 * the 16 rows are adjacent.  Rows form tiles 16*T .. 16*T+R_T-1, R_T =
 * min(16, R - 16*T); row r of tile T, with nsb = K/32 and nb = K/256:
 *   plane A: the 16-byte piece of sub-block s (0..nsb-1) at entry
 *     16*T*nsb + s*R_T + r (entries of 16 bytes from byte 0);
 *   plane B: the 8-byte piece of sub-block s at entry 16*T*nsb + s*R_T + r
 *     (entries of 8 bytes from byte 128*NB);
 *   plane SC: for z = 0..nsb/4-1, the eight scale bytes 8*(z%2) .. 8*(z%2)+7
 *     of block z/2 (the scales of sub-blocks 4z .. 4z+3) at entry
 *     16*T*(nsb/4) + z*R_T + r (entries of 8 bytes from byte 192*NB);
 *   plane D: fp16 d of block b at entry 16*T*nb + b*R_T + r (entries of
 *     2 bytes from byte 208*NB).
 * With it a 64-lane load of 16 rows x 4 sub-blocks reads one contiguous
 * kilobyte, the operand shape of the int8 matrix-core kernel that serves
 * this layout.  Its outputs agree with the other layouts' to fp32 rounding
 * (a different summation order), and its per-sub-block integer sums are
 * identical.
 *
 * Column-planar Q8_1 activations (QMV_ACT_PLANAR), produced by
 * quantize_q8_1_planar: the bytes of each column's K/32 Q8_1 blocks,
 * rearranged inside the column (column n still starts at byte 36*(K/32)*n):
 * the K int8 quants (block b's 32 at byte 32*b of the column), then the K/32
 * fp16 d (block b's at byte K + 2*b), then the K/32 fp16 s (at byte
 * K + 2*(K/32) + 2*b).  The tiled product reads it with aligned 16-byte
 * loads and stores it to LDS unchanged; its outputs are bit-identical to
 * those from the same values in Q8_1 blocks.
 *
 * Conventions for every entry point.
 *   Memory: all data pointers are device pointers owned by the caller; the
 *   library never allocates, frees or synchronizes.  `stream` is a
 *   hipStream_t (NULL: the default stream).  Work is enqueued on `stream` and
 *   returns at once; calls are safe to capture in a HIP graph and are
 *   thread-safe across streams.  Outputs are overwritten, never accumulated.
 *   Errors: 0 on success, a negative QMV_ERR_* code otherwise.  Every argument
 *   check runs on the host before any HIP call, so a rejected call has no
 *   effect.  QMV_ERR_HIP means a launch failed; qmv_last_hip_error() returns
 *   the hipError_t of that failure (per calling thread).
 *   Preconditions the host cannot check: buffers are as large as stated and
 *   do not overlap outputs; activations are finite.
 */
#ifndef QMV_H
#define QMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    QMV_OK = 0,
    QMV_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size */
    QMV_ERR_UNSUPPORTED = -2,   /* K % 256 != 0, ncols not in 1..8, bad layout, too large */
    QMV_ERR_ALIGNMENT = -3,     /* a pointer below its required alignment */
    QMV_ERR_WORKSPACE = -4,     /* workspace missing or too small */
    QMV_ERR_HIP = -5            /* a HIP launch failed */
};

enum { QMV_LAYOUT_GGUF = 0, QMV_LAYOUT_PLANAR = 1, QMV_LAYOUT_TILED = 2 };

/* OR-ed into the layout argument together with QMV_LAYOUT_TILED: the
 * activations are column-planar (see above) instead of Q8_1 blocks. */
enum { QMV_ACT_PLANAR = 16 };

/* Largest supported sizes (larger calls return QMV_ERR_UNSUPPORTED before
 * any HIP call; every launch then stays below 2^32 work-items along x and
 * 65535 workgroups along y): K <= 2^20; products (and their argmax and
 * integer-sum forms) rows <= 2^26 - 1024 = 67,107,840; conversions
 * rows <= 2^31-1 with rows*K/256*8 < 2^32; row gathers nout*K/256 < 2^32;
 * quantizers ncols*K/4 < 2^32; the grouped MoE call as stated there; every
 * weight, activation and output buffer below 2^40 bytes. */

/* Quantize fp32 activations to Q8_1 (PR #2340 "What it changes" names the
 * Q8_1 activation quants).  Per block of 32 values of one column:
 * amax = max|x|, d = amax/127 (fp32 division), q = round-half-away-from-zero
 * of x/d (fp32 division; all zero when d == 0), stored d = fp16(d) and
 * s = fp16(d * sum q), both rounded to nearest even.
 * x: fp32 [ncols][K], 4-byte aligned.  xq: [ncols][K/32] blocks of 36 B,
 * 4-byte aligned.  K % 32 == 0, 1 <= ncols <= 65535. */
int quantize_q8_1(const float *x, void *xq, int64_t K, int ncols, void *stream);

/* As quantize_q8_1 (same arithmetic, same bytes), written in the
 * column-planar layout.  xq: 4-byte aligned (16-byte for the products). */
int quantize_q8_1_planar(const float *x, void *xq, int64_t K, int ncols, void *stream);

/* RMSNorm fused into the Q8_1 quantizer (the norm step ahead of the MMVQ
 * whose fused opt-in PR #1774 "How it was checked" measures end to end; the
 * pages do not define the norm, read here as RMSNorm).  Per column n:
 *   r = 1 / sqrt(sum_i x[n][i]^2 / K + eps), y[i] = (x[n][i] * r) * gamma[i]
 * in fp32 (the sum in a fixed order; IEEE division and square root), then
 * y is quantized exactly as quantize_q8_1 quantizes its input.  One launch,
 * no y in memory.  x: fp32 [ncols][K], gamma: fp32 [K], both 16-byte
 * aligned; eps >= 0 (finite; with eps = 0 an all-zero column has no
 * defined norm); xq: 4-byte aligned, Q8_1 blocks
 * (act_layout 0) or column-planar (act_layout QMV_ACT_PLANAR).
 * K % 32 == 0, 1 <= ncols <= 65535. */
int rmsnorm_quantize_q8_1(const float *x, const float *gamma, float eps, void *xq, int64_t K, int ncols,
                          int act_layout, void *stream);

/* Q6_K weights x Q8_1 activations (the Q6_K dense decode product of PR
 * #2340 "What it changes" and PR #2207 "How it was checked").
 * w: rows x K Q6_K matrix in `layout` (QMV_LAYOUT_GGUF: 210-byte blocks,
 * 4-byte aligned; QMV_LAYOUT_PLANAR, QMV_LAYOUT_TILED: the layouts above,
 * 16-byte aligned).  xq: Q8_1 [ncols][K/32], 4-byte aligned.  out: fp32
 * [ncols][rows], 4-byte aligned.  K % 256 == 0, 1 <= ncols <= 8.
 * GGUF and planar inputs run on the vector ALU (v_dot4_i32_i8); tiled
 * inputs on the int8 matrix cores (v_mfma_i32_16x16x64_i8, each 16-weight
 * scale group kept apart by masking the activation operand).  The matrix
 * cores are used although 1-8 columns are a bandwidth-bound GEMV because the
 * dot4 form is issue-bound on this GPU: at 8 columns of a 10240 x 2560
 * matrix a dot4 wave issues ~830 VALU instructions (~5 us of issue per SIMD,
 * longer than the ~4.5 us weight stream; 8.5 us per call), the matrix-core
 * wave ~450 (6.9 us per call), with HBM traffic 1.01x the weight bytes in
 * both.  layout = QMV_LAYOUT_TILED | QMV_ACT_PLANAR takes
 * column-planar activations (xq 16-byte aligned); any other layout with
 * QMV_ACT_PLANAR is QMV_ERR_UNSUPPORTED. */
int mmvq_q6k(const void *w, int layout, const void *xq, float *out,
             int64_t rows, int64_t K, int ncols, void *stream);

/* One product of a batch (mmvq_q6k_batch): w, xq, out, rows and ncols as
 * the arguments of mmvq_q6k of the same names. */
typedef struct qmv_q6k_job {
    const void *w;
    const void *xq;
    float *out;
    int64_t rows;
    int ncols;
} qmv_q6k_job;

/* Several independent Q6_K products of the same K in one launch -- the
 * decode products of a layer's matrices (each with its own weights,
 * activation columns and outputs), issued together so that the launch
 * ramps up and drains once rather than once per matrix (the pages' decode
 * step runs many such products back to back, PR #2207 "Issue: #1545, #1606
 * (Arc A-series decode)", "Summary").  jobs: host array of njobs
 * (1 <= njobs <= 8) descriptions, read during the call.  Tiled layout only
 * (layout = QMV_LAYOUT_TILED, optionally | QMV_ACT_PLANAR, for every job);
 * each job as for mmvq_q6k (w 16-byte aligned, xq 4-byte aligned or 16 for
 * column-planar activations, out 4-byte aligned, 1 <= ncols <= 8) and the
 * sum of the jobs' rows within the product limit.  Every job's output is
 * bit for bit what mmvq_q6k gives for it alone.  Outputs of different jobs
 * must not overlap each other or any input. */
int mmvq_q6k_batch(const qmv_q6k_job *jobs, int njobs, int layout, int64_t K, void *stream);

/* The same Q6_K x Q8_1 product for many columns at once (the prompt path,
 * which PR #2340 "What it changes" leaves as it is; the arithmetic is the
 * decode product's).  Tiled weights only: layout = QMV_LAYOUT_TILED,
 * optionally | QMV_ACT_PLANAR, with w, xq, out as for mmvq_q6k, and
 * 1 <= ncols <= 65535.  Every output column is bit-for-bit what mmvq_q6k
 * gives for that column alone.  QMV_ERR_UNSUPPORTED also when
 * (ceil(rows/16) + 32) * ceil(ncols/12) >= 2^22. */
int mmq_q6k(const void *w, int layout, const void *xq, float *out,
            int64_t rows, int64_t K, int ncols, void *stream);

/* Q4_K / Q5_K weights (GGUF blocks, 16-byte aligned; 144 and 176 B blocks
 * keep every field aligned, so no planar form is needed) x Q8_1 activations
 * (PR #2340 "What it changes" and PR #2207 "How it was checked" measure
 * these types).  The min term uses the exact integer sum of each Q8_1
 * block's quants.  Arguments as for mmvq_q6k. */
int mmvq_q4k(const void *w, const void *xq, float *out, int64_t rows, int64_t K,
             int ncols, void *stream);
int mmvq_q5k(const void *w, const void *xq, float *out, int64_t rows, int64_t K,
             int ncols, void *stream);

/* Several independent Q4_K (Q5_K) products of the same K issued together,
 * as mmvq_q6k_batch does for Q6_K (a decode step's products of one layer,
 * PR #2207 "Summary"): jobs is a host array of njobs (1 <= njobs <= 8)
 * descriptions, read during the call, each checked as mmvq_q4k (mmvq_q5k)
 * checks its arguments, and the sum of the jobs' rows within the product
 * limit.  Up to four jobs run in one launch; more run in one launch per
 * lanes-per-row class (a function of rows and K; one K gives at most two).
 * Every job's output is bit for bit what mmvq_q4k (mmvq_q5k) gives for it
 * alone.  Outputs of different jobs must not overlap each
 * other or any input. */
int mmvq_q4k_batch(const qmv_q6k_job *jobs, int njobs, int64_t K, void *stream);
int mmvq_q5k_batch(const qmv_q6k_job *jobs, int njobs, int64_t K, void *stream);

/* Load-time conversion of a GGUF Q6_K matrix into the planar layout above
 * (PR #2340 "What it changes").  Out of place; src (2-byte aligned) and dst
 * (16-byte aligned) are rows*K/256*210 bytes and must not overlap.  The
 * caller may free src afterwards. */
int repack_q6k_planar(const void *src, void *dst, int64_t rows, int64_t K, void *stream);
/* Inverse conversion, planar -> GGUF (for tests and for exporting). */
int unpack_q6k_planar(const void *src, void *dst, int64_t rows, int64_t K, void *stream);
/* The same two conversions for the tiled layout above (same sizes,
 * alignments and checks). */
int repack_q6k_tiled(const void *src, void *dst, int64_t rows, int64_t K, void *stream);
int unpack_q6k_tiled(const void *src, void *dst, int64_t rows, int64_t K, void *stream);

/* Row gather within one layout (the draft head's row subset taken from the
 * converted LM head, PR #2340 "What it changes"): dst is the nout x K Q6_K
 * matrix, in the same `layout` as src (rows x K), whose row j is src row
 * ids[j].  ids: int32 [nout], device memory, 4-byte aligned; an id outside
 * [0, rows) yields an all-zero row (device data, so not checked on the host).
 * src/dst: GGUF any alignment, planar and tiled 16-byte aligned; they must
 * not overlap.  Load-time only. */
int gather_q6k_rows(const void *src, int layout, int64_t rows, int64_t K, const int32_t *ids,
                    int64_t nout, void *dst, void *stream);

/* Greedy argmax over the rows of the product (the verify window's next-token
 * choice over an LM head, without writing rows x ncols outputs): for each
 * column n, idx[n] = the row r with the largest out[n][r] of mmvq_q6k and
 * val[n] = that value, bit for bit the fp32 output mmvq_q6k gives for the
 * same inputs; among equal values the lowest row wins, -0 counts as +0.
 * Tiled layout only (QMV_LAYOUT_TILED, optionally | QMV_ACT_PLANAR;
 * others: QMV_ERR_UNSUPPORTED).
 * idx int32 [ncols], val fp32 [ncols] (4-byte aligned); ws: device
 * workspace of at least mmvq_q6k_argmax_workspace(rows, ncols) bytes,
 * 8-byte aligned, overwritten (one 8-byte key per column and 16-row tile,
 * then 256 bytes of per-column reduction state; calls sharing a workspace
 * must not overlap).
 * Other arguments and checks as for mmvq_q6k.  Two launches: the product
 * with per-tile maxima, then one reduction per column.  Outputs must be
 * finite. */
int mmvq_q6k_argmax(const void *w, int layout, const void *xq, int64_t rows, int64_t K,
                    int ncols, int32_t *idx, float *val, void *ws, size_t ws_bytes,
                    void *stream);
size_t mmvq_q6k_argmax_workspace(int64_t rows, int ncols);

/* The k largest outputs of each column of the product (the candidates a
 * verify window keeps when it samples beyond the greedy token; the pages'
 * verify path runs the LM head at 1-8 columns, PR #2207 "Summary", with the
 * draft head taken from the converted head, PR #2340 "What it changes"):
 * for each column n, idx[n][i] and val[n][i] (i = 0..k-1) are the rows and
 * fp32 values of mmvq_q6k's outputs in descending order of value, among
 * equal values the lower row first, -0 counted as +0; the values are bit for
 * bit mmvq_q6k's outputs for the same inputs.  Any layout mmvq_q6k takes.
 * 1 <= k <= 64, k <= rows, and ceil(rows/4096) * k <= 4096 (k = 64 up to
 * 262,144 rows; k = 16 up to 1,048,576).  idx int32 [ncols][k], val fp32
 * [ncols][k] (4-byte aligned); ws: device workspace of at least
 * mmvq_q6k_topk_workspace(rows, ncols, k) bytes, 256-byte aligned,
 * overwritten: the product's fp32 outputs [ncols][rows], then (at the next
 * 256-byte boundary) 8-byte candidate keys.  Three launches: the product,
 * a radix select of the k largest keys of each 4096-row chunk, a radix
 * select of each column's candidates ranked into order.  Other arguments and
 * checks as for mmvq_q6k; outputs must be finite. */
int mmvq_q6k_topk(const void *w, int layout, const void *xq, int64_t rows, int64_t K, int ncols,
                  int k, int32_t *idx, float *val, void *ws, size_t ws_bytes, void *stream);
size_t mmvq_q6k_topk_workspace(int64_t rows, int ncols, int k);

/* Per-sub-block integer sums of the same kernels (for verification):
 * isums int32 [ncols][rows][K/32].  Q6_K: sum over the sub-block's two
 * 16-weight groups of scale * sum (q6-32)*q8.  Q4_K/Q5_K: sum q*q8 of the
 * sub-block, unscaled.  Same arguments and checks as the products. */
int mmvq_q6k_isums(const void *w, int layout, const void *xq, int32_t *isums,
                   int64_t rows, int64_t K, int ncols, void *stream);
int mmvq_q4k_isums(const void *w, const void *xq, int32_t *isums, int64_t rows,
                   int64_t K, int ncols, void *stream);
int mmvq_q5k_isums(const void *w, const void *xq, int32_t *isums, int64_t rows,
                   int64_t K, int ncols, void *stream);

/* Grouped MoE-expert product over a window of T routed tokens (the
 * routed-expert gate/up and down kernels of issue #2801 "[Feature]: SYCL:
 * cheaper IQ weight decodes in the grouped expert kernels"; the token windows
 * and empty expert groups of PR #2746 "B70 validation").  For every token t
 * and slot k (slot = t*topk + k), e = ids[t][k]:
 *   g = gate_e . xq_t, u = up_e . xq_t           (Q4_K MMVQ, d_ff rows)
 *   h = silu(g) * u, silu(g) = g / (1 + exp(-g))  (fp32)
 *   hq = quantize_q8_1(h)                         (d_ff/32 blocks)
 *   y = down_e . hq                               (Q6_K MMVQ, d_model rows)
 *   out[t] = sum over k = 0..topk-1, in that order, of route_w[t][k] * y.
 * Each expert's gate and up rows are read once for all tokens routed to it;
 * its down rows once per routed token with planar down weights (two
 * launches: gate/up, then down and the routed sum by (row block, token);
 * the repeats mostly come from the caches) and once with GGUF down weights
 * (three launches: gate/up, down, the routed sum).  Experts with no token
 * are not read.
 *   w_gate, w_up: Q4_K [E][d_ff][d_model/256] blocks, 16-byte aligned.
 *   w_down: Q6_K [E][d_model][d_ff/256] in down_layout (GGUF: 4-byte
 *     aligned; planar: 16-byte aligned, the repack_q6k_planar of the whole
 *     tensor taken as E*d_model rows).
 *   xq: Q8_1 [T][d_model/32] (4-byte aligned); ids: int32 [T][topk] in
 *   [0, E), distinct within a token; route_w: fp32 [T][topk];
 *   out: fp32 [T][d_model], overwritten.
 *   1 <= T <= 8, 1 <= topk <= 8, d_model and d_ff multiples of 256 (at
 *   most 2^20), E*d_model <= 2^31-1, and d_model/r <= 65535 with r the
 *   down rows per workgroup (4*64/U, U = lanes per down row: the largest of
 *   64, 32, 16 dividing d_ff/32 with at least three units each, else 8), so
 *   d_model <= 262,140 at least.
 *   ws: device workspace of at least grouped_expert_mmvq_workspace() bytes,
 *   256-byte aligned.  Layout (all offsets from ws, S = T*topk):
 *     int32 hdr[64]: hdr[0] = number of distinct experts hit, hdr[1] = number
 *       of ids outside [0, E) (such slots contribute nothing);
 *     int32 expert[S], count[S], first[S] @256: per hit expert (ascending id)
 *       its id, its number of slots and its first position in slot_list;
 *     int32 slot_list[S] @256+12*S: slots grouped by expert, ascending slot
 *       order inside a group;
 *     fp32 h[S][d_ff] @H = align256(256+16*S);
 *     Q8_1 hq[S][d_ff/32] @HQ = align256(H + 4*S*d_ff);
 *     fp32 y[S][d_model] @Y = align256(HQ + 36*S*d_ff/32).
 *   The workspace is overwritten; ids that repeat within a token are handled
 *   (their slots are processed like any other) but break the "read once"
 *   property of gate and up. */
int grouped_expert_mmvq(const void *w_gate, const void *w_up, const void *w_down,
                        int down_layout, const void *xq, const int32_t *ids,
                        const float *route_w, float *out, int E, int T, int topk,
                        int64_t d_model, int64_t d_ff, void *ws, size_t ws_bytes,
                        void *stream);
size_t grouped_expert_mmvq_workspace(int E, int T, int topk, int64_t d_model, int64_t d_ff);

/* grouped_expert_mmvq without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid allocation): the same kernels, arguments, checks and
 * results, with the workspace taken from a 4 MiB device array that the
 * library holds on every GPU it runs on until the process ends.  Calls whose
 * workspace would exceed 4 MiB (grouped_expert_mmvq_workspace() > 4194304)
 * return QMV_ERR_UNSUPPORTED before any HIP call.  The array of the calling
 * thread's current device is used (`stream` must belong to that device);
 * its address is looked up on the first call on each device.  Nothing in it
 * needs clearing between calls (every call writes what it reads), but every
 * call on one GPU shares that GPU's array: calls that overlap in time on one
 * GPU (on different streams, or from several threads) race and must not be
 * issued. */
int grouped_expert_mmvq_noalloc(const void *w_gate, const void *w_up, const void *w_down,
                                int down_layout, const void *xq, const int32_t *ids,
                                const float *route_w, float *out, int E, int T, int topk,
                                int64_t d_model, int64_t d_ff, void *stream);

/* Diagnostics. */
/* Streaming-read calibration: reads `bytes` (a multiple of 16) from src
 * (16-byte aligned) with 16-byte non-temporal loads, four per thread per
 * step, over `blocks` (1..65535) workgroups of 256 threads, or, when blocks
 * is 0, over one workgroup per 16 KiB so that each thread takes one step
 * (then bytes < 2^38).
 * sink (uint32, as many words as workgroups) is written only if a thread's
 * XOR of its data equals a fixed constant.  Its duration at a given size is
 * the achievable read time the MMVQ kernels are measured against. */
int qmv_stream_read(const void *src, int64_t bytes, uint32_t *sink, int blocks, void *stream);

const char *qmv_strerror(int code);
int qmv_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* QMV_H */

// moe.hip -- grouped MoE-expert product over a window of routed tokens.
//
// Three launches on one stream, none needing a host synchronization:
//   gate/up : workgroup (i, tile) looks at slot i (slot = t*topk + k); if
//             slot i is the first slot routed to its expert e, it takes e and
//             32 rows of d_ff: gate and up are read once for all of e's slots
//             (their count is the MMVQ column count), then h = silu(g)*u and
//             its Q8_1 block are written per slot.  Other workgroups exit.
//   down    : the same selection, with a row tile of d_model: Q6_K MMVQ over
//             the expert's requantized slots, y written per slot;
//   combine : out[t] = sum over k, ascending, of route_w[t][k] * y[t][k].
// With planar down weights (and d_ff <= 1024) down and combine are one
// launch by (row block, token) instead (k_moe_down_tok, below).
// The selection is one wave ballot over the slot ids (S <= 64 = one wave),
// and an expert's slots are taken in ascending slot order.  No workgroup
// reads the weights of an expert no slot is routed to.
#include <mutex>

#include "device.hpp"
#include "launch.hpp"

namespace qmv {

// Device scratch for grouped_expert_mmvq_noalloc: the routed chain's
// workspace when the caller cannot allocate one.  In host code `scratch`
// only stands for the symbol; its device address (one copy per GPU) comes
// from hipGetSymbolAddress, looked up once per device and kept.
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t moe_scratch(int device, void **ptr) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[device], [device] {
        // (the calling thread's current device is `device`)
        void *p = nullptr;
        g_scratch_err[device] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[device] = g_scratch_err[device] == hipSuccess ? p : nullptr;
    });
    *ptr = g_scratch_ptr[device];
    return g_scratch_err[device];
}

namespace {
__host__ __device__ inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
}  // namespace

MoeLayout moe_layout(int T, int topk, int64_t d_model, int64_t d_ff) {
    const int64_t S = (int64_t)T * topk;
    MoeLayout L;
    L.off_h = align256(256 + 16 * S);
    L.off_hq = align256(L.off_h + 4 * S * d_ff);
    L.off_y = align256(L.off_hq + (int64_t)kQ81Bytes * S * (d_ff / 32));
    L.total = align256(L.off_y + 4 * S * d_model);
    return L;
}

// Slot selection shared by the gate/up and down kernels.  Every wave loads
// the S slot ids (lane s holds ids[s], or -1 when out of range or s >= S).
// Returns false when slot i is not the first slot of a valid expert; else
// sets e and the mask of e's slots.
__device__ __forceinline__ bool moe_select(const MoeArgs &m, int i, int &e, uint64_t &mask) {
    const int lane = threadIdx.x & (kWave - 1);
    int id = -1;
    if (lane < m.S) {
        id = m.ids[lane];
        if (id < 0 || id >= m.E) id = -1;
    }
    e = __builtin_amdgcn_readlane(id, i);
    if (e < 0) return false;
    mask = __ballot(id == e);
    return (mask & ((1ull << i) - 1)) == 0;
}

// Routing tables of the workspace (documented in qmv.h, for inspection):
// written by one wave, each lane for its own slot, in one pass over the S
// slot ids read as wave-uniform values (v_readlane; no LDS traffic).  Run
// by a workgroup of its own so that no product workgroup waits for it
// (from slot 0's workgroup, with two LDS shuffle passes over 64 lanes, it
// held the gate/up launch 3-4 us longer at one token).
__device__ void moe_write_tables(const MoeArgs &m) {
    const int s = threadIdx.x & (kWave - 1);
    int e = -1;
    if (s < m.S) {
        e = m.ids[s];
        if (e < 0 || e >= m.E) e = -1;
    }
    const uint64_t valid = __ballot(e >= 0);
    // before: valid slots with a smaller expert; pos: earlier slots of this
    // expert; cnt: slots of this expert; lt: the slots with a smaller expert
    int before = 0, pos = 0, cnt = 0;
    uint64_t lt = 0;
    for (int t = 0; t < m.S; t++) {
        const int et = __builtin_amdgcn_readlane(e, t);
        if (et < 0 || e < 0) continue;
        if (et < e) {
            before++;
            lt |= 1ull << t;
        } else if (et == e) {
            cnt++;
            if (t < s) pos++;
        }
    }
    const bool first_occ = e >= 0 && pos == 0;
    const uint64_t fo = __ballot(first_occ);
    const int rank = __popcll(lt & fo);     // distinct experts below e
    int32_t *wsi = reinterpret_cast<int32_t *>(m.ws);
    int32_t *expert = wsi + 64, *count = expert + m.S, *first = count + m.S, *slot_list = first + m.S;
    if (e >= 0) {
        slot_list[before + pos] = s;
        if (first_occ) {
            expert[rank] = e;
            count[rank] = cnt;
            first[rank] = before;
        }
    }
    if (s == 0) {
        wsi[0] = __popcll(fo);
        wsi[1] = m.S - __popcll(valid);
    }
}

// Slot columns per pass of an expert's workgroup.  An expert with more
// routed slots takes further passes, whose weight reads hit L2; few
// column-count variants keep the kernels' register budget small (every
// variant is inlined into the one kernel and the register count is that of
// the union).
#ifndef QMV_MOE_COLS
#define QMV_MOE_COLS 2
#endif
constexpr int kMoeCols = QMV_MOE_COLS;
static_assert(kMoeCols >= 1 && kMoeCols <= 4, "pass width");

// ------------------------------------------------------------- gate / up
constexpr int kGuRows = 32;   // real rows per workgroup: one Q8_1 block of h

template <int N, int U, bool RAGGED>
__device__ __forceinline__ void gateup_n(const MoeArgs &m, int e, const int32_t (&slots)[8], int tile,
                                         uint8_t *lds) {
    constexpr int nthr = U * kWave;
    constexpr int its = its_for(Q4GateUp::IT, N, U, Q4GateUp::SBPU, nthr);
    float *H = reinterpret_cast<float *>(lds);                 // [N][32]
    uint8_t *act = lds + 8 * kGuRows * sizeof(float);
    int sl[N];
#pragma unroll
    for (int n = 0; n < N; n++) sl[n] = slots[n];

    Q4GateUp f;
    f.g.init(m.w_gate, 0, m.d_model);
    f.u.init(m.w_up, 0, m.d_model);
    f.base_row = (int64_t)e * m.d_ff;
    MmvqArgs a;
    a.xq = m.xq;
    a.dump = nullptr;
    a.rows = 2 * m.d_ff;
    a.K = m.d_model;
    a.colpack = 0;
#pragma unroll
    for (int n = 0; n < N; n++) a.colpack |= (uint64_t)(sl[n] / m.topk) << (8 * n);
    a.xstride = m.d_model / 32;
    a.its = its;
    a.nout = N;
    const int64_t row0 = (int64_t)tile * 2 * kGuRows;
    float acc[1][N];
    // the gate/up weight loads of the first kPreUnits units go out with the
    // activation loads (the tile of this 512-thread kernel is small)
    mmvq_rows<Q4GateUp, N, U, 1, nthr, false, Q4GateUp::IT, RAGGED, kPreUnits>(f, a, row0, act, acc);

    const int lane = threadIdx.x & (kWave - 1), u = lane % U;
    const int64_t vrow = lane_row<U, 1>(row0, 0);
    float *hg = reinterpret_cast<float *>(m.ws + m.off_h);
#pragma unroll
    for (int n = 0; n < N; n++) {
        const float up = __shfl_down(acc[0][n], U);
        if ((vrow & 1) == 0 && vrow < a.rows && u == n % U) {
            const float g = acc[0][n];
            const float h = g / (1.0f + expf(-g)) * up;
            const int r = (int)((vrow - row0) >> 1);
            H[n * kGuRows + r] = h;
            hg[(int64_t)sl[n] * m.d_ff + (int64_t)tile * kGuRows + r] = h;
        }
    }
    lds_barrier();
    const int t = threadIdx.x;
    if (t < N * 32) {
        const int n = t >> 5, i = t & 31;
        int slot = sl[0];
#pragma unroll
        for (int k = 1; k < N; k++)
            if (n == k) slot = sl[k];
        uint32_t db, sb;
        const int q = q8_1_quantize32(H[n * kGuRows + i], db, sb);
        uint8_t *hq = m.ws + m.off_hq + ((int64_t)slot * (m.d_ff / 32) + tile) * kQ81Bytes;
        q8_1_store32(hq, i, q, db, sb, true);
    }
}

template <int U, bool RAGGED>
__global__ __launch_bounds__(U *kWave) void k_moe_gateup(MoeArgs m) {
    extern __shared__ __align__(16) uint8_t lds[];
    int e;
    uint64_t mask;
    if (blockIdx.x == gridDim.x - 1) {        // the extra column: tables only
        if (blockIdx.y == 0 && threadIdx.x < kWave) moe_write_tables(m);
        return;
    }
    if (!moe_select(m, blockIdx.x, e, mask)) return;
    int done = 0;
    while (mask) {
        if (done > 0) lds_barrier();
        int32_t sl[8];
        int nc = 0;
#pragma unroll
        for (int n = 0; n < 8; n++) {
            sl[n] = 0;
            if (mask && n < kMoeCols) {
                sl[n] = __ffsll((long long)mask) - 1;
                mask &= mask - 1;
                nc++;
            }
        }
        if (nc == 1) gateup_n<1, U, RAGGED>(m, e, sl, blockIdx.y, lds);
        if constexpr (kMoeCols >= 2) if (nc == 2) gateup_n<2, U, RAGGED>(m, e, sl, blockIdx.y, lds);
        if constexpr (kMoeCols >= 3) if (nc == 3) gateup_n<3, U, RAGGED>(m, e, sl, blockIdx.y, lds);
        if constexpr (kMoeCols >= 4) if (nc == 4) gateup_n<4, U, RAGGED>(m, e, sl, blockIdx.y, lds);
        done += nc;
    }
}

// ------------------------------------------------------------------ down
constexpr int kDnWaves = 4;

template <class F, int N, int U, int IT, bool RAGGED>
__device__ __forceinline__ void down_n(const MoeArgs &m, int e, const int32_t (&slots)[8], int tile,
                                       uint8_t *lds) {
    constexpr int nthr = kDnWaves * kWave;
    constexpr int its = its_for(IT, N, U, F::SBPU, nthr);
    int sl[N];
#pragma unroll
    for (int n = 0; n < N; n++) sl[n] = slots[n];
    F f;
    f.init(m.w_down, (int64_t)m.E * m.d_model, m.d_ff);
    MmvqArgs a;
    a.xq = m.ws + m.off_hq;
    a.dump = nullptr;
    a.rows = (int64_t)(e + 1) * m.d_model;
    a.K = m.d_ff;
    a.colpack = 0;
#pragma unroll
    for (int n = 0; n < N; n++) a.colpack |= (uint64_t)sl[n] << (8 * n);
    a.xstride = m.d_ff / 32;
    a.its = its;
    a.nout = N;
    const int64_t row0 = (int64_t)e * m.d_model + (int64_t)tile * kDnWaves * (kWave / U);
    float acc[1][N];
    mmvq_rows<F, N, U, 1, nthr, false, IT, RAGGED>(f, a, row0, lds, acc);
    const int64_t row = lane_row<U, 1>(row0, 0);
    const int u = (threadIdx.x & (kWave - 1)) % U;
    float *y = reinterpret_cast<float *>(m.ws + m.off_y);
    if (row < a.rows) {
#pragma unroll
        for (int n = 0; n < N; n++)
            if (u == n % U) y[(int64_t)sl[n] * m.d_model + (row - (int64_t)e * m.d_model)] = acc[0][n];
    }
}

template <class F, int U, int IT, bool RAGGED>
__global__ __launch_bounds__(kDnWaves *kWave) void k_moe_down(MoeArgs m) {
    extern __shared__ __align__(16) uint8_t lds[];
    int e;
    uint64_t mask;
    if (!moe_select(m, blockIdx.x, e, mask)) return;
    int done = 0;
    while (mask) {
        if (done > 0) lds_barrier();
        int32_t sl[8];
        int nc = 0;
#pragma unroll
        for (int n = 0; n < 8; n++) {
            sl[n] = 0;
            if (mask && n < kMoeCols) {
                sl[n] = __ffsll((long long)mask) - 1;
                mask &= mask - 1;
                nc++;
            }
        }
        if (nc == 1) down_n<F, 1, U, IT, RAGGED>(m, e, sl, blockIdx.y, lds);
        if constexpr (kMoeCols >= 2) if (nc == 2) down_n<F, 2, U, IT, RAGGED>(m, e, sl, blockIdx.y, lds);
        if constexpr (kMoeCols >= 3) if (nc == 3) down_n<F, 3, U, IT, RAGGED>(m, e, sl, blockIdx.y, lds);
        if constexpr (kMoeCols >= 4) if (nc == 4) down_n<F, 4, U, IT, RAGGED>(m, e, sl, blockIdx.y, lds);
        done += nc;
    }
}

// --------------------------------------------------------------- combine
// out[t][i] = sum over k ascending of route_w[t][k] * y[t*topk+k][i]; slots
// with an out-of-range id add nothing.  All ids, weights and y values are
// loaded before the sum (one round of memory latency, not topk).
__global__ __launch_bounds__(256) void k_moe_combine(MoeArgs m) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int t = blockIdx.y;
    if (i >= m.d_model) return;
    const float *y = reinterpret_cast<const float *>(m.ws + m.off_y);
    int e[8];
    float w[8], v[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int s = t * m.topk + min(k, m.topk - 1);
        e[k] = m.ids[s];
        w[k] = m.route_w[s];
        v[k] = y[(int64_t)s * m.d_model + i];
    }
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; k++)
        if (k < m.topk && e[k] >= 0 && e[k] < m.E) acc = __builtin_fmaf(w[k], v[k], acc);
    m.out[(int64_t)t * m.d_model + i] = acc;
}

// ------------------------------------------------- down + routed sum, by token
// Planar down weights, d_ff / 256 <= kDtMaxUnits: workgroup (x, t) owns
// 8 or 16 rows of d_model for token t and holds one wave per routed slot of
// the token.  Wave k forms y of slot t*topk + k for the workgroup's rows (its
// expert's rows times the slot's requantized h, eight lanes per row, lane u
// taking sub-blocks u, u + 8, ...; the h blocks go out before the slot id is
// back), then after one barrier the token's routed sum of those rows is
// formed in ascending k, as k_moe_combine does.  No workgroup waits on
// another and there is no combine launch.  An expert routed from several
// tokens is read once per token; the repeats are served by the caches
// (measured HBM fetch in the design notes).  y is also written to the
// workspace.
constexpr int kDtMaxUnits = 4;   // d_ff / 256 at most
constexpr int64_t kDtWideGrid = 1024;

// RPL rows per lane (rows r and r + 8 when RPL = 2): 8 * RPL rows per
// workgroup.
template <int UN, int RPL>
__global__ __launch_bounds__(8 * kWave) void k_moe_down_tok(MoeArgs m) {
    constexpr int ROWS = 8 * RPL;
    __shared__ float ylds[8][ROWS];
    __shared__ float wlds[8];                                // route weight of each slot
    __shared__ int vlds[8];                                  // whether its id is in range
    const int nsb = 8 * UN;                                  // d_ff / 32
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x & (kWave - 1);
    const int r = lane >> 3, u = lane & 7;
    const int tk = blockIdx.y, slot = tk * m.topk + wave;    // wave < topk (one wave per slot)
    const int64_t row0 = (int64_t)blockIdx.x * ROWS;
    const uint8_t *hq = m.ws + m.off_hq;
    ActRaw x[UN];
#pragma unroll
    for (int k = 0; k < UN; k++) act_load(x[k], hq, (int64_t)slot * nsb + u + 8 * k);
    const int e = m.ids[slot];
    const float rw = m.route_w[slot];
    const bool ev = e >= 0 && e < m.E;
    if (lane == 0) {
        wlds[wave] = rw;
        vlds[wave] = ev ? 1 : 0;
    }
    if (ev) {
        // sub-blocks u + 8k of a row: with 8 * UN sub-blocks a row,
        // sub-block u + 8k lies in the row's superblock k
        Q6Planar fmt;
        fmt.init(m.w_down, (int64_t)m.E * m.d_model, m.d_ff);
        Q6Planar::Raw w[RPL][UN];
#pragma unroll
        for (int p = 0; p < RPL; p++) {
            const int64_t wrow = (int64_t)e * m.d_model + row0 + r + 8 * p;
            const int64_t i0 = wrow * nsb + u;
#pragma unroll
            for (int k = 0; k < UN; k++) {
                w[p][k].a = fmt.A[i0 + 8 * k];
                w[p][k].b = fmt.B[i0 + 8 * k];
                w[p][k].sc = fmt.SC[i0 + 8 * k];
                w[p][k].d = fmt.D[wrow * UN + k];
            }
        }
        float a[RPL];
#pragma unroll
        for (int p = 0; p < RPL; p++) {
            a[p] = 0.0f;
#pragma unroll
            for (int k = 0; k < UN; k++) {
                int v[8];
                Q6Planar::codes(w[p][k], v);
                const int sc0 = sext8(w[p][k].sc, 0), sc1 = sext8(w[p][k].sc, 1);
                int d0 = sdot4(v[0], (int)x[k].w[1], 0);
                d0 = sdot4(v[1], (int)x[k].w[2], d0);
                d0 = sdot4(v[2], (int)x[k].w[3], d0);
                d0 = sdot4(v[3], (int)x[k].w[4], d0);
                int d1 = sdot4(v[4], (int)x[k].w[5], 0);
                d1 = sdot4(v[5], (int)x[k].w[6], d1);
                d1 = sdot4(v[6], (int)x[k].w[7], d1);
                d1 = sdot4(v[7], (int)x[k].w[8], d1);
                const int isum4 = __mul24(sc0, d0) + __mul24(sc1, d1);   // 4 * isum, exact
                const float da = half_to_float(x[k].w[0]) * 0.25f;
                a[p] = __builtin_fmaf(half_to_float(w[p][k].d) * da, (float)isum4, a[p]);
            }
            a[p] = group_sum<8>(a[p]);
        }
        if (u == 0) {
            float *yws = reinterpret_cast<float *>(m.ws + m.off_y) + (int64_t)slot * m.d_model + row0;
#pragma unroll
            for (int p = 0; p < RPL; p++) {
                ylds[wave][r + 8 * p] = a[p];
                yws[r + 8 * p] = a[p];
            }
        }
    }
    lds_barrier();
    // the routed sum from LDS only: each wave put its slot's route weight
    // and id check there with its y (reading the ids and weights here, a
    // chain of dependent global loads after the barrier, cost 0.1-0.25 us
    // per call at T = 1..8)
    if (threadIdx.x < ROWS) {
        const int rr = threadIdx.x;
        float acc = 0.0f;
        for (int k = 0; k < m.topk; k++)
            if (vlds[k]) acc = __builtin_fmaf(wlds[k], ylds[k][rr], acc);
        m.out[(int64_t)tk * m.d_model + row0 + rr] = acc;
    }
}

// ------------------------------------------------------------------ host
template <int U, bool RAGGED>
static hipError_t launch_gateup_r(const MoeArgs &m, int smax, hipStream_t s) {
    constexpr int nthr = U * kWave;
    size_t act = 0;
    // largest tile over the column counts a workgroup may meet
    for (int n = 1; n <= kMoeCols; n++) {
        size_t b = (size_t)n * its_for(Q4GateUp::IT, n, U, Q4GateUp::SBPU, nthr) * U * Q4GateUp::SBPU *
                   kActBytesPerBlock;
        if (b > act) act = b;
    }
    const size_t lds = 8 * kGuRows * sizeof(float) + act;
    // one workgroup column per slot, plus one that writes the routing tables
    hipLaunchKernelGGL((k_moe_gateup<U, RAGGED>), dim3(smax + 1, (unsigned)(m.d_ff / kGuRows)), dim3(nthr), lds,
                       s, m);
    return hipGetLastError();
}

// Rows that are a whole number of register chunks use the kernels without
// the ragged-chunk code (fewer registers).
template <int U>
static hipError_t launch_gateup(const MoeArgs &m, int smax, hipStream_t s) {
    const int units = (int)(m.d_model / 32 / Q4GateUp::SBPU);
    return units % (U * Q4GateUp::IT) == 0 ? launch_gateup_r<U, false>(m, smax, s)
                                           : launch_gateup_r<U, true>(m, smax, s);
}

template <class F, int U, int IT, bool RAGGED>
static hipError_t launch_down_r(const MoeArgs &m, int smax, hipStream_t s) {
    constexpr int nthr = kDnWaves * kWave;
    size_t lds = 0;
    // largest tile over the column counts a workgroup may meet
    for (int n = 1; n <= kMoeCols; n++) {
        int its = its_for(IT, n, U, F::SBPU, nthr);
        size_t b = (size_t)n * its * U * F::SBPU * kActBytesPerBlock;
        if (b > lds) lds = b;
    }
    hipError_t e = allow_lds(reinterpret_cast<const void *>(&k_moe_down<F, U, IT, RAGGED>), lds);
    if (e != hipSuccess) return e;
    const int64_t rpb = kDnWaves * (kWave / U);
    hipLaunchKernelGGL((k_moe_down<F, U, IT, RAGGED>), dim3(smax, (unsigned)((m.d_model + rpb - 1) / rpb)),
                       dim3(nthr), lds, s, m);
    return hipGetLastError();
}

template <class F, int U, int IT>
static hipError_t launch_down_ui(const MoeArgs &m, int smax, hipStream_t s) {
    const int units = (int)(m.d_ff / 32 / F::SBPU);
    return units % (U * IT) == 0 ? launch_down_r<F, U, IT, false>(m, smax, s)
                                 : launch_down_r<F, U, IT, true>(m, smax, s);
}

template <class F, int U>
static hipError_t launch_down_u(const MoeArgs &m, int smax, hipStream_t s) {
    if constexpr (F::IT > 3) {
        if (depth_for((int)(m.d_ff / 32), U, F::IT) == 3) return launch_down_ui<F, U, 3>(m, smax, s);
    }
    return launch_down_ui<F, U, F::IT>(m, smax, s);
}

template <class F>
static hipError_t launch_down(const MoeArgs &m, int smax, hipStream_t s) {
    switch (choose_u((int)(m.d_ff / 32))) {
    case 8: return launch_down_u<F, 8>(m, smax, s);
    case 16: return launch_down_u<F, 16>(m, smax, s);
    case 32: return launch_down_u<F, 32>(m, smax, s);
    default: return launch_down_u<F, 64>(m, smax, s);
    }
}

bool moe_grid_fits(int S, int64_t d_model, int64_t d_ff, int64_t max_grid_y) {
    // gate/up: d_ff/32 row tiles along y; down: row blocks of kDnWaves waves
    // along y (either down path is taken depending on the window, so both
    // must fit); combine: the T tokens along y
    const int64_t rpb = kDnWaves * (kWave / choose_u((int)(d_ff / 32)));
    return d_ff / kGuRows <= max_grid_y && (d_model + rpb - 1) / rpb <= max_grid_y && S <= max_grid_y;
}

hipError_t launch_moe(const MoeArgs &m, int down_layout, hipStream_t s) {
    const int smax = m.S;   // one workgroup column per slot; non-first slots exit
    // gate/up: eight lanes per row whatever d_model (512-thread workgroups
    // keep the register budget of two waves per SIMD)
    hipError_t err = launch_gateup<8>(m, smax, s);
    if (err != hipSuccess) return err;
    const int un = (int)(m.d_ff / 256);
    if (down_layout == 1 && un <= kDtMaxUnits && m.d_model % 16 == 0) {
        // down and the routed sum in one launch, by (row block, token); two
        // rows per lane once that still gives kDtWideGrid workgroups (one
        // token at d_model 2560: 12.7 -> 12.5 us per call; two: 18.1 ->
        // 18.8 us, so one row there; eight: 46.6 -> 44.5-45.2 us)
        const bool two = (m.d_model / 16) * m.T >= kDtWideGrid;
        const dim3 grid((unsigned)(m.d_model / (two ? 16 : 8)), (unsigned)m.T), block(m.topk * kWave);
        const void *k = nullptr;
        switch (un * 2 + (two ? 1 : 0)) {
        case 2: k = reinterpret_cast<const void *>(&k_moe_down_tok<1, 1>); break;
        case 3: k = reinterpret_cast<const void *>(&k_moe_down_tok<1, 2>); break;
        case 4: k = reinterpret_cast<const void *>(&k_moe_down_tok<2, 1>); break;
        case 5: k = reinterpret_cast<const void *>(&k_moe_down_tok<2, 2>); break;
        case 6: k = reinterpret_cast<const void *>(&k_moe_down_tok<3, 1>); break;
        case 7: k = reinterpret_cast<const void *>(&k_moe_down_tok<3, 2>); break;
        case 8: k = reinterpret_cast<const void *>(&k_moe_down_tok<4, 1>); break;
        default: k = reinterpret_cast<const void *>(&k_moe_down_tok<4, 2>); break;
        }
        void *args[] = {const_cast<MoeArgs *>(&m)};
        return hipLaunchKernel(k, grid, block, args, 0, s);
    }
    err = down_layout == 1 ? launch_down<Q6Planar>(m, smax, s) : launch_down<Q6Gguf>(m, smax, s);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_moe_combine, dim3((unsigned)((m.d_model + 255) / 256), m.T), dim3(256), 0, s, m);
    return hipGetLastError();
}

}  // namespace qmv

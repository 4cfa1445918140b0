// k_qk.hip -- Q4_0 and Q6_K weight matvecs against a Q8_0 activation on gfx950.
//
// What it computes (the current path's MoE kernel runs on Q6_K weights,
// "Current Inference Path -- Architecture Map", section 4; candle keeps GGML
// block order, "Target Inference Architecture: hf2q on mlx-native", section
// 8, Q1; the int8 x int8 product with int32 accumulation of "Design:
// lattice-inference", Current Design):
//     Q4_0: y[r] = sum_b d_w[r,b] * d_x[b] * sum_{i<32} (n[r,32b+i] - 8) * x_q[32b+i]
//     Q6_K: y[r] = sum_k d[r,k/16] * sc[r,k] * d_x[k/2] * sum_{i<16} (q[r,16k+i] - 32) * x_q[16k+i]
//     (+ residual[r]), every inner sum an exact int32 dot.
//
// Device layout (SoA, from GGML blocks by the pack helpers):
//   Q4_0: qs [rows][cols/2] (each 32-value block's 16 code bytes in GGML
//         order: byte j holds value j in its low nibble, value j+16 in its
//         high nibble), d f16 [rows][cols/32];
//   Q6_K: ql [rows][cols/2], qh [rows][cols/4], sc int8 [rows][cols/16],
//         d f16 [rows][cols/256], each 256-value super-block's arrays in GGML
//         order.
//
// Mapping onto CDNA4.  A lane owns one unit of a row per step (lq_qk.h: a
// Q4_0 block or a quarter of a Q6_K super-block) and its exact int32 dots
// with the activation codes in LDS.  A wave owns RPW rows per group; row
// groups are double-buffered (the next group's loads in flight while the
// current one is consumed) and a DPP wave sum finishes each row.  Every
// workgroup copies the activation into LDS first; its loads go out before
// the first weights.
#include <atomic>

#include "lq_device.h"
#include "lq_internal.h"
#include "lq_qk.h"

namespace lq {

namespace {

constexpr int kQkWaves = 8;
constexpr int kQkNT = kQkWaves * 64;
constexpr int kQkMaxCols = 16384;

struct QkArgs {
    QkMat m;
    int rows, cols;
    const int8_t* xq;       // [cols]
    const uint16_t* xd;     // [cols/32]
    const float* res;       // [rows] or NULL (may alias y)
    float* y;               // [rows]
};

// Loads of unit u of a row; dead units and rows read the first bytes of
// row 0 (never used).
template <int FMT>
__device__ __forceinline__ void qk_load(const QkArgs& a, int row, int u, bool live, QkUnit<FMT>& U) {
    qk_load_unit(a.m, a.cols, live ? row : 0, live ? u : 0, U);
}

template <int FMT, int ST, int RPW>
struct QkRows {
    QkUnit<FMT> u[RPW][ST];
};

template <int FMT, int ST, int RPW>
__device__ __forceinline__ void qk_group_load(const QkArgs& a, int64_t grp, int lane, int units,
                                              QkRows<FMT, ST, RPW>& R) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int64_t row = grp * RPW + i;
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int u = st * kWave + lane;
            qk_load(a, (int)row, u, row < a.rows && u < units, R.u[i][st]);
        }
    }
}

template <int FMT, int ST, int RPW>
__device__ __forceinline__ void qk_group_use(const QkArgs& a, int64_t grp, int lane, int units,
                                             const QkRows<FMT, ST, RPW>& R, const int8_t* xl, const float* xs) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int u = st * kWave + lane;
            if (u < units) acc += qk_unit_dot(R.u[i][st], u, xl, xs);
        }
        acc = wave_sum(acc);
        const int64_t row = grp * RPW + i;
        if (lane == 0 && row < a.rows) a.y[row] = a.res ? a.res[row] + acc : acc;
    }
}

template <int FMT, int ST, int RPW>
__global__ __launch_bounds__(kQkNT, 2) void k_qk_mv(QkArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t xl[kQkMaxCols];
    __shared__ float xs[kQkMaxCols / 32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int units = qk_units<FMT>(a.cols);
    const int64_t ngroups = (a.rows + RPW - 1) / RPW;
    const int64_t gstride = (int64_t)gridDim.x * kQkWaves;
    int64_t g = (int64_t)blockIdx.x * kQkWaves + wave;

    // the activation's loads first (16 code bytes and up to one scale per
    // thread and step), then the first row group's weights.  Threads past
    // the activation issue no load: every workgroup reads the activation, and
    // clamped duplicate reads would pile onto one cache line.
    constexpr int XP = kQkMaxCols / 16 / kQkNT;
    int4 xv[XP];
    uint32_t sv[XP];
    const int n16 = a.cols >> 4, nb = a.cols >> 5;
#pragma unroll
    for (int k = 0; k < XP; ++k) {
        const int i = threadIdx.x + kQkNT * k;
        xv[k] = make_int4(0, 0, 0, 0);
        sv[k] = 0;
        if (i < n16) xv[k] = *reinterpret_cast<const int4*>(a.xq + 16 * i);
        if (i < nb) sv[k] = a.xd[i];
    }
    __builtin_amdgcn_sched_barrier(0);
    QkRows<FMT, ST, RPW> A, B;
    qk_group_load<FMT, ST, RPW>(a, g < ngroups ? g : ngroups, lane, units, A);
#pragma unroll
    for (int k = 0; k < XP; ++k) {
        const int i = threadIdx.x + kQkNT * k;
        if (i < n16) *reinterpret_cast<int4*>(xl + 16 * i) = xv[k];
        if (i < nb) xs[i] = f16_to_f32(sv[k]);
    }
    __syncthreads();

    // grid-stride over row groups, the next group's loads issued before the
    // current one is consumed (the last step peeled)
    while (g < ngroups) {
        const int64_t g1 = g + gstride;
        if (g1 >= ngroups) {
            qk_group_use<FMT, ST, RPW>(a, g, lane, units, A, xl, xs);
            break;
        }
        qk_group_load<FMT, ST, RPW>(a, g1, lane, units, B);
        qk_group_use<FMT, ST, RPW>(a, g, lane, units, A, xl, xs);
        const int64_t g2 = g1 + gstride;
        if (g2 >= ngroups) {
            qk_group_use<FMT, ST, RPW>(a, g1, lane, units, B, xl, xs);
            break;
        }
        qk_group_load<FMT, ST, RPW>(a, g2, lane, units, A);
        qk_group_use<FMT, ST, RPW>(a, g1, lane, units, B, xl, xs);
        g = g2;
    }
}

template <int FMT, int ST, int RPW>
void launch_qk(const QkArgs& a, hipStream_t s) {
    // one resident round: workgroups per CU as the occupancy query reports
    // for this instance (1 or 2, by its register count), queried once
    static std::atomic<int> resident_cache{-1};
    int resident = resident_cache.load(std::memory_order_relaxed);
    if (resident < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_qk_mv<FMT, ST, RPW>, kQkNT, 0) != hipSuccess || n < 1)
            n = 1;
        resident = n < 2 ? n : 2;
        resident_cache.store(resident, std::memory_order_relaxed);
    }
    const int64_t groups = (a.rows + RPW - 1) / RPW;
    const int64_t waves = (int64_t)kNumCUs * resident * kQkWaves;
    const int64_t iters = (groups + waves - 1) / waves;
    int64_t grid = (groups + kQkWaves * iters - 1) / (kQkWaves * iters);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((k_qk_mv<FMT, ST, RPW>), dim3((unsigned)grid), dim3(kQkNT), 0, s, a);
}

// steps per row: units / 64 rounded up (Q4_0 up to 8, Q6_K up to 4); two
// rows per wave and group while the double buffer stays small
template <int FMT>
void dispatch_qk(const QkArgs& a, hipStream_t s) {
    const int st = (qk_units<FMT>(a.cols) + kWave - 1) / kWave;
    switch (st) {
        case 1: launch_qk<FMT, 1, 2>(a, s); break;
        case 2: launch_qk<FMT, 2, 2>(a, s); break;
        case 3: launch_qk<FMT, 3, 1>(a, s); break;
        case 4: launch_qk<FMT, 4, 1>(a, s); break;
        default:
            if constexpr (FMT == QK_Q4_0) {       // Q6_K rows of <= 16384 values need at most 4 steps
                switch (st) {
                    case 5: launch_qk<FMT, 5, 1>(a, s); break;
                    case 6: launch_qk<FMT, 6, 1>(a, s); break;
                    case 7: launch_qk<FMT, 7, 1>(a, s); break;
                    default: launch_qk<FMT, 8, 1>(a, s); break;
                }
            }
            break;
    }
}

lq_status qk_check(const char* fn, int64_t rows, int64_t cols, int per, const int8_t* x_qs, const uint16_t* x_d,
                   float* y, const float* residual) {
    if (rows < 0 || cols <= 0 || cols % per)
        return fail(LQ_ERR_SHAPE, "%s: rows=%lld cols=%lld (cols %% %d == 0)", fn, (long long)rows, (long long)cols,
                    per);
    if (cols > kQkMaxCols || rows > 0x7fffffffLL)
        return fail(LQ_ERR_UNSUPPORTED, "%s: cols=%lld > %d", fn, (long long)cols, kQkMaxCols);
    if (rows == 0) return LQ_OK;
    if (!x_qs || !x_d || !y) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x_qs, 16) || !aligned(x_d, 2) || !aligned(y, 4) || (residual && !aligned(residual, 4)))
        return fail(LQ_ERR_ALIGN, "%s: x_qs must be 16-byte aligned", fn);
    return LQ_OK;
}

}  // namespace

}  // namespace lq

using namespace lq;

extern "C" lq_status lq_q4_0_matvec(const lq_q4_0_weight* w, const int8_t* x_qs, const uint16_t* x_d,
                                    const float* residual, float* y, void* stream) {
    const char* fn = "lq_q4_0_matvec";
    if (!w) return fail(LQ_ERR_NULL, "%s: NULL weight", fn);
    lq_status st = qk_check(fn, w->rows, w->cols, 32, x_qs, x_d, y, residual);
    if (st != LQ_OK || w->rows == 0) return st;
    if (!w->qs || !w->d) return fail(LQ_ERR_NULL, "%s: NULL weight array", fn);
    if (!aligned(w->qs, 16) || !aligned(w->d, 2)) return fail(LQ_ERR_ALIGN, "%s: qs must be 16-byte aligned", fn);
    const QkArgs a{QkMat{w->qs, nullptr, nullptr, w->d}, (int)w->rows, (int)w->cols, x_qs, x_d, residual, y};
    dispatch_qk<QK_Q4_0>(a, as_stream(stream));
    return check_launch(fn);
}

extern "C" lq_status lq_q6_k_matvec(const lq_q6_k_weight* w, const int8_t* x_qs, const uint16_t* x_d,
                                    const float* residual, float* y, void* stream) {
    const char* fn = "lq_q6_k_matvec";
    if (!w) return fail(LQ_ERR_NULL, "%s: NULL weight", fn);
    lq_status st = qk_check(fn, w->rows, w->cols, 256, x_qs, x_d, y, residual);
    if (st != LQ_OK || w->rows == 0) return st;
    if (!w->ql || !w->qh || !w->sc || !w->d) return fail(LQ_ERR_NULL, "%s: NULL weight array", fn);
    if (!aligned(w->ql, 16) || !aligned(w->qh, 16) || !aligned(w->sc, 8) || !aligned(w->d, 2))
        return fail(LQ_ERR_ALIGN, "%s: ql and qh must be 16-byte aligned, sc 8-byte aligned", fn);
    const QkArgs a{QkMat{w->ql, w->qh, w->sc, w->d}, (int)w->rows, (int)w->cols, x_qs, x_d, residual, y};
    dispatch_qk<QK_Q6_K>(a, as_stream(stream));
    return check_launch(fn);
}

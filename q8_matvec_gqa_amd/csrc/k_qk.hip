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
constexpr int kQkMaxCols = 16384;
// Waves per workgroup: 8, or 4 for the SwiGLU + Q8_0 epilogue, whose grid is
// one workgroup per 32-output block of h: two 4-wave workgroups fit a CU, so
// the whole grid of the 8B-like gate_up (384 blocks) is one resident round.
template <int EPI> constexpr int qk_waves() { return EPI == EPI_SWIGLU_Q8 ? 4 : kQkWaves; }

// Arguments of the fused format matvec; prologue and epilogue kinds are the
// Q8_0 matvec's (PRO_* and EPI_* of lq_internal.h).
struct QkArgs {
    QkMat m;
    int rows, cols;         // output rows (EPI_SWIGLU_Q8: rows of h; the weight has 2*rows), cols <= 16384
    const int8_t* xq;       // PRO_Q8: codes [cols] and f16 scales [cols/32]
    const uint16_t* xd;
    const float* x;         // PRO_QUANT / PRO_NORM: f32 [cols]
    const float* gamma;     // PRO_NORM (NULL: unit weight)
    float eps;
    const float* res;       // EPI_RESID (may alias y)
    float* y;               // EPI_STORE / EPI_RESID; EPI_SWIGLU_Q8: optional f32 h
    int8_t* yq;             // EPI_SWIGLU_Q8: Q8_0 of h, codes [rows] and scales [rows/32]
    uint16_t* yd;
    int8_t* tap_q;          // optional: workgroup 0 writes the Q8_0 input it built
    uint16_t* tap_d;
    int act;                // EPI_SWIGLU_Q8: LQ_ACT_SILU or LQ_ACT_GELU_TANH
};

// Loads of unit u of a row; dead units and rows read the first bytes of
// row 0 (never used).
template <int FMT>
__device__ __forceinline__ void qk_load(const QkArgs& a, int64_t row, int u, bool live, QkUnit<FMT>& U) {
    qk_load_unit(a.m, a.cols, live ? row : 0, live ? u : 0, U);
}

template <int FMT, int ST, int RPW>
struct QkRows {
    QkUnit<FMT> u[RPW][ST];
};

// Weight rows of group g: RPW consecutive rows, or for the SwiGLU epilogue
// the pair (gate row g, up row g + rows).
template <int EPI, int RPW>
__device__ __forceinline__ int64_t qk_row(const QkArgs& a, int64_t g, int i) {
    if constexpr (EPI == EPI_SWIGLU_Q8) return g + (i & 1) * (int64_t)a.rows;
    return g * RPW + i;
}
template <int EPI, int RPW>
__device__ __forceinline__ bool qk_live(const QkArgs& a, int64_t g, int i) {
    if constexpr (EPI == EPI_SWIGLU_Q8) return g < a.rows;
    return g * RPW + i < a.rows;
}

template <int FMT, int ST, int RPW, int EPI>
__device__ __forceinline__ void qk_group_load(const QkArgs& a, int64_t grp, bool glive, int lane, int units,
                                              QkRows<FMT, ST, RPW>& R) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const bool rl = glive && qk_live<EPI, RPW>(a, grp, i);
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int u = st * kWave + lane;
            qk_load(a, qk_row<EPI, RPW>(a, grp, i), u, rl && u < units, R.u[i][st]);
        }
    }
}

// SwiGLU gate (silu) or GeGLU gate (tanh form of GELU), as the Q8_0 matvec.
__device__ __forceinline__ float qk_gate(float z, int act) {
    if (act == LQ_ACT_GELU_TANH) return 0.5f * z * (1.0f + tanhf(0.7978845608028654f * (z + 0.044715f * z * z * z)));
    return z / (1.0f + expf(-z));
}

template <int FMT, int ST, int RPW, int EPI>
__device__ __forceinline__ void qk_group_use(const QkArgs& a, int64_t grp, int lane, int units,
                                             const QkRows<FMT, ST, RPW>& R, const int8_t* xl, const float* xs,
                                             float* hs) {
    float acc[RPW];
    // each unit's activation read from LDS once for the RPW rows, where the
    // registers allow (the widest rows read it per row)
    constexpr bool HOLD = FMT == QK_Q4_0 ? ST <= 4 : ST <= 2;
    if constexpr (HOLD) {
        QkAct<FMT> A[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int u = st * kWave + lane;
            qk_load_act_l(xl, xs, u < units ? u : 0, A[st]);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float t = 0.0f;
#pragma unroll
            for (int st = 0; st < ST; ++st) {
                const int u = st * kWave + lane;
                if (u < units) t += qk_unit_dot_a(R.u[i][st], u, A[st]);
            }
            acc[i] = wave_sum(t);
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float t = 0.0f;
#pragma unroll
            for (int st = 0; st < ST; ++st) {
                const int u = st * kWave + lane;
                if (u < units) t += qk_unit_dot(R.u[i][st], u, xl, xs);
            }
            acc[i] = wave_sum(t);
        }
    }
    if (lane != 0) return;
    if constexpr (EPI == EPI_SWIGLU_Q8) {
        if (grp < a.rows) {
            const float h = qk_gate(acc[0], a.act) * acc[1];
            hs[grp & 31] = h;                    // the workgroup's 32-value block, quantized at the end
            if (a.y) a.y[grp] = h;
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t row = grp * RPW + i;
            if (row < a.rows) a.y[row] = (EPI == EPI_RESID) ? a.res[row] + acc[i] : acc[i];
        }
    }
}

// Float prologue: quarter blocks (8 values) per thread, the four lanes of a
// quad holding one 32-value block.  QPT quarter blocks per thread at most.
template <int ST, int FMT, int NT> struct QkPro {
    static constexpr int MAXC = FMT == QK_Q4_0 ? ST * 2048 : ST * 4096;          // columns an ST covers
    static constexpr int QPT = ((MAXC < kQkMaxCols ? MAXC : kQkMaxCols) / 8 + NT - 1) / NT;
};
// VGPRs the weight double buffer takes: the norm weights are loaded with
// the input (ahead of the first weights) only while both fit beside it in
// the 256 VGPRs of two waves per SIMD.
template <int FMT, int ST, int RPW, int PRO, int NT> struct QkOcc {
    static constexpr int UNIT = FMT == QK_Q4_0 ? 5 : 15;
    static constexpr int BUF = 2 * RPW * ST * UNIT;
    static constexpr int XREGS = PRO == PRO_Q8 ? 0 : 8 * QkPro<ST, FMT, NT>::QPT;
    static constexpr bool EARLY_G = PRO == PRO_NORM && BUF + 2 * XREGS <= 160;
};

template <int FMT, int ST, int RPW, int PRO, int EPI>
// Arguments one by one, the ones the first loads need leading, so the
// compiler preloads them into SGPRs at dispatch.
__global__ __launch_bounds__(qk_waves<EPI>() * 64, 2) void k_qk_mv(
    const float* p_x, const float* p_gamma, const int8_t* p_xq, const uint16_t* p_xd, const uint8_t* p_q0,
    const uint8_t* p_q1, const int8_t* p_sc, const uint16_t* p_d, int p_rows, int p_cols, float p_eps,
    const float* p_res, float* p_y, int8_t* p_yq, uint16_t* p_yd, int8_t* p_tap_q, uint16_t* p_tap_d, int p_act) {
    const QkArgs a{QkMat{p_q0, p_q1, p_sc, p_d}, p_rows, p_cols, p_xq, p_xd, p_x, p_gamma, p_eps, p_res, p_y, p_yq,
                   p_yd, p_tap_q, p_tap_d, p_act};
    static_assert(EPI != EPI_SWIGLU_Q8 || RPW == 2, "SwiGLU groups are (gate, up) row pairs");
    constexpr int kQkW = qk_waves<EPI>(), kQkNT = kQkW * 64;
    __shared__ __attribute__((aligned(16))) int8_t xl[kQkMaxCols];
    __shared__ float xs[kQkMaxCols / 32];
    __shared__ float red[kQkW];
    __shared__ float hs[EPI == EPI_SWIGLU_Q8 ? 32 : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int units = qk_units<FMT>(a.cols);
    // groups: grid-stride over row groups, or for the SwiGLU epilogue the
    // workgroup's 32 outputs, four per wave
    constexpr bool SW = EPI == EPI_SWIGLU_Q8;
    constexpr int OPW = 32 / kQkW;
    const int64_t ngroups = SW ? a.rows : (a.rows + RPW - 1) / RPW;
    const int64_t gstride = SW ? 1 : (int64_t)gridDim.x * kQkW;
    int64_t g = SW ? (int64_t)blockIdx.x * 32 + wave * OPW : (int64_t)blockIdx.x * kQkW + wave;
    const int64_t gend = SW ? (g + OPW < ngroups ? g + OPW : ngroups) : ngroups;
    const int n16 = a.cols >> 4, nb = a.cols >> 5;
    QkRows<FMT, ST, RPW> A, B;

    if constexpr (PRO == PRO_Q8) {
        // the activation's loads first (16 code bytes and up to one scale per
        // thread and step), then the first row group's weights.  Threads past
        // the activation issue no load: every workgroup reads the activation,
        // and clamped duplicate reads would pile onto one cache line.
        constexpr int XP = kQkMaxCols / 16 / kQkNT;
        int4 xv[XP];
        uint32_t sv[XP];
#pragma unroll
        for (int k = 0; k < XP; ++k) {
            const int i = threadIdx.x + kQkNT * k;
            xv[k] = make_int4(0, 0, 0, 0);
            sv[k] = 0;
            if (i < n16) xv[k] = *reinterpret_cast<const int4*>(a.xq + 16 * i);
            if (i < nb) sv[k] = a.xd[i];
        }
        __builtin_amdgcn_sched_barrier(0);
        qk_group_load<FMT, ST, RPW, EPI>(a, g, g < gend, lane, units, A);
#pragma unroll
        for (int k = 0; k < XP; ++k) {
            const int i = threadIdx.x + kQkNT * k;
            if (i < n16) *reinterpret_cast<int4*>(xl + 16 * i) = xv[k];
            if (i < nb) xs[i] = f16_to_f32(sv[k]);
        }
    } else {
        // f32 input (and the norm weights when the registers allow) first,
        // then the first weights; then RMSNorm (PRO_NORM) and the Q8_0 of the
        // input into LDS, the same rule as every quantizer here
        constexpr int QPT = QkPro<ST, FMT, kQkNT>::QPT;
        constexpr bool EARLY_G = QkOcc<FMT, ST, RPW, PRO, kQkNT>::EARLY_G;
        const int nqb = a.cols >> 3;
        float xf[QPT][8], gf[EARLY_G ? QPT : 1][8];
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int qb = threadIdx.x + kQkNT * k;
            const int qc = qb < nqb ? qb : 0;        // a valid address; the values are dropped below
            if (k * kQkNT < nqb) {
                load8(a.x + 8 * qc, xf[k]);
                if constexpr (EARLY_G) load8((a.gamma ? a.gamma : a.x) + 8 * qc, gf[k]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        qk_group_load<FMT, ST, RPW, EPI>(a, g, g < gend, lane, units, A);
#pragma unroll
        for (int k = 0; k < QPT; ++k)
            if (k * kQkNT >= nqb || threadIdx.x + kQkNT * k >= nqb)
#pragma unroll
                for (int i = 0; i < 8; ++i) xf[k][i] = 0.0f;
        float rinv = 1.0f;
        if constexpr (PRO == PRO_NORM) {
            float ss = 0.0f;
#pragma unroll
            for (int k = 0; k < QPT; ++k)
#pragma unroll
                for (int i = 0; i < 8; ++i) ss += xf[k][i] * xf[k][i];
            ss = wave_sum(ss);
            if (lane == 0) red[wave] = ss;
            __syncthreads();
            ss = 0.0f;
#pragma unroll
            for (int w = 0; w < kQkW; ++w) ss += red[w];
            rinv = 1.0f / sqrtf(ss / (float)a.cols + a.eps);
        }
        const bool tap = a.tap_q != nullptr && blockIdx.x == 0;
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int qb = threadIdx.x + kQkNT * k;
            if (k * kQkNT < nqb) {                   // whole quads are in or out together (nqb % 4 == 0)
                float v[8];
                if constexpr (PRO == PRO_NORM) {
                    float gm[8];
                    if (a.gamma) {
                        if constexpr (EARLY_G) {
#pragma unroll
                            for (int i = 0; i < 8; ++i) gm[i] = gf[k][i];
                        } else {
                            load8(a.gamma + 8 * (qb < nqb ? qb : 0), gm);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) gm[i] = 1.0f;
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = a.gamma ? (xf[k][i] * rinv) * gm[i] : xf[k][i] * rinv;
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = xf[k][i];
                }
                uint32_t packed[2];
                const uint16_t db = quantize_quarter8_packed(v, packed);
                if (qb < nqb) {
                    *reinterpret_cast<uint2*>(xl + 8 * qb) = make_uint2(packed[0], packed[1]);
                    if ((qb & 3) == 0) xs[qb >> 2] = f16_to_f32(db);
                    if (tap) {
                        *reinterpret_cast<uint2*>(a.tap_q + 8 * qb) = make_uint2(packed[0], packed[1]);
                        if ((qb & 3) == 0) a.tap_d[qb >> 2] = db;
                    }
                }
            }
        }
    }
    __syncthreads();

    // the next group's loads issued before the current one is consumed (the
    // last step peeled)
    while (g < gend) {
        const int64_t g1 = g + gstride;
        if (g1 >= gend) {
            qk_group_use<FMT, ST, RPW, EPI>(a, g, lane, units, A, xl, xs, hs);
            break;
        }
        qk_group_load<FMT, ST, RPW, EPI>(a, g1, true, lane, units, B);
        qk_group_use<FMT, ST, RPW, EPI>(a, g, lane, units, A, xl, xs, hs);
        const int64_t g2 = g1 + gstride;
        if (g2 >= gend) {
            qk_group_use<FMT, ST, RPW, EPI>(a, g1, lane, units, B, xl, xs, hs);
            break;
        }
        qk_group_load<FMT, ST, RPW, EPI>(a, g2, true, lane, units, A);
        qk_group_use<FMT, ST, RPW, EPI>(a, g1, lane, units, B, xl, xs, hs);
        g = g2;
    }

    if constexpr (SW) {
        // Q8_0 of the workgroup's 32 outputs: lane i of wave 0 holds value i
        __syncthreads();
        const int64_t b = blockIdx.x;
        if (wave == 0) {
            const bool mine = lane < 32 && 32 * b + lane < a.rows;
            const float v = mine ? hs[lane & 31] : 0.0f;
            const float amax = group_max<32>(fabsf(v));
            const float d = amax / 127.0f;
            const float inv = (d != 0.0f) ? 1.0f / d : 0.0f;
            const float r = fminf(fmaxf(roundf(v * inv), -127.0f), 127.0f);
            if (mine) a.yq[32 * b + lane] = (int8_t)(int32_t)r;
            if (lane == 0) a.yd[b] = f32_to_f16(d);
        }
    }
}

template <int FMT, int ST, int RPW, int PRO, int EPI>
void launch_qk(const QkArgs& a, hipStream_t s, LaunchMarks* mk) {
    auto kern = k_qk_mv<FMT, ST, RPW, PRO, EPI>;
    constexpr int kQkNT = qk_waves<EPI>() * 64;
    int64_t grid;
    if constexpr (EPI == EPI_SWIGLU_Q8) {
        grid = (a.rows + 31) / 32;                   // one workgroup per 32-output block of h
    } else {
        // one resident round: workgroups per CU as the occupancy query reports
        // for this instance (1 or 2, by its register count), queried once
        static std::atomic<int> resident_cache{-1};
        int resident = resident_cache.load(std::memory_order_relaxed);
        if (resident < 0) {
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kQkNT, 0) != hipSuccess || n < 1) n = 1;
            resident = n < 2 ? n : 2;
            resident_cache.store(resident, std::memory_order_relaxed);
        }
        const int64_t groups = (a.rows + RPW - 1) / RPW;
        const int64_t waves = (int64_t)kNumCUs * resident * kQkWaves;
        const int64_t iters = (groups + waves - 1) / waves;
        grid = (groups + kQkWaves * iters - 1) / (kQkWaves * iters);
    }
    if (grid < 1) grid = 1;
    launch_marked(mk, kern, dim3((unsigned)grid), dim3(kQkNT), 0, s, a.x, a.gamma, a.xq, a.xd, a.m.q0, a.m.q1, a.m.sc,
                  a.m.d, a.rows, a.cols, a.eps, a.res, a.y, a.yq, a.yd, a.tap_q, a.tap_d, a.act);
}

// steps per row: units / 64 rounded up (Q4_0 up to 8, Q6_K up to 4); two
// rows per wave and group while the double buffer stays small
template <int FMT, int PRO, int EPI>
bool dispatch_qk(const QkArgs& a, hipStream_t s, LaunchMarks* mk) {
    const int st = (qk_units<FMT>(a.cols) + kWave - 1) / kWave;
    constexpr bool SW = EPI == EPI_SWIGLU_Q8;
    if (SW && FMT == QK_Q6_K && st > 3) return false;
    switch (st) {
        case 1: launch_qk<FMT, 1, 2, PRO, EPI>(a, s, mk); break;
        case 2: launch_qk<FMT, 2, 2, PRO, EPI>(a, s, mk); break;
        case 3: launch_qk<FMT, 3, SW ? 2 : 1, PRO, EPI>(a, s, mk); break;
        case 4:
            // Q6_K gate/up pairs over 16384 columns would not fit the registers
            // (the decode layer refuses hidden > 12288 for a Q6_K gate_up)
            if constexpr (!(SW && FMT == QK_Q6_K)) launch_qk<FMT, 4, SW ? 2 : 1, PRO, EPI>(a, s, mk);
            break;
        default:
            if constexpr (FMT == QK_Q4_0) {       // Q6_K rows of <= 16384 values need at most 4 steps
                switch (st) {
                    case 5: launch_qk<FMT, 5, SW ? 2 : 1, PRO, EPI>(a, s, mk); break;
                    case 6: launch_qk<FMT, 6, SW ? 2 : 1, PRO, EPI>(a, s, mk); break;
                    case 7: launch_qk<FMT, 7, SW ? 2 : 1, PRO, EPI>(a, s, mk); break;
                    default: launch_qk<FMT, 8, SW ? 2 : 1, PRO, EPI>(a, s, mk); break;
                }
            }
            break;
    }
    return true;
}

template <int FMT>
lq_status dispatch_qk_pe(const QkArgs& a, int pro, int epi, hipStream_t s, LaunchMarks* mk) {
#define LQ_QK_PE(P, E)                                                                        \
    if (pro == P && epi == E) {                                                               \
        if (!dispatch_qk<FMT, P, E>(a, s, mk))                                                \
            return fail(LQ_ERR_UNSUPPORTED, "format matvec: Q6_K gate/up pairs over %d columns", a.cols); \
        return check_launch("format matvec");                                                 \
    }
    LQ_QK_PE(PRO_Q8, EPI_STORE) LQ_QK_PE(PRO_Q8, EPI_RESID)
    LQ_QK_PE(PRO_QUANT, EPI_STORE) LQ_QK_PE(PRO_QUANT, EPI_RESID)
    LQ_QK_PE(PRO_NORM, EPI_STORE) LQ_QK_PE(PRO_NORM, EPI_SWIGLU_Q8)
#undef LQ_QK_PE
    return fail(LQ_ERR_UNSUPPORTED, "format matvec: prologue %d / epilogue %d not built", pro, epi);
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

lq_status check_proj_weight(const char* fn, const char* what, int32_t fmt, const lq_q8_weight& q8,
                            const lq_q4_0_weight& q4, const lq_q6_k_weight& q6, int64_t rows, int64_t cols,
                            ProjWeight* out) {
    if (fmt == LQ_FMT_Q8_0) {
        if (q8.rows != rows || q8.cols != cols)
            return fail(LQ_ERR_SHAPE, "%s: %s Q8_0 weight is %lld x %lld, need %lld x %lld", fn, what,
                        (long long)q8.rows, (long long)q8.cols, (long long)rows, (long long)cols);
        lq_status st = check_weight(&q8, fn);
        if (st != LQ_OK) return st;
        *out = ProjWeight{LQ_FMT_Q8_0, q8.qs, nullptr, nullptr, q8.d};
        return LQ_OK;
    }
    if (fmt == LQ_FMT_Q4_0) {
        if (q4.rows != rows || q4.cols != cols || cols % 32)
            return fail(LQ_ERR_SHAPE, "%s: %s Q4_0 weight is %lld x %lld, need %lld x %lld (cols %% 32 == 0)", fn,
                        what, (long long)q4.rows, (long long)q4.cols, (long long)rows, (long long)cols);
        if (!q4.qs || !q4.d) return fail(LQ_ERR_NULL, "%s: %s: NULL weight array", fn, what);
        if (!aligned(q4.qs, 16) || !aligned(q4.d, 2))
            return fail(LQ_ERR_ALIGN, "%s: %s: qs must be 16-byte aligned", fn, what);
        *out = ProjWeight{LQ_FMT_Q4_0, q4.qs, nullptr, nullptr, q4.d};
        return LQ_OK;
    }
    if (fmt == LQ_FMT_Q6_K) {
        if (q6.rows != rows || q6.cols != cols || cols % 256)
            return fail(LQ_ERR_SHAPE, "%s: %s Q6_K weight is %lld x %lld, need %lld x %lld (cols %% 256 == 0)", fn,
                        what, (long long)q6.rows, (long long)q6.cols, (long long)rows, (long long)cols);
        if (!q6.ql || !q6.qh || !q6.sc || !q6.d) return fail(LQ_ERR_NULL, "%s: %s: NULL weight array", fn, what);
        if (!aligned(q6.ql, 16) || !aligned(q6.qh, 16) || !aligned(q6.sc, 8) || !aligned(q6.d, 2))
            return fail(LQ_ERR_ALIGN, "%s: %s: ql and qh must be 16-byte aligned, sc 8-byte aligned", fn, what);
        *out = ProjWeight{LQ_FMT_Q6_K, q6.ql, q6.qh, q6.sc, q6.d};
        return LQ_OK;
    }
    return fail(LQ_ERR_SHAPE, "%s: %s format %d (LQ_FMT_Q8_0, LQ_FMT_Q4_0 or LQ_FMT_Q6_K)", fn, what, (int)fmt);
}

lq_status launch_proj(const ProjWeight& w, const MvArgs& m, int pro, int epi, hipStream_t s, LaunchMarks* mk) {
    if (w.fmt == LQ_FMT_Q8_0) {
        MvArgs a = m;
        a.wq = static_cast<const int8_t*>(w.q0);
        a.wd = w.d;
        return launch_mv(a, pro, epi, s, kMvWgPerCu, mk);
    }
    if (m.rows == 0) return LQ_OK;
    QkArgs a{};
    a.m = QkMat{static_cast<const uint8_t*>(w.q0), static_cast<const uint8_t*>(w.q1), w.sc, w.d};
    a.rows = m.rows; a.cols = m.cols; a.xq = m.xq; a.xd = m.xd; a.x = m.x; a.gamma = m.gamma; a.eps = m.eps;
    a.res = m.res; a.y = m.y; a.yq = m.yq; a.yd = m.yd; a.tap_q = m.tap_q; a.tap_d = m.tap_d; a.act = m.act;
    if (w.fmt == LQ_FMT_Q4_0) return dispatch_qk_pe<QK_Q4_0>(a, pro, epi, s, mk);
    if (w.fmt == LQ_FMT_Q6_K) return dispatch_qk_pe<QK_Q6_K>(a, pro, epi, s, mk);
    return fail(LQ_ERR_SHAPE, "weight format %d", w.fmt);
}

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
    QkArgs a{};
    a.m = QkMat{w->qs, nullptr, nullptr, w->d};
    a.rows = (int)w->rows; a.cols = (int)w->cols; a.xq = x_qs; a.xd = x_d; a.res = residual; a.y = y;
    return dispatch_qk_pe<QK_Q4_0>(a, PRO_Q8, residual ? EPI_RESID : EPI_STORE, as_stream(stream), nullptr);
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
    QkArgs a{};
    a.m = QkMat{w->ql, w->qh, w->sc, w->d};
    a.rows = (int)w->rows; a.cols = (int)w->cols; a.xq = x_qs; a.xd = x_d; a.res = residual; a.y = y;
    return dispatch_qk_pe<QK_Q6_K>(a, PRO_Q8, residual ? EPI_RESID : EPI_STORE, as_stream(stream), nullptr);
}

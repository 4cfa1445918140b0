// k_matvec.hip -- Q8_0 matvec for gfx950.
//
// What it computes ("Design: lattice-inference", Current Design, CPU
// fallback and NEON: int8 x int8 products summed into int32 per block, then
// scaled): for each row r and 32-column block b
//     dot[r,b] = sum_i qs_w[r, 32b+i] * qs_x[32b+i]          (int32, exact)
//     y[r]     = (residual[r]) + sum_b f16(d_w[r,b]) * f16(d_x[b]) * dot[r,b]
//
// Mapping onto CDNA4:
//   * A row is cut into 1 KB chunks.  In each chunk, lane l of a wave owns
//     bytes [16l, 16l+16): one global_load_dwordx4 per lane, so a wave reads
//     1 KB contiguous per instruction (fully coalesced).  Lanes 2j and 2j+1
//     hold the two halves of block j of the chunk.
//   * The matching 16 activation codes and the activation scale of that
//     block are the same for every row, so each lane loads its K-slice of the
//     quantized activation once into VGPRs and reuses it for every row it
//     processes: no LDS traffic in the inner loop.
//   * 4 x v_dot4_i32_i8 give the int32 half-block sum; one DPP quad_perm add
//     with the neighbour lane gives the exact int32 block dot in both lanes.
//     The block dot (|dot| <= 2^19) and the product of the two f16 scales are
//     exact in f32; even lanes accumulate dot * (d_w * d_x).
//   * A wave keeps RPW rows of loads in flight, then reduces each row with a
//     DPP / permlane wave sum.  The grid is sized so every CU gets many waves.
#include <atomic>

#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

__device__ __forceinline__ int dot16(int4 a, int4 b) {
    int p = __builtin_amdgcn_sdot4(a.x, b.x, 0, false);
    p = __builtin_amdgcn_sdot4(a.y, b.y, p, false);
    p = __builtin_amdgcn_sdot4(a.z, b.z, p, false);
    p = __builtin_amdgcn_sdot4(a.w, b.w, p, false);
    return p;
}

// NCH: number of 1 KB chunks per row (cols <= 1024*NCH).  RPW: rows a wave
// loads before consuming them.  DOTS: write every int32 block dot instead of
// y (the block-dot test tap; scales are not read).
template <int NCH, int RPW, bool DOTS>
__global__ __launch_bounds__(256) void k_q8_matvec(const int8_t* __restrict__ wq,
                                                   const uint16_t* __restrict__ wd, int64_t rows,
                                                   int cols, const int8_t* __restrict__ xq,
                                                   const uint16_t* __restrict__ xd,
                                                   const float* res, float* y,
                                                   int32_t* __restrict__ dots) {
    const int lane = threadIdx.x & 63;
    const int nb = cols >> 5;
    int4 xv[NCH];
    float xs[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int off = c * 1024 + lane * 16;
        if (off < cols) {
            xv[c] = *reinterpret_cast<const int4*>(xq + off);
            xs[c] = DOTS ? 0.0f : f16_to_f32(xd[off >> 5]);
        } else {
            xv[c] = make_int4(0, 0, 0, 0);
            xs[c] = 0.0f;
        }
    }
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * 4;
    for (int64_t r0 = gw * RPW; r0 < rows; r0 += nw * RPW) {
        int4 wv[RPW][NCH];
        uint32_t ws[RPW][NCH];
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t r = r0 + i;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int off = c * 1024 + lane * 16;
                if (r < rows && off < cols) {
                    wv[i][c] = load_stream16(wq + r * cols + off);
                    ws[i][c] = DOTS ? 0u : (uint32_t)wd[r * nb + (off >> 5)];
                } else {
                    wv[i][c] = make_int4(0, 0, 0, 0);
                    ws[i][c] = 0;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t r = r0 + i;
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int p = dot16(wv[i][c], xv[c]);
                const int blk = p + dpp_i<kQuadXor1>(p);
                const float t = (float)blk * (f16_to_f32(ws[i][c]) * xs[c]);
                acc += (lane & 1) ? 0.0f : t;
                if constexpr (DOTS) {
                    const int off = c * 1024 + lane * 16;
                    if (!(lane & 1) && r < rows && off < cols) dots[r * nb + (off >> 5)] = blk;
                }
            }
            if constexpr (!DOTS) {
                acc = wave_sum(acc);
                if (lane == 0 && r < rows) y[r] = res ? res[r] + acc : acc;
            }
        }
    }
}

// Any cols (multiple of 32): the activation slice is re-read per chunk.
template <bool DOTS>
__global__ __launch_bounds__(256) void k_q8_matvec_any(const int8_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ wd, int64_t rows,
                                                       int cols, const int8_t* __restrict__ xq,
                                                       const uint16_t* __restrict__ xd,
                                                       const float* res, float* y,
                                                       int32_t* __restrict__ dots) {
    const int lane = threadIdx.x & 63;
    const int nb = cols >> 5;
    const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * 4;
    for (int64_t r = gw; r < rows; r += nw) {
        float acc = 0.0f;
        for (int base = 0; base < cols; base += 1024) {
            const int off = base + lane * 16;
            int4 w4 = make_int4(0, 0, 0, 0), x4 = make_int4(0, 0, 0, 0);
            float sc = 0.0f;
            if (off < cols) {
                w4 = *reinterpret_cast<const int4*>(wq + r * cols + off);
                x4 = *reinterpret_cast<const int4*>(xq + off);
                if constexpr (!DOTS) sc = f16_to_f32(wd[r * nb + (off >> 5)]) * f16_to_f32(xd[off >> 5]);
            }
            const int p = dot16(w4, x4);
            const int blk = p + dpp_i<kQuadXor1>(p);
            acc += (lane & 1) ? 0.0f : (float)blk * sc;
            if constexpr (DOTS) {
                if (!(lane & 1) && off < cols) dots[r * nb + (off >> 5)] = blk;
            }
        }
        if constexpr (!DOTS) {
            acc = wave_sum(acc);
            if (lane == 0) y[r] = res ? res[r] + acc : acc;
        }
    }
}

// ---------------------------------------------------------------------------
// Fused matvec: prologue x -> Q8_0 in LDS, grid-stride rows with prefetch,
// epilogue store / residual / SwiGLU.
//
// Prologues (PRO_*): the workgroup builds the quantized activation itself,
//   Q8    : codes and scales already in memory (copied to LDS);
//   QUANT : f32 x quantized per 32-block into LDS;
//   NORM  : f32 x -> RMSNorm(gamma) -> quantized into LDS.
//   Every workgroup computes the same bits, so the layer needs no separate
//   normalise / quantize launches.  The first row group's weight loads are
//   issued before the prologue so HBM latency overlaps it.
// Epilogues (EPI_*): y[r] = acc; y[r] = res[r] + acc; or, with the gate rows
//   [0, rows) and up rows [rows, 2*rows) of a gate_up weight processed in
//   pairs, y[r] = silu(acc_gate) * acc_up.
// Each wave owns a fixed 16-byte K-slice per 1 KB chunk, so its activation
// slice is copied from LDS to VGPRs once and reused for every row.
// ---------------------------------------------------------------------------
// Waves per SIMD each instance is compiled for: two where the weight double
// buffer and the activation slice fit in 256 VGPRs, else one (long rows,
// wide SwiGLU pairs), rather than spilling.
template <int NCH, int EPI> struct MvWpe {
    static constexpr int value = (NCH > 8 || ((EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8) && NCH > 5)) ? 1 : 2;
};
constexpr int kMaxCols = 16384;

template <int NCH, int RPW>
struct RowGroup {
    int4 w[RPW][NCH];
    uint32_t d[RPW][NCH];
};

// Loads are unconditional, from clamped addresses: rows past the end read
// the first 16 bytes of the matrix in every lane (one cache line, never
// stored), and 16-byte slices past the last column reload the row's last
// slice (their activation slice is zero).  No branches sit between the
// loads, so nothing forces an early wait on them.
template <int NCH, int RPW, int EPI>
__device__ __forceinline__ void load_group(const MvArgs& a, int64_t g, int64_t gend, int lane,
                                           RowGroup<NCH, RPW>& G) {
    const int nb = a.cols >> 5;
    const bool glive = g < gend;          // groups from gend on belong to no one here
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        // SwiGLU pairs: even i -> gate row, odd i -> the matching up row
        int64_t r;
        bool live;
        if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8) {
            const int64_t o = g * (RPW / 2) + i / 2;
            live = glive && o < a.rows;
            r = o + (i & 1) * (int64_t)a.rows;
        } else {
            r = g * RPW + i;
            live = glive && r < a.rows;
        }
        if (!live) r = 0;
        const int8_t* wr = a.wq + r * a.cols;
        const uint16_t* dr = a.wd + r * nb;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            int off = c * 1024 + lane * 16;
            if (off >= a.cols) off = a.cols - 16;
            if (!live) off = 0;
            G.w[i][c] = load_stream16(wr + off);
            G.d[i][c] = dr[off >> 5];
        }
    }
}

// The wave's activation slice (16 bytes of codes and the block scale per
// 1 KB chunk): held in VGPRs, or for long rows (XL) read from LDS at each
// use to keep the register budget for the weight double buffer.
template <int NCH, bool XL>
struct XAct {
    int4 v[XL ? 1 : NCH];
    float s[XL ? 1 : NCH];
    const int8_t* q_lds;
    const uint16_t* s_lds;     // f16 bits
    __device__ __forceinline__ void get(int c, int lane, int4& x4, float& xs) const {
        if constexpr (XL) {
            const int off = c * 1024 + lane * 16;
            x4 = *reinterpret_cast<const int4*>(q_lds + off);
            xs = f16_to_f32(s_lds[off >> 5]);
        } else {
            x4 = v[c];
            xs = s[c];
        }
    }
};

// SwiGLU gate silu(z) = z / (1 + exp(-z)), or the GeGLU gate with the tanh
// form of GELU, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
__device__ __forceinline__ float gate_act(float z, int act) {
    if (act == LQ_ACT_GELU_TANH) return 0.5f * z * (1.0f + tanhf(0.7978845608028654f * (z + 0.044715f * z * z * z)));
    return z / (1.0f + expf(-z));
}

template <int NCH, int RPW, int EPI, bool XL>
__device__ __forceinline__ void consume_group(const MvArgs& a, int64_t g, int lane, const RowGroup<NCH, RPW>& G,
                                              const XAct<NCH, XL>& x, float* hs) {
    if constexpr (EPI == EPI_DOTS) {
        // the block dots exactly as the other epilogues form them; the even
        // lane of each block writes it (slices past the last column, whose
        // loads were clamped, and rows past the end write nothing)
        const int nb = a.cols >> 5;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t r = g * RPW + i;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                int4 x4;
                float xsc;
                x.get(c, lane, x4, xsc);
                const int p = dot16(G.w[i][c], x4);
                const int blk = p + dpp_i<kQuadXor1>(p);
                const int off = c * 1024 + lane * 16;
                if (!(lane & 1) && r < a.rows && off < a.cols) a.dots[r * nb + (off >> 5)] = blk;
            }
        }
        return;
    }
    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        float t = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            int4 x4;
            float xsc;
            x.get(c, lane, x4, xsc);
            const int p = dot16(G.w[i][c], x4);
            const int blk = p + dpp_i<kQuadXor1>(p);
            const float v = (float)blk * (f16_to_f32(G.d[i][c]) * xsc);
            t += (lane & 1) ? 0.0f : v;
        }
        acc[i] = wave_sum(t);
    }
    if (lane != 0) return;
    if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8) {
#pragma unroll
        for (int j = 0; j < RPW / 2; ++j) {
            const int64_t r = g * (RPW / 2) + j;
            if (r < a.rows) {
                const float gt = acc[2 * j], up = acc[2 * j + 1];
                const float h = gate_act(gt, a.act) * up;
                if constexpr (EPI == EPI_SWIGLU_Q8) {
                    hs[r & 31] = h;               // the workgroup's 32-value block, quantized at the end
                    if (a.y) a.y[r] = h;
                } else {
                    a.y[r] = h;
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const int64_t r = g * RPW + i;
            if (r < a.rows) a.y[r] = (EPI == EPI_RESID) ? a.res[r] + acc[i] : acc[i];
        }
    }
}

// The arguments come one by one, the ones every wave reads first leading:
// the compiler can then preload them into SGPRs at dispatch instead of each
// wave fetching them from the kernel-argument buffer before its first load.
template <int NCH, int RPW, int PRO, int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64, (MvWpe<NCH, EPI>::value)) void k_mv(
    const float* p_x, const float* p_gamma, const int8_t* p_xq, const uint16_t* p_xd, const int8_t* p_wq,
    const uint16_t* p_wd, int p_rows, int p_cols, float p_eps, const float* p_res, float* p_y, int8_t* p_yq,
    uint16_t* p_yd, int8_t* p_tap_q, uint16_t* p_tap_d, int p_act, int32_t* p_dots) {
    const MvArgs a{p_wq, p_wd, p_rows, p_cols, p_xq, p_xd, p_x, p_gamma, p_eps, p_res, p_y, p_yq, p_yd, p_tap_q,
                   p_tap_d, p_act, p_dots};
    constexpr int NT = WAVES * 64;
    constexpr bool XL = NCH > 8;                          // activation slice from LDS
    constexpr bool LDS_X = (PRO != PRO_Q8) || XL;
    __shared__ __attribute__((aligned(16))) int8_t xq_s[LDS_X ? kMaxCols : 16];
    __shared__ __attribute__((aligned(16))) uint16_t xs_s[LDS_X ? kMaxCols / 32 : 8];
    __shared__ float red[WAVES];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nb = a.cols >> 5;
    constexpr bool SW = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8;
    constexpr int OUT_PER_GROUP = SW ? RPW / 2 : RPW;
    const int64_t ngroups = (a.rows + OUT_PER_GROUP - 1) / OUT_PER_GROUP;
    // Groups of a wave: grid-stride; or, for EPI_SWIGLU_Q8, the workgroup
    // owns one 32-output block and each wave a contiguous slice of it.
    constexpr int BLK_GROUPS = 32 / OUT_PER_GROUP;
    static_assert(EPI != EPI_SWIGLU_Q8 || BLK_GROUPS % WAVES == 0, "block split over the waves");
    const int64_t gstride = EPI == EPI_SWIGLU_Q8 ? 1 : (int64_t)gridDim.x * WAVES;
    int64_t g = EPI == EPI_SWIGLU_Q8 ? (int64_t)blockIdx.x * BLK_GROUPS + wave * (BLK_GROUPS / WAVES)
                                     : (int64_t)blockIdx.x * WAVES + wave;
    const int64_t gend = EPI == EPI_SWIGLU_Q8 ? (g + BLK_GROUPS / WAVES < ngroups ? g + BLK_GROUPS / WAVES : ngroups)
                                              : ngroups;
    __shared__ float hs[EPI == EPI_SWIGLU_Q8 ? 32 : 1];

    // The prologue's own loads (x, and gamma when it fits in registers; or
    // the Q8 activation that goes to LDS) are issued first, then the first
    // row group's weights: loads retire in order, so the prologue can compute
    // while the weights are in flight.
    // A float activation is handled in quarter blocks of 8 values: the four
    // lanes of a quad hold the quarters of one 32-value block.
    constexpr int QPT = (NCH * 128 + NT - 1) / NT;         // quarter blocks per thread
    constexpr bool EARLY_G = (PRO == PRO_NORM) && QPT <= 4;
    const int nqb = 4 * nb;
    float xf[PRO != PRO_Q8 ? QPT : 1][8];
    float gf[EARLY_G ? QPT : 1][8];
    if constexpr (PRO != PRO_Q8) {
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int qb = threadIdx.x + NT * k;
            const int qc = qb < nqb ? qb : 0;             // valid address; values dropped below
            load8(a.x + 8 * qc, xf[k]);
            if constexpr (EARLY_G) load8((a.gamma ? a.gamma : a.x) + 8 * qc, gf[k]);
        }
    } else if constexpr (XL) {
        // codes and scales straight into LDS (global_load_lds: no registers),
        // 16 bytes per lane, whole waves; slices past the end are not loaded
        using gptr = const __attribute__((address_space(1))) void*;
        using lptr = __attribute__((address_space(3))) void*;
        const int nq16 = a.cols >> 4;
        for (int s0 = wave * 64; s0 < nq16; s0 += NT)
            if (s0 + lane < nq16)
                __builtin_amdgcn_global_load_lds((gptr)(a.xq + 16 * (s0 + lane)), (lptr)(xq_s + 16 * s0), 16, 0, 0);
    }
    // XL Q8 scales: early register loads (the 2-byte LDS copy writes one
    // dword per lane), stored to LDS once the weight loads are in flight
    constexpr int SPT = (PRO == PRO_Q8 && XL) ? (NCH * 32 + NT - 1) / NT : 1;
    uint32_t sc_early[SPT];
    if constexpr (PRO == PRO_Q8 && XL) {
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
            const int b = threadIdx.x + NT * k;
            sc_early[k] = EPI == EPI_DOTS ? 0u : a.xd[b < nb ? b : nb - 1];   // the dots use no scales
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    RowGroup<NCH, RPW> A, B;
    load_group<NCH, RPW, EPI>(a, g, gend, lane, A);      // a wave past the end reads one cache line

    XAct<NCH, XL> x;
    x.q_lds = xq_s;
    x.s_lds = xs_s;
    if constexpr (PRO == PRO_Q8 && !XL) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int off = c * 1024 + lane * 16;
            x.v[c] = make_int4(0, 0, 0, 0);
            x.s[c] = 0.0f;
            if (off < a.cols) {
                x.v[c] = *reinterpret_cast<const int4*>(a.xq + off);
                x.s[c] = EPI == EPI_DOTS ? 0.0f : f16_to_f32(a.xd[off >> 5]);
            }
        }
    } else {
        if constexpr (PRO == PRO_Q8) {
            // the LDS copies and scale loads issued above must have landed;
            // they precede the first group's weight loads (RPW*NCH codes +
            // RPW*NCH scales), so waiting until only those are outstanding
            // does not wait for the weights
            constexpr int WL = 2 * RPW * NCH < 63 ? 2 * RPW * NCH : 63;     // vmcnt holds at most 63
            __builtin_amdgcn_s_waitcnt((WL & 15) | ((WL >> 4) << 14) | (7 << 4) | (15 << 8));
#pragma unroll
            for (int k = 0; k < SPT; ++k) {
                const int b = threadIdx.x + NT * k;
                if (b < nb) xs_s[b] = (uint16_t)sc_early[k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < QPT; ++k)
                if (threadIdx.x + NT * k >= nqb)
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
                for (int w = 0; w < WAVES; ++w) ss += red[w];
                rinv = 1.0f / sqrtf(ss / (float)a.cols + a.eps);
            }
            const bool tap = a.tap_q != nullptr && blockIdx.x == 0;
#pragma unroll
            for (int k = 0; k < QPT; ++k) {
                // whole quads are in or out together (nqb is a multiple of 4)
                const int qb = threadIdx.x + NT * k;
                if (k * NT < nqb) {
                    float v[8];
                    if constexpr (PRO == PRO_NORM) {
                        if (a.gamma) {
                            float gm[8];
                            if constexpr (EARLY_G) {
#pragma unroll
                                for (int i = 0; i < 8; ++i) gm[i] = gf[k][i];
                            } else {
                                load8(a.gamma + 8 * (qb < nqb ? qb : 0), gm);
                            }
#pragma unroll
                            for (int i = 0; i < 8; ++i) v[i] = (xf[k][i] * rinv) * gm[i];
                        } else {
#pragma unroll
                            for (int i = 0; i < 8; ++i) v[i] = xf[k][i] * rinv;
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; ++i) v[i] = xf[k][i];
                    }
                    uint32_t packed[2];
                    const uint16_t db = quantize_quarter8_packed(v, packed);
                    if (qb < nqb) {
                        *reinterpret_cast<uint2*>(xq_s + 8 * qb) = make_uint2(packed[0], packed[1]);
                        if ((qb & 3) == 0) xs_s[qb >> 2] = db;
                        if (tap) {
                            *reinterpret_cast<uint2*>(a.tap_q + 8 * qb) = make_uint2(packed[0], packed[1]);
                            if ((qb & 3) == 0) a.tap_d[qb >> 2] = db;
                        }
                    }
                }
            }
        }
        if constexpr (XL) {
            // slices past the last column read as zero
            for (int i = a.cols + 16 * threadIdx.x; i < NCH * 1024; i += 16 * NT)
                *reinterpret_cast<int4*>(xq_s + i) = make_int4(0, 0, 0, 0);
            for (int b = nb + threadIdx.x; b < NCH * 32; b += NT) xs_s[b] = 0;
        }
        __syncthreads();
        if constexpr (!XL) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int off = c * 1024 + lane * 16;
                x.v[c] = make_int4(0, 0, 0, 0);
                x.s[c] = 0.0f;
                if (off < a.cols) {
                    x.v[c] = *reinterpret_cast<const int4*>(xq_s + off);
                    x.s[c] = f16_to_f32(xs_s[off >> 5]);
                }
            }
        }
    }

    // grid-stride over row groups, the next group's loads issued before the
    // current one is consumed.  Every load sits in straight-line code ahead
    // of its consumer (the last step is peeled), so each wait covers exactly
    // the loads it needs.
    while (g < gend) {
        const int64_t g1 = g + gstride;
        if (g1 >= gend) {
            consume_group<NCH, RPW, EPI, XL>(a, g, lane, A, x, hs);
            break;
        }
        load_group<NCH, RPW, EPI>(a, g1, gend, lane, B);
        consume_group<NCH, RPW, EPI, XL>(a, g, lane, A, x, hs);
        const int64_t g2 = g1 + gstride;
        if (g2 >= gend) {
            consume_group<NCH, RPW, EPI, XL>(a, g1, lane, B, x, hs);
            break;
        }
        load_group<NCH, RPW, EPI>(a, g2, gend, lane, A);
        consume_group<NCH, RPW, EPI, XL>(a, g1, lane, B, x, hs);
        g = g2;
    }

    if constexpr (EPI == EPI_SWIGLU_Q8) {
        // Q8_0 of the workgroup's 32 outputs: lane i of wave 0 holds value i
        // (the same rule as every other quantizer here: d = amax/127,
        // codes round-half-away(v * (1/d)) clamped to +-127)
        __syncthreads();
        const int64_t b = blockIdx.x;
        if (wave == 0) {
            const bool mine = lane < 32 && 32 * b + lane < a.rows;
            const float v = mine ? hs[lane & 31] : 0.0f;
            const float amax = group_max<32>(fabsf(v));      // lanes 0-31: the block's amax
            const float d = amax / 127.0f;
            const float inv = (d != 0.0f) ? 1.0f / d : 0.0f;
            const float r = fminf(fmaxf(roundf(v * inv), -127.0f), 127.0f);
            if (mine) a.yq[32 * b + lane] = (int8_t)(int32_t)r;
            if (lane == 0) a.yd[b] = f32_to_f16(d);
        }
    }
}

// Rows per wave and workgroups per CU for each shape class.
template <int NCH> struct MvShape {
    static constexpr int RPW = NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1);
};

// Grid: never more workgroups than can be resident at once (so no wave of
// late workgroups repeats the prologue), and every wave gets the same number
// of row groups (no half-empty tail).
// Waves per workgroup: every workgroup builds the activation in its
// prologue, so wider workgroups repeat that work fewer times; SwiGLU pairs
// and long rows keep 4 (their register budget allows no more).
template <int NCH, int PRO, int EPI> struct MvWaves {
    static constexpr int value = (NCH > 8 || EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8) ? 4 : 8;
};
template <int NCH, int PRO, int EPI, int RPW_OVER = 0, int WAVES_OVER = 0>
static void launch_mv_nch(const MvArgs& a, hipStream_t s, int wg_per_cu, LaunchMarks* mk) {
    constexpr bool SW = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_Q8;
    if constexpr (EPI == EPI_SWIGLU_Q8 && WAVES_OVER == 0 && NCH <= 4) {
        // fewer 32-output blocks of h than CUs (a narrow FFN, or one GPU's
        // share of a wide one): each block's workgroup takes 16 waves with a
        // pair or two of rows each, so the few busy CUs keep more rows in flight
        if ((a.rows + 31) / 32 < kNumCUs) {
            launch_mv_nch<NCH, PRO, EPI, 0, 16>(a, s, wg_per_cu, mk);
            return;
        }
    }
    if constexpr (RPW_OVER == 0 && !SW && NCH <= 4) {
        // Short rows and few of them: the default groups (4 rows for rows of
        // at most 2 KB, 2 rows up to 4 KB) would put workgroups on only part
        // of the CUs, or give the waves unequal counts.  With at most three
        // rows per 8-wave workgroup slot of every CU, take that many rows
        // per group instead: one group per wave, every CU busy.
        const int64_t waves = (int64_t)kNumCUs * 8;
        if (a.rows <= waves) {
            launch_mv_nch<NCH, PRO, EPI, 1>(a, s, wg_per_cu, mk);
            return;
        }
        if (a.rows <= 2 * waves && MvShape<NCH>::RPW != 2) {
            launch_mv_nch<NCH, PRO, EPI, 2>(a, s, wg_per_cu, mk);
            return;
        }
        if (a.rows > 2 * waves && a.rows <= 3 * waves) {
            launch_mv_nch<NCH, PRO, EPI, 3>(a, s, wg_per_cu, mk);
            return;
        }
    }
    constexpr int RPW = RPW_OVER ? RPW_OVER
                        : SW ? 2 * (MvShape<NCH>::RPW > 1 ? MvShape<NCH>::RPW / 2 : 1) : MvShape<NCH>::RPW;
    constexpr int OUT = SW ? RPW / 2 : RPW;
    constexpr int WAVES = WAVES_OVER ? WAVES_OVER : MvWaves<NCH, PRO, EPI>::value;
    auto kern = k_mv<NCH, RPW, PRO, EPI, WAVES>;
    // workgroups per CU this instance can keep resident (queried once; the
    // value is the same for every caller, so concurrent first calls agree)
    static std::atomic<int> resident_cache{-1};
    int resident = resident_cache.load(std::memory_order_relaxed);
    if (resident < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, WAVES * 64, 0) != hipSuccess || n < 1) n = 1;
        resident = n;
        resident_cache.store(n, std::memory_order_relaxed);
    }
    const int cap_wg = wg_per_cu * 4 / WAVES > 0 ? wg_per_cu * 4 / WAVES : 1;
    const int per_cu = resident < cap_wg ? resident : cap_wg;
    const int64_t groups = (a.rows + OUT - 1) / OUT;
    const int64_t cap_waves = (int64_t)WAVES * kNumCUs * per_cu;
    const int64_t iters = (groups + cap_waves - 1) / cap_waves;
    int64_t grid = (groups + WAVES * iters - 1) / (WAVES * iters);
    if (EPI == EPI_SWIGLU_Q8) grid = (a.rows + 31) / 32;        // one workgroup per 32-output block
    if (grid < 1) grid = 1;
    launch_marked(mk, kern, dim3((unsigned)grid), dim3(WAVES * 64), 0, s, a.x, a.gamma, a.xq, a.xd, a.wq, a.wd,
                  a.rows, a.cols, a.eps, a.res, a.y, a.yq, a.yd, a.tap_q, a.tap_d, a.act, a.dots);
}

template <int PRO, int EPI>
static lq_status launch_mv_pe(const MvArgs& a, hipStream_t s, int wg_per_cu, LaunchMarks* mk) {
    const int nch = (a.cols + 1023) / 1024;
#define LQ_MV2(N) \
    case N: launch_mv_nch<N, PRO, EPI>(a, s, wg_per_cu, mk); break;
    switch (nch) {
        LQ_MV2(1) LQ_MV2(2) LQ_MV2(3) LQ_MV2(4) LQ_MV2(5) LQ_MV2(6) LQ_MV2(7) LQ_MV2(8)
        LQ_MV2(9) LQ_MV2(10) LQ_MV2(11) LQ_MV2(12) LQ_MV2(13) LQ_MV2(14) LQ_MV2(15) LQ_MV2(16)
        default: return fail(LQ_ERR_UNSUPPORTED, "fused matvec: cols > %d", kMaxCols);
    }
#undef LQ_MV2
    return check_launch("fused matvec");
}

lq_status launch_mv(const MvArgs& a, int pro, int epi, hipStream_t s, int wg_per_cu, LaunchMarks* mk) {
    if (a.rows == 0) return LQ_OK;
#define LQ_PE(P, E) \
    if (pro == P && epi == E) return launch_mv_pe<P, E>(a, s, wg_per_cu, mk);
    LQ_PE(PRO_Q8, EPI_STORE) LQ_PE(PRO_Q8, EPI_RESID)
    LQ_PE(PRO_QUANT, EPI_STORE) LQ_PE(PRO_QUANT, EPI_RESID)
    LQ_PE(PRO_NORM, EPI_STORE) LQ_PE(PRO_NORM, EPI_SWIGLU_Q8)
    LQ_PE(PRO_Q8, EPI_DOTS) LQ_PE(PRO_QUANT, EPI_DOTS) LQ_PE(PRO_NORM, EPI_DOTS)
#undef LQ_PE
    return fail(LQ_ERR_UNSUPPORTED, "fused matvec: prologue %d / epilogue %d not built", pro, epi);
}

template <int NCH, bool DOTS>
static void launch_nch(int grid, hipStream_t s, const int8_t* wq, const uint16_t* wd, int64_t rows,
                       int cols, const int8_t* xq, const uint16_t* xd, const float* res, float* y,
                       int32_t* dots) {
    constexpr int RPW = NCH <= 4 ? 4 : (NCH <= 8 ? 2 : 1);
    hipLaunchKernelGGL((k_q8_matvec<NCH, RPW, DOTS>), dim3(grid), dim3(256), 0, s, wq, wd, rows, cols,
                       xq, xd, res, y, dots);
}

static int rows_per_wave(int nch) { return nch <= 4 ? 4 : (nch <= 8 ? 2 : 1); }

template <bool DOTS>
static void dispatch(hipStream_t s, const int8_t* wq, const uint16_t* wd, int64_t rows, int cols,
                     const int8_t* xq, const uint16_t* xd, const float* res, float* y,
                     int32_t* dots) {
    const int nch = (cols + 1023) / 1024;
    const int rpw = nch <= 16 ? rows_per_wave(nch) : 1;
    int64_t waves = (rows + rpw - 1) / rpw;
    int64_t grid = (waves + 3) / 4;
    if (grid > (1 << 20)) grid = 1 << 20;
    const int g = (int)grid;
#define LQ_MV_CASE(N) \
    case N: launch_nch<N, DOTS>(g, s, wq, wd, rows, cols, xq, xd, res, y, dots); break;
    switch (nch) {
        LQ_MV_CASE(1) LQ_MV_CASE(2) LQ_MV_CASE(3) LQ_MV_CASE(4)
        LQ_MV_CASE(5) LQ_MV_CASE(6) LQ_MV_CASE(7) LQ_MV_CASE(8)
        LQ_MV_CASE(9) LQ_MV_CASE(10) LQ_MV_CASE(11) LQ_MV_CASE(12)
        LQ_MV_CASE(13) LQ_MV_CASE(14) LQ_MV_CASE(15) LQ_MV_CASE(16)
        default:
            hipLaunchKernelGGL((k_q8_matvec_any<DOTS>), dim3(g), dim3(256), 0, s, wq, wd, rows, cols, xq,
                               xd, res, y, dots);
    }
#undef LQ_MV_CASE
}

lq_status launch_q8_matvec(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                           const int8_t* xq, const uint16_t* xd, const float* residual, float* y,
                           int32_t* dots, hipStream_t s) {
    if (rows == 0) return LQ_OK;
    if (dots)
        dispatch<true>(s, wq, wd, rows, (int)cols, xq, xd, residual, y, dots);
    else
        dispatch<false>(s, wq, wd, rows, (int)cols, xq, xd, residual, y, dots);
    return check_launch("q8_matvec");
}

static lq_status check_act(const char* fn, const lq_q8_weight* w, const int8_t* x_qs,
                           const uint16_t* x_d) {
    lq_status st = check_weight(w, fn);
    if (st != LQ_OK) return st;
    if (w->rows == 0) return LQ_OK;
    if (w->cols > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "%s: cols too large", fn);
    if (!x_qs || !x_d) return fail(LQ_ERR_NULL, "%s: activation is NULL", fn);
    if (!aligned(x_qs, 16) || !aligned(x_d, 2))
        return fail(LQ_ERR_ALIGN, "%s: x_qs must be 16-byte aligned", fn);
    return LQ_OK;
}

}  // namespace lq

using namespace lq;

extern "C" lq_status lq_q8_matvec(const lq_q8_weight* w, const int8_t* x_qs, const uint16_t* x_d,
                                  const float* residual, float* y, void* stream) {
    lq_status st = check_act("lq_q8_matvec", w, x_qs, x_d);
    if (st != LQ_OK || w->rows == 0) return st;
    if (!y) return fail(LQ_ERR_NULL, "lq_q8_matvec: y is NULL");
    if (!aligned(y, 4) || (residual && !aligned(residual, 4)))
        return fail(LQ_ERR_ALIGN, "lq_q8_matvec: y and residual must be 4-byte aligned");
    if (w->cols <= kMaxCols && w->rows <= 0x7fffffffLL) {
        MvArgs a{};
        a.wq = w->qs; a.wd = w->d; a.rows = (int)w->rows; a.cols = (int)w->cols;
        a.xq = x_qs; a.xd = x_d; a.res = residual; a.y = y;
        return launch_mv(a, PRO_Q8, residual ? EPI_RESID : EPI_STORE, as_stream(stream), kMvWgPerCu);
    }
    return launch_q8_matvec(w->qs, w->d, w->rows, w->cols, x_qs, x_d, residual, y, nullptr,
                            as_stream(stream));
}

extern "C" lq_status lq_q8_block_dots(const lq_q8_weight* w, const int8_t* x_qs, int32_t* dots,
                                      void* stream) {
    if (!w) return fail(LQ_ERR_NULL, "lq_q8_block_dots: weight descriptor is NULL");
    lq_status st = check_weight(w, "lq_q8_block_dots");
    if (st != LQ_OK || w->rows == 0) return st;
    if (!x_qs || !dots) return fail(LQ_ERR_NULL, "lq_q8_block_dots: NULL pointer");
    if (!aligned(x_qs, 16) || !aligned(dots, 4))
        return fail(LQ_ERR_ALIGN, "lq_q8_block_dots: x_qs must be 16-byte aligned");
    if (w->cols > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "lq_q8_block_dots: cols too large");
    if (w->cols <= kMaxCols && w->rows <= 0x7fffffffLL) {
        // the fused kernel lq_q8_matvec runs, with its dots written out
        MvArgs a{};
        a.wq = w->qs; a.wd = w->d; a.rows = (int)w->rows; a.cols = (int)w->cols;
        a.xq = x_qs; a.dots = dots;
        return launch_mv(a, PRO_Q8, EPI_DOTS, as_stream(stream), kMvWgPerCu);
    }
    return launch_q8_matvec(w->qs, w->d, w->rows, w->cols, x_qs, nullptr, nullptr, nullptr, dots,
                            as_stream(stream));
}

extern "C" lq_status lq_q8_block_dots_f32(const lq_q8_weight* w, const float* x, int32_t norm, const float* gamma,
                                          float eps, int32_t* dots, int8_t* x_qs_out, uint16_t* x_d_out,
                                          void* stream) {
    const char* fn = "lq_q8_block_dots_f32";
    if (!w) return fail(LQ_ERR_NULL, "%s: weight descriptor is NULL", fn);
    lq_status st = check_weight(w, fn);
    if (st != LQ_OK || w->rows == 0) return st;
    if (!x || !dots || !x_qs_out || !x_d_out) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (norm != 0 && norm != 1) return fail(LQ_ERR_SHAPE, "%s: norm must be 0 or 1", fn);
    if (!(eps >= 0.0f)) return fail(LQ_ERR_SHAPE, "%s: eps must be >= 0", fn);
    if (!aligned(x, 16) || (gamma && !aligned(gamma, 16)) || !aligned(dots, 4) || !aligned(x_qs_out, 8) ||
        !aligned(x_d_out, 2))
        return fail(LQ_ERR_ALIGN, "%s: x and gamma must be 16-byte aligned, x_qs_out 8-byte aligned", fn);
    if (w->cols > kMaxCols || w->rows > 0x7fffffffLL)
        return fail(LQ_ERR_UNSUPPORTED, "%s: cols > %d", fn, kMaxCols);
    MvArgs a{};
    a.wq = w->qs; a.wd = w->d; a.rows = (int)w->rows; a.cols = (int)w->cols;
    a.x = x; a.gamma = norm ? gamma : nullptr; a.eps = eps; a.dots = dots;
    a.tap_q = x_qs_out; a.tap_d = x_d_out;
    return launch_mv(a, norm ? PRO_NORM : PRO_QUANT, EPI_DOTS, as_stream(stream), kMvWgPerCu);
}

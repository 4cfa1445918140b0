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
    return launch_q8_matvec(w->qs, w->d, w->rows, w->cols, x_qs, nullptr, nullptr, nullptr, dots,
                            as_stream(stream));
}

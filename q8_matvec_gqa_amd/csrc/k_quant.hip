// k_quant.hip -- Q8_0 activation quantization kernels for gfx950:
//   * plain quantize (one lane owns one 32-value block),
//   * RMSNorm fused with the quantize of its output (one workgroup per row),
//   * SwiGLU fused with the quantize of its output.
// The block rule is the Q8_0 activation quantization that feeds the int8 x
// int8 matvec ("Design: lattice-inference", Current Design, CPU fallback and
// NEON): d = amax/127, codes = round-half-away(x / d), scale stored as f16.
#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

__global__ __launch_bounds__(256) void k_q8_quantize(const float* __restrict__ x, int64_t nb,
                                                     int8_t* __restrict__ qs,
                                                     uint16_t* __restrict__ d) {
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nb; b += (int64_t)gridDim.x * 256) {
        float v[32];
        load32(x + 32 * b, v);
        quantize_block32(v, qs + 32 * b, d + b);
    }
}

// One workgroup per row: sum of squares over the row (wave DPP reduction,
// then across the 4 waves in LDS), then every lane normalises and quantizes
// whole 32-blocks.  y = (x * rinv) * gamma.
__global__ __launch_bounds__(256) void k_rmsnorm_q8(const float* __restrict__ x, int64_t n,
                                                    const float* __restrict__ gamma, float eps,
                                                    int8_t* __restrict__ qs,
                                                    uint16_t* __restrict__ d) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const float* xr = x + row * n;
    float ss = 0.0f;
    for (int64_t i = (int64_t)threadIdx.x * 4; i < n; i += 1024) {
        float4 t = *reinterpret_cast<const float4*>(xr + i);
        ss += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float rinv = 1.0f / sqrtf(ss / (float)n + eps);
    const int64_t nb = n / 32;
    for (int64_t b = threadIdx.x; b < nb; b += 256) {
        float v[32];
        load32(xr + 32 * b, v);
        if (gamma) {
            float g[32];
            load32(gamma + 32 * b, g);
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = (v[i] * rinv) * g[i];
        } else {
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = v[i] * rinv;
        }
        quantize_block32(v, qs + row * n + 32 * b, d + row * nb + b);
    }
}

// h = silu(g) * u with silu(z) = z / (1 + exp(-z)); one lane per 32-block of h.
__global__ __launch_bounds__(256) void k_swiglu_q8(const float* __restrict__ gu, int64_t n_rows,
                                                   int64_t ffn, int8_t* __restrict__ qs,
                                                   uint16_t* __restrict__ d) {
    const int64_t nbr = ffn / 32;
    const int64_t nb = n_rows * nbr;
    for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nb; b += (int64_t)gridDim.x * 256) {
        const int64_t r = b / nbr, c = b - r * nbr;
        const float* g = gu + r * 2 * ffn + 32 * c;
        float v[32], u[32];
        load32(g, v);
        load32(g + ffn, u);
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = (v[i] / (1.0f + expf(-v[i]))) * u[i];
        quantize_block32(v, qs + r * ffn + 32 * c, d + b);
    }
}

// out = res + gamma * o / sqrt(mean(o^2) + eps): the weighted RMSNorm with
// residual add ("Current Inference Path -- Architecture Map", section 4,
// rms_norm F=3).  One workgroup, one vector.  out may alias res.
// One workgroup of 1024 threads; every load (o, gamma, res: up to 4 float4
// each per thread for n <= 16384) is issued before the first use, so the
// whole op costs one memory round trip.
constexpr int kNormAddThreads = 1024;
constexpr int kNormAddIters = 4;     // 4 * 1024 * 4 = 16384 elements
__global__ __launch_bounds__(kNormAddThreads) void k_rmsnorm_add(const float* __restrict__ o, int64_t n,
                                                                 const float* __restrict__ gamma, float eps,
                                                                 const float* res, float* out) {
    __shared__ float red[kNormAddThreads / 64];
    const int n4 = (int)(n >> 2);
    float4 ov[kNormAddIters], gv[kNormAddIters], rv[kNormAddIters];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kNormAddIters; ++k) {
        const int i = threadIdx.x + kNormAddThreads * k;
        const int ic = i < n4 ? i : 0;                       // valid address; dropped below
        ov[k] = reinterpret_cast<const float4*>(o)[ic];
        gv[k] = gamma ? reinterpret_cast<const float4*>(gamma)[ic] : make_float4(1.f, 1.f, 1.f, 1.f);
        rv[k] = reinterpret_cast<const float4*>(res)[ic];
    }
#pragma unroll
    for (int k = 0; k < kNormAddIters; ++k)
        if ((int)threadIdx.x + kNormAddThreads * k < n4)
            ss += ov[k].x * ov[k].x + ov[k].y * ov[k].y + ov[k].z * ov[k].z + ov[k].w * ov[k].w;
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = 0.0f;
#pragma unroll
    for (int w = 0; w < kNormAddThreads / 64; ++w) ss += red[w];
    const float rinv = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
    for (int k = 0; k < kNormAddIters; ++k) {
        const int i = threadIdx.x + kNormAddThreads * k;
        if (i < n4) {
            float4 y;
            y.x = rv[k].x + (ov[k].x * rinv) * gv[k].x;
            y.y = rv[k].y + (ov[k].y * rinv) * gv[k].y;
            y.z = rv[k].z + (ov[k].z * rinv) * gv[k].z;
            y.w = rv[k].w + (ov[k].w * rinv) * gv[k].w;
            reinterpret_cast<float4*>(out)[i] = y;
        }
    }
}

static int grid_for(int64_t items, int per_block) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g > 65536) g = 65536;
    return (int)(g < 1 ? 1 : g);
}

lq_status launch_q8_quantize(const float* x, int64_t n_blocks, int8_t* qs, uint16_t* d,
                             hipStream_t s) {
    if (n_blocks == 0) return LQ_OK;
    hipLaunchKernelGGL(k_q8_quantize, dim3(grid_for(n_blocks, 256)), dim3(256), 0, s, x, n_blocks, qs, d);
    return check_launch("q8_quantize");
}

lq_status launch_rmsnorm_q8(const float* x, int64_t n_rows, int64_t n, const float* gamma,
                            float eps, int8_t* qs, uint16_t* d, hipStream_t s) {
    if (n_rows == 0) return LQ_OK;
    hipLaunchKernelGGL(k_rmsnorm_q8, dim3((unsigned)n_rows), dim3(256), 0, s, x, n, gamma, eps, qs, d);
    return check_launch("rmsnorm_q8");
}

lq_status launch_swiglu_q8(const float* gate_up, int64_t n_rows, int64_t ffn, int8_t* qs,
                           uint16_t* d, hipStream_t s) {
    const int64_t nb = n_rows * (ffn / 32);
    if (nb == 0) return LQ_OK;
    hipLaunchKernelGGL(k_swiglu_q8, dim3(grid_for(nb, 256)), dim3(256), 0, s, gate_up, n_rows, ffn, qs, d);
    return check_launch("swiglu_q8");
}

lq_status launch_rmsnorm_add(const float* o, int64_t n, const float* gamma, float eps, const float* res,
                             float* out, hipStream_t s, LaunchMarks* mk) {
    if (n == 0) return LQ_OK;
    launch_marked(mk, k_rmsnorm_add, dim3(1), dim3(kNormAddThreads), 0, s, o, n, gamma, eps, res, out);
    return check_launch("rmsnorm_add");
}

static lq_status check_q8_out(const char* fn, int64_t n_rows, int64_t n, const void* x, int8_t* qs,
                              uint16_t* d) {
    if (n_rows < 0 || n <= 0 || n % 32)
        return fail(LQ_ERR_SHAPE, "%s: n_rows=%lld n=%lld (n must be a positive multiple of 32)", fn,
                    (long long)n_rows, (long long)n);
    if (n_rows == 0) return LQ_OK;
    if (!x || !qs || !d) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || !aligned(qs, 16) || !aligned(d, 2))
        return fail(LQ_ERR_ALIGN, "%s: input and codes must be 16-byte aligned", fn);
    return LQ_OK;
}

}  // namespace lq

using namespace lq;

extern "C" lq_status lq_q8_quantize_act(const float* x, int64_t n_rows, int64_t n, int8_t* qs,
                                        uint16_t* d, void* stream) {
    lq_status st = check_q8_out("lq_q8_quantize_act", n_rows, n, x, qs, d);
    if (st != LQ_OK || n_rows == 0) return st;
    return launch_q8_quantize(x, n_rows * (n / 32), qs, d, as_stream(stream));
}

extern "C" lq_status lq_rmsnorm_q8(const float* x, int64_t n_rows, int64_t n, const float* gamma,
                                   float eps, int8_t* qs, uint16_t* d, void* stream) {
    lq_status st = check_q8_out("lq_rmsnorm_q8", n_rows, n, x, qs, d);
    if (st != LQ_OK || n_rows == 0) return st;
    if (gamma && !aligned(gamma, 16)) return fail(LQ_ERR_ALIGN, "lq_rmsnorm_q8: gamma must be 16-byte aligned");
    if (!(eps >= 0.0f)) return fail(LQ_ERR_SHAPE, "lq_rmsnorm_q8: eps must be >= 0");
    if (n_rows > 0x7fffffff) return fail(LQ_ERR_UNSUPPORTED, "lq_rmsnorm_q8: too many rows");
    return launch_rmsnorm_q8(x, n_rows, n, gamma, eps, qs, d, as_stream(stream));
}

extern "C" lq_status lq_swiglu_q8(const float* gate_up, int64_t n_rows, int64_t ffn, int8_t* qs,
                                  uint16_t* d, void* stream) {
    lq_status st = check_q8_out("lq_swiglu_q8", n_rows, ffn, gate_up, qs, d);
    if (st != LQ_OK || n_rows == 0) return st;
    return launch_swiglu_q8(gate_up, n_rows, ffn, qs, d, as_stream(stream));
}

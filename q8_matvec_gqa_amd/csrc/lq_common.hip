// lq_common.hip -- status reporting and host-only helpers of liblq.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "lq_internal.h"

namespace lq {

static thread_local char g_last_error[512] = "";

lq_status fail(lq_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

lq_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LQ_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return LQ_OK;
}

lq_status check_weight(const lq_q8_weight* w, const char* name) {
    if (!w) return fail(LQ_ERR_NULL, "%s: weight descriptor is NULL", name);
    if (w->rows < 0 || w->cols <= 0 || (w->cols % 32) != 0)
        return fail(LQ_ERR_SHAPE, "%s: rows=%lld cols=%lld (cols must be a positive multiple of 32)",
                    name, (long long)w->rows, (long long)w->cols);
    if (w->rows == 0) return LQ_OK;
    if (!w->qs || !w->d) return fail(LQ_ERR_NULL, "%s: qs or d is NULL", name);
    if (!aligned(w->qs, 16)) return fail(LQ_ERR_ALIGN, "%s: qs must be 16-byte aligned", name);
    if (!aligned(w->d, 2)) return fail(LQ_ERR_ALIGN, "%s: d must be 2-byte aligned", name);
    return LQ_OK;
}

}  // namespace lq

using namespace lq;

extern "C" int32_t lq_version(void) { return 1; }

extern "C" const char* lq_status_string(lq_status s) {
    switch (s) {
        case LQ_OK: return "ok";
        case LQ_ERR_NULL: return "null pointer";
        case LQ_ERR_SHAPE: return "invalid shape";
        case LQ_ERR_ALIGN: return "misaligned pointer or stride";
        case LQ_ERR_WORKSPACE: return "workspace missing or too small";
        case LQ_ERR_HIP: return "HIP runtime error";
        case LQ_ERR_UNSUPPORTED: return "unsupported by the library's kernels";
        default: return "unknown status";
    }
}

extern "C" const char* lq_last_error(void) { return g_last_error; }

// GGML Q8_0 block: f16 scale (2 bytes, little-endian) then 32 int8 codes.
extern "C" lq_status lq_q8_pack_ggml(const void* blocks, int64_t rows, int64_t cols, int8_t* qs,
                                     uint16_t* d) {
    if (rows < 0 || cols <= 0 || cols % 32)
        return fail(LQ_ERR_SHAPE, "lq_q8_pack_ggml: rows=%lld cols=%lld", (long long)rows, (long long)cols);
    if (rows == 0) return LQ_OK;
    if (!blocks || !qs || !d) return fail(LQ_ERR_NULL, "lq_q8_pack_ggml: NULL pointer");
    const uint8_t* src = static_cast<const uint8_t*>(blocks);
    const int64_t nb = rows * (cols / 32);
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = src + 34 * b;
        d[b] = (uint16_t)(blk[0] | (blk[1] << 8));
        memcpy(qs + 32 * b, blk + 2, 32);
    }
    return LQ_OK;
}

extern "C" lq_status lq_q4_0_pack_ggml(const void* blocks, int64_t rows, int64_t cols, uint8_t* qs,
                                       uint16_t* d) {
    if (rows < 0 || cols <= 0 || cols % 32)
        return fail(LQ_ERR_SHAPE, "lq_q4_0_pack_ggml: rows=%lld cols=%lld", (long long)rows, (long long)cols);
    if (rows == 0) return LQ_OK;
    if (!blocks || !qs || !d) return fail(LQ_ERR_NULL, "lq_q4_0_pack_ggml: NULL pointer");
    const uint8_t* src = static_cast<const uint8_t*>(blocks);
    const int64_t nb = rows * (cols / 32);
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = src + 18 * b;
        d[b] = (uint16_t)(blk[0] | (blk[1] << 8));
        memcpy(qs + 16 * b, blk + 2, 16);
    }
    return LQ_OK;
}

extern "C" lq_status lq_q6_k_pack_ggml(const void* blocks, int64_t rows, int64_t cols, uint8_t* ql, uint8_t* qh,
                                       int8_t* sc, uint16_t* d) {
    if (rows < 0 || cols <= 0 || cols % 256)
        return fail(LQ_ERR_SHAPE, "lq_q6_k_pack_ggml: rows=%lld cols=%lld", (long long)rows, (long long)cols);
    if (rows == 0) return LQ_OK;
    if (!blocks || !ql || !qh || !sc || !d) return fail(LQ_ERR_NULL, "lq_q6_k_pack_ggml: NULL pointer");
    const uint8_t* src = static_cast<const uint8_t*>(blocks);
    const int64_t nb = rows * (cols / 256);
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = src + 210 * b;
        memcpy(ql + 128 * b, blk, 128);
        memcpy(qh + 64 * b, blk + 128, 64);
        memcpy(sc + 16 * b, blk + 192, 16);
        d[b] = (uint16_t)(blk[208] | (blk[209] << 8));
    }
    return LQ_OK;
}

extern "C" lq_status lq_rope_table_freqs(int64_t max_ctx, int64_t head_dim, double theta,
                                         const float* freq_factors, float* cos_out, float* sin_out) {
    if (max_ctx < 0 || head_dim <= 0 || head_dim % 2 || !(theta > 0.0))
        return fail(LQ_ERR_SHAPE, "lq_rope_table: max_ctx=%lld head_dim=%lld theta=%g",
                    (long long)max_ctx, (long long)head_dim, theta);
    const int64_t half = head_dim / 2;
    if (freq_factors)
        for (int64_t i = 0; i < half; ++i)
            if (!(freq_factors[i] > 0.0f))
                return fail(LQ_ERR_SHAPE, "lq_rope_table_freqs: freq_factors[%lld] must be > 0", (long long)i);
    if (max_ctx == 0) return LQ_OK;
    if (!cos_out || !sin_out) return fail(LQ_ERR_NULL, "lq_rope_table: NULL output");
    const double lt = log2(theta);
    for (int64_t i = 0; i < half; ++i) {
        double freq = exp2(-(2.0 * (double)i / (double)head_dim) * lt);
        if (freq_factors) freq /= (double)freq_factors[i];
        for (int64_t p = 0; p < max_ctx; ++p) {
            const double a = (double)p * freq;
            cos_out[p * half + i] = (float)cos(a);
            sin_out[p * half + i] = (float)sin(a);
        }
    }
    return LQ_OK;
}

extern "C" lq_status lq_rope_table(int64_t max_ctx, int64_t head_dim, double theta, float* cos_out,
                                   float* sin_out) {
    return lq_rope_table_freqs(max_ctx, head_dim, theta, nullptr, cos_out, sin_out);
}

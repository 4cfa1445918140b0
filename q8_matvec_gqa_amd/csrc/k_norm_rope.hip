// k_norm_rope.hip -- per-head RMSNorm + NeoX RoPE and the KV-cache append.
//
// "Design: lattice-inference" (Current Design, fused_qk_norm_rope: one
// thread per rotation pair) and "Current Inference Path -- Architecture Map"
// (section 4: RMSNorm F=1/F=2, NeoX RoPE pairing (i, i + head_dim/2),
// stride-aware so Q/K are read in place; section 1: in-place KV append).
//
// On CDNA4 one wavefront owns one head: lane l holds the pairs
// i = l, l+64, l+128, l+192 (head_dim <= 512), the sum of squares is a DPP
// wave reduction, and the rotated values are written back in place (q, k)
// or converted straight into the cache row (k, v in the decode layer).
#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

constexpr int kMaxPairs = 4;   // head_dim <= 2 * 64 * kMaxPairs = 512

struct HeadVals {
    float a[kMaxPairs], b[kMaxPairs];
};

__device__ __forceinline__ void head_load(const float* xh, int half, int lane, HeadVals& v, float& ss) {
    ss = 0.0f;
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        const int i = lane + 64 * p;
        v.a[p] = 0.0f;
        v.b[p] = 0.0f;
        if (i < half) {
            v.a[p] = xh[i];
            v.b[p] = xh[i + half];
        }
        ss += v.a[p] * v.a[p] + v.b[p] * v.b[p];
    }
}

__device__ __forceinline__ void head_norm(HeadVals& v, float ss, int hd, int half, int lane,
                                          const float* __restrict__ gamma, float eps) {
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)hd + eps);
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        const int i = lane + 64 * p;
        if (i < half) {
            const float ga = gamma ? gamma[i] : 1.0f;
            const float gb = gamma ? gamma[i + half] : 1.0f;
            v.a[p] = (v.a[p] * rinv) * ga;
            v.b[p] = (v.b[p] * rinv) * gb;
        }
    }
}

__device__ __forceinline__ void head_rope(HeadVals& v, int half, int lane, const float* __restrict__ c,
                                          const float* __restrict__ s) {
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        const int i = lane + 64 * p;
        if (i < half) {
            const float cs = c[i], sn = s[i];
            const float a = v.a[p], b = v.b[p];
            v.a[p] = a * cs - b * sn;
            v.b[p] = a * sn + b * cs;
        }
    }
}

__device__ __forceinline__ void head_store(float* xh, int half, int lane, const HeadVals& v) {
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        const int i = lane + 64 * p;
        if (i < half) {
            xh[i] = v.a[p];
            xh[i + half] = v.b[p];
        }
    }
}

__device__ __forceinline__ void head_store_cache(void* cache, int32_t dtype, int64_t off, int half,
                                                 int lane, const HeadVals& v) {
#pragma unroll
    for (int p = 0; p < kMaxPairs; ++p) {
        const int i = lane + 64 * p;
        if (i < half) {
            if (dtype == LQ_KV_F32) {
                float* c = static_cast<float*>(cache) + off;
                c[i] = v.a[p];
                c[i + half] = v.b[p];
            } else {
                uint16_t* c = static_cast<uint16_t*>(cache) + off;
                c[i] = (uint16_t)f32_to_bf16(v.a[p]);
                c[i + half] = (uint16_t)f32_to_bf16(v.b[p]);
            }
        }
    }
}

// Standalone: n_heads heads at x + h*head_stride, in place.
__global__ __launch_bounds__(256) void k_rmsnorm_rope(float* x, int64_t n_heads, int hd,
                                                      int64_t head_stride,
                                                      const float* __restrict__ gamma, float eps,
                                                      const float* __restrict__ cos_row,
                                                      const float* __restrict__ sin_row) {
    const int64_t head = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (head >= n_heads) return;
    const int lane = threadIdx.x & 63, half = hd >> 1;
    float* xh = x + head * head_stride;
    HeadVals v;
    float ss;
    head_load(xh, half, lane, v, ss);
    head_norm(v, ss, hd, half, lane, gamma, eps);
    if (cos_row) head_rope(v, half, lane, cos_row, sin_row);
    head_store(xh, half, lane, v);
}

// Decode-layer post-projection step.  Waves [0, n_q) handle q heads,
// [n_q, n_q + n_kv) k heads, [n_q + n_kv, n_q + 2 n_kv) v heads; all in
// place on the fused qkv vector, k and v also converted into the caches.
__global__ __launch_bounds__(256) void k_qkv_post(float* qkv, int n_q, int n_kv, int hd,
                                                  const float* __restrict__ g_q,
                                                  const float* __restrict__ g_k, int qk_norm,
                                                  int v_unit_norm, float eps,
                                                  const float* __restrict__ cos_row,
                                                  const float* __restrict__ sin_row, void* kc,
                                                  void* vc, int32_t dtype, int64_t cache_off,
                                                  int64_t head_stride) {
    const int head = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (head >= n_q + 2 * n_kv) return;
    const int lane = threadIdx.x & 63, half = hd >> 1;
    float* xh = qkv + (int64_t)head * hd;
    HeadVals v;
    float ss;
    head_load(xh, half, lane, v, ss);
    if (head < n_q + n_kv) {
        if (qk_norm) head_norm(v, ss, hd, half, lane, head < n_q ? g_q : g_k, eps);
        head_rope(v, half, lane, cos_row, sin_row);
        head_store(xh, half, lane, v);
        if (head >= n_q)
            head_store_cache(kc, dtype, (int64_t)(head - n_q) * head_stride + cache_off, half, lane, v);
    } else {
        if (v_unit_norm) head_norm(v, ss, hd, half, lane, nullptr, eps);
        head_store(xh, half, lane, v);
        head_store_cache(vc, dtype, (int64_t)(head - n_q - n_kv) * head_stride + cache_off, half, lane, v);
    }
}

__global__ __launch_bounds__(256) void k_kv_append(const float* __restrict__ k,
                                                   const float* __restrict__ v, int64_t n_kv, int hd,
                                                   void* kc, void* vc, int32_t dtype,
                                                   int64_t head_stride, int64_t cache_off) {
    const int64_t n = n_kv * hd;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n; i += (int64_t)gridDim.x * 256) {
        const bool is_v = i >= n;
        const int64_t j = is_v ? i - n : i;
        const int64_t g = j / hd, e = j - g * hd;
        const float val = is_v ? v[j] : k[j];
        const int64_t dst = g * head_stride + cache_off + e;
        void* cache = is_v ? vc : kc;
        if (dtype == LQ_KV_F32)
            static_cast<float*>(cache)[dst] = val;
        else
            static_cast<uint16_t*>(cache)[dst] = (uint16_t)f32_to_bf16(val);
    }
}

lq_status launch_rmsnorm_rope(float* x, int64_t n_heads, int64_t hd, int64_t head_stride,
                              const float* gamma, float eps, const float* rope_cos,
                              const float* rope_sin, int64_t pos, hipStream_t s) {
    if (n_heads == 0) return LQ_OK;
    const int64_t half = hd / 2;
    const float* c = rope_cos ? rope_cos + pos * half : nullptr;
    const float* sn = rope_sin ? rope_sin + pos * half : nullptr;
    hipLaunchKernelGGL(k_rmsnorm_rope, dim3((unsigned)((n_heads + 3) / 4)), dim3(256), 0, s, x, n_heads,
                       (int)hd, head_stride, gamma, eps, c, sn);
    return check_launch("rmsnorm_rope");
}

lq_status launch_kv_append(const float* k, const float* v, int64_t n_kv, int64_t hd, void* kc,
                           void* vc, int32_t kv_dtype, int64_t head_stride, int64_t pos_stride,
                           int64_t pos, hipStream_t s) {
    const int64_t n = 2 * n_kv * hd;
    if (n == 0) return LQ_OK;
    int64_t grid = (n + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_kv_append, dim3((unsigned)grid), dim3(256), 0, s, k, v, n_kv, (int)hd, kc, vc,
                       kv_dtype, head_stride, pos * pos_stride);
    return check_launch("kv_append");
}

lq_status launch_qkv_post(float* qkv, int64_t n_q, int64_t n_kv, int64_t hd, const float* g_q,
                          const float* g_k, int32_t qk_norm, int32_t v_unit_norm, float eps,
                          const float* rope_cos, const float* rope_sin, int64_t pos, void* kc,
                          void* vc, int32_t kv_dtype, int64_t head_stride, int64_t pos_stride,
                          hipStream_t s) {
    const int64_t heads = n_q + 2 * n_kv;
    const int64_t half = hd / 2;
    hipLaunchKernelGGL(k_qkv_post, dim3((unsigned)((heads + 3) / 4)), dim3(256), 0, s, qkv, (int)n_q,
                       (int)n_kv, (int)hd, g_q, g_k, qk_norm, v_unit_norm, eps, rope_cos + pos * half,
                       rope_sin + pos * half, kc, vc, kv_dtype, pos * pos_stride, head_stride);
    return check_launch("qkv_post");
}

}  // namespace lq

using namespace lq;

extern "C" lq_status lq_rmsnorm_rope(float* x, int64_t n_heads, int64_t head_dim, int64_t head_stride,
                                     const float* gamma, float eps, const float* rope_cos,
                                     const float* rope_sin, int64_t rope_len, int64_t pos, void* stream) {
    if (n_heads < 0 || head_dim < 2 || head_dim % 2 || head_stride < head_dim || pos < 0)
        return fail(LQ_ERR_SHAPE, "lq_rmsnorm_rope: n_heads=%lld head_dim=%lld head_stride=%lld pos=%lld",
                    (long long)n_heads, (long long)head_dim, (long long)head_stride, (long long)pos);
    if (head_dim > 2 * 64 * kMaxPairs)
        return fail(LQ_ERR_UNSUPPORTED, "lq_rmsnorm_rope: head_dim > %d", 2 * 64 * kMaxPairs);
    if (n_heads == 0) return LQ_OK;
    if (n_heads > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "lq_rmsnorm_rope: too many heads");
    if (!x) return fail(LQ_ERR_NULL, "lq_rmsnorm_rope: x is NULL");
    if ((rope_cos == nullptr) != (rope_sin == nullptr))
        return fail(LQ_ERR_NULL, "lq_rmsnorm_rope: pass both RoPE tables or neither");
    if (rope_cos && pos >= rope_len)
        return fail(LQ_ERR_SHAPE, "lq_rmsnorm_rope: pos=%lld outside the %lld-row RoPE table", (long long)pos,
                    (long long)rope_len);
    if (!(eps >= 0.0f)) return fail(LQ_ERR_SHAPE, "lq_rmsnorm_rope: eps must be >= 0");
    if (!aligned(x, 4)) return fail(LQ_ERR_ALIGN, "lq_rmsnorm_rope: x must be 4-byte aligned");
    return launch_rmsnorm_rope(x, n_heads, head_dim, head_stride, gamma, eps, rope_cos, rope_sin, pos,
                               as_stream(stream));
}

extern "C" lq_status lq_kv_append(const float* k, const float* v, int64_t n_kv, int64_t head_dim,
                                  void* k_cache, void* v_cache, int32_t kv_dtype, int64_t head_stride,
                                  int64_t pos_stride, int64_t max_ctx, int64_t pos, void* stream) {
    if (n_kv < 0 || head_dim <= 0 || pos < 0 || pos >= max_ctx || pos_stride < head_dim || head_stride < 0)
        return fail(LQ_ERR_SHAPE, "lq_kv_append: n_kv=%lld head_dim=%lld pos=%lld pos_stride=%lld",
                    (long long)n_kv, (long long)head_dim, (long long)pos, (long long)pos_stride);
    if (kv_dtype != LQ_KV_F32 && kv_dtype != LQ_KV_BF16)
        return fail(LQ_ERR_SHAPE, "lq_kv_append: kv_dtype %d", kv_dtype);
    if (n_kv == 0) return LQ_OK;
    if (!k || !v || !k_cache || !v_cache) return fail(LQ_ERR_NULL, "lq_kv_append: NULL pointer");
    const size_t es = kv_dtype == LQ_KV_F32 ? 4 : 2;
    if (!aligned(k, 4) || !aligned(v, 4) || !aligned(k_cache, es) || !aligned(v_cache, es))
        return fail(LQ_ERR_ALIGN, "lq_kv_append: misaligned pointer");
    return launch_kv_append(k, v, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride, pos,
                            as_stream(stream));
}

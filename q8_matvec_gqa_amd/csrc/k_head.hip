// k_head.hip -- the output head for gfx950: final RMSNorm, f16 vocab
// projection and logit softcapping in one launch.
//
// What it computes ("Current Inference Path -- Architecture Map", section 3,
// forward pass steps 4, 5 and 7: final RmsNorm, normed times the transposed
// lm_head weight, softcapping as division, tanh and multiplication; section
// 4, lm_head_kernel: the projection on F16 weights; "Target Inference
// Architecture: hf2q on mlx-native", section 3.2: rms_norm, f16_gemm,
// softcap, and section 3.3: lm_head_f16 [vocab, hidden] f16, logits
// [1, vocab] f32):
//     n = norm ? gamma * x / sqrt(mean(x^2) + eps) : x
//     logits[r] = sum_c f16(W[r, c]) * n[c],  then cap * tanh(logits / cap)
//
// Mapping onto CDNA4: the weight (vocab x hidden f16, 1.5 GB for a 262144 x
// 2816 head) is streamed from HBM once, so the kernel is a plain bandwidth
// problem.  Every workgroup builds n in LDS (the prologue's loads go out
// before the first rows' weights); each lane then keeps the f32 n values of
// its 16-byte column chunks in registers.  A wave owns RPW rows per group,
// lane l reads chunk l + 64*st of each row (one coalesced 128-bit load per
// lane and step), converts the 8 halves and accumulates with FMAs; a DPP wave
// sum finishes each row.  Row groups are double-buffered with the next
// group's loads issued before the current one is consumed.
#include <math.h>

#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

namespace {

constexpr int kHeadWaves = 8;
constexpr int kHeadRPW = 2;
constexpr int kHeadMaxHidden = 4096;

struct HeadArgs {
    const uint16_t* w;      // [vocab, hidden] f16 bits
    int64_t vocab;
    int hidden;
    const float* x;         // [hidden]
    const float* gamma;     // [hidden] or NULL (unit weight)
    int norm;
    float eps;
    float cap;              // <= 0: no softcap
    float* logits;          // [vocab]
};

template <int ST>
struct HeadRows {
    int4 w[kHeadRPW][ST];
};

// Unconditional loads: chunks past the row's end read the row's last chunk
// (the same 16 bytes a live lane reads, so the request merges with it; their
// n values are zero) and rows past the end read the first 16 bytes of the
// matrix (never stored).
template <int ST>
__device__ __forceinline__ void head_load(const HeadArgs& a, int64_t grp, int lane, int c16, HeadRows<ST>& R) {
#pragma unroll
    for (int i = 0; i < kHeadRPW; ++i) {
        const int64_t r = grp * kHeadRPW + i;
        const bool live = r < a.vocab;
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int ch = st * kWave + lane;
            const int64_t off = live ? r * a.hidden + 8 * (ch < c16 ? ch : c16 - 1) : 0;
            R.w[i][st] = load_stream16(a.w + off);
        }
    }
}

__device__ __forceinline__ float head_cap(float y, float cap) {
    return cap > 0.0f ? cap * tanhf(y / cap) : y;
}

template <int ST>
__device__ __forceinline__ void head_consume(const HeadArgs& a, int64_t grp, int lane, const HeadRows<ST>& R,
                                             const float (&n)[ST][8]) {
#pragma unroll
    for (int i = 0; i < kHeadRPW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const uint32_t u[4] = {(uint32_t)R.w[i][st].x, (uint32_t)R.w[i][st].y, (uint32_t)R.w[i][st].z,
                                   (uint32_t)R.w[i][st].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc = fmaf(f16_to_f32(u[j] & 0xffffu), n[st][2 * j], acc);
                acc = fmaf(f16_to_f32(u[j] >> 16), n[st][2 * j + 1], acc);
            }
        }
        acc = wave_sum(acc);
        const int64_t r = grp * kHeadRPW + i;
        if (lane == 0 && r < a.vocab) a.logits[r] = head_cap(acc, a.cap);
    }
}

template <int ST>
__global__ __launch_bounds__(kHeadWaves * 64, 2) void k_lm_head(HeadArgs a) {
    constexpr int NT = kHeadWaves * 64;
    __shared__ __attribute__((aligned(16))) float n_s[kHeadMaxHidden];
    __shared__ float red[kHeadWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.hidden, c16 = H >> 3, n4 = H >> 2;
    const int64_t ngroups = (a.vocab + kHeadRPW - 1) / kHeadRPW;
    const int64_t gstride = (int64_t)gridDim.x * kHeadWaves;
    int64_t g = (int64_t)blockIdx.x * kHeadWaves + wave;

    // prologue loads first (x and gamma, 16 bytes per thread and step), then
    // the first row group's weights
    // (threads past the vector issue no load: every workgroup reads x, and
    // clamped duplicates would pile onto one cache line)
    constexpr int XP = (kHeadMaxHidden / 4 + NT - 1) / NT;
    float4 xv[XP], gv[XP];
#pragma unroll
    for (int k = 0; k < XP; ++k) {
        const int i4 = threadIdx.x + NT * k;
        xv[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        gv[k] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if (i4 < n4) {
            xv[k] = reinterpret_cast<const float4*>(a.x)[i4];
            if (a.gamma) gv[k] = reinterpret_cast<const float4*>(a.gamma)[i4];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    HeadRows<ST> A, B;
    head_load<ST>(a, g < ngroups ? g : ngroups, lane, c16, A);

    float rinv = 1.0f;
    if (a.norm) {
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < XP; ++k)
            if (threadIdx.x + NT * k < n4)
                ss += xv[k].x * xv[k].x + xv[k].y * xv[k].y + xv[k].z * xv[k].z + xv[k].w * xv[k].w;
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        ss = 0.0f;
#pragma unroll
        for (int w = 0; w < kHeadWaves; ++w) ss += red[w];
        rinv = 1.0f / sqrtf(ss / (float)H + a.eps);
    }
#pragma unroll
    for (int k = 0; k < XP; ++k) {
        const int i4 = threadIdx.x + NT * k;
        if (i4 < n4) {
            float4 v = xv[k];
            if (a.norm) {
                v.x = (v.x * rinv) * gv[k].x; v.y = (v.y * rinv) * gv[k].y;
                v.z = (v.z * rinv) * gv[k].z; v.w = (v.w * rinv) * gv[k].w;
            }
            reinterpret_cast<float4*>(n_s)[i4] = v;
        }
    }
    __syncthreads();
    float n[ST][8];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        const int ch = st * kWave + lane;
#pragma unroll
        for (int e = 0; e < 8; ++e) n[st][e] = ch < c16 ? n_s[8 * ch + e] : 0.0f;
    }

    // grid-stride over row groups, the next group's loads issued before the
    // current one is consumed (the last step peeled, so each wait covers
    // exactly the loads it needs)
    while (g < ngroups) {
        const int64_t g1 = g + gstride;
        if (g1 >= ngroups) {
            head_consume<ST>(a, g, lane, A, n);
            break;
        }
        head_load<ST>(a, g1, lane, c16, B);
        head_consume<ST>(a, g, lane, A, n);
        const int64_t g2 = g1 + gstride;
        if (g2 >= ngroups) {
            head_consume<ST>(a, g1, lane, B, n);
            break;
        }
        head_load<ST>(a, g2, lane, c16, A);
        head_consume<ST>(a, g1, lane, B, n);
        g = g2;
    }
}

template <int ST>
void launch_head(const HeadArgs& a, hipStream_t s) {
    const int64_t groups = (a.vocab + kHeadRPW - 1) / kHeadRPW;
    const int64_t waves = (int64_t)kNumCUs * 2 * 4;       // one resident round: 2 waves per SIMD
    const int64_t iters = (groups + waves - 1) / waves;
    int64_t grid = (groups + kHeadWaves * iters - 1) / (kHeadWaves * iters);
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_lm_head<ST>, dim3((unsigned)grid), dim3(kHeadWaves * 64), 0, s, a);
}

}  // namespace

}  // namespace lq

using namespace lq;

extern "C" lq_status lq_lm_head_f16(const uint16_t* w, int64_t vocab, int64_t hidden, const float* x,
                                    int32_t norm, const float* gamma, float eps, float softcap, float* logits,
                                    void* stream) {
    const char* fn = "lq_lm_head_f16";
    if (vocab < 0 || hidden <= 0 || hidden % 8)
        return fail(LQ_ERR_SHAPE, "%s: vocab=%lld hidden=%lld (need hidden %% 8 == 0)", fn, (long long)vocab,
                    (long long)hidden);
    if (hidden > kHeadMaxHidden)
        return fail(LQ_ERR_UNSUPPORTED, "%s: hidden=%lld > %d", fn, (long long)hidden, kHeadMaxHidden);
    if (vocab == 0) return LQ_OK;
    if (!w || !x || !logits) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(w, 16) || !aligned(x, 16) || (gamma && !aligned(gamma, 16)) || !aligned(logits, 4))
        return fail(LQ_ERR_ALIGN, "%s: w, x and gamma must be 16-byte aligned", fn);
    HeadArgs a{w, vocab, (int)hidden, x, gamma, norm != 0, eps, softcap, logits};
    const hipStream_t s = as_stream(stream);
    switch ((int)((hidden / 8 + kWave - 1) / kWave)) {
        case 1: launch_head<1>(a, s); break;
        case 2: launch_head<2>(a, s); break;
        case 3: launch_head<3>(a, s); break;
        case 4: launch_head<4>(a, s); break;
        case 5: launch_head<5>(a, s); break;
        case 6: launch_head<6>(a, s); break;
        case 7: launch_head<7>(a, s); break;
        default: launch_head<8>(a, s); break;
    }
    return check_launch(fn);
}

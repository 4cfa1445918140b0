// k_attn.hip -- GQA decode attention over a KV cache for gfx950.
//
// What it computes ("Inference Engine" (larql), BLAS-Fused Attention, How
// it works: scores K.q scaled by 1/sqrt(head_dim), softmax, V^T.p; GQA with
// any ratio; "Design: lattice-inference", Current Design: fused attention
// with online softmax, the GQA group's query rows handled together):
//     s_j = scale * <q_h, K[g, j]>,  out_h = sum_j softmax(s)_j V[g, j],
//     g = h / G for the G = n_q / n_kv query heads of kv head g.
//
// Mapping onto CDNA4 (flash-decoding style split of the positions):
//   * grid = (splits, n_kv); a workgroup of 4 waves owns one kv head and a
//     range of positions; its waves take 64-position tiles round-robin.  All
//     G query heads of the kv head are served from one read of K and V.
//   * K phase: NP consecutive lanes share one position; each lane holds the
//     (pre-scaled) query slice of its 16-byte chunks for all G heads in VGPRs,
//     does CE*G FMAs per 16-byte K load, and the NP partial dots are summed
//     with DPP / permlane group reductions.  Scores go to LDS.
//   * softmax: one lane per position of the tile; running max per head is a
//     wave max, probabilities are exp2 of pre-scaled scores (log2(e) folded
//     into q); the running sum stays per lane until the end.
//   * V phase: VC lanes per position read 16-byte V chunks (coalesced rows)
//     and accumulate p * V for all G heads; p is broadcast from LDS.
//   * end: waves combine (m, l, acc) in LDS; with one split the workgroup
//     writes the normalised output, else a partial that a second kernel
//     rescales and sums over splits.
#include <math.h>

#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

namespace {

constexpr int kTile = 64;        // positions per wave iteration (one per lane in the softmax)
constexpr int kWavesPerWG = 4;
constexpr float kLog2e = 1.4426950408889634f;

template <typename KV> struct KvTraits;
template <> struct KvTraits<float> {
    static constexpr int CE = 4;   // elements per 16-byte chunk
    __device__ static __forceinline__ void unpack(const int4& c, float (&f)[4]) {
        f[0] = __int_as_float(c.x); f[1] = __int_as_float(c.y);
        f[2] = __int_as_float(c.z); f[3] = __int_as_float(c.w);
    }
};
template <> struct KvTraits<uint16_t> {
    static constexpr int CE = 8;
    __device__ static __forceinline__ void unpack(const int4& c, float (&f)[8]) {
        const uint32_t w[4] = {(uint32_t)c.x, (uint32_t)c.y, (uint32_t)c.z, (uint32_t)c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo_to_f32(w[i]);
            f[2 * i + 1] = bf16hi_to_f32(w[i]);
        }
    }
};

struct AttnArgs {
    const float* q;
    const void* kc;
    const void* vc;
    float* out;
    float* part_m;     // [n_kv][nsplit][G]
    float* part_l;
    float* part_acc;   // [n_kv][nsplit][G][hd]
    int64_t head_stride, pos_stride, start, len;
    int hd, G, nsplit, tiles_per_split;
    float qscale;      // scale * log2(e)
};

}  // namespace

// KV: float or uint16_t (bf16).  NP lanes per position and CPL chunks per
// lane in the K phase; GM >= G heads per kv head; VCPL chunks per lane in
// the V phase (head_dim > 64 chunks needs 2).
template <typename KV, int NP, int CPL, int GM, int VCPL>
__global__ __launch_bounds__(256) void k_attn_split(AttnArgs a) {
    constexpr int CE = KvTraits<KV>::CE;
    constexpr int TP = kWave / NP;                 // positions per K step
    constexpr int KB = NP < 8 ? NP : 8;             // K steps per load group
    constexpr int VB = 8;                           // V steps per load group
    __shared__ float red[8 * 512];                  // [G][hd] workgroup accumulator
    __shared__ float sc[kWavesPerWG][kTile][GM];
    __shared__ float wm[kWavesPerWG][GM], wl[kWavesPerWG][GM];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.y, split = blockIdx.x;
    const int hd = a.hd, G = a.G, C = hd / CE;
    const KV* kc = static_cast<const KV*>(a.kc) + (int64_t)g * a.head_stride;
    const KV* vc = static_cast<const KV*>(a.vc) + (int64_t)g * a.head_stride;
    const int64_t end = a.start + a.len;

    // ---- query slice in registers, pre-scaled by scale*log2(e)
    const int kp = lane / NP, kk = lane % NP;
    float qr[GM][CPL][CE];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = kk + c * NP;
#pragma unroll
            for (int e = 0; e < CE; ++e)
                qr[h][c][e] = (h < G && ch < C) ? a.q[(int64_t)(g * G + h) * hd + ch * CE + e] * a.qscale : 0.0f;
        }

    // V-phase lane layout
    const int VC = C < 64 ? C : 64;
    const int VTP = 64 / VC;
    const int vp = lane / VC, vk = lane % VC;
    const bool v_lane = vp < VTP;
    const int vsteps = (kTile + VTP - 1) / VTP;

    float m[GM], l[GM], acc[GM][VCPL][CE];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < VCPL; ++c)
#pragma unroll
            for (int e = 0; e < CE; ++e) acc[h][c][e] = 0.0f;
    }

    const int t0 = split * a.tiles_per_split;
    const int64_t total_tiles = (a.len + kTile - 1) / kTile;
    int t1 = t0 + a.tiles_per_split;
    if (t1 > total_tiles) t1 = (int)total_tiles;

    for (int tb = t0; tb < t1; tb += kWavesPerWG) {
        const int tile = tb + wave;
        const int64_t p0 = a.start + (int64_t)tile * kTile;   // first position of this wave's tile
        const bool tile_ok = tile < t1;

        // ---- K phase: scores for 64 positions
        for (int sb = 0; sb < NP; sb += KB) {
            int4 kr[KB][CPL];
#pragma unroll
            for (int st = 0; st < KB; ++st) {
                const int64_t pos = p0 + (sb + st) * TP + kp;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const int ch = kk + c * NP;
                    kr[st][c] = make_int4(0, 0, 0, 0);
                    if (tile_ok && pos < end && ch < C)
                        kr[st][c] = *reinterpret_cast<const int4*>(kc + pos * a.pos_stride + ch * CE);
                }
            }
#pragma unroll
            for (int st = 0; st < KB; ++st) {
                float part[GM];
#pragma unroll
                for (int h = 0; h < GM; ++h) part[h] = 0.0f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    float kf[CE];
                    KvTraits<KV>::unpack(kr[st][c], kf);
#pragma unroll
                    for (int h = 0; h < GM; ++h)
#pragma unroll
                        for (int e = 0; e < CE; ++e) part[h] = fmaf(qr[h][c][e], kf[e], part[h]);
                }
#pragma unroll
                for (int h = 0; h < GM; ++h) part[h] = group_sum<NP>(part[h]);
                if (kk == 0) {
                    const int pt = (sb + st) * TP + kp;
#pragma unroll
                    for (int h = 0; h < GM; ++h) sc[wave][pt][h] = part[h];
                }
            }
        }
        __syncthreads();

        // ---- softmax over the tile, lane = position
        float alpha[GM];
        {
            const int64_t pos = p0 + lane;
            const bool ok = tile_ok && pos < end;
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                const float s = ok ? sc[wave][lane][h] : -INFINITY;
                const float mt = wave_max(s);
                const float mn = fmaxf(m[h], mt);
                float p = 0.0f;
                if (mn == -INFINITY) {
                    alpha[h] = 1.0f;
                } else {
                    alpha[h] = exp2f(m[h] - mn);
                    p = ok ? exp2f(s - mn) : 0.0f;
                }
                l[h] = l[h] * alpha[h] + p;
                m[h] = mn;
                sc[wave][lane][h] = p;
            }
        }
        __syncthreads();

        // ---- V phase: acc = acc * alpha + sum_j p_j V_j
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
            for (int c = 0; c < VCPL; ++c)
#pragma unroll
                for (int e = 0; e < CE; ++e) acc[h][c][e] *= alpha[h];
        for (int sb = 0; sb < vsteps; sb += VB) {
            int4 vr[VB][VCPL];
#pragma unroll
            for (int st = 0; st < VB; ++st) {
                const int pt = (sb + st) * VTP + vp;
                const int64_t pos = p0 + pt;
#pragma unroll
                for (int c = 0; c < VCPL; ++c) {
                    const int ch = vk + 64 * c;
                    vr[st][c] = make_int4(0, 0, 0, 0);
                    if (tile_ok && v_lane && pt < kTile && pos < end && ch < C)
                        vr[st][c] = *reinterpret_cast<const int4*>(vc + pos * a.pos_stride + ch * CE);
                }
            }
#pragma unroll
            for (int st = 0; st < VB; ++st) {
                const int pt = (sb + st) * VTP + vp;
                if (pt < kTile) {
                    float p[GM];
#pragma unroll
                    for (int h = 0; h < GM; ++h) p[h] = sc[wave][pt][h];
#pragma unroll
                    for (int c = 0; c < VCPL; ++c) {
                        float vf[CE];
                        KvTraits<KV>::unpack(vr[st][c], vf);
#pragma unroll
                        for (int h = 0; h < GM; ++h)
#pragma unroll
                            for (int e = 0; e < CE; ++e) acc[h][c][e] = fmaf(p[h], vf[e], acc[h][c][e]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- combine the waves of this workgroup.  Each wave's running max and
    // sum go to LDS; then the waves, one after another, add their rescaled
    // accumulators (position sub-groups of a wave also one after another)
    // into one [G][hd] buffer, so the order of the float sums is fixed.
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        const float ls = wave_sum(l[h]);
        if (lane == 0) {
            wm[wave][h] = m[h];
            wl[wave][h] = ls;
        }
    }
    __syncthreads();
    float ew[GM];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, wm[w][h]);
        ew[h] = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - M);
    }
    for (int w = 0; w < kWavesPerWG; ++w) {
        if (wave == w && v_lane) {
            for (int v = 0; v < VTP; ++v) {
                if (vp == v) {
#pragma unroll
                    for (int h = 0; h < GM; ++h)
                        if (h < G) {
#pragma unroll
                            for (int c = 0; c < VCPL; ++c) {
                                const int ch = vk + 64 * c;
                                if (ch < C)
#pragma unroll
                                    for (int e = 0; e < CE; ++e) {
                                        float* r = &red[h * hd + ch * CE + e];
                                        const float add = ew[h] * acc[h][c][e];
                                        *r = (w == 0 && v == 0) ? add : *r + add;
                                    }
                            }
                        }
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this sub-group's LDS adds land first
                __builtin_amdgcn_wave_barrier();
            }
        }
        __syncthreads();
    }
    const int n_el = G * hd;
    for (int idx = threadIdx.x; idx < n_el; idx += 256) {
        const int h = idx / hd, d = idx - h * hd;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, wm[w][h]);
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesPerWG; ++w)
            L += (wm[w][h] == -INFINITY) ? 0.0f : exp2f(wm[w][h] - M) * wl[w][h];
        const float S = red[idx];
        if (a.nsplit == 1) {
            a.out[(int64_t)(g * G + h) * hd + d] = S / L;
        } else {
            const int64_t slot = ((int64_t)g * a.nsplit + split) * G + h;
            a.part_acc[slot * hd + d] = S;
            if (d == 0) {
                a.part_m[slot] = M;
                a.part_l[slot] = L;
            }
        }
    }
}

// Rescale and sum the split partials: one thread per output element.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a, int64_t n_q) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_q * a.hd) return;
    const int64_t hq = idx / a.hd;
    const int d = (int)(idx - hq * a.hd);
    const int64_t g = hq / a.G, h = hq - g * a.G;
    float M = -INFINITY;
    for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_m[(g * a.nsplit + s) * a.G + h]);
    float L = 0.0f, S = 0.0f;
    for (int s = 0; s < a.nsplit; ++s) {
        const int64_t slot = (g * a.nsplit + s) * a.G + h;
        const float ms = a.part_m[slot];
        const float e = (ms == -INFINITY) ? 0.0f : exp2f(ms - M);
        L += e * a.part_l[slot];
        S += e * a.part_acc[slot * a.hd + d];
    }
    a.out[idx] = S / L;
}

__global__ void k_fill_zero(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// ---- host side ------------------------------------------------------------

namespace {

struct Plan {
    int nsplit, tiles_per_split;
};

Plan make_plan(int64_t n_kv, int64_t len) {
    const int64_t tiles = (len + kTile - 1) / kTile;
    const int64_t target_wgs = 256;
    int64_t ns = (target_wgs + n_kv - 1) / n_kv;
    if (ns > tiles) ns = tiles;
    if (ns < 1) ns = 1;
    int64_t tps = (tiles + ns - 1) / ns;
    if (tps < 1) tps = 1;
    ns = (tiles + tps - 1) / tps;
    if (ns < 1) ns = 1;
    return Plan{(int)ns, (int)tps};
}

int ce_of(int32_t dtype) { return dtype == LQ_KV_F32 ? 4 : 8; }

template <typename KV, int NP, int CPL, int GM, int VCPL>
void launch_split(dim3 grid, size_t shmem, hipStream_t s, const AttnArgs& a) {
    hipLaunchKernelGGL((k_attn_split<KV, NP, CPL, GM, VCPL>), grid, dim3(256), shmem, s, a);
}

using SplitFn = void (*)(dim3, size_t, hipStream_t, const AttnArgs&);

// Specialised (fast) shapes; everything else takes the generic instance.
struct Variant {
    int32_t dtype;
    int c;       // chunks per row (head_dim / CE)
    int gm;      // exact G
    SplitFn fn;
};

const Variant kVariants[] = {
    {LQ_KV_F32, 16, 2, launch_split<float, 8, 2, 2, 1>},         // head_dim 64, G 2
    {LQ_KV_F32, 16, 4, launch_split<float, 8, 2, 4, 1>},         // head_dim 64, G 4
    {LQ_KV_F32, 32, 4, launch_split<float, 16, 2, 4, 1>},        // head_dim 128, G 4
    {LQ_KV_BF16, 8, 2, launch_split<uint16_t, 8, 1, 2, 1>},      // head_dim 64, G 2
    {LQ_KV_BF16, 8, 4, launch_split<uint16_t, 8, 1, 4, 1>},      // head_dim 64, G 4
    {LQ_KV_BF16, 10, 2, launch_split<uint16_t, 8, 2, 2, 1>},     // head_dim 80, G 2
    {LQ_KV_BF16, 10, 4, launch_split<uint16_t, 8, 2, 4, 1>},     // head_dim 80, G 4
    {LQ_KV_BF16, 16, 2, launch_split<uint16_t, 8, 2, 2, 1>},     // head_dim 128, G 2
    {LQ_KV_BF16, 16, 4, launch_split<uint16_t, 8, 2, 4, 1>},     // head_dim 128, G 4
    {LQ_KV_BF16, 16, 8, launch_split<uint16_t, 16, 1, 8, 1>},    // head_dim 128, G 8
    {LQ_KV_BF16, 32, 2, launch_split<uint16_t, 8, 4, 2, 1>},     // head_dim 256, G 2
    {LQ_KV_BF16, 32, 4, launch_split<uint16_t, 16, 2, 4, 1>},    // head_dim 256, G 4
};

SplitFn pick(int32_t dtype, int64_t hd, int64_t G) {
    const int c = (int)(hd / ce_of(dtype));
    for (const Variant& v : kVariants)
        if (v.dtype == dtype && v.c == c && v.gm == G) return v.fn;
    // generic: one position per K step, up to 8 heads
    if (dtype == LQ_KV_F32) return launch_split<float, 64, 2, 8, 2>;
    return launch_split<uint16_t, 64, 1, 8, 1>;
}

}  // namespace

bool attn_supported(int64_t n_q, int64_t n_kv, int64_t hd, int32_t kv_dtype) {
    if (n_kv <= 0 || n_q % n_kv) return false;
    const int64_t G = n_q / n_kv;
    return G >= 1 && G <= 8 && hd > 0 && hd <= 512 && hd % ce_of(kv_dtype) == 0;
}

size_t attn_workspace_bytes(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len) {
    if (len <= 0 || n_kv <= 0) return 0;
    const Plan p = make_plan(n_kv, len);
    if (p.nsplit == 1) return 0;
    const int64_t slots = n_kv * p.nsplit * (n_q / n_kv);
    return (size_t)(slots * (hd + 2)) * sizeof(float);
}

lq_status launch_attention(const float* q, int64_t n_q, int64_t n_kv, int64_t hd, const void* kc,
                           const void* vc, int32_t kv_dtype, int64_t head_stride,
                           int64_t pos_stride, int64_t start, int64_t len, float scale,
                           float* out, void* ws, hipStream_t s) {
    if (n_q == 0) return LQ_OK;
    if (len == 0) {
        const int64_t n = n_q * hd;
        hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256),
                           0, s, out, n);
        return check_launch("attention(len=0)");
    }
    const int64_t G = n_q / n_kv;
    const Plan p = make_plan(n_kv, len);
    AttnArgs a{};
    a.q = q; a.kc = kc; a.vc = vc; a.out = out;
    a.head_stride = head_stride; a.pos_stride = pos_stride; a.start = start; a.len = len;
    a.hd = (int)hd; a.G = (int)G; a.nsplit = p.nsplit; a.tiles_per_split = p.tiles_per_split;
    a.qscale = scale * kLog2e;
    const int64_t slots = n_kv * p.nsplit * G;
    if (p.nsplit > 1) {
        float* f = static_cast<float*>(ws);
        a.part_m = f;
        a.part_l = f + slots;
        a.part_acc = f + 2 * slots;
    }
    SplitFn fn = pick(kv_dtype, hd, G);
    fn(dim3((unsigned)p.nsplit, (unsigned)n_kv), 0, s, a);
    lq_status st = check_launch("attention split");
    if (st != LQ_OK || p.nsplit == 1) return st;
    const int64_t n = n_q * hd;
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n_q);
    return check_launch("attention combine");
}

}  // namespace lq

using namespace lq;

extern "C" size_t lq_gqa_decode_attn_workspace_size(int64_t n_q, int64_t n_kv, int64_t head_dim,
                                                    int64_t len) {
    if (n_q <= 0 || n_kv <= 0 || head_dim <= 0 || len <= 0 || n_q % n_kv) return 0;
    return attn_workspace_bytes(n_q, n_kv, head_dim, len);
}

extern "C" lq_status lq_gqa_decode_attn(const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                                        const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                        int64_t head_stride, int64_t pos_stride, int64_t max_ctx,
                                        int64_t start, int64_t len, float scale, float* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "lq_gqa_decode_attn";
    if (n_q < 0 || n_kv <= 0 || head_dim <= 0 || (n_q % n_kv) || head_dim % 4)
        return fail(LQ_ERR_SHAPE, "%s: n_q=%lld n_kv=%lld head_dim=%lld (need n_q %% n_kv == 0, head_dim %% 4 == 0)",
                    fn, (long long)n_q, (long long)n_kv, (long long)head_dim);
    if (kv_dtype != LQ_KV_F32 && kv_dtype != LQ_KV_BF16)
        return fail(LQ_ERR_SHAPE, "%s: kv_dtype %d", fn, kv_dtype);
    if (start < 0 || len < 0 || max_ctx < 0 || start + len > max_ctx)
        return fail(LQ_ERR_SHAPE, "%s: window [%lld, %lld) outside [0, %lld)", fn, (long long)start,
                    (long long)(start + len), (long long)max_ctx);
    if (pos_stride < head_dim || head_stride < 0)
        return fail(LQ_ERR_SHAPE, "%s: pos_stride=%lld head_stride=%lld", fn, (long long)pos_stride,
                    (long long)head_stride);
    if (!attn_supported(n_q == 0 ? n_kv : n_q, n_kv, head_dim, kv_dtype))
        return fail(LQ_ERR_UNSUPPORTED, "%s: head_dim=%lld G=%lld dtype=%d not built (head_dim <= 512, G <= 8, "
                    "bf16 head_dim %% 8 == 0)", fn, (long long)head_dim, (long long)(n_q / n_kv), kv_dtype);
    if (n_q == 0) return LQ_OK;
    if (!q || !out || (len > 0 && (!k_cache || !v_cache))) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    const size_t es = kv_dtype == LQ_KV_F32 ? 4 : 2;
    if (len > 0 && (!aligned(k_cache, 16) || !aligned(v_cache, 16) || (pos_stride * es) % 16 ||
                    (head_stride * es) % 16))
        return fail(LQ_ERR_ALIGN, "%s: caches and strides must be 16-byte aligned", fn);
    if (!aligned(q, 4) || !aligned(out, 4)) return fail(LQ_ERR_ALIGN, "%s: q/out misaligned", fn);
    const size_t need = attn_workspace_bytes(n_q, n_kv, head_dim, len);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn, need,
                    workspace_bytes);
    if (n_kv > 65535) return fail(LQ_ERR_UNSUPPORTED, "%s: too many kv heads", fn);
    return launch_attention(q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride, start,
                            len, scale, out, workspace, as_stream(stream));
}

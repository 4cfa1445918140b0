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
//   * grid = (splits, n_kv).  A workgroup of 4 waves owns one kv head and a
//     range of positions; each wave takes TILE-position tiles.  All G query
//     heads of the kv head are served from one read of K and V.
//   * The first tile's K and V loads are issued before anything else, so
//     HBM latency overlaps the prologue.  In the decode layer the prologue
//     also does the per-head q/k RMSNorm + NeoX RoPE of the raw projection,
//     the unit norm of v, and appends k and v at the new position ("Current
//     Inference Path -- Architecture Map", section 3 steps b; the kv-cache
//     append of section 1), so no separate launch is needed for them.
//   * K phase: NP consecutive lanes share one position; each lane holds the
//     (pre-scaled) query slice of its 16-byte chunks for all G heads in VGPRs,
//     does CE*G FMAs per 16-byte K load, and the NP partial dots are summed
//     with DPP / permlane group reductions.  Scores go to LDS.
//   * softmax: one lane per position of the tile; running max per head is a
//     wave max, probabilities are exp2 of pre-scaled scores (log2(e) folded
//     into q); the running sum stays per lane until the end.
//   * V phase: VC lanes per position read 16-byte V chunks (coalesced rows)
//     and accumulate p * V for all G heads; p is broadcast from LDS.
//   * The next tile's K loads are issued before the softmax, its V loads
//     before the next K phase.
//   * end: the waves' (m, l, acc) are combined in LDS in a fixed order; with
//     one split the workgroup writes the normalised output, else a partial
//     that a second kernel rescales and sums over the splits.
#include <math.h>

#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

namespace {

constexpr int kWavesPerWG = 4;
constexpr int kRedFloats = 2048;   // per-wave LDS floats for the final combine
constexpr int kMaxSplitsC = 256;   // splits per kv head (the combine keeps their weights in LDS)
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
    const float* q;          // unfused: final q [n_q, hd]; fused: raw projection [n_q*hd + 2*n_kv*hd]
    const void* kc;
    void* vc_w;              // V cache (written at the new position when fused)
    void* kc_w;
    float* out;
    float* part_m;           // [n_kv][nsplit][G]
    float* part_l;
    float* part_acc;         // [n_kv][nsplit][G][hd]
    const float* g_q;        // fused prologue: per-head norm weights (NULL: no q/k norm)
    const float* g_k;
    const float* rope_cos;   // fused prologue: table rows at the new position
    const float* rope_sin;
    int64_t head_stride, pos_stride, start, len;
    int hd, G, n_q, n_kv, nsplit, tiles_per_split;
    int fused, qk_norm, v_unit_norm;
    float qscale;            // scale * log2(e)
    float eps;
};

}  // namespace

// One head vector of hd floats, by one wave: RMSNorm over the head (optional,
// weights gamma, or none for a unit norm), then NeoX RoPE (optional: element
// i pairs with i + hd/2 and uses the table entry of the lower index), times
// `scale`.  Lane l handles elements l + 64j; it reads the RoPE partner of
// each of its elements straight from `raw`, so lanes exchange nothing but the
// sum of squares.  The result goes to dst (LDS); when kv_dst is set it is
// also stored there as KV (a cache row), and dst then holds the stored value.
template <typename KV>
__device__ __forceinline__ void head_vec(const float* __restrict__ raw, const float* __restrict__ gamma,
                                         const float* __restrict__ cs, const float* __restrict__ sn, int hd,
                                         bool norm, bool rope, float eps, float scale, int lane, float* dst,
                                         KV* kv_dst) {
    constexpr int EPL = 8;                          // hd <= 512
    const int half = hd >> 1;
    float own[EPL], par[EPL];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int i = lane + 64 * j;
        own[j] = 0.0f;
        par[j] = 0.0f;
        if (i < hd) {
            own[j] = raw[i];
            if (rope) par[j] = raw[i < half ? i + half : i - half];
        }
        ss += own[j] * own[j];
    }
    float rinv = 1.0f;
    if (norm) rinv = 1.0f / sqrtf(wave_sum(ss) / (float)hd + eps);
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int i = lane + 64 * j;
        if (i < hd) {
            const bool first = i < half;
            const int pi = first ? i + half : i - half;
            const float av = own[j] * rinv * (gamma ? gamma[i] : 1.0f);
            float y = av;
            if (rope) {
                const float bv = par[j] * rinv * (gamma ? gamma[pi] : 1.0f);
                const int t = first ? i : pi;
                y = first ? av * cs[t] - bv * sn[t] : bv * sn[t] + av * cs[t];
            }
            y *= scale;
            if (kv_dst) {
                if constexpr (sizeof(KV) == 4) {
                    kv_dst[i] = y;
                } else {
                    const uint32_t b = f32_to_bf16(y);
                    kv_dst[i] = (KV)b;
                    y = bf16_to_f32(b);
                }
            }
            dst[i] = y;
        }
    }
}

// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Raw buffer resource over [base, base + bytes): a load at a byte offset at or
// beyond `bytes` returns zeros instead of touching memory, so bounds need no
// branches (gfx9 descriptor word 3).
constexpr uint32_t kOob = 0x80000000u;   // offset that is always out of range (bytes < 2^31)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ int4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_int4((int)v[0], (int)v[1], (int)v[2], (int)v[3]);
}

// One split of the positions of one kv head, all G query heads of it.
//   KV: float or uint16_t (bf16).  CM: chunks (16 bytes) per row at most, so
//   head_dim <= CM * CE; GM: query heads per kv head at most; NP: lanes per
//   position in the K phase; TILE: positions per wave iteration.
// The loops run over CM and GM; rows shorter than CM chunks load zeros past
// their end and query heads past G are zero, so exact shapes (CM*CE ==
// head_dim, GM == G) do no wasted work and padded ones stay correct.
template <typename KV, int CM, int GM, int NP, int TILE>
__global__ __launch_bounds__(256, 2) void k_attn_split(AttnArgs a) {
    constexpr int CE = KvTraits<KV>::CE;
    constexpr int HDM = CM * CE;                  // largest head_dim
    constexpr int CPL = (CM + NP - 1) / NP;       // K chunks per lane
    constexpr int TP = kWave / NP;                // positions per K step
    constexpr int KSTEPS = TILE / TP;
    constexpr int VC = CM < 64 ? CM : 64;         // V lanes per position
    constexpr int VTP = kWave / VC;               // positions per V step
    constexpr int VCPL = (CM + 63) / 64;          // V chunks per lane
    constexpr int VSTEPS = (TILE + VTP - 1) / VTP;
    static_assert(TILE % TP == 0 && TILE <= 64 && HDM <= 512 && GM <= 8, "tile shape");
    constexpr int RED = kWavesPerWG * kRedFloats;

    __shared__ float sc[kWavesPerWG][TILE][GM];   // per wave: scores, then probabilities
    __shared__ float wm[kWavesPerWG][GM], wl[kWavesPerWG][GM];
    __shared__ __attribute__((aligned(16))) float q_lds[GM * HDM];
    __shared__ __attribute__((aligned(16))) float kv_new[2][HDM];     // new k and v rows, as stored
    __shared__ __attribute__((aligned(16))) float red[RED];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.y, split = blockIdx.x;
    const int hd = a.hd, G = a.G, C = hd / CE;
    const int64_t end = a.start + a.len;
    const int64_t ps0 = a.start + (int64_t)split * a.tiles_per_split * TILE;
    const int64_t ps1 = ps0 + (int64_t)a.tiles_per_split * TILE < end ? ps0 + (int64_t)a.tiles_per_split * TILE : end;
    const int n_pos = (int)(ps1 - ps0);
    const int n_tiles = (n_pos + TILE - 1) / TILE;
    const int64_t pos_new = a.fused ? end - 1 : -1;
    const int lp_new = (pos_new >= ps0 && pos_new < ps1) ? (int)(pos_new - ps0) : -1;   // in this split
    const uint32_t pb = (uint32_t)(a.pos_stride * (int64_t)sizeof(KV));            // bytes per position
    const int64_t row0 = (int64_t)g * a.head_stride + ps0 * a.pos_stride;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const KV*>(a.kc) + row0, (uint32_t)n_pos * pb);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const KV*>(a.vc_w) + row0, (uint32_t)n_pos * pb);

    // per-lane byte offsets inside a tile (kOob for chunks past the row)
    const int kp = lane / NP, kk = lane % NP;
    uint32_t koff[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = kk + c * NP;
        koff[c] = ch < C ? (uint32_t)kp * pb + (uint32_t)ch * 16u : kOob;
    }
    const int vp = lane / VC, vk = lane % VC;
    uint32_t voff[VCPL];
#pragma unroll
    for (int c = 0; c < VCPL; ++c) {
        const int ch = vk + 64 * c;
        voff[c] = (vp < VTP && ch < C) ? (uint32_t)vp * pb + (uint32_t)ch * 16u : kOob;
    }

    auto load_k = [&](int t, int4 (&kr)[KSTEPS][CPL]) {
        const uint32_t base = (uint32_t)(t * TILE) * pb;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
            for (int c = 0; c < CPL; ++c) kr[st][c] = bload16(rk, koff[c] + base + (uint32_t)(st * TP) * pb);
    };
    auto load_v = [&](int t, int4 (&vr)[VSTEPS][VCPL]) {
        const uint32_t base = (uint32_t)(t * TILE) * pb;
#pragma unroll
        for (int st = 0; st < VSTEPS; ++st) {
            // a last, partial step must not reach into the next tile
            const bool in = (TILE % VTP == 0) || st * VTP + vp < TILE;
#pragma unroll
            for (int c = 0; c < VCPL; ++c)
                vr[st][c] = bload16(rv, (in ? voff[c] : kOob) + base + (uint32_t)(st * VTP) * pb);
        }
    };

    // ---- first tile in flight before the prologue
    int t = wave;
    int4 kr[KSTEPS][CPL];
    int4 vr[VSTEPS][VCPL];
    load_k(t, kr);
    load_v(t, vr);

    // ---- prologue, one head vector per wave at a time, into LDS: the query
    // heads of this kv head, pre-scaled by scale*log2(e).  In the decode
    // layer the raw projection is normalised and rotated here, and the
    // workgroup whose positions include the new one also builds the new k and
    // v rows and appends them to the caches.
    {
        const bool mine = lp_new >= 0;
        const int items = G + (mine ? 2 : 0);
        for (int it = wave; it < items; it += kWavesPerWG) {
            if (!a.fused) {
                head_vec<KV>(a.q + (int64_t)(g * G + it) * hd, nullptr, nullptr, nullptr, hd, false, false, 0.0f,
                             a.qscale, lane, q_lds + it * HDM, nullptr);
            } else if (it < G) {
                head_vec<KV>(a.q + (int64_t)(g * G + it) * hd, a.qk_norm ? a.g_q : nullptr, a.rope_cos, a.rope_sin,
                             hd, a.qk_norm, true, a.eps, a.qscale, lane, q_lds + it * HDM, nullptr);
            } else {
                const float* kraw = a.q + (int64_t)a.n_q * hd + (int64_t)g * hd;
                const int64_t row = (int64_t)g * a.head_stride + pos_new * a.pos_stride;
                if (it == G)
                    head_vec<KV>(kraw, a.qk_norm ? a.g_k : nullptr, a.rope_cos, a.rope_sin, hd, a.qk_norm, true,
                                 a.eps, 1.0f, lane, kv_new[0], static_cast<KV*>(a.kc_w) + row);
                else
                    head_vec<KV>(kraw + (int64_t)a.n_kv * hd, nullptr, nullptr, nullptr, hd, a.v_unit_norm, false,
                                 a.eps, 1.0f, lane, kv_new[1], static_cast<KV*>(a.vc_w) + row);
            }
        }
        // zero the padding: query heads past G, dims past head_dim
        for (int i = threadIdx.x; i < GM * HDM; i += 256)
            if (i / HDM >= G || i % HDM >= hd) q_lds[i] = 0.0f;
    }
    __syncthreads();
    float qr[GM][CPL][CE];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const int ch = kk + c * NP < CM ? kk + c * NP : 0;    // chunks past CM load zeros from K
#pragma unroll
            for (int e4 = 0; e4 < CE / 4; ++e4) {
                const float4 v = *reinterpret_cast<const float4*>(q_lds + h * HDM + ch * CE + 4 * e4);
                qr[h][c][4 * e4] = v.x; qr[h][c][4 * e4 + 1] = v.y;
                qr[h][c][4 * e4 + 2] = v.z; qr[h][c][4 * e4 + 3] = v.w;
            }
        }

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

    for (; t < n_tiles; t += kWavesPerWG) {
        const int lp0 = t * TILE;                        // first position of the tile, split-local
        const int next = t + kWavesPerWG;
        const int pt_new = (lp_new >= lp0 && lp_new < lp0 + TILE) ? lp_new - lp0 : -1;

        // ---- K phase: scores of the tile
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
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
#pragma unroll
                for (int h = 0; h < GM; ++h) sc[wave][st * TP + kp][h] = part[h];
            }
        }
        if (next < n_tiles) load_k(next, kr);
        if (pt_new >= 0) {
            // the new position: its k row comes from LDS (the cache row was
            // loaded before it was written)
            float sn[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) sn[h] = 0.0f;
            for (int d = lane; d < hd; d += kWave) {
                const float kd = kv_new[0][d];
#pragma unroll
                for (int h = 0; h < GM; ++h) sn[h] = fmaf(q_lds[h * HDM + d], kd, sn[h]);
            }
#pragma unroll
            for (int h = 0; h < GM; ++h) sn[h] = wave_sum(sn[h]);
            if (lane == 0) {
#pragma unroll
                for (int h = 0; h < GM; ++h) sc[wave][pt_new][h] = sn[h];
            }
        }
        wave_lds_sync();

        // ---- softmax over the tile, lane = position
        float alpha[GM], pn[GM];
        {
            const bool ok = lane < TILE && lp0 + lane < n_pos;
#pragma unroll
            for (int h = 0; h < GM; ++h) {
                const float s = ok ? sc[wave][lane < TILE ? lane : 0][h] : -INFINITY;
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
                pn[h] = pt_new >= 0 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), pt_new)) : 0.0f;
                // the new position's V term is added from LDS below
                if (lane < TILE) sc[wave][lane][h] = (lane == pt_new) ? 0.0f : p;
            }
        }
        wave_lds_sync();

        // ---- V phase: acc = acc * alpha + sum_j p_j V_j
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
            for (int c = 0; c < VCPL; ++c)
#pragma unroll
                for (int e = 0; e < CE; ++e) acc[h][c][e] *= alpha[h];
#pragma unroll
        for (int st = 0; st < VSTEPS; ++st) {
            const int pt = st * VTP + vp < TILE ? st * VTP + vp : TILE - 1;   // lanes past the tile load zeros
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
        if (pt_new >= 0 && vp == 0) {
#pragma unroll
            for (int c = 0; c < VCPL; ++c) {
                const int ch = vk + 64 * c;
                if (ch < C) {
#pragma unroll
                    for (int e = 0; e < CE; ++e) {
                        const float vd = kv_new[1][ch * CE + e];
#pragma unroll
                        for (int h = 0; h < GM; ++h) acc[h][c][e] = fmaf(pn[h], vd, acc[h][c][e]);
                    }
                }
            }
        }
        if (next < n_tiles) load_v(next, vr);
        wave_lds_sync();                 // this tile's probabilities are read before the next overwrite
    }

    // ---- combine the waves of this workgroup (fixed order: waves, then
    // position groups), in chunks of heads that fit the LDS buffer
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        const float ls = wave_sum(l[h]);
        if (lane == 0) {
            wm[wave][h] = m[h];
            wl[wave][h] = ls;
        }
    }
    constexpr int per_head = VTP * HDM;
    constexpr int HC = kRedFloats / per_head >= 1 ? kRedFloats / per_head : 1;
    static_assert(per_head <= kRedFloats, "combine buffer");
    for (int h0 = 0; h0 < G; h0 += HC) {
        const int h1 = h0 + HC < G ? h0 + HC : G;
        if (vp < VTP) {
#pragma unroll
            for (int h = 0; h < GM; ++h)
                if (h >= h0 && h < h1) {
#pragma unroll
                    for (int c = 0; c < VCPL; ++c) {
                        const int ch = vk + 64 * c;
                        if (ch < CM)
#pragma unroll
                            for (int e4 = 0; e4 < CE / 4; ++e4)
                                *reinterpret_cast<float4*>(
                                    &red[wave * kRedFloats + ((h - h0) * VTP + vp) * HDM + ch * CE + 4 * e4]) =
                                    make_float4(acc[h][c][4 * e4], acc[h][c][4 * e4 + 1], acc[h][c][4 * e4 + 2],
                                                acc[h][c][4 * e4 + 3]);
                    }
                }
        }
        __syncthreads();
        const int n_el = (h1 - h0) * hd;
        for (int idx = threadIdx.x; idx < n_el; idx += 256) {
            const int hh = idx / hd, d = idx - hh * hd, h = h0 + hh;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, wm[w][h]);
            float L = 0.0f, S = 0.0f;
#pragma unroll
            for (int w = 0; w < kWavesPerWG; ++w) {
                const float ew = (wm[w][h] == -INFINITY) ? 0.0f : exp2f(wm[w][h] - M);
                float sw = 0.0f;
#pragma unroll
                for (int v = 0; v < VTP; ++v) sw += red[w * kRedFloats + (hh * VTP + v) * HDM + d];
                L += ew * wl[w][h];
                S += ew * sw;
            }
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
        __syncthreads();
    }
}

// Rescale and sum the split partials.  One wave per (query head, 64 dims):
// lane s reads the split maxima, the wave forms the split weights
// exp2(m_s - M) and the total L once, then every lane sums its dim over the
// splits with 16 loads in flight.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
    __shared__ float wts[kWavesPerWG][kMaxSplitsC];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int chunks = (a.hd + 63) / 64;
    const int unit = blockIdx.x * kWavesPerWG + wave;
    if (unit >= a.n_q * chunks) return;
    const int hq = unit / chunks, d = (unit - hq * chunks) * 64 + lane;
    const int g = hq / a.G, h = hq - g * a.G;
    const int S = a.nsplit, G = a.G, hd = a.hd;
    const int64_t base = (int64_t)g * S * G + h;          // slot of split s = base + s*G
    float M = -INFINITY;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, a.part_m[base + (int64_t)s * G]);
    M = wave_max(M);
    float L = 0.0f;
    for (int s = lane; s < S; s += 64) {
        const float ms = a.part_m[base + (int64_t)s * G];
        const float e = (ms == -INFINITY) ? 0.0f : exp2f(ms - M);
        wts[wave][s] = e;
        L += e * a.part_l[base + (int64_t)s * G];
    }
    L = wave_sum(L);
    wave_lds_sync();
    if (d >= hd) return;
    const float* acc = a.part_acc + base * hd + d;
    const int64_t stride = (int64_t)G * hd;
    float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int s = 0;
    for (; s + 16 <= S; s += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = acc[(int64_t)(s + u) * stride];
#pragma unroll
        for (int u = 0; u < 16; ++u) sum[u & 3] = fmaf(wts[wave][s + u], v[u], sum[u & 3]);
    }
    for (; s < S; ++s) sum[0] = fmaf(wts[wave][s], acc[(int64_t)s * stride], sum[0]);
    a.out[(int64_t)hq * hd + d] = ((sum[0] + sum[1]) + (sum[2] + sum[3])) / L;
}

__global__ void k_fill_zero(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// ---- host side ------------------------------------------------------------

namespace {

struct Plan {
    int nsplit, tiles_per_split;
};

constexpr int kTargetWGs = 512;    // two workgroups of 4 waves per CU
constexpr int kMaxSplits = kMaxSplitsC;

using SplitFn = void (*)(dim3, hipStream_t, const AttnArgs&, LaunchMarks*);

struct Variant {
    int32_t dtype;
    int c;       // chunks per row (head_dim / CE), exact
    int g;       // G, exact
    int tile;
    SplitFn fn;
};

template <typename KV, int CM, int GM, int NP, int TILE>
void launch_split(dim3 grid, hipStream_t s, const AttnArgs& a, LaunchMarks* mk) {
    launch_marked(mk, k_attn_split<KV, CM, GM, NP, TILE>, grid, dim3(256), 0, s, a);
}

// Exact shapes of the common models; <KV, chunks, G, lanes per position, tile>.
const Variant kVariants[] = {
    {LQ_KV_F32, 16, 2, 32, launch_split<float, 16, 2, 8, 32>},          // head_dim 64
    {LQ_KV_F32, 16, 4, 32, launch_split<float, 16, 4, 8, 32>},
    {LQ_KV_F32, 32, 4, 16, launch_split<float, 32, 4, 16, 16>},         // head_dim 128
    {LQ_KV_BF16, 8, 2, 32, launch_split<uint16_t, 8, 2, 8, 32>},        // head_dim 64
    {LQ_KV_BF16, 8, 4, 32, launch_split<uint16_t, 8, 4, 8, 32>},
    {LQ_KV_BF16, 10, 2, 32, launch_split<uint16_t, 10, 2, 8, 32>},      // head_dim 80
    {LQ_KV_BF16, 10, 4, 32, launch_split<uint16_t, 10, 4, 8, 32>},
    {LQ_KV_BF16, 16, 2, 32, launch_split<uint16_t, 16, 2, 8, 32>},      // head_dim 128
    {LQ_KV_BF16, 16, 4, 32, launch_split<uint16_t, 16, 4, 8, 32>},
    {LQ_KV_BF16, 16, 8, 16, launch_split<uint16_t, 16, 8, 16, 16>},
    {LQ_KV_BF16, 32, 2, 16, launch_split<uint16_t, 32, 2, 16, 16>},     // head_dim 256
    {LQ_KV_BF16, 32, 4, 16, launch_split<uint16_t, 32, 4, 16, 16>},
    {LQ_KV_BF16, 64, 8, 8, launch_split<uint16_t, 64, 8, 64, 8>},       // head_dim 512
};

int ce_of(int32_t dtype) { return dtype == LQ_KV_F32 ? 4 : 8; }

struct Pick {
    SplitFn fn;
    int tile;
};

Pick pick(int32_t dtype, int64_t hd, int64_t G) {
    const int c = (int)(hd / ce_of(dtype));
    for (const Variant& v : kVariants)
        if (v.dtype == dtype && v.c == c && v.g == G) return Pick{v.fn, v.tile};
    // any head_dim <= 512 and G <= 8: padded loops, one position per K step
    if (dtype == LQ_KV_F32) return Pick{launch_split<float, 128, 8, 64, 4>, 4};
    return Pick{launch_split<uint16_t, 64, 8, 64, 8>, 8};
}

Plan make_plan(int64_t n_kv, int64_t len, int tile) {
    const int64_t tiles = (len + tile - 1) / tile;
    int64_t ns = (kTargetWGs + n_kv - 1) / n_kv;
    const int64_t by_tiles = (tiles + kWavesPerWG - 1) / kWavesPerWG;   // every wave gets a tile
    if (ns > by_tiles) ns = by_tiles;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    int64_t tps = (tiles + ns - 1) / ns;
    tps = (tps + kWavesPerWG - 1) / kWavesPerWG * kWavesPerWG;        // whole tiles per wave
    ns = (tiles + tps - 1) / tps;
    if (ns < 1) ns = 1;
    return Plan{(int)ns, (int)tps};
}

}  // namespace

bool attn_supported(int64_t n_q, int64_t n_kv, int64_t hd, int32_t kv_dtype) {
    if (n_kv <= 0 || n_q % n_kv) return false;
    const int64_t G = n_q / n_kv;
    return G >= 1 && G <= 8 && hd > 0 && hd <= 512 && hd % ce_of(kv_dtype) == 0 && hd % 4 == 0;
}

static size_t ws_bytes_for(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len, int32_t dtype) {
    if (len <= 0 || n_kv <= 0) return 0;
    const Plan p = make_plan(n_kv, len, pick(dtype, hd, n_q / n_kv).tile);
    if (p.nsplit == 1) return 0;
    const int64_t slots = n_kv * p.nsplit * (n_q / n_kv);
    return (size_t)(slots * (hd + 2)) * sizeof(float);
}

size_t attn_workspace_bytes(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len) {
    // the larger of the two dtypes' plans, so one query serves both
    const size_t a = ws_bytes_for(n_q, n_kv, hd, len, LQ_KV_F32);
    const size_t b = hd % 8 == 0 ? ws_bytes_for(n_q, n_kv, hd, len, LQ_KV_BF16) : 0;
    return a > b ? a : b;
}

static lq_status launch_common(AttnArgs& a, int64_t n_q, int64_t n_kv, int64_t hd, int32_t kv_dtype,
                               void* ws, hipStream_t s, LaunchMarks* marks = nullptr) {
    const int64_t G = n_q / n_kv;
    const Pick pk = pick(kv_dtype, hd, G);
    const Plan p = make_plan(n_kv, a.len, pk.tile);
    // buffer offsets inside one split stay below 2^31 bytes
    const int64_t es = kv_dtype == LQ_KV_F32 ? 4 : 2;
    if (((int64_t)p.tiles_per_split * pk.tile + 64) * a.pos_stride * es >= (int64_t(1) << 31))
        return fail(LQ_ERR_UNSUPPORTED, "attention: %lld positions of %lld bytes in one split exceed 2 GiB",
                    (long long)p.tiles_per_split * pk.tile, (long long)(a.pos_stride * es));
    a.hd = (int)hd; a.G = (int)G; a.n_q = (int)n_q; a.n_kv = (int)n_kv;
    a.nsplit = p.nsplit; a.tiles_per_split = p.tiles_per_split;
    const int64_t slots = n_kv * p.nsplit * G;
    if (p.nsplit > 1) {
        float* f = static_cast<float*>(ws);
        a.part_m = f;
        a.part_l = f + slots;
        a.part_acc = f + 2 * slots;
    }
    pk.fn(dim3((unsigned)p.nsplit, (unsigned)n_kv), s, a, marks);
    lq_status st = check_launch("attention split");
    if (st != LQ_OK || p.nsplit == 1) return st;
    const int units = (int)(n_q * ((hd + 63) / 64));
    launch_marked(marks, k_attn_combine, dim3((unsigned)((units + kWavesPerWG - 1) / kWavesPerWG)), dim3(256), 0,
                  s, a);
    return check_launch("attention combine");
}

lq_status launch_attention(const float* q, int64_t n_q, int64_t n_kv, int64_t hd, const void* kc,
                           const void* vc, int32_t kv_dtype, int64_t head_stride,
                           int64_t pos_stride, int64_t start, int64_t len, float scale,
                           float* out, void* ws, hipStream_t s) {
    if (n_q == 0) return LQ_OK;
    if (len == 0) {
        const int64_t n = n_q * hd;
        const int64_t grid = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
        hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)grid), dim3(256), 0, s, out, n);
        return check_launch("attention(len=0)");
    }
    AttnArgs a{};
    a.q = q; a.kc = kc; a.vc_w = const_cast<void*>(vc); a.out = out;
    a.head_stride = head_stride; a.pos_stride = pos_stride; a.start = start; a.len = len;
    a.qscale = scale * kLog2e;
    return launch_common(a, n_q, n_kv, hd, kv_dtype, ws, s);
}

lq_status launch_attention_fused(const float* qkv, int64_t n_q, int64_t n_kv, int64_t hd, const float* g_q,
                                 const float* g_k, int32_t qk_norm, int32_t v_unit_norm, float eps,
                                 const float* rope_cos_row, const float* rope_sin_row, void* kc, void* vc,
                                 int32_t kv_dtype, int64_t head_stride, int64_t pos_stride, int64_t start,
                                 int64_t len, float scale, float* out, void* ws, hipStream_t s,
                                 LaunchMarks* marks) {
    AttnArgs a{};
    a.q = qkv; a.kc = kc; a.kc_w = kc; a.vc_w = vc; a.out = out;
    a.g_q = g_q; a.g_k = g_k; a.rope_cos = rope_cos_row; a.rope_sin = rope_sin_row;
    a.head_stride = head_stride; a.pos_stride = pos_stride; a.start = start; a.len = len;
    a.fused = 1; a.qk_norm = qk_norm; a.v_unit_norm = v_unit_norm; a.eps = eps;
    a.qscale = scale * kLog2e;
    return launch_common(a, n_q, n_kv, hd, kv_dtype, ws, s, marks);
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

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

#include <type_traits>

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
    float cap2;              // score softcap times log2(e) (scores are kept in the log2 domain); 0: none
    float eps;
    float* tap_post;         // fused prologue, optional: q, k, v heads after norm / RoPE, before the
                             // attention scale and the cache conversion [n_q*hd + 2*n_kv*hd]
};

// The split kernel's arguments one by one, the ones its first loads need
// leading (the query/projection rows, the caches and the window): the
// compiler preloads the first 16 dwords into SGPRs at dispatch, so no wave
// waits for the kernel-argument buffer before its first load.
#define LQ_ATTN_PARAMS                                                                                      \
    const float *p_q, const void *p_kc, void *p_vc_w, void *p_kc_w, int64_t p_head_stride,                   \
        int64_t p_pos_stride, int64_t p_start, int64_t p_len, float *p_out, float *p_part_m, float *p_part_l, \
        float *p_part_acc, const float *p_g_q, const float *p_g_k, const float *p_rope_cos,                  \
        const float *p_rope_sin, int p_hd, int p_G, int p_n_q, int p_n_kv, int p_nsplit,                     \
        int p_tiles_per_split, int p_fused, int p_qk_norm, int p_v_unit_norm, float p_qscale, float p_cap2,   \
        float p_eps, float *p_tap_post
#define LQ_ATTN_FIELDS(A)                                                                                   \
    (A).q, (A).kc, (A).vc_w, (A).kc_w, (A).head_stride, (A).pos_stride, (A).start, (A).len, (A).out,         \
        (A).part_m, (A).part_l, (A).part_acc, (A).g_q, (A).g_k, (A).rope_cos, (A).rope_sin, (A).hd, (A).G,   \
        (A).n_q, (A).n_kv, (A).nsplit, (A).tiles_per_split, (A).fused, (A).qk_norm, (A).v_unit_norm,        \
        (A).qscale, (A).cap2, (A).eps, (A).tap_post
#define LQ_ATTN_REBUILD                                                                                      \
    AttnArgs a{p_q, p_kc, p_vc_w, p_kc_w, p_out, p_part_m, p_part_l, p_part_acc, p_g_q, p_g_k, p_rope_cos,   \
               p_rope_sin, p_head_stride, p_pos_stride, p_start, p_len, p_hd, p_G, p_n_q, p_n_kv, p_nsplit,   \
               p_tiles_per_split, p_fused, p_qk_norm, p_v_unit_norm, p_qscale, p_cap2, p_eps, p_tap_post}

}  // namespace

// The prologue's head vectors, by one wave each: RMSNorm over the head
// (optional, weights gamma, or none for a unit norm), then NeoX RoPE
// (optional: element i pairs with i + hd/2 and uses the table entry of the
// lower index), times `scale`.  Lane l handles elements l + 64j and reads the
// RoPE partner of each straight from the source, so lanes exchange nothing
// but the sum of squares.  Loading and computing are separate so the loads
// can be issued before the wave's K/V loads (the vector memory counter
// retires loads in order).
struct HeadSrc {
    const float* raw;
    const float* gamma;   // NULL: no weights
    bool norm, rope;
    float scale;
};

template <int EPL>
struct HeadIn {
    float own[EPL], par[EPL], ga[EPL], gb[EPL], cs[EPL], sn[EPL];   // as loaded
};

// Issues the loads only: every load comes from a valid address (absent
// tables are replaced by the source row, elements past hd by element 0) and
// the values are selected in head_finish, so nothing here waits on them.
template <int EPL>
__device__ __forceinline__ void head_load(HeadIn<EPL>& in, const HeadSrc& h, const float* __restrict__ cs,
                                          const float* __restrict__ sn, int hd, int lane) {
    const int half = hd >> 1;
    const float* gp = h.gamma ? h.gamma : h.raw;
    const float* cp = h.rope ? cs : h.raw;
    const float* sp = h.rope ? sn : h.raw;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int i0 = lane + 64 * j;
        const int i = i0 < hd ? i0 : 0;
        const bool first = i < half;
        const int pi = first ? i + half : i - half;
        const int t = first ? i : pi;
        in.own[j] = h.raw[i];
        in.par[j] = h.raw[pi];
        in.ga[j] = gp[i];
        in.gb[j] = gp[pi];
        in.cs[j] = cp[t];
        in.sn[j] = sp[t];
    }
}

// Writes the head to dst (LDS); with kv_dst also stores it as KV (a cache
// row), and dst then holds the stored value.
template <typename KV, int EPL>
__device__ __forceinline__ void head_finish(const HeadIn<EPL>& in, const HeadSrc& h, int hd, float eps, int lane,
                                            float* dst, KV* kv_dst, float* tap) {
    const int half = hd >> 1;
    const bool wg = h.gamma != nullptr;
    float own[EPL];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        own[j] = lane + 64 * j < hd ? in.own[j] : 0.0f;
        ss += own[j] * own[j];
    }
    float rinv = 1.0f;
    if (h.norm) rinv = 1.0f / sqrtf(wave_sum(ss) / (float)hd + eps);
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int i = lane + 64 * j;
        if (i < hd) {
            const float av = own[j] * rinv * (wg ? in.ga[j] : 1.0f);
            float y = av;
            if (h.rope) {
                const float bv = in.par[j] * rinv * (wg ? in.gb[j] : 1.0f);
                y = i < half ? av * in.cs[j] - bv * in.sn[j] : bv * in.sn[j] + av * in.cs[j];
            }
            if (tap) tap[i] = y;
            y *= h.scale;
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

// Contiguous form, for head_dim == 64 * EPL: lane l owns elements
// [l*EPL, (l+1)*EPL), read and written with vector accesses (16-byte aligned
// rows), and the RoPE partner of each element (i +- head_dim/2) is the same
// element of lane l ^ 32, fetched with a cross-half lane swap instead of a
// second load; both halves use the table entries of lane l & 31.
template <int EPL>
struct HeadInV {
    float own[EPL], ga[EPL], cs[EPL], sn[EPL];
};

template <int N>
__device__ __forceinline__ void load_run(float (&d)[N], const float* __restrict__ p) {
    if constexpr (N == 1) {
        d[0] = p[0];
    } else if constexpr (N == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        d[0] = v.x; d[1] = v.y;
    } else {
        static_assert(N % 4 == 0, "run length");
#pragma unroll
        for (int j = 0; j < N; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + j);
            d[j] = v.x; d[j + 1] = v.y; d[j + 2] = v.z; d[j + 3] = v.w;
        }
    }
}

template <int N>
__device__ __forceinline__ void store_run(float* p, const float (&d)[N]) {
    if constexpr (N == 1) {
        p[0] = d[0];
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(d[0], d[1]);
    } else {
#pragma unroll
        for (int j = 0; j < N; j += 4) *reinterpret_cast<float4*>(p + j) = make_float4(d[j], d[j + 1], d[j + 2], d[j + 3]);
    }
}

// the value of v held by lane ^ 32
__device__ __forceinline__ float half_swap(float v, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

template <int EPL>
__device__ __forceinline__ void head_load_v(HeadInV<EPL>& in, const HeadSrc& h, const float* __restrict__ cs,
                                            const float* __restrict__ sn, int lane) {
    const int i0 = lane * EPL, t0 = (lane & 31) * EPL;
    load_run<EPL>(in.own, h.raw + i0);
    load_run<EPL>(in.ga, (h.gamma ? h.gamma : h.raw) + i0);
    load_run<EPL>(in.cs, (h.rope ? cs : h.raw) + t0);
    load_run<EPL>(in.sn, (h.rope ? sn : h.raw) + t0);
}

template <typename KV, int EPL>
__device__ __forceinline__ void head_finish_v(const HeadInV<EPL>& in, const HeadSrc& h, float eps, int lane,
                                              float* dst, KV* kv_dst, float* tap) {
    constexpr int HD = 64 * EPL;
    const bool wg = h.gamma != nullptr;
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) ss += in.own[j] * in.own[j];
    float rinv = 1.0f;
    if (h.norm) rinv = 1.0f / sqrtf(wave_sum(ss) / (float)HD + eps);
    float y[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const float av = in.own[j] * rinv * (wg ? in.ga[j] : 1.0f);
        y[j] = av;
        if (h.rope) {
            const float bv = half_swap(av, lane);
            y[j] = lane < 32 ? av * in.cs[j] - bv * in.sn[j] : bv * in.sn[j] + av * in.cs[j];
        }
    }
    if (tap) store_run<EPL>(tap + lane * EPL, y);
#pragma unroll
    for (int j = 0; j < EPL; ++j) y[j] *= h.scale;
    if (kv_dst) {
        KV* row = kv_dst + lane * EPL;
        if constexpr (sizeof(KV) == 4) {
            store_run<EPL>(reinterpret_cast<float*>(row), y);
        } else {
            uint32_t b[EPL];
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                b[j] = f32_to_bf16(y[j]);
                y[j] = bf16_to_f32(b[j]);
            }
            if constexpr (EPL == 1) {
                row[0] = (KV)b[0];
            } else {
#pragma unroll
                for (int j = 0; j < EPL; j += 2) reinterpret_cast<uint32_t*>(row)[j / 2] = b[j] | (b[j + 1] << 16);
            }
        }
    }
    store_run<EPL>(dst + lane * EPL, y);
}

// Optional score softcap ("Inference Engine" (larql), BLAS-Fused Attention:
// the Gemma cap * tanh(score / cap) after the scaling), applied in the log2
// domain the kernel keeps its scores in: with c2 = cap * log2(e),
// c2 * tanh(u / c2) is log2(e) times the capped natural score.
__device__ __forceinline__ float soft_cap(float u, float c2) {
    return c2 > 0.0f ? c2 * tanhf(u / c2) : u;
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
// K and V rows are read once per call: nontemporal (aux bit 2), which streams
// long contexts about 10% faster than the default policy.
__device__ __forceinline__ int4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
    return make_int4((int)v[0], (int)v[1], (int)v[2], (int)v[3]);
}

// One split of the positions of one kv head, all G query heads of it.
//   KV: float or uint16_t (bf16).  CM: chunks (16 bytes) per row at most, so
//   head_dim <= CM * CE; GM: query heads per kv head at most; NP: lanes per
//   position in the K phase; TILE: positions per wave iteration; EX: the
//   shape is exact (head_dim == CM * CE, G == GM), known at compile time;
//   WPE: waves per SIMD the register budget is set for; NW: waves per
//   workgroup (more waves: fewer splits, so fewer partials to combine).
// Inexact shapes run the same loops over CM and GM: rows shorter than CM
// chunks load zeros past their end and query heads past G are zero.
template <typename KV, int CM, int GM, int NP, int TILE, bool EX, int WPE, int NW>
__global__ __launch_bounds__(NW * 64, WPE) void k_attn_split(LQ_ATTN_PARAMS) {
    LQ_ATTN_REBUILD;
    constexpr int NT = NW * 64;
    constexpr int CE = KvTraits<KV>::CE;
    constexpr int HDM = CM * CE;                  // largest head_dim
    constexpr int EPL = (HDM + 63) / 64;          // prologue elements per lane
    constexpr int CPL = (CM + NP - 1) / NP;       // K chunks per lane
    constexpr int TP = kWave / NP;                // positions per K step
    constexpr int KSTEPS = TILE / TP;
    constexpr int VC = CM < 64 ? CM : 64;         // V lanes per position
    constexpr int VTP = kWave / VC;               // positions per V step
    constexpr int VCPL = (CM + 63) / 64;          // V chunks per lane
    constexpr int VSTEPS = (TILE + VTP - 1) / VTP;
    // softmax: HPP heads side by side, TW lanes (>= TILE) per head
    constexpr int TW = TILE <= 4 ? 4 : TILE <= 8 ? 8 : TILE <= 16 ? 16 : TILE <= 32 ? 32 : 64;
    constexpr int HPP = kWave / TW < GM ? kWave / TW : GM;
    constexpr int NPASS = GM / HPP;
    static_assert(TILE % TP == 0 && TILE <= 64 && HDM <= 512 && GM <= 8 && GM % HPP == 0, "tile shape");
    constexpr int RED = NW * kRedFloats;

    __shared__ float sc[NW][TILE][GM];   // per wave: scores, then probabilities
    __shared__ float wm[NW][GM], wl[NW][GM];
    __shared__ __attribute__((aligned(16))) float q_lds[GM * HDM];
    __shared__ __attribute__((aligned(16))) float kv_new[2][HDM];     // new k and v rows, as stored
    __shared__ __attribute__((aligned(16))) float red[RED];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.y, split = blockIdx.x;
    const int hd = EX ? HDM : a.hd, G = EX ? GM : a.G, C = EX ? CM : hd / CE;
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

    // A tile past the split's end (t >= n_tiles) is still issued, at offsets
    // that are out of range (zeros, no memory access): the loads stay
    // unconditional, so each wait counts exactly the loads issued before it
    // (a branch around them would make the compiler wait for all of them).
    auto load_k = [&](int t, int4 (&kr)[KSTEPS][CPL]) {
        const bool live = t < n_tiles;
        const uint32_t base = (uint32_t)(t * TILE) * pb;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                kr[st][c] = bload16(rk, live ? koff[c] + base + (uint32_t)(st * TP) * pb : kOob);
    };
    auto load_v = [&](int t, int4 (&vr)[VSTEPS][VCPL]) {
        const bool live = t < n_tiles;
        const uint32_t base = (uint32_t)(t * TILE) * pb;
#pragma unroll
        for (int st = 0; st < VSTEPS; ++st) {
            // a last, partial step must not reach into the next tile
            const bool in = live && ((TILE % VTP == 0) || st * VTP + vp < TILE);
#pragma unroll
            for (int c = 0; c < VCPL; ++c)
                vr[st][c] = bload16(rv, in ? voff[c] + base + (uint32_t)(st * VTP) * pb : kOob);
        }
    };

    // ---- prologue items: the G query heads of this kv head (pre-scaled by
    // scale*log2(e)), then, in the workgroup whose split holds the new
    // position, its k and v rows: item j goes to wave j % NW.  In the decode
    // layer they are normalised and rotated here; the new k and v rows are
    // appended to the caches and kept in LDS, where the wave whose tile holds
    // the new position reads them back.
    const bool new_here = lp_new >= 0;
    const int n_qi = wave < G ? (G - wave + NW - 1) / NW : 0;
    const bool has_k = new_here && wave == G % NW, has_v = new_here && wave == (G + 1) % NW;
    const int n_items = n_qi + (has_k ? 1 : 0) + (has_v ? 1 : 0);
    // item i of this wave past its query heads: 0 = k, 1 = v
    auto kv_item = [&](int i) { return (has_k && i == n_qi) ? 0 : 1; };
    auto item_src = [&](int i) -> HeadSrc {
        if (i < n_qi) {
            const float* raw = a.q + (int64_t)(g * G + wave + NW * i) * hd;
            if (!a.fused) return HeadSrc{raw, nullptr, false, false, a.qscale};
            return HeadSrc{raw, a.qk_norm ? a.g_q : nullptr, a.qk_norm != 0, true, a.qscale};
        }
        const float* kraw = a.q + (int64_t)a.n_q * hd + (int64_t)g * hd;
        if (kv_item(i) == 0) return HeadSrc{kraw, a.qk_norm ? a.g_k : nullptr, a.qk_norm != 0, true, 1.0f};
        return HeadSrc{kraw + (int64_t)a.n_kv * hd, nullptr, a.v_unit_norm != 0, false, 1.0f};
    };
    // exact shapes with head_dim == 64 * EPL >= 256 use the contiguous form
    // (measured: for head_dim 128 the strided form is faster)
    constexpr bool VEC = EX && HDM == 64 * EPL && EPL >= 4;
    using HIn = std::conditional_t<VEC, HeadInV<EPL>, HeadIn<EPL>>;
    auto item_load = [&](HIn& in, const HeadSrc& src) {
        if constexpr (VEC) head_load_v<EPL>(in, src, a.rope_cos, a.rope_sin, lane);
        else head_load<EPL>(in, src, a.rope_cos, a.rope_sin, hd, lane);
    };
    auto item_fin = [&](const HIn& in, const HeadSrc& src, float* dst, KV* kv, float* tap) {
        if constexpr (VEC) head_finish_v<KV, EPL>(in, src, a.eps, lane, dst, kv, tap);
        else head_finish<KV, EPL>(in, src, hd, a.eps, lane, dst, kv, tap);
    };
    // the optional tap of the prologue's results: the query heads from split
    // 0 of each kv head, k and v from the workgroup that appends them
    auto item_run = [&](int i, const HIn& in, const HeadSrc& src) {
        if (i < n_qi) {
            const int h = wave + NW * i;
            float* tap = (a.tap_post && split == 0) ? a.tap_post + (int64_t)(g * G + h) * hd : nullptr;
            item_fin(in, src, q_lds + h * HDM, nullptr, tap);
        } else {
            const int64_t row = (int64_t)g * a.head_stride + pos_new * a.pos_stride;
            const int kv = kv_item(i);
            KV* cache = static_cast<KV*>(kv == 0 ? a.kc_w : a.vc_w);
            float* tap = a.tap_post ? a.tap_post + (int64_t)(a.n_q + kv * a.n_kv + g) * hd : nullptr;
            item_fin(in, src, kv_new[kv], cache + row, tap);
        }
    };

    // the items' inputs are read before the wave's first K/V tile (all of
    // them when they fit in registers), the tile before the items are
    // computed
    constexpr int MAXI = (GM + 2 + NW - 1) / NW;
    constexpr int EARLY = MAXI * (VEC ? 4 : 6) * EPL <= (VEC ? 160 : 72) ? MAXI : 1;
    HIn hin[EARLY];
    HeadSrc srcs[EARLY];
#pragma unroll
    for (int i = 0; i < EARLY; ++i) {
        if (i < n_items) {
            srcs[i] = item_src(i);
            item_load(hin[i], srcs[i]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);       // keep these loads ahead of the tile's
    int t = wave;
    int4 kr[KSTEPS][CPL];
    int4 vr[VSTEPS][VCPL];
    load_k(t, kr);
#pragma unroll
    for (int i = 0; i < EARLY; ++i)
        if (i < n_items) item_run(i, hin[i], srcs[i]);
    for (int i = EARLY; i < n_items; ++i) {
        const HeadSrc src = item_src(i);
        item_load(hin[0], src);
        item_run(i, hin[0], src);
    }
    if (!EX) {
        // zero the padding: query heads past G, dims past head_dim
        for (int i = threadIdx.x; i < GM * HDM; i += NT)
            if (i / HDM >= G || i % HDM >= hd) q_lds[i] = 0.0f;
    }
    __syncthreads();
    load_v(t, vr);
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

    // softmax state: lane (hs, sp) keeps head pass*HPP + hs
    const int hs = lane / TW, sp = lane % TW;
    float ms[NPASS], ls[NPASS], acc[GM][VCPL][CE];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        ms[ps] = -INFINITY;
        ls[ps] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int c = 0; c < VCPL; ++c)
#pragma unroll
            for (int e = 0; e < CE; ++e) acc[h][c][e] = 0.0f;

    for (; t < n_tiles; t += NW) {
        const int lp0 = t * TILE;                        // first position of the tile, split-local
        const int next = t + NW;
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
            if constexpr (NP == 64 && GM == 8) {
                // one position per step: reduce-scatter, lane group h holds head h
                const float sum = wave_sum8_scatter(part);
                if ((lane & 7) == 0) sc[wave][st][(lane >> 3) & 7] = soft_cap(sum, a.cap2);
            } else {
#pragma unroll
                for (int h = 0; h < GM; ++h) part[h] = group_sum<NP>(part[h]);
                if (kk == 0) {
#pragma unroll
                    for (int h = 0; h < GM; ++h) sc[wave][st * TP + kp][h] = soft_cap(part[h], a.cap2);
                }
            }
        }
        load_k(next, kr);
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
                for (int h = 0; h < GM; ++h) sc[wave][pt_new][h] = soft_cap(sn[h], a.cap2);
            }
        }
        wave_lds_sync();

        // ---- softmax over the tile: HPP heads at once, lane = (head, position)
        float alpha[GM], pn[GM];
        {
            const bool ok = hs < HPP && sp < TILE && lp0 + sp < n_pos;
            const int spc = sp < TILE ? sp : 0;
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                const int h = ps * HPP + (hs < HPP ? hs : 0);
                const float s = ok ? sc[wave][spc][h] : -INFINITY;
                const float mn = fmaxf(ms[ps], group_max<TW>(s));
                const bool live = mn != -INFINITY;
                const float al = live ? exp2f(ms[ps] - mn) : 1.0f;
                const float p = (ok && live) ? exp2f(s - mn) : 0.0f;
                ls[ps] = ls[ps] * al + p;
                ms[ps] = mn;
#pragma unroll
                for (int j = 0; j < HPP; ++j) {
                    alpha[ps * HPP + j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), j * TW));
                    pn[ps * HPP + j] = pt_new >= 0
                        ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), j * TW + pt_new)) : 0.0f;
                }
                // the new position's V term is added from LDS below
                if (hs < HPP && sp < TILE) sc[wave][sp][h] = (sp == pt_new) ? 0.0f : p;
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
        load_v(next, vr);
        wave_lds_sync();                 // this tile's probabilities are read before the next overwrite
    }

    // ---- combine the waves of this workgroup (fixed order: waves, then
    // position groups), in chunks of heads that fit the LDS buffer
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const float lsum = group_sum<TW>(ls[ps]);
        if (sp == 0 && hs < HPP) {
            wm[wave][ps * HPP + hs] = ms[ps];
            wl[wave][ps * HPP + hs] = lsum;
        }
    }
    // per head: the workgroup maximum, each wave's weight exp2(m_w - M) and
    // the weighted sum of the l's, once, before the per-element loop
    __shared__ float wf[NW][GM], hM[GM], hL[GM];
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w][h]);
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float ew = (wm[w][h] == -INFINITY) ? 0.0f : exp2f(wm[w][h] - M);
            wf[w][h] = ew;
            L += ew * wl[w][h];
        }
        hM[h] = M;
        hL[h] = L;
    }
    // A partial result per output element and wave: with 4 position groups
    // per V step, the wave first sums its groups across lanes (a
    // reduce-scatter over lane bits 5 and 4), leaving lane (vp, vk) the
    // values [vp*Q, (vp+1)*Q) of its chunk vk, then writes one [G][hd] slab.
    constexpr bool RS = VTP == 4 && GM % 4 == 0 && VCPL == 1 && CE == 8;
    if constexpr (RS) {
        constexpr int N = GM * CE, Q = N / 4;
        float hv[N / 2], qv[Q];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float lo = acc[i / CE][0][i % CE], hi = acc[(i + N / 2) / CE][0][(i + N / 2) % CE];
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
            hv[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(hv[i]), __float_as_uint(hv[i + Q]), false,
                                                            false);
            qv[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
        // qv[i] is element (vp*Q + i) % CE of head (vp*Q + i) / CE, chunk vk
        static_assert(GM * HDM <= kRedFloats, "combine buffer");
#pragma unroll
        for (int i = 0; i < Q; i += 4) {
            const int h = (vp * Q + i) / CE, e = (vp * Q + i) % CE;
            *reinterpret_cast<float4*>(&red[wave * kRedFloats + h * HDM + vk * CE + e]) =
                make_float4(qv[i], qv[i + 1], qv[i + 2], qv[i + 3]);
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < G * hd; idx += NT) {
            const int h = idx / hd, d = idx - h * hd;
            float S = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) S += wf[w][h] * red[w * kRedFloats + h * HDM + d];
            if (a.nsplit == 1) {
                a.out[(int64_t)(g * G + h) * hd + d] = S / hL[h];
            } else {
                const int64_t slot = ((int64_t)g * a.nsplit + split) * G + h;
                a.part_acc[slot * hd + d] = S;
                if (d == 0) {
                    a.part_m[slot] = hM[h];
                    a.part_l[slot] = hL[h];
                }
            }
        }
        return;
    }
    constexpr int per_head = VTP * HDM;
    constexpr int HC = kRedFloats / per_head < GM ? kRedFloats / per_head : GM;
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
        for (int idx = threadIdx.x; idx < n_el; idx += NT) {
            const int hh = idx / hd, d = idx - hh * hd, h = h0 + hh;
            float S = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                float sw = 0.0f;
#pragma unroll
                for (int v = 0; v < VTP; ++v) sw += red[w * kRedFloats + (hh * VTP + v) * HDM + d];
                S += wf[w][h] * sw;
            }
            if (a.nsplit == 1) {
                a.out[(int64_t)(g * G + h) * hd + d] = S / hL[h];
            } else {
                const int64_t slot = ((int64_t)g * a.nsplit + split) * G + h;
                a.part_acc[slot * hd + d] = S;
                if (d == 0) {
                    a.part_m[slot] = hM[h];
                    a.part_l[slot] = hL[h];
                }
            }
        }
        __syncthreads();
    }
}

// Rescale and sum the split partials: one workgroup per (query head, 64
// dims), wave w taking the splits s = w (mod 4).  Lane j reads the maximum and
// sum of the wave's split j while every lane's partial-vector loads are
// already in flight; the wave forms its weights exp2(m_s - M_w), sums its
// splits, and wave 0 merges the four waves in a fixed order.
__global__ __launch_bounds__(256) void k_attn_combine(const float* p_part_m, const float* p_part_l,
                                                      const float* p_part_acc, float* p_out, int p_hd, int p_G,
                                                      int p_nsplit) {
    struct {
        const float *part_m, *part_l, *part_acc;
        float* out;
        int hd, G, nsplit;
    } const a{p_part_m, p_part_l, p_part_acc, p_out, p_hd, p_G, p_nsplit};
    constexpr int kBatch = 16;
    __shared__ float wts[kWavesPerWG][kWave];
    __shared__ float gm[kWavesPerWG], gl[kWavesPerWG], gacc[kWavesPerWG][kWave];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hq = blockIdx.y, d = blockIdx.x * kWave + lane;
    const int G = a.G, hd = a.hd, S = a.nsplit;
    const int g = hq / G, h = hq - g * G;
    const int64_t base = (int64_t)g * S * G + h;          // slot of split s = base + s*G
    const int ns = S > wave ? (S - wave + kWavesPerWG - 1) / kWavesPerWG : 0;   // this wave's splits (<= 64)
    const bool dl = d < hd;

    float mj = -INFINITY, lj = 0.0f;
    if (lane < ns) {
        const int64_t slot = base + (int64_t)(wave + kWavesPerWG * lane) * G;
        mj = a.part_m[slot];
        lj = a.part_l[slot];
    }
    // partial vectors: loads from clamped, valid slots; values past the
    // wave's splits are dropped by their zero weight
    const int dc = dl ? d : 0;
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
        const int uc = u < ns ? u : (ns > 0 ? ns - 1 : 0);
        const int64_t slot = base + (int64_t)(ns > 0 ? wave + kWavesPerWG * uc : 0) * G;
        v[u] = a.part_acc[slot * hd + dc];
    }
    const float Mw = wave_max(mj);
    const float wj = (mj == -INFINITY) ? 0.0f : exp2f(mj - Mw);
    const float Lw = wave_sum(wj * lj);
    wts[wave][lane] = wj;
    wave_lds_sync();
    float sum = 0.0f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) sum = fmaf(wts[wave][u], v[u], sum);     // wts is 0 past ns
    for (int u0 = kBatch; u0 < ns; u0 += kBatch) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int uc = u0 + u < ns ? u0 + u : ns - 1;
            v[u] = a.part_acc[(base + (int64_t)(wave + kWavesPerWG * uc) * G) * hd + dc];
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) sum = fmaf(wts[wave][u0 + u < kWave ? u0 + u : kWave - 1], v[u], sum);
    }
    if (lane == 0) {
        gm[wave] = Mw;
        gl[wave] = Lw;
    }
    gacc[wave][lane] = sum;
    __syncthreads();
    if (wave == 0 && dl) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWavesPerWG; ++w) M = fmaxf(M, gm[w]);
        float L = 0.0f, acc = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesPerWG; ++w) {
            const float e = (gm[w] == -INFINITY) ? 0.0f : exp2f(gm[w] - M);
            L = fmaf(e, gl[w], L);
            acc = fmaf(e, gacc[w][lane], acc);
        }
        a.out[(int64_t)hq * hd + d] = acc / L;
    }
}

__global__ void k_fill_zero(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}

// ---- host side ------------------------------------------------------------

namespace {

struct Plan {
    int nsplit, tiles_per_split;
    int cap;     // splits before whole tiles per wave are rounded: no shorter length plans more
};

constexpr int kMaxSplits = kMaxSplitsC;

using SplitFn = void (*)(dim3, hipStream_t, const AttnArgs&, LaunchMarks*);

struct Variant {
    int32_t dtype;
    int c;       // chunks per row (head_dim / CE), exact
    int g;       // G, exact
    int tile;
    int wpe;     // waves per SIMD resident at once
    int nw;      // waves per workgroup
    SplitFn fn;
    int tpw = 1; // tiles per wave at least (more: the next tile's loads overlap this tile's math)
};

template <typename KV, int CM, int GM, int NP, int TILE, int WPE = 2, bool EX = true, int NW = 4>
void launch_split(dim3 grid, hipStream_t s, const AttnArgs& a, LaunchMarks* mk) {
    launch_marked(mk, k_attn_split<KV, CM, GM, NP, TILE, EX, WPE, NW>, grid, dim3(NW * 64), 0, s, LQ_ATTN_FIELDS(a));
}

// Exact shapes of the common models: {dtype, chunks per row, G, positions per
// tile, waves per SIMD, waves per workgroup, kernel, tiles per wave at least}.
// Tiles per wave over 1024 bf16 positions: head_dim 512 with G 8 takes 13.1
// us with 1 against 15.4 with 2 (at 8192 positions the plans coincide).
// head_dim 256 with G 2 was faster with 2 alone (10.1 against 11.1 us) but
// slower inside the decode layer, whose attention prologue normalizes and
// rotates the heads (6.4 against 5.7 us for the split kernel).
const Variant kVariants[] = {
    {LQ_KV_F32, 16, 2, 32, 2, 4, launch_split<float, 16, 2, 8, 32>},          // head_dim 64
    {LQ_KV_F32, 16, 4, 32, 2, 4, launch_split<float, 16, 4, 8, 32>},
    {LQ_KV_F32, 32, 4, 16, 2, 4, launch_split<float, 32, 4, 16, 16>},         // head_dim 128
    {LQ_KV_BF16, 8, 2, 32, 2, 4, launch_split<uint16_t, 8, 2, 8, 32>},        // head_dim 64
    {LQ_KV_BF16, 8, 4, 32, 2, 4, launch_split<uint16_t, 8, 4, 8, 32>},
    {LQ_KV_BF16, 10, 2, 32, 2, 4, launch_split<uint16_t, 10, 2, 8, 32>},      // head_dim 80
    {LQ_KV_BF16, 10, 4, 32, 2, 4, launch_split<uint16_t, 10, 4, 8, 32>},
    {LQ_KV_BF16, 16, 2, 32, 2, 4, launch_split<uint16_t, 16, 2, 8, 32>},      // head_dim 128
    {LQ_KV_BF16, 16, 4, 16, 2, 4, launch_split<uint16_t, 16, 4, 8, 16>, 2},
    {LQ_KV_BF16, 16, 8, 16, 2, 4, launch_split<uint16_t, 16, 8, 16, 16>},
    {LQ_KV_BF16, 32, 2, 8, 2, 4, launch_split<uint16_t, 32, 2, 16, 8>},     // head_dim 256
    {LQ_KV_BF16, 32, 4, 16, 2, 4, launch_split<uint16_t, 32, 4, 16, 16>},
    {LQ_KV_BF16, 64, 8, 4, 2, 8, launch_split<uint16_t, 64, 8, 64, 4, 2, true, 8>},          // head_dim 512
};

int ce_of(int32_t dtype) { return dtype == LQ_KV_F32 ? 4 : 8; }

struct Pick {
    SplitFn fn;
    int tile;
    int wpe;
    int nw;
    int tpw;
};

// vec_ok: the query rows are 16-byte aligned; exact instances with head_dim
// 256 or 512 read them with vector loads, so without it the padded instance
// runs.
Pick pick(int32_t dtype, int64_t hd, int64_t G, bool vec_ok) {
    const int c = (int)(hd / ce_of(dtype));
    if (vec_ok || !(hd == 256 || hd == 512))
        for (const Variant& v : kVariants)
            if (v.dtype == dtype && v.c == c && v.g == G) return Pick{v.fn, v.tile, v.wpe, v.nw, v.tpw};
    // any head_dim <= 512 and G <= 8: padded loops, one position per K step
    if (dtype == LQ_KV_F32) return Pick{launch_split<float, 128, 8, 64, 4, 2, false>, 4, 2, 4, 1};
    return Pick{launch_split<uint16_t, 64, 8, 64, 8, 2, false>, 8, 2, 4, 1};
}

Plan make_plan(int64_t n_kv, int64_t len, const Pick& pk) {
    const int64_t tile = pk.tile, nw = pk.nw;
    const int64_t tiles = (len + tile - 1) / tile;
    int64_t ns = ((int64_t)kNumCUs * pk.wpe * 4 / nw + n_kv - 1) / n_kv;   // one resident round of workgroups
    const int64_t by_tiles = (tiles + nw * pk.tpw - 1) / (nw * pk.tpw);  // every wave gets tpw tiles
    if (ns > by_tiles) ns = by_tiles;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    const int64_t cap = ns;
    int64_t tps = (tiles + ns - 1) / ns;
    tps = (tps + nw - 1) / nw * nw;                                     // whole tiles per wave
    ns = (tiles + tps - 1) / tps;
    if (ns < 1) ns = 1;
    return Plan{(int)ns, (int)tps, (int)cap};
}

}  // namespace

bool attn_supported(int64_t n_q, int64_t n_kv, int64_t hd, int32_t kv_dtype) {
    if (n_kv <= 0 || n_q % n_kv) return false;
    const int64_t G = n_q / n_kv;
    return G >= 1 && G <= 8 && hd > 0 && hd <= 512 && hd % ce_of(kv_dtype) == 0 && hd % 4 == 0;
}

// Partials for the plan of len.  For the decode layer (`layer`): sized for
// the split count before rounding, which bounds the splits of every shorter
// length (the layer sizes its workspace for its longest attention and runs
// shorter ones in it).
static size_t ws_bytes_for(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len, int32_t dtype, bool layer) {
    if (len <= 0 || n_kv <= 0) return 0;
    size_t most = 0;
    for (const bool vec_ok : {true, false}) {
        const Plan p = make_plan(n_kv, len, pick(dtype, hd, n_q / n_kv, vec_ok));
        const int64_t ns = layer ? p.cap : p.nsplit;
        if (ns == 1) continue;
        const int64_t slots = n_kv * ns * (n_q / n_kv);
        const size_t b = (size_t)(slots * (hd + 2)) * sizeof(float);
        most = b > most ? b : most;
    }
    return most;
}

int attn_nsplit(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len, int32_t kv_dtype, bool vec_ok) {
    if (len <= 0 || n_kv <= 0) return 0;
    return make_plan(n_kv, len, pick(kv_dtype, hd, n_q / n_kv, vec_ok)).nsplit;
}

size_t attn_workspace_bytes(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len, bool layer) {
    // the larger of the two dtypes' plans, so one query serves both
    const size_t a = ws_bytes_for(n_q, n_kv, hd, len, LQ_KV_F32, layer);
    const size_t b = hd % 8 == 0 ? ws_bytes_for(n_q, n_kv, hd, len, LQ_KV_BF16, layer) : 0;
    return a > b ? a : b;
}

static lq_status launch_common(AttnArgs& a, int64_t n_q, int64_t n_kv, int64_t hd, int32_t kv_dtype,
                               void* ws, hipStream_t s, LaunchMarks* marks = nullptr) {
    const int64_t G = n_q / n_kv;
    const Pick pk = pick(kv_dtype, hd, G, a.fused || reinterpret_cast<uintptr_t>(a.q) % 16 == 0);
    const Plan p = make_plan(n_kv, a.len, pk);
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
    launch_marked(marks, k_attn_combine, dim3((unsigned)((hd + kWave - 1) / kWave), (unsigned)n_q), dim3(256), 0,
                  s, (const float*)a.part_m, (const float*)a.part_l, (const float*)a.part_acc, a.out, a.hd, a.G,
                  a.nsplit);
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
                                 int64_t len, float scale, float softcap, float* out, void* ws, hipStream_t s,
                                 LaunchMarks* marks, float* tap_post) {
    AttnArgs a{};
    a.tap_post = tap_post;
    a.cap2 = softcap > 0.0f ? softcap * kLog2e : 0.0f;
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

namespace lq {
lq_status check_attention_args(const char* fn, const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                               const void* k_cache, const void* v_cache, int32_t kv_dtype, int64_t head_stride,
                               int64_t pos_stride, int64_t max_ctx, int64_t start, int64_t len, const float* out) {
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
    if (n_q > 65535) return fail(LQ_ERR_UNSUPPORTED, "%s: too many query heads", fn);
    return LQ_OK;
}
}  // namespace lq

extern "C" lq_status lq_gqa_decode_attn(const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                                        const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                        int64_t head_stride, int64_t pos_stride, int64_t max_ctx,
                                        int64_t start, int64_t len, float scale, float* out,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "lq_gqa_decode_attn";
    lq_status st = check_attention_args(fn, q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride,
                                        pos_stride, max_ctx, start, len, out);
    if (st != LQ_OK || n_q == 0) return st;
    const size_t need = attn_workspace_bytes(n_q, n_kv, head_dim, len);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 16)))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn, need,
                    workspace_bytes);
    return launch_attention(q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride, start,
                            len, scale, out, workspace, as_stream(stream));
}

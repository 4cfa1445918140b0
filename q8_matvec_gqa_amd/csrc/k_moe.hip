// k_moe.hip -- MoE routing and the index-driven Q8_0 matvec for gfx950.
//
// "Current Inference Path -- Architecture Map" (section 3 item i: router
// softmax, top-k, expert dispatch, weighted reduction; section 4 moe_kernel:
// each (token, slot) row selects an expert's quantized weights by id) and
// "Target Inference Architecture: hf2q on mlx-native" (section 3.2:
// softmax, argsort, gather, quantized_matmul_id x2, weighted_sum; section
// 6.3: experts byte-contiguous as [num_experts, n, k]).
//
// Decode batches are small (16 tokens x top-8 here), so a (token, slot)
// touches few rows per expert; what matters is that every touched expert's
// weights stream from HBM exactly once.  A gather step lists, per active
// expert, its (token, slot) rows (in the order the gather's LDS atomics hand
// out places, which may vary between runs: each row is computed on its own
// and written to its own slot, so the results do not depend on it); the
// matvec then walks (expert, row block) items over one resident round of
// workgroups, loads each item's weight rows into VGPRs once (the next
// item's while the current one is computed), and applies them to every
// listed slot.  No float atomics are used, so results are deterministic.
#include <math.h>

#include <atomic>

#include "lq_device.h"
#include "lq_internal.h"
#include "lq_qk.h"

namespace lq {

constexpr int kMoeMaxExperts = 4096;
constexpr int kMoeMaxSlots = 8192;

// Workspace layout (int32 units):
//   [0] invalid-id counter, [1] active expert count,
//   [2, 2+E) active expert ids, [2+E, 3+2E) slot offsets per active expert,
//   [3+2E, 3+2E+T*k) slot indices grouped by expert.
struct MoeWs {
    int32_t* base;
    int64_t E;
    __host__ __device__ int32_t* invalid() const { return base; }
    __host__ __device__ int32_t* n_active() const { return base + 1; }
    __host__ __device__ int32_t* active() const { return base + 2; }
    __host__ __device__ int32_t* offsets() const { return base + 2 + E; }
    __host__ __device__ int32_t* slots() const { return base + 3 + 2 * E; }
};

size_t moe_ws_bytes(int64_t T, int64_t k, int64_t n_experts) {
    return round_up((size_t)(3 + 2 * n_experts + T * k) * sizeof(int32_t), 256);
}

// ---- router: one wave per token --------------------------------------------
// Softmax over the token's E logits, then the k largest (ties: lower id);
// the weights are the probabilities themselves.  Lane 0 writes id and weight
// of each pick to ids/w and, when sids is given, the id to sids (LDS).
// PER logits per lane (E <= 64 * PER): the instance for the smallest PER
// that holds E runs (routing is VALU work on one workgroup in k_moe_prep).
template <int PER>
__device__ __forceinline__ void route_token_p(const float* __restrict__ lt, int E, int k, int lane,
                                              int32_t* __restrict__ ids, float* __restrict__ w, int32_t* sids) {
    float v[PER];
    float mx = -INFINITY;
    // straight-line loads (a clamped index, then a select): a load under a
    // branch per element would wait for each one in turn
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = lt[e < E ? e : E - 1];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        v[i] = lane + 64 * i < E ? v[i] : -INFINITY;
        mx = fmaxf(mx, v[i]);
    }
    mx = wave_max(mx);
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < PER; ++i) z += (lane + 64 * i < E) ? expf(v[i] - mx) : 0.0f;
    z = wave_sum(z);
    // pick s lands in lane s; the weights are formed after the k picks, one
    // per lane (k <= 32)
    float pv = 0.0f;
    int pid = 0;
    for (int s = 0; s < k; ++s) {
        // lane-local best (largest value, then lowest id)
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = lane + 64 * i;
            if (e < E && (v[i] > bv || (v[i] == bv && e < bi))) {
                bv = v[i];
                bi = e;
            }
        }
        // wave argmax with the same ordering: the largest value, then the
        // lowest id among the lanes holding it (read from the one lane that
        // holds it unless several do)
        const float m = wave_max(bv);
        const unsigned long long tied = __ballot(bv == m);
        if (__popcll(tied) == 1)
            bi = __builtin_amdgcn_readlane(bi, __ffsll((long long)tied) - 1);
        else
            bi = wave_min_i(bv == m ? bi : 0x7fffffff);
        if (lane == s) {
            pv = m;
            pid = bi;
        }
        // remove the chosen expert, below every real value (NaN never wins)
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (lane + 64 * i == bi) v[i] = __int_as_float(0xff800001u);
    }
    if (lane < k) {
        ids[lane] = pid;
        w[lane] = expf(pv - mx) / z;
        if (sids) sids[lane] = pid;
    }
}

__device__ __forceinline__ void route_token(const float* __restrict__ lt, int E, int k, int lane,
                                            int32_t* __restrict__ ids, float* __restrict__ w, int32_t* sids) {
    if (E <= 64) route_token_p<1>(lt, E, k, lane, ids, w, sids);
    else if (E <= 128) route_token_p<2>(lt, E, k, lane, ids, w, sids);
    else if (E <= 256) route_token_p<4>(lt, E, k, lane, ids, w, sids);
    else if (E <= 512) route_token_p<8>(lt, E, k, lane, ids, w, sids);
    else route_token_p<16>(lt, E, k, lane, ids, w, sids);   // E <= 1024
}

__global__ __launch_bounds__(64) void k_moe_route(const float* __restrict__ logits, int E, int k,
                                                  int32_t* __restrict__ ids, float* __restrict__ w) {
    const int t = blockIdx.x;
    route_token(logits + (int64_t)t * E, E, k, threadIdx.x, ids + (int64_t)t * k, w + (int64_t)t * k, nullptr);
}

// ---- gather: group (token, slot) rows by expert ------------------------------
// One workgroup of kGatherThreads, the slot ids already in LDS.  Counts per
// expert (LDS atomics), one block-wide exclusive scan of (count, active)
// pairs gives each expert its offset and its index in the active list (in
// expert order), and every slot then takes a place in its expert's list.
// Rows of slots with an out-of-range id are zeroed in y0 and y1 (either may
// be NULL) and counted.
constexpr int kGatherThreads = 1024;
constexpr int kGatherEpt = kMoeMaxExperts / kGatherThreads;    // experts per thread

// Exclusive scan of one int per thread over the workgroup; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) tmp[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int t = lane < kGatherThreads / 64 ? tmp[lane] : 0;
#pragma unroll
        for (int off = 1; off < kGatherThreads / 64; off <<= 1) {
            const int y = __shfl_up(t, off);
            if (lane >= off) t += y;
        }
        if (lane < kGatherThreads / 64) tmp[lane] = t;
    }
    __syncthreads();
    const int base = wave ? tmp[wave - 1] : 0;
    *total = tmp[kGatherThreads / 64 - 1];
    __syncthreads();
    return base + x - v;
}

__device__ void gather_lds(const int32_t* sids, int nslots, int E, MoeWs ws, int32_t* cnt, int* tmp, float* y0,
                           int64_t rows0, float* y1, int64_t rows1) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kGatherThreads) cnt[e] = 0;
    __syncthreads();
    for (int i = tid; i < nslots; i += kGatherThreads) {
        const int e = sids[i];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // thread tid owns experts [tid*EPT, tid*EPT + EPT); pack (count << 13 | active)
    int c[kGatherEpt], local = 0;
#pragma unroll
    for (int j = 0; j < kGatherEpt; ++j) {
        const int e = tid * kGatherEpt + j;
        c[j] = e < E ? cnt[e] : 0;
        local += (c[j] << 13) | (c[j] > 0 ? 1 : 0);
    }
    int total;
    int run = block_excl_scan(local, tmp, &total);
    int32_t* act = ws.active();
    int32_t* offs = ws.offsets();
#pragma unroll
    for (int j = 0; j < kGatherEpt; ++j) {
        const int e = tid * kGatherEpt + j;
        if (c[j] > 0) {
            const int idx = run & 0x1fff, off = run >> 13;
            act[idx] = e;
            offs[idx] = off;
            cnt[e] = off;                  // becomes the fill cursor of expert e
        }
        run += (c[j] << 13) | (c[j] > 0 ? 1 : 0);
    }
    __syncthreads();
    // each slot takes the next place in its expert's list; the order inside a
    // list does not change any result (every slot's rows are computed on
    // their own), only which iteration of the matvec handles it
    for (int i = tid; i < nslots; i += kGatherThreads) {
        const int e = sids[i];
        if (e >= 0 && e < E) ws.slots()[atomicAdd(&cnt[e], 1)] = i;
    }
    const int n_active = total & 0x1fff, listed = total >> 13;
    if (tid == 0) {
        offs[n_active] = listed;
        *ws.n_active() = n_active;
        *ws.invalid() = nslots - listed;
    }
    if (listed < nslots) {
        // zero the outputs of invalid slots
        for (int i = 0; i < nslots; ++i) {
            const int e = sids[i];
            if (e >= 0 && e < E) continue;
            if (y0)
                for (int64_t r = tid; r < rows0; r += kGatherThreads) y0[(int64_t)i * rows0 + r] = 0.0f;
            if (y1)
                for (int64_t r = tid; r < rows1; r += kGatherThreads) y1[(int64_t)i * rows1 + r] = 0.0f;
        }
    }
}

__global__ __launch_bounds__(kGatherThreads) void k_moe_gather(const int32_t* __restrict__ ids, int nslots, int E,
                                                               int32_t* wsbase, float* y0, int64_t rows0,
                                                               float* y1, int64_t rows1) {
    __shared__ int32_t sids[kMoeMaxSlots];
    __shared__ int32_t cnt[kMoeMaxExperts];
    __shared__ int tmp[kGatherThreads / 64];
    for (int i = threadIdx.x; i < nslots; i += kGatherThreads) sids[i] = ids[i];
    __syncthreads();
    gather_lds(sids, nslots, E, MoeWs{wsbase, E}, cnt, tmp, y0, rows0, y1, rows1);
}

// The MoE block's first step in one launch: workgroup 0 routes every token
// (one wave per token at a time) and gathers the slots by expert; the other
// workgroups quantize x to Q8_0, kPrepQuantBlocks 32-blocks each (one per
// thread, so each SIMD has one busy wave).
constexpr int kPrepQuantBlocks = 256;
__global__ __launch_bounds__(kGatherThreads) void k_moe_prep(const float* __restrict__ logits,
                                                             const float* __restrict__ x, int T, int E, int k,
                                                             int H, int32_t* __restrict__ ids,
                                                             float* __restrict__ w, int32_t* wsbase,
                                                             int8_t* __restrict__ xq, uint16_t* __restrict__ xd,
                                                             float* y0, int64_t rows0, float* y1, int64_t rows1) {
    __shared__ int32_t sids[kMoeMaxSlots];
    __shared__ int32_t cnt[kMoeMaxExperts];
    __shared__ int tmp[kGatherThreads / 64];
    if (blockIdx.x > 0) {
        const int64_t nbx = (int64_t)T * (H / 32);
        const int64_t b = (int64_t)(blockIdx.x - 1) * kPrepQuantBlocks + threadIdx.x;
        if (threadIdx.x < kPrepQuantBlocks && b < nbx) {
            float v[32];
            load32(x + 32 * b, v);
            quantize_block32(v, xq + 32 * b, xd + b);
        }
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int t = wave; t < T; t += kGatherThreads / 64)
        route_token(logits + (int64_t)t * E, E, k, lane, ids + (int64_t)t * k, w + (int64_t)t * k,
                    sids + (int64_t)t * k);
    __syncthreads();
    gather_lds(sids, T * k, E, MoeWs{wsbase, E}, cnt, tmp, y0, rows0, y1, rows1);
}

__device__ __forceinline__ int dot16(int4 a, int4 b) {
    int p = __builtin_amdgcn_sdot4(a.x, b.x, 0, false);
    p = __builtin_amdgcn_sdot4(a.y, b.y, p, false);
    p = __builtin_amdgcn_sdot4(a.z, b.z, p, false);
    p = __builtin_amdgcn_sdot4(a.w, b.w, p, false);
    return p;
}

// ---- index-driven matvec ------------------------------------------------------
// Items are (active expert ai, row block rb), item = ai * rowblocks + rb for
// ai < n_active.  One resident round of workgroups walks them (workgroup b
// takes items b, b + grid, ...).  Each wave holds RPW weight rows (NCH 1 KB
// chunks each) of its item in VGPRs and applies them to every slot of the
// item's expert, with the dense Q8_0 matvec's lane mapping and block-dot
// arithmetic.  The rows of the workgroup's next item are requested before
// the current item's slots are computed, so each wave keeps a weight stream
// in flight while it computes; workgroups that each load one item and exit
// all load, then all compute, and the memory system idles in between.
//
// Epilogues: ID_STORE writes y[slot, r]; ID_SWIGLU takes the weight's rows
// as gate rows then up rows (rows = 2 * outputs), holds gate row o and up
// row o side by side and writes h[slot, o] = silu(gate) * up (and, when
// given, the gate and up values to y1[slot, :]).
enum { ID_STORE = 0, ID_SWIGLU = 1 };

struct IdArgs {
    const int8_t* wq;
    const uint16_t* wd;
    int rows, cols;              // weight rows per expert (ID_SWIGLU: 2 * outputs), columns
    const int8_t* xq;            // Q8_0 activation rows [*, cols] and scales [*, cols/32]
    const uint16_t* xd;
    int x_per_slot, k;           // activation row of slot s: s (x_per_slot) or s / k
    const int32_t* ws;
    int E, rowblocks;
    float* y;                    // ID_STORE: [slots, rows]; ID_SWIGLU: [slots, rows / 2]
    float* y1;                   // ID_SWIGLU: optional [slots, rows]
};

// Rows and activations are loaded without branches: rows past the expert
// read its last row (never stored) and chunks past cols read the row's last
// 16 bytes, whose products are zeroed through the activation.  The f16
// scales stay raw until they are used: converting them where they are
// loaded would wait for each load in turn.
template <int NCH, int RPW>
struct IdRows {
    int4 w[RPW][NCH];
    uint32_t s[RPW][NCH];      // f16 bits
};

// weight row of the wave's row i (-1: past the weight)
template <int RPW, int EPI>
__device__ __forceinline__ int id_row(const IdArgs& a, int u0, int i) {
    if constexpr (EPI == ID_SWIGLU) {
        const int o = u0 + i / 2, out = a.rows >> 1;
        return o < out ? o + (i & 1) * out : -1;
    } else {
        return u0 + i < a.rows ? u0 + i : -1;
    }
}

template <int NCH, int RPW, int EPI>
__device__ __forceinline__ void id_load_rows(const IdArgs& a, int e, int u0, int lane, IdRows<NCH, RPW>& R) {
    const int cols = a.cols, nb = cols >> 5;
    const int8_t* we = a.wq + (int64_t)e * a.rows * cols;
    const uint16_t* de = a.wd + (int64_t)e * a.rows * nb;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int rr = id_row<RPW, EPI>(a, u0, i);
        const int r = rr >= 0 ? rr : a.rows - 1;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int off = c * 1024 + lane * 16 < cols ? c * 1024 + lane * 16 : cols - 16;
            R.w[i][c] = load_stream16(we + (int64_t)r * cols + off);
            R.s[i][c] = de[(int64_t)r * nb + (off >> 5)];
        }
    }
}

template <int NCH>
struct IdAct {
    int4 v[NCH];
    uint32_t s[NCH];           // f16 bits
};

template <int NCH>
__device__ __forceinline__ void id_load_act(const IdArgs& a, int64_t xrow, int lane, IdAct<NCH>& X) {
    const int cols = a.cols;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int off = c * 1024 + lane * 16 < cols ? c * 1024 + lane * 16 : cols - 16;
        X.v[c] = *reinterpret_cast<const int4*>(a.xq + xrow * cols + off);
        X.s[c] = a.xd[xrow * (cols >> 5) + (off >> 5)];
    }
}

// One slot's codes and f32 scales, zero past cols.
template <int NCH>
__device__ __forceinline__ void id_cook(const IdArgs& a, const IdAct<NCH>& X, int lane, int4 (&xv)[NCH],
                                        float (&xs)[NCH]) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const bool in = c * 1024 + lane * 16 < a.cols;
        xv[c] = in ? X.v[c] : make_int4(0, 0, 0, 0);
        xs[c] = in ? f16_to_f32((uint16_t)X.s[c]) : 0.0f;
    }
}

// Products of the rows in R with one slot's activation, then the epilogue.
// With 4 to 8 rows the row sums come from one reduce-scatter over the wave
// (row i's sum in lanes 8i..8i+7) instead of one full wave sum per row, and
// each lane 16j finishes gate/up pair j (its up row's sum is in lane 16j+8).
template <int NCH, int RPW, int EPI>
__device__ __forceinline__ void id_dots(const IdArgs& a, const IdRows<NCH, RPW>& R, const int4 (&xv)[NCH],
                                        const float (&xs)[NCH], int u0, int slot, int lane) {
    float t[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        t[i] = 0.0f;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int p = dot16(R.w[i][c], xv[c]);
            const int blk = p + dpp_i<kQuadXor1>(p);
            const float v = (float)blk * (f16_to_f32((uint16_t)R.s[i][c]) * xs[c]);
            t[i] += (lane & 1) ? 0.0f : v;
        }
    }
    const int out = EPI == ID_SWIGLU ? a.rows >> 1 : a.rows;
    auto swiglu_store = [&](int o, float gt, float up) {
        a.y[(int64_t)slot * out + o] = (gt / (1.0f + expf(-gt))) * up;
        if (a.y1) {
            a.y1[(int64_t)slot * a.rows + o] = gt;
            a.y1[(int64_t)slot * a.rows + out + o] = up;
        }
    };
    if constexpr (RPW >= 4 && RPW <= 8) {
        float v8[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) v8[h] = h < RPW ? t[h] : 0.0f;
        const float srow = wave_sum8_scatter(v8);
        if constexpr (EPI == ID_SWIGLU) {
            const float up = dpp<kRowRor8>(srow);
            const int j = lane >> 4, o = u0 + j;
            if ((lane & 15) == 0 && j < RPW / 2 && o < out) swiglu_store(o, srow, up);
        } else {
            const int h = lane >> 3;
            if ((lane & 7) == 0 && h < RPW && u0 + h < out) a.y[(int64_t)slot * out + u0 + h] = srow;
        }
    } else {
        float acc[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) acc[i] = wave_sum(t[i]);
        if (lane != 0) return;
        if constexpr (EPI == ID_SWIGLU) {
#pragma unroll
            for (int j = 0; j < RPW / 2; ++j)
                if (u0 + j < out) swiglu_store(u0 + j, acc[2 * j], acc[2 * j + 1]);
        } else {
#pragma unroll
            for (int i = 0; i < RPW; ++i)
                if (u0 + i < out) a.y[(int64_t)slot * out + u0 + i] = acc[i];
        }
    }
}

template <int NCH, int RPW, int EPI>
__global__ __launch_bounds__(256) void k_moe_matvec_id(IdArgs a) {
    const MoeWs ws{const_cast<int32_t*>(a.ws), a.E};
    const int rowblocks = a.rowblocks;
    const int n_items = *ws.n_active() * rowblocks;
    int it = blockIdx.x;
    if (it >= n_items) return;
    const int G = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int UPW = EPI == ID_SWIGLU ? RPW / 2 : RPW;       // outputs per wave
    static_assert(EPI != ID_SWIGLU || RPW % 2 == 0, "gate/up pairs");
    auto expert_of = [&](int item) { return ws.active()[item / rowblocks]; };
    auto u0_of = [&](int item) { return ((item - (item / rowblocks) * rowblocks) * 4 + wave) * UPW; };
    auto xrow_of = [&](int slot) -> int64_t { return a.x_per_slot ? slot : slot / a.k; };
    // the activations of an item's first two slots (the first again when it
    // has one); they are requested before the next item's rows, so waiting
    // for them leaves those rows in flight (loads complete in issue order)
    auto load_first = [&](int item, IdAct<NCH>& X0, IdAct<NCH>& X1) {
        const int ai = item / rowblocks;
        const int s0 = ws.offsets()[ai], s1 = ws.offsets()[ai + 1];
        id_load_act<NCH>(a, xrow_of(ws.slots()[s0]), lane, X0);
        id_load_act<NCH>(a, xrow_of(ws.slots()[s0 + 1 < s1 ? s0 + 1 : s0]), lane, X1);
    };
    auto one = [&](const IdRows<NCH, RPW>& R, const IdAct<NCH>& X, int item, int slot) {
        int4 xv[NCH];
        float xs[NCH];
        id_cook<NCH>(a, X, lane, xv, xs);
        id_dots<NCH, RPW, EPI>(a, R, xv, xs, u0_of(item), slot, lane);
    };
    auto consume = [&](int item, const IdRows<NCH, RPW>& R, const IdAct<NCH>& X0, const IdAct<NCH>& X1) {
        const int ai = item / rowblocks;
        const int s0 = ws.offsets()[ai], s1 = ws.offsets()[ai + 1];
        one(R, X0, item, ws.slots()[s0]);
        if (s0 + 1 < s1) one(R, X1, item, ws.slots()[s0 + 1]);
        for (int si = s0 + 2; si < s1; ++si) {
            const int slot = ws.slots()[si];
            IdAct<NCH> X;
            id_load_act<NCH>(a, xrow_of(slot), lane, X);
            one(R, X, item, slot);
        }
    };
    // items it, it + G, ...: the next item's rows are requested before the
    // current one is consumed, in straight-line code with the last step
    // peeled (as in the dense matvec), so each wait covers exactly the loads
    // it needs
    IdRows<NCH, RPW> A, B;
    IdAct<NCH> X0, X1;
    id_load_rows<NCH, RPW, EPI>(a, expert_of(it), u0_of(it), lane, A);
    for (;;) {
        const int i1 = it + G;
        load_first(it, X0, X1);
        if (i1 >= n_items) {
            consume(it, A, X0, X1);
            break;
        }
        id_load_rows<NCH, RPW, EPI>(a, expert_of(i1), u0_of(i1), lane, B);
        consume(it, A, X0, X1);
        const int i2 = i1 + G;
        load_first(i1, X0, X1);
        if (i2 >= n_items) {
            consume(i1, B, X0, X1);
            break;
        }
        id_load_rows<NCH, RPW, EPI>(a, expert_of(i2), u0_of(i2), lane, A);
        consume(i1, B, X0, X1);
        it = i2;
    }
}

// ---- index-driven Q4_0 / Q6_K matvec -------------------------------------------
// The MoE kernel of the current path runs on Q6_K expert weights ("Current
// Inference Path -- Architecture Map", section 4).  Same decomposition as
// k_moe_matvec_id: blockIdx.x = active-expert index * rowblocks + row block;
// each wave holds the units (lq_qk.h) of RPW rows of its expert in VGPRs and
// applies them to every listed slot, reading the slot's Q8_0 activation from
// memory.  Experts are stacked: expert e's row r is row e*rows + r of the
// arrays.  Dead units and rows read the expert's first unit (never used).
template <int FMT, int ST, int RPW>
__global__ __launch_bounds__(256) void k_moe_qk_matvec_id(QkMat m, int rows, int cols, const int8_t* __restrict__ xq,
                                                          const uint16_t* __restrict__ xd, int x_per_slot, int k,
                                                          const int32_t* __restrict__ wsbase, int E, int rowblocks,
                                                          float* __restrict__ y) {
    const MoeWs ws{const_cast<int32_t*>(wsbase), E};
    const int ai = blockIdx.x / rowblocks, rb = blockIdx.x - ai * rowblocks;
    if (ai >= *ws.n_active()) return;
    const int e = ws.active()[ai];
    const int s0 = ws.offsets()[ai], s1 = ws.offsets()[ai + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = (rb * 4 + wave) * RPW;
    if (r0 >= rows) return;
    const int units = qk_units<FMT>(cols);
    const int64_t er = (int64_t)e * rows;
    QkUnit<FMT> U[RPW][ST];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int r = r0 + i, u = st * 64 + lane;
            const bool live = r < rows && u < units;
            qk_load_unit(m, cols, er + (live ? r : 0), live ? u : 0, U[i][st]);
        }
    for (int si = s0; si < s1; ++si) {
        const int slot = ws.slots()[si];
        const int64_t xrow = x_per_slot ? slot : slot / k;
        const int8_t* xr = xq + xrow * cols;
        const uint16_t* xdr = xd + xrow * (cols >> 5);
        // the slot's activation, loaded once for all RPW rows
        QkAct<FMT> A[ST];
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int u = st * 64 + lane;
            qk_load_act(xr, xdr, u < units ? u : 0, A[st]);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float acc = 0.0f;
#pragma unroll
            for (int st = 0; st < ST; ++st) {
                const int u = st * 64 + lane;
                if (u < units) acc += qk_unit_dot_a(U[i][st], u, A[st]);
            }
            acc = wave_sum(acc);
            const int r = r0 + i;
            if (lane == 0 && r < rows) y[(int64_t)slot * rows + r] = acc;
        }
    }
}

// Q4_0 rows of at most 32 blocks (1024 values, the MoE down projection's
// short rows): lane l holds block l & 31 of row 2p + (l >> 5) of its pair p,
// so each load instruction carries two rows and a row's sum is a half-wave
// sum; the per-row unit form above leaves two thirds of the lanes idle on
// 704-value rows.  Otherwise the same decomposition and arithmetic.
template <int RPW>
__global__ __launch_bounds__(256) void k_moe_q4_id_half(QkMat m, int rows, int cols, const int8_t* __restrict__ xq,
                                                        const uint16_t* __restrict__ xd, int x_per_slot, int k,
                                                        const int32_t* __restrict__ wsbase, int E, int rowblocks,
                                                        float* __restrict__ y) {
    constexpr int NP = RPW / 2;
    static_assert(RPW % 2 == 0, "row pairs");
    const MoeWs ws{const_cast<int32_t*>(wsbase), E};
    const int ai = blockIdx.x / rowblocks, rb = blockIdx.x - ai * rowblocks;
    if (ai >= *ws.n_active()) return;
    const int e = ws.active()[ai];
    const int s0 = ws.offsets()[ai], s1 = ws.offsets()[ai + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5, u = lane & 31;
    const int units = cols >> 5;
    const bool uin = u < units;
    const int r0 = (rb * 4 + wave) * RPW;
    if (r0 >= rows) return;
    const int64_t er = (int64_t)e * rows;
    QkUnit<QK_Q4_0> U[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = r0 + 2 * p + half;
        const bool live = r < rows && uin;
        qk_load_unit(m, cols, er + (live ? r : 0), live ? u : 0, U[p]);
    }
    for (int si = s0; si < s1; ++si) {
        const int slot = ws.slots()[si];
        const int64_t xrow = x_per_slot ? slot : slot / k;
        QkAct<QK_Q4_0> A;
        qk_load_act(xq + xrow * cols, xd + xrow * (cols >> 5), uin ? u : 0, A);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            float acc = uin ? qk_unit_dot_a(U[p], u, A) : 0.0f;
            acc = group_sum<32>(acc);
            const int r = r0 + 2 * p + half;
            if (u == 0 && r < rows) y[(int64_t)slot * rows + r] = acc;
        }
    }
}

// out[t] = sum_s w[t,s] * scale[ids[t,s]] * y[t,s] in slot order; without a
// scale table (escale NULL) every scale is 1, and ids past the table (the
// skipped invalid ids, whose y rows are zero) also count 1.
__global__ __launch_bounds__(256) void k_moe_weighted_sum(const float* __restrict__ y,
                                                          const float* __restrict__ w, int64_t T,
                                                          int k, int64_t rows, const int32_t* __restrict__ ids,
                                                          const float* __restrict__ escale, int E,
                                                          float* __restrict__ out) {
    const int64_t n = T * rows;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t t = i / rows, r = i - t * rows;
        float acc = 0.0f;
        for (int s = 0; s < k; ++s) {
            float ws = w[t * k + s];
            if (escale) {
                const int e = ids[t * k + s];
                if (e >= 0 && e < E) ws *= escale[e];
            }
            acc = fmaf(ws, y[(t * k + s) * rows + r], acc);
        }
        out[i] = acc;
    }
}

// ---- host --------------------------------------------------------------------

lq_status launch_moe_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                           float* w, hipStream_t s) {
    if (T == 0) return LQ_OK;
    hipLaunchKernelGGL(k_moe_route, dim3((unsigned)T), dim3(64), 0, s, logits, (int)E, (int)k, ids, w);
    return check_launch("moe_route");
}

static lq_status launch_gather(const int32_t* ids, int64_t nslots, int64_t E, void* ws, float* y0,
                               int64_t rows0, float* y1, int64_t rows1, hipStream_t s) {
    hipLaunchKernelGGL(k_moe_gather, dim3(1), dim3(kGatherThreads), 0, s, ids, (int)nslots, (int)E,
                       static_cast<int32_t*>(ws), y0, rows0, y1, rows1);
    return check_launch("moe_gather");
}

// One resident round of workgroups (queried once per instance), at most one
// item each.
template <int NCH, int RPW, int EPI>
static void launch_id_t(IdArgs a, int outs, hipStream_t s) {
    constexpr int UPW = EPI == ID_SWIGLU ? RPW / 2 : RPW;
    a.rowblocks = (outs + 4 * UPW - 1) / (4 * UPW);
    auto kern = k_moe_matvec_id<NCH, RPW, EPI>;
    static std::atomic<int> resident_cache{-1};
    int resident = resident_cache.load(std::memory_order_relaxed);
    if (resident < 0) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, 0) != hipSuccess || n < 1) n = 1;
        resident = n * kNumCUs;
        resident_cache.store(resident, std::memory_order_relaxed);
    }
    const int64_t items = (int64_t)a.E * a.rowblocks;
    const unsigned grid = (unsigned)(items < resident ? items : resident);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, a);
}

// Rows per wave (for SwiGLU, half as many gate/up pairs): rows of at most 2
// KB 8, of at most 4 KB 4, longer ones 2.  Measured on the 128-expert block
// (704-byte down rows, 2816-byte gate/up rows): down with 4 / 8 / 16 rows
// 118-120 / 116-121 / 125-133 us per block; gate/up with 2 / 4 / 6 / 8 rows
// 118-121 / 110-114 / 115-118 / 120-127 us (4 rows take 238 VGPRs, two
// waves per SIMD, and still stream faster than 2 rows at three).
template <int EPI>
static lq_status launch_id(const IdArgs& a, int outs, hipStream_t s, const char* what) {
    const int nch = (a.cols + 1023) / 1024;
#define LQ_ID_CASE(N)                                              \
    case N:                                                        \
        launch_id_t<N, (N <= 2 ? 8 : (N <= 4 ? 4 : 2)), EPI>(a, outs, s); \
        break;
    switch (nch) {
        LQ_ID_CASE(1) LQ_ID_CASE(2) LQ_ID_CASE(3) LQ_ID_CASE(4)
        LQ_ID_CASE(5) LQ_ID_CASE(6) LQ_ID_CASE(7) LQ_ID_CASE(8)
        default: return fail(LQ_ERR_UNSUPPORTED, "%s: cols > 8192", what);
    }
#undef LQ_ID_CASE
    return check_launch(what);
}

static lq_status launch_id_gathered(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                                    int64_t E, const int8_t* xq, const uint16_t* xd, int32_t x_per_slot,
                                    int64_t k, const void* ws, float* y, hipStream_t s) {
    IdArgs a{};
    a.wq = wq; a.wd = wd; a.rows = (int)rows; a.cols = (int)cols; a.xq = xq; a.xd = xd;
    a.x_per_slot = x_per_slot; a.k = (int)k; a.ws = static_cast<const int32_t*>(ws); a.E = (int)E; a.y = y;
    return launch_id<ID_STORE>(a, (int)rows, s, "moe_matvec_id");
}

lq_status launch_moe_matvec_id(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                               int64_t n_experts, const int8_t* xq, const uint16_t* xd,
                               int32_t x_per_slot, const int32_t* ids, int64_t T, int64_t k,
                               float* y, void* ws, hipStream_t s) {
    lq_status st = launch_gather(ids, T * k, n_experts, ws, y, rows, nullptr, 0, s);
    if (st != LQ_OK) return st;
    return launch_id_gathered(wq, wd, rows, cols, n_experts, xq, xd, x_per_slot, k, ws, y, s);
}

template <int FMT, int ST, int RPW>
static void launch_qk_id_st(hipStream_t s, const QkMat& m, int rows, int cols, int E, const int8_t* xq,
                            const uint16_t* xd, int x_per_slot, int k, const int32_t* ws, float* y) {
    const int rowblocks = (rows + 4 * RPW - 1) / (4 * RPW);
    hipLaunchKernelGGL((k_moe_qk_matvec_id<FMT, ST, RPW>), dim3((unsigned)(E * rowblocks)), dim3(256), 0, s, m, rows,
                       cols, xq, xd, x_per_slot, k, ws, E, rowblocks, y);
}

// The id-matvec on an already gathered workspace.  Steps per row: Q4_0 up
// to 4, Q6_K up to 2 (cols <= 8192).  Rows per wave: 4 for rows of one step
// (measured on the 128-expert block, Q6_K gate/up and Q4_0 down: 129-134
// us per block against 137-140 with 2 and 137-141 with 8 for Q4_0), else
// 2 (1 for Q4_0's 4 steps).
template <int FMT>
static lq_status launch_qk_id_gathered(const QkMat& m, int64_t rows, int64_t cols, int64_t E, const int8_t* xq,
                                       const uint16_t* xd, int32_t x_per_slot, int64_t k, const void* ws, float* y,
                                       hipStream_t s) {
    const int32_t* w32 = static_cast<const int32_t*>(ws);
    if (FMT == QK_Q4_0 && cols <= 1024) {
        // two rows per load instruction: 8 rows per wave
        constexpr int RPW = 8;
        const int rowblocks = (int)((rows + 4 * RPW - 1) / (4 * RPW));
        hipLaunchKernelGGL((k_moe_q4_id_half<RPW>), dim3((unsigned)(E * rowblocks)), dim3(256), 0, s, m, (int)rows,
                           (int)cols, xq, xd, x_per_slot, (int)k, w32, (int)E, rowblocks, y);
        return check_launch("moe_q4_id_half");
    }
    switch ((qk_units<FMT>((int)cols) + 63) / 64) {
        case 1: launch_qk_id_st<FMT, 1, 4>(s, m, (int)rows, (int)cols, (int)E, xq, xd, x_per_slot, (int)k, w32, y); break;
        case 2: launch_qk_id_st<FMT, 2, 2>(s, m, (int)rows, (int)cols, (int)E, xq, xd, x_per_slot, (int)k, w32, y); break;
        default:
            if constexpr (FMT == QK_Q4_0) {
                launch_qk_id_st<FMT, 4, 1>(s, m, (int)rows, (int)cols, (int)E, xq, xd, x_per_slot, (int)k, w32, y);
                break;
            }
            return fail(LQ_ERR_UNSUPPORTED, "moe matvec: cols > 8192");
    }
    return check_launch("moe_qk_matvec_id");
}

template <int FMT>
static lq_status launch_moe_qk_matvec_id(const QkMat& m, int64_t rows, int64_t cols, int64_t E, const int8_t* xq,
                                         const uint16_t* xd, int32_t x_per_slot, const int32_t* ids, int64_t T,
                                         int64_t k, float* y, void* ws, hipStream_t s) {
    lq_status st = launch_gather(ids, T * k, E, ws, y, rows, nullptr, 0, s);
    if (st != LQ_OK) return st;
    return launch_qk_id_gathered<FMT>(m, rows, cols, E, xq, xd, x_per_slot, k, ws, y, s);
}

lq_status launch_moe_weighted_sum(const float* y, const float* w, int64_t T, int64_t k, int64_t rows,
                                  const int32_t* ids, const float* escale, int64_t E, float* out, hipStream_t s) {
    const int64_t n = T * rows;
    if (n == 0) return LQ_OK;
    int64_t grid = (n + 255) / 256;
    if (grid > 4096) grid = 4096;
    hipLaunchKernelGGL(k_moe_weighted_sum, dim3((unsigned)grid), dim3(256), 0, s, y, w, T, (int)k, rows, ids, escale,
                       (int)E, out);
    return check_launch("moe_weighted_sum");
}

static lq_status check_moe_weight(const char* fn, const lq_q8_weight* w, int64_t n_experts) {
    lq_status st = check_weight(w, fn);
    if (st != LQ_OK) return st;
    if (n_experts <= 0 || n_experts > kMoeMaxExperts)
        return fail(LQ_ERR_UNSUPPORTED, "%s: n_experts=%lld (1..%d)", fn, (long long)n_experts, kMoeMaxExperts);
    if (w->cols > 8192 || w->rows > 0x7fffffffLL / 4)
        return fail(LQ_ERR_UNSUPPORTED, "%s: expert rows=%lld cols=%lld too large", fn, (long long)w->rows,
                    (long long)w->cols);
    return LQ_OK;
}

}  // namespace lq

using namespace lq;

extern "C" lq_status lq_moe_route_topk(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                                       float* w, void* stream) {
    if (T < 0 || E <= 0 || k <= 0 || k > E)
        return fail(LQ_ERR_SHAPE, "lq_moe_route_topk: T=%lld E=%lld k=%lld", (long long)T, (long long)E, (long long)k);
    if (E > 1024 || k > 32) return fail(LQ_ERR_UNSUPPORTED, "lq_moe_route_topk: E <= 1024 and k <= 32");
    if (T == 0) return LQ_OK;
    if (T > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "lq_moe_route_topk: T too large");
    if (!logits || !ids || !w) return fail(LQ_ERR_NULL, "lq_moe_route_topk: NULL pointer");
    if (!aligned(logits, 4) || !aligned(ids, 4) || !aligned(w, 4))
        return fail(LQ_ERR_ALIGN, "lq_moe_route_topk: misaligned pointer");
    return launch_moe_route(logits, T, E, k, ids, w, as_stream(stream));
}

extern "C" size_t lq_moe_workspace_size(int64_t T, int64_t k, int64_t n_experts) {
    if (T < 0 || k <= 0 || n_experts <= 0) return 0;
    return moe_ws_bytes(T, k, n_experts);
}

extern "C" lq_status lq_moe_q8_matvec_id(const lq_q8_weight* w, int64_t n_experts, const int8_t* x_qs,
                                         const uint16_t* x_d, int32_t x_per_slot, const int32_t* ids,
                                         int64_t T, int64_t k, float* y, void* workspace,
                                         size_t workspace_bytes, void* stream) {
    const char* fn = "lq_moe_q8_matvec_id";
    lq_status st = check_moe_weight(fn, w, n_experts);
    if (st != LQ_OK) return st;
    if (T < 0 || k <= 0 || (x_per_slot != 0 && x_per_slot != 1))
        return fail(LQ_ERR_SHAPE, "%s: T=%lld k=%lld x_per_slot=%d", fn, (long long)T, (long long)k, x_per_slot);
    if (T * k > kMoeMaxSlots) return fail(LQ_ERR_UNSUPPORTED, "%s: T*k > %d", fn, kMoeMaxSlots);
    if (T == 0 || w->rows == 0) return LQ_OK;
    if (!x_qs || !x_d || !ids || !y) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x_qs, 16) || !aligned(x_d, 2) || !aligned(ids, 4) || !aligned(y, 4))
        return fail(LQ_ERR_ALIGN, "%s: misaligned pointer", fn);
    const size_t need = moe_ws_bytes(T, k, n_experts);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
    return launch_moe_matvec_id(w->qs, w->d, w->rows, w->cols, n_experts, x_qs, x_d, x_per_slot, ids, T, k, y,
                                workspace, as_stream(stream));
}

// Shared argument checks of the Q4_0 / Q6_K id-matvecs (per = values per
// block of the format).
static lq_status check_moe_qk(const char* fn, int64_t rows, int64_t cols, int per, int64_t n_experts,
                              const int8_t* x_qs, const uint16_t* x_d, int32_t x_per_slot, const int32_t* ids,
                              int64_t T, int64_t k, float* y, void* workspace, size_t workspace_bytes) {
    if (rows < 0 || cols <= 0 || cols % per)
        return fail(LQ_ERR_SHAPE, "%s: rows=%lld cols=%lld (cols %% %d == 0)", fn, (long long)rows, (long long)cols,
                    per);
    if (n_experts <= 0 || n_experts > kMoeMaxExperts)
        return fail(LQ_ERR_UNSUPPORTED, "%s: n_experts=%lld (1..%d)", fn, (long long)n_experts, kMoeMaxExperts);
    if (cols > 8192 || rows > 0x7fffffffLL / 4)
        return fail(LQ_ERR_UNSUPPORTED, "%s: expert rows=%lld cols=%lld too large", fn, (long long)rows,
                    (long long)cols);
    if (T < 0 || k <= 0 || (x_per_slot != 0 && x_per_slot != 1))
        return fail(LQ_ERR_SHAPE, "%s: T=%lld k=%lld x_per_slot=%d", fn, (long long)T, (long long)k, x_per_slot);
    if (T * k > kMoeMaxSlots) return fail(LQ_ERR_UNSUPPORTED, "%s: T*k > %d", fn, kMoeMaxSlots);
    if (T == 0 || rows == 0) return LQ_OK;
    if (!x_qs || !x_d || !ids || !y) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x_qs, 16) || !aligned(x_d, 2) || !aligned(ids, 4) || !aligned(y, 4))
        return fail(LQ_ERR_ALIGN, "%s: misaligned pointer", fn);
    const size_t need = moe_ws_bytes(T, k, n_experts);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
    return LQ_OK;
}

extern "C" lq_status lq_moe_q4_0_matvec_id(const lq_q4_0_weight* w, int64_t n_experts, const int8_t* x_qs,
                                           const uint16_t* x_d, int32_t x_per_slot, const int32_t* ids, int64_t T,
                                           int64_t k, float* y, void* workspace, size_t workspace_bytes,
                                           void* stream) {
    const char* fn = "lq_moe_q4_0_matvec_id";
    if (!w) return fail(LQ_ERR_NULL, "%s: NULL weight", fn);
    lq_status st = check_moe_qk(fn, w->rows, w->cols, 32, n_experts, x_qs, x_d, x_per_slot, ids, T, k, y, workspace,
                                workspace_bytes);
    if (st != LQ_OK || T == 0 || w->rows == 0) return st;
    if (!w->qs || !w->d) return fail(LQ_ERR_NULL, "%s: NULL weight array", fn);
    if (!aligned(w->qs, 16) || !aligned(w->d, 2)) return fail(LQ_ERR_ALIGN, "%s: qs must be 16-byte aligned", fn);
    return launch_moe_qk_matvec_id<QK_Q4_0>(QkMat{w->qs, nullptr, nullptr, w->d}, w->rows, w->cols, n_experts, x_qs,
                                            x_d, x_per_slot, ids, T, k, y, workspace, as_stream(stream));
}

extern "C" lq_status lq_moe_q6_k_matvec_id(const lq_q6_k_weight* w, int64_t n_experts, const int8_t* x_qs,
                                           const uint16_t* x_d, int32_t x_per_slot, const int32_t* ids, int64_t T,
                                           int64_t k, float* y, void* workspace, size_t workspace_bytes,
                                           void* stream) {
    const char* fn = "lq_moe_q6_k_matvec_id";
    if (!w) return fail(LQ_ERR_NULL, "%s: NULL weight", fn);
    lq_status st = check_moe_qk(fn, w->rows, w->cols, 256, n_experts, x_qs, x_d, x_per_slot, ids, T, k, y,
                                workspace, workspace_bytes);
    if (st != LQ_OK || T == 0 || w->rows == 0) return st;
    if (!w->ql || !w->qh || !w->sc || !w->d) return fail(LQ_ERR_NULL, "%s: NULL weight array", fn);
    if (!aligned(w->ql, 16) || !aligned(w->qh, 16) || !aligned(w->sc, 8) || !aligned(w->d, 2))
        return fail(LQ_ERR_ALIGN, "%s: ql and qh must be 16-byte aligned, sc 8-byte aligned", fn);
    return launch_moe_qk_matvec_id<QK_Q6_K>(QkMat{w->ql, w->qh, w->sc, w->d}, w->rows, w->cols, n_experts, x_qs,
                                            x_d, x_per_slot, ids, T, k, y, workspace, as_stream(stream));
}

extern "C" lq_status lq_moe_weighted_sum(const float* y, const float* w, int64_t T, int64_t k, int64_t rows,
                                         float* out, void* stream) {
    if (T < 0 || k <= 0 || rows < 0)
        return fail(LQ_ERR_SHAPE, "lq_moe_weighted_sum: T=%lld k=%lld rows=%lld", (long long)T, (long long)k,
                    (long long)rows);
    if (T == 0 || rows == 0) return LQ_OK;
    if (!y || !w || !out) return fail(LQ_ERR_NULL, "lq_moe_weighted_sum: NULL pointer");
    if (!aligned(y, 4) || !aligned(w, 4) || !aligned(out, 4))
        return fail(LQ_ERR_ALIGN, "lq_moe_weighted_sum: misaligned pointer");
    return launch_moe_weighted_sum(y, w, T, k, rows, nullptr, nullptr, 0, out, as_stream(stream));
}

// ---- whole block ---------------------------------------------------------------
namespace {
struct MoeBuffers {
    int32_t* ids; float* w; int8_t* xq; uint16_t* xd; float* y1; int8_t* hq; uint16_t* hd; float* y2;
    float* h;     // Q8_0 block: act(gate) * up in f32, [T*k, ffn]
    void* gather;
    size_t total;
};

MoeBuffers moe_layout(const lq_moe_desc* m, int64_t T, char* base, const lq_moe_taps* taps) {
    const int64_t H = m->hidden, I = m->ffn, k = m->top_k, S = T * k;
    MoeBuffers b{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += round_up(bytes, 256);
        return p;
    };
    b.gather = take(moe_ws_bytes(T, k, m->n_experts));
    b.ids = reinterpret_cast<int32_t*>(take(S * 4));
    b.w = reinterpret_cast<float*>(take(S * 4));
    b.xq = reinterpret_cast<int8_t*>(take(T * H));
    b.xd = reinterpret_cast<uint16_t*>(take(T * (H / 32) * 2));
    b.y1 = reinterpret_cast<float*>(take(S * 2 * I * 4));
    b.hq = reinterpret_cast<int8_t*>(take(S * I));
    b.hd = reinterpret_cast<uint16_t*>(take(S * (I / 32) * 2));
    b.y2 = reinterpret_cast<float*>(take(S * H * 4));
    b.h = reinterpret_cast<float*>(take(S * I * 4));
    b.total = off;
    if (taps) {
        if (taps->ids) b.ids = taps->ids;
        if (taps->w) b.w = taps->w;
        if (taps->xq) b.xq = taps->xq;
        if (taps->xd) b.xd = taps->xd;
        if (taps->y1) b.y1 = taps->y1;
        if (taps->hq) b.hq = taps->hq;
        if (taps->hd) b.hd = taps->hd;
        if (taps->y2) b.y2 = taps->y2;
    }
    return b;
}
}  // namespace

extern "C" size_t lq_moe_block_workspace_size(const lq_moe_desc* m, int64_t T) {
    if (!m || T < 0 || m->top_k <= 0 || m->n_experts <= 0) return 0;
    return moe_layout(m, T, nullptr, nullptr).total;
}

extern "C" lq_status lq_moe_block(const lq_moe_desc* m, const float* x, const float* logits, int64_t T,
                                  float* out, const lq_moe_taps* taps, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    const char* fn = "lq_moe_block";
    if (!m) return fail(LQ_ERR_NULL, "%s: descriptor is NULL", fn);
    const int64_t H = m->hidden, I = m->ffn, E = m->n_experts, k = m->top_k;
    if (T < 0 || H <= 0 || I <= 0 || H % 32 || I % 32 || k <= 0 || k > E)
        return fail(LQ_ERR_SHAPE, "%s: T=%lld hidden=%lld ffn=%lld E=%lld k=%lld", fn, (long long)T, (long long)H,
                    (long long)I, (long long)E, (long long)k);
    if (m->w_gate_up.rows != 2 * I || m->w_gate_up.cols != H || m->w_down.rows != H || m->w_down.cols != I)
        return fail(LQ_ERR_SHAPE, "%s: expert weight shapes do not match hidden/ffn", fn);
    lq_status st = check_moe_weight(fn, &m->w_gate_up, E);
    if (st == LQ_OK) st = check_moe_weight(fn, &m->w_down, E);
    if (st != LQ_OK) return st;
    if (E > 1024 || k > 32) return fail(LQ_ERR_UNSUPPORTED, "%s: E <= 1024 and k <= 32", fn);
    if (T * k > kMoeMaxSlots) return fail(LQ_ERR_UNSUPPORTED, "%s: T*k > %d", fn, kMoeMaxSlots);
    if (T == 0) return LQ_OK;
    if (!x || !logits || !out) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(out, 4) || !aligned(m->expert_scale, 4))
        return fail(LQ_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
    const size_t need = moe_layout(m, T, nullptr, nullptr).total;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-byte aligned), got %zu", fn, need,
                    workspace_bytes);
    MoeBuffers b = moe_layout(m, T, static_cast<char*>(workspace), taps);
    hipStream_t s = as_stream(stream);
    const int64_t S = T * k;
    const int64_t prep_grid = 1 + (T * (H / 32) + kPrepQuantBlocks - 1) / kPrepQuantBlocks;
    hipLaunchKernelGGL(k_moe_prep, dim3((unsigned)prep_grid), dim3(kGatherThreads), 0, s, logits, x, (int)T, (int)E, (int)k, (int)H,
                       b.ids, b.w, static_cast<int32_t*>(b.gather), b.xq, b.xd, b.y1, 2 * I, b.y2, H);
    if ((st = check_launch("moe_prep")) != LQ_OK) return st;
    // gate/up with SwiGLU in the epilogue (h in f32), the Q8_0 of h, then
    // the down projection
    IdArgs g{};
    g.wq = m->w_gate_up.qs; g.wd = m->w_gate_up.d; g.rows = (int)(2 * I); g.cols = (int)H;
    g.xq = b.xq; g.xd = b.xd; g.x_per_slot = 0; g.k = (int)k;
    g.ws = static_cast<const int32_t*>(b.gather); g.E = (int)E; g.y = b.h; g.y1 = taps ? taps->y1 : nullptr;
    if ((st = launch_id<ID_SWIGLU>(g, (int)I, s, "moe gate/up")) != LQ_OK) return st;
    if ((st = launch_q8_quantize(b.h, S * (I / 32), b.hq, b.hd, s)) != LQ_OK) return st;
    if ((st = launch_id_gathered(m->w_down.qs, m->w_down.d, H, I, E, b.hq, b.hd, 1, k, b.gather, b.y2, s)) != LQ_OK)
        return st;
    return launch_moe_weighted_sum(b.y2, b.w, T, k, H, b.ids, m->expert_scale, m->n_experts, out, s);
}

// ---- whole block, GGML-format experts ------------------------------------------
namespace {
struct GgmlMat {
    QkMat m;
    int fmt;
    int64_t rows, cols;
};

lq_status ggml_mat(const char* fn, const char* what, int32_t fmt, const lq_q4_0_weight& q4,
                   const lq_q6_k_weight& q6, int64_t rows, int64_t cols, GgmlMat* out) {
    if (fmt == LQ_FMT_Q4_0) {
        if (q4.rows != rows || q4.cols != cols || cols % 32)
            return fail(LQ_ERR_SHAPE, "%s: %s Q4_0 weight is %lld x %lld, need %lld x %lld (cols %% 32 == 0)", fn,
                        what, (long long)q4.rows, (long long)q4.cols, (long long)rows, (long long)cols);
        if (!q4.qs || !q4.d) return fail(LQ_ERR_NULL, "%s: %s: NULL weight array", fn, what);
        if (!aligned(q4.qs, 16) || !aligned(q4.d, 2)) return fail(LQ_ERR_ALIGN, "%s: %s: qs must be 16-byte aligned", fn, what);
        *out = GgmlMat{QkMat{q4.qs, nullptr, nullptr, q4.d}, QK_Q4_0, rows, cols};
        return LQ_OK;
    }
    if (fmt == LQ_FMT_Q6_K) {
        if (q6.rows != rows || q6.cols != cols || cols % 256)
            return fail(LQ_ERR_SHAPE, "%s: %s Q6_K weight is %lld x %lld, need %lld x %lld (cols %% 256 == 0)", fn,
                        what, (long long)q6.rows, (long long)q6.cols, (long long)rows, (long long)cols);
        if (!q6.ql || !q6.qh || !q6.sc || !q6.d) return fail(LQ_ERR_NULL, "%s: %s: NULL weight array", fn, what);
        if (!aligned(q6.ql, 16) || !aligned(q6.qh, 16) || !aligned(q6.sc, 8) || !aligned(q6.d, 2))
            return fail(LQ_ERR_ALIGN, "%s: %s: ql and qh must be 16-byte aligned, sc 8-byte aligned", fn, what);
        *out = GgmlMat{QkMat{q6.ql, q6.qh, q6.sc, q6.d}, QK_Q6_K, rows, cols};
        return LQ_OK;
    }
    return fail(LQ_ERR_SHAPE, "%s: %s format %d (LQ_FMT_Q4_0 or LQ_FMT_Q6_K)", fn, what, (int)fmt);
}

lq_status launch_ggml_id(const GgmlMat& g, int64_t E, const int8_t* xq, const uint16_t* xd, int32_t x_per_slot,
                         int64_t k, const void* ws, float* y, hipStream_t s) {
    if (g.fmt == QK_Q4_0) return launch_qk_id_gathered<QK_Q4_0>(g.m, g.rows, g.cols, E, xq, xd, x_per_slot, k, ws, y, s);
    return launch_qk_id_gathered<QK_Q6_K>(g.m, g.rows, g.cols, E, xq, xd, x_per_slot, k, ws, y, s);
}

// the buffers are those of the Q8_0 block of the same sizes
lq_moe_desc as_q8_desc(const lq_moe_ggml_desc* m) {
    lq_moe_desc d{};
    d.hidden = m->hidden; d.ffn = m->ffn; d.n_experts = m->n_experts; d.top_k = m->top_k;
    d.expert_scale = m->expert_scale;
    return d;
}
}  // namespace

extern "C" size_t lq_moe_block_ggml_workspace_size(const lq_moe_ggml_desc* m, int64_t T) {
    if (!m || T < 0 || m->top_k <= 0 || m->n_experts <= 0) return 0;
    const lq_moe_desc d = as_q8_desc(m);
    return moe_layout(&d, T, nullptr, nullptr).total;
}

extern "C" lq_status lq_moe_block_ggml(const lq_moe_ggml_desc* m, const float* x, const float* logits, int64_t T,
                                       float* out, const lq_moe_taps* taps, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    const char* fn = "lq_moe_block_ggml";
    if (!m) return fail(LQ_ERR_NULL, "%s: descriptor is NULL", fn);
    const int64_t H = m->hidden, I = m->ffn, E = m->n_experts, k = m->top_k;
    if (T < 0 || H <= 0 || I <= 0 || H % 32 || I % 32 || k <= 0 || k > E)
        return fail(LQ_ERR_SHAPE, "%s: T=%lld hidden=%lld ffn=%lld E=%lld k=%lld", fn, (long long)T, (long long)H,
                    (long long)I, (long long)E, (long long)k);
    GgmlMat gu{}, dn{};
    lq_status st = ggml_mat(fn, "gate_up", m->gate_up_format, m->gate_up_q4_0, m->gate_up_q6_k, 2 * I, H, &gu);
    if (st == LQ_OK) st = ggml_mat(fn, "down", m->down_format, m->down_q4_0, m->down_q6_k, H, I, &dn);
    if (st != LQ_OK) return st;
    // the router in k_moe_prep holds at most 1024 logits per token
    if (H > 8192 || I > 8192 || E > 1024 || k > 32 || 2 * I * E > 0x7fffffffLL || H * E > 0x7fffffffLL)
        return fail(LQ_ERR_UNSUPPORTED, "%s: hidden and ffn <= 8192, E <= 1024, k <= 32", fn);
    if (T * k > kMoeMaxSlots) return fail(LQ_ERR_UNSUPPORTED, "%s: T*k > %d", fn, kMoeMaxSlots);
    if (T == 0) return LQ_OK;
    if (!x || !logits || !out) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x, 16) || !aligned(logits, 4) || !aligned(out, 4) || !aligned(m->expert_scale, 4))
        return fail(LQ_ERR_ALIGN, "%s: x must be 16-byte aligned", fn);
    const lq_moe_desc d = as_q8_desc(m);
    const size_t need = moe_layout(&d, T, nullptr, nullptr).total;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (256-byte aligned), got %zu", fn, need,
                    workspace_bytes);
    MoeBuffers b = moe_layout(&d, T, static_cast<char*>(workspace), taps);
    hipStream_t s = as_stream(stream);
    const int64_t prep_grid = 1 + (T * (H / 32) + kPrepQuantBlocks - 1) / kPrepQuantBlocks;
    hipLaunchKernelGGL(k_moe_prep, dim3((unsigned)prep_grid), dim3(kGatherThreads), 0, s, logits, x, (int)T, (int)E,
                       (int)k, (int)H, b.ids, b.w, static_cast<int32_t*>(b.gather), b.xq, b.xd, b.y1, 2 * I, b.y2, H);
    if ((st = check_launch("moe_prep")) != LQ_OK) return st;
    // gate/up, then SwiGLU + Q8_0 of h in a launch of its own (measured: a
    // gate/up id-matvec with the SwiGLU and Q8_0 epilogue, one workgroup per
    // 32 outputs as the Q8_0 block does it, was slower on these formats)
    if ((st = launch_ggml_id(gu, E, b.xq, b.xd, 0, k, b.gather, b.y1, s)) != LQ_OK) return st;
    if ((st = launch_swiglu_q8(b.y1, T * k, I, b.hq, b.hd, s)) != LQ_OK) return st;
    if ((st = launch_ggml_id(dn, E, b.hq, b.hd, 1, k, b.gather, b.y2, s)) != LQ_OK) return st;
    return launch_moe_weighted_sum(b.y2, b.w, T, k, H, b.ids, m->expert_scale, m->n_experts, out, s);
}

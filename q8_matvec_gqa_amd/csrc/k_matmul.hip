// k_matmul.hip -- multi-token Q8_0 matmul on gfx950 int8 MFMA.
//
// What it computes ("Design: lattice-inference", Current Design: the Q8_0
// path multiplies int8 weights by int8 activations with int32 accumulation,
// one scale per 32 values; the same product as the decode matvec, for T
// tokens at once, as in prefill or batched decode):
//     Y[t, r] = sum_b f16(dW[r, b]) * f16(dX[t, b]) * sum_{i<32} W[r, 32b+i] * X[t, 32b+i]
//     (+ residual[t, r])
//
// With T >= 16-32 tokens every weight byte feeds T multiply-adds, so the
// block dots form a dense int8 contraction: v_mfma_i32_32x32x32_i8 computes a
// 32-token x 32-row tile of one 32-value block (K = 32 is exactly one Q8_0
// block, so each MFMA result is one block dot per (token, row) and takes its
// two scales before the next block is added).
//
// Memory mapping.  The MFMA operands span 32 rows (lane l holds 16 bytes of
// row l % 32), but reading them that way sends every load instruction to 32
// rows cols bytes apart, and the weight and scale streams then crawl.  So a
// workgroup (4 waves, 32 rows) reads each batch of 16 blocks -- 512
// contiguous bytes of every row of W and X, and the matching runs of both
// scale arrays -- with row-contiguous 16-byte loads, stages them in padded
// LDS tiles (the 16-byte pad puts the 8 rows one b128 read phase touches on
// distinct banks), and each wave runs the MFMAs of a quarter of the batch's
// blocks from LDS.  The next batch's loads are in flight while the current
// one is computed.  The waves' partial tiles are summed in LDS in a fixed
// order.  Few row tiles (a short weight) split the blocks over several
// workgroups per tile; each writes its partial tile to the workspace and an
// ordered reduce launch adds them (and the residual), so results do not
// depend on timing.
#include "lq_device.h"
#include "lq_internal.h"

namespace lq {

namespace {

typedef int v4i_mm __attribute__((ext_vector_type(4)));
typedef int v16i_mm __attribute__((ext_vector_type(16)));
typedef float v16f_mm __attribute__((ext_vector_type(16)));
typedef _Float16 v8h_mm __attribute__((ext_vector_type(8)));
typedef _Float16 v4h_mm __attribute__((ext_vector_type(4)));
typedef int v2i_mm __attribute__((ext_vector_type(2)));

constexpr int kMmTok = 32;                  // tokens per launch (MFMA M); the host loops over chunks
constexpr int kMmKB = 8;                    // Q8_0 blocks per batch: 256 bytes of every row
constexpr int kMmRB = kMmKB * 32 + 16;      // LDS row stride in bytes (16-byte pad)
constexpr int kMmSS = 34;                   // LDS stride of one block's 32 f16 scales
constexpr int kMmNT = 256;                  // 4 waves
constexpr int kMmMaxBlocks = 512;           // cols <= 16384
constexpr int kMmTargetWG = kNumCUs * 3;    // workgroups a launch aims for (3 fit per CU)
constexpr int kMmMaxSplit = 4;              // workgroups per row tile at most

struct MmArgs {
    const int8_t* wq;
    const uint16_t* wd;
    int rows, cols;
    const int8_t* xq;       // [T, cols]
    const uint16_t* xd;     // [T, cols/32]
    int T;                  // tokens (the kernel narrows it to its 32-token chunk)
    const float* res;       // [T, ld] or NULL (ks == 1 only)
    float* y;               // [T, ld] (ks == 1 only)
    int64_t ld;             // row stride of res / y (elements)
    float* part;            // ks > 1: [ks][kMmTok][rows] partial sums
    int ks, bpw;            // workgroups per row tile, blocks per workgroup
    int tiles, nchunk;      // row tiles; 32-token chunks (nchunk > 1 needs ks == 1)
};

// One batch in registers, per thread: kMmNL 16-byte chunks of W and of X,
// kMmNS weight and activation scales.
constexpr int kMmCPR = 2 * kMmKB;                  // 16-byte chunks per row and batch
constexpr int kMmNL = 32 * kMmCPR / kMmNT;         // chunk loads per thread and matrix
constexpr int kMmNS = 32 * kMmKB / kMmNT;          // scales per thread and matrix
struct MmStage {
    int4 w[kMmNL], x[kMmNL];
    uint32_t dw[kMmNS], dx[kMmNS];
};

// A batch's loads (blocks [bs, bs + kMmKB) of every row of the tile).  Load j
// of thread tid takes 16-byte chunk idx % kMmCPR of row idx / kMmCPR (idx =
// tid + 256j), so each wave instruction reads whole contiguous row runs;
// scales likewise (consecutive lanes read one row's consecutive scales).
// They go through buffer resources over the tile's W rows and X tokens
// (built once per workgroup): rows or tokens past the matrix, and the bytes
// past the last row's end that a final partial batch touches, read as zeros
// without a memory access (the range check); chunks of blocks past the
// batch's end read the next blocks of the row and are zeroed through their
// scales.  The per-lane offsets are fixed for the tile and a batch adds only
// its start: one add per load, no 64-bit address arithmetic.  NL / NS:
// chunk loads and scale loads per thread and matrix; R: rows of the tile.
template <int NL, int NS>
struct MmSrc {
    __amdgpu_buffer_rsrc_t w, x, dw, dx;
    uint32_t off[NL];     // row * cols + 16 * chunk
    uint32_t doff[NS];    // 2 * (row * nb + block)
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mm_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int NL, int NS, int R>
__device__ __forceinline__ void mm_src(const MmArgs& a, int row0, int t0, int Tc, int tid, MmSrc<NL, NS>& S) {
    const int nb = a.cols >> 5;
    const int nr = a.rows - row0 < R ? a.rows - row0 : R;
    S.w = mm_rsrc(a.wq + (int64_t)row0 * a.cols, (uint32_t)nr * (uint32_t)a.cols);
    S.x = mm_rsrc(a.xq + (int64_t)t0 * a.cols, (uint32_t)Tc * (uint32_t)a.cols);
    S.dw = mm_rsrc(a.wd + (int64_t)row0 * nb, 2u * (uint32_t)nr * (uint32_t)nb);
    S.dx = mm_rsrc(a.xd + (int64_t)t0 * nb, 2u * (uint32_t)Tc * (uint32_t)nb);
    const int c = tid % kMmCPR;
#pragma unroll
    for (int j = 0; j < NL; ++j) S.off[j] = (uint32_t)((tid + kMmNT * j) / kMmCPR) * (uint32_t)a.cols + 16u * c;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        const int idx = tid + kMmNT * i;
        S.doff[i] = 2u * ((uint32_t)(idx / kMmKB) * (uint32_t)nb + (uint32_t)(idx % kMmKB));
    }
}
template <int NL, int NS>
__device__ __forceinline__ void mm_load_b(const MmSrc<NL, NS>& R, int bs, int4 (&w)[NL], int4 (&x)[NL],
                                          uint32_t (&dw)[NS], uint32_t (&dx)[NS]) {
    const uint32_t cb = (uint32_t)bs * 32u, db = 2u * (uint32_t)bs;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const auto vw = __builtin_amdgcn_raw_buffer_load_b128(R.w, (int)(R.off[j] + cb), 0, 2);   // nontemporal
        const auto vx = __builtin_amdgcn_raw_buffer_load_b128(R.x, (int)(R.off[j] + cb), 0, 0);
        w[j] = make_int4((int)vw[0], (int)vw[1], (int)vw[2], (int)vw[3]);
        x[j] = make_int4((int)vx[0], (int)vx[1], (int)vx[2], (int)vx[3]);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        dw[i] = __builtin_amdgcn_raw_buffer_load_b16(R.dw, (int)(R.doff[i] + db), 0, 0);
        dx[i] = __builtin_amdgcn_raw_buffer_load_b16(R.dx, (int)(R.doff[i] + db), 0, 0);
    }
}


// LDS: W tile [32 rows][kMmRB], X tile [32 tokens][kMmRB], scales as f16
// bits [block][kMmSS] (row or token fastest), zero for blocks past be and
// tokens past T.
__device__ __forceinline__ void mm_store(const MmArgs& a, int bs, int be, int tid, const MmStage& S, int8_t* wl,
                                         int8_t* xl, uint16_t* dwl, uint16_t* dxl) {
    const int c = tid % kMmCPR;
#pragma unroll
    for (int j = 0; j < kMmNL; ++j) {
        const int r = (tid + kMmNT * j) / kMmCPR;
        *reinterpret_cast<int4*>(wl + r * kMmRB + 16 * c) = S.w[j];
        *reinterpret_cast<int4*>(xl + r * kMmRB + 16 * c) = S.x[j];
    }
#pragma unroll
    for (int i = 0; i < kMmNS; ++i) {
        const int idx = tid + kMmNT * i, rr = idx / kMmKB, u = idx % kMmKB;
        const bool uv = bs + u < be;
        dwl[u * kMmSS + rr] = uv ? (uint16_t)S.dw[i] : (uint16_t)0;
        dxl[u * kMmSS + rr] = (uv && rr < a.T) ? (uint16_t)S.dx[i] : (uint16_t)0;
    }
}

__global__ __launch_bounds__(kMmNT, 3) void k_q8_matmul(MmArgs args) {
    __shared__ __attribute__((aligned(16))) int8_t tiles[2 * 32 * kMmRB];   // W tile, then X tile
    int8_t* const wl = tiles;
    int8_t* const xl = tiles + 32 * kMmRB;
    __shared__ __attribute__((aligned(16))) uint16_t dwl[kMmKB * kMmSS];
    __shared__ __attribute__((aligned(16))) uint16_t dxl[kMmKB * kMmSS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, half = lane >> 5;
    // Which row tile, block split and token chunk.  With several chunks the
    // workgroups of one tile's chunks sit next to each other in dispatch
    // order on one XCD (workgroups go round-robin over the 8 XCDs), so the
    // tile's weight rows, read by all of them at about the same time, come
    // from that XCD's L2 after the first read.
    MmArgs a = args;
    int tile, split = 0;
    if (a.nchunk == 1) {
        tile = blockIdx.x / a.ks;
        split = blockIdx.x % a.ks;
    } else {
        const int x = blockIdx.x & 7, q = blockIdx.x >> 3;
        const int chunk = q % a.nchunk;
        tile = 8 * (q / a.nchunk) + x;
        if (tile >= a.tiles) return;          // padding of the grid to whole XCD rounds
        const int64_t t0 = (int64_t)chunk * kMmTok;
        a.xq += t0 * a.cols;
        a.xd += t0 * (a.cols >> 5);
        if (a.res) a.res += t0 * a.ld;
        a.y += t0 * a.ld;
        a.T = a.T - (int)t0 < kMmTok ? a.T - (int)t0 : kMmTok;
    }
    const int row0 = tile * 32;
    const int nb = a.cols >> 5;
    const int b0 = split * a.bpw, b1 = b0 + a.bpw < nb ? b0 + a.bpw : nb;   // host: b0 < b1

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    // Batches in a rotated order: tile t starts at batch t mod nbt, so the
    // workgroups that run side by side read different parts of X (every
    // workgroup reads all of X; in lockstep they would all hit the same few
    // cache lines at once).  The order is fixed per tile (deterministic).
    // Two batches are in flight in registers (P, Q): batch i + 2 is requested
    // as soon as batch i sits in LDS, so the loads never pause while a batch
    // is stored and computed.
    const int nbt = (b1 - b0 + kMmKB - 1) / kMmKB;
    const int rot = tile % nbt;
    auto batch_start = [&](int i) {
        const int j = i + rot < nbt ? i + rot : i + rot - nbt;
        return b0 + kMmKB * j;
    };
    auto batch_end = [&](int bs) { return bs + kMmKB < b1 ? bs + kMmKB : b1; };
    // this wave's blocks of the batch: wave, wave + 4, ...; per block an int8
    // MFMA (the block dots) and an f16 MFMA whose only nonzero k term forms
    // the scale products f16(dX[t]) * f16(dW[r]) (exact in f32) in the same
    // tile layout.  Lane holds tokens 8*(i/4) + 4*half + i%4 of row n.
    auto compute = [&]() {
#pragma unroll
        for (int k = 0; k < kMmKB / 4; ++k) {
            const int u = wave + 4 * k;
            const v4i_mm A = *reinterpret_cast<const v4i_mm*>(xl + n * kMmRB + 32 * u + 16 * half);
            const v4i_mm B = *reinterpret_cast<const v4i_mm*>(wl + n * kMmRB + 32 * u + 16 * half);
            const int xs = dxl[u * kMmSS + n], ws = dwl[u * kMmSS + n];
            const v16i_mm c = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, v16i_mm{}, 0, 0, 0);
            const v2i_mm As = {half ? 0 : xs, 0}, Bs = {half ? 0 : ws, 0};
            const v16f_mm sc = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h_mm, As),
                                                                    __builtin_bit_cast(v4h_mm, Bs), v16f_mm{}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf((float)c[i], sc[i], acc[i]);
        }
    };
    MmSrc<kMmNL, kMmNS> src;
    mm_src<kMmNL, kMmNS, 32>(a, row0, 0, a.T, tid, src);
    auto step = [&](int i, MmStage& S) {
        const int bs = batch_start(i), be = batch_end(bs);
        if (i > 0) __syncthreads();          // every wave is done with the previous batch
        mm_store(a, bs, be, tid, S, wl, xl, dwl, dxl);
        __syncthreads();
        if (i + 2 < nbt) mm_load_b(src, batch_start(i + 2), S.w, S.x, S.dw, S.dx);
        compute();
    };
    MmStage P, Q;
    mm_load_b(src, batch_start(0), P.w, P.x, P.dw, P.dx);
    if (nbt > 1) mm_load_b(src, batch_start(1), Q.w, Q.x, Q.dw, Q.dx);
    for (int i = 0; i < nbt; i += 2) {
        step(i, P);
        if (i + 1 < nbt) step(i + 1, Q);
    }
    // the 4 waves' partial tiles, summed in wave order; thread = (token, row)
    __syncthreads();
    static_assert(4 * 1024 * sizeof(float) <= sizeof(tiles), "partial tiles fit the W and X tiles");
    float* red = reinterpret_cast<float*>(tiles);  // [4][32 tokens][32 rows]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave * 1024 + (8 * (r / 4) + 4 * half + (r & 3)) * 32 + n] = acc[r];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int i = tid + kMmNT * k, t = i >> 5, row = row0 + (i & 31);
        if (t < a.T && row < a.rows) {
            const float s = ((red[i] + red[1024 + i]) + red[2048 + i]) + red[3072 + i];
            if (a.ks == 1) {
                const int64_t o = (int64_t)t * a.ld + row;
                a.y[o] = a.res ? a.res[o] + s : s;
            } else {
                a.part[((int64_t)split * kMmTok + t) * a.rows + row] = s;
            }
        }
    }
}

// ---- wide tiles for longer token batches (prefill) ----------------------------
// With more than 32 tokens a workgroup owns 64 rows x 64 tokens: each batch
// of W and X rows staged in LDS feeds two row tiles and two token tiles, so
// every staged byte serves twice the MFMAs of the 32 x 32 tile.  Wave w
// owns output sub-tile (rows 32*(w&1).., tokens 32*(w>>1)..) over all the
// batch's blocks: no cross-wave reduction.  Same row-contiguous loads and
// rotated batch order as the 32 x 32 kernel, but one batch in flight in
// registers (three workgroups per CU hide the latency better than a second
// batch in one) and the smaller scale MFMA.
constexpr int kMwR = 64, kMwT = 64;
constexpr int kMwNL = kMwR * kMmCPR / kMmNT;     // W (and X) 16-byte chunks per thread and batch
constexpr int kMwNS = kMwR * kMmKB / kMmNT;      // W (and X) scales per thread and batch
constexpr int kMwSS = 66;                        // LDS stride of one block's 64 f16 scales

struct MwStage {
    int4 w[kMwNL], x[kMwNL];
    uint32_t dw[kMwNS], dx[kMwNS];
};

__device__ __forceinline__ void mw_store(int Tc, int bs, int be, int tid, const MwStage& S, int8_t* wl, int8_t* xl,
                                         uint16_t* dwl, uint16_t* dxl) {
    const int c = tid % kMmCPR;
#pragma unroll
    for (int j = 0; j < kMwNL; ++j) {
        const int r = (tid + kMmNT * j) / kMmCPR;
        *reinterpret_cast<int4*>(wl + r * kMmRB + 16 * c) = S.w[j];
        *reinterpret_cast<int4*>(xl + r * kMmRB + 16 * c) = S.x[j];
    }
#pragma unroll
    for (int i = 0; i < kMwNS; ++i) {
        const int idx = tid + kMmNT * i, rr = idx / kMmKB, u = idx % kMmKB;
        const bool uv = bs + u < be;
        dwl[u * kMwSS + rr] = uv ? (uint16_t)S.dw[i] : (uint16_t)0;
        dxl[u * kMwSS + rr] = (uv && rr < Tc) ? (uint16_t)S.dx[i] : (uint16_t)0;
    }
}

// grid: 8 * nchunk * ceil(tiles / 8) over 64-row tiles and 64-token chunks,
// a tile's chunks adjacent on one XCD
__global__ __launch_bounds__(kMmNT, 3) void k_q8_matmul_wide(MmArgs a) {
    __shared__ __attribute__((aligned(16))) int8_t wl[kMwR * kMmRB];
    __shared__ __attribute__((aligned(16))) int8_t xl[kMwT * kMmRB];
    __shared__ __attribute__((aligned(16))) uint16_t dwl[kMmKB * kMwSS];
    __shared__ __attribute__((aligned(16))) uint16_t dxl[kMmKB * kMwSS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 31, half = lane >> 5;
    const int x8 = blockIdx.x & 7, q = blockIdx.x >> 3;
    const int chunk = q % a.nchunk, tile = 8 * (q / a.nchunk) + x8;
    if (tile >= a.tiles) return;                  // padding of the grid to whole XCD rounds
    const int row0 = tile * kMwR, t0 = chunk * kMwT;
    const int Tc = a.T - t0 < kMwT ? a.T - t0 : kMwT;
    const int nb = a.cols >> 5;
    const int rt = wave & 1, tt = wave >> 1;      // this wave's output sub-tile

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    const int nbt = (nb + kMmKB - 1) / kMmKB;
    const int rot = tile % nbt;
    auto batch_start = [&](int i) {
        const int j = i + rot < nbt ? i + rot : i + rot - nbt;
        return kMmKB * j;
    };
    auto batch_end = [&](int bs) { return bs + kMmKB < nb ? bs + kMmKB : nb; };
    // Block u: the block dots (i8 MFMA) and the scale products from the
    // smallest f16 MFMA (32x32x8: two-register operands), its only nonzero k
    // term f16(dX[t]) * f16(dW[r]).  Block u + 1's operands are read from LDS
    // while block u is rescaled, so the LDS latency hides behind the
    // converts and FMAs.
    auto lds_ops = [&](int u, v4i_mm& A, v4i_mm& B, int& xs, int& ws) {
        A = *reinterpret_cast<const v4i_mm*>(xl + (tt * 32 + n) * kMmRB + 32 * u + 16 * half);
        B = *reinterpret_cast<const v4i_mm*>(wl + (rt * 32 + n) * kMmRB + 32 * u + 16 * half);
        xs = dxl[u * kMwSS + tt * 32 + n];
        ws = dwl[u * kMwSS + rt * 32 + n];
    };
    auto compute = [&]() {
        v4i_mm A, B;
        int xs, ws;
        lds_ops(0, A, B, xs, ws);
#pragma unroll
        for (int u = 0; u < kMmKB; ++u) {
            const v16i_mm c = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, v16i_mm{}, 0, 0, 0);
            const v2i_mm As = {half ? 0 : xs, 0}, Bs = {half ? 0 : ws, 0};
            const v16f_mm sc = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(v4h_mm, As),
                                                                    __builtin_bit_cast(v4h_mm, Bs), v16f_mm{}, 0, 0, 0);
            if (u + 1 < kMmKB) lds_ops(u + 1, A, B, xs, ws);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf((float)c[i], sc[i], acc[i]);
        }
    };
    MmSrc<kMwNL, kMwNS> src;
    mm_src<kMwNL, kMwNS, kMwR>(a, row0, t0, Tc, tid, src);
    auto step = [&](int i, MwStage& S) {
        const int bs = batch_start(i), be = batch_end(bs);
        if (i > 0) __syncthreads();
        mw_store(Tc, bs, be, tid, S, wl, xl, dwl, dxl);
        __syncthreads();
        if (i + 1 < nbt) mm_load_b(src, batch_start(i + 1), S.w, S.x, S.dw, S.dx);
        compute();
    };
    // one batch in flight in registers (the next batch's loads overlap this
    // batch's math)
    MwStage P;
    mm_load_b(src, batch_start(0), P.w, P.x, P.dw, P.dx);
    for (int i = 0; i < nbt; ++i) step(i, P);
    // lane holds tokens 8*(r/4) + 4*half + r%4 of row n of the sub-tile
    const int row = row0 + rt * 32 + n;
    if (row < a.rows) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int t = tt * 32 + 8 * (r / 4) + 4 * half + (r & 3);
            if (t < Tc) {
                const int64_t o = (int64_t)(t0 + t) * a.ld + row;
                a.y[o] = a.res ? a.res[o] + acc[r] : acc[r];
            }
        }
    }
}

// y[t, r] = residual[t, r] + sum over the splits in order; V consecutive
// rows per thread (V = 4 needs rows % 4 == 0), every split's load issued
// before the sum.
template <int V>
__global__ __launch_bounds__(256) void k_q8_matmul_reduce(const float* __restrict__ part, int ks, int T, int rows,
                                                          const float* res, float* y, int64_t ld) {
    typedef float vf __attribute__((ext_vector_type(V)));
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
    if (i >= (int64_t)T * rows) return;
    const int t = (int)(i / rows), r = (int)(i % rows);
    vf p[kMmMaxSplit];
#pragma unroll
    for (int k = 0; k < kMmMaxSplit; ++k)
        p[k] = k < ks ? *reinterpret_cast<const vf*>(part + ((int64_t)k * kMmTok + t) * rows + r) : vf{};
    vf s = p[0];
#pragma unroll
    for (int k = 1; k < kMmMaxSplit; ++k) s += p[k];
    const int64_t o = (int64_t)t * ld + r;
    if (res) s += *reinterpret_cast<const vf*>(res + o);
    *reinterpret_cast<vf*>(y + o) = s;
}

// Workgroups per row tile and blocks per workgroup: a short weight splits
// its blocks (in whole batches, at most kMmMaxSplit ways) so that the grid
// fills but does not exceed one resident round.  More than 32 tokens fill
// the grid with token chunks instead: no split.
void mm_plan(int64_t rows, int64_t cols, int64_t T, int* ks, int* bpw) {
    const int64_t tiles = (rows + 31) / 32, nb = cols / 32;
    if (T > kMmTok) {
        *ks = 1;
        *bpw = (int)nb;
        return;
    }
    int best_k = 1;
    int64_t best_b = nb;
    for (int k = 2; k <= kMmMaxSplit; ++k) {
        int64_t b = (nb + k - 1) / k;
        if (nb > kMmKB) b = (b + kMmKB - 1) / kMmKB * kMmKB;
        const int64_t kk = (nb + b - 1) / b;
        if (tiles * kk > kMmTargetWG) break;
        if (kk > best_k) best_k = (int)kk, best_b = b;
    }
    *bpw = (int)best_b;
    *ks = best_k;
}

}  // namespace

}  // namespace lq

using namespace lq;

extern "C" size_t lq_q8_matmul_workspace_size(int64_t rows, int64_t cols, int64_t T) {
    if (rows <= 0 || cols <= 0 || T <= 0 || cols % 32 || cols > 32 * kMmMaxBlocks) return 0;
    int ks, bpw;
    mm_plan(rows, cols, T, &ks, &bpw);
    return ks > 1 ? (size_t)ks * kMmTok * (size_t)rows * sizeof(float) : 0;
}

extern "C" lq_status lq_q8_matmul(const lq_q8_weight* w, const int8_t* x_qs, const uint16_t* x_d, int64_t T,
                                  const float* residual, float* y, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    const char* fn = "lq_q8_matmul";
    lq_status st = check_weight(w, fn);
    if (st != LQ_OK) return st;
    if (T < 0) return fail(LQ_ERR_SHAPE, "%s: T=%lld", fn, (long long)T);
    if (T > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "%s: T=%lld (< 2^31)", fn, (long long)T);
    if (w->cols > 32 * kMmMaxBlocks || w->rows > 0x7fffffffLL)
        return fail(LQ_ERR_UNSUPPORTED, "%s: cols=%lld rows=%lld (cols <= %d)", fn, (long long)w->cols,
                    (long long)w->rows, 32 * kMmMaxBlocks);
    if (T == 0 || w->rows == 0) return LQ_OK;
    if (!x_qs || !x_d || !y) return fail(LQ_ERR_NULL, "%s: NULL pointer", fn);
    if (!aligned(x_qs, 16) || !aligned(x_d, 2) || !aligned(y, 4) || (residual && !aligned(residual, 4)))
        return fail(LQ_ERR_ALIGN, "%s: x_qs must be 16-byte aligned", fn);
    const size_t need = lq_q8_matmul_workspace_size(w->rows, w->cols, T);
    if (need && (!workspace || workspace_bytes < need || !aligned(workspace, 4)))
        return fail(LQ_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
    const hipStream_t s = as_stream(stream);
    const int64_t rows = w->rows, cols = w->cols, nb = cols / 32;
    int ks, bpw;
    mm_plan(rows, cols, T, &ks, &bpw);
    // 64 x 64 tiles once they fill two workgroups per CU; fewer of them
    // leave CUs idle, and the 32 x 32 tiles (every 32-token chunk in one
    // launch) do better there
    const int64_t wtiles = (rows + kMwR - 1) / kMwR, wchunks = (T + kMwT - 1) / kMwT;
    if (T > kMmTok && wtiles * wchunks >= 2 * kNumCUs) {
        const int64_t tiles = wtiles, nchunk = wchunks;
        const int64_t grid = 8 * nchunk * ((tiles + 7) / 8);
        if (grid > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "%s: T=%lld too large", fn, (long long)T);
        MmArgs a{w->qs, w->d, (int)rows, (int)cols, x_qs, x_d, (int)T, residual, y, rows, nullptr, 1, (int)nb,
                 (int)tiles, (int)nchunk};
        hipLaunchKernelGGL(k_q8_matmul_wide, dim3((unsigned)grid), dim3(kMmNT), 0, s, a);
        return check_launch(fn);
    }
    const int64_t tiles = (rows + 31) / 32, nchunk = (T + kMmTok - 1) / kMmTok;
    const int64_t grid = nchunk == 1 ? tiles * ks : 8 * nchunk * ((tiles + 7) / 8);
    if (grid > 0x7fffffffLL) return fail(LQ_ERR_UNSUPPORTED, "%s: T=%lld too large", fn, (long long)T);
    MmArgs a{w->qs, w->d, (int)rows, (int)cols, x_qs, x_d, (int)T, residual, y, rows,
             static_cast<float*>(workspace), ks, bpw, (int)tiles, (int)nchunk};
    hipLaunchKernelGGL(k_q8_matmul, dim3((unsigned)grid), dim3(kMmNT), 0, s, a);
    if (ks > 1) {                                  // T <= 32: one chunk
        const int64_t n = T * rows;
        const bool v4 = rows % 4 == 0 && aligned(y, 16) && (!residual || aligned(residual, 16)) &&
                        aligned(workspace, 16);
        if (v4)
            hipLaunchKernelGGL(k_q8_matmul_reduce<4>, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, s,
                               static_cast<const float*>(workspace), ks, (int)T, (int)rows, residual, y, rows);
        else
            hipLaunchKernelGGL(k_q8_matmul_reduce<1>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                               static_cast<const float*>(workspace), ks, (int)T, (int)rows, residual, y, rows);
    }
    st = check_launch(fn);
    if (st != LQ_OK) return st;
    return LQ_OK;
}

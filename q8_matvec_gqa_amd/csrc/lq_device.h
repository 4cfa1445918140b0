// lq_device.h -- device helpers shared by the gfx950 kernels of liblq.
//
// Wavefront-64 reductions use DPP row permutes inside each 16-lane row and
// gfx950's v_permlane16_swap / v_permlane32_swap across rows, so no LDS
// round trip is needed for a full-wave reduction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lq {

constexpr int kWave = 64;

// ---- number formats --------------------------------------------------------
__device__ __forceinline__ float f16_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
// v_cvt_f16_f32: round to nearest even, f16 subnormals kept (f16 denormals
// are enabled in the default gfx950 FP mode).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// f32 -> bf16, round to nearest even on the bit pattern; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---- 16-byte loads ----------------------------------------------------------
typedef int v4i_t __attribute__((ext_vector_type(4)));
// Streaming (non-temporal) 16-byte load for data read exactly once (weights).
__device__ __forceinline__ int4 load_stream16(const void* p) {
    const v4i_t v = __builtin_nontemporal_load(reinterpret_cast<const v4i_t*>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}

// ---- DPP / permlane --------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor8 = 0x128;      // row_ror:8 (within 16 lanes: lane ^ 8)

// Sum over aligned groups of N consecutive lanes (N = 2..64, power of two);
// every lane of a group receives the group sum.  The mirror steps pair lanes
// whose values are already equal across the sub-groups combined so far, so
// they act as the xor-4 / xor-8 butterfly steps.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power of two");
    if constexpr (N >= 2) v += dpp<kQuadXor1>(v);
    if constexpr (N >= 4) v += dpp<kQuadXor2>(v);
    if constexpr (N >= 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp<kRowMirror>(v);
    if constexpr (N >= 32) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if constexpr (N >= 64) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "power of two");
    if constexpr (N >= 2) v = fmaxf(v, dpp<kQuadXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp<kQuadXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp<kRowHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp<kRowMirror>(v));
    if constexpr (N >= 32) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if constexpr (N >= 64) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return v;
}

// Sums each of v[0..7] over the 64 lanes of the wave and leaves the sum of
// v[h] in the lanes with (lane >> 3) & 7 == h (a reduce-scatter: halves are
// exchanged across lane bits 5, 4 and 3, then 8-lane groups are summed).
__device__ __forceinline__ float wave_sum8_scatter(const float (&v)[8]) {
    const int lane = threadIdx.x & 63;
    float a[4], b[2];
    // bit 5: lanes 0-31 keep heads 0-3, lanes 32-63 heads 4-7
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[h]), __float_as_uint(v[h + 4]), false, false);
        a[h] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // bit 4: keep the first or second pair of the four
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[h]), __float_as_uint(a[h + 2]), false, false);
        b[h] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // bit 3: keep one of the two; the partner (lane ^ 8) sends the other
    const bool hi = (lane & 8) != 0;
    const float send = hi ? b[0] : b[1];
    const float keep = hi ? b[1] : b[0];
    float c = keep + dpp<kRowRor8>(send);
    // bits 0-2
    c += dpp<kQuadXor1>(c);
    c += dpp<kQuadXor2>(c);
    c += dpp<kRowHalfMirror>(c);
    return c;
}

// Minimum of an int over the wave (same DPP/permlane steps as group_max<64>).
__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, dpp_i<kQuadXor1>(v));
    v = min(v, dpp_i<kQuadXor2>(v));
    v = min(v, dpp_i<kRowHalfMirror>(v));
    v = min(v, dpp_i<kRowMirror>(v));
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
    v = min((int)r[0], (int)r[1]);
    r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
    return min((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// ---- Q8_0 block quantization of 32 floats held by one lane ------------------
// Scale d = amax/127 (correctly rounded float division), codes =
// round-half-away-from-zero(x * (1/d)) clamped to [-127, 127], 0 for amax 0.
// Returns the f16 scale bits; the 32 codes come back packed 4 per word.
__device__ __forceinline__ uint16_t quantize_block32_packed(const float (&v)[32], uint32_t (&packed)[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float db = amax / 127.0f;
    const float inv = (db != 0.0f) ? 1.0f / db : 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = roundf(v[4 * w + j] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            word |= ((uint32_t)(int32_t)r & 0xffu) << (8 * j);
        }
        packed[w] = word;
    }
    return f32_to_f16(db);
}

// The same quantizer with a 32-value block spread over the 4 lanes of a quad
// (8 values each, lane & 3 = quarter): the block's amax is a quad max, every
// lane packs its own 8 codes and returns the block's f16 scale.  All four
// lanes of the quad must be active.
__device__ __forceinline__ uint16_t quantize_quarter8_packed(const float (&v)[8], uint32_t (&packed)[2]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, dpp<kQuadXor1>(amax));
    amax = fmaxf(amax, dpp<kQuadXor2>(amax));
    const float db = amax / 127.0f;
    const float inv = (db != 0.0f) ? 1.0f / db : 0.0f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float r = roundf(v[4 * w + j] * inv);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            word |= ((uint32_t)(int32_t)r & 0xffu) << (8 * j);
        }
        packed[w] = word;
    }
    return f32_to_f16(db);
}

__device__ __forceinline__ void store_codes32(int8_t* qs, const uint32_t (&packed)[8]) {
    int4* q4 = reinterpret_cast<int4*>(qs);
    q4[0] = make_int4((int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]);
    q4[1] = make_int4((int)packed[4], (int)packed[5], (int)packed[6], (int)packed[7]);
}

// Quantize 32 floats and write 32 codes (two 16-byte stores) and the f16 scale.
__device__ __forceinline__ void quantize_block32(const float (&v)[32], int8_t* __restrict__ qs,
                                                 uint16_t* __restrict__ d) {
    uint32_t packed[8];
    const uint16_t db = quantize_block32_packed(v, packed);
    store_codes32(qs, packed);
    *d = db;
}

__device__ __forceinline__ void load8(const float* __restrict__ p, float (&v)[8]) {
    const float4* p4 = reinterpret_cast<const float4*>(p);
    const float4 a = p4[0], b = p4[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load32(const float* __restrict__ p, float (&v)[32]) {
    const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float4 t = p4[i];
        v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
}

}  // namespace lq

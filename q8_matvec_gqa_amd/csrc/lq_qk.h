// lq_qk.h -- device decode of Q4_0 and Q6_K weight units, shared by the
// dense matvec (k_qk.hip) and the index-driven MoE matvec (k_moe.hip).
//
// Layouts (SoA per matrix; GGML block order inside each array, as GGML's
// Q4_0 / Q6_K blocks define it -- formats named in "Current Inference Path --
// Architecture Map", section 4, and "Target Inference Architecture: hf2q on
// mlx-native", section 8, Q1):
//   Q4_0: qs [rows][cols/2], byte j of a 32-value block holds value j (low
//         nibble) and value j+16 (high nibble); d f16 [rows][cols/32].
//   Q6_K: ql [rows][cols/2], qh [rows][cols/4], sc int8 [rows][cols/16],
//         d f16 [rows][cols/256]; value i of a 256-value super-block (h =
//         i/128, g = (i%128)/32, l = i%32) has its low 4 bits in
//         ql[64h + 32(g%2) + l] (low nibble for g < 2, high for g >= 2) and its
//         high 2 bits at bits 2g, 2g+1 of qh[32h + l]; scale sc[i/16].
//
// A lane's unit: a Q4_0 block (32 values, one 16-byte load), or a quarter of
// a Q6_K super-block: the 16 positions l = 16p..16p+15 of each 32-value
// quarter g of half h (two 16-byte ql loads, one qh load; 64 values in four
// groups of 16 at value offsets v0 + 32g).  The stored bits n of each value
// (0..15 for Q4_0, 0..63 for Q6_K) go into v_dot4_i32_i8 as they are, against
// the Q8_0 activation codes; the offset (8 or 32) comes off afterwards as the
// offset times the sum of the activation codes, so the int32 dots are exact.
#pragma once
#include "lq_device.h"

namespace lq {

enum { QK_Q4_0 = 0, QK_Q6_K = 1 };

template <int FMT>
struct QkUnit;
template <>
struct QkUnit<QK_Q4_0> {
    int4 q;
    uint32_t d;
};
template <>
struct QkUnit<QK_Q6_K> {
    int4 l0, l1, h;
    uint2 sc;
    uint32_t d;
};

// One matrix's arrays (Q4_0 uses q0 = qs and d).
struct QkMat {
    const uint8_t* q0;      // Q4_0 qs / Q6_K ql
    const uint8_t* q1;      // Q6_K qh
    const int8_t* sc;       // Q6_K sub-scales
    const uint16_t* d;      // Q4_0 block scales / Q6_K super-scales
};

template <int FMT>
__host__ __device__ __forceinline__ int qk_units(int cols) { return FMT == QK_Q4_0 ? cols >> 5 : cols >> 6; }

// Loads of unit u of row r.
__device__ __forceinline__ void qk_load_unit(const QkMat& m, int cols, int64_t r, int u, QkUnit<QK_Q4_0>& U) {
    U.q = load_stream16(m.q0 + r * (cols >> 1) + 16 * u);
    U.d = m.d[r * (cols >> 5) + u];
}
__device__ __forceinline__ void qk_load_unit(const QkMat& m, int cols, int64_t r, int u, QkUnit<QK_Q6_K>& U) {
    const int sb = u >> 2, h = (u >> 1) & 1, p = u & 1;
    const uint8_t* ql = m.q0 + r * (cols >> 1) + sb * 128 + h * 64 + p * 16;
    U.l0 = load_stream16(ql);
    U.l1 = load_stream16(ql + 32);
    U.h = load_stream16(m.q1 + r * (cols >> 2) + sb * 64 + h * 32 + p * 16);
    U.sc = *reinterpret_cast<const uint2*>(m.sc + r * (cols >> 4) + sb * 16 + h * 8);
    U.d = m.d[r * (cols >> 8) + sb];
}

__device__ __forceinline__ int qk_dot16(const int (&w)[4], const int4 x) {
    int s = __builtin_amdgcn_sdot4(w[0], x.x, 0, false);
    s = __builtin_amdgcn_sdot4(w[1], x.y, s, false);
    s = __builtin_amdgcn_sdot4(w[2], x.z, s, false);
    return __builtin_amdgcn_sdot4(w[3], x.w, s, false);
}

// Q6_K: first value of unit u's group 0 (groups g at + 32g, 16 values each;
// each group lies in the Q8_0 activation block (v0 >> 5) + g).
__device__ __forceinline__ int qk6_v0(int u) { return (u >> 2) * 256 + ((u >> 1) & 1) * 128 + (u & 1) * 16; }

// Q6_K: the sub-scales of unit u's four groups (byte p + 2g of the half's 8).
__device__ __forceinline__ void qk6_subscales(const QkUnit<QK_Q6_K>& U, int u, float (&c)[4]) {
    const int p = u & 1;
    const uint32_t s01 = p ? U.sc.x >> 8 : U.sc.x, s23 = p ? U.sc.y >> 8 : U.sc.y;
    c[0] = (float)(int8_t)(s01 & 0xFF);
    c[1] = (float)(int8_t)((s01 >> 16) & 0xFF);
    c[2] = (float)(int8_t)(s23 & 0xFF);
    c[3] = (float)(int8_t)((s23 >> 16) & 0xFF);
}

// A unit's activation held in registers, so that the rows of one wave share
// one load of it: Q4_0 the block's 32 codes and scale, Q6_K the four groups'
// 16 codes each and the scales of their Q8_0 blocks.
template <int FMT>
struct QkAct;
template <>
struct QkAct<QK_Q4_0> {
    int4 lo, hi;
    float s;
    int sum;        // sum of the block's 32 codes
};
template <>
struct QkAct<QK_Q6_K> {
    int4 x[4];
    float s[4];
    int sum[4];     // sum of each group's 16 codes
};
// Sum of 16 int8 codes (v_dot4 against ones).
__device__ __forceinline__ int qk_sum16(const int4 x, int acc) {
    acc = __builtin_amdgcn_sdot4(x.x, 0x01010101, acc, false);
    acc = __builtin_amdgcn_sdot4(x.y, 0x01010101, acc, false);
    acc = __builtin_amdgcn_sdot4(x.z, 0x01010101, acc, false);
    return __builtin_amdgcn_sdot4(x.w, 0x01010101, acc, false);
}
__device__ __forceinline__ void qk_load_act(const int8_t* xq, const uint16_t* xd, int u, QkAct<QK_Q4_0>& A) {
    A.lo = *reinterpret_cast<const int4*>(xq + 32 * u);
    A.hi = *reinterpret_cast<const int4*>(xq + 32 * u + 16);
    A.s = f16_to_f32(xd[u]);
    A.sum = qk_sum16(A.hi, qk_sum16(A.lo, 0));
}
__device__ __forceinline__ void qk_load_act(const int8_t* xq, const uint16_t* xd, int u, QkAct<QK_Q6_K>& A) {
    const int v0 = qk6_v0(u);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        A.x[g] = *reinterpret_cast<const int4*>(xq + v0 + 32 * g);
        A.s[g] = f16_to_f32(xd[(v0 >> 5) + g]);
        A.sum[g] = qk_sum16(A.x[g], 0);
    }
}
// The same from the activation in LDS (codes xq, f32 scales xs per block).
__device__ __forceinline__ void qk_load_act_l(const int8_t* xq, const float* xs, int u, QkAct<QK_Q4_0>& A) {
    A.lo = *reinterpret_cast<const int4*>(xq + 32 * u);
    A.hi = *reinterpret_cast<const int4*>(xq + 32 * u + 16);
    A.s = xs[u];
    A.sum = qk_sum16(A.hi, qk_sum16(A.lo, 0));
}
__device__ __forceinline__ void qk_load_act_l(const int8_t* xq, const float* xs, int u, QkAct<QK_Q6_K>& A) {
    const int v0 = qk6_v0(u);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        A.x[g] = *reinterpret_cast<const int4*>(xq + v0 + 32 * g);
        A.s[g] = xs[(v0 >> 5) + g];
        A.sum[g] = qk_sum16(A.x[g], 0);
    }
}

// The unsigned codes' dots less the offset times the activation sum: a Q4_0
// value is n - 8 and a Q6_K value n - 32 for its stored bits n, so
// sum_i (n_i - o) x_i = sum_i n_i x_i - o * sum_i x_i, exactly in int32.
// The stored bits go into v_dot4 as they are (n <= 63 is a valid int8).
__device__ __forceinline__ int qk4_dot_act(const QkUnit<QK_Q4_0>& U, const QkAct<QK_Q4_0>& A) {
    const uint32_t q[4] = {(uint32_t)U.q.x, (uint32_t)U.q.y, (uint32_t)U.q.z, (uint32_t)U.q.w};
    int lo[4], hi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo[i] = (int)(q[i] & 0x0F0F0F0Fu);
        hi[i] = (int)((q[i] >> 4) & 0x0F0F0F0Fu);
    }
    return qk_dot16(hi, A.hi) + qk_dot16(lo, A.lo) - 8 * A.sum;
}
__device__ __forceinline__ void qk6_dots_act(const QkUnit<QK_Q6_K>& U, const QkAct<QK_Q6_K>& A, int (&dots)[4]) {
    const uint32_t L0[4] = {(uint32_t)U.l0.x, (uint32_t)U.l0.y, (uint32_t)U.l0.z, (uint32_t)U.l0.w};
    const uint32_t L1[4] = {(uint32_t)U.l1.x, (uint32_t)U.l1.y, (uint32_t)U.l1.z, (uint32_t)U.l1.w};
    const uint32_t H[4] = {(uint32_t)U.h.x, (uint32_t)U.h.y, (uint32_t)U.h.z, (uint32_t)U.h.w};
    int g0[4], g1[4], g2[4], g3[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        g0[i] = (int)((L0[i] & 0x0F0F0F0Fu) | ((H[i] << 4) & 0x30303030u));
        g1[i] = (int)((L1[i] & 0x0F0F0F0Fu) | ((H[i] << 2) & 0x30303030u));
        g2[i] = (int)(((L0[i] >> 4) & 0x0F0F0F0Fu) | (H[i] & 0x30303030u));
        g3[i] = (int)(((L1[i] >> 4) & 0x0F0F0F0Fu) | ((H[i] >> 2) & 0x30303030u));
    }
    dots[0] = qk_dot16(g0, A.x[0]) - 32 * A.sum[0];
    dots[1] = qk_dot16(g1, A.x[1]) - 32 * A.sum[1];
    dots[2] = qk_dot16(g2, A.x[2]) - 32 * A.sum[2];
    dots[3] = qk_dot16(g3, A.x[3]) - 32 * A.sum[3];
}
// qk_unit_dot's and qk_unit_dot_h's arithmetic, in the same order, on a held
// activation.
__device__ __forceinline__ float qk_unit_dot_a(const QkUnit<QK_Q4_0>& U, int, const QkAct<QK_Q4_0>& A) {
    const int dot = qk4_dot_act(U, A);
    return (f16_to_f32(U.d) * A.s) * (float)dot;
}
__device__ __forceinline__ float qk_unit_dot_a(const QkUnit<QK_Q6_K>& U, int u, const QkAct<QK_Q6_K>& A) {
    int dots[4];
    qk6_dots_act(U, A, dots);
    float c[4];
    qk6_subscales(U, u, c);
    float s = (c[0] * A.s[0]) * (float)dots[0];
    s = fmaf(c[1] * A.s[1], (float)dots[1], s);
    s = fmaf(c[2] * A.s[2], (float)dots[2], s);
    s = fmaf(c[3] * A.s[3], (float)dots[3], s);
    return f16_to_f32(U.d) * s;
}

// A unit's contribution to its row with its activation read in place:
// codes xq and f32 scales xs per block (from LDS), or f16 scale bits xd (from
// global memory); the same arithmetic as qk_unit_dot_a.
__device__ __forceinline__ float qk_unit_dot(const QkUnit<QK_Q4_0>& U, int u, const int8_t* xq, const float* xs) {
    QkAct<QK_Q4_0> A;
    qk_load_act_l(xq, xs, u, A);
    return qk_unit_dot_a(U, u, A);
}
// (Q6_K: group by group, so that only one group's codes are live at a time)
__device__ __forceinline__ float qk_unit_dot(const QkUnit<QK_Q6_K>& U, int u, const int8_t* xq, const float* xs) {
    const int v0 = qk6_v0(u);
    const uint32_t L0[4] = {(uint32_t)U.l0.x, (uint32_t)U.l0.y, (uint32_t)U.l0.z, (uint32_t)U.l0.w};
    const uint32_t L1[4] = {(uint32_t)U.l1.x, (uint32_t)U.l1.y, (uint32_t)U.l1.z, (uint32_t)U.l1.w};
    const uint32_t H[4] = {(uint32_t)U.h.x, (uint32_t)U.h.y, (uint32_t)U.h.z, (uint32_t)U.h.w};
    int dots[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int4 x = *reinterpret_cast<const int4*>(xq + v0 + 32 * g);
        int n[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = g & 1 ? L1[i] : L0[i];
            const uint32_t l4 = g < 2 ? lo & 0x0F0F0F0Fu : (lo >> 4) & 0x0F0F0F0Fu;
            const int sh = 4 - 2 * g;            // bits 2g, 2g+1 of qh to bits 4, 5
            const uint32_t h2 = (sh >= 0 ? H[i] << sh : H[i] >> -sh) & 0x30303030u;
            n[i] = (int)(l4 | h2);
        }
        dots[g] = qk_dot16(n, x) - 32 * qk_sum16(x, 0);
    }
    float c[4];
    qk6_subscales(U, u, c);
    const float* xsv = xs + (v0 >> 5);
    float s = (c[0] * xsv[0]) * (float)dots[0];
    s = fmaf(c[1] * xsv[1], (float)dots[1], s);
    s = fmaf(c[2] * xsv[2], (float)dots[2], s);
    s = fmaf(c[3] * xsv[3], (float)dots[3], s);
    return f16_to_f32(U.d) * s;
}
template <int FMT>
__device__ __forceinline__ float qk_unit_dot_h(const QkUnit<FMT>& U, int u, const int8_t* xq, const uint16_t* xd) {
    QkAct<FMT> A;
    qk_load_act(xq, xd, u, A);
    return qk_unit_dot_a(U, u, A);
}

}  // namespace lq

/*
 * oracle.c -- plain, slow CPU reference for the single-token decode layer.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg; never by the GPU product path.  Every function
 * is the plain definition of one step, written loop by loop, with double
 * accumulation and float storage at stage boundaries.  No blocking, fusion or
 * reordering beyond what the definition states.
 *
 * Sources (web pages, cited by title and section):
 *   [LAT]  "Design: lattice-inference" -- Current Design (CPU fallback and
 *          NEON: the Q8_0 matvec multiplies int8 weights by int8 activations
 *          with int32 accumulation), Invariants (INV-2/3/7), Model
 *          Compatibility Matrix.
 *   [CUR]  "Current Inference Path -- Architecture Map" (hf2q) -- section 3
 *          (per-token decode sequence), section 4 (rms_norm_kernel F=1/2/3,
 *          rope_kernel Neox/Norm), section 7 (SDPA start_offset note).
 *   [ENG]  "Inference Engine" (larql) -- BLAS-Fused Attention, How it works
 *          (scores, 1/sqrt(head_dim) scale, two-pass softmax accumulated in
 *          f64, weighted V) and Supported features (GQA with any ratio).
 *   [TGT]  "Target Inference Architecture: hf2q on mlx-native" -- section 3.2
 *          (decode op list incl. MoE softmax / argsort / gather /
 *          quantized_matmul_id / weighted_sum; final rms_norm, f16_gemm
 *          lm_head and softcap), section 3.3 (buffer flow: expert_gate_up_3d
 *          [E, 2*I, H], expert_down_3d [E, H, I], KV caches [1, kv_heads,
 *          max_cache, head_dim], lm_head_f16 [vocab, hidden], logits
 *          [1, vocab]), section 6.3 (GGML block layout, non-zero start
 *          offsets).
 * Where the pages leave a step open, the reading taken is stated at the
 * function.
 *
 * Pins (tests/test_oracle_pins.py) tie every function to something other
 * than itself.  orc_decode_layer is pinned as a whole by special cases with
 * closed forms (all-zero O and down projections return x bit for bit; at
 * position 0 every head's attention output is its kv head's new v row) and
 * against an independent composition of its pinned stages; no external value
 * for a whole layer on random weights exists.  One limit:
 *   orc_q6_k_dequant / orc_q6_k_matvec -- parity unpinned against GGML
 *          itself: the element order is pinned to the layout as read from
 *          the pages (no GGML fixture is available offline).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ======================================================================== */
/* Number formats                                                           */
/* ======================================================================== */

/* IEEE 754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * Round-to-nearest-even is done exactly in double: every float is exact in
 * double, the quotient by a power of two is exact, and nearbyint() rounds
 * ties to even under the default rounding mode. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
    double v = fabs((double)x);
    /* The largest finite binary16 is 65504; halfway to the next step (65520)
     * and above rounds to infinity. */
    if (v >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (v < ldexp(1.0, -14)) {
        /* subnormal range: integer multiples of 2^-24 */
        double m = nearbyint(ldexp(v, 24));   /* 0 .. 1024; 1024 encodes 2^-14 */
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e2;
    (void)frexp(v, &e2);                      /* v = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                           /* v in [2^E, 2^(E+1)) */
    double m = nearbyint(ldexp(v, 10 - E));   /* 1024 .. 2048 */
    if (m == 2048.0) { m = 1024.0; E += 1; }
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0));
}

float orc_f16_to_f32(uint16_t h)
{
    int s = (h >> 15) & 1, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0)       v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else              v = ldexp((double)(1024 + f), e - 25);
    return (float)(s ? -v : v);
}

/* bfloat16 keeps the binary32 exponent and 7 fraction bits. */
uint16_t orc_f32_to_bf16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0u);
    double v = fabs((double)x);
    if (isinf(x)) return (uint16_t)(sign | 0x7f80u);
    if (v < ldexp(1.0, -126)) {
        /* binary32 subnormals: multiples of 2^-133 in bfloat16 */
        double m = nearbyint(ldexp(v, 133));  /* 0 .. 128; 128 encodes 2^-126 */
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e2;
    (void)frexp(v, &e2);
    int E = e2 - 1;
    double m = nearbyint(ldexp(v, 7 - E));    /* 128 .. 256 */
    if (m == 256.0) { m = 128.0; E += 1; }
    if (E + 127 >= 255) return (uint16_t)(sign | 0x7f80u);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)(m - 128.0));
}

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static double kv_elem(const void* base, int32_t dtype, int64_t idx)
{
    if (dtype == 0) return (double)((const float*)base)[idx];
    return (double)orc_bf16_to_f32(((const uint16_t*)base)[idx]);
}

static void kv_store(void* base, int32_t dtype, int64_t idx, float v)
{
    if (dtype == 0) ((float*)base)[idx] = v;
    else ((uint16_t*)base)[idx] = orc_f32_to_bf16(v);
}

/* ======================================================================== */
/* Q8_0                                                                     */
/* ======================================================================== */

/* Q8_0 activation quantization ([LAT] Current Design: the NEON path feeds
 * int8 x int8 products, so activations are Q8_0 blocks of 32 codes and one
 * f16 scale, the GGML block format of [TGT] section 6.3).
 * Reading taken (the pages print no rule): symmetric absmax scaling per block
 * in float: d = amax / 127; inv = 1/d (0 for an all-zero block);
 * q = round-half-away-from-zero(x * inv), clamped to [-127, 127]; the stored
 * scale is d rounded to f16.  The codes use the float d, not its f16 image. */
void orc_q8_quantize(const float* x, int64_t n, int8_t* qs, uint16_t* d)
{
    for (int64_t b = 0; b < n / 32; ++b) {
        const float* xb = x + 32 * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) {
            float a = fabsf(xb[i]);
            if (a > amax) amax = a;
        }
        float db = amax / 127.0f;
        float inv = (db != 0.0f) ? 1.0f / db : 0.0f;
        for (int i = 0; i < 32; ++i) {
            float v = xb[i] * inv;
            float r = roundf(v);                 /* ties away from zero */
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            qs[32 * b + i] = (int8_t)r;
        }
        d[b] = orc_f32_to_f16(db);
    }
}

/* Integer block dot ([LAT] Current Design, NEON matvec: int8 x int8 products
 * summed into an int32 per block).  |dot| <= 32*128*128, exact in int32. */
void orc_q8_block_dots(const int8_t* wq, int64_t rows, int64_t cols,
                       const int8_t* xq, int32_t* dots)
{
    int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < nb; ++b) {
            int32_t acc = 0;
            for (int i = 0; i < 32; ++i)
                acc += (int32_t)wq[r * cols + 32 * b + i] * (int32_t)xq[32 * b + i];
            dots[r * nb + b] = acc;
        }
}

/* Q8_0 matvec: y[r] = sum over blocks of d_w * d_x * dot, in double and in
 * block order, rounded once to float; the residual (if any) is added in
 * double before that rounding ([LAT] Current Design; [TGT] section 3.2
 * quantized_matmul, then add for the residual). */
void orc_q8_matvec(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                   const int8_t* xq, const uint16_t* xd, const float* residual, float* y)
{
    int64_t nb = cols / 32;
    for (int64_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            int32_t dot = 0;
            for (int i = 0; i < 32; ++i)
                dot += (int32_t)wq[r * cols + 32 * b + i] * (int32_t)xq[32 * b + i];
            acc += (double)orc_f16_to_f32(wd[r * nb + b]) *
                   (double)orc_f16_to_f32(xd[b]) * (double)dot;
        }
        if (residual) acc += (double)residual[r];
        y[r] = (float)acc;
    }
}

/* The same product for T tokens ([LAT] Current Design, applied row by row of
 * a token batch): y[t] = W x[t] (+ residual[t]), one matvec per token. */
void orc_q8_matmul(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                   const int8_t* xq, const uint16_t* xd, int64_t T, const float* residual, float* y)
{
    for (int64_t t = 0; t < T; ++t)
        orc_q8_matvec(wq, wd, rows, cols, xq + t * cols, xd + t * (cols / 32),
                      residual ? residual + t * rows : NULL, y + t * rows);
}

/* ======================================================================== */
/* Other GGML weight formats against Q8_0 activations                       */
/* ======================================================================== */

/* [CUR] section 4 (the MoE kernel of the current path runs on Q6_K weights)
 * and [TGT] section 8 (Q1: candle keeps GGML block order) name GGML's Q4_0
 * and Q6_K beside Q8_0 without their bit layouts.  The layouts here are
 * GGML's published block definitions as this oracle reads them (blocks in
 * order, f16 little-endian):
 *   Q4_0: 18 bytes per 32 values: f16 d, then 16 code bytes.  Byte j holds
 *         value j in its low nibble and value j+16 in its high nibble;
 *         w = d * (n - 8).
 *   Q6_K: 210 bytes per 256 values: ql[128], qh[64], int8 sc[16], f16 d.
 *         Value i, with h = i/128, g = (i%128)/32, l = i%32, takes its low 4
 *         bits from ql[64h + 32(g%2) + l] (the low nibble for g < 2, the high
 *         one for g >= 2) and its high 2 bits from bits 2g and 2g+1 of
 *         qh[32h + l]; w = d * sc[i/16] * (q - 32).
 * The product with a Q8_0 activation takes the int8 x int8 path of [LAT]
 * Current Design: exact int32 dots over each run of values that share their
 * scales (a Q4_0 block; 16 values of Q6_K, which sit inside one activation
 * block), times those scales. */
static void q4_0_codes(const uint8_t* blk, int8_t* q, double* d)
{
    *d = (double)orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int j = 0; j < 16; ++j) {
        q[j] = (int8_t)((blk[2 + j] & 0x0F) - 8);
        q[j + 16] = (int8_t)((blk[2 + j] >> 4) - 8);
    }
}

static void q6_k_codes(const uint8_t* blk, int8_t* q, double* d, int8_t* sc)
{
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    for (int k = 0; k < 16; ++k) sc[k] = (int8_t)blk[192 + k];
    *d = (double)orc_f16_to_f32((uint16_t)(blk[208] | (blk[209] << 8)));
    for (int i = 0; i < 256; ++i) {
        const int h = i / 128, g = (i % 128) / 32, l = i % 32;
        const uint8_t lb = ql[64 * h + 32 * (g % 2) + l];
        const int lo = g < 2 ? (lb & 0x0F) : (lb >> 4);
        const int hi = (qh[32 * h + l] >> (2 * g)) & 3;
        q[i] = (int8_t)((lo | (hi << 4)) - 32);
    }
}

/* Dequantized values (for pins): n values from consecutive blocks. */
void orc_q4_0_dequant(const uint8_t* blocks, int64_t n, double* w)
{
    int8_t q[32];
    double d;
    for (int64_t b = 0; b < n / 32; ++b) {
        q4_0_codes(blocks + 18 * b, q, &d);
        for (int i = 0; i < 32; ++i) w[32 * b + i] = d * (double)q[i];
    }
}

void orc_q6_k_dequant(const uint8_t* blocks, int64_t n, double* w)
{
    int8_t q[256], sc[16];
    double d;
    for (int64_t b = 0; b < n / 256; ++b) {
        q6_k_codes(blocks + 210 * b, q, &d, sc);
        for (int i = 0; i < 256; ++i) w[256 * b + i] = d * (double)sc[i / 16] * (double)q[i];
    }
}

/* y[r] = residual[r] + sum over blocks of d_w * d_x * dot (Q4_0 weights,
 * row-major GGML blocks [rows, cols/32]); double, in block order. */
void orc_q4_0_matvec(const uint8_t* blocks, int64_t rows, int64_t cols, const int8_t* xq,
                     const uint16_t* xd, const float* residual, float* y)
{
    const int64_t nb = cols / 32;
    int8_t q[32];
    double d;
    for (int64_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            q4_0_codes(blocks + 18 * (r * nb + b), q, &d);
            int32_t dot = 0;
            for (int i = 0; i < 32; ++i) dot += (int32_t)q[i] * (int32_t)xq[32 * b + i];
            acc += d * (double)orc_f16_to_f32(xd[b]) * (double)dot;
        }
        if (residual) acc += (double)residual[r];
        y[r] = (float)acc;
    }
}

/* The same for Q6_K weights (GGML blocks [rows, cols/256]): one int32 dot
 * per 16 values, times d * sc and the scale of the activation block that
 * holds them. */
void orc_q6_k_matvec(const uint8_t* blocks, int64_t rows, int64_t cols, const int8_t* xq,
                     const uint16_t* xd, const float* residual, float* y)
{
    const int64_t nsb = cols / 256;
    int8_t q[256], sc[16];
    double d;
    for (int64_t r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (int64_t b = 0; b < nsb; ++b) {
            q6_k_codes(blocks + 210 * (r * nsb + b), q, &d, sc);
            for (int k = 0; k < 16; ++k) {
                const int64_t c0 = 256 * b + 16 * k;
                int32_t dot = 0;
                for (int i = 0; i < 16; ++i) dot += (int32_t)q[16 * k + i] * (int32_t)xq[c0 + i];
                acc += d * (double)sc[k] * (double)orc_f16_to_f32(xd[c0 / 32]) * (double)dot;
            }
        }
        if (residual) acc += (double)residual[r];
        y[r] = (float)acc;
    }
}

/* ======================================================================== */
/* Norms, RoPE, activation                                                  */
/* ======================================================================== */

/* RMSNorm ([CUR] section 4, rms_norm_kernel: F=1 unit weight, F=2 weighted).
 * Reading taken: gamma multiplies directly (no 1+gamma offset). */
void orc_rmsnorm(const float* x, int64_t n, const float* gamma, double eps, float* y)
{
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += (double)x[i] * (double)x[i];
    double rinv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) {
        double g = gamma ? (double)gamma[i] : 1.0;
        y[i] = (float)(g * (double)x[i] * rinv);
    }
}

/* RoPE table ([LAT] Current Design: rope_table_max_seq_len is a precomputed
 * table; the angle is the usual pos * theta^(-2i/hd)), computed in double and
 * stored as float. */
void orc_rope_table(int64_t max_ctx, int64_t hd, double theta, float* cos_t, float* sin_t)
{
    orc_rope_table_freqs(max_ctx, hd, theta, NULL, cos_t, sin_t);
}

/* The table with per-pair frequency factors ([CUR] section 2, step 3: the
 * global layers' rope_freqs vector, a frequency mask over the head_dim/2
 * pairs).  Reading taken: each factor divides its pair's frequency (so +inf
 * leaves the pair unrotated). */
void orc_rope_table_freqs(int64_t max_ctx, int64_t hd, double theta, const float* factors,
                          float* cos_t, float* sin_t)
{
    int64_t half = hd / 2;
    for (int64_t p = 0; p < max_ctx; ++p)
        for (int64_t i = 0; i < half; ++i) {
            double inv_freq = pow(theta, -2.0 * (double)i / (double)hd);
            if (factors) inv_freq = inv_freq / (double)factors[i];
            double a = (double)p * inv_freq;
            cos_t[p * half + i] = (float)cos(a);
            sin_t[p * half + i] = (float)sin(a);
        }
}

/* NeoX RoPE ([CUR] section 4, rope_kernel Neox variant; the one the Gemma
 * path uses): element i is paired with i + hd/2 and the pair is rotated by the
 * table angle. */
void orc_rope_neox(float* x, int64_t hd, const float* cos_row, const float* sin_row)
{
    int64_t half = hd / 2;
    for (int64_t i = 0; i < half; ++i) {
        double a = (double)x[i], b = (double)x[i + half];
        double c = (double)cos_row[i], s = (double)sin_row[i];
        x[i] = (float)(a * c - b * s);
        x[i + half] = (float)(a * s + b * c);
    }
}

/* SwiGLU gate ([TGT] section 3.2 gate/up/mul; SiLU gating as the dense
 * SwiGLU MLP of [CUR] section 2). */
void orc_silu_mul(const float* g, const float* u, int64_t n, float* h)
{
    for (int64_t i = 0; i < n; ++i) {
        double z = (double)g[i];
        h[i] = (float)((z / (1.0 + exp(-z))) * (double)u[i]);
    }
}

/* GeGLU gate: gelu(gate) * up with the tanh form of GELU ([TGT] section 3.2
 * lists gelu among the decode ops; the Gemma MLP gates with it).  Reading
 * taken: the tanh approximation 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715
 * z^3))), the form Gemma-family MLPs use; the pages name no variant. */
void orc_gelu_mul(const float* g, const float* u, int64_t n, float* h)
{
    const double k = sqrt(2.0 / acos(-1.0));   /* sqrt(2 / pi) */
    for (int64_t i = 0; i < n; ++i) {
        double z = (double)g[i];
        double gz = 0.5 * z * (1.0 + tanh(k * (z + 0.044715 * z * z * z)));
        h[i] = (float)(gz * (double)u[i]);
    }
}

/* ======================================================================== */
/* Attention                                                                */
/* ======================================================================== */

/* Decode attention ([ENG] BLAS-Fused Attention, How it works: scores K.q,
 * scale 1/sqrt(head_dim), two-pass softmax with f64 accumulation, output
 * V^T.p; GQA with any ratio).  Reading taken for the head map: consecutive
 * query heads share a KV head, g = h / (n_q / n_kv).  Offsets and strides are
 * element counts ([CUR] section 7: the start offset must not be confused
 * with a byte count). */
void orc_attention(const float* q, int64_t n_q, int64_t n_kv, int64_t hd,
                   const void* k_cache, const void* v_cache, int32_t kv_dtype,
                   int64_t head_stride, int64_t pos_stride,
                   int64_t start, int64_t len, double scale, double softcap, float* out)
{
    int64_t G = n_q / n_kv;
    double* s = (double*)malloc((size_t)(len > 0 ? len : 1) * sizeof(double));
    double* o = (double*)malloc((size_t)hd * sizeof(double));
    for (int64_t h = 0; h < n_q; ++h) {
        int64_t g = h / G;
        const float* qh = q + h * hd;
        double m = -INFINITY;
        for (int64_t j = 0; j < len; ++j) {
            int64_t base = g * head_stride + (start + j) * pos_stride;
            double acc = 0.0;
            for (int64_t d = 0; d < hd; ++d)
                acc += (double)qh[d] * kv_elem(k_cache, kv_dtype, base + d);
            s[j] = scale * acc;
            /* optional score softcap ([ENG] BLAS-Fused Attention: the Gemma
             * tanh(score / cap) * cap after the scaling) */
            if (softcap > 0.0) s[j] = softcap * tanh(s[j] / softcap);
            if (s[j] > m) m = s[j];
        }
        double z = 0.0;
        for (int64_t j = 0; j < len; ++j) { s[j] = exp(s[j] - m); z += s[j]; }
        for (int64_t d = 0; d < hd; ++d) o[d] = 0.0;
        for (int64_t j = 0; j < len; ++j) {
            double p = s[j] / z;
            int64_t base = g * head_stride + (start + j) * pos_stride;
            for (int64_t d = 0; d < hd; ++d) o[d] += p * kv_elem(v_cache, kv_dtype, base + d);
        }
        for (int64_t d = 0; d < hd; ++d) out[h * hd + d] = (float)o[d];
    }
    free(s);
    free(o);
}

/* ======================================================================== */
/* MoE                                                                      */
/* ======================================================================== */

/* Router ([TGT] section 3.2: softmax, argsort, gather of the top-k
 * probabilities; [CUR] section 3 item i).  Softmax is strictly increasing in
 * the logit, so the k largest probabilities are those of the k largest
 * logits; the selection compares the float logits (exact), ties going to the
 * lower expert id.  Reading taken: no renormalisation of the k weights and no
 * per-expert scale (both are open on the pages). */
void orc_moe_route(const float* logits, int64_t T, int64_t E, int64_t k,
                   int32_t* ids, float* w)
{
    char* taken = (char*)malloc((size_t)E);
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        double m = -INFINITY, z = 0.0;
        for (int64_t e = 0; e < E; ++e) if ((double)l[e] > m) m = (double)l[e];
        for (int64_t e = 0; e < E; ++e) z += exp((double)l[e] - m);
        memset(taken, 0, (size_t)E);
        for (int64_t s = 0; s < k; ++s) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[t * k + s] = (int32_t)best;
            w[t * k + s] = (float)(exp((double)l[best] - m) / z);
        }
    }
    free(taken);
}

/* MoE block ([CUR] section 3 item i and section 4 moe_kernel: each
 * (token, slot) row selects one expert's quantized weights by id; [TGT]
 * section 3.2: gate_up, SwiGLU, down, weighted sum over the k slots; the
 * "loop" mode of [CUR] section 1 is exactly this per-slot loop). */
void orc_moe_block(const orc_moe* m, const float* x, const float* logits, float* out,
                   orc_moe_trace* tr)
{
    int64_t H = m->hidden, I = m->ffn, K = m->top_k, T = m->tokens;
    int32_t* ids = (int32_t*)malloc((size_t)(T * K) * sizeof(int32_t));
    float* w = (float*)malloc((size_t)(T * K) * sizeof(float));
    int8_t* xq = (int8_t*)malloc((size_t)H);
    uint16_t* xd = (uint16_t*)malloc((size_t)(H / 32) * sizeof(uint16_t));
    float* y1 = (float*)malloc((size_t)(2 * I) * sizeof(float));
    float* h = (float*)malloc((size_t)I * sizeof(float));
    int8_t* hq = (int8_t*)malloc((size_t)I);
    uint16_t* hd = (uint16_t*)malloc((size_t)(I / 32) * sizeof(uint16_t));
    float* y2 = (float*)malloc((size_t)H * sizeof(float));
    double* acc = (double*)malloc((size_t)H * sizeof(double));

    orc_moe_route(logits, T, m->n_experts, K, ids, w);
    if (tr && tr->ids) memcpy(tr->ids, ids, (size_t)(T * K) * sizeof(int32_t));
    if (tr && tr->w) memcpy(tr->w, w, (size_t)(T * K) * sizeof(float));

    int64_t gu_rows = 2 * I;
    for (int64_t t = 0; t < T; ++t) {
        orc_q8_quantize(x + t * H, H, xq, xd);
        if (tr && tr->xq) memcpy(tr->xq + t * H, xq, (size_t)H);
        if (tr && tr->xd) memcpy(tr->xd + t * (H / 32), xd, (size_t)(H / 32) * sizeof(uint16_t));
        for (int64_t j = 0; j < H; ++j) acc[j] = 0.0;
        for (int64_t s = 0; s < K; ++s) {
            int64_t e = ids[t * K + s];
            orc_q8_matvec(m->gu_qs + e * gu_rows * H, m->gu_d + e * gu_rows * (H / 32),
                          gu_rows, H, xq, xd, NULL, y1);
            orc_silu_mul(y1, y1 + I, I, h);
            orc_q8_quantize(h, I, hq, hd);
            orc_q8_matvec(m->dn_qs + e * H * I, m->dn_d + e * H * (I / 32),
                          H, I, hq, hd, NULL, y2);
            int64_t slot = t * K + s;
            if (tr && tr->y1) memcpy(tr->y1 + slot * gu_rows, y1, (size_t)gu_rows * sizeof(float));
            if (tr && tr->hq) memcpy(tr->hq + slot * I, hq, (size_t)I);
            if (tr && tr->hd) memcpy(tr->hd + slot * (I / 32), hd, (size_t)(I / 32) * sizeof(uint16_t));
            if (tr && tr->y2) memcpy(tr->y2 + slot * H, y2, (size_t)H * sizeof(float));
            /* per-expert output scale ([TGT] section 3.2: gather of
             * per_expert_scale, then weight * scale) */
            double ws = (double)w[slot];
            if (m->expert_scale) ws *= (double)m->expert_scale[e];
            for (int64_t j = 0; j < H; ++j) acc[j] += ws * (double)y2[j];
        }
        for (int64_t j = 0; j < H; ++j) out[t * H + j] = (float)acc[j];
    }
    free(ids); free(w); free(xq); free(xd); free(y1); free(h);
    free(hq); free(hd); free(y2); free(acc);
}

/* ======================================================================== */
/* Decode layer                                                             */
/* ======================================================================== */

/* One decode token through one layer.
 * kind 0 (pre-norm layer with SwiGLU FFN, the Qwen3 family of [LAT]):
 *   x -> RMSNorm(g_in) -> Q8 -> fused QKV ([LAT] INV-7) -> per-head q/k
 *   RMSNorm -> NeoX RoPE -> append k, v at pos -> attention over the causal
 *   (or windowed) context -> Q8 -> O projection + x = x1 -> RMSNorm(g_post)
 *   -> Q8 -> gate/up -> silu(g)*u -> Q8 -> down + x1.
 * kind 1 (Gemma attention block, [CUR] section 3 items a-d): as above through
 *   the attention, with V unit-normed before the append, then
 *   O projection -> RMSNorm(g_post) -> + x.
 * Window reading taken: window W attends the W most recent positions
 * including the current one, [pos-W+1, pos]. */
void orc_decode_layer(const orc_layer* L, float* x, int64_t pos, orc_layer_trace* tr)
{
    int64_t H = L->hidden, hd = L->head_dim, nq = L->n_q, nkv = L->n_kv, I = L->ffn;
    int64_t qd = nq * hd, kvd = nkv * hd, half = hd / 2;
    int64_t qkv_rows = qd + 2 * kvd;
    size_t fmax = (size_t)(H > qkv_rows ? H : qkv_rows);
    if ((size_t)(2 * I) > fmax) fmax = (size_t)(2 * I);
    if ((size_t)qd > fmax) fmax = (size_t)qd;

    float* n = (float*)malloc(fmax * sizeof(float));
    int8_t* q8 = (int8_t*)malloc(fmax);
    uint16_t* d8 = (uint16_t*)malloc((fmax / 32 + 1) * sizeof(uint16_t));
    float* qkv = (float*)malloc((size_t)qkv_rows * sizeof(float));
    float* att = (float*)malloc((size_t)qd * sizeof(float));
    float* x1 = (float*)malloc((size_t)H * sizeof(float));
    float* tmp = (float*)malloc(fmax * sizeof(float));

    /* input norm + quantize */
    orc_rmsnorm(x, H, L->g_in, L->eps, n);
    orc_q8_quantize(n, H, q8, d8);
    if (tr && tr->xq) memcpy(tr->xq, q8, (size_t)H);
    if (tr && tr->xd) memcpy(tr->xd, d8, (size_t)(H / 32) * sizeof(uint16_t));

    /* fused QKV projection */
    orc_q8_matvec(L->qkv_qs, L->qkv_d, qkv_rows, H, q8, d8, NULL, qkv);
    if (tr && tr->qkv) memcpy(tr->qkv, qkv, (size_t)qkv_rows * sizeof(float));

    float* q = qkv;
    float* k = qkv + qd;
    float* v = qkv + qd + kvd;
    const float* c_row = L->rope_cos + pos * half;
    const float* s_row = L->rope_sin + pos * half;
    for (int64_t h = 0; h < nq; ++h) {
        if (L->qk_norm) { orc_rmsnorm(q + h * hd, hd, L->g_q, L->eps, tmp); memcpy(q + h * hd, tmp, (size_t)hd * sizeof(float)); }
        orc_rope_neox(q + h * hd, hd, c_row, s_row);
    }
    for (int64_t g = 0; g < nkv; ++g) {
        if (L->qk_norm) { orc_rmsnorm(k + g * hd, hd, L->g_k, L->eps, tmp); memcpy(k + g * hd, tmp, (size_t)hd * sizeof(float)); }
        orc_rope_neox(k + g * hd, hd, c_row, s_row);
        if (L->v_unit_norm) { orc_rmsnorm(v + g * hd, hd, NULL, L->eps, tmp); memcpy(v + g * hd, tmp, (size_t)hd * sizeof(float)); }
    }
    if (tr && tr->q) memcpy(tr->q, q, (size_t)qd * sizeof(float));
    if (tr && tr->k) memcpy(tr->k, k, (size_t)kvd * sizeof(float));
    if (tr && tr->v) memcpy(tr->v, v, (size_t)kvd * sizeof(float));

    /* KV append at pos (cache layout [n_kv, max_ctx, hd]) */
    int64_t hs = L->max_ctx * hd;
    for (int64_t g = 0; g < nkv; ++g)
        for (int64_t d = 0; d < hd; ++d) {
            kv_store(L->k_cache, L->kv_dtype, g * hs + pos * hd + d, k[g * hd + d]);
            kv_store(L->v_cache, L->kv_dtype, g * hs + pos * hd + d, v[g * hd + d]);
        }

    /* attention */
    int64_t start = 0;
    if (L->window > 0 && pos - L->window + 1 > 0) start = pos - L->window + 1;
    orc_attention(q, nq, nkv, hd, L->k_cache, L->v_cache, L->kv_dtype, hs, hd,
                  start, pos - start + 1, L->attn_scale, L->attn_softcap, att);
    if (tr && tr->attn) memcpy(tr->attn, att, (size_t)qd * sizeof(float));

    orc_q8_quantize(att, qd, q8, d8);
    if (tr && tr->aq) memcpy(tr->aq, q8, (size_t)qd);
    if (tr && tr->ad) memcpy(tr->ad, d8, (size_t)(qd / 32) * sizeof(uint16_t));

    if (L->kind == 0) {
        orc_q8_matvec(L->o_qs, L->o_d, H, qd, q8, d8, x, x1);
    } else {
        orc_q8_matvec(L->o_qs, L->o_d, H, qd, q8, d8, NULL, tmp);
        orc_rmsnorm(tmp, H, L->g_post, L->eps, n);
        for (int64_t i = 0; i < H; ++i) x1[i] = (float)((double)x[i] + (double)n[i]);
    }
    if (tr && tr->x1) memcpy(tr->x1, x1, (size_t)H * sizeof(float));

    if (L->kind == 0 && I > 0) {
        float* gu = (float*)malloc((size_t)(2 * I) * sizeof(float));
        orc_rmsnorm(x1, H, L->g_post, L->eps, n);
        orc_q8_quantize(n, H, q8, d8);
        if (tr && tr->nq) memcpy(tr->nq, q8, (size_t)H);
        if (tr && tr->nd) memcpy(tr->nd, d8, (size_t)(H / 32) * sizeof(uint16_t));
        orc_q8_matvec(L->gu_qs, L->gu_d, 2 * I, H, q8, d8, NULL, gu);
        if (tr && tr->gu) memcpy(tr->gu, gu, (size_t)(2 * I) * sizeof(float));
        if (L->ffn_act == 1) orc_gelu_mul(gu, gu + I, I, tmp);
        else orc_silu_mul(gu, gu + I, I, tmp);
        orc_q8_quantize(tmp, I, q8, d8);
        if (tr && tr->hq) memcpy(tr->hq, q8, (size_t)I);
        if (tr && tr->hd) memcpy(tr->hd, d8, (size_t)(I / 32) * sizeof(uint16_t));
        orc_q8_matvec(L->dn_qs, L->dn_d, H, I, q8, d8, x1, x);
        free(gu);
    } else {
        memcpy(x, x1, (size_t)H * sizeof(float));
    }
    free(n); free(q8); free(d8); free(qkv); free(att); free(x1); free(tmp);
}

/* ======================================================================== */
/* Output head                                                              */
/* ======================================================================== */

/* Final norm, vocab projection and logit softcapping ([CUR] section 3,
 * forward pass steps 4, 5 and 7: the final RmsNorm, normed times the
 * transposed lm_head weight, softcapping as a division, tanh and
 * multiplication; section 4, lm_head_kernel: the projection runs on F16
 * weights; [TGT] section 3.2: rms_norm, f16_gemm, softcap; section 3.3:
 * lm_head_f16 [vocab, hidden] f16, logits [1, vocab] f32).
 * Readings taken: norm == 0 uses x as given (already normed); the softcap
 * is cap * tanh(y / cap) and cap <= 0 turns it off. */
void orc_lm_head(const uint16_t* w, int64_t vocab, int64_t hidden, const float* x, int32_t norm,
                 const float* gamma, double eps, double cap, float* logits)
{
    float* n = (float*)malloc((size_t)hidden * sizeof(float));
    if (norm) {
        orc_rmsnorm(x, hidden, gamma, eps, n);
    } else {
        for (int64_t c = 0; c < hidden; ++c) n[c] = x[c];
    }
    for (int64_t r = 0; r < vocab; ++r) {
        const uint16_t* row = w + r * hidden;
        double acc = 0.0;
        for (int64_t c = 0; c < hidden; ++c) acc += (double)orc_f16_to_f32(row[c]) * (double)n[c];
        if (cap > 0.0) acc = cap * tanh(acc / cap);
        logits[r] = (float)acc;
    }
    free(n);
}

/*
 * oracle.h -- plain, slow CPU reference for the single-token decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU product
 * path never links, imports or calls it, and it shares no code with it.
 *
 * Conventions
 *   - Accumulation is in double (binary64); every stage boundary is stored as
 *     float (binary32), which is how the pages' engines keep activations
 *     ("Target Inference Architecture: hf2q on mlx-native", section 8, Q4:
 *     the forward pass is end-to-end F32).
 *   - f16 and bf16 values are passed as uint16_t bit patterns.
 *   - Q8_0 data is structure-of-arrays: int8 codes [rows, cols] row-major and
 *     one f16 scale per 32 consecutive codes [rows, cols/32].
 *   - KV caches are [n_kv, max_ctx, head_dim] with element strides given
 *     explicitly; dtype 0 = f32, 1 = bf16.
 *   - Nothing here allocates GPU memory or checks arguments beyond what the
 *     definitions need; callers pass well-formed sizes.
 */
#ifndef LQ_ORACLE_H
#define LQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats ------------------------------------------------------ */
uint16_t orc_f32_to_f16(float x);      /* IEEE binary16, round-to-nearest-even, subnormals kept */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_bf16(float x);     /* bfloat16 (top half of binary32), round-to-nearest-even */
float    orc_bf16_to_f32(uint16_t b);

/* ---- Q8_0 ---------------------------------------------------------------- */
/* Quantize n values (n % 32 == 0) block by block. */
void orc_q8_quantize(const float* x, int64_t n, int8_t* qs, uint16_t* d);
/* Exact int32 dot product of every 32-wide block of every row with x. */
void orc_q8_block_dots(const int8_t* wq, int64_t rows, int64_t cols,
                       const int8_t* xq, int32_t* dots);
/* y[r] = residual[r] + sum_b d_w[r,b] * d_x[b] * dot[r,b]  (residual may be NULL). */
void orc_q8_matvec(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                   const int8_t* xq, const uint16_t* xd, const float* residual, float* y);

/* y[t] = W x[t] (+ residual[t]) for t < T: x [T, cols], y [T, rows]. */
void orc_q8_matmul(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                   const int8_t* xq, const uint16_t* xd, int64_t T, const float* residual, float* y);

/* ---- other GGML weight formats (GGML blocks, row-major) ------------------ */
void orc_q4_0_dequant(const uint8_t* blocks, int64_t n, double* w);
void orc_q6_k_dequant(const uint8_t* blocks, int64_t n, double* w);
void orc_q4_0_matvec(const uint8_t* blocks, int64_t rows, int64_t cols, const int8_t* xq,
                     const uint16_t* xd, const float* residual, float* y);
void orc_q6_k_matvec(const uint8_t* blocks, int64_t rows, int64_t cols, const int8_t* xq,
                     const uint16_t* xd, const float* residual, float* y);

/* ---- norms, RoPE, activation --------------------------------------------- */
/* y = gamma * x / sqrt(mean(x^2) + eps); gamma == NULL means unit weight. */
void orc_rmsnorm(const float* x, int64_t n, const float* gamma, double eps, float* y);
/* cos/sin tables [max_ctx, hd/2]: angle(pos, i) = pos * theta^(-2i/hd). */
void orc_rope_table(int64_t max_ctx, int64_t hd, double theta, float* cos_t, float* sin_t);
/* ... with angle / factors[i] (factors NULL: all 1). */
void orc_rope_table_freqs(int64_t max_ctx, int64_t hd, double theta, const float* factors,
                          float* cos_t, float* sin_t);
/* NeoX rotation of one head in place: pairs (i, i + hd/2). */
void orc_rope_neox(float* x, int64_t hd, const float* cos_row, const float* sin_row);
/* h = silu(g) * u, silu(z) = z / (1 + exp(-z)). */
void orc_silu_mul(const float* g, const float* u, int64_t n, float* h);
/* h = gelu(g) * u, gelu(z) = 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
void orc_gelu_mul(const float* g, const float* u, int64_t n, float* h);

/* ---- output head --------------------------------------------------------- */
/* n = norm ? rmsnorm(x; gamma, eps) : x;  logits[r] = sum_c f16(w[r,c]) * n[c];
 * then logits = cap * tanh(logits / cap) when cap > 0. */
void orc_lm_head(const uint16_t* w, int64_t vocab, int64_t hidden, const float* x, int32_t norm,
                 const float* gamma, double eps, double cap, float* logits);

/* ---- attention ----------------------------------------------------------- */
/* For each query head h (kv head g = h / (n_q/n_kv)) attend over cache
 * positions [start, start+len): two-pass softmax in double, scores optionally
 * soft-capped (softcap > 0: s -> softcap * tanh(s / softcap)). out is [n_q, hd]. */
void orc_attention(const float* q, int64_t n_q, int64_t n_kv, int64_t hd,
                   const void* k_cache, const void* v_cache, int32_t kv_dtype,
                   int64_t head_stride, int64_t pos_stride,
                   int64_t start, int64_t len, double scale, double softcap, float* out);

/* ---- MoE ----------------------------------------------------------------- */
/* Per token: softmax over E logits, the k largest (ties: lower expert id),
 * weights = their probabilities (no renormalisation). */
void orc_moe_route(const float* logits, int64_t T, int64_t E, int64_t k,
                   int32_t* ids, float* w);

typedef struct orc_moe {
    int64_t hidden, ffn, n_experts, top_k, tokens;
    const int8_t* gu_qs;  const uint16_t* gu_d;    /* [E, 2*ffn, hidden] */
    const int8_t* dn_qs;  const uint16_t* dn_d;    /* [E, hidden, ffn]   */
    const float* expert_scale;                     /* [E] or NULL (all 1) */
} orc_moe;

typedef struct orc_moe_trace {       /* every pointer may be NULL */
    int32_t* ids; float* w;          /* [T, k] */
    int8_t* xq; uint16_t* xd;        /* [T, hidden] codes, [T, hidden/32] scales */
    float* y1;                       /* [T, k, 2*ffn] */
    int8_t* hq; uint16_t* hd;        /* [T, k, ffn], [T, k, ffn/32] */
    float* y2;                       /* [T, k, hidden] */
} orc_moe_trace;

/* out[t] = sum_s w[t,s] * W_down[e] . Q8(silu(g) * u),  [g;u] = W_gate_up[e] . Q8(x[t]). */
void orc_moe_block(const orc_moe* m, const float* x, const float* logits, float* out,
                   orc_moe_trace* trace);

/* ---- decode layer -------------------------------------------------------- */
typedef struct orc_layer {
    int64_t hidden, n_q, n_kv, head_dim, ffn;   /* ffn == 0: attention block only */
    int64_t max_ctx, window;                     /* window == 0: full causal context */
    double eps, attn_scale;
    int32_t kv_dtype;                            /* 0 f32, 1 bf16 */
    int32_t kind;                                /* 0 pre-norm + SwiGLU FFN; 1 attention block with post-attention norm */
    int32_t qk_norm, v_unit_norm;
    const int8_t* qkv_qs; const uint16_t* qkv_d; /* [n_q*hd + 2*n_kv*hd, hidden] */
    const int8_t* o_qs;   const uint16_t* o_d;   /* [hidden, n_q*hd] */
    const int8_t* gu_qs;  const uint16_t* gu_d;  /* [2*ffn, hidden] (gate rows, then up rows) */
    const int8_t* dn_qs;  const uint16_t* dn_d;  /* [hidden, ffn] */
    const float *g_in, *g_q, *g_k, *g_post;      /* norm weights */
    void *k_cache, *v_cache;                     /* [n_kv, max_ctx, hd], updated at pos */
    const float *rope_cos, *rope_sin;            /* [max_ctx, hd/2] */
    int32_t ffn_act;                             /* 0 silu(gate) * up; 1 gelu_tanh(gate) * up */
    double attn_softcap;                         /* > 0: scores become cap * tanh(s / cap) */
} orc_layer;

typedef struct orc_layer_trace {    /* every pointer may be NULL */
    int8_t* xq; uint16_t* xd;       /* Q8 of the input norm output */
    float* qkv;                     /* raw fused projection */
    float* q; float* k; float* v;   /* after norms and RoPE (k, v as appended, before cache rounding) */
    float* attn;                    /* attention output [n_q*hd] */
    int8_t* aq; uint16_t* ad;       /* Q8 of the attention output */
    float* x1;                      /* after the attention residual */
    int8_t* nq; uint16_t* nd;       /* Q8 of the second norm output (kind 0) */
    float* gu;                      /* gate/up projection [2*ffn] */
    int8_t* hq; uint16_t* hd;       /* Q8 of silu(g)*u */
} orc_layer_trace;

/* One token at position pos: x [hidden] is updated in place; the caches are
 * written at pos. */
void orc_decode_layer(const orc_layer* L, float* x, int64_t pos, orc_layer_trace* trace);

#ifdef __cplusplus
}
#endif
#endif

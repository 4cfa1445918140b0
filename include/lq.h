/*
 * lq.h -- C ABI of the Q8_0 single-token decode-layer library for AMD
 * Instinct MI355X (gfx950).  Library: liblq.so (hand-written HIP kernels).
 *
 * The operations are the decode hot path that these inference-engine design
 * pages describe (cited by page title and section):
 *   [LAT] "Design: lattice-inference": Current Design (Q8_0 NEON matvec with
 *         int8 x int8 products into int32; fused attention with online
 *         softmax; fused per-head Q/K norm + RoPE), Invariants INV-2
 *         (head_dim % 4 == 0), INV-3 (num_heads % kv_heads == 0), INV-7
 *         (fused QKV weight [q_dim + 2*kv_dim, hidden]), INV-8 (buffers
 *         pre-allocated, no allocation in the forward pass).
 *   [CUR] "Current Inference Path -- Architecture Map" (hf2q): section 3
 *         (per-token decode sequence), section 4 (rms_norm F=1/2/3, NeoX
 *         RoPE, index-driven quantized matvec for MoE), section 7 (KV views
 *         with a non-zero start offset; offsets are element counts).
 *   [ENG] "Inference Engine" (larql): BLAS-Fused Attention (scale
 *         1/sqrt(head_dim), softmax, GQA with any ratio).
 *   [TGT] "Target Inference Architecture: hf2q on mlx-native": section 3.2
 *         (decode op list), section 3.3 (buffer flow and layouts), section
 *         4.2 (buffers carry no shape metadata; the caller tracks shapes),
 *         section 6.3 (GGML block layout; [num_experts, n, k] expert layout).
 *
 * Conventions (all entry points)
 *   - Every pointer named as device memory is caller-owned GPU memory; the
 *     library never allocates or frees on these calls.  Host pointers are
 *     named as such.  Scratch space comes in through (workspace,
 *     workspace_bytes), sized by the matching *_workspace_size() query.
 *   - stream is a hipStream_t passed as void* (NULL: the null stream).  Calls
 *     only enqueue work; none synchronizes the host.
 *   - Sizes, offsets and strides are int64_t ELEMENT counts, never bytes.
 *   - f16 and bf16 values are uint16_t bit patterns.
 *   - A nonzero lq_status means nothing was enqueued (argument checks run on
 *     the host before any launch), except LQ_ERR_HIP, which reports a launch
 *     failure.  lq_last_error() then returns a message (thread-local).
 *     Faults inside kernels surface at the caller's next synchronization.
 *   - Zero-sized work (rows == 0, n_rows == 0, ...) is a no-op returning
 *     LQ_OK.
 *   - Calls are stateless and reentrant; concurrent calls must not share
 *     output or workspace buffers.
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t lq_status;
#define LQ_OK               0
#define LQ_ERR_NULL         1   /* a required pointer is NULL */
#define LQ_ERR_SHAPE        2   /* sizes violate the operation's definition */
#define LQ_ERR_ALIGN        3   /* a pointer or stride breaks the alignment below */
#define LQ_ERR_WORKSPACE    4   /* workspace NULL or smaller than the query says */
#define LQ_ERR_HIP          5   /* the HIP runtime reported an error on launch */
#define LQ_ERR_UNSUPPORTED  6   /* valid by definition, outside what the library's kernels cover */

#define LQ_KV_F32   0
#define LQ_KV_BF16  1

/* Q8_0 weight matrix in structure-of-arrays form ([LAT] Current Design;
 * GGML Q8_0 semantics per [TGT] section 6.3): row r, block b (32 columns)
 * dequantizes to f16(d[r*cols/32 + b]) * qs[r*cols + 32*b + i].
 *   qs:  device, int8 [rows, cols], row-major, 16-byte aligned.
 *   d:   device, f16 bits [rows, cols/32], 2-byte aligned.
 *   cols must be a positive multiple of 32.
 * lq_q8_pack_ggml() converts the interleaved 34-byte GGML blocks to this. */
typedef struct lq_q8_weight {
    const int8_t*   qs;
    const uint16_t* d;
    int64_t rows;
    int64_t cols;
} lq_q8_weight;

/* Weight formats.  Q8_0 is this library's native format; Q4_0 and Q6_K are
 * the other GGML block formats the pages name.  Zero (a zero-initialized
 * descriptor) is Q8_0. */
#define LQ_FMT_Q8_0  0
#define LQ_FMT_Q4_0  1
#define LQ_FMT_Q6_K  2

/* Other GGML weight formats ([CUR] section 4: the current path's MoE kernel
 * runs on Q6_K weights; [TGT] section 8, Q1: GGML block order).  Device
 * layout, SoA (lq_q4_0_pack_ggml / lq_q6_k_pack_ggml convert GGML blocks):
 *   Q4_0: qs  uint8 [rows, cols/2]: each 32-value block's 16 code bytes in
 *             GGML order (byte j: value j in the low nibble, value j+16 in
 *             the high nibble), 16-byte aligned;
 *         d   f16 bits [rows, cols/32].     w = d * (n - 8).
 *   Q6_K: ql  uint8 [rows, cols/2] and qh uint8 [rows, cols/4] (the low 4
 *             and high 2 code bits, each 256-value super-block's bytes in
 *             GGML order), both 16-byte aligned;
 *         sc  int8 [rows, cols/16] (one scale per 16 values), 8-byte aligned;
 *         d   f16 bits [rows, cols/256].   w = d * sc[i/16] * (q - 32),
 *         where value i (h = i/128, g = (i%128)/32, l = i%32) takes its low
 *         bits from ql[64h + 32(g%2) + l] (low nibble for g < 2, high for
 *         g >= 2) and its high bits from bits 2g, 2g+1 of qh[32h + l]. */
typedef struct lq_q4_0_weight {
    const uint8_t*  qs;
    const uint16_t* d;
    int64_t rows;
    int64_t cols;
} lq_q4_0_weight;

typedef struct lq_q6_k_weight {
    const uint8_t*  ql;
    const uint8_t*  qh;
    const int8_t*   sc;
    const uint16_t* d;
    int64_t rows;
    int64_t cols;
} lq_q6_k_weight;

/* ---------------------------------------------------------------- misc */
int32_t     lq_version(void);
const char* lq_status_string(lq_status s);
const char* lq_last_error(void);

/* Host-only helper: GGML Q8_0 blocks (per 32 values: f16 scale, then 32
 * int8 codes; 34 bytes, [TGT] section 6.3 "GGML block order") for a
 * [rows, cols] matrix, row-major, into SoA qs [rows, cols] and d
 * [rows, cols/32].  All pointers are HOST memory.  cols % 32 == 0. */
lq_status lq_q8_pack_ggml(const void* blocks, int64_t rows, int64_t cols,
                          int8_t* qs, uint16_t* d);

/* Host-only helpers: GGML Q4_0 blocks (18 bytes per 32 values: f16 d, 16
 * code bytes) and Q6_K blocks (210 bytes per 256 values: ql[128], qh[64],
 * int8 sc[16], f16 d) of a [rows, cols] matrix, row-major, into the SoA
 * arrays above.  All pointers are HOST memory.  cols % 32 (Q4_0) or % 256
 * (Q6_K) == 0. */
lq_status lq_q4_0_pack_ggml(const void* blocks, int64_t rows, int64_t cols, uint8_t* qs, uint16_t* d);
lq_status lq_q6_k_pack_ggml(const void* blocks, int64_t rows, int64_t cols, uint8_t* ql, uint8_t* qh,
                            int8_t* sc, uint16_t* d);

/* Host-only helper: RoPE cos/sin tables [max_ctx, head_dim/2] for angle
 * pos * theta^(-2i/head_dim), computed in double and stored as float
 * ([LAT] Current Design: rope_table_max_seq_len).  HOST memory. */
lq_status lq_rope_table(int64_t max_ctx, int64_t head_dim, double theta,
                        float* cos_out, float* sin_out);

/* The same table with per-pair frequency factors (the Gemma global layers'
 * rope_freqs vector of [CUR] section 2, step 3, item 4, a frequency mask of
 * head_dim/2 entries; sliding and global layers also use their own theta,
 * item 5, which is a second table): angle = pos * theta^(-2i/head_dim) /
 * freq_factors[i].  A factor of +inf leaves pair i unrotated.  freq_factors:
 * HOST f32 [head_dim/2], every entry > 0, or NULL (all 1).  HOST memory. */
lq_status lq_rope_table_freqs(int64_t max_ctx, int64_t head_dim, double theta, const float* freq_factors,
                              float* cos_out, float* sin_out);

/* ---------------------------------------------------------------- Q8_0 */
/* Quantize n_rows independent vectors of n floats (n % 32 == 0) to Q8_0:
 * per 32-block d = amax/127 (float), codes = round-half-away(x * (1/d))
 * clamped to [-127, 127] (0 when amax == 0), scale stored as f16 (RNE).
 * x: device f32 [n_rows, n], 16-byte aligned.  qs: device int8 [n_rows, n],
 * 16-byte aligned.  d: device f16 bits [n_rows, n/32]. */
lq_status lq_q8_quantize_act(const float* x, int64_t n_rows, int64_t n,
                             int8_t* qs, uint16_t* d, void* stream);

/* Fused RMSNorm + Q8_0 quantize of n_rows vectors of n floats:
 * y = gamma * x / sqrt(mean(x^2) + eps) ([CUR] section 4, F=2 weighted;
 * gamma == NULL gives the unit-weight F=1 form), then as
 * lq_q8_quantize_act.  gamma: device f32 [n]. */
lq_status lq_rmsnorm_q8(const float* x, int64_t n_rows, int64_t n, const float* gamma,
                        float eps, int8_t* qs, uint16_t* d, void* stream);

/* SwiGLU + Q8_0 quantize: for each of n_rows rows of gate_up [n_rows, 2*ffn]
 * (gate in columns [0, ffn), up in [ffn, 2*ffn)), h = silu(gate) * up with
 * silu(z) = z / (1 + exp(-z)), then quantize h as lq_q8_quantize_act
 * ([TGT] section 3.2: gate, activation, up, mul).  ffn % 32 == 0.
 * gate_up: device f32, 16-byte aligned. */
lq_status lq_swiglu_q8(const float* gate_up, int64_t n_rows, int64_t ffn,
                       int8_t* qs, uint16_t* d, void* stream);

/* Q8_0 matvec ([LAT] Current Design, NEON 4-row matvec): for every row r,
 *   dot[r,b] = sum_{i<32} qs_w[r,32b+i] * x_qs[32b+i]        (int32, exact)
 *   y[r]     = residual[r] + sum_b f16(d_w[r,b]) * f16(x_d[b]) * dot[r,b]
 * with the float sum in an unspecified order (each term is exact in f32
 * before accumulation).  residual may be NULL.  x_qs: device int8 [cols],
 * 16-byte aligned; x_d: device f16 bits [cols/32]; y, residual: device f32
 * [rows].  y may alias residual. */
lq_status lq_q8_matvec(const lq_q8_weight* w, const int8_t* x_qs, const uint16_t* x_d,
                       const float* residual, float* y, void* stream);

/* Test tap: the int32 block dots dot[r,b] of the Q8_0 matvec ([LAT] Current
 * Design: int8 x int8 products summed into int32 per block), written to dots
 * (device int32 [rows, cols/32]).  For cols <= 16384 they come from the
 * fused matvec kernel that lq_q8_matvec and lq_decode_layer run (same
 * weight loads, lane-to-slice mapping and block-dot routine, with an
 * epilogue that stores the dots instead of y); for longer rows from the
 * kernel lq_q8_matvec runs there.  x_qs: device int8 [cols], 16-byte
 * aligned.  No scales are read: the dots do not depend on them. */
lq_status lq_q8_block_dots(const lq_q8_weight* w, const int8_t* x_qs, int32_t* dots,
                           void* stream);

/* Test tap: the same block dots when the fused matvec builds its Q8_0 input
 * in-kernel from a float vector, as the decode layer's projections do
 * ([CUR] section 4: rms_norm F=2 weighted, F=1 unit): norm == 0 quantizes
 * x as lq_q8_quantize_act; norm == 1 first applies y = gamma * x /
 * sqrt(mean(x^2) + eps) (gamma NULL: unit weight), as lq_rmsnorm_q8.
 * The Q8_0 input the kernel built is written to x_qs_out (device int8
 * [cols], 8-byte aligned) and x_d_out (device f16 bits [cols/32]), so the
 * dots can be checked against it.  x, gamma: device f32 [cols], 16-byte
 * aligned.  cols <= 16384 (LQ_ERR_UNSUPPORTED beyond). */
lq_status lq_q8_block_dots_f32(const lq_q8_weight* w, const float* x, int32_t norm, const float* gamma,
                               float eps, int32_t* dots, int8_t* x_qs_out, uint16_t* x_d_out,
                               void* stream);

/* Q4_0 and Q6_K weight matvecs against a Q8_0 activation, on the int8 x
 * int8 path of [LAT] Current Design: an exact int32 dot over each run of
 * values that share their scales (a Q4_0 block; 16 Q6_K values, which lie in
 * one activation block), then
 *   Q4_0: y[r] = residual[r] + sum_b d[r,b] * f16(x_d[b]) * dot
 *   Q6_K: y[r] = residual[r] + sum_k d[r,k/16] * sc[r,k] * f16(x_d[k/2]) * dot
 * with the float sum in an unspecified order.  Weights as above, cols <=
 * 16384 (LQ_ERR_UNSUPPORTED beyond).  x_qs: device int8 [cols], 16-byte
 * aligned; x_d: device f16 bits [cols/32]; y, residual: device f32 [rows]
 * (residual may be NULL and may alias y).  rows == 0 is a no-op. */
lq_status lq_q4_0_matvec(const lq_q4_0_weight* w, const int8_t* x_qs, const uint16_t* x_d,
                         const float* residual, float* y, void* stream);
lq_status lq_q6_k_matvec(const lq_q6_k_weight* w, const int8_t* x_qs, const uint16_t* x_d,
                         const float* residual, float* y, void* stream);

/* Multi-token Q8_0 matmul: the decode matvec for T tokens at once (prefill,
 * batched decode) in one launch ([LAT] Current Design: int8 weights times
 * int8 activations with int32 accumulation, one f16 scale per 32 values):
 *   y[t, r] = residual[t, r] + sum_b f16(d_w[r,b]) * f16(x_d[t,b]) * dot_b(W[r], X[t])
 * with dot_b the exact int32 dot of block b.  Runs on int8 MFMA; the float
 * sum is in an unspecified but fixed order (results do not vary from run to
 * run).
 *   w: as for lq_q8_matvec, cols <= 16384 (LQ_ERR_UNSUPPORTED beyond).
 *   x_qs: device int8 [T, cols], 16-byte aligned; x_d: device f16 bits [T, cols/32].
 *   residual: device f32 [T, rows] or NULL; y: device f32 [T, rows]; y may
 *   alias residual.
 *   workspace: device memory of lq_q8_matmul_workspace_size(rows, cols, T)
 *   bytes (4-byte aligned; may be NULL when that size is 0), holding partial
 *   sums when a short weight splits its blocks over several workgroups
 *   (T <= 32 only; the size is 0 for more tokens).
 * T == 0 or rows == 0 is a no-op; T >= 2^31, or a launch of 2^31 or more
 * workgroups, is LQ_ERR_UNSUPPORTED. */
size_t lq_q8_matmul_workspace_size(int64_t rows, int64_t cols, int64_t T);
lq_status lq_q8_matmul(const lq_q8_weight* w, const int8_t* x_qs, const uint16_t* x_d, int64_t T,
                       const float* residual, float* y, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ---------------------------------------------------------------- norm + RoPE */
/* In place, for each of n_heads heads of head_dim floats starting at
 * x + h*head_stride ([LAT] Current Design: fused_qk_norm_rope; [CUR]
 * section 4: RMSNorm, then the NeoX rotation of pairs (i, i + head_dim/2)):
 *   x <- gamma * x / sqrt(mean(x^2) + eps)   (gamma NULL: unit weight)
 *   (a, b) <- (a*c - b*s, a*s + b*c),  c, s = rope_cos/sin[pos*head_dim/2 + i]
 * rope_cos == rope_sin == NULL skips the rotation.  head_dim even, 2..512.
 * x: device f32, 4-byte aligned; gamma: device f32 [head_dim];
 * rope tables: device f32 [rope_len, head_dim/2] (see lq_rope_table), with
 * pos < rope_len. */
lq_status lq_rmsnorm_rope(float* x, int64_t n_heads, int64_t head_dim, int64_t head_stride,
                          const float* gamma, float eps, const float* rope_cos,
                          const float* rope_sin, int64_t rope_len, int64_t pos, void* stream);

/* KV-cache append in place ([CUR] section 1 kv-cache-kernel in-place;
 * [TGT] section 6.1 step 6): for every kv head g and dim e,
 *   k_cache[g*head_stride + pos*pos_stride + e] = cvt(k[g*head_dim + e])
 * (same for v), cvt = identity (LQ_KV_F32) or f32->bf16 round-to-nearest-
 * even (LQ_KV_BF16).  k, v: device f32 [n_kv, head_dim].  max_ctx is the
 * number of positions allocated per head: pos < max_ctx. */
lq_status lq_kv_append(const float* k, const float* v, int64_t n_kv, int64_t head_dim,
                       void* k_cache, void* v_cache, int32_t kv_dtype,
                       int64_t head_stride, int64_t pos_stride, int64_t max_ctx, int64_t pos,
                       void* stream);

/* ---------------------------------------------------------------- attention */
/* GQA decode attention ([ENG] BLAS-Fused Attention; [LAT] fused_attention
 * with online softmax, GQA rows per workgroup): for every query head h,
 * with kv head g = h / (n_q / n_kv) (consecutive query heads share a kv
 * head) and positions j in [start, start + len):
 *   s_j   = scale * <q[h], K[g, j]>
 *   out_h = sum_j softmax(s)_j * V[g, j]
 * K[g, j] starts at element g*head_stride + j*pos_stride of the cache
 * (element offsets, never bytes: [CUR] section 7).  The GPU computes the
 * softmax online over splits of the positions and combines the splits.
 *   q: device f32 [n_q, head_dim]; out: device f32 [n_q, head_dim].
 *   caches: device f32 or bf16 (kv_dtype), 16-byte aligned, with
 *   head_stride and pos_stride multiples of 16 bytes; max_ctx is the number
 *   of positions allocated per head: start + len <= max_ctx.
 * Shapes: n_q % n_kv == 0 (INV-3), head_dim % 4 == 0 (INV-2); the kernels
 * also need head_dim % 8 == 0 for bf16, head_dim <= 512 and
 * n_q / n_kv <= 8 (else LQ_ERR_UNSUPPORTED).  len == 0 writes zeros. */
size_t lq_gqa_decode_attn_workspace_size(int64_t n_q, int64_t n_kv, int64_t head_dim,
                                         int64_t len);
lq_status lq_gqa_decode_attn(const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                             const void* k_cache, const void* v_cache, int32_t kv_dtype,
                             int64_t head_stride, int64_t pos_stride, int64_t max_ctx,
                             int64_t start, int64_t len, float scale, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* The same attention for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): arguments,
 * results and errors as lq_gqa_decode_attn, with no workspace.  The split
 * partials go to a device array inside the library, 16 MiB on each GPU,
 * held from module load until the process ends.  Shapes whose partials
 * (lq_gqa_decode_attn_workspace_size) exceed it are refused with
 * LQ_ERR_UNSUPPORTED: every shape of up to 510 kv heads fits.  Every call on
 * a GPU shares that GPU's array, so calls that overlap on one GPU (several
 * streams or host threads) race on it; calls in one stream do not.  The
 * first call on a device looks up the array's address there (the current
 * device must be the stream's); no call allocates or frees memory. */
lq_status lq_gqa_decode_attn_noalloc(const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                                     const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                     int64_t head_stride, int64_t pos_stride, int64_t max_ctx,
                                     int64_t start, int64_t len, float scale, float* out, void* stream);

/* ---------------------------------------------------------------- output head */
/* Final norm, vocab projection on f16 weights and logit softcapping
 * ([CUR] section 3, forward pass steps 4, 5 and 7; section 4,
 * lm_head_kernel: the projection runs on F16 weights; [TGT] section 3.2:
 * rms_norm, f16_gemm, softcap; section 3.3: lm_head_f16 [vocab, hidden] f16,
 * logits [1, vocab] f32), in one launch:
 *   n = norm ? gamma * x / sqrt(mean(x^2) + eps) : x   (gamma NULL: unit weight)
 *   logits[r] = sum_c f16(w[r, c]) * n[c]
 *   if softcap > 0: logits[r] = softcap * tanh(logits[r] / softcap)
 *   w: device f16 bits [vocab, hidden], row-major, 16-byte aligned.
 *   x, gamma: device f32 [hidden], 16-byte aligned.  logits: device f32 [vocab].
 * hidden % 8 == 0 (LQ_ERR_SHAPE) and, for the kernel as written, hidden <= 4096
 * (LQ_ERR_UNSUPPORTED).  vocab == 0 is a no-op.  Float results follow the
 * library's tolerance (the f16 products are exact; sums are f32). */
lq_status lq_lm_head_f16(const uint16_t* w, int64_t vocab, int64_t hidden, const float* x, int32_t norm,
                         const float* gamma, float eps, float softcap, float* logits, void* stream);

/* ---------------------------------------------------------------- MoE */
/* Router ([TGT] section 3.2: softmax, argsort, gather of the top-k
 * probabilities): per token t, p = softmax(logits[t, :E]); ids[t, s] are
 * the k experts with the largest logits (equivalently probabilities), in
 * descending order, ties to the lower id; w[t, s] = p[ids[t, s]] (no
 * renormalisation).  logits: device f32 [T, E]; ids: device int32 [T, k];
 * w: device f32 [T, k].  E <= 1024, k <= min(E, 32). */
lq_status lq_moe_route_topk(const float* logits, int64_t T, int64_t E, int64_t k,
                            int32_t* ids, float* w, void* stream);

/* Index-driven Q8_0 matvec, one row-set per (token, slot) ([CUR] section 4,
 * moe_kernel: each (token, slot) selects an expert's quantized weights by
 * id; [TGT] section 6.3: experts byte-contiguous as [n_experts, rows, cols]):
 *   y[t, s, r] = sum_b f16(dW_e[r,b]) * f16(dx[b]) * dot(W_e[r, b], x[b]),
 *   e = ids[t, s],  x = x_qs/x_d row t (x_per_slot == 0) or row t*k + s
 *   (x_per_slot == 1).
 * w describes ONE expert (rows, cols); expert e's codes start at
 * w->qs + e*rows*cols and its scales at w->d + e*rows*cols/32.  Each touched
 * expert's weights are streamed once for all of its (t, s) rows.
 * ids live on the device and are not checked on the host: a (t, s) whose id
 * is outside [0, n_experts) gets y = 0 and increments the int32 counter at
 * the start of the workspace (read it after synchronizing).
 * y: device f32 [T, k, rows]. */
size_t lq_moe_workspace_size(int64_t T, int64_t k, int64_t n_experts);
lq_status lq_moe_q8_matvec_id(const lq_q8_weight* w, int64_t n_experts,
                              const int8_t* x_qs, const uint16_t* x_d, int32_t x_per_slot,
                              const int32_t* ids, int64_t T, int64_t k, float* y,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The same index-driven matvec with Q4_0 or Q6_K expert weights (the
 * current path's MoE kernel runs on Q6_K, [CUR] section 4), on the int8
 * path of lq_q4_0_matvec / lq_q6_k_matvec.  w describes ONE expert (rows,
 * cols); the arrays hold n_experts experts back to back, expert e's row r
 * being row e*rows + r of each array.  cols <= 8192; ids, workspace, x and
 * y as for lq_moe_q8_matvec_id. */
lq_status lq_moe_q4_0_matvec_id(const lq_q4_0_weight* w, int64_t n_experts, const int8_t* x_qs,
                                const uint16_t* x_d, int32_t x_per_slot, const int32_t* ids, int64_t T,
                                int64_t k, float* y, void* workspace, size_t workspace_bytes, void* stream);
lq_status lq_moe_q6_k_matvec_id(const lq_q6_k_weight* w, int64_t n_experts, const int8_t* x_qs,
                                const uint16_t* x_d, int32_t x_per_slot, const int32_t* ids, int64_t T,
                                int64_t k, float* y, void* workspace, size_t workspace_bytes, void* stream);

/* Weighted sum over slots ([TGT] section 3.2 weighted_sum):
 * out[t, r] = sum_{s<k} w[t, s] * y[t, s, r], slots summed in order s = 0..k-1.
 * y: device f32 [T, k, rows]; w: device f32 [T, k]; out: device f32 [T, rows]. */
lq_status lq_moe_weighted_sum(const float* y, const float* w, int64_t T, int64_t k,
                              int64_t rows, float* out, void* stream);

/* Whole MoE FFN block for T tokens ([CUR] section 3 item i, fused path):
 * route -> Q8(x) -> gate_up id-matvec -> SwiGLU + Q8 -> down id-matvec ->
 * weighted sum.  No host synchronization.  n_experts <= 1024 and
 * top_k <= 32 (the router's limits, as lq_moe_route_topk), T * top_k <=
 * 8192; LQ_ERR_UNSUPPORTED beyond. */
typedef struct lq_moe_desc {
    int64_t hidden, ffn, n_experts, top_k;
    lq_q8_weight w_gate_up;   /* one expert: rows 2*ffn (gate rows, then up rows), cols hidden */
    lq_q8_weight w_down;      /* one expert: rows hidden, cols ffn */
    const float* expert_scale;  /* device f32 [n_experts], or NULL (all 1): per-expert output scale
                                   ([TGT] section 3.2: gather of per_expert_scale, weight * scale) */
} lq_moe_desc;

/* Optional device buffers; a non-NULL tap replaces the workspace buffer for
 * that intermediate, so the caller can read it after synchronizing. */
typedef struct lq_moe_taps {
    int32_t* ids; float* w;           /* [T, k] */
    int8_t* xq; uint16_t* xd;         /* [T, hidden], [T, hidden/32] */
    float* y1;                        /* [T, k, 2*ffn] */
    int8_t* hq; uint16_t* hd;         /* [T, k, ffn], [T, k, ffn/32] */
    float* y2;                        /* [T, k, hidden] */
} lq_moe_taps;

size_t lq_moe_block_workspace_size(const lq_moe_desc* m, int64_t T);
lq_status lq_moe_block(const lq_moe_desc* m, const float* x, const float* logits, int64_t T,
                       float* out, const lq_moe_taps* taps,
                       void* workspace, size_t workspace_bytes, void* stream);

/* The same MoE block with Q4_0 or Q6_K expert weights (the current path's
 * MoE runs Q6_K experts through the index-driven matvec, [CUR] section 4;
 * [TGT] section 3.2 lists the same block op by op): route -> Q8(x) ->
 * gate_up id-matvec -> SwiGLU + Q8 -> down id-matvec -> weighted sum, with
 * the id-matvecs of lq_moe_q4_0_matvec_id / lq_moe_q6_k_matvec_id.
 * gate_up_format and down_format are LQ_FMT_Q4_0 or LQ_FMT_Q6_K and name
 * which of the two weight descriptors of each matrix is used (the other is
 * ignored); each describes ONE expert as in lq_moe_q4_0_matvec_id: gate_up
 * rows 2*ffn (gate rows, then up rows) by hidden columns, down rows hidden by
 * ffn columns, the experts back to back.  hidden and ffn <= 8192 and
 * multiples of 32 (Q4_0) or 256 (Q6_K) where they are a weight's columns.
 * Taps, workspace, expert_scale and errors as for lq_moe_block; the y1 tap
 * holds the gate_up outputs before SwiGLU. */
typedef struct lq_moe_ggml_desc {
    int64_t hidden, ffn, n_experts, top_k;
    int32_t gate_up_format, down_format;
    lq_q4_0_weight gate_up_q4_0;
    lq_q6_k_weight gate_up_q6_k;
    lq_q4_0_weight down_q4_0;
    lq_q6_k_weight down_q6_k;
    const float* expert_scale;  /* device f32 [n_experts], or NULL (all 1) */
} lq_moe_ggml_desc;

size_t lq_moe_block_ggml_workspace_size(const lq_moe_ggml_desc* m, int64_t T);
lq_status lq_moe_block_ggml(const lq_moe_ggml_desc* m, const float* x, const float* logits, int64_t T,
                            float* out, const lq_moe_taps* taps,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- decode layer */
#define LQ_LAYER_PRENORM_FFN     0   /* x -> norm -> QKV -> qk-norm/RoPE -> KV append -> attn -> O + x
                                        -> norm -> gate_up -> SwiGLU -> down + x1 */
#define LQ_LAYER_ATTN_POSTNORM   1   /* Gemma attention block: ... -> attn -> O -> norm -> + x */

/* FFN gate activation of LQ_LAYER_PRENORM_FFN: h = act(gate) * up. */
#define LQ_ACT_SILU        0   /* SwiGLU: silu(z) = z / (1 + exp(-z)) */
#define LQ_ACT_GELU_TANH   1   /* GeGLU, the Gemma MLP gate ([TGT] section 3.2 lists gelu in the
                                  decode op list): 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */

typedef struct lq_layer_desc {
    int64_t hidden, n_q, n_kv, head_dim;
    int64_t ffn;              /* used by LQ_LAYER_PRENORM_FFN */
    int64_t max_ctx;          /* positions allocated per kv head in each cache */
    int64_t window;           /* 0: full causal context; W: positions [pos-W+1, pos] */
    float eps, attn_scale;
    int32_t kind;
    int32_t kv_dtype;
    int32_t qk_norm;          /* per-head RMSNorm of q (g_q) and k (g_k) */
    int32_t v_unit_norm;      /* unit-weight RMSNorm of v ([CUR] section 3, rms_norm_unit) */
    lq_q8_weight w_qkv;       /* [n_q*hd + 2*n_kv*hd, hidden] (INV-7): q rows, k rows, v rows */
    lq_q8_weight w_o;         /* [hidden, n_q*hd] */
    lq_q8_weight w_gate_up;   /* [2*ffn, hidden]: gate rows, then up rows */
    lq_q8_weight w_down;      /* [hidden, ffn] */
    const float *g_in;        /* [hidden] input norm */
    const float *g_q, *g_k;   /* [head_dim] */
    const float *g_post;      /* [hidden] post-attention norm */
    void *k_cache, *v_cache;  /* [n_kv, max_ctx, head_dim], contiguous */
    const float *rope_cos, *rope_sin;   /* [max_ctx, head_dim/2] */
    int32_t ffn_act;          /* LQ_ACT_SILU (0) or LQ_ACT_GELU_TANH */
    float attn_softcap;       /* > 0: each scaled score s becomes cap * tanh(s / cap) before the softmax
                                 (the optional Gemma score softcap of [ENG] BLAS-Fused Attention);
                                 0: none */
    int32_t w_format[4];      /* formats of the projections, in the order qkv, o, gate_up, down
                                 ([CUR] section 4: the current path runs GGML Q6_K weights; [TGT]
                                 section 8, Q1: GGML block order).  LQ_FMT_Q8_0 (0, the default)
                                 takes w_qkv / w_o / w_gate_up / w_down above; LQ_FMT_Q4_0 and
                                 LQ_FMT_Q6_K take w_q4_0[i] / w_q6_k[i] below, with the same rows
                                 and cols (Q6_K: cols % 256 == 0; a Q6_K gate_up needs hidden <=
                                 12288, else LQ_ERR_UNSUPPORTED).  The activations stay Q8_0, the
                                 prologues and epilogues are the same, so is the launch count. */
    lq_q4_0_weight w_q4_0[4];
    lq_q6_k_weight w_q6_k[4];
} lq_layer_desc;

/* Optional device buffers for the layer's intermediates; read them after
 * synchronizing.  qkv, attn and x1 replace the workspace buffer of that
 * intermediate; h (silu(gate) * up, never otherwise stored) is written when
 * given.  xq/xd, aq/ad and nq/nd are the quantized inputs that the matvec
 * kernels build in on-chip memory; when a tap is given, one workgroup also
 * writes its copy there.  hq/hd (given together, else neither is written)
 * replace the workspace buffer of the quantized h that the gate_up
 * epilogue produces and the down projection reads. */
typedef struct lq_layer_taps {
    int8_t* xq; uint16_t* xd;  /* Q8 of the input norm [hidden], [hidden/32] */
    float* qkv;                /* raw fused projection [n_q*hd + 2*n_kv*hd] */
    float* attn;               /* attention output [n_q*hd] */
    int8_t* aq; uint16_t* ad;  /* Q8 of the attention output */
    float* x1;                 /* PRENORM_FFN: x + O projection; ATTN_POSTNORM: the O
                                  projection before the post-attention norm [hidden] */
    int8_t* nq; uint16_t* nd;  /* Q8 of the post-attention norm (PRENORM_FFN) */
    float* h;                  /* silu(gate) * up [ffn] */
    int8_t* hq; uint16_t* hd;  /* Q8 of h */
    float* qkv_post;           /* q and k after the per-head norm and RoPE, v after its optional
                                  unit norm, as f32 before the attention scale and before the
                                  conversion to the cache dtype [n_q*hd + 2*n_kv*hd]: the cache
                                  rows written at pos are exactly cvt(k), cvt(v) of these */
} lq_layer_taps;

/* One decode token through one layer ([CUR] section 3 sequence; [TGT]
 * section 3.2, one queue and no intermediate host synchronization): x
 * (device f32 [hidden]) is updated in place; k and v of the token are
 * written into the caches at pos (pos < max_ctx); attention covers the
 * window ending at pos.  taps may be NULL.
 * The kernels need head_dim % 8 == 0 (<= 512), hidden, n_q*head_dim
 * and ffn <= 16384, and 16-byte aligned x, norm weights, RoPE tables and
 * caches (LQ_ERR_UNSUPPORTED / LQ_ERR_ALIGN otherwise). */
size_t lq_decode_layer_workspace_size(const lq_layer_desc* L);
lq_status lq_decode_layer(const lq_layer_desc* L, float* x, int64_t pos,
                          const lq_layer_taps* taps, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Measurement entry point: lq_decode_layer with every kernel launched with a
 * start/stop hipEvent_t pair on `stream` (hipExtLaunchKernelGGL: the runtime
 * stamps the events at that dispatch's own start and end), so a caller can
 * time each kernel of the layer on the stream it runs on.  Kernel k uses
 * events[2k] and events[2k+1].  events: host array of n_events hipEvent_t
 * handles (passed as void*) created by the caller; n_events must be at
 * least 2 * lq_decode_layer_kernel_count(L).  Same results as
 * lq_decode_layer. */
int32_t lq_decode_layer_kernel_count(const lq_layer_desc* L);
lq_status lq_decode_layer_timed(const lq_layer_desc* L, float* x, int64_t pos,
                                const lq_layer_taps* taps, void* workspace, size_t workspace_bytes,
                                void* const* events, int32_t n_events, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LQ_H */

// lq_internal.h -- host-side internals of liblq: error reporting and the
// unchecked launchers that the public entry points and the composites
// (decode layer, MoE block) share.  Every launcher assumes its arguments were
// validated by the caller.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lq.h"

namespace lq {

constexpr int kNumCUs = 256;   // MI355X compute units

// Optional per-kernel timing for the measurement entry point of the decode
// layer: kernel k of a run gets the start/stop event pair (ev[2k], ev[2k+1]),
// stamped by the runtime at that dispatch's own start and end.
struct LaunchMarks {
    void* const* ev;
    int n, k;
    bool next(hipEvent_t* start, hipEvent_t* stop) {
        const bool ok = ev && 2 * k + 1 < n;
        if (ok) {
            *start = reinterpret_cast<hipEvent_t>(ev[2 * k]);
            *stop = reinterpret_cast<hipEvent_t>(ev[2 * k + 1]);
        }
        ++k;
        return ok;
    }
};

// Launches a kernel, with start/stop events when timing marks are given.
template <typename K, typename... Args>
inline void launch_marked(LaunchMarks* mk, K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                          Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (mk && mk->next(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

// Records a thread-local message for lq_last_error() and returns s.
lq_status fail(lq_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Maps a pending HIP launch error to LQ_ERR_HIP.
lq_status check_launch(const char* what);

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Validates an lq_q8_weight (pointers, cols % 32, alignment).
lq_status check_weight(const lq_q8_weight* w, const char* name);

// ---- launchers (k_quant.hip) ------------------------------------------------
lq_status launch_q8_quantize(const float* x, int64_t n_blocks, int8_t* qs, uint16_t* d,
                             hipStream_t s);
lq_status launch_rmsnorm_q8(const float* x, int64_t n_rows, int64_t n, const float* gamma,
                            float eps, int8_t* qs, uint16_t* d, hipStream_t s);
lq_status launch_swiglu_q8(const float* gate_up, int64_t n_rows, int64_t ffn, int8_t* qs,
                           uint16_t* d, hipStream_t s);
// out = res + gamma * o / sqrt(mean(o^2) + eps) for one vector (n % 4 == 0).
lq_status launch_rmsnorm_add(const float* o, int64_t n, const float* gamma, float eps, const float* res,
                             float* out, hipStream_t s, struct LaunchMarks* mk = nullptr);

// ---- launchers (k_matvec.hip) -----------------------------------------------
lq_status launch_q8_matvec(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                           const int8_t* xq, const uint16_t* xd, const float* residual, float* y,
                           int32_t* dots, hipStream_t s);

// Fused matvec (see k_matvec.hip): prologue PRO_* builds the Q8_0 input,
// epilogue EPI_* stores, adds a residual or applies SwiGLU to row pairs;
// EPI_SWIGLU_Q8 also quantizes the SwiGLU output to Q8_0 (yq, yd), each
// workgroup owning whole 32-value blocks.
enum { PRO_Q8 = 0, PRO_QUANT = 1, PRO_NORM = 2 };
// EPI_DOTS writes every int32 block dot (dots[r*cols/32 + b]) instead of y:
// the test tap of the block dots this kernel forms.
enum { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_SWIGLU_Q8 = 3, EPI_DOTS = 4 };
constexpr int kMvWgPerCu = 4;   // upper bound on resident workgroups of 4 waves per CU
struct MvArgs {
    const int8_t* wq;
    const uint16_t* wd;
    int rows;            // output rows (SwiGLU: rows of h; the weight has 2*rows)
    int cols;            // <= 16384
    const int8_t* xq;    // PRO_Q8: codes and scales in memory
    const uint16_t* xd;
    const float* x;      // PRO_QUANT / PRO_NORM: f32 input
    const float* gamma;  // PRO_NORM (NULL: unit weight)
    float eps;
    const float* res;    // EPI_RESID (may alias y)
    float* y;            // EPI_SWIGLU_Q8: optional (NULL: f32 output not written)
    int8_t* yq;          // EPI_SWIGLU_Q8: Q8_0 codes [rows] and scales [rows/32]
    uint16_t* yd;
    int8_t* tap_q;       // optional: workgroup 0 writes the Q8_0 input it built
    uint16_t* tap_d;
    int act;             // EPI_SWIGLU*: gate activation, LQ_ACT_SILU or LQ_ACT_GELU_TANH
    int32_t* dots;       // EPI_DOTS: int32 [rows, cols/32]
};
lq_status launch_mv(const MvArgs& a, int pro, int epi, hipStream_t s, int wg_per_cu,
                    LaunchMarks* mk = nullptr);

// A projection weight in any of the library's formats: LQ_FMT_Q8_0 (q0 =
// codes, d = scales), LQ_FMT_Q4_0 (q0 = qs, d) or LQ_FMT_Q6_K (q0 = ql, q1 =
// qh, sc, d); device arrays as include/lq.h lays them out.
struct ProjWeight {
    int fmt;
    const void* q0;
    const void* q1;
    const int8_t* sc;
    const uint16_t* d;
};
// The fused matvec of MvArgs (prologue, epilogue, taps; wq/wd ignored) on a
// weight of any format: the Q8_0 kernels for LQ_FMT_Q8_0, the Q4_0 / Q6_K
// kernels of k_qk.hip otherwise (same prologues and epilogues; EPI_SWIGLU
// without Q8 and EPI_DOTS only for Q8_0).
lq_status launch_proj(const ProjWeight& w, const MvArgs& m, int pro, int epi, hipStream_t s,
                      LaunchMarks* mk = nullptr);
// Validates the weight of format fmt among the three descriptors (shape
// rows x cols, pointers, alignment) and fills *out.
lq_status check_proj_weight(const char* fn, const char* what, int32_t fmt, const lq_q8_weight& q8,
                            const lq_q4_0_weight& q4, const lq_q6_k_weight& q6, int64_t rows, int64_t cols,
                            ProjWeight* out);

// ---- launchers (k_norm_rope.hip) ----------------------------------------------
lq_status launch_rmsnorm_rope(float* x, int64_t n_heads, int64_t hd, int64_t head_stride,
                              const float* gamma, float eps, const float* rope_cos,
                              const float* rope_sin, int64_t pos, hipStream_t s);
lq_status launch_kv_append(const float* k, const float* v, int64_t n_kv, int64_t hd, void* kc,
                           void* vc, int32_t kv_dtype, int64_t head_stride, int64_t pos_stride,
                           int64_t pos, hipStream_t s);
// Decode-layer step after the QKV projection: per-head q/k RMSNorm (if
// qk_norm) + NeoX RoPE in place on qkv, optional unit norm of v, then the
// append of k and v at pos.
lq_status launch_qkv_post(float* qkv, int64_t n_q, int64_t n_kv, int64_t hd, const float* g_q,
                          const float* g_k, int32_t qk_norm, int32_t v_unit_norm, float eps,
                          const float* rope_cos, const float* rope_sin, int64_t pos, void* kc,
                          void* vc, int32_t kv_dtype, int64_t head_stride, int64_t pos_stride,
                          hipStream_t s);

// ---- launchers (k_attn.hip) ---------------------------------------------------
bool attn_supported(int64_t n_q, int64_t n_kv, int64_t hd, int32_t kv_dtype);
// Split partials of an attention over len positions; `layer`: the decode
// layer's region, which also serves every shorter length.
size_t attn_workspace_bytes(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len, bool layer = false);
// splits the layer's attention uses (1: no combine launch); vec_ok: 16-byte aligned query rows
int attn_nsplit(int64_t n_q, int64_t n_kv, int64_t hd, int64_t len, int32_t kv_dtype, bool vec_ok);
// The host-side checks of lq_gqa_decode_attn other than the workspace's.
lq_status check_attention_args(const char* fn, const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                               const void* k_cache, const void* v_cache, int32_t kv_dtype, int64_t head_stride,
                               int64_t pos_stride, int64_t max_ctx, int64_t start, int64_t len, const float* out);
lq_status launch_attention(const float* q, int64_t n_q, int64_t n_kv, int64_t hd, const void* kc,
                           const void* vc, int32_t kv_dtype, int64_t head_stride,
                           int64_t pos_stride, int64_t start, int64_t len, float scale,
                           float* out, void* ws, hipStream_t s);
// Decode-layer attention with the per-head q/k RMSNorm + NeoX RoPE, the v
// unit norm and the KV append (at start + len - 1) done in the kernel's
// prologue; qkv is the raw fused projection.  rope rows are at that position.
// tap_post (optional, [n_q*hd + 2*n_kv*hd]) receives q, k and v after that
// prologue, before the attention scale and the cache conversion.
lq_status launch_attention_fused(const float* qkv, int64_t n_q, int64_t n_kv, int64_t hd, const float* g_q,
                                 const float* g_k, int32_t qk_norm, int32_t v_unit_norm, float eps,
                                 const float* rope_cos_row, const float* rope_sin_row, void* kc, void* vc,
                                 int32_t kv_dtype, int64_t head_stride, int64_t pos_stride, int64_t start,
                                 int64_t len, float scale, float softcap, float* out, void* ws, hipStream_t s,
                                 LaunchMarks* marks = nullptr, float* tap_post = nullptr);

// ---- launchers (k_moe.hip) ----------------------------------------------------
size_t moe_ws_bytes(int64_t T, int64_t k, int64_t n_experts);
lq_status launch_moe_route(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* ids,
                           float* w, hipStream_t s);
lq_status launch_moe_matvec_id(const int8_t* wq, const uint16_t* wd, int64_t rows, int64_t cols,
                               int64_t n_experts, const int8_t* xq, const uint16_t* xd,
                               int32_t x_per_slot, const int32_t* ids, int64_t T, int64_t k,
                               float* y, void* ws, hipStream_t s);
// out[t] = sum_s w[t,s] * escale[ids[t,s]] * y[t,s] (escale NULL: scale 1; ids, E only read with escale)
lq_status launch_moe_weighted_sum(const float* y, const float* w, int64_t T, int64_t k, int64_t rows,
                                  const int32_t* ids, const float* escale, int64_t E, float* out, hipStream_t s);

}  // namespace lq

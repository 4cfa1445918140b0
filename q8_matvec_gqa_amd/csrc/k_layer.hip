// k_layer.hip -- one decode token through one transformer layer.
//
// The step order is the per-token decode sequence of "Current Inference
// Path -- Architecture Map" (section 3: input norm, Q/K/V projections,
// Q/K norms, V unit norm, RoPE, KV append, SDPA, O projection, post-
// attention norm, residual, MLP) with the fused QKV weight of "Design:
// lattice-inference" (INV-7), run as one queue of kernels with no host
// synchronization inside ("Target Inference Architecture: hf2q on
// mlx-native", section 3.2 and design principle P2: one commit per forward
// pass).  Every intermediate lives in the caller's workspace (INV-8: no
// allocation in the forward pass), or in a caller tap buffer.
#include <math.h>
#include "lq_device.h"
#include "lq_internal.h"

namespace lq {
namespace {

struct LayerBuffers {
    float* qkv;
    float* attn;
    float* x1;
    int8_t* hq;          // Q8_0 of silu(gate) * up, written by the gate_up epilogue
    uint16_t* hd;
    void* attn_ws;
    size_t total;
};

int64_t max_attn_len(const lq_layer_desc* L) {
    return (L->window > 0 && L->window < L->max_ctx) ? L->window : L->max_ctx;
}

LayerBuffers layout(const lq_layer_desc* L, char* base, const lq_layer_taps* taps) {
    const int64_t H = L->hidden, qd = L->n_q * L->head_dim, kvd = L->n_kv * L->head_dim;
    const int64_t I = L->kind == LQ_LAYER_PRENORM_FFN ? L->ffn : 0;
    LayerBuffers b{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += round_up(bytes ? bytes : 1, 256);
        return p;
    };
    b.qkv = reinterpret_cast<float*>(take((qd + 2 * kvd) * 4));
    b.attn = reinterpret_cast<float*>(take(qd * 4));
    b.x1 = reinterpret_cast<float*>(take(H * 4));
    b.hq = reinterpret_cast<int8_t*>(take(I));
    b.hd = reinterpret_cast<uint16_t*>(take(I / 32 * 2));
    b.attn_ws = take(attn_workspace_bytes(L->n_q, L->n_kv, L->head_dim, max_attn_len(L), true));
    b.total = off;
    if (taps) {
        if (taps->qkv) b.qkv = taps->qkv;
        if (taps->attn) b.attn = taps->attn;
        if (taps->x1) b.x1 = taps->x1;
        if (taps->hq && taps->hd) {
            b.hq = taps->hq;
            b.hd = taps->hd;
        }
    }
    return b;
}

// rows x cols of projection i (qkv, o, gate_up, down) as its format's descriptor states them
bool weight_is(const lq_layer_desc* L, int i, int64_t rows, int64_t cols) {
    const lq_q8_weight* q8[4] = {&L->w_qkv, &L->w_o, &L->w_gate_up, &L->w_down};
    int64_t r = q8[i]->rows, c = q8[i]->cols;
    if (L->w_format[i] == LQ_FMT_Q4_0) {
        r = L->w_q4_0[i].rows; c = L->w_q4_0[i].cols;
    } else if (L->w_format[i] == LQ_FMT_Q6_K) {
        r = L->w_q6_k[i].rows; c = L->w_q6_k[i].cols;
    }
    return r == rows && c == cols;
}

lq_status validate(const lq_layer_desc* L, const float* x, int64_t pos, ProjWeight (&pw)[4]) {
    const char* fn = "lq_decode_layer";
    if (!L) return fail(LQ_ERR_NULL, "%s: descriptor is NULL", fn);
    const int64_t H = L->hidden, nq = L->n_q, nkv = L->n_kv, hd = L->head_dim;
    if (L->kind != LQ_LAYER_PRENORM_FFN && L->kind != LQ_LAYER_ATTN_POSTNORM)
        return fail(LQ_ERR_SHAPE, "%s: kind %d", fn, L->kind);
    if (H <= 0 || H % 32 || nq <= 0 || nkv <= 0 || nq % nkv || hd <= 0 || hd % 4 || (nq * hd) % 32)
        return fail(LQ_ERR_SHAPE, "%s: hidden=%lld n_q=%lld n_kv=%lld head_dim=%lld", fn, (long long)H,
                    (long long)nq, (long long)nkv, (long long)hd);
    if (L->kv_dtype != LQ_KV_F32 && L->kv_dtype != LQ_KV_BF16)
        return fail(LQ_ERR_SHAPE, "%s: kv_dtype %d", fn, L->kv_dtype);
    if (L->max_ctx <= 0 || pos < 0 || pos >= L->max_ctx || L->window < 0)
        return fail(LQ_ERR_SHAPE, "%s: pos=%lld max_ctx=%lld window=%lld", fn, (long long)pos,
                    (long long)L->max_ctx, (long long)L->window);
    if (!(L->eps >= 0.0f)) return fail(LQ_ERR_SHAPE, "%s: eps must be >= 0", fn);
    if (L->ffn_act != LQ_ACT_SILU && L->ffn_act != LQ_ACT_GELU_TANH)
        return fail(LQ_ERR_SHAPE, "%s: ffn_act %d", fn, L->ffn_act);
    if (!(L->attn_softcap >= 0.0f) || L->attn_softcap == INFINITY)
        return fail(LQ_ERR_SHAPE, "%s: attn_softcap must be finite and >= 0", fn);
    for (int i = 0; i < 4; ++i)
        if (L->w_format[i] != LQ_FMT_Q8_0 && L->w_format[i] != LQ_FMT_Q4_0 && L->w_format[i] != LQ_FMT_Q6_K)
            return fail(LQ_ERR_SHAPE, "%s: w_format[%d] = %d", fn, i, L->w_format[i]);
    if (!weight_is(L, 0, nq * hd + 2 * nkv * hd, H) || !weight_is(L, 1, H, nq * hd))
        return fail(LQ_ERR_SHAPE, "%s: w_qkv must be [%lld, %lld] and w_o [%lld, %lld]", fn,
                    (long long)(nq * hd + 2 * nkv * hd), (long long)H, (long long)H, (long long)(nq * hd));
    if (L->kind == LQ_LAYER_PRENORM_FFN) {
        const int64_t I = L->ffn;
        if (I <= 0 || I % 32 || !weight_is(L, 2, 2 * I, H) || !weight_is(L, 3, H, I))
            return fail(LQ_ERR_SHAPE, "%s: ffn=%lld with w_gate_up [2*ffn, hidden] and w_down [hidden, ffn]", fn,
                        (long long)I);
    }
    if (hd > 512 || hd % 8 || !attn_supported(nq, nkv, hd, L->kv_dtype))
        return fail(LQ_ERR_UNSUPPORTED, "%s: head_dim=%lld G=%lld kv_dtype=%d not built", fn, (long long)hd,
                    (long long)(nq / nkv), L->kv_dtype);
    lq_status st;
    const lq_q8_weight* q8[4] = {&L->w_qkv, &L->w_o, &L->w_gate_up, &L->w_down};
    const char* names[4] = {"w_qkv", "w_o", "w_gate_up", "w_down"};
    const int n_proj = L->kind == LQ_LAYER_PRENORM_FFN ? 4 : 2;
    for (int i = 0; i < n_proj; ++i) {
        const int64_t rows = i == 0 ? nq * hd + 2 * nkv * hd : i == 2 ? 2 * L->ffn : H;
        const int64_t cols = i == 1 ? nq * hd : i == 3 ? L->ffn : H;
        if ((st = check_proj_weight(fn, names[i], L->w_format[i], *q8[i], L->w_q4_0[i], L->w_q6_k[i], rows, cols,
                                    &pw[i])) != LQ_OK)
            return st;
    }
    if (L->kind == LQ_LAYER_PRENORM_FFN && !L->g_post) return fail(LQ_ERR_NULL, "%s: g_post is NULL", fn);
    if (!x || !L->g_in || !L->k_cache || !L->v_cache || !L->rope_cos || !L->rope_sin)
        return fail(LQ_ERR_NULL, "%s: NULL pointer (x, g_in, caches and RoPE tables are required)", fn);
    if (L->qk_norm && (!L->g_q || !L->g_k)) return fail(LQ_ERR_NULL, "%s: qk_norm needs g_q and g_k", fn);
    if (!aligned(x, 16) || !aligned(L->g_in, 16) || (L->g_post && !aligned(L->g_post, 16)) ||
        (L->g_q && !aligned(L->g_q, 16)) || (L->g_k && !aligned(L->g_k, 16)) || !aligned(L->rope_cos, 16) ||
        !aligned(L->rope_sin, 16) || !aligned(L->k_cache, 16) || !aligned(L->v_cache, 16))
        return fail(LQ_ERR_ALIGN, "%s: x, norm weights, RoPE tables and caches must be 16-byte aligned", fn);
    const size_t es = L->kv_dtype == LQ_KV_F32 ? 4 : 2;
    if ((hd * es) % 16) return fail(LQ_ERR_ALIGN, "%s: cache rows must be a multiple of 16 bytes", fn);
    if (H > 16384 || nq * hd > 16384 || (L->kind == LQ_LAYER_PRENORM_FFN && L->ffn > 16384) ||
        nq * hd + 2 * nkv * hd > 0x7fffffffLL || 2 * L->ffn > 0x7fffffffLL)
        return fail(LQ_ERR_UNSUPPORTED, "%s: matvec inputs are limited to 16384 columns", fn);
    if (L->kind == LQ_LAYER_PRENORM_FFN && L->w_format[2] == LQ_FMT_Q6_K && H > 12288)
        return fail(LQ_ERR_UNSUPPORTED, "%s: a Q6_K gate_up needs hidden <= 12288", fn);
    return LQ_OK;
}

lq_status validate_taps(const lq_layer_taps* t) {
    if (!t) return LQ_OK;
    const void* f32s[] = {t->qkv, t->attn, t->x1, t->h, t->xq, t->aq, t->nq, t->hq, t->qkv_post};
    for (const void* p : f32s)
        if (p && !aligned(p, 16)) return fail(LQ_ERR_ALIGN, "lq_decode_layer: tap buffers must be 16-byte aligned");
    const void* d16[] = {t->xd, t->ad, t->nd, t->hd};
    for (const void* p : d16)
        if (p && !aligned(p, 2)) return fail(LQ_ERR_ALIGN, "lq_decode_layer: scale taps must be 2-byte aligned");
    return LQ_OK;
}

}  // namespace
}  // namespace lq

using namespace lq;

extern "C" size_t lq_decode_layer_workspace_size(const lq_layer_desc* L) {
    if (!L || L->hidden <= 0 || L->n_q <= 0 || L->n_kv <= 0 || L->head_dim <= 0 || L->max_ctx <= 0) return 0;
    return layout(L, nullptr, nullptr).total;
}

namespace {
using Marks = LaunchMarks;

int kernel_count(const lq_layer_desc* L, int64_t len) {
    // QKV, attention (+ split combine), O, then gate_up and down, or the post-norm add
    const bool combine = attn_nsplit(L->n_q, L->n_kv, L->head_dim, len, L->kv_dtype, true) > 1;
    return 3 + (combine ? 1 : 0) + (L->kind == LQ_LAYER_PRENORM_FFN ? 2 : 1);
}

lq_status run_layer(const lq_layer_desc* L, float* x, int64_t pos, const lq_layer_taps* taps, void* workspace,
                    size_t workspace_bytes, Marks& mk, hipStream_t s);
}  // namespace

extern "C" int32_t lq_decode_layer_kernel_count(const lq_layer_desc* L) {
    if (!L) return 0;
    return kernel_count(L, (L->window > 0 && L->window < L->max_ctx) ? L->window : L->max_ctx);
}

extern "C" lq_status lq_decode_layer(const lq_layer_desc* L, float* x, int64_t pos, const lq_layer_taps* taps,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    Marks mk{nullptr, 0, 0};
    return run_layer(L, x, pos, taps, workspace, workspace_bytes, mk, as_stream(stream));
}

extern "C" lq_status lq_decode_layer_timed(const lq_layer_desc* L, float* x, int64_t pos,
                                           const lq_layer_taps* taps, void* workspace, size_t workspace_bytes,
                                           void* const* events, int32_t n_events, void* stream) {
    if (!events) return fail(LQ_ERR_NULL, "lq_decode_layer_timed: events is NULL");
    if (!L) return fail(LQ_ERR_NULL, "lq_decode_layer_timed: descriptor is NULL");
    if (pos < 0 || pos >= L->max_ctx) return fail(LQ_ERR_SHAPE, "lq_decode_layer_timed: pos out of range");
    int64_t start = 0;
    if (L->window > 0 && pos - L->window + 1 > 0) start = pos - L->window + 1;
    const int need = 2 * kernel_count(L, pos - start + 1);
    if (n_events < need)
        return fail(LQ_ERR_SHAPE, "lq_decode_layer_timed: needs %d events, got %d", need, n_events);
    Marks mk{events, n_events, 0};
    return run_layer(L, x, pos, taps, workspace, workspace_bytes, mk, as_stream(stream));
}

namespace {
lq_status run_layer(const lq_layer_desc* L, float* x, int64_t pos, const lq_layer_taps* taps, void* workspace,
                    size_t workspace_bytes, Marks& mk, hipStream_t s) {
    ProjWeight pw[4] = {};
    lq_status st = validate(L, x, pos, pw);
    if (st != LQ_OK) return st;
    if ((st = validate_taps(taps)) != LQ_OK) return st;
    const size_t need = layout(L, nullptr, nullptr).total;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(LQ_ERR_WORKSPACE, "lq_decode_layer: workspace needs %zu bytes (256-byte aligned), got %zu", need,
                    workspace_bytes);
    const LayerBuffers b = layout(L, static_cast<char*>(workspace), taps);
    const int64_t H = L->hidden, nq = L->n_q, nkv = L->n_kv, hd = L->head_dim, qd = nq * hd;
    const int64_t head_stride = L->max_ctx * hd, pos_stride = hd;
    int64_t start = 0;
    if (L->window > 0 && pos - L->window + 1 > 0) start = pos - L->window + 1;
    const int64_t len = pos - start + 1;

    const lq_layer_taps T = taps ? *taps : lq_layer_taps{};
    MvArgs m{};

    // attention block: QKV projection with the input RMSNorm + Q8 built in-kernel
    m = MvArgs{};
    m.rows = (int)(nq * hd + 2 * nkv * hd); m.cols = (int)H;
    m.x = x; m.gamma = L->g_in; m.eps = L->eps; m.y = b.qkv; m.tap_q = T.xq; m.tap_d = T.xd;
    if ((st = launch_proj(pw[0], m, PRO_NORM, EPI_STORE, s, &mk)) != LQ_OK) return st;
    // attention, with the per-head norms, RoPE and the KV append in its prologue
    const int64_t half = hd / 2;
    if ((st = launch_attention_fused(b.qkv, nq, nkv, hd, L->g_q, L->g_k, L->qk_norm, L->v_unit_norm, L->eps,
                                     L->rope_cos + pos * half, L->rope_sin + pos * half, L->k_cache, L->v_cache,
                                     L->kv_dtype, head_stride, pos_stride, start, len, L->attn_scale,
                                     L->attn_softcap, b.attn,
                                     b.attn_ws, s, &mk, T.qkv_post)) != LQ_OK)
        return st;
    // O projection, quantizing the attention output in-kernel
    m = MvArgs{};
    m.rows = (int)H; m.cols = (int)qd;
    m.x = b.attn; m.y = b.x1; m.tap_q = T.aq; m.tap_d = T.ad;
    if (L->kind == LQ_LAYER_ATTN_POSTNORM) {
        if ((st = launch_proj(pw[1], m, PRO_QUANT, EPI_STORE, s, &mk)) != LQ_OK) return st;
        return launch_rmsnorm_add(b.x1, H, L->g_post, L->eps, x, x, s, &mk);
    }
    m.res = x;
    if ((st = launch_proj(pw[1], m, PRO_QUANT, EPI_RESID, s, &mk)) != LQ_OK) return st;
    // FFN: gate/up with the post-attention RMSNorm + Q8 in-kernel, SwiGLU on
    // row pairs, and the Q8_0 of the SwiGLU output built by the workgroup that
    // owns each 32-value block
    const int64_t I = L->ffn;
    m = MvArgs{};
    m.rows = (int)I; m.cols = (int)H;
    m.x = b.x1; m.gamma = L->g_post; m.eps = L->eps; m.y = T.h; m.yq = b.hq; m.yd = b.hd; m.act = L->ffn_act;
    m.tap_q = T.nq; m.tap_d = T.nd;
    if ((st = launch_proj(pw[2], m, PRO_NORM, EPI_SWIGLU_Q8, s, &mk)) != LQ_OK) return st;
    // down projection on the Q8_0 h, plus the residual
    m = MvArgs{};
    m.rows = (int)H; m.cols = (int)I;
    m.xq = b.hq; m.xd = b.hd; m.res = b.x1; m.y = x;
    return launch_proj(pw[3], m, PRO_Q8, EPI_RESID, s, &mk);
}
}  // namespace

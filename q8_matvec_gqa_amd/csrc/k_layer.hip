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
#include "lq_device.h"
#include "lq_internal.h"

namespace lq {
namespace {

struct LayerBuffers {
    int8_t* xq; uint16_t* xd;
    float* qkv;
    float* attn;
    int8_t* aq; uint16_t* ad;
    float* x1;
    int8_t* nq; uint16_t* nd;
    float* gu;
    int8_t* hq; uint16_t* hd;
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
    b.xq = reinterpret_cast<int8_t*>(take(H));
    b.xd = reinterpret_cast<uint16_t*>(take(H / 32 * 2));
    b.qkv = reinterpret_cast<float*>(take((qd + 2 * kvd) * 4));
    b.attn = reinterpret_cast<float*>(take(qd * 4));
    b.aq = reinterpret_cast<int8_t*>(take(qd));
    b.ad = reinterpret_cast<uint16_t*>(take(qd / 32 * 2));
    b.x1 = reinterpret_cast<float*>(take(H * 4));
    b.nq = reinterpret_cast<int8_t*>(take(H));
    b.nd = reinterpret_cast<uint16_t*>(take(H / 32 * 2));
    b.gu = reinterpret_cast<float*>(take(2 * I * 4));
    b.hq = reinterpret_cast<int8_t*>(take(I));
    b.hd = reinterpret_cast<uint16_t*>(take(I / 32 * 2));
    b.attn_ws = take(attn_workspace_bytes(L->n_q, L->n_kv, L->head_dim, max_attn_len(L)));
    b.total = off;
    if (taps) {
        if (taps->xq) b.xq = taps->xq;
        if (taps->xd) b.xd = taps->xd;
        if (taps->qkv) b.qkv = taps->qkv;
        if (taps->attn) b.attn = taps->attn;
        if (taps->aq) b.aq = taps->aq;
        if (taps->ad) b.ad = taps->ad;
        if (taps->x1) b.x1 = taps->x1;
        if (taps->nq) b.nq = taps->nq;
        if (taps->nd) b.nd = taps->nd;
        if (taps->gu) b.gu = taps->gu;
        if (taps->hq) b.hq = taps->hq;
        if (taps->hd) b.hd = taps->hd;
    }
    return b;
}

bool weight_is(const lq_q8_weight& w, int64_t rows, int64_t cols) { return w.rows == rows && w.cols == cols; }

lq_status validate(const lq_layer_desc* L, const float* x, int64_t pos) {
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
    if (!weight_is(L->w_qkv, nq * hd + 2 * nkv * hd, H) || !weight_is(L->w_o, H, nq * hd))
        return fail(LQ_ERR_SHAPE, "%s: w_qkv must be [%lld, %lld] and w_o [%lld, %lld]", fn,
                    (long long)(nq * hd + 2 * nkv * hd), (long long)H, (long long)H, (long long)(nq * hd));
    if (L->kind == LQ_LAYER_PRENORM_FFN) {
        const int64_t I = L->ffn;
        if (I <= 0 || I % 32 || !weight_is(L->w_gate_up, 2 * I, H) || !weight_is(L->w_down, H, I))
            return fail(LQ_ERR_SHAPE, "%s: ffn=%lld with w_gate_up [2*ffn, hidden] and w_down [hidden, ffn]", fn,
                        (long long)I);
    }
    if (hd > 512 || !attn_supported(nq, nkv, hd, L->kv_dtype))
        return fail(LQ_ERR_UNSUPPORTED, "%s: head_dim=%lld G=%lld kv_dtype=%d not built", fn, (long long)hd,
                    (long long)(nq / nkv), L->kv_dtype);
    lq_status st;
    if ((st = check_weight(&L->w_qkv, fn)) != LQ_OK) return st;
    if ((st = check_weight(&L->w_o, fn)) != LQ_OK) return st;
    if (L->kind == LQ_LAYER_PRENORM_FFN) {
        if ((st = check_weight(&L->w_gate_up, fn)) != LQ_OK) return st;
        if ((st = check_weight(&L->w_down, fn)) != LQ_OK) return st;
        if (!L->g_post) return fail(LQ_ERR_NULL, "%s: g_post is NULL", fn);
    }
    if (!x || !L->g_in || !L->k_cache || !L->v_cache || !L->rope_cos || !L->rope_sin)
        return fail(LQ_ERR_NULL, "%s: NULL pointer (x, g_in, caches and RoPE tables are required)", fn);
    if (L->qk_norm && (!L->g_q || !L->g_k)) return fail(LQ_ERR_NULL, "%s: qk_norm needs g_q and g_k", fn);
    if (!aligned(x, 16) || !aligned(L->g_in, 16) || (L->g_post && !aligned(L->g_post, 16)) ||
        !aligned(L->k_cache, 16) || !aligned(L->v_cache, 16))
        return fail(LQ_ERR_ALIGN, "%s: x, norm weights and caches must be 16-byte aligned", fn);
    const size_t es = L->kv_dtype == LQ_KV_F32 ? 4 : 2;
    if ((hd * es) % 16) return fail(LQ_ERR_ALIGN, "%s: cache rows must be a multiple of 16 bytes", fn);
    return LQ_OK;
}

}  // namespace
}  // namespace lq

using namespace lq;

extern "C" size_t lq_decode_layer_workspace_size(const lq_layer_desc* L) {
    if (!L || L->hidden <= 0 || L->n_q <= 0 || L->n_kv <= 0 || L->head_dim <= 0 || L->max_ctx <= 0) return 0;
    return layout(L, nullptr, nullptr).total;
}

extern "C" lq_status lq_decode_layer(const lq_layer_desc* L, float* x, int64_t pos, const lq_layer_taps* taps,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    lq_status st = validate(L, x, pos);
    if (st != LQ_OK) return st;
    const size_t need = layout(L, nullptr, nullptr).total;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(LQ_ERR_WORKSPACE, "lq_decode_layer: workspace needs %zu bytes (256-byte aligned), got %zu", need,
                    workspace_bytes);
    const LayerBuffers b = layout(L, static_cast<char*>(workspace), taps);
    hipStream_t s = as_stream(stream);
    const int64_t H = L->hidden, nq = L->n_q, nkv = L->n_kv, hd = L->head_dim, qd = nq * hd;
    const int64_t head_stride = L->max_ctx * hd, pos_stride = hd;
    int64_t start = 0;
    if (L->window > 0 && pos - L->window + 1 > 0) start = pos - L->window + 1;
    const int64_t len = pos - start + 1;

    // attention block
    if ((st = launch_rmsnorm_q8(x, 1, H, L->g_in, L->eps, b.xq, b.xd, s)) != LQ_OK) return st;
    if ((st = launch_q8_matvec(L->w_qkv.qs, L->w_qkv.d, L->w_qkv.rows, H, b.xq, b.xd, nullptr, b.qkv, nullptr, s)) !=
        LQ_OK)
        return st;
    if ((st = launch_qkv_post(b.qkv, nq, nkv, hd, L->g_q, L->g_k, L->qk_norm, L->v_unit_norm, L->eps, L->rope_cos,
                              L->rope_sin, pos, L->k_cache, L->v_cache, L->kv_dtype, head_stride, pos_stride, s)) !=
        LQ_OK)
        return st;
    if ((st = launch_attention(b.qkv, nq, nkv, hd, L->k_cache, L->v_cache, L->kv_dtype, head_stride, pos_stride,
                               start, len, L->attn_scale, b.attn, b.attn_ws, s)) != LQ_OK)
        return st;
    if ((st = launch_q8_quantize(b.attn, qd / 32, b.aq, b.ad, s)) != LQ_OK) return st;
    if (L->kind == LQ_LAYER_ATTN_POSTNORM) {
        // o (into the x1 buffer) -> post-attention norm -> + x
        if ((st = launch_q8_matvec(L->w_o.qs, L->w_o.d, H, qd, b.aq, b.ad, nullptr, b.x1, nullptr, s)) != LQ_OK)
            return st;
        return launch_rmsnorm_add(b.x1, H, L->g_post, L->eps, x, x, s);
    }
    if ((st = launch_q8_matvec(L->w_o.qs, L->w_o.d, H, qd, b.aq, b.ad, x, b.x1, nullptr, s)) != LQ_OK) return st;
    // FFN block
    const int64_t I = L->ffn;
    if ((st = launch_rmsnorm_q8(b.x1, 1, H, L->g_post, L->eps, b.nq, b.nd, s)) != LQ_OK) return st;
    if ((st = launch_q8_matvec(L->w_gate_up.qs, L->w_gate_up.d, 2 * I, H, b.nq, b.nd, nullptr, b.gu, nullptr, s)) !=
        LQ_OK)
        return st;
    if ((st = launch_swiglu_q8(b.gu, 1, I, b.hq, b.hd, s)) != LQ_OK) return st;
    return launch_q8_matvec(L->w_down.qs, L->w_down.d, H, I, b.hq, b.hd, b.x1, x, nullptr, s);
}

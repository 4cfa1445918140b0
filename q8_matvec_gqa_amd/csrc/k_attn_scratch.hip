// k_attn_scratch.hip -- GQA decode attention for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): lq_gqa_decode_attn with the split partials kept in a
// file-scope device array instead of a caller workspace.
//
// The array lives in the code object, so each GPU the library runs on holds
// its own copy at its own address from module load until the process ends.
// The host-side `scratch` is only a stand-in for that array: its device
// address comes from hipGetSymbolAddress, once per device with that device
// current, and only that address is handed to kernels.  Every call on a GPU
// shares the GPU's array: calls that overlap on one GPU (two streams, two
// host threads) race on it.  The split kernel writes every partial the
// combine kernel reads, so no call depends on what a previous call left
// there and nothing needs clearing.
#include <mutex>

#include "lq_internal.h"

namespace lq {
namespace {

// 16 MiB per device.  The partials of every shape with up to 510 kv heads
// fit (head_dim <= 512, up to 8 query heads per kv head, any length); the
// largest plans (511 kv heads with head_dim 512 and 8 query heads each, 16.8
// MB) are refused.  Shapes of more kv heads need no partials (one split).
constexpr size_t kAttnScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kAttnScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void* ptr = nullptr;
};
ScratchSlot g_slots[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call there).
lq_status scratch_address(const char* fn, void** out) {
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LQ_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(LQ_ERR_UNSUPPORTED, "%s: device %d >= %d", fn, dev, kMaxDevices);
    ScratchSlot& s = g_slots[dev];
    std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
    if (s.err != hipSuccess || !s.ptr)
        return fail(LQ_ERR_HIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev,
                    hipGetErrorString(s.err));
    *out = s.ptr;
    return LQ_OK;
}

}  // namespace
}  // namespace lq

using namespace lq;

extern "C" lq_status lq_gqa_decode_attn_noalloc(const float* q, int64_t n_q, int64_t n_kv, int64_t head_dim,
                                                const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                                int64_t head_stride, int64_t pos_stride, int64_t max_ctx,
                                                int64_t start, int64_t len, float scale, float* out,
                                                void* stream) {
    const char* fn = "lq_gqa_decode_attn_noalloc";
    lq_status st = check_attention_args(fn, q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride,
                                        pos_stride, max_ctx, start, len, out);
    if (st != LQ_OK || n_q == 0) return st;
    const size_t need = attn_workspace_bytes(n_q, n_kv, head_dim, len);
    if (need > kAttnScratchBytes)
        return fail(LQ_ERR_UNSUPPORTED, "%s: this shape needs %zu bytes of split partials; the library's scratch "
                    "array holds %zu (use lq_gqa_decode_attn with a workspace)", fn, need, kAttnScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_address(fn, &ws)) != LQ_OK) return st;
    return launch_attention(q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride, start,
                            len, scale, out, ws, as_stream(stream));
}

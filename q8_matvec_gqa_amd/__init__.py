"""Python binding of liblq (include/lq.h): argument marshalling only.

Every function has the name of its C entry point and takes the same
arguments in the same order.  Device buffers may be passed as torch tensors
(their data_ptr() is used) or as raw integer addresses; `stream` defaults to
torch's current stream.  A nonzero lq_status raises LqError carrying the
status and lq_last_error().  No computation happens here: every step of the
path runs in the HIP kernels of liblq.so, and importing this package fails
loudly when that library has not been built.
"""
import ctypes as C
import os

# PyTorch carries its own HIP runtime (libamdhip64.so.7).  Loading it first
# makes liblq.so bind to that same runtime, so the process has one HIP/HSA
# runtime and torch's device pointers and streams are valid in liblq.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()' or python q8_matvec_gqa_amd/build.py)")

_lib = C.CDLL(LIB_PATH)

LQ_OK, LQ_ERR_NULL, LQ_ERR_SHAPE, LQ_ERR_ALIGN, LQ_ERR_WORKSPACE, LQ_ERR_HIP, LQ_ERR_UNSUPPORTED = range(7)
LQ_KV_F32, LQ_KV_BF16 = 0, 1
LQ_LAYER_PRENORM_FFN, LQ_LAYER_ATTN_POSTNORM = 0, 1
LQ_ACT_SILU, LQ_ACT_GELU_TANH = 0, 1

_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_F = C.c_float
_SZ = C.c_size_t


class LqError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"lq status {status} ({lq_status_string(status)}): {msg}")
        self.status = status


class lq_q8_weight(C.Structure):
    _fields_ = [("qs", _P), ("d", _P), ("rows", _I64), ("cols", _I64)]


class lq_q4_0_weight(C.Structure):
    _fields_ = [("qs", _P), ("d", _P), ("rows", _I64), ("cols", _I64)]


class lq_q6_k_weight(C.Structure):
    _fields_ = [("ql", _P), ("qh", _P), ("sc", _P), ("d", _P), ("rows", _I64), ("cols", _I64)]


class lq_moe_desc(C.Structure):
    _fields_ = [("hidden", _I64), ("ffn", _I64), ("n_experts", _I64), ("top_k", _I64),
                ("w_gate_up", lq_q8_weight), ("w_down", lq_q8_weight), ("expert_scale", _P)]


class lq_moe_taps(C.Structure):
    _fields_ = [(n, _P) for n in ("ids", "w", "xq", "xd", "y1", "hq", "hd", "y2")]


LQ_FMT_Q8_0, LQ_FMT_Q4_0, LQ_FMT_Q6_K = 0, 1, 2


class lq_moe_ggml_desc(C.Structure):
    _fields_ = [("hidden", _I64), ("ffn", _I64), ("n_experts", _I64), ("top_k", _I64),
                ("gate_up_format", _I32), ("down_format", _I32),
                ("gate_up_q4_0", lq_q4_0_weight), ("gate_up_q6_k", lq_q6_k_weight),
                ("down_q4_0", lq_q4_0_weight), ("down_q6_k", lq_q6_k_weight), ("expert_scale", _P)]


class lq_layer_desc(C.Structure):
    _fields_ = [
        ("hidden", _I64), ("n_q", _I64), ("n_kv", _I64), ("head_dim", _I64), ("ffn", _I64),
        ("max_ctx", _I64), ("window", _I64), ("eps", _F), ("attn_scale", _F),
        ("kind", _I32), ("kv_dtype", _I32), ("qk_norm", _I32), ("v_unit_norm", _I32),
        ("w_qkv", lq_q8_weight), ("w_o", lq_q8_weight), ("w_gate_up", lq_q8_weight),
        ("w_down", lq_q8_weight),
        ("g_in", _P), ("g_q", _P), ("g_k", _P), ("g_post", _P),
        ("k_cache", _P), ("v_cache", _P), ("rope_cos", _P), ("rope_sin", _P),
        ("ffn_act", _I32), ("attn_softcap", _F),
        ("w_format", _I32 * 4), ("w_q4_0", lq_q4_0_weight * 4), ("w_q6_k", lq_q6_k_weight * 4),
    ]


class lq_layer_taps(C.Structure):
    _fields_ = [(n, _P) for n in ("xq", "xd", "qkv", "attn", "aq", "ad", "x1", "nq", "nd", "h", "hq", "hd",
                                  "qkv_post")]


_W = C.POINTER(lq_q8_weight)
_SIGS = {
    "lq_version": (_I32, []),
    "lq_status_string": (C.c_char_p, [_I32]),
    "lq_last_error": (C.c_char_p, []),
    "lq_q8_pack_ggml": (_I32, [_P, _I64, _I64, _P, _P]),
    "lq_q4_0_pack_ggml": (_I32, [_P, _I64, _I64, _P, _P]),
    "lq_q6_k_pack_ggml": (_I32, [_P, _I64, _I64, _P, _P, _P, _P]),
    "lq_rope_table": (_I32, [_I64, _I64, C.c_double, _P, _P]),
    "lq_q8_quantize_act": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "lq_rmsnorm_q8": (_I32, [_P, _I64, _I64, _P, _F, _P, _P, _P]),
    "lq_swiglu_q8": (_I32, [_P, _I64, _I64, _P, _P, _P]),
    "lq_q8_matvec": (_I32, [_W, _P, _P, _P, _P, _P]),
    "lq_q4_0_matvec": (_I32, [C.POINTER(lq_q4_0_weight), _P, _P, _P, _P, _P]),
    "lq_q6_k_matvec": (_I32, [C.POINTER(lq_q6_k_weight), _P, _P, _P, _P, _P]),
    "lq_q8_block_dots": (_I32, [_W, _P, _P, _P]),
    "lq_q8_block_dots_f32": (_I32, [_W, _P, _I32, _P, _F, _P, _P, _P, _P]),
    "lq_rmsnorm_rope": (_I32, [_P, _I64, _I64, _I64, _P, _F, _P, _P, _I64, _I64, _P]),
    "lq_kv_append": (_I32, [_P, _P, _I64, _I64, _P, _P, _I32, _I64, _I64, _I64, _I64, _P]),
    "lq_gqa_decode_attn_workspace_size": (_SZ, [_I64, _I64, _I64, _I64]),
    "lq_gqa_decode_attn": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _I64, _I64, _I64, _I64, _I64,
                                  _F, _P, _P, _SZ, _P]),
    "lq_gqa_decode_attn_noalloc": (_I32, [_P, _I64, _I64, _I64, _P, _P, _I32, _I64, _I64, _I64, _I64, _I64,
                                          _F, _P, _P]),
    "lq_rope_table_freqs": (_I32, [_I64, _I64, C.c_double, _P, _P, _P]),
    "lq_q8_matmul_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "lq_q8_matmul": (_I32, [_W, _P, _P, _I64, _P, _P, _P, _SZ, _P]),
    "lq_lm_head_f16": (_I32, [_P, _I64, _I64, _P, _I32, _P, C.c_float, C.c_float, _P, _P]),
    "lq_moe_route_topk": (_I32, [_P, _I64, _I64, _I64, _P, _P, _P]),
    "lq_moe_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "lq_moe_q8_matvec_id": (_I32, [_W, _I64, _P, _P, _I32, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "lq_moe_q4_0_matvec_id": (_I32, [C.POINTER(lq_q4_0_weight), _I64, _P, _P, _I32, _P, _I64, _I64, _P, _P, _SZ,
                                      _P]),
    "lq_moe_q6_k_matvec_id": (_I32, [C.POINTER(lq_q6_k_weight), _I64, _P, _P, _I32, _P, _I64, _I64, _P, _P, _SZ,
                                      _P]),
    "lq_moe_weighted_sum": (_I32, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "lq_moe_block_ggml_workspace_size": (_SZ, [C.POINTER(lq_moe_ggml_desc), _I64]),
    "lq_moe_block_ggml": (_I32, [C.POINTER(lq_moe_ggml_desc), _P, _P, _I64, _P, C.POINTER(lq_moe_taps), _P, _SZ,
                                 _P]),
    "lq_moe_block_workspace_size": (_SZ, [C.POINTER(lq_moe_desc), _I64]),
    "lq_moe_block": (_I32, [C.POINTER(lq_moe_desc), _P, _P, _I64, _P, C.POINTER(lq_moe_taps), _P, _SZ,
                            _P]),
    "lq_decode_layer_workspace_size": (_SZ, [C.POINTER(lq_layer_desc)]),
    "lq_decode_layer": (_I32, [C.POINTER(lq_layer_desc), _P, _I64, C.POINTER(lq_layer_taps), _P, _SZ,
                               _P]),
    "lq_decode_layer_kernel_count": (_I32, [C.POINTER(lq_layer_desc)]),
    "lq_decode_layer_timed": (_I32, [C.POINTER(lq_layer_desc), _P, _I64, C.POINTER(lq_layer_taps), _P, _SZ,
                                     C.POINTER(_P), _I32, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def exported_names():
    return list(_SIGS)


def _ptr(a):
    """Device or host address of a tensor / integer / None."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    if hasattr(a, "ctypes"):          # numpy array (host helpers)
        return a.ctypes.data
    raise TypeError(f"cannot take the address of {type(a)}")


def _stream(s):
    if s is not None:
        return s if isinstance(s, int) else s.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ref(s):
    return None if s is None else C.byref(s)


def _check(status, check=True):
    if status != LQ_OK and check:
        raise LqError(status, lq_last_error())
    return status


# ---------------------------------------------------------------- misc
def lq_version():
    return _lib.lq_version()


def lq_status_string(s):
    return _lib.lq_status_string(s).decode()


def lq_last_error():
    return _lib.lq_last_error().decode()


def q8_weight(qs, d, rows=None, cols=None):
    """lq_q8_weight for codes `qs` [rows, cols] and scales `d` [rows, cols/32]
    (tensors or addresses; rows/cols taken from qs.shape when omitted)."""
    if rows is None:
        rows, cols = qs.shape[-2], qs.shape[-1]
    w = lq_q8_weight(_ptr(qs), _ptr(d), rows, cols)
    w._keep = (qs, d)     # the struct holds raw addresses: keep the buffers alive with it
    return w


def lq_q8_pack_ggml(blocks, rows, cols, qs, d, check=True):
    return _check(_lib.lq_q8_pack_ggml(_ptr(blocks), rows, cols, _ptr(qs), _ptr(d)), check)


def lq_q4_0_pack_ggml(blocks, rows, cols, qs, d, check=True):
    return _check(_lib.lq_q4_0_pack_ggml(_ptr(blocks), rows, cols, _ptr(qs), _ptr(d)), check)


def lq_q6_k_pack_ggml(blocks, rows, cols, ql, qh, sc, d, check=True):
    return _check(_lib.lq_q6_k_pack_ggml(_ptr(blocks), rows, cols, _ptr(ql), _ptr(qh), _ptr(sc), _ptr(d)), check)


def q4_0_weight(qs, d, rows, cols):
    """lq_q4_0_weight over device arrays qs [rows, cols/2] and d [rows, cols/32]."""
    w = lq_q4_0_weight(_ptr(qs), _ptr(d), rows, cols)
    w._keep = (qs, d)
    return w


def q6_k_weight(ql, qh, sc, d, rows, cols):
    """lq_q6_k_weight over device arrays ql, qh, sc and d (see include/lq.h)."""
    w = lq_q6_k_weight(_ptr(ql), _ptr(qh), _ptr(sc), _ptr(d), rows, cols)
    w._keep = (ql, qh, sc, d)
    return w


def lq_rope_table(max_ctx, head_dim, theta, cos_out, sin_out, check=True):
    return _check(_lib.lq_rope_table(max_ctx, head_dim, theta, _ptr(cos_out), _ptr(sin_out)), check)


def lq_rope_table_freqs(max_ctx, head_dim, theta, freq_factors, cos_out, sin_out, check=True):
    return _check(_lib.lq_rope_table_freqs(max_ctx, head_dim, theta, _ptr(freq_factors), _ptr(cos_out),
                                           _ptr(sin_out)), check)


# ---------------------------------------------------------------- Q8_0
def lq_q8_quantize_act(x, n_rows, n, qs, d, stream=None, check=True):
    return _check(_lib.lq_q8_quantize_act(_ptr(x), n_rows, n, _ptr(qs), _ptr(d), _stream(stream)), check)


def lq_rmsnorm_q8(x, n_rows, n, gamma, eps, qs, d, stream=None, check=True):
    return _check(_lib.lq_rmsnorm_q8(_ptr(x), n_rows, n, _ptr(gamma), eps, _ptr(qs), _ptr(d),
                                     _stream(stream)), check)


def lq_swiglu_q8(gate_up, n_rows, ffn, qs, d, stream=None, check=True):
    return _check(_lib.lq_swiglu_q8(_ptr(gate_up), n_rows, ffn, _ptr(qs), _ptr(d), _stream(stream)), check)


def lq_q8_matvec(w, x_qs, x_d, residual, y, stream=None, check=True):
    return _check(_lib.lq_q8_matvec(_ref(w), _ptr(x_qs), _ptr(x_d), _ptr(residual), _ptr(y),
                                    _stream(stream)), check)


def lq_q4_0_matvec(w, x_qs, x_d, residual, y, stream=None, check=True):
    return _check(_lib.lq_q4_0_matvec(_ref(w), _ptr(x_qs), _ptr(x_d), _ptr(residual), _ptr(y), _stream(stream)),
                  check)


def lq_q6_k_matvec(w, x_qs, x_d, residual, y, stream=None, check=True):
    return _check(_lib.lq_q6_k_matvec(_ref(w), _ptr(x_qs), _ptr(x_d), _ptr(residual), _ptr(y), _stream(stream)),
                  check)


def lq_q8_block_dots(w, x_qs, dots, stream=None, check=True):
    return _check(_lib.lq_q8_block_dots(_ref(w), _ptr(x_qs), _ptr(dots), _stream(stream)), check)


def lq_q8_block_dots_f32(w, x, norm, gamma, eps, dots, x_qs_out, x_d_out, stream=None, check=True):
    return _check(_lib.lq_q8_block_dots_f32(_ref(w), _ptr(x), int(norm), _ptr(gamma), eps, _ptr(dots),
                                            _ptr(x_qs_out), _ptr(x_d_out), _stream(stream)), check)


# ---------------------------------------------------------------- norm / RoPE / KV
def lq_rmsnorm_rope(x, n_heads, head_dim, head_stride, gamma, eps, rope_cos, rope_sin, rope_len, pos,
                    stream=None, check=True):
    return _check(_lib.lq_rmsnorm_rope(_ptr(x), n_heads, head_dim, head_stride, _ptr(gamma), eps,
                                       _ptr(rope_cos), _ptr(rope_sin), rope_len, pos, _stream(stream)), check)


def lq_kv_append(k, v, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride, max_ctx, pos,
                 stream=None, check=True):
    return _check(_lib.lq_kv_append(_ptr(k), _ptr(v), n_kv, head_dim, _ptr(k_cache), _ptr(v_cache),
                                    kv_dtype, head_stride, pos_stride, max_ctx, pos, _stream(stream)), check)


# ---------------------------------------------------------------- attention
def lq_gqa_decode_attn_workspace_size(n_q, n_kv, head_dim, length):
    return _lib.lq_gqa_decode_attn_workspace_size(n_q, n_kv, head_dim, length)


def lq_gqa_decode_attn(q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride,
                       max_ctx, start, length, scale, out, workspace, workspace_bytes, stream=None,
                       check=True):
    return _check(_lib.lq_gqa_decode_attn(_ptr(q), n_q, n_kv, head_dim, _ptr(k_cache), _ptr(v_cache),
                                          kv_dtype, head_stride, pos_stride, max_ctx, start, length,
                                          scale, _ptr(out), _ptr(workspace), workspace_bytes,
                                          _stream(stream)), check)


def lq_gqa_decode_attn_noalloc(q, n_q, n_kv, head_dim, k_cache, v_cache, kv_dtype, head_stride, pos_stride,
                               max_ctx, start, length, scale, out, stream=None, check=True):
    return _check(_lib.lq_gqa_decode_attn_noalloc(_ptr(q), n_q, n_kv, head_dim, _ptr(k_cache), _ptr(v_cache),
                                                  kv_dtype, head_stride, pos_stride, max_ctx, start, length,
                                                  scale, _ptr(out), _stream(stream)), check)


# ---------------------------------------------------------------- MoE
def lq_q8_matmul_workspace_size(rows, cols, T):
    return _lib.lq_q8_matmul_workspace_size(rows, cols, T)


def lq_q8_matmul(w, x_qs, x_d, T, residual, y, workspace, workspace_bytes, stream=None, check=True):
    return _check(_lib.lq_q8_matmul(_ref(w), _ptr(x_qs), _ptr(x_d), T, _ptr(residual), _ptr(y), _ptr(workspace),
                                    workspace_bytes, _stream(stream)), check)


def lq_lm_head_f16(w, vocab, hidden, x, norm, gamma, eps, softcap, logits, stream=None, check=True):
    return _check(_lib.lq_lm_head_f16(_ptr(w), vocab, hidden, _ptr(x), int(norm), _ptr(gamma), eps, softcap,
                                      _ptr(logits), _stream(stream)), check)


def lq_moe_route_topk(logits, T, E, k, ids, w, stream=None, check=True):
    return _check(_lib.lq_moe_route_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream(stream)), check)


def lq_moe_workspace_size(T, k, n_experts):
    return _lib.lq_moe_workspace_size(T, k, n_experts)


def lq_moe_q8_matvec_id(w, n_experts, x_qs, x_d, x_per_slot, ids, T, k, y, workspace, workspace_bytes,
                        stream=None, check=True):
    return _check(_lib.lq_moe_q8_matvec_id(_ref(w), n_experts, _ptr(x_qs), _ptr(x_d), x_per_slot, _ptr(ids),
                                           T, k, _ptr(y), _ptr(workspace), workspace_bytes,
                                           _stream(stream)), check)


def lq_moe_q4_0_matvec_id(w, n_experts, x_qs, x_d, x_per_slot, ids, T, k, y, workspace, workspace_bytes,
                          stream=None, check=True):
    return _check(_lib.lq_moe_q4_0_matvec_id(_ref(w), n_experts, _ptr(x_qs), _ptr(x_d), x_per_slot, _ptr(ids), T, k,
                                             _ptr(y), _ptr(workspace), workspace_bytes, _stream(stream)), check)


def lq_moe_q6_k_matvec_id(w, n_experts, x_qs, x_d, x_per_slot, ids, T, k, y, workspace, workspace_bytes,
                          stream=None, check=True):
    return _check(_lib.lq_moe_q6_k_matvec_id(_ref(w), n_experts, _ptr(x_qs), _ptr(x_d), x_per_slot, _ptr(ids), T, k,
                                             _ptr(y), _ptr(workspace), workspace_bytes, _stream(stream)), check)


def lq_moe_weighted_sum(y, w, T, k, rows, out, stream=None, check=True):
    return _check(_lib.lq_moe_weighted_sum(_ptr(y), _ptr(w), T, k, rows, _ptr(out), _stream(stream)), check)


def lq_moe_block_workspace_size(desc, T):
    return _lib.lq_moe_block_workspace_size(_ref(desc), T)


def lq_moe_block(desc, x, logits, T, out, taps, workspace, workspace_bytes, stream=None, check=True):
    return _check(_lib.lq_moe_block(_ref(desc), _ptr(x), _ptr(logits), T, _ptr(out), _ref(taps),
                                    _ptr(workspace), workspace_bytes, _stream(stream)), check)


def lq_moe_block_ggml_workspace_size(desc, T):
    return _lib.lq_moe_block_ggml_workspace_size(_ref(desc), T)


def lq_moe_block_ggml(desc, x, logits, T, out, taps, workspace, workspace_bytes, stream=None, check=True):
    return _check(_lib.lq_moe_block_ggml(_ref(desc), _ptr(x), _ptr(logits), T, _ptr(out), _ref(taps),
                                         _ptr(workspace), workspace_bytes, _stream(stream)), check)


# ---------------------------------------------------------------- layer
def lq_decode_layer_workspace_size(desc):
    return _lib.lq_decode_layer_workspace_size(_ref(desc))


def lq_decode_layer(desc, x, pos, taps, workspace, workspace_bytes, stream=None, check=True):
    return _check(_lib.lq_decode_layer(_ref(desc), _ptr(x), pos, _ref(taps), _ptr(workspace),
                                       workspace_bytes, _stream(stream)), check)


def lq_decode_layer_kernel_count(desc):
    return _lib.lq_decode_layer_kernel_count(_ref(desc))


def lq_decode_layer_timed(desc, x, pos, taps, workspace, workspace_bytes, events, stream=None, check=True):
    """events: list of torch.cuda.Event (created with enable_timing) or raw hipEvent_t addresses."""
    handles = [e if isinstance(e, int) else e.cuda_event for e in events]
    arr = (_P * len(handles))(*handles)
    return _check(_lib.lq_decode_layer_timed(_ref(desc), _ptr(x), pos, _ref(taps), _ptr(workspace),
                                             workspace_bytes, arr, len(handles), _stream(stream)), check)

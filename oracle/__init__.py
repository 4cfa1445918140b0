"""ctypes binding of the CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The GPU product path never imports this
package.  All arrays are numpy, C-contiguous; f16/bf16 travel as uint16 bit
patterns.
"""
import contextlib
import ctypes as C
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_D = C.c_double


class OrcLayer(C.Structure):
    _fields_ = [
        ("hidden", _I64), ("n_q", _I64), ("n_kv", _I64), ("head_dim", _I64), ("ffn", _I64),
        ("max_ctx", _I64), ("window", _I64),
        ("eps", _D), ("attn_scale", _D),
        ("kv_dtype", _I32), ("kind", _I32), ("qk_norm", _I32), ("v_unit_norm", _I32),
        ("qkv_qs", _P), ("qkv_d", _P), ("o_qs", _P), ("o_d", _P),
        ("gu_qs", _P), ("gu_d", _P), ("dn_qs", _P), ("dn_d", _P),
        ("g_in", _P), ("g_q", _P), ("g_k", _P), ("g_post", _P),
        ("k_cache", _P), ("v_cache", _P), ("rope_cos", _P), ("rope_sin", _P),
        ("ffn_act", _I32), ("attn_softcap", _D),
    ]


class OrcLayerTrace(C.Structure):
    _fields_ = [(n, _P) for n in (
        "xq", "xd", "qkv", "q", "k", "v", "attn", "aq", "ad", "x1", "nq", "nd", "gu", "hq", "hd")]


class OrcMoe(C.Structure):
    _fields_ = [
        ("hidden", _I64), ("ffn", _I64), ("n_experts", _I64), ("top_k", _I64), ("tokens", _I64),
        ("gu_qs", _P), ("gu_d", _P), ("dn_qs", _P), ("dn_d", _P), ("expert_scale", _P),
    ]


class OrcMoeTrace(C.Structure):
    _fields_ = [(n, _P) for n in ("ids", "w", "xq", "xd", "y1", "hq", "hd", "y2")]


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        src = os.path.join(_HERE, "oracle.c")
        if (not os.path.exists(path)) or os.path.getmtime(path) < os.path.getmtime(src):
            _build.build()
        _lib = _load(path)
    return _lib


@contextlib.contextmanager
def using(path):
    """Temporarily route every call to another build of the oracle (used by
    the tests that plant mistakes in copies of oracle.c)."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _load(path):
    L = C.CDLL(path)
    L.orc_f32_to_f16.restype = C.c_uint16
    L.orc_f32_to_f16.argtypes = [C.c_float]
    L.orc_f16_to_f32.restype = C.c_float
    L.orc_f16_to_f32.argtypes = [C.c_uint16]
    L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_f32_to_bf16.argtypes = [C.c_float]
    L.orc_bf16_to_f32.restype = C.c_float
    L.orc_bf16_to_f32.argtypes = [C.c_uint16]
    L.orc_q8_quantize.argtypes = [_P, _I64, _P, _P]
    L.orc_q8_block_dots.argtypes = [_P, _I64, _I64, _P, _P]
    L.orc_q8_matvec.argtypes = [_P, _P, _I64, _I64, _P, _P, _P, _P]
    L.orc_q8_matmul.argtypes = [_P, _P, _I64, _I64, _P, _P, _I64, _P, _P]
    L.orc_q4_0_dequant.argtypes = [_P, _I64, _P]
    L.orc_q6_k_dequant.argtypes = [_P, _I64, _P]
    L.orc_q4_0_matvec.argtypes = [_P, _I64, _I64, _P, _P, _P, _P]
    L.orc_q6_k_matvec.argtypes = [_P, _I64, _I64, _P, _P, _P, _P]
    L.orc_rmsnorm.argtypes = [_P, _I64, _P, _D, _P]
    L.orc_rope_table.argtypes = [_I64, _I64, _D, _P, _P]
    L.orc_rope_table_freqs.argtypes = [_I64, _I64, _D, _P, _P, _P]
    L.orc_rope_neox.argtypes = [_P, _I64, _P, _P]
    L.orc_silu_mul.argtypes = [_P, _P, _I64, _P]
    L.orc_gelu_mul.argtypes = [_P, _P, _I64, _P]
    L.orc_attention.argtypes = [_P, _I64, _I64, _I64, _P, _P, _I32, _I64, _I64,
                                _I64, _I64, _D, _D, _P]
    L.orc_lm_head.argtypes = [_P, _I64, _I64, _P, _I32, _P, _D, _D, _P]
    L.orc_moe_route.argtypes = [_P, _I64, _I64, _I64, _P, _P]
    L.orc_moe_block.argtypes = [C.POINTER(OrcMoe), _P, _P, _P, C.POINTER(OrcMoeTrace)]
    L.orc_decode_layer.argtypes = [C.POINTER(OrcLayer), _P, _I64, C.POINTER(OrcLayerTrace)]
    return L


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def f32_to_f16(x):
    x = np.asarray(x, dtype=np.float32).ravel()
    f = lib().orc_f32_to_f16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def f16_to_f32(h):
    h = np.asarray(h, dtype=np.uint16).ravel()
    f = lib().orc_f16_to_f32
    return np.array([f(int(v)) for v in h], dtype=np.float32)


def f32_to_bf16(x):
    x = np.asarray(x, dtype=np.float32).ravel()
    f = lib().orc_f32_to_bf16
    return np.array([f(float(v)) for v in x], dtype=np.uint16)


def bf16_to_f32(b):
    b = np.asarray(b, dtype=np.uint16).ravel()
    f = lib().orc_bf16_to_f32
    return np.array([f(int(v)) for v in b], dtype=np.float32)


# ---------------------------------------------------------------- Q8_0
def q8_quantize(x):
    """x: float32 [..., n] (n % 32 == 0) -> (codes int8 [..., n], scales uint16 [..., n/32])."""
    x = _c(x, np.float32)
    n = x.size
    qs = np.empty(x.shape, dtype=np.int8)
    d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=np.uint16)
    lib().orc_q8_quantize(_ptr(x), n, _ptr(qs), _ptr(d))
    return qs, d


def q8_block_dots(wq, xq):
    wq = _c(wq, np.int8)
    xq = _c(xq, np.int8)
    rows, cols = wq.shape
    out = np.empty((rows, cols // 32), dtype=np.int32)
    lib().orc_q8_block_dots(_ptr(wq), rows, cols, _ptr(xq), _ptr(out))
    return out


def q8_matvec(wq, wd, xq, xd, residual=None):
    wq = _c(wq, np.int8)
    wd = _c(wd, np.uint16)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.uint16)
    rows, cols = wq.shape
    res = None if residual is None else _c(residual, np.float32)
    y = np.empty(rows, dtype=np.float32)
    lib().orc_q8_matvec(_ptr(wq), _ptr(wd), rows, cols, _ptr(xq), _ptr(xd), _ptr(res), _ptr(y))
    return y


def q8_matmul(wq, wd, xq, xd, residual=None):
    """xq [T, cols] int8, xd [T, cols/32] f16 bits -> y [T, rows]."""
    wq = _c(wq, np.int8)
    wd = _c(wd, np.uint16)
    xq = _c(xq, np.int8)
    xd = _c(xd, np.uint16)
    rows, cols = wq.shape
    T = xq.shape[0]
    res = None if residual is None else _c(residual, np.float32)
    y = np.empty((T, rows), dtype=np.float32)
    lib().orc_q8_matmul(_ptr(wq), _ptr(wd), rows, cols, _ptr(xq), _ptr(xd), T, _ptr(res), _ptr(y))
    return y


# ---------------------------------------------------------------- other GGML formats
_QK = {"q4_0": (32, 18), "q6_k": (256, 210)}   # values and bytes per GGML block


def q_dequant(fmt, blocks, n):
    """GGML blocks (uint8, n values' worth) -> float64 values."""
    per, nbytes = _QK[fmt]
    blocks = _c(blocks, np.uint8)
    assert n % per == 0 and blocks.size == n // per * nbytes
    w = np.empty(n, dtype=np.float64)
    getattr(lib(), f"orc_{fmt}_dequant")(_ptr(blocks), n, _ptr(w))
    return w


def q_matvec(fmt, blocks, rows, cols, xq, xd, residual=None):
    """Q4_0 / Q6_K weight (GGML blocks, row-major) times a Q8_0 activation."""
    per, nbytes = _QK[fmt]
    blocks = _c(blocks, np.uint8)
    assert cols % per == 0 and blocks.size == rows * (cols // per) * nbytes
    xq = _c(xq, np.int8)
    xd = _c(xd, np.uint16)
    res = None if residual is None else _c(residual, np.float32)
    y = np.empty(rows, dtype=np.float32)
    getattr(lib(), f"orc_{fmt}_matvec")(_ptr(blocks), rows, cols, _ptr(xq), _ptr(xd), _ptr(res), _ptr(y))
    return y


# ---------------------------------------------------------------- norms etc.
def rmsnorm(x, gamma=None, eps=1e-6):
    x = _c(x, np.float32)
    g = None if gamma is None else _c(gamma, np.float32)
    y = np.empty_like(x)
    lib().orc_rmsnorm(_ptr(x), x.size, _ptr(g), float(eps), _ptr(y))
    return y


def lm_head(w, x, gamma=None, norm=True, eps=1e-6, cap=0.0):
    """w: uint16 f16 bits [vocab, hidden]; returns f32 logits [vocab]."""
    w = _c(w, np.uint16)
    x = _c(x, np.float32)
    g = None if gamma is None else _c(gamma, np.float32)
    vocab, hidden = w.shape
    out = np.empty(vocab, dtype=np.float32)
    lib().orc_lm_head(_ptr(w), vocab, hidden, _ptr(x), int(bool(norm)), _ptr(g), float(eps), float(cap), _ptr(out))
    return out


def rope_table(max_ctx, hd, theta):
    c = np.empty((max_ctx, hd // 2), dtype=np.float32)
    s = np.empty((max_ctx, hd // 2), dtype=np.float32)
    lib().orc_rope_table(max_ctx, hd, float(theta), _ptr(c), _ptr(s))
    return c, s


def rope_table_freqs(max_ctx, hd, theta, factors):
    f = None if factors is None else _c(factors, np.float32)
    c = np.empty((max_ctx, hd // 2), dtype=np.float32)
    s = np.empty((max_ctx, hd // 2), dtype=np.float32)
    lib().orc_rope_table_freqs(max_ctx, hd, float(theta), _ptr(f), _ptr(c), _ptr(s))
    return c, s


def rope_neox(x, cos_row, sin_row):
    x = _c(x, np.float32).copy()
    lib().orc_rope_neox(_ptr(x), x.size, _ptr(_c(cos_row, np.float32)), _ptr(_c(sin_row, np.float32)))
    return x


def silu_mul(g, u):
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty_like(g)
    lib().orc_silu_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def gelu_mul(g, u):
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty_like(g)
    lib().orc_gelu_mul(_ptr(g), _ptr(u), g.size, _ptr(h))
    return h


def attention(q, n_q, n_kv, hd, k_cache, v_cache, kv_dtype, head_stride, pos_stride,
              start, length, scale, softcap=0.0):
    """kv_dtype 0: caches are float32 arrays; 1: caches are uint16 bf16 bit patterns."""
    q = _c(q, np.float32)
    kd = np.float32 if kv_dtype == 0 else np.uint16
    k_cache = _c(k_cache, kd)
    v_cache = _c(v_cache, kd)
    out = np.empty(n_q * hd, dtype=np.float32)
    lib().orc_attention(_ptr(q), n_q, n_kv, hd, _ptr(k_cache), _ptr(v_cache), kv_dtype,
                        head_stride, pos_stride, start, length, float(scale), float(softcap), _ptr(out))
    return out


# ---------------------------------------------------------------- MoE
def moe_route(logits, k):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    lib().orc_moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w))
    return ids, w


def moe_block(hidden, ffn, n_experts, top_k, gu_qs, gu_d, dn_qs, dn_d, x, logits, trace=False,
              expert_scale=None):
    x = _c(x, np.float32)
    logits = _c(logits, np.float32)
    T = x.shape[0]
    gu_qs = _c(gu_qs, np.int8); gu_d = _c(gu_d, np.uint16)
    dn_qs = _c(dn_qs, np.int8); dn_d = _c(dn_d, np.uint16)
    es = None if expert_scale is None else _c(expert_scale, np.float32)
    m = OrcMoe(hidden, ffn, n_experts, top_k, T, _ptr(gu_qs), _ptr(gu_d), _ptr(dn_qs), _ptr(dn_d), _ptr(es))
    out = np.empty((T, hidden), dtype=np.float32)
    tr = OrcMoeTrace()
    arrays = {}
    if trace:
        arrays = dict(
            ids=np.empty((T, top_k), np.int32), w=np.empty((T, top_k), np.float32),
            xq=np.empty((T, hidden), np.int8), xd=np.empty((T, hidden // 32), np.uint16),
            y1=np.empty((T, top_k, 2 * ffn), np.float32),
            hq=np.empty((T, top_k, ffn), np.int8), hd=np.empty((T, top_k, ffn // 32), np.uint16),
            y2=np.empty((T, top_k, hidden), np.float32))
        for name, a in arrays.items():
            setattr(tr, name, _ptr(a))
    lib().orc_moe_block(C.byref(m), _ptr(x), _ptr(logits), _ptr(out), C.byref(tr))
    return (out, arrays) if trace else out


# ---------------------------------------------------------------- layer
def decode_layer(cfg, w, x, pos, k_cache, v_cache, trace=False):
    """Run one decode layer in place on copies.

    cfg: dict with hidden, n_q, n_kv, head_dim, ffn, max_ctx, window, eps,
         attn_scale, kv_dtype (0/1), kind (0/1), qk_norm, v_unit_norm.
    w:   dict of numpy arrays qkv_qs, qkv_d, o_qs, o_d, gu_qs, gu_d, dn_qs,
         dn_d, g_in, g_q, g_k, g_post, rope_cos, rope_sin (missing ones None).
    Returns (x_out, k_cache_out, v_cache_out, trace_arrays).
    """
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    x = _c(x, np.float32).copy()
    kd = np.float32 if cfg["kv_dtype"] == 0 else np.uint16
    kc = _c(k_cache, kd).copy()
    vc = _c(v_cache, kd).copy()
    keep = {}

    def P(name, dtype):
        a = w.get(name)
        if a is None:
            return None
        a = _c(a, dtype)
        keep[name] = a
        return _ptr(a)

    L = OrcLayer(
        hidden=H, n_q=nq, n_kv=nkv, head_dim=hd, ffn=I,
        max_ctx=cfg["max_ctx"], window=cfg.get("window", 0),
        eps=cfg["eps"], attn_scale=cfg["attn_scale"],
        kv_dtype=cfg["kv_dtype"], kind=cfg["kind"],
        qk_norm=cfg.get("qk_norm", 1), v_unit_norm=cfg.get("v_unit_norm", 0),
        qkv_qs=P("qkv_qs", np.int8), qkv_d=P("qkv_d", np.uint16),
        o_qs=P("o_qs", np.int8), o_d=P("o_d", np.uint16),
        gu_qs=P("gu_qs", np.int8), gu_d=P("gu_d", np.uint16),
        dn_qs=P("dn_qs", np.int8), dn_d=P("dn_d", np.uint16),
        g_in=P("g_in", np.float32), g_q=P("g_q", np.float32),
        g_k=P("g_k", np.float32), g_post=P("g_post", np.float32),
        k_cache=_ptr(kc), v_cache=_ptr(vc),
        rope_cos=P("rope_cos", np.float32), rope_sin=P("rope_sin", np.float32),
        ffn_act=cfg.get("ffn_act", 0), attn_softcap=cfg.get("attn_softcap", 0.0))
    tr = OrcLayerTrace()
    arrays = {}
    if trace:
        qd, kvd = nq * hd, nkv * hd
        arrays = dict(
            xq=np.empty(H, np.int8), xd=np.empty(H // 32, np.uint16),
            qkv=np.empty(qd + 2 * kvd, np.float32),
            q=np.empty(qd, np.float32), k=np.empty(kvd, np.float32), v=np.empty(kvd, np.float32),
            attn=np.empty(qd, np.float32), aq=np.empty(qd, np.int8), ad=np.empty(qd // 32, np.uint16),
            x1=np.empty(H, np.float32))
        if cfg["kind"] == 0 and I > 0:
            arrays.update(nq=np.empty(H, np.int8), nd=np.empty(H // 32, np.uint16),
                          gu=np.empty(2 * I, np.float32),
                          hq=np.empty(I, np.int8), hd=np.empty(I // 32, np.uint16))
        for name, a in arrays.items():
            setattr(tr, name, _ptr(a))
    lib().orc_decode_layer(C.byref(L), _ptr(x), int(pos), C.byref(tr))
    return x, kc, vc, arrays

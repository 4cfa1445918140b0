"""Layer-level parity rules shared by the GPU layer tests and smoke().

Two checks beyond the per-stage (teacher-forced) ones:

* check_kv_row: the cache row the decode layer appends at `pos` is compared
  byte for byte.  The attention prologue reports its own f32 k / v (the
  qkv_post tap); the row must be exactly cvt(tap) (identity for f32, the
  oracle's f32 -> bf16 round-to-nearest-even for bf16), the tap must meet the
  float tolerance against the oracle, and the row may differ from the
  oracle's own cvt(oracle value) only by one bf16 step where a rounding
  midpoint lies between the GPU's f32 and the oracle's f32.

* free_running: the whole layer computed by the oracle from the original
  inputs, stage by stage.  At every point where a float becomes a discrete
  value (the Q8_0 codes and scales of a quantized activation, the bf16 cache
  row) the GPU's discrete values are checked against the oracle's float
  (near-boundary rule) and then carried forward, so that every difference
  between the GPU's layer output and this reference traces back to a counted
  flip; the output must then meet the float tolerance everywhere.
"""
import numpy as np

import oracle
from lqtest import assert_close, assert_q8_near


def _bf16_dec(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def check_kv_row(row_gpu, tap, ref, kv_dtype, what):
    """row_gpu: the cache row written at pos (f32 values or bf16 bits);
    tap: the GPU's f32 values before conversion; ref: the oracle's f32 values
    of the same step.  Returns the number of bf16 codes that differ from the
    oracle's own conversion (each one a checked boundary flip)."""
    row_gpu = np.asarray(row_gpu).ravel()
    tap = np.asarray(tap, np.float32).ravel()
    ref = np.asarray(ref, np.float32).ravel()
    assert_close(tap, ref, what + " (f32 before the cache conversion)")
    if kv_dtype == 0:
        assert np.array_equal(row_gpu.view(np.uint32), tap.view(np.uint32)), what + ": f32 row != its values"
        return 0
    row_gpu = row_gpu.view(np.uint16)
    assert np.array_equal(row_gpu, oracle.f32_to_bf16(tap)), what + ": bf16 row != RNE of the kernel's f32"
    want = oracle.f32_to_bf16(ref)
    diff = np.nonzero(row_gpu != want)[0]
    if diff.size:
        g, o = row_gpu[diff].astype(np.int32), want[diff].astype(np.int32)
        # adjacent bf16 values (same sign, codes one apart); the midpoint
        # between them must separate the two f32 values
        assert np.all(((g ^ o) & 0x8000) == 0) and np.all(np.abs(g - o) == 1), \
            what + ": bf16 differs by more than one step"
        a, b = _bf16_dec(row_gpu[diff]).astype(np.float64), _bf16_dec(want[diff]).astype(np.float64)
        mid = (a + b) / 2
        lo = np.minimum(tap[diff], ref[diff]).astype(np.float64)
        hi = np.maximum(tap[diff], ref[diff]).astype(np.float64)
        assert np.all((lo <= mid) & (mid <= hi)), what + ": bf16 flip without a rounding midpoint between the values"
        assert diff.size <= max(2, row_gpu.size // 100), f"{what}: {diff.size} bf16 flips"
    return int(diff.size)


def proj_matvec(w, key, xq, xd, residual=None):
    """The oracle's product of projection `key` ("qkv", "o", "gu", "dn") with a
    Q8_0 activation: its Q8_0 matvec, or the GGML-format matvec when the
    inputs carry that projection as Q4_0 / Q6_K blocks."""
    f = w.get(key + "_fmt")
    if f is None:
        return oracle.q8_matvec(w[key + "_qs"], w[key + "_d"], xq, xd, residual=residual)
    blocks = w[key + "_blocks"]
    rows, cols = blocks.shape[0], blocks.shape[1] * (32 if f == "q4_0" else 256)
    return oracle.q_matvec(f, blocks, rows, cols, xq, xd, residual=residual)


def post_rope(cfg, qkv, gq, gk, cos_row, sin_row):
    """The oracle's per-head steps after the QKV projection: RMSNorm (g_q / g_k)
    and NeoX RoPE of every q and k head, the optional unit norm of v."""
    nq, nkv, hd, eps = cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["eps"]
    qd, kvd = nq * hd, nkv * hd
    post = np.asarray(qkv, np.float32).copy()
    for h in range(nq + nkv):
        v = post[h * hd:(h + 1) * hd]
        if cfg["qk_norm"]:
            v = oracle.rmsnorm(v, gq if h < nq else gk, eps)
        post[h * hd:(h + 1) * hd] = oracle.rope_neox(v, cos_row, sin_row)
    if cfg["v_unit_norm"]:
        for g in range(nkv):
            s = slice(qd + kvd + g * hd, qd + kvd + (g + 1) * hd)
            post[s] = oracle.rmsnorm(post[s], None, eps)
    return post


def free_running(cfg, w, T, kc_gpu, vc_gpu, rope_cos, rope_sin, what="layer"):
    """The oracle's layer from the original inputs, carrying the GPU's discrete
    values forward at accepted rounding-boundary flips (see the module
    docstring).  T: the layer's taps (host arrays; xd/ad/nd/hd as uint16).
    kc_gpu / vc_gpu: the GPU's caches after the layer.  Returns (output,
    {stage: flips})."""
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    pos, eps, kind = cfg["pos"], cfg["eps"], cfg["kind"]
    qd, kvd = nq * hd, nkv * hd
    act, cap = cfg.get("ffn_act", 0), cfg.get("attn_softcap", 0.0)
    flips = {}
    # input RMSNorm and its Q8_0
    xn = oracle.rmsnorm(w["x"], w["g_in"], eps)
    flips["xq"] = assert_q8_near(T["xq"], T["xd"], xn, what + ": input norm Q8")
    qkv = proj_matvec(w, "qkv", T["xq"], T["xd"])
    post = post_rope(cfg, qkv, w.get("g_q"), w.get("g_k"), rope_cos[pos], rope_sin[pos])
    # the appended row: the oracle's conversion, or the GPU's at boundary flips
    kc, vc = w["k_cache"].copy(), w["v_cache"].copy()
    flips["kv"] = 0
    for cache, cache_gpu, off, name in ((kc, kc_gpu, qd, "k"), (vc, vc_gpu, qd + kvd, "v")):
        ref = post[off:off + kvd]
        tap = T["qkv_post"][off:off + kvd]
        if cfg["kv_dtype"] == 0:
            cache[:, pos] = ref.reshape(nkv, hd)
            continue
        flips["kv"] += check_kv_row(cache_gpu[:, pos], tap, ref, 1, f"{what}: {name} row (free-running)")
        cache[:, pos] = cache_gpu[:, pos]
    start = max(0, pos - cfg["window"] + 1) if cfg["window"] else 0
    att = oracle.attention(post[:qd], nq, nkv, hd, kc, vc, cfg["kv_dtype"], cfg["max_ctx"] * hd, hd, start,
                           pos - start + 1, cfg["attn_scale"], softcap=cap)
    flips["aq"] = assert_q8_near(T["aq"], T["ad"], att, what + ": attention Q8")
    if kind == 0:
        x1 = proj_matvec(w, "o", T["aq"], T["ad"], residual=w["x"])
        flips["nq"] = assert_q8_near(T["nq"], T["nd"], oracle.rmsnorm(x1, w["g_post"], eps), what + ": post norm Q8")
        gu = proj_matvec(w, "gu", T["nq"], T["nd"])
        gate = oracle.gelu_mul if act == 1 else oracle.silu_mul
        h = gate(gu[:I], gu[I:])
        flips["hq"] = assert_q8_near(T["hq"], T["hd"], h, what + ": Q8 of act(gate) * up")
        out = proj_matvec(w, "dn", T["hq"], T["hd"], residual=x1)
    else:
        o = proj_matvec(w, "o", T["aq"], T["ad"])
        out = (w["x"].astype(np.float64) + oracle.rmsnorm(o, w["g_post"], eps)).astype(np.float32)
    return out, flips

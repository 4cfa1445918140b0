"""Seeded synthetic inputs for the decode-layer hot path.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no quantization, normalisation, rotation, softmax or
dot products).  Both the GPU path and the CPU oracle receive exactly these
arrays.

Distributions (the workloads below):
  * Q8_0 weight codes: int8 uniform on [-127, 127].
  * Q8_0 weight scales: |N(0, 0.02)| / 127 stored as IEEE f16 (numpy's
    float16 cast); about 30% of them are f16 subnormals.
  * activations x: N(0, 1) float32.
  * norm weights gamma: N(1, 0.1) float32.
  * KV cache: N(0, 1); float32 caches keep the draw, bfloat16 caches keep
    the top 16 bits of the float32 draw (a truncation, which is a way of
    drawing bf16 values, not the path's f32->bf16 rounding).
  * MoE router logits: N(0, 1) float32.
  * output head (f16 weights): N(0, 0.02) cast to IEEE f16; its input is
    N(0, 1) float32 and its norm weight N(1, 0.1).
Draw order per layer: x, g_in, W_qkv, g_q, g_k, W_o, g_post, [W_gate_up,
W_down], K cache, V cache.  MoE: x, logits, W_gate_up (all experts),
W_down (all experts).
"""
import numpy as np

# Workloads by name: one decode token per layer.  The cache holds `ctx`
# positions, the new token sits at pos = ctx - 1 and is appended there.
WORKLOADS = {
    "tiny_h1024": dict(kind=0, hidden=1024, n_q=16, n_kv=8, head_dim=64, ffn=3072,
                       kv_dtype=0, ctx=128, window=0),
    "qwen3_4b_like_h2560": dict(kind=0, hidden=2560, n_q=32, n_kv=8, head_dim=80, ffn=9728,
                                kv_dtype=1, ctx=2048, window=0),
    "qwen3_8b_like_h4096": dict(kind=0, hidden=4096, n_q=32, n_kv=8, head_dim=128, ffn=12288,
                                kv_dtype=1, ctx=8192, window=0),
    "gemma4_sliding_h2816": dict(kind=1, hidden=2816, n_q=16, n_kv=8, head_dim=256, ffn=0,
                                 kv_dtype=1, ctx=8192, window=1024),
    "gemma4_global_h2816": dict(kind=1, hidden=2816, n_q=16, n_kv=2, head_dim=512, ffn=0,
                                kv_dtype=1, ctx=8192, window=0),
    # one GPU's share of the 8B-like layer under 8-way tensor parallelism: 4
    # query heads with their 1 kv head, a 1536-wide FFN slice (QKV 768 x 4096,
    # O 4096 x 512, gate_up 3072 x 4096, down 4096 x 1536); on one GPU the
    # residual is added locally where the sharded layer would all-reduce
    "qwen3_8b_like_h4096_tp8_share": dict(kind=0, hidden=4096, n_q=4, n_kv=1, head_dim=128, ffn=1536,
                                          kv_dtype=1, ctx=8192, window=0),
}
MOE_WORKLOADS = {
    "moe_e128_top8_t16": dict(hidden=2816, ffn=704, n_experts=128, top_k=8, tokens=16),
}
HEADLINE = "qwen3_8b_like_h4096"
COMMON = dict(eps=1e-6, theta=1e6)


def layer_cfg(name):
    c = dict(WORKLOADS[name])
    c.update(COMMON)
    c["max_ctx"] = c["ctx"]
    c["pos"] = c["ctx"] - 1
    c["qk_norm"] = 1
    c["v_unit_norm"] = 1 if c["kind"] == 1 else 0
    c["attn_scale"] = 1.0 / np.sqrt(c["head_dim"])
    return c


def q8_weight(rng, rows, cols):
    """(codes int8 [rows, cols], scales uint16 f16-bits [rows, cols/32])."""
    qs = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    d = (np.abs(rng.normal(0.0, 0.02, size=(rows, cols // 32))) / 127.0)
    return qs, d.astype(np.float16).view(np.uint16)


def q4_0_blocks(rng, rows, cols):
    """GGML Q4_0 blocks uint8 [rows, cols/32, 18]: f16 scale bytes (little
    endian; |N(0, 0.02)|/8, so d*(n-8) spreads like the Q8_0 weights) then 16
    random code bytes."""
    nb = cols // 32
    blk = np.empty((rows, nb, 18), np.uint8)
    d = (np.abs(rng.normal(0.0, 0.02, size=(rows, nb))) / 8.0).astype(np.float16).view(np.uint16)
    blk[..., 0] = d & 0xFF
    blk[..., 1] = d >> 8
    blk[..., 2:] = rng.integers(0, 256, size=(rows, nb, 16), dtype=np.uint8)
    return blk


def q6_k_blocks(rng, rows, cols):
    """GGML Q6_K blocks uint8 [rows, cols/256, 210]: 192 random bytes of
    low/high code bits, 16 random int8 sub-scales (the full range), then the
    f16 super-scale bytes (|N(0, 1)| * 2e-5, so weights spread about 0.02;
    many are f16-subnormal)."""
    nsb = cols // 256
    blk = np.empty((rows, nsb, 210), np.uint8)
    blk[..., :208] = rng.integers(0, 256, size=(rows, nsb, 208), dtype=np.uint8)
    d = (np.abs(rng.normal(0.0, 1.0, size=(rows, nsb))) * 2e-5).astype(np.float16).view(np.uint16)
    blk[..., 208] = d & 0xFF
    blk[..., 209] = d >> 8
    return blk


# The output head of the Gemma-4 shape the pages quote (vocab 262144, hidden 2816).
HEAD = dict(vocab=262144, hidden=2816, eps=1e-6, softcap=30.0)


def f16_weight(rng, rows, cols, std=0.02):
    """f16 bits [rows, cols]: N(0, std) cast to IEEE binary16 by numpy."""
    return (rng.standard_normal((rows, cols)) * std).astype(np.float16).view(np.uint16)


def activations(rng, *shape):
    return rng.standard_normal(shape, dtype=np.float32)


def gamma(rng, n):
    return (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)


def kv_cache(rng, n_kv, ctx, hd, kv_dtype):
    """[n_kv, ctx, hd] float32 (dtype 0) or bf16 bit patterns (dtype 1)."""
    a = rng.standard_normal((n_kv, ctx, hd), dtype=np.float32)
    if kv_dtype == 0:
        return a
    return (a.view(np.uint32) >> 16).astype(np.uint16)


PROJECTIONS = ("qkv", "o", "gu", "dn")     # the layer's four weights, in lq_layer_desc.w_format order


def layer_inputs(name, seed=0, formats=None):
    """All inputs of one decode layer of workload `name` (numpy, CPU).
    formats: optional {"qkv" | "o" | "gu" | "dn": "q4_0" | "q6_k"}; those
    projections are drawn as GGML blocks (w[key + "_blocks"], with
    w[key + "_fmt"]) in place of Q8_0 codes and scales, in the same draw
    order."""
    c = layer_cfg(name)
    rng = np.random.Generator(np.random.PCG64(seed))
    H, nq, nkv, hd, I = c["hidden"], c["n_q"], c["n_kv"], c["head_dim"], c["ffn"]
    w = {}

    def proj(key, rows, cols):
        f = (formats or {}).get(key)
        if f is None:
            w[key + "_qs"], w[key + "_d"] = q8_weight(rng, rows, cols)
        else:
            w[key + "_fmt"] = f
            w[key + "_blocks"] = (q4_0_blocks if f == "q4_0" else q6_k_blocks)(rng, rows, cols)

    w["x"] = activations(rng, H)
    w["g_in"] = gamma(rng, H)
    proj("qkv", nq * hd + 2 * nkv * hd, H)
    w["g_q"] = gamma(rng, hd)
    w["g_k"] = gamma(rng, hd)
    proj("o", H, nq * hd)
    w["g_post"] = gamma(rng, H)
    if I > 0:
        proj("gu", 2 * I, H)
        proj("dn", H, I)
    w["k_cache"] = kv_cache(rng, nkv, c["max_ctx"], hd, c["kv_dtype"])
    w["v_cache"] = kv_cache(rng, nkv, c["max_ctx"], hd, c["kv_dtype"])
    return c, w


def moe_inputs(name, seed=0, **over):
    """The MoE workload `name`, or its shape with fields replaced by `over`
    (tokens, hidden, ffn, n_experts, top_k)."""
    c = dict(MOE_WORKLOADS[name])
    c.update(over)
    rng = np.random.Generator(np.random.PCG64(seed))
    H, I, E, T = c["hidden"], c["ffn"], c["n_experts"], c["tokens"]
    w = {}
    w["x"] = activations(rng, T, H)
    w["logits"] = activations(rng, T, E)
    qs, d = q8_weight(rng, E * 2 * I, H)
    w["gu_qs"], w["gu_d"] = qs.reshape(E, 2 * I, H), d.reshape(E, 2 * I, H // 32)
    qs, d = q8_weight(rng, E * H, I)
    w["dn_qs"], w["dn_d"] = qs.reshape(E, H, I), d.reshape(E, H, I // 32)
    return c, w

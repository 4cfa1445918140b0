"""Per-operation parity of the HIP path (through the C ABI) with the oracle.

Bar: integer work (Q8_0 codes and scales from identical float inputs, int32
block dots, MoE ids) bit-exact; float outputs within |gpu - ref| <=
max(1e-3 |ref|, 1e-4).  Quantized codes of float values that the two sides
compute in different rounding orders use the near-boundary rule of
tests/lqtest.py.  Sizes span several tiles with ragged tails, plus the
workloads' full shapes.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

lq = pytest.importorskip("q8_matvec_gqa_amd")
from lqtest import (assert_close, assert_q8_near, dev, empty, host, sync, torch_mod,  # noqa: E402
                    workspace)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------------------------ quantize
def test_quantize_golden_blocks():
    from test_oracle_pins import load_golden_blocks
    cases = load_golden_blocks()
    x = np.concatenate([c["x"] for c in cases])
    xq, xd = empty(x.size, np.int8), empty(x.size // 32, np.uint16)
    lq.lq_q8_quantize_act(dev(x), 1, x.size, xq, xd)
    sync()
    assert np.array_equal(host(xq), np.concatenate([c["q"] for c in cases]))
    assert np.array_equal(host(xd, np.uint16), np.array([c["d"] for c in cases], np.uint16))


@pytest.mark.parametrize("n_rows,n,scale", [(1, 32, 1.0), (3, 4096, 1.0), (7, 12288, 1.0),
                                            (5, 9728, 1e-3), (2, 2816, 3e-6), (1, 64 * 1000 + 32, 50.0)])
def test_quantize_bit_exact(n_rows, n, scale):
    x = (synthetic.activations(rng(n), n_rows, n) * np.float32(scale)).astype(np.float32)
    x[0, :32] = 0.0                                             # an all-zero block
    xq, xd = empty((n_rows, n), np.int8), empty((n_rows, n // 32), np.uint16)
    lq.lq_q8_quantize_act(dev(x), n_rows, n, xq, xd)
    sync()
    rq, rd = oracle.q8_quantize(x)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(xd, np.uint16), rd)   # includes f16-subnormal scales at scale 3e-6


@pytest.mark.parametrize("n_rows,n", [(1, 1024), (1, 4096), (2, 2816), (3, 2560)])
def test_rmsnorm_q8(n_rows, n):
    r = rng(100 + n)
    x = synthetic.activations(r, n_rows, n) * 3
    g = synthetic.gamma(r, n)
    xq, xd = empty((n_rows, n), np.int8), empty((n_rows, n // 32), np.uint16)
    lq.lq_rmsnorm_q8(dev(x), n_rows, n, dev(g), 1e-6, xq, xd)
    sync()
    for i in range(n_rows):
        ref = oracle.rmsnorm(x[i], g, 1e-6)
        assert_q8_near(host(xq)[i], host(xd, np.uint16)[i], ref, f"row {i}")
    lq.lq_rmsnorm_q8(dev(x), n_rows, n, None, 1e-6, xq, xd)    # unit-weight form
    sync()
    for i in range(n_rows):
        assert_q8_near(host(xq)[i], host(xd, np.uint16)[i], oracle.rmsnorm(x[i], None, 1e-6), f"unit {i}")


@pytest.mark.parametrize("n_rows,ffn", [(1, 3072), (1, 12288), (128, 704), (3, 96)])
def test_swiglu_q8(n_rows, ffn):
    gu = synthetic.activations(rng(ffn + n_rows), n_rows, 2 * ffn) * 2
    hq, hd = empty((n_rows, ffn), np.int8), empty((n_rows, ffn // 32), np.uint16)
    lq.lq_swiglu_q8(dev(gu), n_rows, ffn, hq, hd)
    sync()
    for i in range(n_rows):
        ref = oracle.silu_mul(gu[i, :ffn], gu[i, ffn:])
        assert_q8_near(host(hq)[i], host(hd, np.uint16)[i], ref, f"row {i}")


# ------------------------------------------------------------------ block dots / matvec
DOT_SHAPES = [(1, 32), (3, 64), (5, 1024), (37, 1056), (64, 2560), (9, 2816), (17, 4096), (4, 9728),
              (13, 12288), (3, 16384), (2, 17408)]     # 17408 > 16 KB: the generic path
# rows at the thresholds where rows of at most 4 KB change rows per group
# (one row up to 2048 rows, two up to 4096, three up to 6144), with ragged
# last groups and a ragged last 1 KB chunk
THRESHOLD_SHAPES = [(2048, 1024), (2049, 1024), (4096, 1056), (4097, 3072), (6143, 2080), (6145, 4096)]


@pytest.mark.parametrize("rows,cols", DOT_SHAPES + THRESHOLD_SHAPES)
def test_block_dots_bit_exact(rows, cols):
    r = rng(rows * 7 + cols)
    wq = r.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    wq[0, :32] = -128                                     # extreme block: 524288
    xq = r.integers(-127, 128, size=cols, dtype=np.int8)
    xq[:32] = -128
    wd = np.zeros((rows, cols // 32), np.uint16)
    dots = empty((rows, cols // 32), np.int32)
    lq.lq_q8_block_dots(lq.q8_weight(dev(wq), dev(wd)), dev(xq), dots)
    sync()
    ref = oracle.q8_block_dots(wq, xq)
    assert ref[0, 0] == 524288
    assert np.array_equal(host(dots), ref)


def _layer_projections():
    """(tag, rows, cols, prologue) for every projection of the layer workloads:
    QKV and gate_up build their input with the RMSNorm prologue, O with the
    quantize prologue, down reads the Q8_0 of h; plus the MoE experts' shapes."""
    out = []
    for name, c in synthetic.WORKLOADS.items():
        H, qd, kvd, I = c["hidden"], c["n_q"] * c["head_dim"], c["n_kv"] * c["head_dim"], c["ffn"]
        out += [(name + ":qkv", qd + 2 * kvd, H, "norm"), (name + ":o", H, qd, "quant")]
        if I:
            out += [(name + ":gate_up", 2 * I, H, "norm"), (name + ":down", H, I, "q8")]
    m = synthetic.MOE_WORKLOADS["moe_e128_top8_t16"]
    out += [("moe:gate_up", 2 * m["ffn"], m["hidden"], "q8"), ("moe:down", m["hidden"], m["ffn"], "q8")]
    return out


@pytest.mark.parametrize("tag,rows,cols,pro", _layer_projections(), ids=lambda v: str(v))
def test_block_dots_layer_projections(tag, rows, cols, pro):
    """The int32 block dots of the fused matvec kernel the layer runs, at every
    projection shape of the layer workloads, through the prologue each one
    uses there: bit-exact against the oracle's integer sums of the Q8_0 input
    the kernel built (which itself must match the oracle's quantization)."""
    r = rng(rows + 11 * cols)
    wq, wd = synthetic.q8_weight(r, rows, cols)
    wq[rows - 1, -32:] = -128                              # extreme block in the last row
    W = lq.q8_weight(dev(wq), dev(wd))
    dots = empty((rows, cols // 32), np.int32)
    print(f"[dots] {tag} {rows}x{cols} prologue {pro}", flush=True)
    if pro == "q8":
        xq, _ = oracle.q8_quantize(synthetic.activations(r, cols))
        lq.lq_q8_block_dots(W, dev(xq), dots)
        sync()
    else:
        x = synthetic.activations(r, cols) * 2
        g = synthetic.gamma(r, cols)
        xq_d, xd_d = empty(cols, np.int8), empty(cols // 32, np.uint16)
        lq.lq_q8_block_dots_f32(W, dev(x), pro == "norm", dev(g), 1e-6, dots, xq_d, xd_d)
        sync()
        xq, xd = host(xq_d), host(xd_d, np.uint16)
        if pro == "norm":
            assert_q8_near(xq, xd, oracle.rmsnorm(x, g, 1e-6), tag + " input Q8")
        else:
            rq, rd = oracle.q8_quantize(x)                  # identical float input: bit-exact
            assert np.array_equal(xq, rq) and np.array_equal(xd, rd)
    assert np.array_equal(host(dots), oracle.q8_block_dots(wq, xq)), tag


MATVEC_SHAPES = DOT_SHAPES[1:] + [(6144, 4096), (4096, 4096), (24576, 4096), (4096, 12288),
                                  (10240, 2816), (2816, 8192), (1, 4096), (255, 3072)]
MATVEC_SHAPES += THRESHOLD_SHAPES


@pytest.mark.parametrize("rows,cols", MATVEC_SHAPES)
def test_matvec(rows, cols):
    r = rng(rows + 3 * cols)
    wq, wd = synthetic.q8_weight(r, rows, cols)
    x = synthetic.activations(r, cols)
    xq, xd = oracle.q8_quantize(x)
    res = synthetic.activations(r, rows)
    W = lq.q8_weight(dev(wq), dev(wd))
    y = empty(rows, np.float32)
    lq.lq_q8_matvec(W, dev(xq), dev(xd), None, y)
    y_res = dev(res)
    lq.lq_q8_matvec(W, dev(xq), dev(xd), y_res, y_res)        # y aliases residual
    sync()
    assert_close(host(y), oracle.q8_matvec(wq, wd, xq, xd), "matvec")
    assert_close(host(y_res), oracle.q8_matvec(wq, wd, xq, xd, residual=res), "matvec+residual")


def test_matvec_deterministic():
    r = rng(5)
    wq, wd = synthetic.q8_weight(r, 24576, 4096)
    xq, xd = oracle.q8_quantize(synthetic.activations(r, 4096))
    W = lq.q8_weight(dev(wq), dev(wd))
    a, b = empty(24576, np.float32), empty(24576, np.float32)
    lq.lq_q8_matvec(W, dev(xq), dev(xd), None, a)
    lq.lq_q8_matvec(W, dev(xq), dev(xd), None, b)
    sync()
    assert np.array_equal(host(a), host(b))


# ------------------------------------------------------------------ norm + RoPE, KV append
@pytest.mark.parametrize("n_heads,hd,stride,use_gamma,use_rope,pos", [
    (16, 64, 64, True, True, 127), (32, 80, 96, True, True, 2047), (32, 128, 128, True, True, 8191),
    (8, 256, 256, False, True, 5000), (2, 512, 520, True, False, 0), (3, 2, 2, True, True, 7)])
def test_rmsnorm_rope(n_heads, hd, stride, use_gamma, use_rope, pos):
    r = rng(hd + pos)
    x = synthetic.activations(r, n_heads * stride) * 2
    g = synthetic.gamma(r, hd) if use_gamma else None
    ctx = pos + 1
    c = np.zeros((ctx, hd // 2), np.float32)
    s = np.zeros((ctx, hd // 2), np.float32)
    lq.lq_rope_table(ctx, hd, 1e6, c, s)
    xt = dev(x)
    lq.lq_rmsnorm_rope(xt, n_heads, hd, stride, None if g is None else dev(g), 1e-6,
                       dev(c) if use_rope else None, dev(s) if use_rope else None, ctx, pos)
    sync()
    got = host(xt)
    oc, os_ = oracle.rope_table(ctx, hd, 1e6)
    want = x.copy()
    for h in range(n_heads):
        v = oracle.rmsnorm(x[h * stride:h * stride + hd], g, 1e-6)
        if use_rope:
            v = oracle.rope_neox(v, oc[pos], os_[pos])
        want[h * stride:h * stride + hd] = v
    assert_close(got, want, "rmsnorm_rope")     # includes the untouched gaps between heads


@pytest.mark.parametrize("dtype", [0, 1])
def test_kv_append(dtype):
    r = rng(11 + dtype)
    n_kv, hd, ctx, pos = 8, 128, 64, 37
    kc = synthetic.kv_cache(r, n_kv, ctx, hd, dtype)
    vc = synthetic.kv_cache(r, n_kv, ctx, hd, dtype)
    k = synthetic.activations(r, n_kv * hd)
    v = synthetic.activations(r, n_kv * hd)
    kt, vt = dev(kc), dev(vc)
    lq.lq_kv_append(dev(k), dev(v), n_kv, hd, kt, vt, dtype, ctx * hd, hd, ctx, pos)
    sync()
    dt = np.float32 if dtype == 0 else np.uint16
    gk, gv = host(kt, dt), host(vt, dt)
    ek, ev = kc.copy(), vc.copy()
    conv = (lambda a: a) if dtype == 0 else oracle.f32_to_bf16
    ek[:, pos] = conv(k).reshape(n_kv, hd)
    ev[:, pos] = conv(v).reshape(n_kv, hd)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


# ------------------------------------------------------------------ attention
def run_attn(q, n_q, n_kv, hd, kc, vc, dtype, hs, ps, max_ctx, start, length, scale):
    out = empty(n_q * hd, np.float32)
    need = lq.lq_gqa_decode_attn_workspace_size(n_q, n_kv, hd, length)
    ws = workspace(need)
    qd = q if not isinstance(q, np.ndarray) else dev(q)
    lq.lq_gqa_decode_attn(qd, n_q, n_kv, hd, dev(kc), dev(vc), dtype, hs, ps, max_ctx, start, length,
                          scale, out, ws, ws.numel())
    sync()
    return host(out)


ATTN_CASES = [
    # n_q, n_kv, hd, dtype, ctx, start, len
    (16, 8, 64, 0, 128, 0, 128),          # tiny layer shape
    (32, 8, 80, 1, 2048, 0, 2048),        # 4B-like
    (32, 8, 128, 1, 8192, 0, 8192),       # 8B-like (headline)
    (16, 8, 256, 1, 8192, 7168, 1024),    # Gemma sliding: window with start > 0
    (16, 2, 512, 1, 8192, 0, 8192),       # Gemma global
    (32, 8, 128, 1, 300, 0, 1),           # one position
    (32, 8, 128, 1, 300, 0, 63), (32, 8, 128, 1, 300, 0, 65), (32, 8, 128, 1, 3000, 1, 2999),
    (8, 8, 64, 1, 200, 10, 150),          # G = 1 (generic instance)
    (20, 4, 64, 1, 500, 3, 333),          # G = 5 (generic instance)
    (16, 2, 128, 1, 1000, 0, 1000),       # G = 8
    (8, 2, 96, 0, 700, 100, 555),         # f32, head_dim 96 (generic)
    (8, 2, 512, 0, 200, 0, 200),          # f32, head_dim 512 (two chunks per lane in V)
    (4, 4, 8, 1, 130, 0, 130),            # head_dim 8: one 16-byte chunk per row
    (32, 8, 128, 1, 65536, 0, 65536),     # long context: 64 splits of 1024 positions (16 tiles per wave)
    # head_dim 512, G 8, bf16 (the Gemma-global instance): ragged tiles, one and four kv heads, long context
    (16, 2, 512, 1, 300, 0, 1),           # one position
    (16, 2, 512, 1, 300, 0, 17),          # a few tiles and one position
    (8, 1, 512, 1, 1000, 5, 995),         # one kv head, start > 0, a ragged last tile
    (32, 4, 512, 1, 3000, 100, 1500),     # four kv heads, a window
    (16, 2, 512, 1, 65536, 0, 65536),     # long context: several tiles per wave
    # the same heads from 2048 positions on, where the scores run on the matrix cores
    (16, 2, 512, 1, 2048, 0, 2048),       # the first length that does
    (8, 1, 512, 1, 3000, 7, 2501),        # one kv head, start > 0, a ragged last 16-position tile
    (32, 4, 512, 1, 5000, 100, 4099),     # four kv heads, a window, ragged
]


@pytest.mark.parametrize("n_q,n_kv,hd,dtype,ctx,start,length", ATTN_CASES)
def test_attention(n_q, n_kv, hd, dtype, ctx, start, length):
    r = rng(n_q * hd + ctx + start)
    kc = synthetic.kv_cache(r, n_kv, ctx, hd, dtype)
    vc = synthetic.kv_cache(r, n_kv, ctx, hd, dtype)
    q = synthetic.activations(r, n_q * hd)
    scale = 1 / math.sqrt(hd)
    got = run_attn(q, n_q, n_kv, hd, kc, vc, dtype, ctx * hd, hd, ctx, start, length, scale)
    want = oracle.attention(q, n_q, n_kv, hd, kc, vc, dtype, ctx * hd, hd, start, length, scale)
    assert_close(got, want, "attention")


def test_attention_strided_layout():
    """Cache laid out [ctx, n_kv, hd]: head stride hd, position stride n_kv*hd."""
    r = rng(77)
    n_q, n_kv, hd, ctx = 32, 8, 128, 1500
    kc = synthetic.kv_cache(r, ctx, n_kv, hd, 1)
    vc = synthetic.kv_cache(r, ctx, n_kv, hd, 1)
    q = synthetic.activations(r, n_q * hd)
    got = run_attn(q, n_q, n_kv, hd, kc, vc, 1, hd, n_kv * hd, ctx, 200, 1300, 0.1)
    want = oracle.attention(q, n_q, n_kv, hd, kc, vc, 1, hd, n_kv * hd, 200, 1300, 0.1)
    assert_close(got, want, "attention strided")


@pytest.mark.parametrize("hd,n_kv,n_q", [(128, 8, 32), (256, 8, 16), (512, 2, 16)])
def test_attention_unaligned_query(hd, n_kv, n_q):
    """q 4-byte but not 16-byte aligned: the exact instances read query rows
    with vector loads, so the padded instance must take the call."""
    r = rng(91 + hd)
    ctx = 1200
    kc = synthetic.kv_cache(r, n_kv, ctx, hd, 1)
    vc = synthetic.kv_cache(r, n_kv, ctx, hd, 1)
    q = synthetic.activations(r, n_q * hd)
    qd = dev(np.concatenate([np.zeros(1, np.float32), q]))[1:]
    assert qd.data_ptr() % 16 == 4
    got = run_attn(qd, n_q, n_kv, hd, kc, vc, 1, ctx * hd, hd, ctx, 5, 1190, 0.07)
    want = oracle.attention(q, n_q, n_kv, hd, kc, vc, 1, ctx * hd, hd, 5, 1190, 0.07)
    assert_close(got, want, "attention unaligned q")


def test_attention_empty_window_writes_zeros():
    out = dev(np.full(64 * 4, 7.0, np.float32))
    lq.lq_gqa_decode_attn(dev(np.zeros(256, np.float32)), 4, 2, 64, None, None, 1, 64 * 10, 64, 10, 0, 0,
                          0.125, out, None, 0)
    sync()
    assert np.all(host(out) == 0)


def test_attention_deterministic():
    r = rng(3)
    n_q, n_kv, hd, ctx = 32, 8, 128, 8192
    kc = synthetic.kv_cache(r, n_kv, ctx, hd, 1)
    vc = synthetic.kv_cache(r, n_kv, ctx, hd, 1)
    q = synthetic.activations(r, n_q * hd)
    a = run_attn(q, n_q, n_kv, hd, kc, vc, 1, ctx * hd, hd, ctx, 0, ctx, 0.088)
    b = run_attn(q, n_q, n_kv, hd, kc, vc, 1, ctx * hd, hd, ctx, 0, ctx, 0.088)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ multi-token matmul
def run_matmul(W, rows, cols, xq, xd, T, res, y):
    nws = lq.lq_q8_matmul_workspace_size(rows, cols, T)
    ws = empty(max(nws // 4, 1), np.float32)
    lq.lq_q8_matmul(W, xq, xd, T, res, y, ws, nws)
    sync()


@pytest.mark.parametrize("T,rows,cols", [
    (32, 4096, 4096),     # a batch of 32 on the 8B-like O projection
    (1, 96, 64),          # one token, two blocks
    (17, 1000, 1024),     # ragged tokens and rows
    (45, 300, 2816),      # two token chunks (32 + 13), Gemma width
    (33, 64, 16384),      # widest rows
    (16, 6144, 4096),     # 8B-like QKV, half a tile of tokens
    (32, 24576, 4096),    # 8B-like gate_up (no block split)
    (8, 4096, 12288),     # 8B-like down (block split over 6 workgroups)
    (32, 33, 32),         # one block, a one-row ragged tile
    (200, 1000, 2048),    # prefill-like: 7 token chunks in one launch (6 full + 8 tokens), ragged rows
    (512, 256, 1024),     # 16 chunks over 8 row tiles
    (512, 4096, 256),     # 64 x 64 tiles (512 of them), one batch
    (1000, 2050, 512),    # 64 x 64 tiles with ragged rows and tokens, two batches
    (520, 3650, 352),     # 64 x 64 tiles, ragged rows and tokens, a partial last batch (8 + 3 blocks)
])
def test_q8_matmul(T, rows, cols):
    r = rng(T * 7 + rows + cols)
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = (np.abs(r.standard_normal((T, cols // 32))) * 0.05).astype(np.float16).view(np.uint16)
    res = synthetic.activations(r, T, rows)
    y = empty(T * rows, np.float32)
    run_matmul(lq.q8_weight(dev(wq), dev(wd)), rows, cols, dev(xq), dev(xd), T, dev(res), y)
    want = oracle.q8_matmul(wq, wd, xq, xd, residual=res)
    assert_close(host(y).reshape(T, rows), want, "q8 matmul")


def test_q8_matmul_prefill_full_size_sampled():
    """The bench's prefill launch (512 tokens on the 8B-like gate_up weight,
    64 x 64 tiles): sampled tokens against the oracle matvec of each."""
    r = rng(512)
    T, rows, cols = 512, 24576, 4096
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = (np.abs(r.standard_normal((T, cols // 32))) * 0.05).astype(np.float16).view(np.uint16)
    y = empty(T * rows, np.float32)
    run_matmul(lq.q8_weight(dev(wq), dev(wd)), rows, cols, dev(xq), dev(xd), T, None, y)
    Y = host(y).reshape(T, rows)
    for t in (0, 63, 64, 300, 511):
        assert_close(Y[t], oracle.q8_matvec(wq, wd, xq[t], xd[t]), f"token {t}")


@pytest.mark.parametrize("rows,cols", [(4096, 4096), (24576, 1024)])
def test_q8_matmul_in_place_and_repeatable(rows, cols):
    """y aliasing the residual (the residual-add form of a projection) gives
    the same as separate buffers, and two runs agree bit for bit (the split
    partials are summed in a fixed order)."""
    r = rng(rows + 3 * cols)
    T = 20
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = (np.abs(r.standard_normal((T, cols // 32))) * 0.05).astype(np.float16).view(np.uint16)
    res = synthetic.activations(r, T, rows)
    W = lq.q8_weight(dev(wq), dev(wd))
    y1 = empty(T * rows, np.float32)
    run_matmul(W, rows, cols, dev(xq), dev(xd), T, dev(res), y1)
    y2 = dev(res)
    run_matmul(W, rows, cols, dev(xq), dev(xd), T, y2, y2)
    assert np.array_equal(host(y1).reshape(T, rows), host(y2).reshape(T, rows))
    assert_close(host(y1).reshape(T, rows), oracle.q8_matmul(wq, wd, xq, xd, residual=res), "q8 matmul")


def test_q8_matmul_subnormal_scales():
    """Q8_0 scales are f16 including its subnormals: blocks whose weight or
    activation scale is subnormal (or zero) keep their exact products, with
    no flush to zero.  Rows 0-63 have only subnormal weight scales, tokens
    0-7 only subnormal activation scales; each region is checked with an
    absolute floor far below its own magnitude."""
    r = rng(77)
    T, rows, cols = 32, 256, 1024
    nb = cols // 32
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    wsub = r.integers(1, 1024, (rows, nb)).astype(np.uint16)                     # f16 subnormal bit patterns
    wd = np.where(r.random((rows, nb)) < 0.5, wsub, wd).astype(np.uint16)
    wd[:64] = wsub[:64]
    wd[:, 3] = 0                                                                  # a zero scale
    xsub = r.integers(1, 1024, (T, nb)).astype(np.uint16)
    xd = (np.abs(r.standard_normal((T, nb))) * 0.05).astype(np.float16).view(np.uint16)
    xd = np.where(r.random((T, nb)) < 0.5, xsub, xd).astype(np.uint16)
    xd[:8] = xsub[:8]
    y = empty(T * rows, np.float32)
    run_matmul(lq.q8_weight(dev(wq), dev(wd)), rows, cols, dev(xq), dev(xd), T, None, y)
    got = host(y).reshape(T, rows)
    want = oracle.q8_matmul(wq, wd, xq, xd)
    assert_close(got, want, "q8 matmul, mixed scales")
    both = np.abs(want[:8, :64]).mean()
    assert 1e-6 < both < 1e-3
    assert_close(got[:8, :64], want[:8, :64], "subnormal x subnormal", atol=both * 1e-5)
    assert_close(got[8:, :64], want[8:, :64], "subnormal weight scales", atol=np.abs(want[8:, :64]).mean() * 1e-5)
    assert_close(got[:8, 64:], want[:8, 64:], "subnormal activation scales", atol=np.abs(want[:8, 64:]).mean() * 1e-5)


def test_q8_matmul_workspace_checked():
    r = rng(5)
    rows, cols, T = 4096, 4096, 4
    need = lq.lq_q8_matmul_workspace_size(rows, cols, T)
    assert need > 0
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = np.ones((T, cols // 32), np.float16).view(np.uint16)
    y = empty(T * rows, np.float32)
    ws = empty(need // 4, np.float32)
    st = lq.lq_q8_matmul(lq.q8_weight(dev(wq), dev(wd)), dev(xq), dev(xd), T, None, y, ws, need - 4, check=False)
    assert st == lq.LQ_ERR_WORKSPACE


def test_q8_matmul_matches_matvec_rows():
    """Every token row of the MFMA matmul equals the decode matvec of that
    token to the float tolerance (same block dots, different combine order)."""
    r = rng(404)
    T, rows, cols = 24, 512, 2048
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = (np.abs(r.standard_normal((T, cols // 32))) * 0.05).astype(np.float16).view(np.uint16)
    W = lq.q8_weight(dev(wq), dev(wd))
    y = empty(T * rows, np.float32)
    run_matmul(W, rows, cols, dev(xq), dev(xd), T, None, y)
    Y = host(y).reshape(T, rows)
    for t in (0, 5, 23):
        yt = empty(rows, np.float32)
        lq.lq_q8_matvec(W, dev(xq[t]), dev(xd[t]), None, yt)
        sync()
        assert_close(Y[t], host(yt), f"token {t}")


# ------------------------------------------------------------------ Q4_0 / Q6_K weights
def ggml_weight(fmt, r, rows, cols):
    """Random GGML blocks, packed on the host by the library's helper and
    uploaded: (blocks, lq weight struct)."""
    if fmt == "q4_0":
        b = synthetic.q4_0_blocks(r, rows, cols)
        qs = np.zeros((rows, cols // 2), np.uint8)
        d = np.zeros((rows, cols // 32), np.uint16)
        lq.lq_q4_0_pack_ggml(b, rows, cols, qs, d)
        return b, lq.q4_0_weight(dev(qs), dev(d), rows, cols)
    b = synthetic.q6_k_blocks(r, rows, cols)
    ql = np.zeros((rows, cols // 2), np.uint8)
    qh = np.zeros((rows, cols // 4), np.uint8)
    sc = np.zeros((rows, cols // 16), np.int8)
    d = np.zeros((rows, cols // 256), np.uint16)
    lq.lq_q6_k_pack_ggml(b, rows, cols, ql, qh, sc, d)
    return b, lq.q6_k_weight(dev(ql), dev(qh), dev(sc), dev(d), rows, cols)


def run_qk(fmt, W, xq, xd, res, y):
    (lq.lq_q4_0_matvec if fmt == "q4_0" else lq.lq_q6_k_matvec)(W, xq, xd, res, y)
    sync()


@pytest.mark.parametrize("fmt,rows,cols", [
    ("q4_0", 4096, 4096),      # the 8B-like O projection
    ("q4_0", 24576, 4096),     # 8B-like gate_up
    ("q4_0", 4096, 12288),     # 8B-like down (6 steps per row)
    ("q4_0", 1000, 2816),      # Gemma width, ragged rows, a partial step
    ("q4_0", 33, 32),          # one block
    ("q4_0", 5, 16384),        # widest rows (8 steps)
    ("q6_k", 4096, 4096),
    ("q6_k", 24576, 4096),
    ("q6_k", 4096, 12288),     # 3 steps, one row per wave
    ("q6_k", 1000, 2816),      # 11 super-blocks: 44 of 64 lanes
    ("q6_k", 7, 256),          # one super-block
    ("q6_k", 9, 16384),        # widest rows (4 steps)
])
def test_ggml_format_matvec(fmt, rows, cols):
    r = rng(rows * 3 + cols + len(fmt))
    b, W = ggml_weight(fmt, r, rows, cols)
    xq = r.integers(-127, 128, cols).astype(np.int8)
    xd = (np.abs(r.standard_normal(cols // 32)) * 0.05).astype(np.float16).view(np.uint16)
    res = synthetic.activations(r, rows)
    y = empty(rows, np.float32)
    run_qk(fmt, W, dev(xq), dev(xd), dev(res), y)
    assert_close(host(y), oracle.q_matvec(fmt, b, rows, cols, xq, xd, residual=res), f"{fmt} matvec")
    # no residual, and the residual aliasing y
    run_qk(fmt, W, dev(xq), dev(xd), None, y)
    want = oracle.q_matvec(fmt, b, rows, cols, xq, xd)
    assert_close(host(y), want, f"{fmt} matvec, no residual")
    y2 = dev(res)
    run_qk(fmt, W, dev(xq), dev(xd), y2, y2)
    assert_close(host(y2), want + res, f"{fmt} matvec, in place")


@pytest.mark.parametrize("fmt", ["q4_0", "q6_k"])
def test_ggml_format_extreme_codes(fmt):
    """All-extreme codes (nibble 0 and 15; 6-bit 0 and 63), int8 sub-scales
    at -128 and 127 and +-127 activations: the int32 dots and the offsets
    at their limits."""
    r = rng(11 if fmt == "q4_0" else 12)
    rows, cols = 64, 2048
    b, _ = ggml_weight(fmt, r, rows, cols)
    if fmt == "q4_0":
        b[..., 2:] = np.where(r.random(b[..., 2:].shape) < 0.5, 0x00, 0xFF)
        qs = np.ascontiguousarray(b[..., 2:]).reshape(rows, cols // 2)
        d = b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8)
        W = lq.q4_0_weight(dev(qs), dev(d), rows, cols)
    else:
        b[..., :192] = np.where(r.random(b[..., :192].shape) < 0.5, 0x00, 0xFF)
        b[..., 192:208] = np.where(r.random(b[..., 192:208].shape) < 0.5, 0x80, 0x7F)
        ql = np.ascontiguousarray(b[..., :128]).reshape(rows, cols // 2)
        qh = np.ascontiguousarray(b[..., 128:192]).reshape(rows, cols // 4)
        sc = np.ascontiguousarray(b[..., 192:208]).view(np.int8).reshape(rows, cols // 16)
        d = b[..., 208].astype(np.uint16) | (b[..., 209].astype(np.uint16) << 8)
        W = lq.q6_k_weight(dev(ql), dev(qh), dev(sc), dev(d), rows, cols)
    xq = np.where(r.random(cols) < 0.5, -127, 127).astype(np.int8)
    xd = np.full(cols // 32, 0x2C00, np.uint16)       # f16 1/16
    y = empty(rows, np.float32)
    run_qk(fmt, W, dev(xq), dev(xd), None, y)
    assert_close(host(y), oracle.q_matvec(fmt, b, rows, cols, xq, xd), f"{fmt} extremes")


@pytest.mark.parametrize("fmt,E,rows,cols,T,k", [
    ("q4_0", 12, 200, 704, 5, 3),
    ("q6_k", 12, 200, 512, 5, 3),
    ("q6_k", 128, 1408, 2816, 16, 8),    # the MoE workload's gate/up on Q6_K experts
    ("q4_0", 128, 2816, 704, 16, 8),     # its down projection on Q4_0 experts
    ("q4_0", 6, 33, 1024, 4, 2),         # two rows per load: every lane of a half-wave holds a block
    ("q4_0", 5, 97, 32, 3, 2),           # one block per row, odd rows
    ("q4_0", 3, 17, 1056, 3, 2),         # 33 blocks: the one-row-per-load form again
    ("q4_0", 4, 64, 8192, 3, 2),         # widest rows (4 steps per lane)
    ("q6_k", 4, 33, 8192, 3, 2),         # Q6_K widest (2 steps), ragged row blocks
])
def test_moe_ggml_format_matvec_id(fmt, E, rows, cols, T, k):
    """The index-driven matvec on Q4_0 / Q6_K experts: every valid (t, s) equals
    the pinned oracle matvec of its expert; invalid ids give zeros."""
    r = rng(E + rows + cols + T)
    b, W = ggml_weight(fmt, r, E * rows, cols)
    W.rows = rows                                         # the struct describes one expert
    x = synthetic.activations(r, T * k, cols)
    xq, xd = oracle.q8_quantize(x)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, 0] = 99
    if T > 2:
        ids[1, 0] = ids[2, 1] = ids[0, 1]                  # an expert with several slots
    call = lq.lq_moe_q4_0_matvec_id if fmt == "q4_0" else lq.lq_moe_q6_k_matvec_id
    y = dev(np.full((T * k, rows), 5.0, np.float32))
    ws = workspace(lq.lq_moe_workspace_size(T, k, E))
    for per_slot in (1, 0):
        xq_use = xq if per_slot else np.ascontiguousarray(xq[::k])
        xd_use = xd if per_slot else np.ascontiguousarray(xd[::k])
        call(W, E, dev(xq_use), dev(xd_use), per_slot, dev(ids), T, k, y, ws, ws.numel())
        sync()
        got = host(y).reshape(T, k, rows)
        for t in range(T):
            for s in range(k):
                e = ids[t, s]
                xi = t * k + s if per_slot else t
                if 0 <= e < E:
                    ref = oracle.q_matvec(fmt, b[e * rows:(e + 1) * rows], rows, cols, xq_use[xi], xd_use[xi])
                    assert_close(got[t, s], ref, f"{fmt} slot {t},{s}")
                else:
                    assert np.all(got[t, s] == 0)


# ------------------------------------------------------------------ output head
@pytest.mark.parametrize("vocab,hidden,norm,cap", [
    (1000, 2816, True, 30.0),    # the Gemma-4 head width, ragged row count
    (777, 64, True, 0.0),        # one chunk per lane, no softcap
    (513, 520, False, 0.0),      # 65 chunks: the second step has one live lane
    (300, 4096, True, 5.0),      # widest supported row, a cap that bites
    (1, 8, True, 30.0),          # a single row of one chunk
])
def test_lm_head(vocab, hidden, norm, cap):
    r = rng(vocab + hidden)
    w = synthetic.f16_weight(r, vocab, hidden, 0.05)
    x = synthetic.activations(r, hidden)
    g = synthetic.gamma(r, hidden)
    out = empty(vocab, np.float32)
    lq.lq_lm_head_f16(dev(w), vocab, hidden, dev(x), int(norm), dev(g), 1e-6, cap, out)
    sync()
    want = oracle.lm_head(w, x, g, norm=norm, eps=1e-6, cap=cap)
    assert_close(host(out), want, "lm_head")


@pytest.mark.gpu
def test_lm_head_full_size_sampled():
    """The 262144 x 2816 head at full size (weights drawn on the GPU), checked
    on 256 sampled rows against the oracle."""
    torch = torch_mod()
    H = synthetic.HEAD
    V, D = H["vocab"], H["hidden"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    w = (torch.randn(V, D, device="cuda", generator=gen) * 0.02).half().view(torch.int16)
    x = torch.randn(D, device="cuda", generator=gen)
    g = 1.0 + 0.1 * torch.randn(D, device="cuda", generator=gen)
    out = torch.empty(V, dtype=torch.float32, device="cuda")
    lq.lq_lm_head_f16(w, V, D, x, 1, g, H["eps"], H["softcap"], out)
    sync()
    idx = np.sort(np.random.default_rng(5).choice(V, 256, replace=False))
    rows = w[torch.from_numpy(idx).cuda()].cpu().numpy().view(np.uint16)
    want = oracle.lm_head(rows, x.cpu().numpy(), g.cpu().numpy(), norm=True, eps=H["eps"], cap=H["softcap"])
    assert_close(host(out)[idx], want, "lm_head full size")
    del w
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ MoE pieces
def test_moe_route():
    r = rng(21)
    logits = synthetic.activations(r, 16, 128)
    logits[5, 7] = logits[5, 100] = 4.0                    # tie: lower id first
    ids, w = empty((16, 8), np.int32), empty((16, 8), np.float32)
    lq.lq_moe_route_topk(dev(logits), 16, 128, 8, ids, w)
    sync()
    rid, rw = oracle.moe_route(logits, 8)
    assert np.array_equal(host(ids), rid)
    assert host(ids)[5, 0] == 7 and host(ids)[5, 1] == 100
    assert_close(host(w), rw, "route weights")


def test_moe_matvec_id_and_weighted_sum():
    r = rng(22)
    E, rows, cols, T, k = 12, 200, 704, 5, 3
    wq, wd = synthetic.q8_weight(r, E * rows, cols)
    wq, wd = wq.reshape(E, rows, cols), wd.reshape(E, rows, cols // 32)
    x = synthetic.activations(r, T * k, cols)
    xq, xd = oracle.q8_quantize(x)
    ids = r.integers(0, E, size=(T, k)).astype(np.int32)
    ids[0, 0] = ids[1, 0] = ids[2, 1] = 4                   # an expert with several slots
    ids[4, 2] = 99                                          # out of range: zeros and counted
    ids[3, 1] = -1
    wqt, wdt = dev(wq), dev(wd)
    W = lq.lq_q8_weight(wqt.data_ptr(), wdt.data_ptr(), rows, cols)
    y = dev(np.full((T * k, rows), 5.0, np.float32))
    ws = workspace(lq.lq_moe_workspace_size(T, k, E))
    for per_slot in (1, 0):
        xrows = slice(None) if per_slot else slice(0, T * k, k)    # per token: rows 0, k, 2k, ...
        xq_use = xq if per_slot else np.ascontiguousarray(xq[xrows])
        xd_use = xd if per_slot else np.ascontiguousarray(xd[xrows])
        lq.lq_moe_q8_matvec_id(W, E, dev(xq_use), dev(xd_use), per_slot, dev(ids), T, k, y, ws, ws.numel())
        sync()
        got = host(y).reshape(T, k, rows)
        for t in range(T):
            for s in range(k):
                e = ids[t, s]
                xi = t * k + s if per_slot else t
                if 0 <= e < E:
                    ref = oracle.q8_matvec(wq[e], wd[e], xq_use[xi if per_slot else t], xd_use[xi if per_slot else t])
                    assert_close(got[t, s], ref, f"slot {t},{s}")
                else:
                    assert np.all(got[t, s] == 0)
        assert host(ws[:4].view(dtype=torch_mod().int32))[0] == 2     # invalid-id counter
    # weighted sum over slots, slots in order
    wts = synthetic.activations(r, T, k)
    out = empty((T, rows), np.float32)
    lq.lq_moe_weighted_sum(y, dev(wts), T, k, rows, out)
    sync()
    want = np.einsum("ts,tsr->tr", wts.astype(np.float64), host(y).reshape(T, k, rows).astype(np.float64))
    assert_close(host(out), want, "weighted sum")

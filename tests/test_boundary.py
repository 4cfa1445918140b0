"""The C-ABI boundary without a GPU.

* liblq.so loads and exports every function that include/lq.h declares,
  and the Python binding covers exactly those names.
* Argument validation runs on the host before any launch: every invalid
  call returns its documented status and touches no device (fake, aligned
  addresses are enough).  Zero-sized work returns LQ_OK with no launch.
* The host-only helpers (GGML block packing, RoPE tables) run here and are
  checked against numpy and the oracle.
"""
import ctypes as C
import math
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lq.h")

lq = pytest.importorskip("q8_matvec_gqa_amd")

A = 0x10000   # a fake, 256-byte aligned device address: validation never dereferences it.
# Every call below is invalid or empty, so none of them launches a kernel.
S0 = 0        # explicit null stream: no torch.cuda involvement


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(lq_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_symbols_exported():
    names = header_functions()
    assert len(names) >= 20, names
    lib = C.CDLL(lq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/lq.h but not exported"
    assert sorted(lq.exported_names()) == names


def test_status_strings():
    assert lq.lq_version() >= 1
    for s in range(7):
        assert lq.lq_status_string(s)
    assert lq.lq_status_string(99) == "unknown status"


def st(fn, *args, **kw):
    return fn(*args, stream=S0, check=False, **kw)


def test_quantize_validation():
    assert st(lq.lq_q8_quantize_act, A, 1, 33, A, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_q8_quantize_act, A, -1, 32, A, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_q8_quantize_act, None, 1, 32, A, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_q8_quantize_act, A + 4, 1, 32, A, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q8_quantize_act, A, 0, 32, None, None) == lq.LQ_OK        # empty: no launch
    assert st(lq.lq_rmsnorm_q8, A, 1, 64, A + 4, 1e-6, A, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_rmsnorm_q8, A, 1, 64, A, -1.0, A, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_swiglu_q8, A, 1, 48, A, A) == lq.LQ_ERR_SHAPE


def test_matvec_validation():
    w = lq.lq_q8_weight(A, A, 10, 64)
    assert st(lq.lq_q8_matvec, None, A, A, None, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_q8_matvec, lq.lq_q8_weight(A, A, 10, 48), A, A, None, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_q8_matvec, lq.lq_q8_weight(A + 8, A, 10, 64), A, A, None, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q8_matvec, w, A + 1, A, None, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q8_matvec, w, A, A, None, None) == lq.LQ_ERR_NULL
    assert st(lq.lq_q8_matvec, lq.lq_q8_weight(None, None, 0, 64), None, None, None, None) == lq.LQ_OK
    assert st(lq.lq_q8_block_dots, w, A, None) == lq.LQ_ERR_NULL
    f = lq.lq_q8_block_dots_f32
    assert st(f, w, A, 1, A, 1e-6, A, A, None) == lq.LQ_ERR_NULL
    assert st(f, w, A, 2, A, 1e-6, A, A, A) == lq.LQ_ERR_SHAPE
    assert st(f, w, A, 1, A, -1.0, A, A, A) == lq.LQ_ERR_SHAPE
    assert st(f, w, A + 4, 1, A, 1e-6, A, A, A) == lq.LQ_ERR_ALIGN
    assert st(f, w, A, 0, None, 0.0, A, A + 4, A) == lq.LQ_ERR_ALIGN
    assert st(f, lq.lq_q8_weight(A, A, 10, 16384 + 32), A, 0, None, 0.0, A, A, A) == lq.LQ_ERR_UNSUPPORTED
    assert st(f, lq.lq_q8_weight(None, None, 0, 64), None, 0, None, 0.0, None, None, None) == lq.LQ_OK


def test_ggml_format_validation():
    w4 = lq.lq_q4_0_weight(A, A, 10, 64)
    assert st(lq.lq_q4_0_matvec, None, A, A, None, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_q4_0_matvec, lq.lq_q4_0_weight(A, A, 10, 48), A, A, None, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_q4_0_matvec, lq.lq_q4_0_weight(A, A, 10, 16384 + 32), A, A, None, A) == lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_q4_0_matvec, lq.lq_q4_0_weight(A + 8, A, 10, 64), A, A, None, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q4_0_matvec, lq.lq_q4_0_weight(None, A, 10, 64), A, A, None, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_q4_0_matvec, w4, A + 1, A, None, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q4_0_matvec, w4, A, A, None, None) == lq.LQ_ERR_NULL
    assert st(lq.lq_q4_0_matvec, lq.lq_q4_0_weight(None, None, 0, 64), None, None, None, None) == lq.LQ_OK
    w6 = lq.lq_q6_k_weight(A, A, A, A, 10, 512)
    assert st(lq.lq_q6_k_matvec, lq.lq_q6_k_weight(A, A, A, A, 10, 384), A, A, None, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_q6_k_matvec, lq.lq_q6_k_weight(A, A, A, A, 10, 16384 + 256), A, A, None, A) == \
        lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_q6_k_matvec, lq.lq_q6_k_weight(A, A + 8, A, A, 10, 512), A, A, None, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q6_k_matvec, lq.lq_q6_k_weight(A, A, A + 4, A, 10, 512), A, A, None, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q6_k_matvec, lq.lq_q6_k_weight(A, A, None, A, 10, 512), A, A, None, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_q6_k_matvec, w6, A, None, None, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_q6_k_matvec, lq.lq_q6_k_weight(None, None, None, None, 0, 256), None, None, None, None) == \
        lq.LQ_OK


def test_attention_noalloc_validation():
    """The allocation-free attention validates like lq_gqa_decode_attn, and
    refuses shapes whose split partials exceed its 16 MiB array (the size
    query proves each refused shape needs more, so nothing can launch)."""
    f = lq.lq_gqa_decode_attn_noalloc
    assert st(f, A, 32, 8, 128, A, A, 1, 8192 * 128, 128, 8192, 0, 8192, 0.1, None) == lq.LQ_ERR_NULL
    assert st(f, A, 30, 8, 128, A, A, 1, 8192 * 128, 128, 8192, 0, 8192, 0.1, A) == lq.LQ_ERR_SHAPE
    assert st(f, A, 32, 8, 128, A, A, 1, 8192 * 128, 128, 8192, 100, 8192, 0.1, A) == lq.LQ_ERR_SHAPE
    assert st(f, A, 32, 8, 128, A + 8, A, 1, 8192 * 128, 128, 8192, 0, 8192, 0.1, A) == lq.LQ_ERR_ALIGN
    assert st(f, A, 32, 8, 1024, A, A, 1, 8192 * 1024, 1024, 8192, 0, 8192, 0.1, A) == lq.LQ_ERR_UNSUPPORTED
    assert st(f, None, 0, 8, 128, None, None, 1, 8192 * 128, 128, 8192, 0, 8192, 0.1, None) == lq.LQ_OK
    n_q, n_kv, hd, ctx = 511 * 8, 511, 512, 4096
    assert lq.lq_gqa_decode_attn_workspace_size(n_q, n_kv, hd, ctx) > 16 << 20
    assert st(f, A, n_q, n_kv, hd, A, A, 0, ctx * hd, hd, ctx, 0, ctx, 0.05, A) == lq.LQ_ERR_UNSUPPORTED
    assert "scratch" in lq.lq_last_error()
    # every shape of up to 510 kv heads fits
    worst = max(lq.lq_gqa_decode_attn_workspace_size(n * g, n, d, 65536)
                for n in (1, 2, 8, 64, 255, 256, 257, 500, 510) for g in (1, 2, 4, 8) for d in (64, 128, 256, 512))
    assert worst <= 16 << 20


def test_moe_ggml_format_validation():
    w4 = lq.lq_q4_0_weight(A, A, 64, 704)
    w6 = lq.lq_q6_k_weight(A, A, A, A, 64, 512)
    for fn, w in ((lq.lq_moe_q4_0_matvec_id, w4), (lq.lq_moe_q6_k_matvec_id, w6)):
        assert st(fn, None, 8, A, A, 0, A, 4, 2, A, A, 1 << 20) == lq.LQ_ERR_NULL
        assert st(fn, w, 0, A, A, 0, A, 4, 2, A, A, 1 << 20) == lq.LQ_ERR_UNSUPPORTED
        assert st(fn, w, 8, A, A, 2, A, 4, 2, A, A, 1 << 20) == lq.LQ_ERR_SHAPE
        assert st(fn, w, 8, A + 4, A, 0, A, 4, 2, A, A, 1 << 20) == lq.LQ_ERR_ALIGN
        assert st(fn, w, 8, A, A, 0, A, 4, 2, A, None, 0) == lq.LQ_ERR_WORKSPACE
        assert st(fn, w, 8, A, A, 0, A, 0, 2, A, None, 0) == lq.LQ_OK          # T == 0: no launch
    assert st(lq.lq_moe_q4_0_matvec_id, lq.lq_q4_0_weight(A, A, 64, 48), 8, A, A, 0, A, 4, 2, A, A, 1 << 20) == \
        lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_q6_k_matvec_id, lq.lq_q6_k_weight(A, A, A, A, 64, 704), 8, A, A, 0, A, 4, 2, A, A,
              1 << 20) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_q6_k_matvec_id, lq.lq_q6_k_weight(A, A, A, A, 64, 8192 + 256), 8, A, A, 0, A, 4, 2, A, A,
              1 << 20) == lq.LQ_ERR_UNSUPPORTED


def test_ggml_format_pack_host():
    """The pack helpers move every GGML block field to its SoA array (host
    memory only), and reject bad shapes."""
    import synthetic
    rng = np.random.default_rng(9)
    rows, cols = 5, 512
    b4 = synthetic.q4_0_blocks(rng, rows, cols)
    qs = np.zeros((rows, cols // 2), np.uint8)
    d = np.zeros((rows, cols // 32), np.uint16)
    lq.lq_q4_0_pack_ggml(b4, rows, cols, qs, d)
    assert np.array_equal(qs.reshape(rows, cols // 32, 16), b4[..., 2:])
    assert np.array_equal(d, b4[..., 0].astype(np.uint16) | (b4[..., 1].astype(np.uint16) << 8))
    b6 = synthetic.q6_k_blocks(rng, rows, cols)
    ql = np.zeros((rows, cols // 2), np.uint8)
    qh = np.zeros((rows, cols // 4), np.uint8)
    sc = np.zeros((rows, cols // 16), np.int8)
    d6 = np.zeros((rows, cols // 256), np.uint16)
    lq.lq_q6_k_pack_ggml(b6, rows, cols, ql, qh, sc, d6)
    assert np.array_equal(ql.reshape(rows, cols // 256, 128), b6[..., :128])
    assert np.array_equal(qh.reshape(rows, cols // 256, 64), b6[..., 128:192])
    assert np.array_equal(sc.view(np.uint8).reshape(rows, cols // 256, 16), b6[..., 192:208])
    assert np.array_equal(d6, b6[..., 208].astype(np.uint16) | (b6[..., 209].astype(np.uint16) << 8))
    assert lq.lq_q4_0_pack_ggml(b4, rows, 48, qs, d, check=False) == lq.LQ_ERR_SHAPE
    assert lq.lq_q6_k_pack_ggml(b6, rows, 384, ql, qh, sc, d6, check=False) == lq.LQ_ERR_SHAPE
    assert lq.lq_q6_k_pack_ggml(None, rows, 512, ql, qh, sc, d6, check=False) == lq.LQ_ERR_NULL


def test_matmul_validation_and_workspace():
    w = lq.lq_q8_weight(A, A, 4096, 4096)
    need = lq.lq_q8_matmul_workspace_size(4096, 4096, 32)
    # a short weight splits its blocks: one f32 partial tile per split, reused per 32-token chunk
    assert need > 0 and need % (32 * 4096 * 4) == 0
    assert lq.lq_q8_matmul_workspace_size(4096, 4096, 33) == 0         # > 32 tokens: chunks fill the grid
    assert lq.lq_q8_matmul_workspace_size(24576, 4096, 32) == 0       # enough row tiles: no split
    assert lq.lq_q8_matmul_workspace_size(4096, 4096, 0) == 0
    assert lq.lq_q8_matmul_workspace_size(4096, 48, 8) == 0
    assert st(lq.lq_q8_matmul, w, A, A, -1, None, A, A, need) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_q8_matmul, w, A, A, 1 << 31, None, A, A, need) == lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_q8_matmul, lq.lq_q8_weight(A, A, 10, 32 * 513), A, A, 4, None, A, A, 1 << 20) == \
        lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_q8_matmul, w, None, A, 4, None, A, A, need) == lq.LQ_ERR_NULL
    assert st(lq.lq_q8_matmul, w, A + 4, A, 4, None, A, A, need) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_q8_matmul, w, A, A, 4, None, A, None, need) == lq.LQ_ERR_WORKSPACE
    assert st(lq.lq_q8_matmul, w, A, A, 4, None, A, A, need - 4) == lq.LQ_ERR_WORKSPACE
    assert st(lq.lq_q8_matmul, w, None, None, 0, None, None, None, 0) == lq.LQ_OK     # T == 0: no launch


def test_lm_head_validation():
    assert st(lq.lq_lm_head_f16, A, 10, 36, A, 1, A, 1e-6, 0.0, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_lm_head_f16, A, 10, 8192, A, 1, A, 1e-6, 0.0, A) == lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_lm_head_f16, None, 10, 64, A, 1, A, 1e-6, 0.0, A) == lq.LQ_ERR_NULL
    assert st(lq.lq_lm_head_f16, A + 4, 10, 64, A, 1, A, 1e-6, 0.0, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_lm_head_f16, A, 10, 64, A, 1, A + 8, 1e-6, 0.0, A) == lq.LQ_ERR_ALIGN
    assert st(lq.lq_lm_head_f16, None, 0, 64, None, 1, None, 1e-6, 0.0, None) == lq.LQ_OK   # empty: no launch


def test_norm_rope_kv_validation():
    assert st(lq.lq_rmsnorm_rope, A, 4, 63, 63, None, 1e-6, None, None, 0, 0) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_rmsnorm_rope, A, 4, 1024, 1024, None, 1e-6, None, None, 0, 0) == lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_rmsnorm_rope, A, 4, 64, 32, None, 1e-6, None, None, 0, 0) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_rmsnorm_rope, A, 4, 64, 64, None, 1e-6, A, None, 10, 0) == lq.LQ_ERR_NULL
    assert st(lq.lq_rmsnorm_rope, A, 4, 64, 64, None, 1e-6, A, A, 10, 10) == lq.LQ_ERR_SHAPE   # pos past the table
    assert st(lq.lq_rmsnorm_rope, A, 0, 64, 64, None, 1e-6, None, None, 0, 0) == lq.LQ_OK
    assert st(lq.lq_kv_append, A, A, 2, 64, A, A, 7, 64 * 8, 64, 8, 0) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_kv_append, A, A, 2, 64, A, A, 1, 64 * 8, 32, 8, 0) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_kv_append, A, A, 2, 64, A, A, 1, 64 * 8, 64, 8, 8) == lq.LQ_ERR_SHAPE     # pos past the cache


def test_attention_validation():
    def call(n_q=8, n_kv=2, hd=64, dtype=1, hs=64 * 100, ps=64, max_ctx=100, start=0, length=100,
             ws=A, wsb=1 << 20):
        return st(lq.lq_gqa_decode_attn, A, n_q, n_kv, hd, A, A, dtype, hs, ps, max_ctx, start, length,
                  0.125, A, ws, wsb)
    assert call(n_q=7) == lq.LQ_ERR_SHAPE                      # INV-3
    assert call(hd=66, ps=66, hs=6600) == lq.LQ_ERR_SHAPE      # INV-2
    assert call(start=50, length=51) == lq.LQ_ERR_SHAPE        # window past the allocation
    assert call(start=-1, length=10) == lq.LQ_ERR_SHAPE
    assert call(hd=1024, ps=1024, hs=102400) == lq.LQ_ERR_UNSUPPORTED
    assert call(n_q=18, n_kv=2) == lq.LQ_ERR_UNSUPPORTED       # G = 9
    assert call(hd=68, ps=68, hs=6800) == lq.LQ_ERR_UNSUPPORTED   # bf16 needs head_dim % 8
    assert call(ps=60) == lq.LQ_ERR_SHAPE
    assert call(dtype=1, ps=68, hs=6800) == lq.LQ_ERR_ALIGN    # 136-byte rows are not 16-byte multiples
    need = lq.lq_gqa_decode_attn_workspace_size(32, 8, 128, 8192)
    assert need > 0
    assert st(lq.lq_gqa_decode_attn, A, 32, 8, 128, A, A, 1, 128 * 8192, 128, 8192, 0, 8192, 0.1, A,
              A, need - 1) == lq.LQ_ERR_WORKSPACE
    assert st(lq.lq_gqa_decode_attn, A, 32, 8, 128, A, A, 1, 128 * 8192, 128, 8192, 0, 8192, 0.1, A,
              None, need) == lq.LQ_ERR_WORKSPACE
    # workspace need grows with the attended length (the layer sizes it for the longest window)
    sizes = [lq.lq_gqa_decode_attn_workspace_size(32, 8, 128, n) for n in (1, 64, 1000, 4096, 8192, 65536)]
    assert sizes == sorted(sizes)


def test_moe_validation():
    w = lq.lq_q8_weight(A, A, 1408, 2816)
    wsb = lq.lq_moe_workspace_size(16, 8, 128)
    assert wsb > 0
    assert st(lq.lq_moe_route_topk, A, 16, 128, 0, A, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_route_topk, A, 16, 128, 129, A, A) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_route_topk, A, 16, 2048, 8, A, A) == lq.LQ_ERR_UNSUPPORTED
    assert st(lq.lq_moe_q8_matvec_id, w, 128, A, A, 2, A, 16, 8, A, A, wsb) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_q8_matvec_id, w, 128, A, A, 0, A, 16, 8, A, A, wsb - 4) == lq.LQ_ERR_WORKSPACE
    assert st(lq.lq_moe_q8_matvec_id, w, 0, A, A, 0, A, 16, 8, A, A, wsb) == lq.LQ_ERR_UNSUPPORTED
    d = lq.lq_moe_desc(2816, 704, 128, 8, lq.lq_q8_weight(A, A, 1408, 2816), lq.lq_q8_weight(A, A, 2816, 704))
    need = lq.lq_moe_block_workspace_size(d, 16)
    assert need > 0
    assert st(lq.lq_moe_block, d, A, A, 16, A, None, A, need - 1) == lq.LQ_ERR_WORKSPACE
    bad = lq.lq_moe_desc(2816, 704, 128, 8, lq.lq_q8_weight(A, A, 1400, 2816), lq.lq_q8_weight(A, A, 2816, 704))
    assert st(lq.lq_moe_block, bad, A, A, 16, A, None, A, need) == lq.LQ_ERR_SHAPE


def test_moe_block_ggml_validation():
    H, I, E, k = 2816, 704, 128, 8
    gu6, dn4 = lq.lq_q6_k_weight(A, A, A, A, 2 * I, H), lq.lq_q4_0_weight(A, A, H, I)

    def desc(gf=lq.LQ_FMT_Q6_K, df=lq.LQ_FMT_Q4_0, gu=gu6, dn=dn4, dn6=lq.lq_q6_k_weight()):
        return lq.lq_moe_ggml_desc(H, I, E, k, gf, df, gate_up_q6_k=gu, down_q4_0=dn, down_q6_k=dn6)

    d = desc()
    need = lq.lq_moe_block_ggml_workspace_size(d, 16)
    assert need == lq.lq_moe_block_workspace_size(
        lq.lq_moe_desc(H, I, E, k, lq.lq_q8_weight(A, A, 2 * I, H), lq.lq_q8_weight(A, A, H, I)), 16)
    assert st(lq.lq_moe_block_ggml, None, A, A, 16, A, None, A, need) == lq.LQ_ERR_NULL
    assert st(lq.lq_moe_block_ggml, d, A, A, 16, A, None, A, need - 1) == lq.LQ_ERR_WORKSPACE
    assert st(lq.lq_moe_block_ggml, d, A, A, 0, A, None, A, need) == lq.LQ_OK          # T == 0: no launch
    assert st(lq.lq_moe_block_ggml, desc(gf=7), A, A, 16, A, None, A, need) == lq.LQ_ERR_SHAPE
    # Q6_K down would need ffn % 256 == 0 (704 is not); a wrong row count
    assert st(lq.lq_moe_block_ggml, desc(df=lq.LQ_FMT_Q6_K, dn6=lq.lq_q6_k_weight(A, A, A, A, H, I)), A, A, 16, A,
              None, A, need) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_block_ggml, desc(gu=lq.lq_q6_k_weight(A, A, A, A, 2 * I - 1, H)), A, A, 16, A, None, A,
              need) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_moe_block_ggml, desc(dn=lq.lq_q4_0_weight(A + 4, A, H, I)), A, A, 16, A, None, A,
              need) == lq.LQ_ERR_ALIGN
    # the router holds at most 1024 logits per token, as in lq_moe_block
    big = lq.lq_moe_ggml_desc(H, I, 1025, k, lq.LQ_FMT_Q6_K, lq.LQ_FMT_Q4_0, gate_up_q6_k=gu6, down_q4_0=dn4)
    nbig = lq.lq_moe_block_ggml_workspace_size(big, 16)
    assert st(lq.lq_moe_block_ggml, big, A, A, 16, A, None, A, nbig) == lq.LQ_ERR_UNSUPPORTED


def _layer_desc(**over):
    H, nq, nkv, hd, I, ctx = 4096, 32, 8, 128, 12288, 8192
    d = lq.lq_layer_desc(
        hidden=H, n_q=nq, n_kv=nkv, head_dim=hd, ffn=I, max_ctx=ctx, window=0, eps=1e-6,
        attn_scale=1 / math.sqrt(hd), kind=0, kv_dtype=1, qk_norm=1, v_unit_norm=0,
        w_qkv=lq.lq_q8_weight(A, A, nq * hd + 2 * nkv * hd, H), w_o=lq.lq_q8_weight(A, A, H, nq * hd),
        w_gate_up=lq.lq_q8_weight(A, A, 2 * I, H), w_down=lq.lq_q8_weight(A, A, H, I),
        g_in=A, g_q=A, g_k=A, g_post=A, k_cache=A, v_cache=A, rope_cos=A, rope_sin=A)
    for k, v in over.items():
        setattr(d, k, v)
    return d


def test_layer_validation():
    d = _layer_desc()
    need = lq.lq_decode_layer_workspace_size(d)
    assert need > 0
    call = lambda desc, pos=8191, wsb=need, ws=A: st(lq.lq_decode_layer, desc, A, pos, None, ws, wsb)
    assert call(d, wsb=need - 1) == lq.LQ_ERR_WORKSPACE
    assert call(d, ws=A + 16) == lq.LQ_ERR_WORKSPACE          # workspace must be 256-byte aligned
    assert call(d, pos=8192) == lq.LQ_ERR_SHAPE
    assert call(_layer_desc(n_q=30)) == lq.LQ_ERR_SHAPE       # 30 % 8
    assert call(_layer_desc(kind=5)) == lq.LQ_ERR_SHAPE
    assert call(_layer_desc(w_o=lq.lq_q8_weight(A, A, 4096, 4000))) == lq.LQ_ERR_SHAPE
    assert call(_layer_desc(ffn=12300)) == lq.LQ_ERR_SHAPE
    assert call(_layer_desc(g_in=None)) == lq.LQ_ERR_NULL
    assert call(_layer_desc(rope_cos=None)) == lq.LQ_ERR_NULL
    assert call(_layer_desc(k_cache=A + 2)) == lq.LQ_ERR_ALIGN
    assert call(_layer_desc(window=-1)) == lq.LQ_ERR_SHAPE
    assert lq.lq_decode_layer_workspace_size(None) == 0
    n = lq.lq_decode_layer_kernel_count(d)
    assert n == 6                                            # QKV, attention split + combine, O, gate_up, down
    assert st(lq.lq_decode_layer_timed, d, A, 8191, None, A, need, [A] * (2 * n - 1)) == lq.LQ_ERR_SHAPE
    assert st(lq.lq_decode_layer_timed, d, A, 8192, None, A, need, [A] * (2 * n)) == lq.LQ_ERR_SHAPE


def test_layer_workspace_covers_shorter_contexts():
    """The decode layer sizes its attention partials for its longest
    attention (max_ctx, or the window) and runs every shorter one in the same
    region, so the workspace must never shrink as max_ctx grows: a shorter
    attention can plan more splits than a longer one after the whole-tile
    rounding (8192 positions: 64 splits per kv head; 8193: 43)."""
    prev = 0
    for ctx in list(range(8150, 8260)) + [16384, 16385, 65536, 65537]:
        n = lq.lq_decode_layer_workspace_size(_layer_desc(max_ctx=ctx))
        assert n >= prev, (ctx, n, prev)
        prev = n


def test_layer_ggml_format_validation():
    """Projections in GGML formats (lq_layer_desc.w_format): the chosen
    descriptor's shape, pointers and alignment are checked before any launch."""
    H, nq, nkv, hd, I = 4096, 32, 8, 128, 12288
    d = _layer_desc()
    need = lq.lq_decode_layer_workspace_size(d)
    call = lambda desc: st(lq.lq_decode_layer, desc, A, 8191, None, A, need)

    def with_formats(fmts, q4=None, q6=None):
        desc = _layer_desc()
        for i, f in enumerate(fmts):
            desc.w_format[i] = f
        for i, w in (q4 or {}).items():
            desc.w_q4_0[i] = w
        for i, w in (q6 or {}).items():
            desc.w_q6_k[i] = w
        return desc

    Q8, Q4, Q6 = lq.LQ_FMT_Q8_0, lq.LQ_FMT_Q4_0, lq.LQ_FMT_Q6_K
    good_q6_gu = lq.lq_q6_k_weight(A, A, A, A, 2 * I, H)
    good_q4_dn = lq.lq_q4_0_weight(A, A, H, I)
    assert call(with_formats([Q8, Q8, 7, Q8])) == lq.LQ_ERR_SHAPE                           # unknown format
    assert call(with_formats([Q8, Q8, Q6, Q4])) == lq.LQ_ERR_SHAPE                          # descriptors left empty
    assert call(with_formats([Q8, Q8, Q6, Q4], q4={3: lq.lq_q4_0_weight(A, A, H, I + 32)},
                             q6={2: good_q6_gu})) == lq.LQ_ERR_SHAPE                         # wrong cols
    assert call(with_formats([Q8, Q8, Q6, Q4], q4={3: lq.lq_q4_0_weight(None, A, H, I)},
                             q6={2: good_q6_gu})) == lq.LQ_ERR_NULL
    assert call(with_formats([Q8, Q8, Q6, Q4], q4={3: good_q4_dn},
                             q6={2: lq.lq_q6_k_weight(A, A, A + 4, A, 2 * I, H)})) == lq.LQ_ERR_ALIGN
    assert call(with_formats([Q8, Q6, Q8, Q8], q6={1: lq.lq_q6_k_weight(A, A, A, A, H, 4000)})) == lq.LQ_ERR_SHAPE
    # a Q6_K QKV needs cols % 256 == 0
    d6 = _layer_desc(hidden=4000, w_qkv=lq.lq_q8_weight(A, A, nq * hd + 2 * nkv * hd, 4000),
                     w_o=lq.lq_q8_weight(A, A, 4000, nq * hd), w_gate_up=lq.lq_q8_weight(A, A, 2 * I, 4000),
                     w_down=lq.lq_q8_weight(A, A, 4000, I))
    d6.w_format[0] = Q6
    d6.w_q6_k[0] = lq.lq_q6_k_weight(A, A, A, A, nq * hd + 2 * nkv * hd, 4000)
    assert call(d6) == lq.LQ_ERR_SHAPE
    # a Q6_K gate_up over more than 12288 columns is refused up front
    big = _layer_desc(hidden=16384, w_qkv=lq.lq_q8_weight(A, A, nq * hd + 2 * nkv * hd, 16384),
                      w_o=lq.lq_q8_weight(A, A, 16384, nq * hd), w_down=lq.lq_q8_weight(A, A, 16384, I))
    big.w_format[2] = Q6
    big.w_q6_k[2] = lq.lq_q6_k_weight(A, A, A, A, 2 * I, 16384)
    assert st(lq.lq_decode_layer, big, A, 8191, None, A, lq.lq_decode_layer_workspace_size(big)) == \
        lq.LQ_ERR_UNSUPPORTED


def test_pack_ggml_host():
    rng = np.random.default_rng(0)
    rows, cols = 5, 96
    qs = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    d = rng.integers(0, 1 << 16, size=(rows, cols // 32), dtype=np.uint16)
    blocks = np.zeros((rows * cols // 32, 34), dtype=np.uint8)
    blocks[:, 0:2] = d.reshape(-1, 1).view(np.uint8).reshape(-1, 2)   # little-endian f16 scale
    blocks[:, 2:] = qs.reshape(-1, 32).view(np.uint8)
    out_qs = np.zeros_like(qs)
    out_d = np.zeros_like(d)
    lq.lq_q8_pack_ggml(blocks, rows, cols, out_qs, out_d)
    assert np.array_equal(out_qs, qs) and np.array_equal(out_d, d)
    assert lq.lq_q8_pack_ggml(blocks, rows, 33, out_qs, out_d, check=False) == lq.LQ_ERR_SHAPE


@pytest.mark.parametrize("hd", [64, 80, 128, 256, 512])
def test_rope_table_host(hd):
    ctx, theta = 8192, 1e6
    c = np.zeros((ctx, hd // 2), np.float32)
    s = np.zeros((ctx, hd // 2), np.float32)
    lq.lq_rope_table(ctx, hd, theta, c, s)
    oc, os_ = oracle.rope_table(ctx, hd, theta)
    # the two tables are independent double-precision evaluations rounded to
    # float; they may differ in the last float bit
    assert np.abs(c.astype(np.float64) - oc).max() <= 2 ** -23
    assert np.abs(s.astype(np.float64) - os_).max() <= 2 ** -23
    assert lq.lq_rope_table(ctx, 63, theta, c, s, check=False) == lq.LQ_ERR_SHAPE


def test_rope_table_freqs_host():
    """The frequency-factor table (host helper) against the oracle's, with a
    mask that leaves the upper pairs unrotated."""
    ctx, hd, theta = 4096, 512, 1e6
    f = np.ones(hd // 2, np.float32)
    f[64:] = np.inf
    f[10] = 4.0
    c = np.zeros((ctx, hd // 2), np.float32)
    s = np.zeros((ctx, hd // 2), np.float32)
    lq.lq_rope_table_freqs(ctx, hd, theta, f, c, s)
    oc, os_ = oracle.rope_table_freqs(ctx, hd, theta, f)
    assert np.abs(c.astype(np.float64) - oc).max() <= 2 ** -23
    assert np.abs(s.astype(np.float64) - os_).max() <= 2 ** -23
    assert np.all(c[:, 64:] == 1.0) and np.all(s[:, 64:] == 0.0)
    bad = f.copy()
    bad[3] = 0.0
    assert lq.lq_rope_table_freqs(ctx, hd, theta, bad, c, s, check=False) == lq.LQ_ERR_SHAPE

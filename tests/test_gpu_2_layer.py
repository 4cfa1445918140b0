"""Decode-layer and MoE-block parity: the whole path through lq_decode_layer /
lq_moe_block on every workload at full size.

Teacher-forced: every stage of the oracle is fed the GPU's own input to that
stage (read back from the tap buffers) and must match the GPU's output of the
stage (bit-exact for Q8_0 of an identical float input; the near-boundary rule
for Q8_0 of a recomputed float; 1e-3 / 1e-4 for floats).  The KV append is
checked byte for byte (tests/layercheck.py: check_kv_row).  Free-running: the
oracle's whole layer from the original inputs, carrying the GPU's discrete
values forward only at counted, checked rounding-boundary flips
(layercheck.free_running), must match the GPU's layer output to the float
tolerance; with no flip at all, so must the oracle's own composed layer
(orc_decode_layer).
"""
import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

lq = pytest.importorskip("q8_matvec_gqa_amd")
from q8_matvec_gqa_amd.layers import DeviceLayer, DeviceMoe  # noqa: E402
from lqtest import assert_close, assert_q8_near, dev, host, sync, torch_mod  # noqa: E402
from layercheck import check_kv_row, free_running, post_rope, proj_matvec  # noqa: E402

LAYERS = list(synthetic.WORKLOADS)


def oracle_cfg(cfg):
    return dict(cfg)


@pytest.mark.parametrize("name", LAYERS)
def test_layer_teacher_forced(name):
    run_teacher_forced(name)


# the Gemma fidelity options: GeGLU gate (tanh GELU) and the attention score softcap
@pytest.mark.parametrize("name,act,cap", [
    ("tiny_h1024", 1, 0.0),
    ("qwen3_4b_like_h2560", 1, 1.5),
    ("gemma4_sliding_h2816", 0, 1.5),
    ("gemma4_global_h2816", 0, 3.0),
])
def test_layer_variants_teacher_forced(name, act, cap):
    run_teacher_forced(name, act, cap)


def test_layer_rope_freqs_teacher_forced():
    """Gemma global layer with a RoPE frequency mask: the first 64 of the 256
    pairs rotate (one at a quarter of its frequency), the rest do not."""
    f = np.ones(256, np.float32)
    f[64:] = np.inf
    f[7] = 4.0
    run_teacher_forced("gemma4_global_h2816", freqs=f)


# GGML weight formats in the layer ("Current Inference Path -- Architecture Map",
# section 4: the current path runs GGML Q6_K weights): the 8B-like layer with
# a Q6_K gate_up and a Q4_0 down, every projection Q4_0, the other pairing,
# and the Gemma block with Q6_K QKV and Q4_0 O
@pytest.mark.parametrize("name,formats", [
    ("qwen3_8b_like_h4096", {"gu": "q6_k", "dn": "q4_0"}),
    ("qwen3_4b_like_h2560", {"qkv": "q4_0", "o": "q4_0", "gu": "q4_0", "dn": "q4_0"}),
    ("tiny_h1024", {"qkv": "q6_k", "o": "q6_k", "gu": "q4_0", "dn": "q6_k"}),
    ("gemma4_sliding_h2816", {"qkv": "q6_k", "o": "q4_0"}),
], ids=["8b-gu_q6k-dn_q40", "4b-all_q40", "tiny-mixed", "gemma_sliding-q6k_q40"])
def test_layer_ggml_formats_teacher_forced(name, formats):
    run_teacher_forced(name, formats=formats)


@pytest.mark.parametrize("fmt", ["q6_k", "q4_0"])
def test_layer_ggml_wide_rows(fmt, monkeypatch):
    """Every projection in one GGML format on 6144-wide rows: two 64-unit
    steps per Q6_K row (QKV, and gate_up through the SwiGLU + Q8_0 epilogue)
    and three per Q4_0 row, which no workload shape reaches."""
    cfg = dict(synthetic.WORKLOADS["qwen3_8b_like_h4096"], hidden=6144, ffn=2048, ctx=256)
    monkeypatch.setitem(synthetic.WORKLOADS, "wide_h6144", cfg)
    run_teacher_forced("wide_h6144", formats={"qkv": fmt, "o": fmt, "gu": fmt, "dn": fmt})


def run_teacher_forced(name, act=0, cap=0.0, freqs=None, formats=None):
    torch = torch_mod()
    cfg, w = synthetic.layer_inputs(name, seed=0, formats=formats)
    cfg = dict(cfg, ffn_act=act, attn_softcap=cap, rope_freqs=freqs)
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    pos, kind = cfg["pos"], cfg["kind"]
    qd, kvd = nq * hd, nkv * hd
    print(f"[layer] {name} pos={pos} act={act} softcap={cap} formats={formats}", flush=True)
    L = DeviceLayer(cfg, w, torch)
    taps, bufs = L.make_taps()
    x = dev(w["x"])
    L.run(x, pos, taps)
    sync()
    T = {k: host(v) for k, v in bufs.items()}
    for k in ("xd", "ad", "nd", "hd"):
        if k in T:
            T[k] = T[k].view(np.uint16)
    kv_np = np.float32 if cfg["kv_dtype"] == 0 else np.uint16
    kc_gpu = host(L.t["k_cache"], kv_np)
    vc_gpu = host(L.t["v_cache"], kv_np)
    out_gpu = host(x)
    if freqs is None:
        oc, os_ = oracle.rope_table(cfg["max_ctx"], hd, cfg["theta"])
    else:
        oc, os_ = oracle.rope_table_freqs(cfg["max_ctx"], hd, cfg["theta"], freqs)
    eps = cfg["eps"]
    flips = 0

    # 1. input norm + quantize
    flips += assert_q8_near(T["xq"], T["xd"], oracle.rmsnorm(w["x"], w["g_in"], eps), "input norm Q8")
    # 2. raw QKV projection from the GPU's Q8 input
    assert_close(T["qkv"], proj_matvec(w, "qkv", T["xq"], T["xd"]), "qkv projection")
    # per-head norms and RoPE of the GPU's raw projection (the oracle's steps),
    # against the attention prologue's own f32 results
    post = post_rope(cfg, T["qkv"], w["g_q"], w["g_k"], oc[pos], os_[pos])
    assert_close(T["qkv_post"][:qd], post[:qd], "q after norm and RoPE")
    # 3. KV append, byte for byte: the row at pos is exactly cvt() of the
    # prologue's k and v, which meet the tolerance against the oracle's; any
    # code differing from cvt() of the oracle's value is a checked bf16 flip
    flips += check_kv_row(kc_gpu[:, pos], T["qkv_post"][qd:qd + kvd], post[qd:qd + kvd], cfg["kv_dtype"],
                          "k appended")
    flips += check_kv_row(vc_gpu[:, pos], T["qkv_post"][qd + kvd:], post[qd + kvd:], cfg["kv_dtype"],
                          "v appended")
    others = np.ones(cfg["max_ctx"], bool)
    others[pos] = False
    assert np.array_equal(kc_gpu[:, others], w["k_cache"][:, others])
    assert np.array_equal(vc_gpu[:, others], w["v_cache"][:, others])
    # 4. attention from the oracle's q (of the GPU's projection) and the GPU's caches
    start = max(0, pos - cfg["window"] + 1) if cfg["window"] else 0
    att = oracle.attention(post[:qd], nq, nkv, hd, kc_gpu, vc_gpu, cfg["kv_dtype"],
                           cfg["max_ctx"] * hd, hd, start, pos - start + 1, cfg["attn_scale"], softcap=cap)
    assert_close(T["attn"], att, "attention")
    # 5. quantize of the attention output: identical float input -> bit-exact
    aq, ad = oracle.q8_quantize(T["attn"])
    assert np.array_equal(T["aq"], aq) and np.array_equal(T["ad"], ad)
    # 6. O projection (+ residual for the pre-norm layer)
    if kind == 0:
        assert_close(T["x1"], proj_matvec(w, "o", T["aq"], T["ad"], residual=w["x"]), "x1")
        flips += assert_q8_near(T["nq"], T["nd"], oracle.rmsnorm(T["x1"], w["g_post"], eps), "post norm Q8")
        gu = proj_matvec(w, "gu", T["nq"], T["nd"])
        gate = oracle.gelu_mul if act == 1 else oracle.silu_mul
        assert_close(T["h"], gate(gu[:I], gu[I:]), "act(gate) * up")
        hq, hd_ = oracle.q8_quantize(T["h"])                 # identical float input -> bit-exact
        assert np.array_equal(T["hq"], hq) and np.array_equal(T["hd"], hd_)
        assert_close(out_gpu, proj_matvec(w, "dn", T["hq"], T["hd"], residual=T["x1"]),
                     "layer output")
    else:
        assert_close(T["x1"], proj_matvec(w, "o", T["aq"], T["ad"]), "o projection")
        n = oracle.rmsnorm(T["x1"], w["g_post"], eps)
        assert_close(out_gpu, (w["x"].astype(np.float64) + n).astype(np.float32), "block output")

    # free-running: the oracle's layer from the original inputs, the GPU's
    # discrete values carried forward only at checked boundary flips
    ref_fr, fr_flips = free_running(cfg, w, T, kc_gpu, vc_gpu, oc, os_, name)
    err = assert_close(out_gpu, ref_fr, "free-running layer output")
    n_fr = sum(fr_flips.values())
    if n_fr == 0 and not formats:
        # the oracle's own composed layer (Q8_0 weights only)
        ow = dict(w)
        ow["rope_cos"], ow["rope_sin"] = oc, os_
        ref_out, _, _, _ = oracle.decode_layer(oracle_cfg(cfg), ow, w["x"], pos, w["k_cache"], w["v_cache"])
        assert_close(out_gpu, ref_out, "free-running layer output (orc_decode_layer)")
    print(f"[layer] {name}: free-running max rel err {err:.2e}; flips carried forward {fr_flips}; "
          f"teacher-forced flips {flips}", flush=True)


def test_layer_deterministic_and_repeatable():
    """Same inputs twice -> bit-identical outputs and caches (the only race
    detector available: any unsynchronized read-after-write would show)."""
    torch = torch_mod()
    cfg, w = synthetic.layer_inputs(synthetic.HEADLINE, seed=1)
    L = DeviceLayer(cfg, w, torch)
    outs = []
    for _ in range(2):
        L.t["k_cache"].copy_(dev(w["k_cache"]))
        L.t["v_cache"].copy_(dev(w["v_cache"]))
        x = dev(w["x"])
        L.run(x, cfg["pos"])
        sync()
        outs.append((host(x), host(L.t["k_cache"]).copy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


def test_layer_timed_matches():
    """The measurement entry point runs the same kernels: identical outputs."""
    torch = torch_mod()
    cfg, w = synthetic.layer_inputs("qwen3_4b_like_h2560", seed=3)
    L = DeviceLayer(cfg, w, torch)
    n = lq.lq_decode_layer_kernel_count(L.desc)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for e in evs:
        e.record()
    outs = []
    for timed in (False, True):
        L.t["k_cache"].copy_(dev(w["k_cache"]))
        L.t["v_cache"].copy_(dev(w["v_cache"]))
        x = dev(w["x"])
        if timed:
            lq.lq_decode_layer_timed(L.desc, x, cfg["pos"], None, L.ws, L.ws_bytes, evs)
        else:
            L.run(x, cfg["pos"])
        sync()
        outs.append(host(x))
    assert np.array_equal(outs[0], outs[1])
    ts = [evs[2 * k].elapsed_time(evs[2 * k + 1]) for k in range(n)]
    assert all(t > 0 for t in ts), ts


@pytest.mark.parametrize("name,pos", [("gemma4_sliding_h2816", p) for p in (0, 1, 63, 64, 1023, 1024, 5000)]
                         + [("gemma4_global_h2816", p) for p in (0, 1, 15, 16, 17, 100, 2000)])
def test_layer_positions(name, pos):
    """Early positions (window not full yet, start 0) and late ones (start > 0)
    of the sliding-window block, and early and late positions of the
    full-context block (the new row at different places of its tile and
    split), against the free-running oracle."""
    torch = torch_mod()
    cfg, w = synthetic.layer_inputs(name, seed=2)
    L = DeviceLayer(cfg, w, torch)
    taps, bufs = L.make_taps()
    x = dev(w["x"])
    L.run(x, pos, taps)
    sync()
    hd, nq, nkv = cfg["head_dim"], cfg["n_q"], cfg["n_kv"]
    oc, os_ = oracle.rope_table(cfg["max_ctx"], hd, cfg["theta"])
    kc_gpu = host(L.t["k_cache"], np.uint16)
    vc_gpu = host(L.t["v_cache"], np.uint16)
    qkv = host(bufs["qkv"])
    post = post_rope(dict(cfg, pos=pos), qkv, w["g_q"], w["g_k"], oc[pos], os_[pos])
    q = post[:nq * hd]
    kvd, tap = nkv * hd, host(bufs["qkv_post"])
    check_kv_row(kc_gpu[:, pos], tap[nq * hd:nq * hd + kvd], post[nq * hd:nq * hd + kvd], 1, f"k at pos {pos}")
    check_kv_row(vc_gpu[:, pos], tap[nq * hd + kvd:], post[nq * hd + kvd:], 1, f"v at pos {pos}")
    start = max(0, pos - cfg["window"] + 1) if cfg["window"] else 0
    att = oracle.attention(q, nq, nkv, hd, kc_gpu, vc_gpu, 1, cfg["max_ctx"] * hd, hd, start,
                           pos - start + 1, cfg["attn_scale"])
    assert_close(host(bufs["attn"]), att, f"{name}: attention at pos {pos}")


def test_layer_workspace_serves_shorter_attention():
    """A layer sized for its longest attention (max_ctx 8193: 33 splits per
    kv head after the whole-tile rounding) running a shorter one (8192
    positions: 64 splits): the partials fit the workspace, nothing past it is
    written (a guard region keeps its bytes), and the attention matches the
    oracle."""
    torch = torch_mod()
    cfg, w = synthetic.layer_inputs("tiny_h1024", seed=5)
    hd, nq, nkv, M, pos = cfg["head_dim"], cfg["n_q"], cfg["n_kv"], 8193, 8191
    r = np.random.Generator(np.random.PCG64(8193))
    cfg = dict(cfg, max_ctx=M)
    w = dict(w, k_cache=synthetic.kv_cache(r, nkv, M, hd, 0), v_cache=synthetic.kv_cache(r, nkv, M, hd, 0))
    print(f"[ws] tiny_h1024 with max_ctx {M} at pos {pos}", flush=True)
    L = DeviceLayer(cfg, w, torch)
    guard = 1 << 20
    buf = torch.full((L.ws_bytes + guard,), 0xA5, dtype=torch.uint8, device="cuda")
    L.ws = buf[:L.ws_bytes]
    taps, bufs = L.make_taps()
    x = dev(w["x"])
    L.run(x, pos, taps)
    sync()
    assert bool((buf[L.ws_bytes:] == 0xA5).all()), "write past the layer workspace"
    oc, os_ = oracle.rope_table(M, hd, cfg["theta"])
    kc, vc = host(L.t["k_cache"]), host(L.t["v_cache"])
    post = post_rope(dict(cfg, pos=pos), host(bufs["qkv"]), w["g_q"], w["g_k"], oc[pos], os_[pos])
    att = oracle.attention(post[:nq * hd], nq, nkv, hd, kc, vc, 0, M * hd, hd, 0, pos + 1, cfg["attn_scale"])
    assert_close(host(bufs["attn"]), att, "attention with 64 splits in a workspace sized at max_ctx")


def _check_moe_block(cfg, w, escale, tag):
    """One MoE block on the GPU with every tap, checked stage by stage against
    the oracle fed the GPU's own inputs (teacher-forced), then free-running
    from the original inputs with only checked Q8_0 flips of h carried
    forward.  Returns (max rel err free-running, flips)."""
    torch = torch_mod()
    T_, H, I, E, k = cfg["tokens"], cfg["hidden"], cfg["ffn"], cfg["n_experts"], cfg["top_k"]
    if escale is not None:
        w = dict(w, expert_scale=escale)
    M = DeviceMoe(cfg, w, torch)
    taps, bufs = M.make_taps()
    x, logits = dev(w["x"]), dev(w["logits"])
    out = torch.empty(T_ * H, dtype=torch.float32, device="cuda")
    M.run(x, logits, out, taps)
    sync()
    G = {n: host(v) for n, v in bufs.items()}
    G["xd"], G["hd"] = G["xd"].view(np.uint16), G["hd"].view(np.uint16)
    ids = G["ids"].reshape(T_, k)
    rid, rw = oracle.moe_route(w["logits"], k)
    assert np.array_equal(ids, rid), f"{tag}: routing ids"
    assert_close(G["w"].reshape(T_, k), rw, f"{tag}: route weights")
    xq, xd = oracle.q8_quantize(w["x"])
    assert np.array_equal(G["xq"].reshape(T_, H), xq) and np.array_equal(G["xd"].reshape(T_, H // 32), xd), \
        f"{tag}: Q8_0 of x"
    y1 = G["y1"].reshape(T_, k, 2 * I)
    hq = G["hq"].reshape(T_, k, I)
    hd = G["hd"].reshape(T_, k, I // 32)
    y2 = G["y2"].reshape(T_, k, H)
    for t in range(T_):
        for s in range(k):
            e = ids[t, s]
            assert_close(y1[t, s], oracle.q8_matvec(w["gu_qs"][e], w["gu_d"][e], xq[t], xd[t]), f"{tag}: y1 {t},{s}")
            assert_q8_near(hq[t, s], hd[t, s], oracle.silu_mul(y1[t, s, :I], y1[t, s, I:]), f"{tag}: h {t},{s}")
            assert_close(y2[t, s], oracle.q8_matvec(w["dn_qs"][e], w["dn_d"][e], hq[t, s], hd[t, s]),
                         f"{tag}: y2 {t},{s}")
    ws = G["w"].reshape(T_, k).astype(np.float64)
    if escale is not None:
        ws = ws * escale[ids].astype(np.float64)
    want = np.einsum("ts,tsh->th", ws, y2.astype(np.float64))
    got = host(out).reshape(T_, H)
    assert_close(got, want, f"{tag}: weighted sum")
    # free-running: the oracle's block from the original inputs (routing and
    # Q8(x) are bit-exact above), carrying the GPU's Q8_0 of h forward only
    # where it is a checked boundary flip of the oracle's own h
    ref_fr = np.zeros((T_, H), np.float64)
    fr_flips = 0
    for t in range(T_):
        for s in range(k):
            e = rid[t, s]
            y1o = oracle.q8_matvec(w["gu_qs"][e], w["gu_d"][e], xq[t], xd[t])
            fr_flips += assert_q8_near(hq[t, s], hd[t, s], oracle.silu_mul(y1o[:I], y1o[I:]),
                                       f"{tag}: free-running h {t},{s}")
            y2o = oracle.q8_matvec(w["dn_qs"][e], w["dn_d"][e], hq[t, s], hd[t, s])
            ws_ = float(rw[t, s]) * (float(escale[e]) if escale is not None else 1.0)
            ref_fr[t] += ws_ * y2o.astype(np.float64)
    err = assert_close(got, ref_fr, f"{tag}: free-running MoE block")
    if fr_flips == 0:
        ref = oracle.moe_block(H, I, E, k, w["gu_qs"], w["gu_d"], w["dn_qs"], w["dn_d"], w["x"], w["logits"],
                               expert_scale=escale)
        assert_close(got, ref, f"{tag}: free-running MoE block (orc_moe_block)")
    return err, fr_flips, len(np.unique(ids))


@pytest.mark.parametrize("scaled", [False, True])
def test_moe_block_teacher_forced(scaled):
    """The MoE workload at full size."""
    name = list(synthetic.MOE_WORKLOADS)[0]
    cfg, w = synthetic.moe_inputs(name, seed=0)
    escale = synthetic.gamma(np.random.default_rng(77), cfg["n_experts"]) if scaled else None
    print(f"[moe] {name} per-expert scale={scaled}", flush=True)
    err, flips, touched = _check_moe_block(cfg, w, escale, name)
    print(f"[moe] free-running max rel err {err:.2e}; flips carried forward {flips}; "
          f"{touched} experts touched", flush=True)


# (tokens, hidden, ffn, experts, top_k, scaled, tied logits): the block's
# shape limits and edge cases beside the workload.
MOE_SHAPES = [
    (1, 512, 256, 8, 2, False, False),       # one token
    (16, 512, 256, 100, 6, True, False),     # experts not a multiple of 64
    (8, 2048, 1536, 8, 2, False, False),     # 2 KB rows in both matrices
    (4, 3072, 2560, 4, 2, False, False),     # 3 KB rows
    (5, 4096, 4096, 4, 2, False, False),     # the widest fused gate/up rows (4 KB)
    (16, 256, 128, 64, 32, False, False),    # 512 slots, top-32
    (8, 512, 256, 32, 4, False, True),       # tied logits: the lower id first
    (16, 256, 128, 1024, 8, False, False),   # 1024 experts
    (40, 512, 256, 16, 4, True, False),      # 40 tokens
]


@pytest.mark.parametrize("T,H,I,E,k,scaled,tied", MOE_SHAPES)
def test_moe_block_shapes(T, H, I, E, k, scaled, tied):
    name = list(synthetic.MOE_WORKLOADS)[0]
    cfg, w = synthetic.moe_inputs(name, seed=40 + T + E, tokens=T, hidden=H, ffn=I, n_experts=E, top_k=k)
    if tied:
        w["logits"] = np.round(w["logits"]).astype(np.float32)      # few distinct values: many ties
    escale = synthetic.gamma(np.random.default_rng(78), E) if scaled else None
    tag = f"moe T={T} H={H} I={I} E={E} k={k}"
    print(f"[moe] {tag} scaled={scaled} tied={tied}", flush=True)
    err, flips, touched = _check_moe_block(cfg, w, escale, tag)
    print(f"[moe] max rel err {err:.2e}; flips {flips}; {touched} experts touched", flush=True)


def _ggml_experts(fmt, r, rows, cols, E):
    """E experts of random GGML blocks ([E*rows] rows), packed by the
    library's host helper and uploaded; the struct describes one expert."""
    if fmt == "q4_0":
        b = synthetic.q4_0_blocks(r, E * rows, cols)
        qs = np.zeros((E * rows, cols // 2), np.uint8)
        d = np.zeros((E * rows, cols // 32), np.uint16)
        lq.lq_q4_0_pack_ggml(b, E * rows, cols, qs, d)
        return b, lq.q4_0_weight(dev(qs), dev(d), rows, cols)
    b = synthetic.q6_k_blocks(r, E * rows, cols)
    ql = np.zeros((E * rows, cols // 2), np.uint8)
    qh = np.zeros((E * rows, cols // 4), np.uint8)
    sc = np.zeros((E * rows, cols // 16), np.int8)
    d = np.zeros((E * rows, cols // 256), np.uint16)
    lq.lq_q6_k_pack_ggml(b, E * rows, cols, ql, qh, sc, d)
    return b, lq.q6_k_weight(dev(ql), dev(qh), dev(sc), dev(d), rows, cols)


@pytest.mark.parametrize("gu_fmt,dn_fmt,small", [
    ("q6_k", "q4_0", False),     # the MoE workload at full size, with the pages' formats (Q6_K gate/up, Q4_0 down)
    ("q4_0", "q6_k", True),      # the other pairing: 16 experts, 5 tokens, top-4, hidden 512, ffn 256
    ("q6_k", "q4_0", "wide"),    # hidden 8192 (> 4096: the id-matvec and a separate SwiGLU launch)
])
def test_moe_block_ggml_teacher_forced(gu_fmt, dn_fmt, small):
    """The MoE block on GGML-format experts: routing, Q8(x), each slot's
    gate_up and down id-matvec against the pinned oracle matvec of its
    expert fed the GPU's own inputs, the Q8_0 of h near the oracle's, and the
    weighted sum."""
    torch = torch_mod()
    r = np.random.default_rng(31 if small is True else 33 if small else 32)
    if small:
        T_, H, I, E, k = (5, 512, 256, 16, 4) if small is True else (3, 8192, 128, 8, 2)
        x = synthetic.activations(r, T_, H)
        logits = r.standard_normal((T_, E)).astype(np.float32)
    else:
        name = list(synthetic.MOE_WORKLOADS)[0]
        cfg, w = synthetic.moe_inputs(name, seed=6)
        T_, H, I, E, k = cfg["tokens"], cfg["hidden"], cfg["ffn"], cfg["n_experts"], cfg["top_k"]
        x, logits = w["x"], w["logits"]
    print(f"[moe ggml] gate_up {gu_fmt}, down {dn_fmt}, T={T_} H={H} I={I} E={E} k={k}", flush=True)
    bgu, Wgu = _ggml_experts(gu_fmt, r, 2 * I, H, E)
    bdn, Wdn = _ggml_experts(dn_fmt, r, H, I, E)
    fmt = {"q4_0": lq.LQ_FMT_Q4_0, "q6_k": lq.LQ_FMT_Q6_K}
    d = lq.lq_moe_ggml_desc(H, I, E, k, fmt[gu_fmt], fmt[dn_fmt])
    setattr(d, "gate_up_" + gu_fmt, Wgu)
    setattr(d, "down_" + dn_fmt, Wdn)
    e = lambda n, dt: torch.empty(n, dtype=dt, device="cuda")
    bufs = dict(ids=e(T_ * k, torch.int32), w=e(T_ * k, torch.float32), xq=e(T_ * H, torch.int8),
                xd=e(T_ * H // 32, torch.int16), y1=e(T_ * k * 2 * I, torch.float32), hq=e(T_ * k * I, torch.int8),
                hd=e(T_ * k * I // 32, torch.int16), y2=e(T_ * k * H, torch.float32))
    taps = lq.lq_moe_taps(**{n: v.data_ptr() for n, v in bufs.items()})
    nws = lq.lq_moe_block_ggml_workspace_size(d, T_)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out = torch.empty(T_ * H, dtype=torch.float32, device="cuda")
    lq.lq_moe_block_ggml(d, dev(x), dev(logits), T_, out, taps, ws, nws)
    sync()
    G = {n: host(v) for n, v in bufs.items()}
    G["xd"], G["hd"] = G["xd"].view(np.uint16), G["hd"].view(np.uint16)
    ids = G["ids"].reshape(T_, k)
    rid, rw = oracle.moe_route(logits, k)
    assert np.array_equal(ids, rid)
    assert_close(G["w"].reshape(T_, k), rw, "route weights")
    xq, xd = oracle.q8_quantize(x)
    assert np.array_equal(G["xq"].reshape(T_, H), xq) and np.array_equal(G["xd"].reshape(T_, H // 32), xd)
    y1 = G["y1"].reshape(T_, k, 2 * I)
    hq, hd = G["hq"].reshape(T_, k, I), G["hd"].reshape(T_, k, I // 32)
    y2 = G["y2"].reshape(T_, k, H)
    for t in range(T_):
        for s in range(k):
            ex = ids[t, s]
            assert_close(y1[t, s], oracle.q_matvec(gu_fmt, bgu[ex * 2 * I:(ex + 1) * 2 * I], 2 * I, H, xq[t], xd[t]),
                         f"y1 {t},{s}")
            assert_q8_near(hq[t, s], hd[t, s], oracle.silu_mul(y1[t, s, :I], y1[t, s, I:]), f"h {t},{s}")
            assert_close(y2[t, s], oracle.q_matvec(dn_fmt, bdn[ex * H:(ex + 1) * H], H, I, hq[t, s], hd[t, s]),
                         f"y2 {t},{s}")
    want = np.einsum("ts,tsh->th", G["w"].reshape(T_, k).astype(np.float64), y2.astype(np.float64))
    assert_close(host(out).reshape(T_, H), want, "weighted sum")

"""Benchmark: single-token decode layer (Q8_0 matvecs + GQA attention) on one MI355X.

A step is one decode token through a stack of R distinct synthetic layers of
the workload (default qwen3_8b_like_h4096: hidden 4096, 32/8 heads, head_dim
128, SwiGLU 12288, bf16 KV cache of 8192 positions).  R is chosen so the
stack holds >= 2 GB of weights and KV (>= 8 layers), so every layer streams
from HBM instead of the 256 MB Infinity Cache.  The stack is captured once as
a HIP graph and replayed; `value` is microseconds per token per layer.

Also measured inside this run, with HIP events on the launch stream:
  * roofline: the dominant kernel (the Q8_0 matvec instance that carries
    most of the layer's bytes) -- algorithmic bytes per launch / average
    launch duration, against 8 TB/s;
  * the GQA attention kernel the same way (extra field);
  * cpu_baseline: the plain C oracle running the same layer on one host
    thread (a bounded sample of full layer calls).

Prints one JSON line.  python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synthetic  # noqa: E402

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- inputs
FMT_BYTES = {"q8_0": 34 / 32, "q4_0": 18 / 32, "q6_k": 210 / 256}   # weight bytes per value


def device_layer_inputs(cfg, seed, torch, formats=None):
    """Layer inputs drawn directly on the GPU (same distributions as
    synthetic.py; bf16 KV drawn as the top half of float32 normals).
    formats: optional {"qkv" | "o" | "gu" | "dn": "q4_0" | "q6_k"}; those
    projections are random GGML arrays in the library's device layout (code
    bytes uniform, f16 scales as synthetic.py's blocks)."""
    import q8_matvec_gqa_amd as lq
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]

    def rbytes(*shape):
        return torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=g)

    def f16(shape, scale):
        return (torch.randn(shape, device="cuda", generator=g).abs() * scale).half().view(torch.int16)

    def q8(rows, cols):
        qs = torch.randint(-127, 128, (rows, cols), dtype=torch.int8, device="cuda", generator=g)
        d = (torch.randn(rows, cols // 32, device="cuda", generator=g).abs() * (0.02 / 127)).half()
        return qs, d.view(torch.int16)

    def proj(w, key, rows, cols):
        f = (formats or {}).get(key)
        if f is None:
            w[key + "_qs"], w[key + "_d"] = q8(rows, cols)
        elif f == "q4_0":
            w[key + "_fmt"] = f
            w[key + "_dev"] = lq.q4_0_weight(rbytes(rows, cols // 2), f16((rows, cols // 32), 0.02 / 8), rows, cols)
        else:
            w[key + "_fmt"] = f
            w[key + "_dev"] = lq.q6_k_weight(rbytes(rows, cols // 2), rbytes(rows, cols // 4),
                                             rbytes(rows, cols // 16).view(torch.int8), f16((rows, cols // 256), 2e-5),
                                             rows, cols)

    def gamma(n):
        return 1.0 + 0.1 * torch.randn(n, device="cuda", generator=g)

    def kv():
        a = torch.randn(nkv, cfg["max_ctx"], hd, device="cuda", generator=g)
        if cfg["kv_dtype"] == 0:
            return a
        return (a.view(torch.int32) >> 16).to(torch.int16)

    w = {"x": torch.randn(H, device="cuda", generator=g), "g_in": gamma(H)}
    proj(w, "qkv", nq * hd + 2 * nkv * hd, H)
    w["g_q"], w["g_k"] = gamma(hd), gamma(hd)
    proj(w, "o", H, nq * hd)
    w["g_post"] = gamma(H)
    if I:
        proj(w, "gu", 2 * I, H)
        proj(w, "dn", H, I)
    w["k_cache"], w["v_cache"] = kv(), kv()
    return w


def layer_bytes(cfg, formats=None):
    """Algorithmic HBM bytes of one decode layer: weights in their format
    (Q8_0 34 B per 32 values; Q4_0 18 per 32, Q6_K 210 per 256), the KV
    positions attended (read once), activations in and out."""
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    es = 4 if cfg["kv_dtype"] == 0 else 2
    L = min(cfg["window"], cfg["pos"] + 1) if cfg["window"] else cfg["pos"] + 1
    mats = [("qkv", nq * hd + 2 * nkv * hd, H), ("o", H, nq * hd)] + ([("gu", 2 * I, H), ("dn", H, I)] if I else [])
    mv = sum(matvec_bytes(r, c, fmt=(formats or {}).get(k, "q8_0")) for k, r, c in mats)
    attn = attn_bytes(nq, nkv, hd, L, es)
    return mv, attn


def matvec_bytes(rows, cols, residual=False, fmt="q8_0"):
    return int(rows * cols * FMT_BYTES[fmt]) + cols + cols // 16 + 4 * rows + (4 * rows if residual else 0)


def attn_bytes(nq, nkv, hd, L, es):
    return 2 * nkv * L * hd * es + 4 * nq * hd * 2


# ---------------------------------------------------------------- GPU parts
def time_stack(layers, xs, pos, steps, warmup, torch):
    """Graph-captured stack of layers: returns (ms per step, eager ms per step)."""
    stream = torch.cuda.Stream()
    R = len(layers)
    # eager reference (launch-overhead included), a few steps
    torch.cuda.synchronize()
    for i in range(R):
        layers[i].run(xs[i], pos)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        for i in range(R):
            layers[i].run(xs[i], pos)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / 3
    # capture one step (R layers) as a graph
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(R):
                layers[i].run(xs[i], pos)
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, eager_ms


def layer_kernels(cfg, nsplit_used, formats=None):
    """Names and algorithmic bytes of the kernels the decode layer launches,
    in launch order (matching lq_decode_layer_timed's events)."""
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    es = 4 if cfg["kv_dtype"] == 0 else 2
    pos = cfg["pos"]
    L = min(cfg["window"], pos + 1) if cfg["window"] else pos + 1
    qkv_rows = nq * hd + 2 * nkv * hd
    fm = formats or {}
    wb = {("qkv", qkv_rows, H), ("o", H, nq * hd), ("gu", 2 * I, H), ("dn", H, I)}
    wbytes = {k: int(r * c * FMT_BYTES[fm.get(k, "q8_0")]) for k, r, c in wb}
    q8w = lambda r, c: r * c * 34 // 32
    ks = [("qkv_matvec", "k_mv<NCH=%d,NORM,STORE>" % math.ceil(H / 1024),
           wbytes["qkv"] + 8 * H + 4 * qkv_rows),
          ("attn_split", "k_attn_split", attn_bytes(nq, nkv, hd, L, es) + 4 * qkv_rows)]
    if nsplit_used:
        ks.append(("attn_combine", "k_attn_combine", 0))
    if cfg["kind"] == 0:
        ks += [("o_matvec", "k_mv<NCH=%d,QUANT,RESID>" % math.ceil(nq * hd / 1024), wbytes["o"] + 4 * nq * hd + 8 * H),
               ("gate_up_matvec", "k_mv<NCH=%d,NORM,SWIGLU_Q8>" % math.ceil(H / 1024), wbytes["gu"] + 8 * H + q8w(1, I)),
               ("down_matvec", "k_mv<NCH=%d,Q8,RESID>" % math.ceil(I / 1024), wbytes["dn"] + q8w(1, I) + 8 * H)]
    else:
        ks += [("o_matvec", "k_mv<NCH=%d,QUANT,STORE>" % math.ceil(nq * hd / 1024), wbytes["o"] + 4 * nq * hd + 4 * H),
               ("post_norm_add", "k_rmsnorm_add", 16 * H)]
    return ks


def spin_cycles(torch, ms):
    """Argument of torch.cuda._sleep (a spin kernel that touches no memory)
    for about `ms` milliseconds on this device, from one timed probe."""
    probe = 1 << 20
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(probe)
    e0.record()
    torch.cuda._sleep(probe)
    e1.record()
    torch.cuda.synchronize()
    per_ms = probe / max(e0.elapsed_time(e1), 1e-3)
    return int(min(max(per_ms * ms, 1 << 16), 1 << 34))


def kernel_measurements(cfg, layers, xs, torch, rounds, formats=None):
    """Times every kernel of the decode layer with start/stop HIP events that
    the runtime stamps at each dispatch of the layer (lq_decode_layer_timed),
    on the stream the layer runs on.  Each round enqueues all R layers back
    to back behind a ~2 ms spin kernel (no memory traffic), so the host has
    queued every launch before the first one starts and the kernels run one
    after another as in the graph replay (no host gaps, each kernel starting
    as the previous one drains).  A device copy as the wait would leave the
    Infinity Cache full of dirty lines, whose write-back then competes with
    the first layers' reads."""
    import q8_matvec_gqa_amd as lq
    n_k = lq.lq_decode_layer_kernel_count(layers[0].desc)
    R = len(layers)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_k)] for _ in range(R)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    names = layer_kernels(cfg, n_k == (6 if cfg["kind"] == 0 else 5), formats)
    assert len(names) == n_k, (len(names), n_k)
    if hasattr(torch.cuda, "_sleep"):
        cycles = spin_cycles(torch, 2.0)
        busy = lambda: torch.cuda._sleep(cycles)
    else:
        # without torch's spin kernel: a read-only reduction (no dirty lines left behind)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        busy = lambda: src.sum()
    times = [[] for _ in range(n_k)]
    for r in range(rounds + 1):
        busy()                                    # keeps the GPU busy while the host enqueues
        for li, lay in enumerate(layers):
            lq.lq_decode_layer_timed(lay.desc, xs[li], cfg["pos"], None, lay.ws, lay.ws_bytes, evs[li])
        torch.cuda.synchronize()
        if r == 0:
            continue                              # warm round
        for li in range(R):
            for k in range(n_k):
                times[k].append(evs[li][2 * k].elapsed_time(evs[li][2 * k + 1]) * 1e3)
    per = {}
    for (tag, kernel, b), ts in zip(names, times):
        per[tag] = dict(kernel=kernel, launches=len(ts), avg_us=float(np.mean(ts)), min_us=float(np.min(ts)),
                        bytes=int(b))
    return per


def measure_layer(workload, steps, warmup, rounds, min_stack_bytes, torch, formats=None):
    """A graph-captured stack of R distinct layers (>= min_stack_bytes of
    weights and KV, so the Infinity Cache cannot serve them), timed over
    `steps` replays, plus per-kernel launch durations from HIP events.
    formats: GGML weight formats of some projections (see device_layer_inputs)."""
    from q8_matvec_gqa_amd.layers import DeviceLayer
    cfg = synthetic.layer_cfg(workload)
    mv_b, at_b = layer_bytes(cfg, formats)
    R = max(8, math.ceil(min_stack_bytes / (mv_b + at_b)))
    tag = workload + (" " + ",".join(f"{k}={v}" for k, v in formats.items()) if formats else "")
    log(f"workload {tag}: {(mv_b + at_b) / 1e6:.1f} MB/layer, stack of {R} layers")
    layers, xs = [], []
    for i in range(R):
        w = device_layer_inputs(cfg, seed=1000 + i, torch=torch, formats=formats)
        layers.append(DeviceLayer(cfg, w, torch))
        xs.append(w["x"])
    torch.cuda.synchronize()
    ms_step, eager_ms = time_stack(layers, xs, cfg["pos"], steps, warmup, torch)
    us_layer = ms_step * 1e3 / R
    log(f"{tag}: {us_layer:.2f} us/token/layer (graph), eager {eager_ms * 1e3 / R:.2f}")
    per = kernel_measurements(cfg, layers, xs, torch, rounds, formats)
    at_us = per["attn_split"]["avg_us"] + (per["attn_combine"]["avg_us"] if "attn_combine" in per else 0.0)
    at_bytes = per["attn_split"]["bytes"]
    at_gbs = at_bytes / (at_us * 1e3)
    mv_tags = [t for t in per if t.endswith("_matvec")]
    mv_us = sum(per[t]["avg_us"] for t in mv_tags)
    mv_bytes = sum(per[t]["bytes"] for t in mv_tags)
    del layers, xs
    return {
        "R": R, "ms_step": ms_step, "us_layer": us_layer, "eager_us_layer": eager_ms * 1e3 / R,
        "layer_bytes": mv_b + at_b, "per": per,
        "attn": {"bound": "hbm", "kernel": "k_attn_split+k_attn_combine", "achieved": round(at_gbs, 1),
                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(at_gbs / HBM_PEAK_GBS, 4),
                 "bytes_per_launch": at_bytes, "avg_launch_us": round(at_us, 3)},
        "matvec": {"us": round(mv_us, 3), "bytes": mv_bytes, "GBps": round(mv_bytes / (mv_us * 1e3), 1),
                   "frac": round(mv_bytes / (mv_us * 1e3) / HBM_PEAK_GBS, 4)},
    }


def device_moe_inputs(c, seed, torch):
    """MoE block inputs drawn on the GPU (same distributions as synthetic.py)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    H, I, E, T = c["hidden"], c["ffn"], c["n_experts"], c["tokens"]

    def q8(rows, cols):
        qs = torch.randint(-127, 128, (rows, cols), dtype=torch.int8, device="cuda", generator=g)
        d = (torch.randn(rows, cols // 32, device="cuda", generator=g).abs() * (0.02 / 127)).half()
        return qs, d.view(torch.int16)

    w = {"x": torch.randn(T, H, device="cuda", generator=g), "logits": torch.randn(T, E, device="cuda", generator=g)}
    w["gu_qs"], w["gu_d"] = q8(E * 2 * I, H)
    w["dn_qs"], w["dn_d"] = q8(E * H, I)
    return w


def measure_moe(name, steps, torch):
    """The MoE block (route, gather, id-matvecs, SwiGLU, weighted sum) on R
    replicas of all expert weights, graph-captured.  Algorithmic bytes: the
    experts the routing touches (counted per replica from the same top-k)
    at 34 B per 32 weights, plus activations."""
    from q8_matvec_gqa_amd.layers import DeviceMoe
    c = dict(synthetic.MOE_WORKLOADS[name])
    H, I, E, T, k = c["hidden"], c["ffn"], c["n_experts"], c["tokens"], c["top_k"]
    expert_bytes = 3 * I * H * 34 // 32
    R = max(2, math.ceil(1.5e9 / (E * expert_bytes)))
    mods, ins, outs, touched = [], [], [], []
    for i in range(R):
        w = device_moe_inputs(c, 2000 + i, torch)
        mods.append(DeviceMoe(c, w, torch))
        ins.append((w["x"], w["logits"]))
        outs.append(torch.empty(T, H, device="cuda"))
        ids = torch.topk(torch.softmax(w["logits"].double(), dim=1), k, dim=1).indices
        touched.append(int(torch.unique(ids).numel()))
        del w
    block_bytes = [n * expert_bytes + T * H * 8 + T * E * 4 for n in touched]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    for i in range(R):
        mods[i].run(ins[i][0], ins[i][1], outs[i])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(R):
                mods[i].run(ins[i][0], ins[i][1], outs[i])
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us_block = e0.elapsed_time(e1) * 1e3 / (steps * R)
    mean_bytes = sum(block_bytes) / R
    gbs = mean_bytes / (us_block * 1e3)
    log(f"{name}: {us_block:.2f} us/block ({us_block / T:.2f} us/token), {gbs:.1f} GB/s, "
        f"touched experts {touched}")
    del mods, ins, outs, graph
    return {"workload": name, "us_per_block": round(us_block, 3), "tokens": T,
            "us_per_token": round(us_block / T, 3), "touched_experts": touched,
            "bytes_per_block": int(mean_bytes), "GBps": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "replicas": R, "graph": True}


def graph_us(torch, calls, steps):
    """calls(stream) issues one round of launches; it is run once eagerly,
    captured as a HIP graph on a side stream and replayed `steps` times, so
    no host launch overhead is timed.  Returns microseconds per replay."""
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        calls(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            calls(stream)
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e3 / steps


def measure_matmul(T, steps, torch):
    """The multi-token Q8_0 matmul (int8 MFMA) on the 8B-like layer's four
    projections for a batch of T tokens, over R distinct replicas of the
    weights (>= 2 GB, beyond the Infinity Cache).  Algorithmic bytes per call:
    weights + T rows of Q8_0 input + T rows of f32 output."""
    import q8_matvec_gqa_amd as lq
    cfg = synthetic.layer_cfg("qwen3_8b_like_h4096")
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    shapes = {"qkv": (nq * hd + 2 * nkv * hd, H), "o": (H, nq * hd), "gate_up": (2 * I, H), "down": (H, I)}
    per_rep = sum(r * c * 34 // 32 for r, c in shapes.values())
    R = max(2, math.ceil(2e9 / per_rep))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4000)
    reps = []
    for _ in range(R):
        ws = {}
        for k, (r, c) in shapes.items():
            qs = torch.randint(-127, 128, (r, c), dtype=torch.int8, device="cuda", generator=gen)
            d = (torch.randn(r, c // 32, device="cuda", generator=gen).abs() * (0.02 / 127)).half().view(torch.int16)
            ws[k] = (lq.q8_weight(qs, d), qs, d)
        reps.append(ws)
    xs = {}
    for k, (r, c) in shapes.items():
        xs[k] = (torch.randint(-127, 128, (T, c), dtype=torch.int8, device="cuda", generator=gen),
                 (torch.rand(T, c // 32, device="cuda", generator=gen) * 0.05).half().view(torch.int16),
                 torch.empty(T, r, device="cuda"))
    nws = max(lq.lq_q8_matmul_workspace_size(r, c, T) for r, c in shapes.values())
    work = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
    res = {}
    total_us = 0.0
    for k, (r, c) in shapes.items():
        xq, xd, y = xs[k]

        def calls(stream):
            for ws in reps:
                lq.lq_q8_matmul(ws[k][0], xq, xd, T, None, y, work, nws, stream=stream)

        us = graph_us(torch, calls, steps) / R
        nbytes = r * c * 34 // 32 + T * c * 34 // 32 + T * r * 4
        res[k] = {"rows": r, "cols": c, "us": round(us, 3), "GBps": round(nbytes / (us * 1e3), 1),
                  "frac": round(nbytes / (us * 1e3) / HBM_PEAK_GBS, 4),
                  "TOPs": round(2.0 * T * r * c / (us * 1e-6) / 1e12, 1)}
        total_us += us
        log(f"q8_matmul T={T} {k:8s} {r}x{c}: {us:.2f} us, {res[k]['GBps']:.1f} GB/s, {res[k]['TOPs']:.1f} TOP/s")
    del reps, xs, work
    return {"workload": f"q8_matmul_t{T}_qwen3_8b_like_h4096", "tokens": T, "replicas": R,
            "us_four_projections": round(total_us, 3), "us_per_token_four_projections": round(total_us / T, 3),
            "per_matrix": res, "mfma": "v_mfma_i32_32x32x32_i8"}


def measure_ggml_formats(steps, torch):
    """The Q4_0 and Q6_K weight matvecs (Q8_0 activation) on the 8B-like
    layer's four projection shapes, one token, over R distinct weight
    replicas (>= 2 GB, beyond the Infinity Cache).  Algorithmic bytes per
    call: the format's weight bytes (Q4_0 18 and Q6_K 210 per 32 / 256
    values) + the Q8_0 input + the f32 output."""
    import q8_matvec_gqa_amd as lq
    cfg = synthetic.layer_cfg("qwen3_8b_like_h4096")
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    shapes = {"qkv": (nq * hd + 2 * nkv * hd, H), "o": (H, nq * hd), "gate_up": (2 * I, H), "down": (H, I)}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5000)
    out = {}
    for fmt, bpv in (("q4_0", 18 / 32), ("q6_k", 210 / 256)):
        per_rep = sum(r * c * bpv for r, c in shapes.values())
        R = max(2, math.ceil(2e9 / per_rep))

        def rbytes(*shape):
            return torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=gen)

        def f16(shape, scale):
            return (torch.randn(shape, device="cuda", generator=gen).abs() * scale).half().view(torch.int16)

        reps = []
        for _ in range(R):
            ws = {}
            for k, (r, c) in shapes.items():
                if fmt == "q4_0":
                    ws[k] = lq.q4_0_weight(rbytes(r, c // 2), f16((r, c // 32), 0.02 / 8), r, c)
                else:
                    ws[k] = lq.q6_k_weight(rbytes(r, c // 2), rbytes(r, c // 4), rbytes(r, c // 16).view(torch.int8),
                                           f16((r, c // 256), 2e-5), r, c)
            reps.append(ws)
        call = lq.lq_q4_0_matvec if fmt == "q4_0" else lq.lq_q6_k_matvec
        res = {}
        total = 0.0
        for k, (r, c) in shapes.items():
            xq = torch.randint(-127, 128, (c,), dtype=torch.int8, device="cuda", generator=gen)
            xd = (torch.rand(c // 32, device="cuda", generator=gen) * 0.05).half().view(torch.int16)
            y = torch.empty(r, device="cuda")

            def calls(stream):
                for ws in reps:
                    call(ws[k], xq, xd, None, y, stream=stream)

            us = graph_us(torch, calls, steps) / R
            nbytes = r * c * bpv + c * 34 / 32 + 4 * r
            res[k] = {"rows": r, "cols": c, "us": round(us, 3), "GBps": round(nbytes / (us * 1e3), 1),
                      "frac": round(nbytes / (us * 1e3) / HBM_PEAK_GBS, 4)}
            total += us
            log(f"{fmt}_matvec {k:8s} {r}x{c}: {us:.2f} us, {res[k]['GBps']:.1f} GB/s")
        out[fmt] = {"workload": f"{fmt}_matvec_qwen3_8b_like_h4096", "replicas": R,
                    "us_four_projections": round(total, 3), "per_matrix": res}
        del reps
        torch.cuda.empty_cache()
    return out


def measure_moe_formats(steps, torch):
    """The index-driven matvec on Q6_K and Q4_0 experts at the MoE workload
    (16 tokens, top-8 of 128 experts): the gate/up projection [2*ffn, hidden]
    per expert, ids from a softmax top-k of N(0,1) logits, R replicas of all
    experts (>= 1.5 GB).  Algorithmic bytes: the touched experts' weights in
    the format, plus the per-token Q8_0 input and the f32 output."""
    import q8_matvec_gqa_amd as lq
    c = dict(synthetic.MOE_WORKLOADS["moe_e128_top8_t16"])
    H, I, E, T, k = c["hidden"], c["ffn"], c["n_experts"], c["tokens"], c["top_k"]
    rows, cols = 2 * I, H
    gen = torch.Generator(device="cuda")
    gen.manual_seed(6000)
    out = {}
    for fmt, bpv in (("q6_k", 210 / 256), ("q4_0", 18 / 32)):
        expert_bytes = rows * cols * bpv
        R = max(2, math.ceil(1.5e9 / (E * expert_bytes)))

        def rbytes(*shape):
            return torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=gen)

        def f16(shape, scale):
            return (torch.randn(shape, device="cuda", generator=gen).abs() * scale).half().view(torch.int16)

        reps = []
        for _ in range(R):
            n = E * rows
            if fmt == "q4_0":
                W = lq.q4_0_weight(rbytes(n, cols // 2), f16((n, cols // 32), 0.02 / 8), rows, cols)
            else:
                W = lq.q6_k_weight(rbytes(n, cols // 2), rbytes(n, cols // 4), rbytes(n, cols // 16).view(torch.int8),
                                   f16((n, cols // 256), 2e-5), rows, cols)
            logits = torch.randn(T, E, device="cuda", generator=gen)
            ids = torch.topk(torch.softmax(logits.double(), dim=1), k, dim=1).indices.to(torch.int32).contiguous()
            reps.append((W, ids, int(torch.unique(ids).numel())))
        xq = torch.randint(-127, 128, (T, cols), dtype=torch.int8, device="cuda", generator=gen)
        xd = (torch.rand(T, cols // 32, device="cuda", generator=gen) * 0.05).half().view(torch.int16)
        y = torch.empty(T * k, rows, device="cuda")
        nws = lq.lq_moe_workspace_size(T, k, E)
        work = torch.empty(nws, dtype=torch.uint8, device="cuda")
        call = lq.lq_moe_q4_0_matvec_id if fmt == "q4_0" else lq.lq_moe_q6_k_matvec_id

        def calls(stream):
            for W, ids, _ in reps:
                call(W, E, xq, xd, 0, ids, T, k, y, work, nws, stream=stream)

        us = graph_us(torch, calls, steps) / R
        touched = sum(t for _, _, t in reps) / R
        nbytes = touched * expert_bytes + T * cols * 34 / 32 + T * k * rows * 4
        out[fmt] = {"workload": f"moe_e128_top8_t16_gate_up_{fmt}", "replicas": R, "us": round(us, 3),
                    "touched_experts": round(touched, 1), "GBps": round(nbytes / (us * 1e3), 1),
                    "frac": round(nbytes / (us * 1e3) / HBM_PEAK_GBS, 4)}
        log(f"moe {fmt} gate/up id-matvec {rows}x{cols} x {E} experts: {us:.2f} us, "
            f"{touched:.1f} touched, {out[fmt]['GBps']:.1f} GB/s")
        del reps, work
        torch.cuda.empty_cache()
    return out


def measure_moe_block_ggml(steps, torch):
    """The whole MoE block (lq_moe_block_ggml) on the pages' expert formats,
    Q6_K gate/up and Q4_0 down, at the MoE workload (16 tokens, top-8 of 128
    experts), R replicas of all experts (>= 1.5 GB) with their own logits.
    Algorithmic bytes: the touched experts' gate/up and down weights in their
    formats, plus x, logits and the output (f32)."""
    import q8_matvec_gqa_amd as lq
    c = dict(synthetic.MOE_WORKLOADS["moe_e128_top8_t16"])
    H, I, E, T, k = c["hidden"], c["ffn"], c["n_experts"], c["tokens"], c["top_k"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7000)

    def rbytes(*shape):
        return torch.randint(0, 256, shape, dtype=torch.uint8, device="cuda", generator=gen)

    def f16(shape, scale):
        return (torch.randn(shape, device="cuda", generator=gen).abs() * scale).half().view(torch.int16)

    expert_bytes = 2 * I * H * 210 / 256 + H * I * 18 / 32
    R = max(2, math.ceil(1.5e9 / (E * expert_bytes)))
    reps = []
    for _ in range(R):
        n = E * 2 * I
        gu = lq.q6_k_weight(rbytes(n, H // 2), rbytes(n, H // 4), rbytes(n, H // 16).view(torch.int8),
                            f16((n, H // 256), 2e-5), 2 * I, H)
        dn = lq.q4_0_weight(rbytes(E * H, I // 2), f16((E * H, I // 32), 0.02 / 8), H, I)
        d = lq.lq_moe_ggml_desc(H, I, E, k, lq.LQ_FMT_Q6_K, lq.LQ_FMT_Q4_0, gate_up_q6_k=gu, down_q4_0=dn)
        d._keep = (gu, dn)
        logits = torch.randn(T, E, device="cuda", generator=gen)
        touched = int(torch.unique(torch.topk(logits, k, dim=1).indices).numel())
        reps.append((d, logits, touched))
    x = torch.randn(T, H, device="cuda", generator=gen)
    out = torch.empty(T, H, device="cuda")
    nws = lq.lq_moe_block_ggml_workspace_size(reps[0][0], T)
    work = torch.empty(nws, dtype=torch.uint8, device="cuda")

    def calls(stream):
        for d, logits, _ in reps:
            lq.lq_moe_block_ggml(d, x, logits, T, out, None, work, nws, stream=stream)

    us = graph_us(torch, calls, steps) / R
    touched = sum(t for _, _, t in reps) / R
    nbytes = touched * expert_bytes + T * H * 4 * 2 + T * E * 4
    gbs = nbytes / (us * 1e3)
    log(f"moe block q6_k gate/up + q4_0 down, 128 experts, 16 tokens: {us:.2f} us/block, {touched:.1f} touched, "
        f"{gbs:.1f} GB/s")
    del reps, work
    torch.cuda.empty_cache()
    return {"workload": "moe_e128_top8_t16_q6_k_gate_up_q4_0_down", "replicas": R, "us_per_block": round(us, 3),
            "us_per_token": round(us / T, 3), "touched_experts": round(touched, 1), "GBps": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def measure_head(steps, torch):
    """The output head (final norm, f16 vocab projection, softcap) at the
    Gemma-4 shape: vocab x hidden f16 weights (1.5 GB, beyond the Infinity
    Cache) read once per call.  Algorithmic bytes: weights + x + gamma +
    logits."""
    import q8_matvec_gqa_amd as lq
    H = synthetic.HEAD
    V, D = H["vocab"], H["hidden"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3000)
    w = (torch.randn(V, D, device="cuda", generator=gen) * 0.02).half().view(torch.int16)
    x = torch.randn(D, device="cuda", generator=gen)
    g = 1.0 + 0.1 * torch.randn(D, device="cuda", generator=gen)
    out = torch.empty(V, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(3):
        lq.lq_lm_head_f16(w, V, D, x, 1, g, H["eps"], H["softcap"], out, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        lq.lq_lm_head_f16(w, V, D, x, 1, g, H["eps"], H["softcap"], out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = V * D * 2 + D * 8 + V * 4
    gbs = nbytes / (us * 1e3)
    log(f"lm_head_v{V}_h{D}: {us:.2f} us/call, {gbs:.1f} GB/s")
    del w, x, g, out
    return {"workload": f"lm_head_v{V}_h{D}", "us_per_call": round(us, 3), "bytes_per_call": nbytes,
            "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "dtype": "f16 weights, f32 math",
            "softcap": H["softcap"]}


def measure_attn_context(steps, torch, ctx=65536):
    """GQA decode attention alone (split kernel + combine) with the 8B-like
    heads at a long bf16 context, where every wave streams 16 tiles: the
    regime in which the split kernel is bound by HBM rather than by latency.
    Two K/V cache pairs alternate (2 x 268 MB, beyond the Infinity Cache).
    Algorithmic bytes: K and V once, q in, the output out."""
    import q8_matvec_gqa_amd as lq
    n_q, n_kv, hd = 32, 8, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4000)
    pairs = [tuple((torch.randn(n_kv * ctx * hd, device="cuda", generator=gen) * 0.5).bfloat16().view(torch.int16)
                   for _ in range(2)) for _ in range(2)]
    q = torch.randn(n_q * hd, device="cuda", generator=gen)
    out = torch.empty(n_q * hd, dtype=torch.float32, device="cuda")
    nws = lq.lq_gqa_decode_attn_workspace_size(n_q, n_kv, hd, ctx)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(hd)

    def calls(stream):
        for k, v in pairs:
            lq.lq_gqa_decode_attn(q, n_q, n_kv, hd, k, v, 1, ctx * hd, hd, ctx, 0, ctx, scale, out, ws, nws,
                                  stream=stream)

    us = graph_us(torch, calls, steps) / len(pairs)
    nbytes = attn_bytes(n_q, n_kv, hd, ctx, 2)
    gbs = nbytes / (us * 1e3)
    log(f"attention n_q {n_q} n_kv {n_kv} hd {hd} bf16 x {ctx} positions: {us:.2f} us/call, {gbs:.1f} GB/s")
    del pairs, q, out, ws
    torch.cuda.empty_cache()
    return {"workload": f"gqa_attn_q{n_q}_kv{n_kv}_hd{hd}_bf16_ctx{ctx}", "kernel": "k_attn_split+k_attn_combine",
            "us_per_call": round(us, 3), "bytes_per_call": nbytes, "GBps": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def calib_copy(torch, nbytes=1 << 30, reps=3):
    """A plain elementwise copy of known size (reads nbytes, writes nbytes),
    run for the PMC calibration of FETCH_SIZE / WRITE_SIZE."""
    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)          # the only negation kernel in the run
    torch.cuda.synchronize()
    return nbytes


# ---------------------------------------------------------------- profiles
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join("q8_matvec_gqa_amd", "csrc")


def kernel_sources():
    """Every device source of the library: a summary taken before any of them
    changed no longer describes the kernels that run."""
    d = os.path.join(ROOT, CSRC)
    return sorted(os.path.join(CSRC, f) for f in os.listdir(d) if f.endswith((".hip", ".h")))


def source_hash(paths=None):
    import hashlib
    h = hashlib.sha256()
    for p in (kernel_sources() if paths is None else paths):
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def layer_kernel_patterns(cfg):
    """rocprofv3 kernel-name patterns of the decode layer's kernels (template
    arguments: NCH, RPW, prologue, epilogue, waves for k_mv)."""
    import re
    H, qd, I = cfg["hidden"], cfg["n_q"] * cfg["head_dim"], cfg["ffn"]
    nch = lambda c: math.ceil(c / 1024)
    kv = "float" if cfg["kv_dtype"] == 0 else "unsigned short"
    ce = 4 if cfg["kv_dtype"] == 0 else 8
    pats = {"qkv_matvec": r"k_mv<%d, \d+, 2, 0, \d+>" % nch(H),
            "attn_split": r"k_attn_split<%s, %d, %d, " % (kv, cfg["head_dim"] // ce, cfg["n_q"] // cfg["n_kv"]),
            "attn_combine": r"k_attn_combine",
            "o_matvec": r"k_mv<%d, \d+, 1, %d, \d+>" % (nch(qd), 1 if cfg["kind"] == 0 else 0)}
    if cfg["kind"] == 0:
        pats["gate_up_matvec"] = r"k_mv<%d, \d+, 2, 3, \d+>" % nch(H)
        pats["down_matvec"] = r"k_mv<%d, \d+, 0, 1, \d+>" % nch(I)
    else:
        pats["post_norm_add"] = r"k_rmsnorm_add"
    return {t: re.compile(p) for t, p in pats.items()}


def _kernel_match(name, tag, cfg=None):
    """rocprofv3 kernel names -> the layer's kernel tags (headline workload by default)."""
    if tag == "copy":
        return "neg" in name.lower()
    pats = layer_kernel_patterns(cfg or synthetic.layer_cfg(synthetic.HEADLINE))
    return pats[tag].search(name) is not None


def summarize_pmc(fetch_dir, write_dir, workload, out_path, command):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel of the layer
    and of the calibration copy -> HBM bytes per launch, written as a text
    summary (one line per kernel)."""
    cfg = synthetic.layer_cfg(workload)
    tags = list(layer_kernel_patterns(cfg)) + ["copy"]

    def per_kernel(d, counter):
        rows = _read_csv(_find(d, "counter_collection.csv"))
        out = {t: [] for t in tags}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            for tag in out:
                if _kernel_match(r["Kernel_Name"], tag, cfg):
                    out[tag].append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v) if v else float("nan"), len(v)) for k, v in out.items()}

    f = per_kernel(fetch_dir, "FETCH_SIZE")
    w = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = 1 << 30
    f_scale = copy_bytes / (f["copy"][0] * 1024.0)
    w_scale = copy_bytes / (w["copy"][0] * 1024.0)
    algo = dict((t, b) for t, _, b in layer_kernels(cfg, True))
    lines = [
        f"# HBM traffic per launch of the decode layer's kernels, {workload}",
        f"command_fetch: {command.replace('WRITE_SIZE', 'FETCH_SIZE')}",
        f"command_write: {command.replace('FETCH_SIZE', 'WRITE_SIZE')}",
        f"source_sha256: {source_hash()}",
        f"copy_calibration_bytes: {copy_bytes}",
        f"copy_fetch_kib: {f['copy'][0]:.1f}  (scale {f_scale:.4f})",
        f"copy_write_kib: {w['copy'][0]:.1f}  (scale {w_scale:.4f})",
        "kernel | dispatches | fetch_kib | write_kib | traffic_bytes | algorithmic_bytes | traffic_over_algorithmic",
    ]
    for t in tags[:-1]:
        fb, wb = f[t][0] * 1024.0 * f_scale, w[t][0] * 1024.0 * w_scale
        a = algo.get(t, 0)
        ratio = f"{(fb + wb) / a:.4f}" if a else "-"
        lines.append(f"{t} | {f[t][1]} | {f[t][0]:.1f} | {w[t][0]:.1f} | {int(round(fb + wb))} | {a} | {ratio}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _summary(path):
    """(key: value header, {kernel: [columns]}) of a committed summary, or None
    when it is missing or the kernel sources changed since it was taken."""
    if not os.path.exists(path):
        return None
    kv, rows = {}, {}
    with open(path) as f:
        for line in f:
            line = line.rstrip("\n")
            if " | " in line:
                c = [x.strip() for x in line.split(" | ")]
                rows[c[0]] = c[1:]
            elif ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash():
        return None
    return kv, rows


def load_traffic(workload, tag="gate_up_matvec"):
    """traffic_bytes per launch of a layer kernel from the committed PMC
    summary, or None (missing, or the sources changed since it was taken)."""
    s = _summary(os.path.join(PROFILES, f"decode_layer_{workload}.pmc.txt"))
    if s is None or tag not in s[1]:
        return None
    v = s[1][tag][3]
    return int(v) if v.isdigit() else None


def load_trace_avg(workload, tag="gate_up_matvec", phase="timed"):
    """Average duration (us) of a layer kernel in one phase of the committed
    rocprofv3 kernel trace of the bench command ("timed": the dispatches
    that the bench's per-kernel events time; "graph": the graph replays), or
    None."""
    s = _summary(os.path.join(PROFILES, f"decode_layer_{workload}.trace.txt"))
    if s is None:
        return None
    key = f"{tag}@{phase}"
    if key not in s[1]:
        return None
    return float(s[1][key][1])


def stack_layers(cfg, min_stack_bytes=2.0e9):
    mv_b, at_b = layer_bytes(cfg)
    return max(8, math.ceil(min_stack_bytes / (mv_b + at_b)))


def trace_phases(R, steps, warmup, rounds):
    """Dispatch index ranges, per kernel of the measured workload's layer and
    in launch order, of measure_layer's phases: the eager reference (one warm
    and three timed calls of each of the R layers), the graph warmup, the
    graph replays, then the per-kernel event rounds (one warm round)."""
    a = 4 * R
    b = a + warmup * R
    c = b + steps * R
    d = c + R
    e = d + rounds * R
    return {"eager": (0, a), "graph": (b, c), "timed": (d, e)}


def summarize_counters(dirs, out_path, command, title):
    """Per-kernel averages (over dispatches) of every counter in one or more
    rocprofv3 --pmc output folders (one pass each) -> a text summary."""
    import statistics
    per = {}
    for d in dirs:
        rows = _read_csv(_find(d, "counter_collection.csv"))
        acc = {}
        for r in rows:
            n = r["Kernel_Name"]
            if "lq::" not in n:
                continue
            key = (n, r["Dispatch_Id"], r["Counter_Name"])
            acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        for (n, _, c), v in acc.items():
            per.setdefault(n, {}).setdefault(c, []).append(v)
    lines = [f"# {title}", f"command: {command}", f"source_sha256: {source_hash()}",
             "kernel | counter | dispatches | average per dispatch"]
    for n in sorted(per):
        for c in sorted(per[n]):
            v = per[n][c]
            lines.append(f"{n} | {c} | {len(v)} | {statistics.mean(v):.1f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(trace_dir, out_dir, workload, command, steps=20, warmup=5, rounds=5):
    """Kernel-trace statistics of a bench run -> a text summary: every lq
    kernel (average duration over all its dispatches), then each kernel of
    the measured workload's layer per phase of the bench (the workload runs
    first, so its dispatches lead each kernel's list)."""
    import statistics
    rows = _read_csv(_find(trace_dir, "kernel_trace.csv"))
    groups = {}
    for r in rows:
        n = r["Kernel_Name"]
        if "lq::" not in n:
            continue
        groups.setdefault(n, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    cfg = synthetic.layer_cfg(workload)
    R = stack_layers(cfg)
    phases = trace_phases(R, steps, warmup, rounds)
    lines = [f"# rocprofv3 kernel trace of bench.py, {workload}", f"command: {command}",
             f"source_sha256: {source_hash()}",
             f"phases: {R} layers; per kernel and in launch order, dispatches [a, b) of each phase: "
             + ", ".join(f"{k} {v}" for k, v in phases.items()),
             "kernel | dispatches | avg_us | median_us | min_us | max_us"]
    durs = {n: [(e - s_) / 1e3 for s_, e in sorted(v)] for n, v in groups.items()}
    for n, ts in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{n} | {len(ts)} | {statistics.mean(ts):.3f} | {statistics.median(ts):.3f} | "
                     f"{min(ts):.3f} | {max(ts):.3f}")
    lines.append("layer kernel@phase | dispatches | avg_us | median_us | min_us | max_us")
    first = {n: min(v)[0] for n, v in groups.items()}
    for tag, pat in layer_kernel_patterns(cfg).items():
        # several instances can match (another workload's shape of the same
        # step): the workload's own is the one dispatched first
        names = sorted((n for n in durs if pat.search(n)), key=lambda n: first[n])
        if not names:
            continue
        ts = durs[names[0]]
        for ph, (a, b) in phases.items():
            sub = ts[a:b]
            if sub:
                lines.append(f"{tag}@{ph} | {len(sub)} | {statistics.mean(sub):.3f} | {statistics.median(sub):.3f} | "
                             f"{min(sub):.3f} | {max(sub):.3f}")
    out = os.path.join(out_dir, f"decode_layer_{workload}.trace.txt")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(workload, seconds):
    """The oracle (plain C, as it stands) on the same layer: full layer calls,
    first on one host thread, then on one thread per available core (at most
    16, the machine's CPU share per GPU; each thread runs whole calls on its own
    copies, and ctypes releases the GIL during a call).  `value` is the
    all-core wall time per layer call."""
    import threading

    import oracle
    cfg, w = synthetic.layer_inputs(workload, seed=0)
    oc, os_ = oracle.rope_table(cfg["max_ctx"], cfg["head_dim"], cfg["theta"])
    ow = dict(w, rope_cos=oc, rope_sin=os_)

    def calls_until(deadline, counts, i):
        n = 0
        while True:
            oracle.decode_layer(cfg, ow, w["x"], cfg["pos"], w["k_cache"], w["v_cache"])
            n += 1
            if time.perf_counter() >= deadline:
                break
        counts[i] = n

    half = seconds / 2
    counts = [0]
    t0 = time.perf_counter()
    calls_until(t0 + half, counts, 0)
    dt1 = time.perf_counter() - t0
    single_us = dt1 / counts[0] * 1e6
    n_thr = max(1, min(16, len(os.sched_getaffinity(0))))
    counts = [0] * n_thr
    t0 = time.perf_counter()
    ths = [threading.Thread(target=calls_until, args=(t0 + half, counts, i)) for i in range(n_thr)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    dt = time.perf_counter() - t0
    all_us = dt / sum(counts) * 1e6
    return dict(value=round(all_us, 1), unit="us/token/layer", cores=n_thr, kind="oracle",
                single_thread_us=round(single_us, 1), cpu_model=cpu_model(),
                sample=f"{sum(counts)} full decode-layer calls of {workload} (pos {cfg['pos']}) on {n_thr} host "
                       f"threads in {dt:.1f} s, after {dt1:.1f} s of single-thread calls; f64 "
                       f"accumulation, plain C, no SIMD intrinsics")


def context_figures(us_layer):
    """The pages' own figures, on other hardware and other workloads: context,
    not targets."""
    return {
        "hf2q_decode_tok_per_s": {
            "value": [86, 105], "target": 102, "hardware": "Apple M5 Max",
            "workload": "Gemma-4 26B MoE decode (whole model, DWQ weights)",
            "source": "Target Inference Architecture: hf2q on mlx-native, header (Phase 0 verdict and target)"},
        "larql_amx_f32_TFLOPS": {
            "value": [2, 4], "hardware": "Apple M-series AMX through Accelerate (cblas_sgemm)",
            "source": "Inference Engine (larql), Compute Backend: CPU Backend"},
        "this_run_36_layer_stack_tok_per_s": {
            "value": round(1e6 / (36 * us_layer), 1),
            "note": "36 layers of this workload back to back (layers only: no embedding, head or sampling)"},
    }


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=synthetic.HEADLINE, choices=list(synthetic.WORKLOADS))
    ap.add_argument("--min-stack-bytes", type=float, default=2.0e9)
    ap.add_argument("--rounds", type=int, default=5, help="rounds of per-launch kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--headline-only", action="store_true", help="skip the other configs and the MoE block")
    ap.add_argument("--calib-copy", action="store_true", help="also run the PMC calibration copy (1 GiB)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary from two rocprofv3 --pmc output folders and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write the kernel-trace summary from a rocprofv3 --kernel-trace folder and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar=("NAME", "DIR"),
                    help="write profiles/NAME.txt: per-kernel counter averages from rocprofv3 --pmc folders, and exit")
    ap.add_argument("--only", choices=["attn_long_context", "moe_block", "lm_head", "q8_matmul", "q8_matmul_prefill"],
                    help="run only this extra measurement (for profiling) and print its JSON")
    ap.add_argument("--command", default="", help="the profiled command, recorded in the summary")
    ap.add_argument("--profiles-dir", default=PROFILES, help="where the summaries are written")
    args = ap.parse_args()
    if args.summarize_pmc:
        os.makedirs(args.profiles_dir, exist_ok=True)
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      os.path.join(args.profiles_dir, f"decode_layer_{args.workload}.pmc.txt"), args.command)
        return
    if args.summarize_trace:
        os.makedirs(args.profiles_dir, exist_ok=True)
        summarize_trace(args.summarize_trace, args.profiles_dir, args.workload, args.command, args.steps, args.warmup,
                        args.rounds)
        return
    if args.summarize_counters:
        name, dirs = args.summarize_counters[0], args.summarize_counters[1:]
        os.makedirs(args.profiles_dir, exist_ok=True)
        summarize_counters(dirs, os.path.join(args.profiles_dir, name + ".txt"), args.command,
                           f"rocprofv3 counters per kernel ({name})")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import q8_matvec_gqa_amd as lq  # noqa: F401  (fails loudly without liblq.so)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.only:
        fn = {"attn_long_context": lambda: measure_attn_context(max(5, args.steps // 5), torch),
              "moe_block": lambda: measure_moe(list(synthetic.MOE_WORKLOADS)[0], max(10, args.steps // 2), torch),
              "lm_head": lambda: measure_head(max(10, args.steps // 2), torch),
              "q8_matmul": lambda: measure_matmul(32, max(5, args.steps // 10), torch),
              "q8_matmul_prefill": lambda: measure_matmul(512, max(3, args.steps // 20), torch)}[args.only]
        print(json.dumps({args.only: fn()}), flush=True)
        return
    cfg = synthetic.layer_cfg(args.workload)
    m = measure_layer(args.workload, args.steps, args.warmup, args.rounds, args.min_stack_bytes, torch)
    per, us_layer, R = m["per"], m["us_layer"], m["R"]
    per_layer_bytes = m["layer_bytes"]
    for tag, p in per.items():
        gbs = p["bytes"] / (p["avg_us"] * 1e3)
        log(f"{tag:16s} {p['avg_us']:8.2f} us avg ({p['min_us']:.2f} min) {gbs:8.1f} GB/s  [{p['kernel']}]")
    dom_tag = "gate_up_matvec" if "gate_up_matvec" in per else "qkv_matvec"
    dom = per[dom_tag]
    dom_gbs = dom["bytes"] / (dom["avg_us"] * 1e3)
    result = {
        "metric": "decode-layer us/token + achieved HBM GB/s (% peak), Q8_0 matvec & GQA attn",
        "value": round(us_layer, 3),
        "unit": "us/token/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8xi8->i32 (Q8_0) + f32; bf16 KV",
        "data": "synthetic",
        "config": {"workload": args.workload, "hidden": cfg["hidden"], "n_q": cfg["n_q"], "n_kv": cfg["n_kv"],
                   "head_dim": cfg["head_dim"], "ffn": cfg["ffn"], "kv_len": cfg["pos"] + 1,
                   "kv_dtype": "bf16" if cfg["kv_dtype"] else "f32", "layers_per_step": R,
                   "tokens_per_step": 1, "graph": True},
        "layer_bytes": per_layer_bytes,
        "layer_GBps": round(per_layer_bytes / (us_layer * 1e3), 1),
        "eager_us_per_layer": round(m["eager_us_layer"], 3),
        "roofline": {"bound": "hbm", "kernel": dom["kernel"] + " (" + dom_tag + ")", "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic(args.workload, dom_tag),
                     "bytes_per_launch": dom["bytes"], "avg_launch_us": round(dom["avg_us"], 3),
                     "trace_avg_launch_us": load_trace_avg(args.workload, dom_tag, "timed"),
                     "trace_graph_avg_launch_us": load_trace_avg(args.workload, dom_tag, "graph")},
        "attn_roofline": dict(m["attn"], traffic_split=load_traffic(args.workload, "attn_split")),
        "matvec_total": m["matvec"],
        "kernels": {t: {k: (round(v, 3) if isinstance(v, float) else v) for k, v in p.items()}
                    for t, p in per.items()},
    }
    del m
    torch.cuda.empty_cache()
    if not args.headline_only:
        others = {}
        for wl in synthetic.WORKLOADS:
            if wl == args.workload:
                continue
            o = measure_layer(wl, max(10, args.steps // 4), 3, 2, args.min_stack_bytes, torch)
            others[wl] = {"us_per_layer": round(o["us_layer"], 3), "layers_per_step": o["R"],
                          "layer_bytes": o["layer_bytes"],
                          "layer_GBps": round(o["layer_bytes"] / (o["us_layer"] * 1e3), 1),
                          "layer_frac": round(o["layer_bytes"] / (o["us_layer"] * 1e3) / HBM_PEAK_GBS, 4),
                          "attn": o["attn"], "matvec": o["matvec"],
                          "kernels_us": {t: round(p["avg_us"], 3) for t, p in o["per"].items()}}
            del o
            torch.cuda.empty_cache()
        result["other_configs"] = others
        # the headline layer with GGML-format projections (same launches, other weight bytes)
        gl = {}
        for name, fm in (("gu_q6_k+dn_q4_0", {"gu": "q6_k", "dn": "q4_0"}),
                         ("all_q4_0", {"qkv": "q4_0", "o": "q4_0", "gu": "q4_0", "dn": "q4_0"}),
                         ("all_q6_k", {"qkv": "q6_k", "o": "q6_k", "gu": "q6_k", "dn": "q6_k"})):
            o = measure_layer(args.workload, max(10, args.steps // 4), 3, 2, args.min_stack_bytes, torch, formats=fm)
            gl[name] = {"us_per_layer": round(o["us_layer"], 3), "layers_per_step": o["R"],
                        "layer_bytes": o["layer_bytes"],
                        "layer_GBps": round(o["layer_bytes"] / (o["us_layer"] * 1e3), 1),
                        "layer_frac": round(o["layer_bytes"] / (o["us_layer"] * 1e3) / HBM_PEAK_GBS, 4),
                        "matvec": o["matvec"],
                        "kernels_us": {t: round(p["avg_us"], 3) for t, p in o["per"].items()}}
            del o
            torch.cuda.empty_cache()
        result["ggml_layers"] = gl
        for name in synthetic.MOE_WORKLOADS:
            result["moe_block"] = measure_moe(name, max(10, args.steps // 2), torch)
            torch.cuda.empty_cache()
        result["lm_head"] = measure_head(max(10, args.steps // 2), torch)
        torch.cuda.empty_cache()
        result["q8_matmul"] = measure_matmul(32, max(5, args.steps // 10), torch)
        torch.cuda.empty_cache()
        result["q8_matmul_prefill"] = measure_matmul(512, max(3, args.steps // 20), torch)
        result["attn_long_context"] = measure_attn_context(max(5, args.steps // 5), torch)
        torch.cuda.empty_cache()
        result["ggml_formats"] = measure_ggml_formats(max(5, args.steps // 5), torch)
        torch.cuda.empty_cache()
        result["moe_ggml_formats"] = measure_moe_formats(max(5, args.steps // 5), torch)
        result["moe_block_ggml"] = measure_moe_block_ggml(max(5, args.steps // 5), torch)
        torch.cuda.empty_cache()
    if args.calib_copy:
        calib_copy(torch)
    result["context"] = context_figures(us_layer)
    if not args.no_cpu:
        log("oracle CPU baseline")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

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
def device_layer_inputs(cfg, seed, torch):
    """Layer inputs drawn directly on the GPU (same distributions as
    synthetic.py; bf16 KV drawn as the top half of float32 normals)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]

    def q8(rows, cols):
        qs = torch.randint(-127, 128, (rows, cols), dtype=torch.int8, device="cuda", generator=g)
        d = (torch.randn(rows, cols // 32, device="cuda", generator=g).abs() * (0.02 / 127)).half()
        return qs, d.view(torch.int16)

    def gamma(n):
        return 1.0 + 0.1 * torch.randn(n, device="cuda", generator=g)

    def kv():
        a = torch.randn(nkv, cfg["max_ctx"], hd, device="cuda", generator=g)
        if cfg["kv_dtype"] == 0:
            return a
        return (a.view(torch.int32) >> 16).to(torch.int16)

    w = {"x": torch.randn(H, device="cuda", generator=g), "g_in": gamma(H)}
    w["qkv_qs"], w["qkv_d"] = q8(nq * hd + 2 * nkv * hd, H)
    w["g_q"], w["g_k"] = gamma(hd), gamma(hd)
    w["o_qs"], w["o_d"] = q8(H, nq * hd)
    w["g_post"] = gamma(H)
    if I:
        w["gu_qs"], w["gu_d"] = q8(2 * I, H)
        w["dn_qs"], w["dn_d"] = q8(H, I)
    w["k_cache"], w["v_cache"] = kv(), kv()
    return w


def layer_bytes(cfg):
    """Algorithmic HBM bytes of one decode layer: Q8_0 weights at 34 B per 32,
    the KV positions attended (read once), activations in and out."""
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    es = 4 if cfg["kv_dtype"] == 0 else 2
    L = min(cfg["window"], cfg["pos"] + 1) if cfg["window"] else cfg["pos"] + 1
    mats = [(nq * hd + 2 * nkv * hd, H), (H, nq * hd)] + ([(2 * I, H), (H, I)] if I else [])
    mv = sum(matvec_bytes(r, c) for r, c in mats)
    attn = attn_bytes(nq, nkv, hd, L, es)
    return mv, attn


def matvec_bytes(rows, cols, residual=False):
    return rows * cols * 34 // 32 + cols + cols // 16 + 4 * rows + (4 * rows if residual else 0)


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


def layer_kernels(cfg, nsplit_used):
    """Names and algorithmic bytes of the kernels the decode layer launches,
    in launch order (matching lq_decode_layer_timed's events)."""
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    es = 4 if cfg["kv_dtype"] == 0 else 2
    pos = cfg["pos"]
    L = min(cfg["window"], pos + 1) if cfg["window"] else pos + 1
    qkv_rows = nq * hd + 2 * nkv * hd
    q8w = lambda r, c: r * c * 34 // 32
    ks = [("qkv_matvec", "k_mv<NCH=%d,NORM,STORE>" % math.ceil(H / 1024),
           q8w(qkv_rows, H) + 8 * H + 4 * qkv_rows),
          ("attn_split", "k_attn_split", attn_bytes(nq, nkv, hd, L, es) + 4 * qkv_rows)]
    if nsplit_used:
        ks.append(("attn_combine", "k_attn_combine", 0))
    if cfg["kind"] == 0:
        ks += [("o_matvec", "k_mv<NCH=%d,QUANT,RESID>" % math.ceil(nq * hd / 1024), q8w(H, nq * hd) + 4 * nq * hd + 8 * H),
               ("gate_up_matvec", "k_mv<NCH=%d,NORM,SWIGLU>" % math.ceil(H / 1024), q8w(2 * I, H) + 8 * H + 4 * I),
               ("down_matvec", "k_mv<NCH=%d,QUANT,RESID>" % math.ceil(I / 1024), q8w(H, I) + 4 * I + 8 * H)]
    else:
        ks += [("o_matvec", "k_mv<NCH=%d,QUANT,STORE>" % math.ceil(nq * hd / 1024), q8w(H, nq * hd) + 4 * nq * hd + 4 * H),
               ("post_norm_add", "k_rmsnorm_add", 16 * H)]
    return ks


def kernel_measurements(cfg, layers, xs, torch, rounds):
    """Times every kernel of the decode layer with start/stop HIP events that
    the runtime stamps at each dispatch of the layer (lq_decode_layer_timed),
    on the stream the layer runs on."""
    import q8_matvec_gqa_amd as lq
    n_k = lq.lq_decode_layer_kernel_count(layers[0].desc)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_k)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    names = layer_kernels(cfg, n_k == (6 if cfg["kind"] == 0 else 5))
    assert len(names) == n_k, (len(names), n_k)
    times = [[] for _ in range(n_k)]
    for r in range(rounds + 1):
        for li, lay in enumerate(layers):
            lq.lq_decode_layer_timed(lay.desc, xs[li], cfg["pos"], None, lay.ws, lay.ws_bytes, evs)
            torch.cuda.synchronize()
            if r == 0:
                continue                      # warm round
            for k in range(n_k):
                times[k].append(evs[2 * k].elapsed_time(evs[2 * k + 1]) * 1e3)
    per = {}
    for (tag, kernel, b), ts in zip(names, times):
        per[tag] = dict(kernel=kernel, launches=len(ts), avg_us=float(np.mean(ts)), min_us=float(np.min(ts)),
                        bytes=int(b))
    return per


def cpu_baseline(workload, seconds):
    import oracle
    cfg, w = synthetic.layer_inputs(workload, seed=0)
    oc, os_ = oracle.rope_table(cfg["max_ctx"], cfg["head_dim"], cfg["theta"])
    ow = dict(w, rope_cos=oc, rope_sin=os_)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.decode_layer(cfg, ow, w["x"], cfg["pos"], w["k_cache"], w["v_cache"])
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return dict(value=round(dt / n * 1e6, 1), unit="us/token/layer", cores=1, kind="oracle",
                sample=f"{n} full decode-layer calls of {workload} (pos {cfg['pos']}) on one host thread, "
                       f"{dt:.1f} s; f64 accumulation, plain C, no SIMD intrinsics")


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=synthetic.HEADLINE, choices=list(synthetic.WORKLOADS))
    ap.add_argument("--min-stack-bytes", type=float, default=2.0e9)
    ap.add_argument("--rounds", type=int, default=5, help="rounds of per-launch kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import q8_matvec_gqa_amd as lq  # noqa: F401  (fails loudly without liblq.so)
    from q8_matvec_gqa_amd.layers import DeviceLayer

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synthetic.layer_cfg(args.workload)
    mv_b, at_b = layer_bytes(cfg)
    per_layer_bytes = mv_b + at_b
    R = max(8, math.ceil(args.min_stack_bytes / per_layer_bytes))
    log(f"workload {args.workload}: {per_layer_bytes / 1e6:.1f} MB/layer, stack of {R} layers")
    layers, xs = [], []
    for i in range(R):
        w = device_layer_inputs(cfg, seed=1000 + i, torch=torch)
        layers.append(DeviceLayer(cfg, w, torch))
        xs.append(w["x"])
    torch.cuda.synchronize()
    log("stack built; timing graph replays")
    ms_step, eager_ms = time_stack(layers, xs, cfg["pos"], args.steps, args.warmup, torch)
    us_layer = ms_step * 1e3 / R
    log(f"{us_layer:.2f} us/token/layer (graph), eager {eager_ms * 1e3 / R:.2f}")
    per = kernel_measurements(cfg, layers, xs, torch, args.rounds)
    dom_tag = "gate_up_matvec" if "gate_up_matvec" in per else "qkv_matvec"
    dom = per[dom_tag]
    dom_gbs = dom["bytes"] / (dom["avg_us"] * 1e3)
    at_us = per["attn_split"]["avg_us"] + (per["attn_combine"]["avg_us"] if "attn_combine" in per else 0.0)
    at_bytes = per["attn_split"]["bytes"]
    at_gbs = at_bytes / (at_us * 1e3)
    mv_tags = [t for t in per if t.endswith("_matvec")]
    mv_us = sum(per[t]["avg_us"] for t in mv_tags)
    mv_bytes = sum(per[t]["bytes"] for t in mv_tags)
    for tag, p in per.items():
        gbs = p["bytes"] / (p["avg_us"] * 1e3)
        log(f"{tag:16s} {p['avg_us']:8.2f} us avg ({p['min_us']:.2f} min) {gbs:8.1f} GB/s  [{p['kernel']}]")
    result = {
        "metric": "decode-layer us/token + achieved HBM GB/s (% peak), Q8_0 matvec & GQA attn",
        "value": round(us_layer, 3),
        "unit": "us/token/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
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
        "eager_us_per_layer": round(eager_ms * 1e3 / R, 3),
        "roofline": {"bound": "hbm", "kernel": dom["kernel"] + " (" + dom_tag + ")", "achieved": round(dom_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": dom["bytes"], "avg_launch_us": round(dom["avg_us"], 3)},
        "attn_roofline": {"bound": "hbm", "kernel": "k_attn_split+k_attn_combine", "achieved": round(at_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(at_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": at_bytes, "avg_launch_us": round(at_us, 3)},
        "matvec_total": {"us": round(mv_us, 3), "bytes": mv_bytes, "GBps": round(mv_bytes / (mv_us * 1e3), 1),
                         "frac": round(mv_bytes / (mv_us * 1e3) / HBM_PEAK_GBS, 4)},
        "kernels": {t: {k: (round(v, 3) if isinstance(v, float) else v) for k, v in p.items()}
                    for t, p in per.items()},
    }
    if not args.no_cpu:
        log("oracle CPU baseline")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

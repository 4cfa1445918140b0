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


def time_launches(fns, torch, rounds):
    """Per-launch HIP-event timing on the current stream (the one the library
    launches on).  fns: list of (tag, callable).  Returns {tag: [ms, ...]}."""
    out = {}
    for _ in range(rounds):
        evs = []
        for tag, fn in fns:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((tag, a, b))
        torch.cuda.synchronize()
        for tag, a, b in evs:
            out.setdefault(tag, []).append(a.elapsed_time(b))
    return out


def kernel_measurements(cfg, layers, torch, rounds):
    import q8_matvec_gqa_amd as lq
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    es = 4 if cfg["kv_dtype"] == 0 else 2
    pos = cfg["pos"]
    start = max(0, pos - cfg["window"] + 1) if cfg["window"] else 0
    L = pos - start + 1
    # matvec launches exactly as the layer makes them (same entry, same shapes)
    shapes = [("qkv", nq * hd + 2 * nkv * hd, H, False), ("o", H, nq * hd, True)]
    if I:
        shapes += [("gate_up", 2 * I, H, False), ("down", H, I, True)]
    scratch = {}
    fns = []
    for li, lay in enumerate(layers):
        t = lay.t
        for tag, rows, cols, res in shapes:
            key = {"qkv": "qkv", "o": "o", "gate_up": "gu", "down": "dn"}[tag]
            W = lq.q8_weight(t[key + "_qs"], t[key + "_d"])
            if cols not in scratch:
                scratch[cols] = (torch.randint(-127, 128, (cols,), dtype=torch.int8, device="cuda"),
                                 (torch.rand(cols // 32, device="cuda") * 0.01 + 0.001).half().view(torch.int16))
            xq, xd = scratch[cols]
            y = torch.empty(rows, device="cuda")
            r = torch.zeros(rows, device="cuda") if res else None
            fns.append((f"matvec:{tag}", (lambda W=W, xq=xq, xd=xd, r=r, y=y:
                                          lq.lq_q8_matvec(W, xq, xd, r, y))))
    # attention launches as the layer makes them
    ws_need = lq.lq_gqa_decode_attn_workspace_size(nq, nkv, hd, L)
    ws = torch.empty(max(ws_need, 256), dtype=torch.uint8, device="cuda")
    q = torch.randn(nq * hd, device="cuda")
    o = torch.empty(nq * hd, device="cuda")
    for lay in layers:
        kc, vc = lay.t["k_cache"], lay.t["v_cache"]
        fns.append(("attn", (lambda kc=kc, vc=vc: lq.lq_gqa_decode_attn(
            q, nq, nkv, hd, kc, vc, cfg["kv_dtype"], cfg["max_ctx"] * hd, hd, cfg["max_ctx"], start, L,
            cfg["attn_scale"], o, ws, ws.numel()))))
    for tag, fn in fns[: len(fns)]:          # warm every launch once
        fn()
    torch.cuda.synchronize()
    times = time_launches(fns, torch, rounds)
    per = {}
    for tag, ts in times.items():
        if tag.startswith("matvec:"):
            name = tag.split(":")[1]
            rows, cols, res = [(r_, c_, s_) for t_, r_, c_, s_ in shapes if t_ == name][0]
            b = matvec_bytes(rows, cols, res)
            kernel = f"k_q8_matvec<NCH={math.ceil(cols / 1024)}>"
        else:
            b = attn_bytes(nq, nkv, hd, L, es)
            kernel = "k_attn_split+k_attn_combine"
        per[tag] = dict(kernel=kernel, launches=len(ts), avg_us=1e3 * float(np.mean(ts)),
                        min_us=1e3 * float(np.min(ts)), bytes=b)
    # group by kernel instance, as a profiler aggregates by kernel name
    groups = {}
    for tag, p in per.items():
        g_ = groups.setdefault(p["kernel"], dict(launches=0, time_us=0.0, bytes=0))
        g_["launches"] += p["launches"]
        g_["time_us"] += p["avg_us"] * p["launches"]
        g_["bytes"] += p["bytes"] * p["launches"]
    return per, groups


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
    per, groups = kernel_measurements(cfg, layers, torch, args.rounds)
    dom = max((g for g in groups if g.startswith("k_q8_matvec")), key=lambda g: groups[g]["time_us"])
    gd = groups[dom]
    dom_bytes = gd["bytes"] / gd["launches"]
    dom_us = gd["time_us"] / gd["launches"]
    dom_gbs = dom_bytes / dom_us / 1e3
    ga = groups["k_attn_split+k_attn_combine"]
    at_us = ga["time_us"] / ga["launches"]
    at_gbs = (ga["bytes"] / ga["launches"]) / at_us / 1e3
    for tag, p in sorted(per.items()):
        log(f"{tag:16s} {p['avg_us']:8.2f} us avg ({p['min_us']:.2f} min) "
            f"{p['bytes'] / p['avg_us'] / 1e3:8.1f} GB/s")
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
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": int(dom_bytes), "avg_launch_us": round(dom_us, 3)},
        "attn_roofline": {"bound": "hbm", "kernel": "k_attn_split+k_attn_combine", "achieved": round(at_gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(at_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": int(ga["bytes"] / ga["launches"]), "avg_launch_us": round(at_us, 3)},
        "kernels": {t: {k: (round(v, 3) if isinstance(v, float) else v) for k, v in p.items()}
                    for t, p in sorted(per.items())},
    }
    if not args.no_cpu:
        log("oracle CPU baseline")
        result["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

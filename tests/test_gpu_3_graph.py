"""HIP graph capture and replay of the composites.

The bench times the decode layer as a captured graph, so replays must give
exactly what eager calls give: each test captures the call once on a side
stream, then replays it several times with unrelated eager work and a
synchronization between replays, and compares every replay bit for bit with
the eager result of the same step.  (The library clears its scratch memory
with kernels, never with memsets, so nothing in a captured graph depends on
a memset node.)
"""
import numpy as np
import pytest

import synthetic

pytestmark = pytest.mark.gpu

lq = pytest.importorskip("q8_matvec_gqa_amd")
from q8_matvec_gqa_amd.layers import DeviceLayer, DeviceMoe  # noqa: E402
from lqtest import dev, host, sync, torch_mod, workspace  # noqa: E402

REPLAYS = 3


def unrelated_eager_work(torch):
    a = torch.randn(1 << 20, device="cuda")
    (a * 2.0 + 1.0).sum().item()
    torch.cuda.synchronize()


def capture(torch, fn):
    """Capture fn(stream) into a graph on a side stream (nothing executes)."""
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,formats", [("tiny_h1024", None), (synthetic.HEADLINE, None),
                                          ("gemma4_global_h2816", None),
                                          (synthetic.HEADLINE, {"gu": "q6_k", "dn": "q4_0"})])
def test_layer_graph_replays(name, formats):
    """Three chained decode steps (x updated in place, the new position's
    k/v rewritten each step): the graph's replays equal the eager steps."""
    torch = torch_mod()
    cfg, w = synthetic.layer_inputs(name, seed=5, formats=formats)
    print(f"[graph] layer {name} formats={formats}", flush=True)
    L = DeviceLayer(cfg, w, torch)

    def reset():
        L.t["k_cache"].copy_(dev(w["k_cache"]))
        L.t["v_cache"].copy_(dev(w["v_cache"]))

    reset()
    x = dev(w["x"])
    eager = []
    for _ in range(REPLAYS):
        L.run(x, cfg["pos"])
        sync()
        eager.append((host(x), host(L.t["k_cache"]).copy()))

    reset()
    xg = dev(w["x"])
    g = capture(torch, lambda s: L.run(xg, cfg["pos"], stream=s))
    for i in range(REPLAYS):
        unrelated_eager_work(torch)
        g.replay()
        sync()
        assert np.array_equal(host(xg), eager[i][0]), f"replay {i}: layer output"
        assert np.array_equal(host(L.t["k_cache"]), eager[i][1]), f"replay {i}: k cache"


def test_moe_block_graph_replays():
    """Routing, gather, id-matvecs and the weighted sum in a graph: every
    replay rebuilds the expert lists and gives the eager output."""
    torch = torch_mod()
    name = list(synthetic.MOE_WORKLOADS)[0]
    cfg, w = synthetic.moe_inputs(name, seed=2)
    print(f"[graph] moe {name}", flush=True)
    M = DeviceMoe(cfg, w, torch)
    x, logits = dev(w["x"]), dev(w["logits"])
    out = torch.empty(cfg["tokens"] * cfg["hidden"], dtype=torch.float32, device="cuda")
    M.run(x, logits, out)
    sync()
    want = host(out)
    out.fill_(7.0)
    g = capture(torch, lambda s: M.run(x, logits, out, stream=s))
    for i in range(REPLAYS):
        unrelated_eager_work(torch)
        out.fill_(float(i + 3))
        g.replay()
        sync()
        assert np.array_equal(host(out), want), f"replay {i}"


@pytest.mark.parametrize("T,rows,cols", [
    (32, 4096, 4096),     # split blocks: partials in the workspace, then the ordered reduce
    (512, 4096, 1024),    # 64 x 64 tiles, no workspace
])
def test_matmul_graph_replays(T, rows, cols):
    """The matmul in a graph, residual aliasing y: each replay adds W x to
    the result of the previous one, as the eager calls do."""
    torch = torch_mod()
    print(f"[graph] matmul T={T} {rows}x{cols}", flush=True)
    r = np.random.default_rng(8)
    wq, wd = synthetic.q8_weight(r, rows, cols)
    xq = r.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = (np.abs(r.standard_normal((T, cols // 32))) * 0.05).astype(np.float16).view(np.uint16)
    y0 = synthetic.activations(r, T, rows)
    W = lq.q8_weight(dev(wq), dev(wd))
    nws = lq.lq_q8_matmul_workspace_size(rows, cols, T)
    assert (nws > 0) == (T <= 32)
    ws = workspace(nws)
    xqd, xdd = dev(xq), dev(xd)
    y = dev(y0)
    eager = []
    for _ in range(REPLAYS):
        lq.lq_q8_matmul(W, xqd, xdd, T, y, y, ws, nws)
        sync()
        eager.append(host(y))
    yg = dev(y0)
    g = capture(torch, lambda s: lq.lq_q8_matmul(W, xqd, xdd, T, yg, yg, ws, nws, stream=s))
    for i in range(REPLAYS):
        unrelated_eager_work(torch)
        g.replay()
        sync()
        assert np.array_equal(host(yg), eager[i]), f"replay {i}"

"""lq_gqa_decode_attn_noalloc: the GQA decode attention with its split
partials in the library's own device scratch array instead of a caller
workspace.  Checked against lq_gqa_decode_attn (same kernels, same plan:
bit-identical outputs) and the oracle (1e-3 rel / 1e-4 abs), on two calls in
a row and a third smaller one, so a stale scratch from an earlier call would
show."""
import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

lq = pytest.importorskip("q8_matvec_gqa_amd")
from lqtest import assert_close, dev, empty, host, sync, workspace  # noqa: E402

# (n_q, n_kv, head_dim, kv dtype, ctx, start, len): the Gemma-global and
# 8B-like attentions, then a smaller call (f32 cache, a window with start > 0)
CASES = [(16, 2, 512, 1, 8192, 0, 8192), (32, 8, 128, 1, 8192, 0, 8192), (16, 8, 64, 0, 256, 20, 100)]


def test_noalloc_matches_workspace_entry_two_calls():
    for n_q, n_kv, hd, dt, ctx, start, ln in CASES:
        print(f"[noalloc] n_q={n_q} n_kv={n_kv} hd={hd} dtype={dt} ctx={ctx} window=[{start}, {start + ln})",
              flush=True)
        r = np.random.Generator(np.random.PCG64(1000 + hd))
        q = synthetic.activations(r, n_q * hd)
        kc = synthetic.kv_cache(r, n_kv, ctx, hd, dt)
        vc = synthetic.kv_cache(r, n_kv, ctx, hd, dt)
        qd, kd, vd = dev(q), dev(kc), dev(vc)
        scale = 1.0 / np.sqrt(hd)
        out_ws, out_na = empty(n_q * hd, np.float32), empty(n_q * hd, np.float32)
        nws = lq.lq_gqa_decode_attn_workspace_size(n_q, n_kv, hd, ln)
        ws = workspace(nws)
        lq.lq_gqa_decode_attn(qd, n_q, n_kv, hd, kd, vd, dt, ctx * hd, hd, ctx, start, ln, scale, out_ws, ws, nws)
        lq.lq_gqa_decode_attn_noalloc(qd, n_q, n_kv, hd, kd, vd, dt, ctx * hd, hd, ctx, start, ln, scale, out_na)
        sync()
        a, b = host(out_na), host(out_ws)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "noalloc differs from the workspace entry point"
        ref = oracle.attention(q, n_q, n_kv, hd, kc, vc, dt, ctx * hd, hd, start, ln, scale)
        assert_close(a, ref, "noalloc attention")


SCRATCH_BYTES = 16 << 20


def test_noalloc_rejects_oversized_partials():
    """A shape whose partials exceed the scratch array is refused on the host.
    The call passes fake aligned addresses, so it is made only after the
    host-side size query shows that this shape needs more than the array
    holds (the entry point then returns before any launch)."""
    n_q, n_kv, hd, ctx = 511 * 8, 511, 512, 4096     # f32 cache: the padded instance, two splits per kv head
    need = lq.lq_gqa_decode_attn_workspace_size(n_q, n_kv, hd, ctx)
    assert need > SCRATCH_BYTES, need                # else the call below would launch on fake addresses
    A = 0x10000
    st = lq.lq_gqa_decode_attn_noalloc(A, n_q, n_kv, hd, A, A, 0, ctx * hd, hd, ctx, 0, ctx, 0.05, A, stream=0,
                                       check=False)
    assert st == lq.LQ_ERR_UNSUPPORTED
    assert "scratch" in lq.lq_last_error()

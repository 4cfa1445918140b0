"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte model behind every GB/s figure, and the kernel-name matching used to
read rocprofv3 output."""
import os
import subprocess
import sys

import bench
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_byte_model():
    """The 8B-like layer's bytes, written out from the storage formats:
    Q8_0 weights at 34 bytes per 32 values, f32 activations, bf16 K and V
    read once over the 8192 positions attended."""
    cfg = synthetic.layer_cfg(synthetic.HEADLINE)
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    assert (H, nq, nkv, hd, I, cfg["pos"] + 1) == (4096, 32, 8, 128, 12288, 8192)
    names = {tag: b for tag, _, b in bench.layer_kernels(cfg, True)}
    q8 = lambda r, c: r * c * 34 // 32
    # gate_up: the weight pair, x and gamma in (f32), the Q8_0 of h out
    assert names["gate_up_matvec"] == q8(2 * I, H) + 4 * H + 4 * H + q8(1, I) == 107000576
    # down: the weight, the Q8_0 of h in, residual in and x out (f32)
    assert names["down_matvec"] == q8(H, I) + q8(1, I) + 4 * H + 4 * H
    # attention: K and V once, q in and the output (f32), plus the projection read back
    kv = 2 * nkv * 8192 * hd * 2
    assert names["attn_split"] == kv + 4 * nq * hd * 2 + 4 * (nq * hd + 2 * nkv * hd)
    mv, at = bench.layer_bytes(cfg)
    assert at == kv + 4 * nq * hd * 2
    assert mv + at == 238765568


def test_rocprof_kernel_name_matching():
    gate_up = "void lq::k_mv<4, 2, 2, 3, 4>(lq::MvArgs)"
    qkv = "void lq::k_mv<4, 2, 2, 0, 8>(lq::MvArgs)"
    assert bench._kernel_match(gate_up, "gate_up_matvec")
    assert not bench._kernel_match(qkv, "gate_up_matvec")


def test_layer_kernel_patterns_are_exclusive():
    """Each kernel the 8B-like layer launches matches exactly one tag of the
    rocprofv3 summaries (names as rocprofv3 prints them)."""
    names = {
        "qkv_matvec": "void lq::k_mv<4, 2, 2, 0, 8>(lq::MvArgs)",
        "attn_split": "void lq::k_attn_split<unsigned short, 16, 4, 8, 16, true, 2, 4>(lq::(anonymous "
                      "namespace)::AttnArgs)",
        "attn_combine": "lq::k_attn_combine(lq::(anonymous namespace)::AttnArgs)",
        "o_matvec": "void lq::k_mv<4, 2, 1, 1, 8>(lq::MvArgs)",
        "gate_up_matvec": "void lq::k_mv<4, 2, 2, 3, 4>(lq::MvArgs)",
        "down_matvec": "void lq::k_mv<12, 1, 0, 1, 4>(lq::MvArgs)",
    }
    pats = bench.layer_kernel_patterns(synthetic.layer_cfg(synthetic.HEADLINE))
    assert set(pats) == set(names)
    for tag, name in names.items():
        hits = [t for t, p in pats.items() if p.search(name)]
        assert hits == [tag], (name, hits)


def test_context_figures_are_the_pages():
    c = bench.context_figures(57.5)
    assert c["hf2q_decode_tok_per_s"]["value"] == [86, 105]
    assert c["larql_amx_f32_TFLOPS"]["value"] == [2, 4]


def test_trace_summary_takes_the_workload_instance_dispatched_first(tmp_path):
    """Two instances match the gate_up pattern (the headline's and another
    workload's 16-wave one, dispatched later): the per-phase rows come from
    the headline's, whose dispatches come first in the trace."""
    import csv
    trace = tmp_path / "trace"
    trace.mkdir()
    head = "void lq::k_mv<4, 2, 2, 3, 4>(lq::MvArgs)"
    other = "void lq::k_mv<4, 2, 2, 3, 16>(lq::MvArgs)"
    rows = []
    for i in range(315):                       # the headline's dispatches: 10 us each
        rows.append((head, 1_000_000 + 100_000 * i, 1_000_000 + 100_000 * i + 10_000))
    for i in range(400):                       # another workload's, later: 5 us each
        rows.append((other, 90_000_000 + 100_000 * i, 90_000_000 + 100_000 * i + 5_000))
    with open(trace / "bt_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)
    bench.summarize_trace(str(trace), str(tmp_path), synthetic.HEADLINE, "test", steps=20, warmup=5, rounds=5)
    text = (tmp_path / f"decode_layer_{synthetic.HEADLINE}.trace.txt").read_text()
    timed = [line for line in text.splitlines() if line.startswith("gate_up_matvec@timed")]
    assert timed == ["gate_up_matvec@timed | 45 | 10.000 | 10.000 | 10.000 | 10.000"]

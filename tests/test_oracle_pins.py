"""Pins of the CPU oracle against things other than itself.

Every check here compares the oracle with a closed form, an invariant, a
hand-derived fixture (tests/golden/), a library routine (numpy, scipy,
torch CPU) or brute force over a differently-ordered computation.  The
checks are chosen so that a plausible slip (dropped term, wrong sign, wrong
pairing, transposed operand, wrong rounding rule) fails at least one of them;
tests/test_oracle_mutants.py plants such slips in copies of the oracle and
verifies that.
"""
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------
def pin_f16():
    # every binary16 pattern: decode against numpy, and encode round-trips
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = allbits.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(allbits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(got[~finite]) == np.isnan(ref[~finite]))
    enc = oracle.f32_to_f16(ref[finite])
    assert np.array_equal(enc, allbits[finite])
    # midpoints between neighbours (ties), and values just off them, vs numpy's cast
    pos = allbits[(allbits < 0x7bff)]
    lo = pos.view(np.float16).astype(np.float64)
    hi = (pos + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)           # exact in float32
    probes = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)),
                             np.nextafter(mid, np.float32(-np.inf)), -mid])
    probes = probes[::7]                               # a spread sample keeps it quick
    with np.errstate(over="ignore"):
        want = probes.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(probes), want)
    # overflow edge: 65504 is the largest finite, 65520 rounds to infinity
    assert oracle.f32_to_f16([65504.0, 65519.996, 65520.0])[2] == 0x7c00
    assert oracle.f32_to_f16([65519.996])[0] == 0x7bff


def pin_bf16():
    import torch
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),     # f32 subnormals
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, both parities of bit 16
    u = rng.integers(0, 2 ** 31, size=2000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xffff0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), want)
    back = oracle.bf16_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_f16_conversion():
    pin_f16()


def test_bf16_conversion():
    pin_bf16()


# ----------------------------------------------------------------------------
# Q8_0 quantizer
# ----------------------------------------------------------------------------
def load_golden_blocks():
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, "q8_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# case:"):
                cur = {"name": line.split(":", 1)[1].split()[0]}
            elif line.startswith("x:"):
                cur["x"] = np.array([float(v) for v in line[2:].split()], dtype=np.float32)
            elif line.startswith("q:"):
                cur["q"] = np.array([int(v) for v in line[2:].split()], dtype=np.int8)
            elif line.startswith("d:"):
                cur["d"] = int(line[2:].strip(), 16)
                cases.append(cur)
    return cases


def pin_quantize_golden():
    cases = load_golden_blocks()
    assert len(cases) == 7
    for c in cases:
        assert c["x"].size == 32 and c["q"].size == 32, c["name"]
        qs, d = oracle.q8_quantize(c["x"])
        assert np.array_equal(qs, c["q"]), (c["name"], qs, c["q"])
        assert int(d[0]) == c["d"], (c["name"], hex(int(d[0])))


def pin_quantize_invariants():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 256)) * rng.uniform(1e-3, 1e3, size=(64, 1))).astype(np.float32)
    qs, d = oracle.q8_quantize(x)
    xb = x.reshape(64, 8, 32).astype(np.float64)
    qb = qs.reshape(64, 8, 32).astype(np.float64)
    amax = np.abs(x.reshape(64, 8, 32)).max(axis=2)
    dfl = (amax / np.float32(127)).astype(np.float32)              # float division, as defined
    # stored scale = f16 image of amax/127 (numpy's float16 cast as the rounding authority)
    assert np.array_equal(d.reshape(64, 8), dfl.astype(np.float16).view(np.uint16))
    # the element with the largest magnitude maps to +-127, and every code is
    # within half a step of x / d
    assert np.all(np.abs(qb).max(axis=2) == 127)
    err = np.abs(xb / dfl[..., None].astype(np.float64) - qb)
    assert err.max() <= 0.5 + 1e-4
    assert np.all(np.sign(qb) * np.sign(xb) >= 0)                  # no sign flips


def test_quantize_golden():
    pin_quantize_golden()


def test_quantize_invariants():
    pin_quantize_invariants()


# ----------------------------------------------------------------------------
# block dots and matvec
# ----------------------------------------------------------------------------
def pin_block_dots():
    rng = np.random.default_rng(3)
    rows, cols = 7, 96                           # non-square, several blocks
    wq = rng.integers(-128, 128, size=(rows, cols), dtype=np.int8)
    xq = rng.integers(-128, 128, size=cols, dtype=np.int8)
    got = oracle.q8_block_dots(wq, xq)
    want = (wq.astype(np.int64) * xq.astype(np.int64)).reshape(rows, cols // 32, 32).sum(axis=2)
    assert np.array_equal(got, want)
    # extremes: 32 * (-128) * (-128) = 524288 fits int32 exactly
    ext = oracle.q8_block_dots(np.full((1, 32), -128, np.int8), np.full(32, -128, np.int8))
    assert ext[0, 0] == 524288
    ext = oracle.q8_block_dots(np.full((1, 32), 127, np.int8), np.full(32, -128, np.int8))
    assert ext[0, 0] == -32 * 127 * 128


def pin_matvec():
    rng = np.random.default_rng(4)
    rows, cols = 37, 160
    wq, wd = synthetic.q8_weight(rng, rows, cols)
    xq = rng.integers(-127, 128, size=cols, dtype=np.int8)
    xd = (np.abs(rng.normal(0, 0.05, size=cols // 32)).astype(np.float16)).view(np.uint16)
    res = rng.standard_normal(rows).astype(np.float32)
    # brute force: dequantize each operand with numpy's f16 decode, then one f64 dot
    wdq = wq.astype(np.float64) * np.repeat(wd.view(np.float16).astype(np.float64), 32, axis=1)
    xdq = xq.astype(np.float64) * np.repeat(xd.view(np.float16).astype(np.float64), 32)
    want = wdq @ xdq
    got = oracle.q8_matvec(wq, wd, xq, xd).astype(np.float64)
    assert np.allclose(got, want, rtol=2e-7, atol=1e-12 * np.abs(want).max())
    got_r = oracle.q8_matvec(wq, wd, xq, xd, residual=res).astype(np.float64)
    assert np.allclose(got_r, want + res, rtol=2e-7, atol=1e-7)
    # one-hot: a single non-zero code gives d_w * d_x * q_w * q_x exactly
    xq1 = np.zeros(cols, np.int8); xq1[70] = -3
    xd1 = np.zeros(cols // 32, np.uint16); xd1[2] = 0x3800          # 0.5
    y1 = oracle.q8_matvec(wq, wd, xq1, xd1)
    exact = wq[:, 70].astype(np.float64) * -3 * 0.5 * wd[:, 2].view(np.float16).astype(np.float64)
    assert np.array_equal(y1.astype(np.float64), exact.astype(np.float32).astype(np.float64))


def test_block_dots():
    pin_block_dots()


def test_matvec():
    pin_matvec()


# ----------------------------------------------------------------------------
# RMSNorm, RoPE, SwiGLU
# ----------------------------------------------------------------------------
def pin_rmsnorm():
    n = 96
    c = 3.0
    g = np.linspace(0.5, 1.5, n).astype(np.float32)
    y = oracle.rmsnorm(np.full(n, c, np.float32), g, eps=1e-6)
    want = g.astype(np.float64) * c / math.sqrt(c * c + 1e-6)
    assert np.allclose(y, want, rtol=1e-7, atol=0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal(n).astype(np.float32) * 7
    u = oracle.rmsnorm(x, None, eps=0.0).astype(np.float64)
    assert abs(np.mean(u * u) - 1.0) < 1e-6                       # unit RMS
    assert np.all(np.sign(u) == np.sign(x))
    # scale invariance and per-element gamma
    assert np.allclose(oracle.rmsnorm(x * 4, None, eps=0.0), u, rtol=1e-6)
    yg = oracle.rmsnorm(x, g, eps=0.0).astype(np.float64)
    assert np.allclose(yg, u * g, rtol=1e-6)


def pin_rope():
    hd, theta = 64, 1e6
    cos_t, sin_t = oracle.rope_table(40, hd, theta)
    # table entries against the math library
    for p, i in [(0, 0), (1, 0), (7, 3), (39, 31), (13, 17)]:
        a = p * theta ** (-2.0 * i / hd)
        assert cos_t[p, i] == np.float32(math.cos(a)) and sin_t[p, i] == np.float32(math.sin(a))
    rng = np.random.default_rng(6)
    x = rng.standard_normal(hd).astype(np.float32)
    # pos 0 is the identity
    assert np.array_equal(oracle.rope_neox(x, cos_t[0], sin_t[0]), x)
    # NeoX pairing and rotation direction: e_0 rotates into (cos, sin) on (0, hd/2)
    e0 = np.zeros(hd, np.float32); e0[0] = 1
    r = oracle.rope_neox(e0, cos_t[5], sin_t[5])
    assert r[0] == cos_t[5, 0] and r[hd // 2] == sin_t[5, 0] and np.count_nonzero(r) == 2
    # pair norms preserved
    y = oracle.rope_neox(x, cos_t[9], sin_t[9]).astype(np.float64)
    xx = x.astype(np.float64)
    n0 = xx[:hd // 2] ** 2 + xx[hd // 2:] ** 2
    n1 = y[:hd // 2] ** 2 + y[hd // 2:] ** 2
    assert np.allclose(n0, n1, rtol=1e-5)
    # relative position: <R(m) q, R(n) k> depends on m - n only
    k = rng.standard_normal(hd).astype(np.float32)
    for m, n in [(30, 10), (25, 5), (39, 19)]:
        lhs = np.dot(oracle.rope_neox(x, cos_t[m], sin_t[m]).astype(np.float64),
                     oracle.rope_neox(k, cos_t[n], sin_t[n]).astype(np.float64))
        rhs = np.dot(oracle.rope_neox(x, cos_t[m - n], sin_t[m - n]).astype(np.float64),
                     k.astype(np.float64))
        assert abs(lhs - rhs) < 1e-4 * (1 + abs(rhs))


def pin_silu():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5, -0.75], np.float32)
    u = np.array([5.0, 2.0, 2.0, 1.0, 1.0, -3.0, 4.0], np.float32)
    h = oracle.silu_mul(g, u).astype(np.float64)
    want = scipy.special.expit(g.astype(np.float64)) * g * u
    assert h[0] == 0.0
    assert np.allclose(h, want, rtol=1e-7, atol=1e-30)
    assert abs(h[3] - 30.0) < 1e-6                                 # silu(z) -> z


def pin_lm_head():
    rng = np.random.default_rng(7)
    vocab, hidden = 48, 96
    wf = (rng.standard_normal((vocab, hidden)) * 0.05).astype(np.float16)
    w = wf.view(np.uint16)
    x = rng.standard_normal(hidden).astype(np.float32)
    gamma = (1.0 + 0.1 * rng.standard_normal(hidden)).astype(np.float32)
    # no norm, no cap: numpy's own f16 decode and an f64 product
    want = wf.astype(np.float64) @ x.astype(np.float64)
    got = oracle.lm_head(w, x, norm=False)
    assert np.allclose(got, want, rtol=1e-6, atol=1e-30)
    # one-hot input: a single term, n_c = gamma_c * s / sqrt(s^2 / hidden + eps)
    c, sv, eps = 17, 3.0, 1e-6
    e = np.zeros(hidden, np.float32)
    e[c] = sv
    nc = np.float32(gamma[c] * sv / math.sqrt(sv * sv / hidden + eps))
    got = oracle.lm_head(w, e, gamma, norm=True, eps=eps)
    assert np.allclose(got, wf[:, c].astype(np.float64) * float(nc), rtol=1e-6)
    # the norm: a constant input and an all-ones weight give hidden * c / sqrt(c^2 + eps)
    ones = np.full((3, hidden), 1.0, np.float16).view(np.uint16)
    got = oracle.lm_head(ones, np.full(hidden, 0.5, np.float32), None, norm=True, eps=eps)
    assert np.allclose(got, hidden * 0.5 / math.sqrt(0.25 + eps), rtol=1e-6)
    # softcap: cap * tanh(y / cap); cap * atanh(1/2) maps to cap / 2, large values saturate
    cap = 30.0
    big = np.zeros((4, hidden), np.float16)
    big[0, 0] = cap * math.atanh(0.5) / 1.0
    big[1, 0] = 2000.0
    big[2, 0] = -2000.0
    big[3, 0] = 0.01
    one = np.zeros(hidden, np.float32)
    one[0] = 1.0
    got = oracle.lm_head(big.view(np.uint16), one, norm=False, cap=cap).astype(np.float64)
    y0 = float(big[0, 0])
    assert abs(got[0] - cap * math.tanh(y0 / cap)) < 1e-5 and abs(got[0] - cap / 2) < 0.02
    assert abs(got[1] - cap) < 1e-5 and abs(got[2] + cap) < 1e-5
    assert abs(got[3] - float(big[3, 0])) < 1e-7


def test_lm_head():
    pin_lm_head()


def pin_gelu():
    z = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.5, -2.5, 10.0, -10.0, 0.03], np.float32)
    one = np.ones_like(z)
    h = oracle.gelu_mul(z, one).astype(np.float64)
    hn = oracle.gelu_mul(-z, one).astype(np.float64)
    assert h[0] == 0.0
    # the tanh form is odd around z/2: gelu(z) - gelu(-z) = z exactly
    assert np.allclose(h - hn, z.astype(np.float64), rtol=1e-6, atol=1e-7)
    # and it approximates z * Phi(z) (the normal CDF) to well under 1e-3
    exact = z.astype(np.float64) * scipy.special.ndtr(z.astype(np.float64))
    assert np.max(np.abs(h - exact)) < 1e-3
    assert abs(h[7] - 10.0) < 1e-6 and abs(h[8]) < 1e-6
    # the up factor multiplies
    u = np.full_like(z, -3.0)
    assert np.allclose(oracle.gelu_mul(z, u), -3.0 * h, rtol=1e-6)


def pin_attention_softcap():
    # one head, two positions whose scaled scores (100 and 200) both saturate a
    # cap of 2: the capped scores are equal, so the output is the mean of V
    hd = 4
    q = np.array([1.0, 0.0, 0.0, 0.0], np.float32)
    k = np.zeros((1, 2, hd), np.float32)
    k[0, 0, 0], k[0, 1, 0] = 100.0, 200.0
    v = np.zeros((1, 2, hd), np.float32)
    v[0, 0] = [1.0, 2.0, 3.0, 4.0]
    v[0, 1] = [5.0, -6.0, 7.0, 0.5]
    capped = oracle.attention(q, 1, 1, hd, k, v, 0, 2 * hd, hd, 0, 2, 1.0, softcap=2.0)
    assert np.allclose(capped, (v[0, 0] + v[0, 1]) / 2, rtol=1e-6)
    plain = oracle.attention(q, 1, 1, hd, k, v, 0, 2 * hd, hd, 0, 2, 1.0)
    assert np.allclose(plain, v[0, 1], rtol=1e-6)
    # a very large cap changes nothing at ordinary scores
    rng = np.random.default_rng(2)
    q = rng.standard_normal(2 * 16).astype(np.float32)
    kc = rng.standard_normal((1, 40, 16)).astype(np.float32)
    vc = rng.standard_normal((1, 40, 16)).astype(np.float32)
    a = oracle.attention(q, 2, 1, 16, kc, vc, 0, 40 * 16, 16, 0, 40, 0.25)
    b = oracle.attention(q, 2, 1, 16, kc, vc, 0, 40 * 16, 16, 0, 40, 0.25, softcap=1e12)
    assert np.allclose(a, b, rtol=1e-6, atol=1e-7)


def test_gelu():
    pin_gelu()


def test_attention_softcap():
    pin_attention_softcap()


def pin_rope_freqs():
    hd, theta, ctx = 32, 1e4, 40
    c0, s0 = oracle.rope_table(ctx, hd, theta)
    c1, s1 = oracle.rope_table_freqs(ctx, hd, theta, np.ones(hd // 2, np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    # a factor of 2 halves every angle: position p reads like position p/2
    c2, s2 = oracle.rope_table_freqs(ctx, hd, theta, np.full(hd // 2, 2.0, np.float32))
    assert np.array_equal(c2[0::2][:ctx // 2], c0[:ctx // 2]) and np.array_equal(s2[0::2][:ctx // 2], s0[:ctx // 2])
    # an infinite factor leaves the pair unrotated; the others are untouched
    f = np.ones(hd // 2, np.float32)
    f[5:] = np.inf
    c3, s3 = oracle.rope_table_freqs(ctx, hd, theta, f)
    assert np.all(c3[:, 5:] == 1.0) and np.all(s3[:, 5:] == 0.0)
    assert np.array_equal(c3[:, :5], c0[:, :5]) and np.array_equal(s3[:, :5], s0[:, :5])


def test_rope_freqs():
    pin_rope_freqs()


def pin_matmul():
    rng = np.random.default_rng(12)
    T, rows, cols = 5, 40, 96
    wq, wd = synthetic.q8_weight(rng, rows, cols)
    xq = rng.integers(-127, 128, (T, cols)).astype(np.int8)
    xd = (np.abs(rng.standard_normal((T, cols // 32))) * 0.05).astype(np.float16).view(np.uint16)
    res = rng.standard_normal((T, rows)).astype(np.float32)

    def deq(q, d):
        return q.astype(np.float64) * np.repeat(d.view(np.float16).astype(np.float64), 32, axis=-1)

    want = deq(xq, xd) @ deq(wq, wd).T + res.astype(np.float64)
    got = oracle.q8_matmul(wq, wd, xq, xd, residual=res)
    assert got.shape == (T, rows)
    assert np.allclose(got, want, rtol=1e-6, atol=1e-6)
    assert oracle.q8_matmul(wq, wd, xq[:0], xd[:0]).shape == (0, rows)


def test_matmul():
    pin_matmul()


def pin_q4_0():
    # layout: d = 1, byte j = j | (15 - j) << 4 -> values j - 8 (j < 16) in the
    # low nibbles, then 7 - (j - 16) in the high ones (value j + 16 of byte j)
    blk = np.zeros(18, np.uint8)
    blk[0:2] = [0x00, 0x3C]                       # f16 1.0
    blk[2:] = [j | ((15 - j) << 4) for j in range(16)]
    want = np.array([j - 8 for j in range(16)] + [7 - j for j in range(16)], np.float64)
    assert np.array_equal(oracle.q_dequant("q4_0", blk, 32), want)
    # the scale multiplies: f16 0.5, and the smallest subnormal 2^-24
    blk[0:2] = [0x00, 0x38]
    assert np.array_equal(oracle.q_dequant("q4_0", blk, 32), 0.5 * want)
    blk[0:2] = [0x01, 0x00]
    assert np.array_equal(oracle.q_dequant("q4_0", blk, 32), 2.0 ** -24 * want)
    # the matvec equals the pinned Q8_0 matvec of the same codes (n - 8 as int8)
    rng = np.random.default_rng(31)
    rows, cols = 12, 160
    b = synthetic.q4_0_blocks(rng, rows, cols)
    code = b[..., 2:]
    q8 = np.concatenate([(code & 15).astype(np.int16) - 8, (code >> 4).astype(np.int16) - 8], axis=-1)
    q8 = q8.reshape(rows, cols).astype(np.int8)
    d = (b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8))
    xq = rng.integers(-127, 128, cols).astype(np.int8)
    xd = (np.abs(rng.standard_normal(cols // 32)) * 0.05).astype(np.float16).view(np.uint16)
    res = rng.standard_normal(rows).astype(np.float32)
    got = oracle.q_matvec("q4_0", b, rows, cols, xq, xd, residual=res)
    assert np.array_equal(got, oracle.q8_matvec(q8, d, xq, xd, residual=res))


def _q6_block(d_bits=0x3C00):
    blk = np.zeros(210, np.uint8)
    blk[192:208] = 1
    blk[208:210] = [d_bits & 0xFF, d_bits >> 8]
    return blk


def pin_q6_k():
    # all code bits zero: q = 0 - 32 everywhere
    blk = _q6_block()
    assert np.array_equal(oracle.q_dequant("q6_k", blk, 256), np.full(256, -32.0))
    # hand-placed bits, values derived from the layout statement:
    #   ql[0] = 0x5A: low nibble 10 -> value 0, high nibble 5 -> value 64
    #   qh[0] = 0b11100100: bit pairs 0,1,2,3 -> values 0, 32, 64, 96
    #   ql[32] = 0x0C: low nibble 12 -> value 32 (high nibble 0 -> value 96)
    #   second half: ql[64 + 5] = 0xF3 -> value 128 + 5 (3) and 128 + 69 (15);
    #   qh[32 + 5] = 0b00000010 -> value 128 + 5 gets high bits 2
    blk[0] = 0x5A
    blk[128] = 0b11100100
    blk[32] = 0x0C
    blk[64 + 5] = 0xF3
    blk[128 + 32 + 5] = 0b00000010
    w = oracle.q_dequant("q6_k", blk, 256)
    want = np.full(256, -32.0)
    want[0] = 10 + (0 << 4) - 32
    want[32] = 12 + (1 << 4) - 32
    want[64] = 5 + (2 << 4) - 32
    want[96] = 0 + (3 << 4) - 32
    want[128 + 5] = 3 + (2 << 4) - 32
    want[128 + 69] = 15 - 32
    assert np.array_equal(w, want)
    # sub-scales run in value order, 16 values each; d multiplies
    blk = _q6_block(0x3800)                        # d = 0.5
    blk[192:208] = np.arange(16, dtype=np.int8).view(np.uint8) - 7
    w = oracle.q_dequant("q6_k", blk, 256)
    assert np.array_equal(w, 0.5 * np.repeat(np.arange(16) - 7.0, 16) * -32.0)
    # every stored code bit reaches exactly one value, and each value gets
    # six distinct bit weights (1, 2, 4, 8 from ql, 16, 32 from qh)
    base = oracle.q_dequant("q6_k", _q6_block(), 256)
    seen = np.zeros((256, 6), int)
    for byte in range(192):
        for bit in range(8):
            blk = _q6_block()
            blk[byte] = 1 << bit
            diff = oracle.q_dequant("q6_k", blk, 256) - base
            hit = np.nonzero(diff)[0]
            assert hit.size == 1, (byte, bit)
            k = int(round(np.log2(diff[hit[0]])))
            assert diff[hit[0]] == 2.0 ** k and 0 <= k < 6
            seen[hit[0], k] += 1
    assert np.array_equal(seen, np.ones((256, 6), int))
    # the matvec is the int8 path: per 16 values an exact dot, times d * sc
    # and the activation block's scale; equal to the f64 dot of the values
    rng = np.random.default_rng(32)
    rows, cols = 6, 512
    b = synthetic.q6_k_blocks(rng, rows, cols)
    xq = rng.integers(-127, 128, cols).astype(np.int8)
    xd = (np.abs(rng.standard_normal(cols // 32)) * 0.05).astype(np.float16).view(np.uint16)
    x = xq.astype(np.float64) * np.repeat(xd.view(np.float16).astype(np.float64), 32)
    W = oracle.q_dequant("q6_k", b, rows * cols).reshape(rows, cols)
    got = oracle.q_matvec("q6_k", b, rows, cols, xq, xd)
    assert np.allclose(got, W @ x, rtol=1e-6, atol=1e-9)
    got = oracle.q_matvec("q6_k", b, rows, cols, xq, xd, residual=np.ones(rows, np.float32))
    assert np.allclose(got, W @ x + 1.0, rtol=1e-6, atol=1e-9)


def test_q4_0():
    pin_q4_0()


def test_q6_k():
    pin_q6_k()


def test_rmsnorm():
    pin_rmsnorm()


def test_rope():
    pin_rope()


def test_silu():
    pin_silu()


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def _bf16(a):
    return (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_attention():
    rng = np.random.default_rng(8)
    n_q, n_kv, hd, ctx = 8, 2, 32, 50
    G = n_q // n_kv
    K = rng.standard_normal((n_kv, ctx, hd)).astype(np.float32)
    V = rng.standard_normal((n_kv, ctx, hd)).astype(np.float32)
    q = rng.standard_normal(n_q * hd).astype(np.float32)
    scale = 1 / math.sqrt(hd)
    hs, ps = ctx * hd, hd
    # brute force with scipy's softmax over the window, both dtypes
    for dtype in (0, 1):
        Kc, Vc = (K, V) if dtype == 0 else (_bf16(K), _bf16(V))
        Kf = K.astype(np.float64) if dtype == 0 else _bf16_f64(Kc)
        Vf = V.astype(np.float64) if dtype == 0 else _bf16_f64(Vc)
        for start, length in [(0, ctx), (17, 20), (49, 1)]:
            got = oracle.attention(q, n_q, n_kv, hd, Kc, Vc, dtype, hs, ps, start, length, scale)
            for h in range(n_q):
                g = h // G
                s = Kf[g, start:start + length] @ q[h * hd:(h + 1) * hd].astype(np.float64) * scale
                want = scipy.special.softmax(s) @ Vf[g, start:start + length]
                assert np.allclose(got[h * hd:(h + 1) * hd], want, rtol=1e-6, atol=1e-7)
    # one position: output is that V row exactly
    got = oracle.attention(q, n_q, n_kv, hd, K, V, 0, hs, ps, 33, 1, scale)
    for h in range(n_q):
        assert np.array_equal(got[h * hd:(h + 1) * hd], V[h // G, 33])
    # q = 0: uniform weights, output is the mean of V over the window
    got = oracle.attention(np.zeros_like(q), n_q, n_kv, hd, K, V, 0, hs, ps, 5, 40, scale)
    for h in range(n_q):
        assert np.allclose(got[h * hd:(h + 1) * hd], V[h // G, 5:45].astype(np.float64).mean(0), rtol=1e-6, atol=1e-7)
    # GQA head map: V constant per kv head -> output of head h is h // G
    Vg = np.broadcast_to(np.arange(n_kv, dtype=np.float32)[:, None, None], V.shape).copy()
    got = oracle.attention(q, n_q, n_kv, hd, K, Vg, 0, hs, ps, 0, ctx, scale)
    for h in range(n_q):
        assert np.allclose(got[h * hd:(h + 1) * hd], h // G, atol=1e-6)
    # one dominant score picks that row
    Kd = K.copy(); Kd[:, 21] = 0
    for g in range(n_kv):
        Kd[g, 21] = 50 * q[g * G * hd:(g * G + 1) * hd]
    got = oracle.attention(q, n_q, n_kv, hd, Kd, V, 0, hs, ps, 0, ctx, scale)
    for g in range(n_kv):
        assert np.allclose(got[g * G * hd:(g * G + 1) * hd], V[g, 21], atol=1e-6)
    # non-default strides: a cache laid out [ctx, n_kv, hd] gives the same result
    Kt = np.ascontiguousarray(K.transpose(1, 0, 2)); Vt = np.ascontiguousarray(V.transpose(1, 0, 2))
    a = oracle.attention(q, n_q, n_kv, hd, K, V, 0, hs, ps, 3, 30, scale)
    b = oracle.attention(q, n_q, n_kv, hd, Kt, Vt, 0, hd, n_kv * hd, 3, 30, scale)
    assert np.array_equal(a, b)
    # the method's own reformulation (online softmax in f64) matches the two-pass form
    g, h = 1, 5
    m, l, acc = -np.inf, 0.0, np.zeros(hd)
    for j in range(ctx):
        s = float(np.dot(K[g, j].astype(np.float64), q[h * hd:(h + 1) * hd].astype(np.float64)) * scale)
        mn = max(m, s)
        c = math.exp(m - mn) if m != -np.inf else 0.0
        l = l * c + math.exp(s - mn)
        acc = acc * c + math.exp(s - mn) * V[g, j].astype(np.float64)
        m = mn
    got = oracle.attention(q, n_q, n_kv, hd, K, V, 0, hs, ps, 0, ctx, scale)
    assert np.allclose(got[h * hd:(h + 1) * hd], acc / l, rtol=1e-6, atol=1e-7)


def test_attention():
    pin_attention()


# ----------------------------------------------------------------------------
# MoE
# ----------------------------------------------------------------------------
def pin_moe_route():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((16, 128)).astype(np.float32)
    logits[3, 10] = logits[3, 90] = 5.0                            # exact tie: lower id first
    ids, w = oracle.moe_route(logits, 8)
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, order)
    assert ids[3, 0] == 10 and ids[3, 1] == 90
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, order, axis=1), rtol=1e-6)


def pin_moe_block():
    rng = np.random.default_rng(10)
    H, I, E, k, T = 64, 32, 6, 2, 3
    gq, gd = synthetic.q8_weight(rng, E * 2 * I, H)
    dq, dd = synthetic.q8_weight(rng, E * H, I)
    gq, gd = gq.reshape(E, 2 * I, H), gd.reshape(E, 2 * I, H // 32)
    dq, dd = dq.reshape(E, H, I), dd.reshape(E, H, I // 32)
    x = rng.standard_normal((T, H)).astype(np.float32) * 3
    logits = rng.standard_normal((T, E)).astype(np.float32)
    out, tr = oracle.moe_block(H, I, E, k, gq, gd, dq, dd, x, logits, trace=True)

    def deq(q, d):
        return q.astype(np.float64) * np.repeat(d.view(np.float16).astype(np.float64), 32, axis=-1)

    # brute force in numpy over dequantized operands; the quantized inputs of
    # each matvec are the oracle's (pinned separately above)
    for t in range(T):
        acc = np.zeros(H)
        for s in range(k):
            e = tr["ids"][t, s]
            y1 = deq(gq[e], gd[e]) @ deq(tr["xq"][t], tr["xd"][t])
            assert np.allclose(tr["y1"][t, s], y1, rtol=1e-6, atol=1e-7)
            g32 = tr["y1"][t, s].astype(np.float64)          # stage boundary is float32
            h = (scipy.special.expit(g32[:I]) * g32[:I] * g32[I:]).astype(np.float32)
            hq, hd = oracle.q8_quantize(h)
            diff = hq.astype(int) - tr["hq"][t, s].astype(int)
            assert np.abs(diff).max() <= 1 and np.count_nonzero(diff) <= 1
            y2 = deq(dq[e], dd[e]) @ deq(tr["hq"][t, s], tr["hd"][t, s])
            assert np.allclose(tr["y2"][t, s], y2, rtol=1e-6, atol=1e-7)
            acc += tr["w"][t, s] * y2
        assert np.allclose(out[t], acc, rtol=1e-6, atol=1e-6)
    # per-expert output scale: all 2 doubles the block exactly; a one-hot table
    # keeps only the slots routed to that expert
    out2 = oracle.moe_block(H, I, E, k, gq, gd, dq, dd, x, logits, expert_scale=np.full(E, 2.0, np.float32))
    assert np.array_equal(out2, 2.0 * out)
    e1 = int(tr["ids"][0, 0])
    one = np.zeros(E, np.float32)
    one[e1] = 1.5
    out1 = oracle.moe_block(H, I, E, k, gq, gd, dq, dd, x, logits, expert_scale=one)
    for t in range(T):
        want = sum(1.5 * float(tr["w"][t, s]) * tr["y2"][t, s].astype(np.float64)
                   for s in range(k) if tr["ids"][t, s] == e1) + np.zeros(H)
        assert np.allclose(out1[t], want, rtol=1e-6, atol=1e-7)
    # one expert, k = 1, weight 1: the block is the plain two-matvec FFN
    out1, tr1 = oracle.moe_block(H, I, 1, 1, gq[:1], gd[:1], dq[:1], dd[:1], x, logits[:, :1], trace=True)
    assert np.allclose(tr1["w"], 1.0)
    y1 = oracle.q8_matvec(gq[0], gd[0], *oracle.q8_quantize(x[1]))
    h = oracle.silu_mul(y1[:I], y1[I:])
    y2 = oracle.q8_matvec(dq[0], dd[0], *oracle.q8_quantize(h))
    assert np.array_equal(out1[1], y2)


def test_moe_route():
    pin_moe_route()


def test_moe_block():
    pin_moe_block()


# ----------------------------------------------------------------------------
# decode layer: composition of the pinned stages, checked against a numpy
# float64 re-composition (brute force) on a small shape
# ----------------------------------------------------------------------------
def _np_layer(cfg, w, x, pos, kc, vc):
    """Independent numpy composition of the layer (float64 math, float32 at
    stage boundaries, the oracle's pinned quantizer for the Q8 steps)."""
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    eps = cfg["eps"]

    def deq(q, d):
        return q.astype(np.float64) * np.repeat(d.view(np.float16).astype(np.float64), 32, axis=-1)

    def rms(v, g):
        v = v.astype(np.float64)
        r = v / np.sqrt(np.mean(v * v) + eps)
        return (r * (1.0 if g is None else g.astype(np.float64))).astype(np.float32)

    def mv(qname, a, res=None):
        aq, ad = oracle.q8_quantize(a)
        y = deq(w[qname + "_qs"], w[qname + "_d"]) @ deq(aq, ad)
        if res is not None:
            y = y + res.astype(np.float64)
        return y.astype(np.float32)

    half = hd // 2
    ang = pos * cfg["theta"] ** (-2.0 * np.arange(half) / hd)
    c, s = np.cos(ang).astype(np.float32).astype(np.float64), np.sin(ang).astype(np.float32).astype(np.float64)

    def rope(v):
        v = v.astype(np.float64)
        a, b = v[:half], v[half:]
        return np.concatenate([a * c - b * s, a * s + b * c]).astype(np.float32)

    qkv = mv("qkv", rms(x, w["g_in"]))
    qd, kvd = nq * hd, nkv * hd
    q = np.concatenate([rope(rms(qkv[h * hd:(h + 1) * hd], w["g_q"])) for h in range(nq)])
    k = np.concatenate([rope(rms(qkv[qd + g * hd:qd + (g + 1) * hd], w["g_k"])) for g in range(nkv)])
    v = qkv[qd + kvd:]
    if cfg["v_unit_norm"]:
        v = np.concatenate([rms(v[g * hd:(g + 1) * hd], None) for g in range(nkv)])
    kc, vc = kc.copy(), vc.copy()
    if cfg["kv_dtype"] == 0:
        kc[:, pos] = k.reshape(nkv, hd); vc[:, pos] = v.reshape(nkv, hd)
        Kf, Vf = kc.astype(np.float64), vc.astype(np.float64)
    else:
        import torch
        kb = torch.from_numpy(k.reshape(nkv, hd)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        vb = torch.from_numpy(v.reshape(nkv, hd)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        kc[:, pos] = kb; vc[:, pos] = vb
        Kf, Vf = _bf16_f64(kc), _bf16_f64(vc)
    start = max(0, pos - cfg["window"] + 1) if cfg["window"] else 0
    G = nq // nkv
    att = np.concatenate([
        scipy.special.softmax(Kf[h // G, start:pos + 1] @ q[h * hd:(h + 1) * hd].astype(np.float64)
                              * cfg["attn_scale"]) @ Vf[h // G, start:pos + 1] for h in range(nq)
    ]).astype(np.float32)
    if cfg["kind"] == 0:
        x1 = mv("o", att, res=x)
        gu = mv("gu", rms(x1, w["g_post"]))
        h = (scipy.special.expit(gu[:I].astype(np.float64)) * gu[:I] * gu[I:]).astype(np.float32)
        return mv("dn", h, res=x1)
    o = mv("o", att)
    return (x.astype(np.float64) + rms(o, w["g_post"])).astype(np.float32)


def _small_layer(kind, kv_dtype, seed):
    rng = np.random.default_rng(seed)
    cfg = dict(kind=kind, hidden=128, n_q=4, n_kv=2, head_dim=32, ffn=96 if kind == 0 else 0,
               kv_dtype=kv_dtype, ctx=24, window=8 if kind == 1 else 0, eps=1e-6, theta=1e6,
               max_ctx=24, qk_norm=1, v_unit_norm=1 if kind == 1 else 0)
    cfg["attn_scale"] = 1 / math.sqrt(cfg["head_dim"])
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    w = dict(g_in=synthetic.gamma(rng, H), g_q=synthetic.gamma(rng, hd), g_k=synthetic.gamma(rng, hd),
             g_post=synthetic.gamma(rng, H))
    w["qkv_qs"], w["qkv_d"] = synthetic.q8_weight(rng, nq * hd + 2 * nkv * hd, H)
    w["o_qs"], w["o_d"] = synthetic.q8_weight(rng, H, nq * hd)
    if I:
        w["gu_qs"], w["gu_d"] = synthetic.q8_weight(rng, 2 * I, H)
        w["dn_qs"], w["dn_d"] = synthetic.q8_weight(rng, H, I)
    w["rope_cos"], w["rope_sin"] = oracle.rope_table(cfg["max_ctx"], hd, cfg["theta"])
    x = synthetic.activations(rng, H)
    kc = synthetic.kv_cache(rng, nkv, cfg["max_ctx"], hd, kv_dtype)
    vc = synthetic.kv_cache(rng, nkv, cfg["max_ctx"], hd, kv_dtype)
    return cfg, w, x, kc, vc


def pin_layer(kind, kv_dtype, seed=11):
    cfg, w, x, kc, vc = _small_layer(kind, kv_dtype, seed)
    pos = cfg["ctx"] - 1
    got, kc2, vc2, tr = oracle.decode_layer(cfg, w, x, pos, kc, vc, trace=True)
    want = _np_layer(cfg, w, x, pos, kc, vc)
    err = np.abs(got.astype(np.float64) - want)
    assert np.all(err <= np.maximum(1e-3 * np.abs(want), 1e-4)), err.max()
    # only row pos of each cache changes
    changed = np.any(kc2 != kc, axis=2)
    assert not changed[:, :pos].any() and not changed[:, pos + 1:].any()


@pytest.mark.parametrize("kind,kv_dtype", [(0, 0), (0, 1), (1, 1)])
def test_layer_composition(kind, kv_dtype):
    pin_layer(kind, kv_dtype)


# ---- whole-layer special cases: closed forms that do not go through the
# oracle's attention or wiring ("Current Inference Path -- Architecture Map",
# section 3: residual adds around the attention block and the MLP; "Inference
# Engine" (larql), BLAS-Fused Attention: softmax over the attended positions)

@pytest.mark.parametrize("kind,kv_dtype", [(0, 0), (0, 1), (1, 1)])
def test_layer_zero_projections_is_identity(kind, kv_dtype):
    """With all-zero O and down codes the attention block and the MLP add
    exact zeros to the residual stream, so the layer returns x bit for bit
    (the Gemma block: o = 0, RMSNorm(0) = 0).  A dropped, doubled or
    misrouted residual fails this."""
    cfg, w, x, kc, vc = _small_layer(kind, kv_dtype, 5)
    w["o_qs"] = np.zeros_like(w["o_qs"])
    if kind == 0:
        w["dn_qs"] = np.zeros_like(w["dn_qs"])
    got, _, _, _ = oracle.decode_layer(cfg, w, x, cfg["ctx"] - 1, kc, vc)
    assert np.array_equal(got.view(np.uint32), x.astype(np.float32).view(np.uint32))


def _deq(q, d):
    return q.astype(np.float64) * np.repeat(d.view(np.float16).astype(np.float64), 32, axis=-1)


@pytest.mark.parametrize("kind,kv_dtype", [(0, 0), (0, 1), (1, 1)])
def test_layer_one_position_closed_form(kind, kv_dtype):
    """At position 0 the attention covers one position, so every query head's
    softmax weight is exactly 1 and its output is the new v row of its kv head
    (as stored in the cache): no scores, no softmax.  RoPE at angle 0 is the
    identity, so the new k row is the normed k.  The layer output is then a
    closed form of the projections alone; two kv heads with distinct v rows
    also pin the query-head -> kv-head map (h // G)."""
    cfg, w, x, kc, vc = _small_layer(kind, kv_dtype, 7)
    H, nq, nkv, hd, I = cfg["hidden"], cfg["n_q"], cfg["n_kv"], cfg["head_dim"], cfg["ffn"]
    eps, G = cfg["eps"], nq // nkv
    got, kc2, vc2, _ = oracle.decode_layer(cfg, w, x, 0, kc, vc)

    def rms(v, g):
        v = v.astype(np.float64)
        r = v / np.sqrt(np.mean(v * v) + eps)
        return (r * (1.0 if g is None else g.astype(np.float64))).astype(np.float32)

    def mv(name, a):
        aq, ad = oracle.q8_quantize(a)
        return (_deq(w[name + "_qs"], w[name + "_d"]) @ _deq(aq, ad)).astype(np.float32)

    def stored(v):           # the cache's own rounding of a row
        if kv_dtype == 0:
            return v.astype(np.float64)
        import torch
        b = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return _bf16_f64(b)

    qkv = mv("qkv", rms(x, w["g_in"]))
    qd, kvd = nq * hd, nkv * hd
    v = qkv[qd + kvd:].reshape(nkv, hd)
    if cfg["v_unit_norm"]:
        v = np.stack([rms(v[g], None) for g in range(nkv)])
    k = np.stack([rms(qkv[qd + g * hd:qd + (g + 1) * hd], w["g_k"]) for g in range(nkv)])
    tol = lambda a, b: np.all(np.abs(a - b) <= np.maximum(1e-3 * np.abs(b), 1e-4))
    read = (lambda c: c.astype(np.float64)) if kv_dtype == 0 else _bf16_f64
    assert tol(read(kc2[:, 0]), stored(k)) and tol(read(vc2[:, 0]), stored(v))
    att = np.concatenate([stored(v[h // G]) for h in range(nq)]).astype(np.float32)
    assert not np.allclose(v[0], v[1])                  # distinct kv heads: the map is observable
    if kind == 0:
        x1 = (x.astype(np.float64) + mv("o", att)).astype(np.float32)
        gu = mv("gu", rms(x1, w["g_post"])).astype(np.float64)
        h = (gu[:I] / (1.0 + np.exp(-gu[:I])) * gu[I:]).astype(np.float32)
        want = x1.astype(np.float64) + mv("dn", h)
    else:
        want = x.astype(np.float64) + rms(mv("o", att), w["g_post"])
    assert tol(got.astype(np.float64), want), np.abs(got - want).max()

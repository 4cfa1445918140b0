"""Helpers shared by the GPU parity tests: device transfers, the float
tolerance rule and the acceptance rule for Q8_0 codes computed from float
inputs that differ by rounding."""
import numpy as np

import oracle

RTOL, ATOL = 1e-3, 1e-4     # |gpu - ref| <= max(RTOL * |ref|, ATOL), elementwise


def torch_mod():
    import torch
    return torch


def dev(a):
    """numpy -> device tensor (uint16 travels as int16 bits)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda")


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(shape, dtype):
    torch = torch_mod()
    tmap = {np.float32: torch.float32, np.int8: torch.int8, np.uint16: torch.int16,
            np.int32: torch.int32, np.uint8: torch.uint8}
    return torch.empty(shape, dtype=tmap[dtype], device="cuda")


def workspace(nbytes):
    torch = torch_mod()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device="cuda")


def sync():
    torch_mod().cuda.synchronize()


def assert_close(gpu, ref, what="", rtol=RTOL, atol=ATOL):
    g = np.asarray(gpu, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    assert g.shape == r.shape, (what, g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    err = np.abs(g - r)
    lim = np.maximum(rtol * np.abs(r), atol)
    bad = err > lim
    if bad.any():
        i = int(np.argmax(err / lim))
        raise AssertionError(f"{what}: {int(bad.sum())}/{bad.size} outside tolerance; worst at {i}: "
                             f"gpu={g[i]!r} ref={r[i]!r}")
    return float((err / np.maximum(np.abs(r), 1e-30)).max())


def q8_reference_ratio(x):
    """x * (1/d) per element in float32, the quantity the codes round."""
    x = np.asarray(x, np.float32).reshape(-1, 32)
    amax = np.abs(x).max(axis=1)
    d = (amax / np.float32(127)).astype(np.float32)
    inv = np.where(d != 0, np.float32(1) / np.where(d != 0, d, np.float32(1)), np.float32(0)).astype(np.float32)
    return (x * inv[:, None]).astype(np.float32)


def assert_q8_near(gpu_qs, gpu_d, ref_x, what="", delta=2e-4, max_flip_frac=1e-3):
    """GPU codes/scales of a vector whose float input may differ from the
    oracle's by rounding: codes must equal the oracle's, except a +-1 change
    where the oracle's x/d lies within `delta` of a rounding boundary (.5);
    scales equal or one f16 step apart.  Returns the number of flipped codes."""
    ref_x = np.asarray(ref_x, np.float32).ravel()
    rq, rd = oracle.q8_quantize(ref_x)
    gq = np.asarray(gpu_qs, np.int8).ravel().astype(np.int32)
    gd = np.asarray(gpu_d).view(np.uint16).ravel().astype(np.int32)
    rq = rq.ravel().astype(np.int32)
    rd = rd.ravel().astype(np.int32)
    dd = np.abs(gd - rd)
    assert dd.max() <= 1, f"{what}: scale bits differ by {dd.max()} (f16 steps)"
    diff = gq - rq
    flips = np.nonzero(diff)[0]
    if flips.size:
        assert np.abs(diff[flips]).max() == 1, f"{what}: code differs by more than 1"
        r = np.abs(q8_reference_ratio(ref_x).ravel()[flips]).astype(np.float64)
        dist = np.abs(r - (np.floor(r) + 0.5))
        assert dist.max() <= delta, f"{what}: flipped code not at a rounding boundary (dist {dist.max():.3g})"
        assert flips.size <= max(2, max_flip_frac * gq.size), f"{what}: {flips.size} flips"
    return int(flips.size)

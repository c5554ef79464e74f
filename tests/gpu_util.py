"""Helpers for the GPU parity tests: move seeded inputs to the device, call the
library through its C ABI binding, and compare with the oracle by the rules
the tests state.  Nothing here computes any part of the method."""
from __future__ import annotations

import sys

import numpy as np

Y_RTOL = 1e-5       # fp32 outputs: relative error bound
GAMMA_RTOL = 1e-6   # gamma: relative error bound (fp64 sums in different orders)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch


def to_dev_bits(x_bits: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).to("cuda")


def to_dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    torch_mod().cuda.synchronize()
    return t.cpu().numpy()


def check_gamma(g_gpu: np.float32, g_or: np.float32, tag: str) -> bool:
    """gamma within the stated relative bound; returns whether the bits agree."""
    g_gpu = np.float32(g_gpu)
    g_or = np.float32(g_or)
    if g_or == 0:
        assert g_gpu == 0, tag
        return True
    assert abs(float(g_gpu) - float(g_or)) <= GAMMA_RTOL * abs(float(g_or)), (tag, g_gpu, g_or)
    same = g_gpu.view(np.uint32) == g_or.view(np.uint32)
    if not same:
        log("[%s] gamma differs in the last bits: gpu %r oracle %r" % (tag, g_gpu, g_or))
    return bool(same)


def compare_codes(codes_gpu: np.ndarray, q_or: np.ndarray, w: np.ndarray, g_or: np.float32,
                  gamma_same: bool, tag: str) -> np.ndarray:
    """Ternary codes must be bit-exact.  Only if the two gammas differ in their
    last bits may a code differ, and then only for a weight whose quotient
    W / (gamma + 1e-5) (oracle gamma) lies within the gamma tolerance of a
    rounding threshold (0.5 or 1.5).  Returns the weight rows with any such
    difference (excluded from accumulator checks)."""
    diff = codes_gpu != q_or
    if not diff.any():
        return np.zeros(0, dtype=np.int64)
    assert not gamma_same, "%s: %d ternary codes differ with identical gamma" % (tag, int(diff.sum()))
    d = np.float64(np.float32(np.float32(g_or) + np.float32(1e-5)))
    t = np.abs(w[diff].astype(np.float64)) / d
    band = 4 * GAMMA_RTOL
    near = (np.abs(t - 0.5) <= band * 0.5) | (np.abs(t - 1.5) <= band * 1.5)
    assert near.all(), "%s: code differences away from a rounding threshold" % tag
    rows = np.unique(np.nonzero(diff)[0])
    log("[%s] %d codes in %d rows differ at a threshold (gamma last-bit difference)" % (tag, int(diff.sum()), len(rows)))
    return rows


def compare_y(y_gpu: np.ndarray, y_or: np.ndarray, tag: str):
    y_gpu = y_gpu.astype(np.float64)
    y_or = y_or.astype(np.float64)
    zero = y_or == 0
    assert (y_gpu[zero] == 0).all(), "%s: non-zero output where the oracle gives 0" % tag
    err = np.abs(y_gpu - y_or)
    bound = Y_RTOL * np.abs(y_or)
    bad = err > bound
    assert not bad.any(), "%s: %d outputs beyond rel %.0e (worst rel %.3e)" % (
        tag, int(bad.sum()), Y_RTOL, float((err[~zero] / np.abs(y_or[~zero])).max()))


# RMSNorm ahead of the quantisation: the kernels take the codes of x * gain
# with the per-token factor r folded into a' (rmsnorm_scales), the oracle
# follows the listing (x_norm = (x * r) * gain, then the absmax rule).  The
# two evaluations of t = x_norm * 127 / a' differ by at most about 12 fp32
# roundings of t (2^-24 each), so a code may be the other neighbour only where
# the oracle's t lies within 2^-19 |t| of a rounding tie; a' agrees to within
# 6 ulps (each side's a' is within 3 roundings of the exact max|x_norm|).
NORM_TIE_BAND = 2.0 ** -19
NORM_AMAX_ULPS = 6


def assert_within_ulps(a, b, ulps, tag):
    a = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    d = np.abs(a - b)
    assert d.max(initial=0) <= ulps, (tag, int(d.max(initial=0)))


def check_norm_codes(xq_gpu, a_gpu, xq_or, a_or, xn_or, tag) -> np.ndarray:
    """Codes and a' of the RMSNorm path against the oracle's (listing order).
    Returns, per token, the number of codes that took the other neighbour of
    a tie: the accumulators of that token may differ by at most that much."""
    assert_within_ulps(a_gpu, a_or, NORM_AMAX_ULPS, tag + " a'")
    t = np.abs(xn_or.astype(np.float64) * (127.0 / a_or.astype(np.float64))[:, None])
    near = np.abs(t - np.floor(t) - 0.5) <= NORM_TIE_BAND * t
    diff = np.abs(xq_gpu.astype(np.int64) - xq_or.astype(np.int64))
    assert diff.max(initial=0) <= 1, "%s: a code differs by more than one" % tag
    assert np.all(near[diff != 0]), "%s: %d codes differ away from a rounding tie" % (tag, int((diff != 0).sum() - near[diff != 0].sum()))
    flips = diff.sum(axis=1)
    if flips.any():
        log("[%s] %d codes took the other neighbour of a tie" % (tag, int(flips.sum())))
    return flips


def compare_acc_flips(acc_gpu: np.ndarray, acc_or: np.ndarray, flips: np.ndarray, tag: str):
    """Accumulators: bit-exact for tokens without flipped codes; otherwise
    within the number of flipped codes (each moves acc by a weight in
    {-1, 0, 1})."""
    d = np.abs(acc_gpu.astype(np.int64) - acc_or.astype(np.int64))
    assert np.all(d <= flips[:, None]), "%s: accumulators differ beyond the flipped codes" % tag


def compare_y_flips(y_gpu: np.ndarray, y_or: np.ndarray, flips: np.ndarray, w_scale, a_or: np.ndarray, tag: str):
    """y within Y_RTOL, plus the flipped codes' weight per token."""
    y_gpu = y_gpu.astype(np.float64)
    y_or = y_or.astype(np.float64)
    allow = flips[:, None] * np.float64(w_scale) * a_or.astype(np.float64)[:, None] / 127.0
    zero = (y_or == 0) & (allow == 0)
    assert (y_gpu[zero] == 0).all(), "%s: non-zero output where the oracle gives 0" % tag
    assert np.all(np.abs(y_gpu - y_or) <= Y_RTOL * np.abs(y_or) + allow * (1 + Y_RTOL)), "%s: y" % tag

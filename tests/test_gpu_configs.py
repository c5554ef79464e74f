"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark uses (decode entry point for m <= 16, batched otherwise).

For each distinct matrix shape of a workload (layer 0): gamma within 1e-6
relative, every ternary code and every int8 activation code bit-exact, and
the int32 accumulators bit-exact / fp32 outputs within 1e-5 relative -- on
every output where the oracle can afford the whole contraction, otherwise on
all outputs of the first and last token plus 4096 random (token, row) pairs,
each computed by the oracle one by one.

The fused entry points the decode benchmark times (the quantisation, or
RMSNorm and the quantisation, in the decode prologue; the fp32 quantisation
for the down projection) run at every matrix shape of the decode workloads
with one and two tokens; their codes, a', accumulators and outputs are
compared on every output (RMSNorm: with the per-position tie allowance of
tests/gpu_util.py).  The fused binary decode (1-bit sign weights) runs at
every such shape with one token, compared the same way.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (check_gamma, check_norm_codes, compare_acc_flips, compare_codes, compare_y,
                            compare_y_flips, host, log, to_dev, to_dev_bits, torch_mod)

pytestmark = pytest.mark.gpu

FULL_ORACLE_MACS = 4e9

CASES = [(wl.key, j) for wl in synth.WORKLOADS for j in range(len(wl.matrices))]


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("wkey,j", CASES, ids=["%s-%s" % (k, synth.BY_KEY[k].matrices[j].name) for k, j in CASES])
def test_workload_matrix_full_size(blq, wkey, j):
    torch = torch_mod()
    wl = synth.BY_KEY[wkey]
    mat = wl.matrices[j]
    n, k = mat.n, mat.k
    tag = "%s/%s n=%d k=%d" % (wkey, mat.name, n, k)
    log("case", tag)
    w = synth.latent_weights(synth.seed_for(wl, 0, j, synth.ROLE_WEIGHT), n, k)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    g_or = oracle.gamma(w)
    same = check_gamma(host(gamma)[0], g_or, tag)
    q_or = oracle.ternarize(w, g_or)
    bad_rows = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), q_or, w, g_or, same, tag)
    rng = np.random.default_rng(j)
    for m in wl.ms:
        log("  m=%d" % m)
        x = synth.activations_bf16(synth.seed_for(wl, 0, j, synth.ROLE_ACT, extra=m), m, k, wl.outlier_frac)
        xq_d, amax_d = blq.bitlinear_quant_act(to_dev_bits(x))
        xq_or, amax_or = oracle.quant_act(x)
        assert np.array_equal(host(xq_d), xq_or), tag
        assert np.array_equal(host(amax_d), amax_or), tag
        acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
        fwd = blq.bitlinear_forward if m <= blq.BITLINEAR_FORWARD_MAX_M else blq.bitlinear_forward_batched
        y = host(fwd(packed, gamma, n, k, xq_d, amax_d, acc=acc_d))
        acc = host(acc_d)
        if m * n * k <= FULL_ORACLE_MACS:
            rows = np.repeat(np.arange(m), n)
            cols = np.tile(np.arange(n), m)
        else:
            ends = np.array(sorted({0, m - 1}))
            rows = np.concatenate([np.repeat(ends, n), rng.integers(0, m, 4096)])
            cols = np.concatenate([np.tile(np.arange(n), len(ends)), rng.integers(0, n, 4096)])
        keep = ~np.isin(cols, bad_rows)
        rows, cols = rows[keep], cols[keep]
        acc_or = oracle.contract_pairs(xq_or, q_or, rows, cols)
        assert np.array_equal(acc[rows, cols], acc_or), tag
        # dequantise the sampled accumulators with the oracle, one token at a time
        y_or = np.empty(len(rows), np.float32)
        for t in np.unique(rows):
            sel = rows == t
            y_or[sel] = oracle.dequant(acc_or[sel][None, :], g_or, amax_or[t:t + 1])[0]
        compare_y(y[rows, cols], y_or, tag)
    if min(wl.ms) <= 2:  # a decode workload: the fused entry points it times, at one and two tokens
        fused_checks(blq, wl, j, packed, gamma, q_or, g_or, bad_rows, tag)
        binary_fused_check(blq, wl, j, w, tag)


def fused_checks(blq, wl, j, packed, gamma, q_or, g_or, bad_rows, tag):
    torch = torch_mod()
    n, k = wl.matrices[j].n, wl.matrices[j].k
    keep = np.setdiff1d(np.arange(n), bad_rows)
    gain = synth.norm_gain(synth.seed_for(wl, 0, j, synth.ROLE_GAIN), k)
    for m in (1, 2):
        if not blq.bitlinear_quant_forward_supported(m, k):
            continue
        x = synth.activations_bf16(synth.seed_for(wl, 0, j, synth.ROLE_ACT, extra=100 + m), m, k, wl.outlier_frac)
        xd = to_dev_bits(x)
        for kind in ("plain", "rmsnorm", "f32"):
            if kind == "f32" and m != 1:
                continue
            t = "%s fused %s m=%d" % (tag, kind, m)
            log("  " + t)
            acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
            xq_d = torch.empty((m, k), dtype=torch.int8, device="cuda")
            a_d = torch.empty(m, dtype=torch.float32, device="cuda")
            flips = np.zeros(m, np.int64)
            if kind == "plain":
                y_d = blq.bitlinear_quant_forward(packed, gamma, n, k, xd, acc=acc_d, xq=xq_d, x_absmax=a_d)
                xq_o, a_o = oracle.quant_act(x)
                assert np.array_equal(host(xq_d), xq_o) and np.array_equal(host(a_d), a_o), t
            elif kind == "rmsnorm":
                y_d = blq.bitlinear_rmsnorm_quant_forward(packed, gamma, n, k, xd, gain=to_dev(gain), acc=acc_d,
                                                          xq=xq_d, x_absmax=a_d)
                xq_o, a_o, _, xn_o = oracle.rmsnorm_quant_act(x, gain, with_xnorm=True)
                flips = check_norm_codes(host(xq_d), host(a_d), xq_o, a_o, xn_o, t)
            else:
                xf = synth.activations_f32(synth.seed_for(wl, 0, j, synth.ROLE_ACT, extra=200 + m), m, k, 0.5)
                y_d = blq.bitlinear_quant_forward_f32(packed, gamma, n, k, to_dev(xf), acc=acc_d, xq=xq_d,
                                                      x_absmax=a_d)
                xq_o, a_o = oracle.quant_act_f32(xf)
                assert np.array_equal(host(xq_d), xq_o) and np.array_equal(host(a_d), a_o), t
            acc_o = oracle.contract(xq_o, q_or)
            compare_acc_flips(host(acc_d)[:, keep], acc_o[:, keep], flips, t)
            compare_y_flips(host(y_d)[:, keep], oracle.dequant(acc_o, g_or, a_o)[:, keep], flips, g_or, a_o, t)


def binary_fused_check(blq, wl, j, w, tag):
    """The fused binary decode (1-bit sign weights, the layer scale an input)
    the binary decode records time, at one token: codes, a' and accumulators
    bit-exact on every output, y within 1e-5."""
    torch = torch_mod()
    n, k = wl.matrices[j].n, wl.matrices[j].k
    if not blq.bitlinear_quant_forward_binary_supported(1, k):
        return
    t = "%s fused binary m=1" % tag
    log("  " + t)
    s = np.float32(np.abs(w).astype(np.float64).mean())  # a stand-in for the learned layer scale
    packed = blq.bitlinear_pack_binary(to_dev(w))
    x = synth.activations_bf16(synth.seed_for(wl, 0, j, synth.ROLE_ACT, extra=300), 1, k, wl.outlier_frac)
    acc_d = torch.empty((1, n), dtype=torch.int32, device="cuda")
    xq_d = torch.empty((1, k), dtype=torch.int8, device="cuda")
    a_d = torch.empty(1, dtype=torch.float32, device="cuda")
    y_d = blq.bitlinear_quant_forward_binary(packed, to_dev(np.array([s], np.float32)), n, k, to_dev_bits(x),
                                             acc=acc_d, xq=xq_d, x_absmax=a_d)
    ref = oracle.forward_binary(x, w, s)
    assert np.array_equal(host(xq_d), ref["xq"]) and np.array_equal(host(a_d), ref["amax"]), t
    assert np.array_equal(host(acc_d), ref["acc"]), t
    compare_y(host(y_d), ref["y"], t)

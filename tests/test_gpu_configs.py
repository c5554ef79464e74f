"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark uses (decode entry point for m <= 16, batched otherwise).

For each distinct matrix shape of a workload (layer 0): gamma within 1e-6
relative, every ternary code and every int8 activation code bit-exact, and
the int32 accumulators bit-exact / fp32 outputs within 1e-5 relative -- on
every output where the oracle can afford the whole contraction, otherwise on
all outputs of the first and last token plus 4096 random (token, row) pairs,
each computed by the oracle one by one.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gamma, compare_codes, compare_y, host, log, to_dev, to_dev_bits, torch_mod

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
    del w
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

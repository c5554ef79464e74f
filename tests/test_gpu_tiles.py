"""Full-output GPU parity of every matrix-core configuration the batched
forward selects at the workloads' shapes, on ragged sizes the oracle can
contract in full ("BitNet b1.58 in Production", "The Mathematical
Mechanism", items 3-4).

The batched forward picks its output tile by the matrix width and token
count, and splits the k extent over several workgroups when the output tiles
are too few to fill the device.  Each case below forces one of those
configurations at a size with ragged token and row tails:
  * wide matrices (n >= 16384, the gate+up projections);
  * mid-width matrices (n around 6144, the QKV projections), with more and
    with fewer than 64 tokens;
  * narrow matrices with long rows (n = 4096 / 8192, the O and down
    projections), including the k-sliced grid that 64 tokens give and the
    two-k-group workgroups that 129..256 output tiles take (200 x 4112,
    130 x 6160);
  * the SwiGLU epilogue on wide gate / up matrices;
for ternary and for binary weights.  Bar: codes, accumulators bit-exact on
every output; y within 1e-5 relative and exactly 0 where the oracle's is 0.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gamma, compare_codes, compare_y, host, log, to_dev, to_dev_bits, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


TILE_CASES = [
    (130, 16400, 1024),   # wide: ragged n (16400 = 64 * 256 + 16) and m
    (65, 16400, 512),
    (130, 6160, 1024),    # mid width, more than 64 tokens
    (65, 6160, 1024),
    (40, 6160, 2048),     # mid width, fewer than 64 tokens
    (64, 8192, 8192),     # 128 output tiles: the k extent is split
    (200, 4112, 4096),    # narrow, long rows
    (513, 4096, 1024),    # 512 tokens plus a one-token tail
    (200, 4112, 1040),    # two k-groups with a ragged last k-step (1040 = 4 * 256 + 16)
    (130, 16400, 1040),   # the wide tile with the same ragged k-step
    (64, 8192, 4112),     # k-sliced grid whose last slice ends in a ragged k-step
    (256, 8192, 256),     # two k-groups, one k-step (fewer steps than the ring's stages)
    (130, 6160, 16),      # two k-groups, one partial k-step of 16 columns
]


@pytest.mark.parametrize("m,n,k", TILE_CASES)
def test_batched_tile_ternary(blq, m, n, k):
    torch = torch_mod()
    tag = "batched tile m=%d n=%d k=%d" % (m, n, k)
    log("case", tag)
    w = synth.latent_weights((301, n, k), n, k)
    x = synth.activations_bf16((302, m, k), m, k, 0.005)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    xq_d, a_d = blq.bitlinear_quant_act(to_dev_bits(x))
    acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y_d = blq.bitlinear_forward_batched(packed, gamma, n, k, xq_d, a_d, acc=acc_d)
    y_noacc = blq.bitlinear_forward_batched(packed, gamma, n, k, xq_d, a_d)
    ref = oracle.forward(x, w)
    same = check_gamma(host(gamma)[0], ref["gamma"], tag)
    bad = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), ref["q"], w, ref["gamma"], same, tag)
    keep = np.setdiff1d(np.arange(n), bad)
    assert np.array_equal(host(xq_d), ref["xq"]) and np.array_equal(host(a_d), ref["amax"]), tag
    assert np.array_equal(host(acc_d)[:, keep], ref["acc"][:, keep]), tag
    compare_y(host(y_d)[:, keep], ref["y"][:, keep], tag)
    # with and without the optional accumulators: the same y bits
    assert np.array_equal(host(y_noacc), host(y_d)), tag


@pytest.mark.parametrize("m,n,k", TILE_CASES)
def test_batched_tile_binary(blq, m, n, k):
    torch = torch_mod()
    tag = "batched binary tile m=%d n=%d k=%d" % (m, n, k)
    log("case", tag)
    s = np.float32(0.0173)
    w = synth.latent_weights((303, n, k), n, k)
    x = synth.activations_bf16((304, m, k), m, k, 0.005)
    packed = blq.bitlinear_pack_binary(to_dev(w))
    sd = torch.from_numpy(np.array([s], np.float32)).cuda()
    xq_d, a_d = blq.bitlinear_quant_act(to_dev_bits(x))
    acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y_d = blq.bitlinear_forward_binary(packed, sd, n, k, xq_d, a_d, acc=acc_d)
    ref = oracle.forward_binary(x, w, s)
    assert np.array_equal(host(blq.bitlinear_unpack_binary(packed, n, k)), ref["b"]), tag
    assert np.array_equal(host(acc_d), ref["acc"]), tag
    compare_y(host(y_d), ref["y"], tag)


@pytest.mark.parametrize("m,f,k", [(17, 8208, 512), (130, 8208, 512), (64, 14336, 1024)])
def test_batched_swiglu_wide(blq, m, f, k):
    """Gate / up matrices of at least 8192 features: the wide SwiGLU tile."""
    torch = torch_mod()
    tag = "batched swiglu m=%d f=%d k=%d" % (m, f, k)
    log("case", tag)
    wg = synth.latent_weights((305, f, k), f, k)
    wu = synth.latent_weights((306, f, k), f, k)
    x = synth.activations_bf16((307, m, k), m, k, 0.005)
    pg, gg = blq.bitlinear_pack_weights(to_dev(wg))
    pu, gu = blq.bitlinear_pack_weights(to_dev(wu))
    xq_d, a_d = blq.bitlinear_quant_act(to_dev_bits(x))
    acc_d = torch.empty((m, 2 * f), dtype=torch.int32, device="cuda")
    h_d = blq.bitlinear_forward_swiglu(pg, gg, pu, gu, f, k, xq_d, a_d, acc=acc_d)
    xq_o, a_o = oracle.quant_act(x)
    assert np.array_equal(host(xq_d), xq_o), tag
    keep = np.arange(f)
    accs = []
    for p, gd, w, name in ((pg, gg, wg, "gate"), (pu, gu, wu, "up")):
        g_o = oracle.gamma(w)
        q_o = oracle.ternarize(w, g_o)
        same = check_gamma(host(gd)[0], g_o, tag + " " + name)
        bad = compare_codes(host(blq.bitlinear_unpack_weights(p, f, k)), q_o, w, g_o, same, tag + " " + name)
        keep = np.setdiff1d(keep, bad)
        accs.append((g_o, oracle.contract(xq_o, q_o)))
    acc = host(acc_d)
    assert np.array_equal(acc[:, :f][:, keep], accs[0][1][:, keep]), tag
    assert np.array_equal(acc[:, f:][:, keep], accs[1][1][:, keep]), tag
    h_o = oracle.swiglu(oracle.dequant(accs[0][1], accs[0][0], a_o), oracle.dequant(accs[1][1], accs[1][0], a_o))
    compare_y(host(h_d)[:, keep], h_o[:, keep], tag)

"""GPU parity of the steps on either side of the contraction, against the CPU
oracle on the same seeded inputs:

  * RMSNorm ahead of the activation quantisation ("BitNet b1.58 in
    Production", listing "bit_linear.py"), standalone and fused into the
    decode forward;
  * per-token quantisation from fp32 (the SwiGLU output feeding the down
    projection).

Bar of the RMSNorm path: the oracle normalises first and quantises x_norm
(the listing's order); the kernels quantise x * gain and fold r into a'.  A
code may take the other neighbour only where the oracle's x_norm * 127 / a'
lies within 2^-19 of a rounding tie (relative), position by position; a'
within 6 ulps; accumulators bit-exact for every token without such a code
and otherwise within the number of such codes; y within 1e-5 relative plus
those codes' weight.  The fp32 quantisation: codes, a' and accumulators
bit-exact.  y within 1e-5 relative and exactly 0 where the oracle's is 0.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (assert_within_ulps, check_gamma, check_norm_codes, compare_acc_flips, compare_codes,
                            compare_y, compare_y_flips, host, log, to_dev, to_dev_bits, torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


def gain_of(kind, seed, k):
    if kind == "none":
        return None
    g = synth.norm_gain(seed, k)
    return -g if kind == "negated" else g


NORM_SHAPES = [(1, 8), (1, 2560), (3, 4096), (5, 6912), (2, 1000), (4, 1003), (7, 28672), (16, 2048),
               (2, 40000), (1, 1)]


@pytest.mark.parametrize("m,k", NORM_SHAPES)
@pytest.mark.parametrize("gain_kind", ["none", "synthetic", "negated"])
def test_rmsnorm_quant_parity(blq, m, k, gain_kind):
    tag = "rmsnorm m=%d k=%d gain=%s" % (m, k, gain_kind)
    log("case", tag)
    x = synth.activations_bf16((101, m, k), m, k, 0.01)
    w = gain_of(gain_kind, (102, k), k)
    xq_d, a_d = blq.bitlinear_rmsnorm_quant_act(to_dev_bits(x), gain=None if w is None else to_dev(w))
    xq_o, a_o, _, xn_o = oracle.rmsnorm_quant_act(x, w, with_xnorm=True)
    check_norm_codes(host(xq_d), host(a_d), xq_o, a_o, xn_o, tag)


def test_rmsnorm_quant_degenerate(blq):
    k = 512
    x = synth.activations_bf16((103,), 7, k)
    x[1] = 0                                     # all-zero token
    x[2] = synth.fp32_to_bf16_bits(np.full(k, 2.0 ** -20, dtype=np.float32))  # eps dominates
    x[3, 1:] = 0                                 # one non-zero value
    x[6] = synth.fp32_to_bf16_bits(np.full(k, 1.5, dtype=np.float32))  # constant token
    w = synth.norm_gain((104,), k)
    tiny = np.full(k, 2.0 ** -30, dtype=np.float32)  # max|x_norm| below the 1e-8 floor on every token
    for gname, gain, eps in (("none", None, oracle.RMS_EPS), ("set", w, 0.0), ("set", w, 1.0),
                             ("zero", np.zeros(k, dtype=np.float32), oracle.RMS_EPS),
                             ("tiny", tiny, oracle.RMS_EPS), ("tiny", tiny, 0.0)):
        tag = "degenerate gain=%s eps=%r" % (gname, eps)
        log("case", tag)
        xq_d, a_d = blq.bitlinear_rmsnorm_quant_act(to_dev_bits(x), gain=None if gain is None else to_dev(gain), eps=eps)
        # with eps = 0 the all-zero token has no x_norm (0 / 0): outside the contract
        rows = np.array([t for t in range(x.shape[0]) if not (eps == 0.0 and t == 1)])
        xq_o, a_o, _, xn_o = oracle.rmsnorm_quant_act(x[rows], gain, eps=eps, with_xnorm=True)
        check_norm_codes(host(xq_d)[rows], host(a_d)[rows], xq_o, a_o, xn_o, tag)
        assert np.all(np.isfinite(host(a_d))), tag
        if gname == "tiny" and eps == 0.0:
            # constant token 1.5: x_norm = 2^-30 exactly, below the floor, so the
            # scale is 127 / 1e-8: every code is Round(2^-30 * 1.27e10) = 12
            assert np.all(host(xq_d)[6] == 12), tag


def test_rmsnorm_quant_misaligned(blq):
    torch = torch_mod()
    m, k = 3, 1024
    x = synth.activations_bf16((105,), m, k + 1)
    w = synth.norm_gain((106,), k + 1)
    xd = to_dev_bits(x)[:, 1:].contiguous()      # fresh buffer, aligned
    base = to_dev_bits(x).view(-1)[1:1 + m * k].view(m, k)   # 2-byte aligned view
    wd = to_dev(w)[1:]                            # 4-byte aligned view
    for xin, xh in ((xd, x[:, 1:]), (base, x.reshape(-1)[1:1 + m * k].reshape(m, k))):
        xq_d, a_d = blq.bitlinear_rmsnorm_quant_act(xin, gain=wd)
        xq_o, a_o, _, xn_o = oracle.rmsnorm_quant_act(np.ascontiguousarray(xh), w[1:], with_xnorm=True)
        check_norm_codes(host(xq_d), host(a_d), xq_o, a_o, xn_o, "misaligned")
    torch.cuda.synchronize()


def test_rmsnorm_quant_rejects_bad_eps(blq):
    x = to_dev_bits(synth.activations_bf16((107,), 1, 64))
    for eps in (-1.0, float("inf"), float("nan")):
        with pytest.raises(blq.BitlinearError) as e:
            blq.bitlinear_rmsnorm_quant_act(x, eps=eps)
        assert e.value.status == blq.BITLINEAR_E_VALUE


# ---------------------------------------------------------------------------
# fused RMSNorm + quantisation + decode forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(2560, 2560), (700, 1000), (3840, 2560), (2560, 6912), (64, 14336), (33, 1003),
                                 (601 * 16 - 7, 300)])  # last: 601 row blocks, several per workgroup
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16])
@pytest.mark.parametrize("gain_kind", ["none", "synthetic"])
def test_rmsnorm_quant_forward_parity(blq, n, k, m, gain_kind):
    if not blq.bitlinear_quant_forward_supported(m, k):
        pytest.skip("m*k codes beyond the on-chip budget of the fused path")
    torch = torch_mod()
    tag = "rmsnorm_quant_forward n=%d k=%d m=%d gain=%s" % (n, k, m, gain_kind)
    log("case", tag)
    w = synth.latent_weights((108, n, k), n, k)
    x = synth.activations_bf16((109, m, k), m, k, 0.01)
    gn = gain_of(gain_kind, (110, k), k)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
    xq_d = torch.empty((m, k), dtype=torch.int8, device="cuda")
    a_d = torch.empty(m, dtype=torch.float32, device="cuda")
    y_d = blq.bitlinear_rmsnorm_quant_forward(packed, gamma, n, k, to_dev_bits(x), gain=None if gn is None else to_dev(gn),
                                              acc=acc_d, xq=xq_d, x_absmax=a_d)
    g_or = oracle.gamma(w)
    q_or = oracle.ternarize(w, g_or)
    same = check_gamma(host(gamma)[0], g_or, tag)
    bad_rows = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), q_or, w, g_or, same, tag)
    keep = np.setdiff1d(np.arange(n), bad_rows)
    xq_o, a_o, _, xn_o = oracle.rmsnorm_quant_act(x, gn, with_xnorm=True)
    flips = check_norm_codes(host(xq_d), host(a_d), xq_o, a_o, xn_o, tag)
    acc_o = oracle.contract(xq_o, q_or)
    compare_acc_flips(host(acc_d)[:, keep], acc_o[:, keep], flips, tag)
    compare_y_flips(host(y_d)[:, keep], oracle.dequant(acc_o, g_or, a_o)[:, keep], flips, g_or, a_o, tag)
    # the fused prologue computes the standalone kernel's codes, and its a' to
    # within one ulp (fp64 mean squares summed in different orders)
    xq_s, a_s = blq.bitlinear_rmsnorm_quant_act(to_dev_bits(x), gain=None if gn is None else to_dev(gn))
    assert np.array_equal(host(xq_s), host(xq_d)), tag
    assert_within_ulps(host(a_s), host(a_d), 1, tag)


# ---------------------------------------------------------------------------
# quantisation from fp32
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 1), (1, 7), (3, 1023), (2, 1024), (5, 13824), (1, 28672), (64, 6912),
                                 (3, 40000), (16, 14336)])
def test_quant_act_f32_parity(blq, m, k):
    tag = "quant_f32 m=%d k=%d" % (m, k)
    log("case", tag)
    x = synth.activations_f32((111, m, k), m, k, 3.0)
    if m > 1:
        x[m // 2] = 0.0
    xq_d, a_d = blq.bitlinear_quant_act_f32(to_dev(x))
    xq_o, a_o = oracle.quant_act_f32(x)
    assert np.array_equal(host(xq_d), xq_o), tag
    assert np.array_equal(host(a_d), a_o), tag


def test_quant_act_f32_misaligned(blq):
    m, k = 4, 2048
    x = synth.activations_f32((112,), m, k + 1)
    base = to_dev(x).view(-1)[1:1 + m * k].view(m, k)    # 4-byte aligned view
    xq_d, a_d = blq.bitlinear_quant_act_f32(base)
    xq_o, a_o = oracle.quant_act_f32(x.reshape(-1)[1:1 + m * k].reshape(m, k))
    assert np.array_equal(host(xq_d), xq_o) and np.array_equal(host(a_d), a_o)


# ---------------------------------------------------------------------------
# fp32 quantisation fused into the decode forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(2560, 6912), (700, 1000), (4096, 14336), (33, 1003)])
@pytest.mark.parametrize("m", [1, 2, 8])
def test_quant_forward_f32_parity(blq, n, k, m):
    if not blq.bitlinear_quant_forward_supported(m, k):
        pytest.skip("m*k codes beyond the on-chip budget of the fused path")
    torch = torch_mod()
    tag = "quant_forward_f32 n=%d k=%d m=%d" % (n, k, m)
    log("case", tag)
    w = synth.latent_weights((113, n, k), n, k)
    x = synth.activations_f32((114, m, k), m, k, 0.5)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
    xq_d = torch.empty((m, k), dtype=torch.int8, device="cuda")
    a_d = torch.empty(m, dtype=torch.float32, device="cuda")
    y_d = blq.bitlinear_quant_forward_f32(packed, gamma, n, k, to_dev(x), acc=acc_d, xq=xq_d, x_absmax=a_d)
    g_or = oracle.gamma(w)
    q_or = oracle.ternarize(w, g_or)
    same = check_gamma(host(gamma)[0], g_or, tag)
    bad_rows = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), q_or, w, g_or, same, tag)
    keep = np.setdiff1d(np.arange(n), bad_rows)
    xq_o, a_o = oracle.quant_act_f32(x)
    assert np.array_equal(host(xq_d), xq_o) and np.array_equal(host(a_d), a_o), tag
    acc_o = oracle.contract(xq_o, q_or)
    assert np.array_equal(host(acc_d)[:, keep], acc_o[:, keep]), tag
    compare_y(host(y_d)[:, keep], oracle.dequant(acc_o, g_or, a_o)[:, keep], tag)

"""GPU parity of the table-lookup decode forward (bitlinear_forward_lut,
"BitNet 1-bit LLM Inference Framework", section "How the LUT Kernel Works")
against the CPU oracle on the same seeded inputs, and bitwise against the
matrix-core decode kernel.

Bar: as every forward -- int32 accumulators bit-exact, y within 1e-5
relative and exactly 0 where the oracle's is 0.  The table holds exact
integer partial sums, so y also equals bitlinear_forward's bit for bit.
Shapes span several 16 x 256 tiles with ragged tails, n large enough that
each persistent workgroup serves many 16-row blocks, and the largest k whose
table fits on chip.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gamma, compare_codes, compare_y, host, log, to_dev, to_dev_bits, torch_mod

pytestmark = pytest.mark.gpu

K_MAX = 39 * 256  # largest k whose 16-byte-per-column table fits 158 KiB


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


def run_case(blq, n, k, m, seed, w=None, x=None):
    tag = "lut n=%d k=%d m=%d seed=%d" % (n, k, m, seed)
    log("case", tag)
    torch = torch_mod()
    if w is None:
        w = synth.latent_weights(seed, n, k)
    if x is None:
        x = synth.activations_bf16(seed + 1000, m, k, 0.01)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    xq_d, amax_d = blq.bitlinear_quant_act(to_dev_bits(x))
    acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y_d = blq.bitlinear_forward_lut(packed, gamma, n, k, xq_d, amax_d, acc=acc_d)
    ref = oracle.forward(x, w)
    same = check_gamma(host(gamma)[0], ref["gamma"], tag)
    bad = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), ref["q"], w, ref["gamma"], same, tag)
    assert np.array_equal(host(xq_d), ref["xq"]), tag
    keep = np.setdiff1d(np.arange(n), bad)
    acc = host(acc_d)
    assert np.array_equal(acc[:, keep], ref["acc"][:, keep]), tag
    compare_y(host(y_d)[:, keep], ref["y"][:, keep], tag)
    # the matrix-core decode kernel on the same device operands: bitwise equal
    acc2 = torch.empty_like(acc_d)
    y2 = blq.bitlinear_forward(packed, gamma, n, k, xq_d, amax_d, acc=acc2)
    assert torch.equal(acc_d, acc2), tag
    assert torch.equal(y_d, y2), tag
    return acc


SHAPES = [(16, 256), (17, 257), (48, 1000), (200, 2048), (257, 4112), (64, 6912), (5, 1), (40, 16)]


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 2, 5, 16])
def test_lut_forward_parity(blq, n, k, m):
    run_case(blq, n, k, m, seed=n + 13 * k + m)


@pytest.mark.parametrize("n,k", [(20000, 2560), (12345, 4096), (3000, K_MAX)])
def test_lut_forward_many_row_blocks(blq, n, k):
    """More 16-row blocks than resident workgroups: each builds its table once
    and serves several blocks."""
    run_case(blq, n, k, 1, seed=n + k)


def test_lut_forward_degenerate(blq):
    run_case(blq, 30, 500, 2, seed=1, w=np.zeros((30, 500), np.float32))
    x = synth.activations_bf16(5, 3, 512, 0.01)
    x[1] = 0
    run_case(blq, 40, 512, 3, seed=2, x=x)
    # largest accumulators the table path can meet: codes +-127, weights all +1 / all -1
    k = K_MAX
    w = np.full((16, k), 0.5, np.float32)
    w[1] = -0.5
    xb = synth.fp32_to_bf16_bits(np.stack([np.ones(k, np.float32), -np.ones(k, np.float32)]))
    acc = run_case(blq, 16, k, 2, seed=3, w=w, x=xb)
    assert acc[0, 0] == 127 * k and acc[1, 0] == -127 * k and acc[0, 1] == -127 * k


def test_lut_forward_stays_in_bounds(blq):
    torch = torch_mod()
    n, k, m = 100, 3000, 3
    w = synth.latent_weights(4, n, k)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    xq, amax = blq.bitlinear_quant_act(to_dev_bits(synth.activations_bf16(4, m, k, 0.01)))
    guard = 64
    yb = torch.full((m * n + 2 * guard,), float("nan"), device="cuda")
    ab = torch.full((m * n + 2 * guard,), -7, dtype=torch.int32, device="cuda")
    blq.bitlinear_forward_lut(packed, gamma, n, k, xq, amax, y=yb[guard:guard + m * n].view(m, n),
                              acc=ab[guard:guard + m * n].view(m, n))
    y2 = blq.bitlinear_forward_lut(packed, gamma, n, k, xq, amax)
    assert torch.equal(yb[guard:guard + m * n].view(m, n), y2)
    yh, ah = host(yb), host(ab)
    assert np.isnan(yh[:guard]).all() and np.isnan(yh[-guard:]).all()
    assert (ah[:guard] == -7).all() and (ah[-guard:] == -7).all()


def test_lut_forward_unsupported(blq):
    torch = torch_mod()
    assert blq.bitlinear_forward_lut_supported(K_MAX)
    assert not blq.bitlinear_forward_lut_supported(K_MAX + 1)
    n = 32
    for m, k in ((1, K_MAX + 1), (17, 256)):
        packed, gamma = blq.bitlinear_pack_weights(to_dev(synth.latent_weights(1, n, k)))
        xq, amax = blq.bitlinear_quant_act(to_dev_bits(synth.activations_bf16(1, m, k, 0.0)))
        with pytest.raises(blq.BitlinearError) as e:
            blq.bitlinear_forward_lut(packed, gamma, n, k, xq, amax)
        assert e.value.status == blq.BITLINEAR_E_UNSUPPORTED
    torch.cuda.synchronize()

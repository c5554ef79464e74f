"""GPU parity of the variant modes against the CPU oracle on the same seeded
inputs:
  V1 per-tensor activation quantisation with Q_b = 128 ("BitNet 1-bit LLM
     Inference Framework", the BitLinear class under "The Core Structure of
     BitNet b1.58") and its forward;
  V2 one binary16 scale per output channel ("BitNet-2B-4T: Inside the
     2B-Parameter, 4T-Token 1-Bit LLM", "Weight Representation: Ternary +
     Scale, Not Pure Binary");
  V3 binary sign weights with a per-layer scale ("BitNet's 1-Bit Transformer:
     Architecture Breakdown", "Binary Weight Matrices with Learnable Scaling").

Bar: int8 codes, binary16 scale bits, ternary / sign codes and int32
accumulators bit-exact; the per-tensor max bit-exact; y within 1e-5 relative
and exactly 0 where the oracle's is 0 (the GPU forms the scale in fp32 with at
most three roundings, the oracle in binary64 with one).  Expected values come
only from the oracle applied to the seeded inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check_gamma, compare_codes, compare_y, host, log, to_dev, to_dev_bits, torch_mod

pytestmark = pytest.mark.gpu

SHAPES = [(16, 256), (17, 257), (48, 1000), (200, 2048), (257, 4112), (64, 6912), (5, 1), (40, 16), (33, 768)]
MS = [1, 2, 5, 16, 17, 64, 130]


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


def scalar_dev(v):
    return to_dev(np.array([v], np.float32))


# ---------------------------------------------------------------------------
# V1: per-tensor activations, Q_b = 128
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 1), (1, 7), (3, 255), (1, 16384), (2, 8193), (1, 28672), (64, 4096),
                                 (300, 4112), (16, 2560)])
def test_tensor_quant_parity(blq, m, k):
    tag = "tensor quant m=%d k=%d" % (m, k)
    log("case", tag)
    x = synth.activations_bf16(m * 7 + k, m, k, 0.01)
    xq, g = blq.bitlinear_quant_act_tensor(to_dev_bits(x))
    xq_o, g_o = oracle.quant_act_tensor(x)
    assert host(g)[0] == g_o, tag
    assert np.array_equal(host(xq), xq_o), tag
    assert xq_o.min() == -128 or xq_o.max() == 127, tag  # the max element sits at an end of the range


def test_tensor_quant_special_inputs(blq):
    torch = torch_mod()
    # all zero: codes 0, g = 0
    xq, g = blq.bitlinear_quant_act_tensor(to_dev_bits(np.zeros((3, 100), np.uint16)))
    assert host(g)[0] == 0 and not host(xq).any()
    # the max is a negative value in the last token; a tiny tensor where the epsilon matters
    for x in (synth.activations_bf16(3, 4, 3000, 0.0), synth.fp32_to_bf16_bits(np.array([[2.0 ** -27, 0, -2.0 ** -28]], np.float32))):
        x = x.copy()
        if x.shape[1] == 3000:
            x[3, 1234] = synth.fp32_to_bf16_bits(np.array([-50.0], np.float32))[0]
        xq, g = blq.bitlinear_quant_act_tensor(to_dev_bits(x))
        xq_o, g_o = oracle.quant_act_tensor(x)
        assert host(g)[0] == g_o and np.array_equal(host(xq), xq_o)
    # misaligned views of x and xq (scalar paths)
    x = synth.activations_bf16(9, 5, 9000, 0.01)
    buf = torch.zeros(x.size + 1, dtype=torch.int16, device="cuda")
    buf[1:] = to_dev_bits(x).reshape(-1)
    qbuf = torch.zeros(x.size + 3, dtype=torch.int8, device="cuda")
    xq, g = blq.bitlinear_quant_act_tensor(buf[1:].view(5, 9000), xq=qbuf[3:].view(5, 9000))
    xq_o, g_o = oracle.quant_act_tensor(x)
    assert host(g)[0] == g_o and np.array_equal(host(xq), xq_o)


def tensor_forward_case(blq, n, k, m, seed, w=None, x=None):
    tag = "tensor forward n=%d k=%d m=%d" % (n, k, m)
    log("case", tag)
    torch = torch_mod()
    if w is None:
        w = synth.latent_weights(seed, n, k)
    if x is None:
        x = synth.activations_bf16(seed + 1, m, k, 0.01)
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    ref = oracle.forward_tensor_act(x, w)
    same = check_gamma(host(gamma)[0], ref["gamma"], tag)
    bad = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), ref["q"], w, ref["gamma"], same, tag)
    keep = np.setdiff1d(np.arange(n), bad)
    xq, g = blq.bitlinear_quant_act_tensor(to_dev_bits(x))
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y = blq.bitlinear_forward_tensor_act(packed, gamma, n, k, xq, g, acc=acc)
    assert np.array_equal(host(xq), ref["xq"]), tag
    assert host(g)[0] == ref["gx"], tag
    assert np.array_equal(host(acc)[:, keep], ref["acc"][:, keep]), tag
    compare_y(host(y)[:, keep], ref["y"][:, keep], tag)
    return host(acc)


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", MS)
def test_tensor_forward_parity(blq, n, k, m):
    tensor_forward_case(blq, n, k, m, seed=3 * n + k + m)


def test_tensor_forward_extremes(blq):
    """codes -128 against weights -1: acc = 128 k at the largest k allowed."""
    k = (1 << 18) - 1
    w = np.full((16, k), -0.5, np.float32)
    w[1] = 0.5
    x = synth.fp32_to_bf16_bits(np.stack([-np.ones(k, np.float32), np.ones(k, np.float32)]))
    acc = tensor_forward_case(blq, 16, k, 2, seed=0, w=w, x=x)
    assert acc[0, 0] == 128 * k and acc[1, 0] == -127 * k and acc[0, 1] == -128 * k


# ---------------------------------------------------------------------------
# V2: per-row binary16 scales
# ---------------------------------------------------------------------------

def rowscale_pack_case(blq, w, tag):
    n, k = w.shape
    packed, scales = blq.bitlinear_pack_weights_rowscale(to_dev(w))
    s_o = oracle.row_scales(w)
    assert np.array_equal(host(scales).view(np.uint16), s_o), tag
    q_o = oracle.ternarize_rows(w, s_o)
    assert np.array_equal(host(blq.bitlinear_unpack_weights(packed, n, k)), q_o), tag
    return packed, scales, s_o, q_o


@pytest.mark.parametrize("n,k", SHAPES)
def test_rowscale_pack_parity(blq, n, k):
    w = synth.latent_weights(n + 5 * k, n, k)
    # rows at very different scales, a zero row, a row with a subnormal binary16 scale
    w = w * (2.0 ** (np.arange(n) % 7 - 3)).astype(np.float32)[:, None]
    w[n // 2] = 0.0
    if n > 2:
        w[1] = np.float32(3e-6)
    rowscale_pack_case(blq, w.astype(np.float32), "rowscale pack n=%d k=%d" % (n, k))


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", MS)
def test_rowscale_forward_parity(blq, n, k, m):
    tag = "rowscale forward n=%d k=%d m=%d" % (n, k, m)
    log("case", tag)
    torch = torch_mod()
    seed = 5 * n + k + m
    w = synth.latent_weights(seed, n, k) * (1.0 + (np.arange(n) % 5)).astype(np.float32)[:, None]
    w = w.astype(np.float32)
    x = synth.activations_bf16(seed + 2, m, k, 0.01)
    packed, scales, s_o, q_o = rowscale_pack_case(blq, w, tag)
    xq, amax = blq.bitlinear_quant_act(to_dev_bits(x))
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y = blq.bitlinear_forward_rowscale(packed, scales, n, k, xq, amax, acc=acc)
    ref = oracle.forward_rowscale(x, w)
    assert np.array_equal(ref["s16"], s_o)
    assert np.array_equal(host(acc), ref["acc"]), tag
    compare_y(host(y), ref["y"], tag)


# ---------------------------------------------------------------------------
# V3: binary sign weights
# ---------------------------------------------------------------------------

def decode_binary_layout(raw: np.ndarray, n: int, k: int) -> np.ndarray:
    """Sign codes from the packed bytes, read by the layout the header states
    (independent of the library's own unpack)."""
    kt = (k + 511) // 512
    words = raw.view(np.uint32)
    out = np.empty((n, k), np.int8)
    for r in range(n):
        for c in range(k):
            t, cc = divmod(c, 512)
            g, cw = divmod(cc, 128)
            s, col = divmod(cw, 32)
            slot = (r % 16) + 16 * g
            word = words[((r // 16) * kt + t) * 256 + slot * 4 + s]
            bit = 8 * (col % 4) + 7 - col // 4
            out[r, c] = -1 if (int(word) >> bit) & 1 else 1
    return out


@pytest.mark.parametrize("n,k", [(16, 256), (17, 257), (5, 1), (33, 600)])
def test_binary_pack_layout(blq, n, k):
    w = synth.latent_weights(n * k, n, k)
    special = np.array([0.0, -0.0, -1e-30], np.float32)[:k]
    w[0, :special.size] = special
    packed = blq.bitlinear_pack_binary(to_dev(w))
    b_o = oracle.binarize(w)
    assert np.array_equal(decode_binary_layout(host(packed), n, k), b_o)
    assert np.array_equal(host(blq.bitlinear_unpack_binary(packed, n, k)), b_o)


def binary_case(blq, n, k, m, seed, s=0.0173, fused=False, w=None, x=None):
    tag = "binary n=%d k=%d m=%d%s" % (n, k, m, " fused" if fused else "")
    log("case", tag)
    torch = torch_mod()
    if w is None:
        w = synth.latent_weights(seed, n, k)
    if x is None:
        x = synth.activations_bf16(seed + 3, m, k, 0.01)
    packed = blq.bitlinear_pack_binary(to_dev(w))
    ref = oracle.forward_binary(x, w, np.float32(s))
    assert np.array_equal(host(blq.bitlinear_unpack_binary(packed, n, k)), ref["b"]), tag
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    if fused and not blq.bitlinear_quant_forward_binary_supported(m, k):
        with pytest.raises(blq.BitlinearError) as e:
            blq.bitlinear_quant_forward_binary(packed, scalar_dev(s), n, k, to_dev_bits(x))
        assert e.value.status == blq.BITLINEAR_E_UNSUPPORTED
        return None
    if fused:
        xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
        amax = torch.empty(m, dtype=torch.float32, device="cuda")
        y = blq.bitlinear_quant_forward_binary(packed, scalar_dev(s), n, k, to_dev_bits(x), acc=acc, xq=xq,
                                               x_absmax=amax)
    else:
        xq, amax = blq.bitlinear_quant_act(to_dev_bits(x))
        y = blq.bitlinear_forward_binary(packed, scalar_dev(s), n, k, xq, amax, acc=acc)
    assert np.array_equal(host(xq), ref["xq"]), tag
    assert np.array_equal(host(amax), ref["amax"]), tag
    assert np.array_equal(host(acc), ref["acc"]), tag
    compare_y(host(y), ref["y"], tag)
    return host(acc)


@pytest.mark.parametrize("n,k", SHAPES + [(64, 4352), (16, 8448)])
@pytest.mark.parametrize("m", MS + [300])
def test_binary_forward_parity(blq, n, k, m):
    binary_case(blq, n, k, m, seed=7 * n + k + m)


@pytest.mark.parametrize("n,k", SHAPES + [(2560, 6912), (601 * 16 - 7, 300)])  # last: 601 row blocks
@pytest.mark.parametrize("m", [1, 3, 16])
def test_binary_fused_forward_parity(blq, n, k, m):
    binary_case(blq, n, k, m, seed=11 * n + k + m, fused=True)


def test_binary_forward_long_rows_and_extremes(blq):
    # codes that do not fit on chip at m = 16 (global-operand decode kernel), odd tile count
    binary_case(blq, 40, 28672 + 256, 16, seed=4)
    # +-127 codes against all +1 / all -1 rows
    k = 1 << 18
    w = np.full((16, k), 0.5, np.float32)
    w[1] = -0.5
    x = synth.fp32_to_bf16_bits(np.stack([np.ones(k, np.float32), -np.ones(k, np.float32)]))
    acc = binary_case(blq, 16, k, 2, seed=5, w=w, x=x)
    assert acc[0, 0] == 127 * k and acc[1, 0] == -127 * k and acc[0, 1] == -127 * k


def test_variant_forwards_stay_in_bounds(blq):
    torch = torch_mod()
    n, k = 100, 3000
    w = synth.latent_weights(12, n, k)
    pb = blq.bitlinear_pack_binary(to_dev(w))
    pr, sc = blq.bitlinear_pack_weights_rowscale(to_dev(w))
    pt, gm = blq.bitlinear_pack_weights(to_dev(w))
    for m in (3, 70):
        x = to_dev_bits(synth.activations_bf16(13 + m, m, k, 0.01))
        xq, amax = blq.bitlinear_quant_act(x)
        xqt, g = blq.bitlinear_quant_act_tensor(x)
        calls = [lambda y, a: blq.bitlinear_forward_binary(pb, scalar_dev(0.02), n, k, xq, amax, y=y, acc=a),
                 lambda y, a: blq.bitlinear_forward_rowscale(pr, sc, n, k, xq, amax, y=y, acc=a),
                 lambda y, a: blq.bitlinear_forward_tensor_act(pt, gm, n, k, xqt, g, y=y, acc=a)]
        for call in calls:
            guard = 64
            yb = torch.full((m * n + 2 * guard,), float("nan"), device="cuda")
            ab = torch.full((m * n + 2 * guard,), -7, dtype=torch.int32, device="cuda")
            call(yb[guard:guard + m * n].view(m, n), ab[guard:guard + m * n].view(m, n))
            y2 = call(None, None)
            assert torch.equal(yb[guard:guard + m * n].view(m, n), y2)
            yh, ah = host(yb), host(ab)
            assert np.isnan(yh[:guard]).all() and np.isnan(yh[-guard:]).all()
            assert (ah[:guard] == -7).all() and (ah[-guard:] == -7).all()

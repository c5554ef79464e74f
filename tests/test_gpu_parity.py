"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.

Bar (stated once, applied everywhere):
  * int8 activation codes, ternary codes and int32 accumulators: bit-exact;
  * a' (per-token absmax): bit-exact (it is a max of exact values);
  * gamma: within 1e-6 relative (fp64 sums in different orders, one rounding
    to fp32 each; in practice the bits agree);
  * fp32 outputs y: within 1e-5 relative, and exactly 0 where the oracle's is 0.
Shapes span several 16 x 256 weight tiles with ragged tails in n and k, token
counts on both sides of the decode/batched split, and the degenerate cases of
the method (all-zero weights, all-zero tokens, k = 1).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (check_gamma, compare_codes, compare_y, host, log, to_dev, to_dev_bits,
                            torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def blq():
    torch_mod()
    import bitlinear_quant_act_amd as m
    m.load_library()
    return m


def gpu_pack(blq, w: np.ndarray):
    packed, gamma = blq.bitlinear_pack_weights(to_dev(w))
    return packed, gamma


def run_case(blq, n, k, m, seed, batched, outliers=0.01, w=None, x=None, check_acc=True):
    tag = "n=%d k=%d m=%d seed=%d %s" % (n, k, m, seed, "batched" if batched else "decode")
    log("case", tag)
    if w is None:
        w = synth.latent_weights(seed, n, k)
    if x is None:
        x = synth.activations_bf16(seed + 1000, m, k, outliers)
    packed, gamma = gpu_pack(blq, w)
    xq_d, amax_d = blq.bitlinear_quant_act(to_dev_bits(x))
    torch = torch_mod()
    acc_d = torch.empty((m, n), dtype=torch.int32, device="cuda")
    fwd = blq.bitlinear_forward_batched if batched else blq.bitlinear_forward
    y_d = fwd(packed, gamma, n, k, xq_d, amax_d, acc=acc_d)
    ref = oracle.forward(x, w)
    g_same = check_gamma(host(gamma)[0], ref["gamma"], tag)
    codes = host(blq.bitlinear_unpack_weights(packed, n, k))
    bad_rows = compare_codes(codes, ref["q"], w, ref["gamma"], g_same, tag)
    assert np.array_equal(host(xq_d), ref["xq"]), tag
    assert np.array_equal(host(amax_d), ref["amax"]), tag
    keep = np.setdiff1d(np.arange(n), bad_rows)
    acc = host(acc_d)
    if check_acc:
        assert np.array_equal(acc[:, keep], ref["acc"][:, keep]), tag
    compare_y(host(y_d)[:, keep], ref["y"][:, keep], tag)
    return acc, host(y_d)


def test_native_library_is_loaded(blq):
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert blq.LIB_PATH in maps


# ---------------------------------------------------------------------------
# activation quantisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,k", [(1, 1), (1, 7), (3, 255), (2, 256), (5, 257), (1, 2048), (4, 2560),
                                 (9, 4096), (16, 6912), (1, 28672), (64, 8192), (512, 4096),
                                 (3, 40000), (65, 1000), (77, 2056), (100, 14336), (66, 28672)])
def test_quant_act_parity(blq, m, k):
    log("quant m=%d k=%d" % (m, k))
    x = synth.activations_bf16(m * 7 + k, m, k, 0.01)
    xq, amax = blq.bitlinear_quant_act(to_dev_bits(x))
    rq, ra = oracle.quant_act(x)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(amax), ra)


def test_quant_act_special_tokens(blq):
    k = 512
    x = np.zeros((6, k), dtype=np.float32)
    x[1, 3] = 1e-12                                   # below the 1e-8 floor
    x[2, :10] = [127 / 64, 5 / 128, 7 / 128, 3 / 128, 1 / 128, -5 / 128, -3 / 128, 9 / 128, 0.5, -127 / 64]
    x[3] = np.linspace(-3, 3, k)
    x[4] = 3.3e38 * np.sign(np.linspace(-1, 1, k))    # near the top of the bf16 range
    x[5, ::2] = 2.0 ** -126                           # smallest normal values
    xb = synth.fp32_to_bf16_bits(x)
    xq, amax = blq.bitlinear_quant_act(to_dev_bits(xb))
    rq, ra = oracle.quant_act(xb)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(host(amax), ra)
    assert (host(xq)[0] == 0).all()


def test_quant_act_misaligned_rows(blq):
    """Rows that start off a 16-byte boundary take the general path."""
    torch = torch_mod()
    m, k = 3, 1000
    x = synth.activations_bf16(77, m, k, 0.01)
    base = torch.zeros(m * k + 8, dtype=torch.int16, device="cuda")
    base[1:1 + m * k] = to_dev_bits(x).view(-1)
    xv = base[1:1 + m * k].view(m, k)
    out = torch.zeros(m * k + 8, dtype=torch.int8, device="cuda")
    xq = out[3:3 + m * k].view(m, k)
    _, amax = blq.bitlinear_quant_act(xv, xq=xq)
    rq, ra = oracle.quant_act(x)
    assert np.array_equal(host(xq), rq) and np.array_equal(host(amax), ra)
    o = host(out)
    assert (o[:3] == 0).all() and (o[3 + m * k:] == 0).all()


# ---------------------------------------------------------------------------
# pack / unpack
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", [(1, 1), (3, 5), (16, 256), (17, 257), (33, 1000), (128, 2048),
                                 (100, 4099), (2048, 2048)])
def test_pack_parity(blq, n, k):
    tag = "pack n=%d k=%d" % (n, k)
    log(tag)
    w = synth.latent_weights(n * 31 + k, n, k)
    packed, gamma = gpu_pack(blq, w)
    g_or = oracle.gamma(w)
    same = check_gamma(host(gamma)[0], g_or, tag)
    codes = host(blq.bitlinear_unpack_weights(packed, n, k))
    compare_codes(codes, oracle.ternarize(w, g_or), w, g_or, same, tag)
    assert packed.numel() == blq.bitlinear_packed_bytes(n, k)


def test_pack_degenerate_weights(blq):
    for name, w in [("zeros", np.zeros((20, 300), np.float32)),
                    ("constant", np.full((20, 300), 0.37, np.float32)),
                    ("negative constant", np.full((20, 300), -1e-3, np.float32)),
                    ("single", np.array([[-0.25]], np.float32))]:
        log("pack", name)
        packed, gamma = gpu_pack(blq, w)
        g_or = oracle.gamma(w)
        assert host(gamma)[0] == g_or, name
        assert np.array_equal(host(blq.bitlinear_unpack_weights(packed, *w.shape)), oracle.ternarize(w, g_or)), name


def test_pack_misaligned_weights(blq):
    torch = torch_mod()
    n, k = 40, 600
    w = synth.latent_weights(5, n, k)
    base = torch.zeros(n * k + 4, dtype=torch.float32, device="cuda")
    base[1:1 + n * k] = to_dev(w).view(-1)
    packed, gamma = blq.bitlinear_pack_weights(base[1:1 + n * k].view(n, k))
    g_or = oracle.gamma(w)
    same = check_gamma(host(gamma)[0], g_or, "misaligned")
    compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), oracle.ternarize(w, g_or), w, g_or, same,
                  "misaligned")


def test_pack_is_deterministic(blq):
    w = synth.latent_weights(99, 300, 3000)
    p1, g1 = gpu_pack(blq, w)
    p2, g2 = gpu_pack(blq, w)
    assert np.array_equal(host(p1), host(p2)) and host(g1)[0] == host(g2)[0]


# ---------------------------------------------------------------------------
# forward: decode and batched paths
# ---------------------------------------------------------------------------

SHAPES = [(16, 256), (17, 257), (48, 1000), (200, 2048), (257, 4112), (64, 6912), (5, 1), (40, 16)]
# 601 row blocks (the last one ragged) on the decode kernels' persistent grid:
# three row blocks per workgroup for all but the last, which takes two; two
# tiles per row block, so most waves of a workgroup have none
MANY_ROW_BLOCKS = (601 * 16 - 7, 300)


@pytest.mark.parametrize("n,k", SHAPES + [MANY_ROW_BLOCKS])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 9, 16])
def test_forward_decode_parity(blq, n, k, m):
    run_case(blq, n, k, m, seed=n + 7 * k + m, batched=False)


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("m", [1, 9, 17, 64, 100, 129, 300])
def test_forward_batched_parity(blq, n, k, m):
    run_case(blq, n, k, m, seed=n + 11 * k + m, batched=True)


def test_forward_degenerate(blq):
    # all-zero weights: gamma 0, every output exactly 0
    run_case(blq, 30, 500, 3, seed=1, batched=False, w=np.zeros((30, 500), np.float32))
    run_case(blq, 30, 500, 70, seed=1, batched=True, w=np.zeros((30, 500), np.float32))
    # an all-zero token beside ordinary ones
    x = synth.activations_bf16(5, 4, 512, 0.01)
    x[2] = 0
    run_case(blq, 40, 512, 4, seed=2, batched=False, x=x)
    run_case(blq, 40, 512, 4, seed=2, batched=True, x=x)
    # extreme accumulators: every code +-127 against all-(+1) weights
    k = 28672
    w = np.full((16, k), 0.5, np.float32)
    w[1] = -0.5
    xb = synth.fp32_to_bf16_bits(np.stack([np.ones(k, np.float32), -np.ones(k, np.float32)]))
    acc, _ = run_case(blq, 16, k, 2, seed=3, batched=False, w=w, x=xb)
    assert acc[0, 0] == 127 * k and acc[1, 0] == -127 * k and acc[0, 1] == -127 * k
    acc, _ = run_case(blq, 16, k, 2, seed=3, batched=True, w=w, x=xb)
    assert acc[0, 0] == 127 * k


def test_batched_k_slices_stay_in_bounds(blq):
    """Sizes the matrix-core path splits over k (zeroed int32 sums in y's or
    acc's memory, atomics, an in-place finish): bitwise equal with and
    without acc, deterministic, and guard bands around y and acc intact."""
    torch = torch_mod()
    for n, k, m in ((100, 5000, 70), (33, 28672, 20)):
        w = synth.latent_weights(n + k, n, k)
        packed, gamma = gpu_pack(blq, w)
        x = synth.activations_bf16(m + k, m, k, 0.01)
        xq, amax = blq.bitlinear_quant_act(to_dev_bits(x))
        guard = 64
        yb = torch.full((m * n + 2 * guard,), float("nan"), device="cuda")
        ab = torch.full((m * n + 2 * guard,), -7, dtype=torch.int32, device="cuda")
        y1 = yb[guard:guard + m * n].view(m, n)
        a1 = ab[guard:guard + m * n].view(m, n)
        blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax, y=y1, acc=a1)
        y2 = blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax)
        y3 = blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax)
        assert torch.equal(y1, y2) and torch.equal(y2, y3), (n, k, m)
        assert torch.isnan(yb[:guard]).all() and torch.isnan(yb[-guard:]).all()
        assert (ab[:guard] == -7).all() and (ab[-guard:] == -7).all()
        ref = oracle.forward(x, w)
        g_same = check_gamma(host(gamma)[0], ref["gamma"], "k-slices")
        bad = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), ref["q"], w, ref["gamma"], g_same,
                            "k-slices")
        keep = np.setdiff1d(np.arange(n), bad)
        assert np.array_equal(host(a1)[:, keep], ref["acc"][:, keep])
        compare_y(host(y1)[:, keep], ref["y"][:, keep], "k-slices")


def test_batched_k_slices_in_a_graph(blq):
    """The split path's three launches (zero fill, k-slices, finish) captured
    in a HIP graph: every replay, with eager work between replays, matches
    the eager result bit for bit."""
    torch = torch_mod()
    n, k, m = 96, 8192, 40
    w = synth.latent_weights(77, n, k)
    packed, gamma = gpu_pack(blq, w)
    xq, amax = blq.bitlinear_quant_act(to_dev_bits(synth.activations_bf16(78, m, k, 0.01)))
    y_ref = blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax)
    a_ref = torch.empty((m, n), dtype=torch.int32, device="cuda")
    blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax, acc=a_ref)
    y = torch.empty((m, n), device="cuda")
    a = torch.empty((m, n), dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax, y=y, acc=a)
    for _ in range(3):
        y.fill_(float("nan"))
        a.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(a, a_ref)
        blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax)  # eager work between replays
        torch.cuda.synchronize()


def test_decode_and_batched_agree_bitwise(blq):
    torch = torch_mod()
    n, k = 300, 4096
    w = synth.latent_weights(3, n, k)
    packed, gamma = gpu_pack(blq, w)
    for m in (1, 5, 16):
        xq, amax = blq.bitlinear_quant_act(to_dev_bits(synth.activations_bf16(m, m, k, 0.005)))
        a1 = torch.empty((m, n), dtype=torch.int32, device="cuda")
        a2 = torch.empty((m, n), dtype=torch.int32, device="cuda")
        blq.bitlinear_forward(packed, gamma, n, k, xq, amax, acc=a1)
        blq.bitlinear_forward_batched(packed, gamma, n, k, xq, amax, acc=a2)
        assert torch.equal(a1, a2)


def test_forward_is_deterministic_and_stays_in_bounds(blq):
    """Two runs are bitwise equal; guard bands around every output stay intact."""
    torch = torch_mod()
    n, k, m = 100, 3000, 7
    w = synth.latent_weights(4, n, k)
    packed, gamma = gpu_pack(blq, w)
    xq, amax = blq.bitlinear_quant_act(to_dev_bits(synth.activations_bf16(4, m, k, 0.01)))
    for fwd in (blq.bitlinear_forward, blq.bitlinear_forward_batched):
        guard = 64
        yb = torch.full((m * n + 2 * guard,), float("nan"), device="cuda")
        ab = torch.full((m * n + 2 * guard,), -7, dtype=torch.int32, device="cuda")
        y1 = yb[guard:guard + m * n].view(m, n)
        a1 = ab[guard:guard + m * n].view(m, n)
        fwd(packed, gamma, n, k, xq, amax, y=y1, acc=a1)
        y2 = fwd(packed, gamma, n, k, xq, amax)
        assert torch.equal(y1, y2)
        yh, ah = host(yb), host(ab)
        assert np.isnan(yh[:guard]).all() and np.isnan(yh[-guard:]).all()
        assert (ah[:guard] == -7).all() and (ah[-guard:] == -7).all()


def test_forward_on_a_side_stream(blq):
    torch = torch_mod()
    n, k, m = 64, 2048, 3
    w = synth.latent_weights(8, n, k)
    x = synth.activations_bf16(8, m, k, 0.01)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        wd = to_dev(w)
        xd = to_dev_bits(x)
        packed, gamma = blq.bitlinear_pack_weights(wd, stream=s)
        xq, amax = blq.bitlinear_quant_act(xd, stream=s)
        y = blq.bitlinear_forward(packed, gamma, n, k, xq, amax, stream=s)
    s.synchronize()
    ref = oracle.forward(x, w)
    compare_y(y.cpu().numpy(), ref["y"], "side stream")


# ---------------------------------------------------------------------------
# fused activation quantisation + decode forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k", SHAPES + [(2560, 6912), (64, 14336), MANY_ROW_BLOCKS])
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 16])
def test_quant_forward_parity(blq, n, k, m):
    if not blq.bitlinear_quant_forward_supported(m, k):
        pytest.skip("m*k beyond the fused path's on-chip budget")
    torch = torch_mod()
    tag = "fused n=%d k=%d m=%d" % (n, k, m)
    log("case", tag)
    w = synth.latent_weights(n + 13 * k + m, n, k)
    x = synth.activations_bf16(n + 17 * k + m, m, k, 0.01)
    packed, gamma = gpu_pack(blq, w)
    xd = to_dev_bits(x)
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    amax = torch.empty(m, dtype=torch.float32, device="cuda")
    y = blq.bitlinear_quant_forward(packed, gamma, n, k, xd, acc=acc, xq=xq, x_absmax=amax)
    ref = oracle.forward(x, w)
    g_same = check_gamma(host(gamma)[0], ref["gamma"], tag)
    bad = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), ref["q"], w, ref["gamma"], g_same, tag)
    keep = np.setdiff1d(np.arange(n), bad)
    assert np.array_equal(host(xq), ref["xq"]), tag
    assert np.array_equal(host(amax), ref["amax"]), tag
    assert np.array_equal(host(acc)[:, keep], ref["acc"][:, keep]), tag
    compare_y(host(y)[:, keep], ref["y"][:, keep], tag)
    # the two-launch path gives the same bits
    xq2, amax2 = blq.bitlinear_quant_act(xd)
    y2 = blq.bitlinear_forward(packed, gamma, n, k, xq2, amax2)
    assert torch.equal(y, y2), tag


def test_quant_forward_long_row_one_token(blq):
    """One token of more than 32768 values: the fused prologue reads the row
    again for the quantisation instead of keeping it in registers."""
    torch = torch_mod()
    n, k, m = 300, 40000, 1
    assert blq.bitlinear_quant_forward_supported(m, k)
    w = synth.latent_weights(23, n, k)
    x = synth.activations_bf16(24, m, k, 0.01)
    packed, gamma = gpu_pack(blq, w)
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    amax = torch.empty(m, dtype=torch.float32, device="cuda")
    y = blq.bitlinear_quant_forward(packed, gamma, n, k, to_dev_bits(x), acc=acc, xq=xq, x_absmax=amax)
    ref = oracle.forward(x, w)
    same = check_gamma(host(gamma)[0], ref["gamma"], "fused k=40000")
    bad = compare_codes(host(blq.bitlinear_unpack_weights(packed, n, k)), ref["q"], w, ref["gamma"], same,
                        "fused k=40000")
    keep = np.setdiff1d(np.arange(n), bad)
    assert np.array_equal(host(xq), ref["xq"]) and np.array_equal(host(amax), ref["amax"])
    assert np.array_equal(host(acc)[:, keep], ref["acc"][:, keep])
    compare_y(host(y)[:, keep], ref["y"][:, keep], "fused k=40000")


def test_quant_forward_without_optional_outputs(blq):
    torch = torch_mod()
    n, k, m = 300, 2560, 1
    w = synth.latent_weights(21, n, k)
    x = synth.activations_bf16(22, m, k, 0.0)
    packed, gamma = gpu_pack(blq, w)
    y = blq.bitlinear_quant_forward(packed, gamma, n, k, to_dev_bits(x))
    compare_y(host(y), oracle.forward(x, w)["y"], "fused, no optional outputs")


def test_quant_forward_misaligned_input(blq):
    torch = torch_mod()
    n, k, m = 48, 1000, 3
    w = synth.latent_weights(31, n, k)
    x = synth.activations_bf16(32, m, k, 0.01)
    packed, gamma = gpu_pack(blq, w)
    base = torch.zeros(m * k + 8, dtype=torch.int16, device="cuda")
    base[1:1 + m * k] = to_dev_bits(x).view(-1)
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y = blq.bitlinear_quant_forward(packed, gamma, n, k, base[1:1 + m * k].view(m, k), acc=acc)
    ref = oracle.forward(x, w)
    assert np.array_equal(host(acc), ref["acc"])
    compare_y(host(y), ref["y"], "fused misaligned")


def test_quant_forward_unsupported_sizes(blq):
    torch = torch_mod()
    n, k = 32, 14336
    w = torch.zeros((n, k), dtype=torch.float32, device="cuda")
    packed, gamma = blq.bitlinear_pack_weights(w)
    x = torch.zeros((16, k), dtype=torch.int16, device="cuda")
    assert not blq.bitlinear_quant_forward_supported(16, k)
    with pytest.raises(blq.BitlinearError) as e:
        blq.bitlinear_quant_forward(packed, gamma, n, k, x)
    assert e.value.status == blq.BITLINEAR_E_UNSUPPORTED

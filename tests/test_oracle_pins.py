"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these compares the oracle with itself: each check uses a closed form,
an exact rational computation, a brute-force enumeration in plain Python
integers, an invariant of the definition, a hand-worked fixture in
tests/golden/, or an independent library routine (numpy, torch on the CPU).

Definitions pinned ("BitNet b1.58 in Production: 1-Bit LLMs and Energy
Benchmarks", section "The Mathematical Mechanism"):
  item 1  gamma = mean |W|, W_q = Clip(Round(W / (gamma + eps)), -1, 1)
  item 2  x_q = Clip(Round(x * Q_b / (max|x| + eps)), -Q_b, Q_b), Q_b = 127
  item 3  acc = sum of +x (w = +1), nothing (w = 0), -x (w = -1)
  item 4  y = acc * gamma * max|x| / Q_b
and ("BitNet 1-bit LLM Inference Framework: Running Large Language Models on
CPU", section "How the LUT Kernel Works") the 2-bit codes 00 = 0, 01 = +1,
10 = -1 and the scalar conditional-add loop; section "The Difference in How
Computation Works" gives the mask form (W == 1) @ x - (W == -1) @ x.
"""
from __future__ import annotations

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS_W = np.float32(1e-5)


# ---------------------------------------------------------------------------
# helpers independent of the oracle
# ---------------------------------------------------------------------------

def f32_nearest(fr: Fraction) -> np.float32:
    """Correctly rounded binary32 of an exact rational (ties to even mantissa)."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        if best is None or d < best[0]:
            best = (d, cand)
        elif d == best[0]:
            # tie: even mantissa
            if int(np.float32(cand).view(np.uint32)) % 2 == 0:
                best = (d, cand)
    return np.float32(best[1])


def bits(v: np.ndarray) -> np.ndarray:
    return synth.fp32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


# ---------------------------------------------------------------------------
# O1 gamma
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(3, 7), (64, 1000), (1, 1)])
@pytest.mark.parametrize("c", [0.015625, 0.0173, 3.0])
def test_gamma_constant_magnitude(oracle_mod, shape, c):
    """|W| == c everywhere => gamma == c exactly (the binary64 sum of at most
    2^22 copies of a binary32 value is exact, and so is the division)."""
    c = np.float32(c)
    rng = np.random.default_rng(5)
    signs = np.where(rng.random(shape) < 0.5, -1.0, 1.0).astype(np.float32)
    w = signs * c
    assert oracle_mod.gamma(w) == c


@pytest.mark.parametrize("shape", [(4, 8), (16, 64), (2, 2)])
def test_gamma_exact_rational(oracle_mod, shape):
    """Weights on a 2^-12 grid with n*k a power of two: the mean is exact, so
    gamma must be the correctly rounded binary32 of the exact rational mean."""
    rng = np.random.default_rng(11)
    ints = rng.integers(-4096, 4097, size=shape)
    w = (ints.astype(np.float64) / 4096.0).astype(np.float32)
    exact = sum(Fraction(abs(int(v)), 4096) for v in ints.ravel()) / (shape[0] * shape[1])
    assert oracle_mod.gamma(w) == f32_nearest(exact)


def test_gamma_vs_numpy_pairwise_sum(oracle_mod):
    """numpy's pairwise binary64 summation and the oracle's sequential one
    round to the same binary32 (or 1 ulp apart in a rare boundary case)."""
    w = synth.latent_weights(123, 700, 900)
    ref = np.float32(np.abs(w.astype(np.float64)).sum() / w.size)
    assert ulp_diff(oracle_mod.gamma(w), ref) <= 1


def test_gamma_normal_expectation(oracle_mod):
    """E|W| = sigma * sqrt(2/pi) for W ~ N(0, sigma^2); 4M samples give a
    relative standard error of ~3.8e-4, checked at 5 sigma."""
    w = synth.latent_weights(7, 2000, 2000)
    expect = 0.02 * math.sqrt(2.0 / math.pi)
    assert abs(float(oracle_mod.gamma(w)) / expect - 1.0) < 2e-3


# ---------------------------------------------------------------------------
# O2-O3 ternary RoundClip
# ---------------------------------------------------------------------------

def _gamma_for_denominator(d: float) -> np.float32:
    """A binary32 gamma with fl32(gamma + 1e-5) == d exactly."""
    g = np.float32(np.float32(d) - EPS_W)
    assert np.float32(g + EPS_W) == np.float32(d)
    return g


def test_ternary_ties_unit_denominator(oracle_mod):
    """d = gamma + 1e-5 == 1 exactly, so W/d == W and the rounding rule is
    visible directly.  Expected codes from Round-half-even then Clip."""
    g = _gamma_for_denominator(1.0)
    half_up = np.nextafter(np.float32(0.5), np.float32(1))
    half_dn = np.nextafter(np.float32(0.5), np.float32(0))
    w = np.array([[0.5, -0.5, half_up, -half_up, half_dn, 1.5, 2.5, -1.5, -2.5,
                   1.0, -1.0, 0.0, 100.0, -100.0, 0.75, -0.25]], dtype=np.float32)
    expect = [0, 0, 1, -1, 0, 1, 1, -1, -1, 1, -1, 0, 1, -1, 1, 0]
    assert oracle_mod.ternarize(w, g).ravel().tolist() == expect


def test_ternary_ties_half_denominator(oracle_mod):
    """d == 0.5 exactly: W = 0.25 is the tie 0.5 -> 0; W = 0.75 is 1.5 -> 2
    -> clip 1; the neighbour above 0.25 rounds to 1.  A dropped epsilon would
    make d = 0.49999 and turn the first tie into +1."""
    g = _gamma_for_denominator(0.5)
    w = np.array([[0.25, 0.75, np.nextafter(np.float32(0.25), np.float32(1)), -0.25,
                   0.125, -0.75]], dtype=np.float32)
    assert oracle_mod.ternarize(w, g).ravel().tolist() == [0, 1, 1, 0, 0, -1]


def test_ternary_closed_forms(oracle_mod):
    """W == 0: gamma == 0 and the epsilon alone keeps W/d finite -> all 0.
    W == +c: every W/d = c/(c+1e-5) is in (0.5, 1] -> +1; W == -c -> -1."""
    z = np.zeros((5, 9), dtype=np.float32)
    g0 = oracle_mod.gamma(z)
    assert g0 == 0.0
    assert (oracle_mod.ternarize(z, g0) == 0).all()
    for c in (1e-4, 0.02, 7.0):
        w = np.full((4, 6), c, dtype=np.float32)
        g = oracle_mod.gamma(w)
        assert (oracle_mod.ternarize(w, g) == 1).all()
        assert (oracle_mod.ternarize(-w, g) == -1).all()


def test_ternary_sign_symmetry(oracle_mod):
    w = synth.latent_weights(3, 300, 300)
    g = oracle_mod.gamma(w)
    assert np.array_equal(oracle_mod.ternarize(-w, g), -oracle_mod.ternarize(w, g))


def test_ternary_zero_and_clip_fraction(oracle_mod):
    """Fraction of zero codes is P(|W| <= d/2) and of codes whose quotient
    reaches the clip is P(|W| >= 3d/2) for W ~ N(0, 0.02^2): erf closed forms
    (binomial standard error ~2.3e-4, checked at ~5 sigma)."""
    w = synth.latent_weights(0, 2048, 2048)
    g = oracle_mod.gamma(w)
    q = oracle_mod.ternarize(w, g)
    d = float(np.float32(g + EPS_W))
    sig = 0.02 * math.sqrt(2.0)
    p_zero = math.erf(0.5 * d / sig)
    p_clip = 1.0 - math.erf(1.5 * d / sig)
    assert abs((q == 0).mean() - p_zero) < 1.2e-3
    t = np.abs(w.astype(np.float64)) / d
    assert abs((t >= 1.5).mean() - p_clip) < 1.2e-3
    # the analytic values for N(0, 0.02) latents (~31% zeros, ~23% clipped)
    assert abs(p_zero - 0.3102) < 2e-3 and abs(p_clip - 0.2311) < 2e-3


def test_ternary_vs_torch_listing_expression(oracle_mod):
    """The page's weight_quant expression evaluated by torch on the CPU in
    binary32 (torch.round is half-to-even), with the additive 1e-5 reading."""
    torch = pytest.importorskip("torch")
    w = synth.latent_weights(21, 512, 777)
    g = oracle_mod.gamma(w)
    tw = torch.from_numpy(w)
    denom = torch.tensor(g, dtype=torch.float32) + torch.tensor(1e-5, dtype=torch.float32)
    ref = torch.clamp(torch.round(tw / denom), -1, 1).to(torch.int8).numpy()
    assert np.array_equal(oracle_mod.ternarize(w, g), ref)


# ---------------------------------------------------------------------------
# O4 canonical 2-bit packing
# ---------------------------------------------------------------------------

CODE = {0: 0b00, 1: 0b01, -1: 0b10}


def test_pack_all_81_valid_bytes(oracle_mod):
    seen = set()
    for combo in itertools.product((-1, 0, 1), repeat=4):
        q = np.array([combo], dtype=np.int8)
        b = oracle_mod.pack_canonical(q)
        expect = sum(CODE[v] << (2 * i) for i, v in enumerate(combo))
        assert b.tolist() == [[expect]]
        assert oracle_mod.unpack_canonical(b, 1, 4).tolist() == [list(combo)]
        seen.add(expect)
    assert len(seen) == 81


def test_unpack_rejects_all_175_invalid_bytes(oracle_mod):
    rejected = 0
    for v in range(256):
        fields = [(v >> (2 * i)) & 3 for i in range(4)]
        b = np.array([[v]], dtype=np.uint8)
        if 3 in fields:
            with pytest.raises(oracle_mod.OracleError):
                oracle_mod.unpack_canonical(b, 1, 4)
            rejected += 1
        else:
            oracle_mod.unpack_canonical(b, 1, 4)
    assert rejected == 175


def test_pack_golden_bytes(oracle_mod):
    with open(os.path.join(GOLDEN, "pack_canonical.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array([c["codes"]], dtype=np.int8)
        assert oracle_mod.pack_canonical(q).ravel().tolist() == c["bytes"], c["note"]
        assert oracle_mod.unpack_canonical(np.array(c["bytes"], np.uint8), 1, c["k"]).ravel().tolist() == c["codes"]


def test_unpack_rejects_nonzero_padding(oracle_mod):
    # k = 5: the second byte may only use its lowest field
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.unpack_canonical(np.array([0, 0b0100], np.uint8), 1, 5)


@pytest.mark.parametrize("n,k", [(1, 1), (3, 5), (17, 255), (8, 2048), (5, 1027)])
def test_pack_roundtrip_random(oracle_mod, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    b = oracle_mod.pack_canonical(q)
    assert b.shape == (n, (k + 3) // 4)
    assert np.array_equal(oracle_mod.unpack_canonical(b, n, k), q)


# ---------------------------------------------------------------------------
# O5 per-token activation quantization
# ---------------------------------------------------------------------------

def test_quant_ties_round_half_even(oracle_mod):
    """a' = 127/64 is exact in bf16, so s = fl32(127 / a') = 64 exactly and
    x = j/128 lands on j/2: the .5 cases expose the rounding rule (round half
    away from zero would give 3, 4, 2, 1, -3, -2 instead)."""
    vals = [127 / 64, 5 / 128, 7 / 128, 3 / 128, 1 / 128, -5 / 128, -3 / 128, 0.0, 9 / 128, 64 / 128]
    assert np.float32(127.0) / np.float32(127 / 64) == np.float32(64.0)
    xq, amax = oracle_mod.quant_act(bits([vals]))
    assert amax.tolist() == [np.float32(127 / 64)]
    assert xq.ravel().tolist() == [127, 2, 4, 2, 0, -2, -2, 0, 4, 32]


def test_quant_golden_scale(oracle_mod):
    """a' = 2: s = 63.5 exactly; 63.5 -> 64 (tie to even), -31.75 -> -32."""
    xq, amax = oracle_mod.quant_act(bits([[1.0, -0.5, 2.0, 0.25]]))
    assert xq.tolist() == [[64, -32, 127, 16]] and amax.tolist() == [2.0]


def test_quant_invariants(oracle_mod):
    x = synth.activations_bf16(9, 64, 1536, 0.01)
    xq, amax = oracle_mod.quant_act(x)
    xf = synth.bf16_bits_to_fp32(x)
    # a' is the exact per-token max |x| (all tokens far above the 1e-8 floor)
    assert np.array_equal(amax, np.abs(xf).max(axis=1))
    # the max element always maps to +-127; -128 never appears
    assert (np.abs(xq.astype(np.int32)).max(axis=1) == 127).all()
    assert xq.min() >= -127
    # odd symmetry
    xq_neg, amax_neg = oracle_mod.quant_act(x ^ np.uint16(0x8000))
    assert np.array_equal(xq_neg, -xq) and np.array_equal(amax_neg, amax)
    # exact power-of-two scaling of the token leaves the codes unchanged
    for j in (-3, 5):
        xs = synth.fp32_to_bf16_bits(xf * np.float32(2.0 ** j))
        assert np.array_equal(synth.bf16_bits_to_fp32(xs), xf * np.float32(2.0 ** j))
        xq_s, amax_s = oracle_mod.quant_act(xs)
        assert np.array_equal(xq_s, xq)
        assert np.array_equal(amax_s, amax * np.float32(2.0 ** j))


def test_quant_zero_and_tiny_tokens(oracle_mod):
    x = np.zeros((3, 40), dtype=np.uint16)
    x[1, 5] = bits([[1e-12]])[0, 0]          # below the 1e-8 floor
    x[2, 7] = bits([[-3.0]])[0, 0]
    xq, amax = oracle_mod.quant_act(x)
    assert (xq[0] == 0).all() and amax[0] == np.float32(1e-8)
    # a 1e-12 element against a' = 1e-8: 1e-12 * 127e8 = 0.0127 -> 0
    assert (xq[1] == 0).all() and amax[1] == np.float32(1e-8)
    assert xq[2, 7] == -127 and (np.delete(xq[2], 7) == 0).all() and amax[2] == 3.0


@pytest.mark.parametrize("amax_val", [127 / 64, 3.0, 0.0078125, 1.7e4, 3.3e38])
def test_quant_exhaustive_bf16_vs_torch(oracle_mod, amax_val):
    """Every finite bf16 pattern with |x| <= a' as a token element, against the
    page's activation_quant expression evaluated by torch (binary32)."""
    torch = pytest.importorskip("torch")
    all_bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = synth.bf16_bits_to_fp32(all_bits)
    a_bits = bits([[amax_val]])[0, 0]
    a = synth.bf16_bits_to_fp32(np.array([a_bits]))[0]
    keep = np.isfinite(vals) & (np.abs(vals) <= a)
    cand = all_bits[keep]
    width = 4096
    pad = (-len(cand)) % (width - 1)
    cand = np.concatenate([cand, np.zeros(pad, np.uint16)])
    rows = cand.reshape(-1, width - 1)
    x = np.concatenate([np.full((rows.shape[0], 1), a_bits, np.uint16), rows], axis=1)
    xq, amax = oracle_mod.quant_act(x)
    tx = torch.from_numpy(synth.bf16_bits_to_fp32(x))
    qmax = 127
    scale = torch.max(torch.abs(tx), dim=-1, keepdim=True)[0].clamp(min=1e-8)
    ref = torch.clamp(torch.round(tx * (qmax / scale)), -qmax, qmax).to(torch.int8).numpy()
    assert np.array_equal(xq, ref)
    assert np.array_equal(amax, scale.squeeze(1).numpy())


# ---------------------------------------------------------------------------
# O6 contraction
# ---------------------------------------------------------------------------

def _rand_xq(rng, m, k):
    return rng.integers(-127, 128, size=(m, k)).astype(np.int8)


def test_contract_closed_forms(oracle_mod):
    rng = np.random.default_rng(2)
    m, n, k = 5, 7, 333
    xq = _rand_xq(rng, m, k)
    rowsum = xq.astype(np.int64).sum(axis=1)
    ones = np.ones((n, k), np.int8)
    assert np.array_equal(oracle_mod.contract(xq, ones), np.repeat(rowsum[:, None], n, 1))
    assert np.array_equal(oracle_mod.contract(xq, -ones), -np.repeat(rowsum[:, None], n, 1))
    assert (oracle_mod.contract(xq, np.zeros((n, k), np.int8)) == 0).all()
    # one-hot rows pick single activations (with sign)
    pos = rng.integers(0, k, size=n)
    sgn = np.where(np.arange(n) % 2 == 0, 1, -1)
    oh = np.zeros((n, k), np.int8)
    oh[np.arange(n), pos] = sgn
    expect = xq[:, pos].astype(np.int64) * sgn[None, :]
    assert np.array_equal(oracle_mod.contract(xq, oh), expect)


def test_contract_brute_force_4x8(oracle_mod):
    """All 3^8 = 6561 ternary rows of K = 8 against 4 tokens (including the
    +-127 extremes), checked against a plain-Python integer double loop and
    against the mask form (W == 1) @ x - (W == -1) @ x."""
    q = np.array(list(itertools.product((-1, 0, 1), repeat=8)), dtype=np.int8)
    rng = np.random.default_rng(4)
    xq = np.stack([np.full(8, 127), np.full(8, -127),
                   np.array([127, -127, 0, 1, -1, 64, -64, 3]),
                   rng.integers(-127, 128, 8)]).astype(np.int8)
    acc = oracle_mod.contract(xq, q)
    assert acc.shape == (4, 6561)
    xl = xq.astype(int).tolist()
    ql = q.astype(int).tolist()
    brute = [[sum(a * w for a, w in zip(xl[i], ql[j])) for j in range(6561)] for i in range(4)]
    assert acc.tolist() == brute
    mask = ((q == 1).astype(np.int64) @ xq.T.astype(np.int64)
            - (q == -1).astype(np.int64) @ xq.T.astype(np.int64)).T
    assert np.array_equal(acc, mask)


@pytest.mark.parametrize("m,n,k", [(1, 300, 1000), (5, 129, 2049), (16, 64, 4096)])
def test_contract_vs_numpy_int64(oracle_mod, m, n, k):
    rng = np.random.default_rng(m + n + k)
    xq = _rand_xq(rng, m, k)
    q = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
    ref = xq.astype(np.int64) @ q.T.astype(np.int64)
    assert np.array_equal(oracle_mod.contract(xq, q), ref)


def test_contract_k_permutation_invariance(oracle_mod):
    rng = np.random.default_rng(8)
    xq = _rand_xq(rng, 3, 517)
    q = rng.integers(-1, 2, size=(11, 517)).astype(np.int8)
    perm = rng.permutation(517)
    assert np.array_equal(oracle_mod.contract(xq, q), oracle_mod.contract(xq[:, perm], q[:, perm]))


def test_contract_overflow_bound_at_largest_k(oracle_mod):
    """|acc| <= 127 K; at K = 28672 the extreme is 3,641,344 < 2^31, reached
    exactly by all-127 activations against all-(+1) weights."""
    k = 28672
    xq = np.full((2, k), 127, np.int8)
    xq[1] = -127
    q = np.ones((3, k), np.int8)
    q[1] = -1
    q[2, ::2] = -1
    acc = oracle_mod.contract(xq, q)
    assert acc.tolist() == [[127 * k, -127 * k, 0], [-127 * k, 127 * k, 0]]
    assert 127 * k == 3641344 < 2 ** 31


def test_contract_rejects_non_ternary(oracle_mod):
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.contract(np.ones((1, 4), np.int8), np.array([[0, 2, 0, 0]], np.int8))


def test_contract_pairs_match_full(oracle_mod):
    rng = np.random.default_rng(10)
    xq = _rand_xq(rng, 6, 300)
    q = rng.integers(-1, 2, size=(20, 300)).astype(np.int8)
    full = xq.astype(np.int64) @ q.T.astype(np.int64)
    rows = rng.integers(0, 6, 50)
    cols = rng.integers(0, 20, 50)
    assert np.array_equal(oracle_mod.contract_pairs(xq, q, rows, cols), full[rows, cols])


# ---------------------------------------------------------------------------
# O7 dequantization
# ---------------------------------------------------------------------------

def test_dequant_exact_rational(oracle_mod):
    """y is the correctly rounded binary32 of acc * gamma * a' / 127 (the
    binary64 evaluation may differ by one ulp only at a rounding boundary)."""
    rng = np.random.default_rng(12)
    m, n = 6, 40
    acc = rng.integers(-3641344, 3641345, size=(m, n)).astype(np.int32)
    acc[0, :5] = 0
    g = np.float32(0.0159)
    amax = (rng.random(m) * 20 + 0.25).astype(np.float32)
    y = oracle_mod.dequant(acc, g, amax)
    exact = [[f32_nearest(Fraction(int(acc[i, j])) * Fraction(float(g)) * Fraction(float(amax[i])) / 127)
              for j in range(n)] for i in range(m)]
    d = ulp_diff(y, np.array(exact, np.float32))
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    assert ((y == 0) == (acc == 0)).all()


# ---------------------------------------------------------------------------
# end to end: hand-worked examples
# ---------------------------------------------------------------------------

def test_golden_end_to_end(oracle_mod):
    with open(os.path.join(GOLDEN, "bitlinear_small.json")) as f:
        exs = json.load(f)["examples"]
    for ex in exs:
        w = np.array(ex["w"], np.float32)
        x = bits(ex["x"])
        r = oracle_mod.forward(x, w)
        assert r["gamma"] == f32_nearest(Fraction(ex["gamma"])), ex["name"]
        assert r["q"].tolist() == ex["q"], ex["name"]
        amax = [np.float32(1e-8) if a == "1e-8f" else f32_nearest(Fraction(a)) for a in ex["amax"]]
        assert r["amax"].tolist() == amax, ex["name"]
        assert r["xq"].tolist() == ex["xq"], ex["name"]
        assert r["acc"].tolist() == ex["acc"], ex["name"]
        y = np.array([[f32_nearest(Fraction(v)) for v in row] for row in ex["y"]], np.float32)
        assert ulp_diff(r["y"], y).max() <= 1, ex["name"]


# ---------------------------------------------------------------------------
# RMSNorm ahead of the quantization ("BitNet b1.58 in Production", listing
# "bit_linear.py": x_norm = nn.RMSNorm(in_features)(x), then
# activation_quant(x_norm)).  The oracle forms x_norm value by value:
# r = 1 / sqrt(mean x^2 + eps) (binary64, rounded once to binary32),
# x_norm = (x * r) * w in binary32, then the per-token absmax rule.
# ---------------------------------------------------------------------------

RMS_EPS = float(np.finfo(np.float32).eps)
# |x_norm * s| of two evaluations that differ by a few roundings (a binary32
# mean square summed in another order, or binary64 throughout) differ by at
# most 2^-19 |x_norm * s|; a code may differ only where the value lies that
# close to a rounding tie
TIE_BAND = 2.0 ** -19


def _r_exact(x_bits_row, eps):
    """1 / sqrt(mean x^2 + eps) from the exact rational mean square."""
    xs = synth.bf16_bits_to_fp32(x_bits_row).astype(np.float64)
    ms = sum(Fraction(float(v)) ** 2 for v in xs) / len(xs) + Fraction(float(np.float32(eps)))
    return 1.0 / math.sqrt(float(ms))


def _near_tie(t):
    t = np.abs(np.asarray(t, dtype=np.float64))
    return np.abs(t - np.floor(t) - 0.5) <= TIE_BAND * t + 1e-30


def _listing_activation_quant(torch, xn):
    """activation_quant of the listing, evaluated by torch in xn's dtype."""
    qmax = 2 ** (8 - 1) - 1
    scale = torch.max(torch.abs(xn), dim=-1, keepdim=True)[0].clamp(min=1e-8)
    x_scaled = xn * (qmax / scale)
    return torch.clamp(torch.round(x_scaled), -qmax, qmax), scale[:, 0], x_scaled


def test_rmsnorm_r_is_the_rounded_reciprocal_rms(oracle_mod):
    """r is the reciprocal rms of the exact rational mean square, rounded to
    binary32 (within one ulp: a binary64 evaluation rounded twice), and
    x_norm is x times that binary32 r, times the gain, each product rounded
    to binary32."""
    x = synth.activations_bf16(11, 5, 384, 0.01)
    w = synth.norm_gain(23, 384)
    _, _, r, xn = oracle_mod.rmsnorm_quant_act(x, w, with_xnorm=True)
    xf = synth.bf16_bits_to_fp32(x)
    for t in range(5):
        assert abs(int(ulp_diff(r[t], f32_nearest(Fraction(_r_exact(x[t], RMS_EPS)))))) <= 1
        assert np.array_equal(xn[t], (xf[t] * np.float32(r[t])) * w)


def test_rmsnorm_power_of_two_rms_gives_the_gain(oracle_mod):
    """|x| == 2^j everywhere and eps = 0: r = 2^-j exactly, so x_norm = +-w
    exactly and the codes, a' and x_norm are those of the plain quantiser
    applied to the token +-w (w bf16-exact)."""
    k = 300
    rng = np.random.default_rng(19)
    w = synth.bf16_bits_to_fp32(bits(synth.norm_gain(20, k)))
    for j in (-3, 0, 5):
        signs = np.where(rng.random(k) < 0.5, -1.0, 1.0).astype(np.float32)
        x = bits((signs * np.float32(2.0 ** j))[None, :])
        xq, a, r, xn = oracle_mod.rmsnorm_quant_act(x, w, eps=0.0, with_xnorm=True)
        assert r[0] == np.float32(2.0 ** -j)
        assert np.array_equal(xn[0], signs * w)
        xq0, a0 = oracle_mod.quant_act(bits((signs * w)[None, :]))
        assert np.array_equal(xq, xq0) and a[0] == a0[0] == np.abs(w).max()


def test_rmsnorm_vs_torch_fp32_listing(oracle_mod):
    """torch's own rms_norm in binary32 followed by the listing's
    activation_quant: codes equal except at values within the tie band,
    a' within 1e-6 relative (torch sums the squares in binary32)."""
    torch = pytest.importorskip("torch")
    for seed, (m, k) in ((12, (6, 512)), (21, (3, 4096)), (22, (2, 1001))):
        x = synth.activations_bf16(seed, m, k, 0.01)
        w = synth.norm_gain(seed + 1, k)
        xq, a, _ = oracle_mod.rmsnorm_quant_act(x, w)
        xf = torch.from_numpy(synth.bf16_bits_to_fp32(x))
        xn = torch.nn.functional.rms_norm(xf, (k,), torch.from_numpy(w), RMS_EPS)
        codes, scale, t = _listing_activation_quant(torch, xn)
        codes, scale, t = codes.numpy(), scale.numpy(), t.numpy()
        assert np.allclose(a, scale, rtol=1e-6, atol=0)
        diff = codes.astype(np.int64) - xq.astype(np.int64)
        assert np.all(np.abs(diff) <= 1)
        assert np.all(_near_tie(t)[diff != 0])


def test_rmsnorm_vs_torch_fp64_listing(oracle_mod):
    """The same listing evaluated by torch in binary64 throughout."""
    torch = pytest.importorskip("torch")
    m, k = 6, 512
    x = synth.activations_bf16(12, m, k, 0.01)
    w = synth.norm_gain(13, k)
    xq, a, _ = oracle_mod.rmsnorm_quant_act(x, w)
    xf = torch.from_numpy(synth.bf16_bits_to_fp32(x).astype(np.float64))
    xn = torch.nn.functional.rms_norm(xf, (k,), torch.from_numpy(w.astype(np.float64)), RMS_EPS)
    codes, scale, t = _listing_activation_quant(torch, xn)
    codes, scale, t = codes.numpy(), scale.numpy(), t.numpy()
    assert np.allclose(a, scale, rtol=4e-7, atol=0)
    diff = codes.astype(np.int64) - xq.astype(np.int64)
    assert np.all(np.abs(diff) <= 1)
    assert np.all(_near_tie(t)[diff != 0])


def test_rmsnorm_invariances(oracle_mod):
    x = synth.activations_bf16(14, 4, 256)
    w = synth.norm_gain(15, 256)
    xq, a, _ = oracle_mod.rmsnorm_quant_act(x, w, eps=0.0)
    # power-of-two scaling of x (exact in bf16), eps = 0: r scales inversely
    # and exactly, so x_norm, the codes and a' are unchanged
    xs = bits(synth.bf16_bits_to_fp32(x) * np.float32(8.0))
    xq2, a2, _ = oracle_mod.rmsnorm_quant_act(xs, w, eps=0.0)
    assert np.array_equal(xq, xq2) and np.array_equal(a, a2)
    # negated gain: negated codes, same a'
    xq3, a3, _ = oracle_mod.rmsnorm_quant_act(x, -w, eps=0.0)
    assert np.array_equal(xq3, -xq) and np.array_equal(a3, a)
    assert np.abs(xq).max() == 127


def test_rmsnorm_closed_forms(oracle_mod):
    k = 64
    # constant token c: x_norm = c * r everywhere, every code is sign(c) * 127,
    # a' = |c| / sqrt(c^2 + eps)
    for c in (0.75, -3.0, 40.0):
        x = bits(np.full((1, k), c, dtype=np.float32))
        xq, a, r = oracle_mod.rmsnorm_quant_act(x)
        assert np.all(xq == np.sign(c) * 127)
        ref = np.float32(abs(c) / math.sqrt(c * c + float(np.float32(RMS_EPS))))
        assert abs(int(ulp_diff(a[0], ref))) <= 1
    # eps dominates a tiny token: r ~ 1 / sqrt(eps)
    tiny = 2.0 ** -20
    x = bits(np.full((1, k), tiny, dtype=np.float32))
    _, a, r = oracle_mod.rmsnorm_quant_act(x)
    ref = tiny / math.sqrt(tiny * tiny + float(np.float32(RMS_EPS)))
    assert abs(float(a[0]) - ref) <= 1e-6 * ref
    # all-zero token, or a gain of zero: codes 0, a' at its floor, no NaN
    z = np.zeros((1, k), dtype=np.uint16)
    xq, a, r = oracle_mod.rmsnorm_quant_act(z)
    assert np.all(xq == 0) and a[0] == np.float32(1e-8) and np.isfinite(r[0])
    x = synth.activations_bf16(16, 1, k)
    xq, a, _ = oracle_mod.rmsnorm_quant_act(x, np.zeros(k, dtype=np.float32))
    assert np.all(xq == 0) and a[0] == np.float32(1e-8)


def test_rmsnorm_floor_binds_on_the_normalised_token(oracle_mod):
    """The 1e-8 floor of the listing's activation_quant applies to
    max|x_norm|: a constant token (x_norm = c * r * w everywhere) with a gain
    small enough that x_norm stays below 1e-8 is quantised with the scale
    127 / 1e-8, not stretched to +-127."""
    k = 32
    c = 1.5
    for w_val, code in ((2.0 ** -30, 12), (-(2.0 ** -31), -6), (2.0 ** -40, 0)):
        x = bits(np.full((1, k), c, dtype=np.float32))
        w = np.full(k, w_val, dtype=np.float32)
        xq, a, _ = oracle_mod.rmsnorm_quant_act(x, w, eps=0.0)
        t = abs(w_val) * 127.0 / 1e-8      # c * r = 1 exactly with eps = 0
        assert abs(abs(t) - math.floor(abs(t)) - 0.5) > 1e-3        # away from a tie
        assert np.all(xq == code) and round(t) == abs(code)
        assert a[0] == np.float32(1e-8)


# ---------------------------------------------------------------------------
# quantization from binary32 (the SwiGLU output feeding the next BitLinear)
# ---------------------------------------------------------------------------

def test_quant_f32_matches_bf16_rule_on_bf16_values(oracle_mod):
    x = synth.activations_bf16(17, 7, 300, 0.01)
    xq0, a0 = oracle_mod.quant_act(x)
    xq, a = oracle_mod.quant_act_f32(synth.bf16_bits_to_fp32(x))
    assert np.array_equal(xq, xq0) and np.array_equal(a, a0)


def test_quant_f32_vs_torch_listing_expression(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(18)
    x = (rng.standard_normal((9, 777)) * 3).astype(np.float32)
    x[3] = 0.0
    xq, a = oracle_mod.quant_act_f32(x)
    xt = torch.from_numpy(x)
    scale = xt.abs().max(dim=-1, keepdim=True)[0].clamp(min=1e-8)
    ref = torch.clamp(torch.round(xt * (127.0 / scale)), -127, 127).to(torch.int8).numpy()
    assert np.array_equal(xq, ref)
    assert np.array_equal(a, scale[:, 0].numpy())


# ---------------------------------------------------------------------------
# SwiGLU ("BitNet 1-bit LLM Inference Framework", section "A Deep Look at the
# BitNet Architecture": down_proj(silu(gate_proj(x)) * up_proj(x)))
# ---------------------------------------------------------------------------

def test_swiglu_known_values_and_limits(oracle_mod):
    sig1 = 0.7310585786300049  # logistic(1)
    g = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 2.0, 0.0], dtype=np.float32)
    u = np.array([5.0, 1.0, 1.0, 3.0, 3.0, 0.0, -2.0], dtype=np.float32)
    h = oracle_mod.swiglu(g, u)
    assert h[0] == 0.0 and h[5] == 0.0 and h[6] == 0.0
    assert h[1] == np.float32(sig1)
    assert h[2] == np.float32(sig1 - 1.0)
    assert h[3] == np.float32(120.0)            # sigmoid(40) rounds to 1
    assert abs(float(h[4])) < 1e-15


def test_swiglu_identities(oracle_mod):
    rng = np.random.default_rng(19)
    g = (rng.standard_normal(5000) * 3).astype(np.float32)
    u = rng.standard_normal(5000).astype(np.float32)
    one = np.ones_like(g)
    # silu(g) - silu(-g) = g
    d = oracle_mod.swiglu(g, one).astype(np.float64) - oracle_mod.swiglu(-g, one).astype(np.float64)
    assert np.allclose(d, g, rtol=2e-7, atol=1e-7)
    # linear in u: power-of-two scaling is exact
    assert np.array_equal(oracle_mod.swiglu(g, u * np.float32(4.0)), oracle_mod.swiglu(g, u) * np.float32(4.0))


def test_swiglu_vs_torch_silu(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(20)
    g = (rng.standard_normal((13, 257)) * 4).astype(np.float32)
    u = rng.standard_normal((13, 257)).astype(np.float32)
    h = oracle_mod.swiglu(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g.astype(np.float64))) * torch.from_numpy(u.astype(np.float64))).numpy()
    assert np.all(np.abs(ulp_diff(h, ref.astype(np.float32))) <= 1)


# ---------------------------------------------------------------------------
# variant modes
# ---------------------------------------------------------------------------
# V1 "BitNet 1-bit LLM Inference Framework", "The Core Structure of BitNet
#    b1.58": the BitLinear class quantizes activations with one max over the
#    whole tensor, Q_b = 2^7, x * Q_b / (max + 1e-8) clamped to [-Q_b, Q_b - 1]
#    and then rounded, and de-quantizes by w_scale * x_scale / 2^7.
# V2 "BitNet-2B-4T: Inside the 2B-Parameter, 4T-Token 1-Bit LLM", "Weight
#    Representation: Ternary + Scale, Not Pure Binary": one FP16 scale per
#    output channel.
# V3 "BitNet's 1-Bit Transformer: Architecture Breakdown", "Binary Weight
#    Matrices with Learnable Scaling": W_bit = s * sign(W).

def test_v1_tensor_quant_hand_values():
    """g = 1, and 1 + 1e-8 rounds to 1 in binary32 (its ulp is 2^-23), so each
    code is round(clamp(128 x)): 128 -> 127 (clamp), -128 kept, 0.75 -> 96,
    2.5/128 -> tie 2.5 -> 2 (even), 0.5 -> 64, -0.25 -> -32; 0.1 is the bf16
    value 0.10009765625, 128 of it is 12.8125 -> 13."""
    import oracle
    x = bits([[1.0, -1.0, 0.75, 2.5 / 128], [0.5, 0.0, -0.25, 0.1]])
    xq, g = oracle.quant_act_tensor(x)
    assert g == np.float32(1.0)
    assert xq.tolist() == [[127, -128, 96, 2], [64, 0, -32, 13]]


def test_v1_one_scale_for_the_tensor():
    """The max is over |x| of every token: g = 4 from token 0's -4, so token
    1's 1 and -0.5 give 32 and -16 (per token they would be 127 and -64),
    and token 0's -4 gives -128 (Q_b = 128, not 127)."""
    import oracle
    xq, g = oracle.quant_act_tensor(bits([[-4.0, 1.0], [1.0, -0.5]]))
    assert g == np.float32(4.0)
    assert xq.tolist() == [[-128, 32], [32, -16]]


def test_v1_ties_and_epsilon():
    """Ties go to even on both sides; the 1e-8 is added to the max: a lone
    2^-27 gives 128 * 2^-27 / (2^-27 + 1e-8) = 54.65 -> 55 (without the
    epsilon it would be 127, with max(g, 1e-8) it would be 95); an all-zero
    tensor gives codes 0 and g = 0."""
    import oracle
    xq, _ = oracle.quant_act_tensor(bits([[1.0, 2.5 / 128, -2.5 / 128, 3.5 / 128, -3.5 / 128]]))
    assert xq.tolist() == [[127, 2, -2, 4, -4]]
    fr = Fraction(128) * Fraction(2) ** -27 / Fraction(float(np.float32(2.0 ** -27) + np.float32(1e-8)))
    assert abs(float(fr) - 54.65) < 0.01
    xq, _ = oracle.quant_act_tensor(bits([[2.0 ** -27, 0.0]]))
    assert xq.tolist() == [[55, 0]]
    xq, g = oracle.quant_act_tensor(np.zeros((3, 5), np.uint16))
    assert g == 0.0 and not xq.any()


def test_v1_dequant_and_contraction():
    """y = acc * gamma * g / 2^7: 64 * 0.5 * 2 / 128 = 0.5 and -3 * 0.5 * 2 /
    128 = -0.0234375, both exact; the contraction of codes that include -128
    equals a plain integer product (brute force)."""
    import oracle
    y = oracle.dequant_tensor(np.array([[64, -3]], np.int32), 0.5, 2.0)
    assert y.tolist() == [[0.5, -0.0234375]]
    rng = np.random.default_rng(5)
    xq = rng.integers(-128, 128, size=(3, 37)).astype(np.int8)
    xq[0, :] = -128
    q = rng.integers(-1, 2, size=(4, 37)).astype(np.int8)
    q[1, :] = -1
    acc = oracle.contract_q128(xq, q)
    ref = [[sum(int(a) * int(b) for a, b in zip(xr, qr)) for qr in q] for xr in xq]
    assert acc.tolist() == ref
    assert acc[0, 1] == 128 * 37


def test_v2_f16_encoding_matches_numpy():
    """binary16 rounding against numpy's float32 -> float16 conversion on a
    log-spread sweep, exact ties (normal and subnormal) and the range ends;
    decoding against numpy on every non-NaN bit pattern."""
    import oracle
    rng = np.random.default_rng(11)
    v = (rng.choice([-1.0, 1.0], 3000) * 2.0 ** rng.uniform(-30, 17, 3000)).astype(np.float32)
    special = [0.0, -0.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24, 1.5 * 2 ** -24, 2 ** -25, 2.5 * 2 ** -24,
               2 ** -14, 2 ** -14 - 2 ** -25, 65504, 65519, 65520, 7e4, -65520, 6.1e-5, 1e-9, 0.1, 0.85]
    v = np.concatenate([v, np.array(special, np.float32)])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16_bits(v), ref)
    allbits = np.arange(65536, dtype=np.uint16)
    h = allbits.view(np.float16)
    ok = ~np.isnan(h)
    dec = oracle.f16_bits_to_f32(allbits[ok])
    assert np.array_equal(dec.view(np.uint32), h[ok].astype(np.float32).view(np.uint32))


def test_v2_row_scales_hand_values():
    """Row absmeans: 0.625 (exact); 0.1 -> binary32 0.1f -> binary16 1638 *
    2^-14 = 0.0999755859375 (bits 0x2E66); 0 -> 0; 3e-6 -> subnormal round(3e-6
    * 2^24) = 50 quanta (bits 50); 0.85 -> 1741 * 2^-11 (bits 0x3ACD)."""
    import oracle
    w = np.array([[1, -1, 0.5, 0], [0.1] * 4, [0] * 4, [3e-6] * 4, [0.85, -0.85, 0.85, -0.85]], np.float32)
    s16 = oracle.row_scales(w)
    assert s16.tolist() == [0x3900, 0x2E66, 0, 50, 0x3ACD]
    assert oracle.f16_bits_to_f32(s16).tolist() == [0.625, 0.0999755859375, 0.0, 50 * 2.0 ** -24, 1741 / 2048]


def test_v2_codes_follow_each_rows_scale():
    """Row 1 is 10 x row 0: each row's own scale gives both the codes
    [1, 1, 1, 0] (0.4 / 0.8501 = 0.47 -> 0), with scales 0.85009765625 and
    8.5; one scale for the matrix (4.675) would zero row 0."""
    import oracle
    w = np.array([[1, 1, 1, 0.4], [10, 10, 10, 4]], np.float32)
    s16 = oracle.row_scales(w)
    assert oracle.f16_bits_to_f32(s16).tolist() == [1741 / 2048, 8.5]
    assert oracle.ternarize_rows(w, s16).tolist() == [[1, 1, 1, 0], [1, 1, 1, 0]]


def test_v2_threshold_uses_scale_plus_epsilon():
    """With a stored scale of 0.5 the rounding tie sits at 0.5 * (0.5 +
    1e-5) = 0.250005: 0.250004 -> 0 and 0.250006 -> 1 (without the epsilon
    both would be 1)."""
    import oracle
    w = np.array([[0.250004, 0.250006, -0.250004, -0.250006]], np.float32)
    assert oracle.ternarize_rows(w, np.array([0x3800], np.uint16)).tolist() == [[0, 1, 0, -1]]


def test_v2_reduces_to_the_tensor_rules_row_by_row():
    """Row r of the variant equals the main path's ternarization and
    de-quantization with gamma = that row's stored scale."""
    import oracle
    w = synth.latent_weights(21, 7, 300)
    s16 = oracle.row_scales(w)
    q = oracle.ternarize_rows(w, s16)
    sf = oracle.f16_bits_to_f32(s16)
    for r in range(7):
        assert np.array_equal(q[r:r + 1], oracle.ternarize(w[r:r + 1], sf[r]))
    xq, amax = oracle.quant_act(synth.activations_bf16(22, 3, 300, 0.01))
    acc = oracle.contract(xq, q)
    y = oracle.dequant_rows(acc, s16, amax)
    for j in range(7):
        assert np.array_equal(y[:, j:j + 1], oracle.dequant(acc[:, j:j + 1], sf[j], amax))
    y1 = oracle.dequant_rows(np.array([[127]], np.int32), np.array([0x3800], np.uint16), np.array([2.0], np.float32))
    assert y1.tolist() == [[1.0]]


def test_v3_sign_with_zero_as_plus_one():
    import oracle
    w = np.array([[-0.0, 0.0, -1e-30, 3.0, -2.0, 1e-45, -1e-45]], np.float32)
    assert oracle.binarize(w).tolist() == [[1, 1, -1, 1, -1, 1, -1]]


def test_v3_forward_hand_values():
    """x = [1, 0.5, -0.25]: a' = 1, codes [127, 64, -32] (63.5 -> 64, -31.75 ->
    -32); signs [1, -1, -1] and [1, 1, 1] give acc 95 and 159; with s = 0.25,
    y = acc * 0.25 / 127."""
    import oracle
    r = oracle.forward_binary(bits([[1.0, 0.5, -0.25]]), np.array([[0.3, -0.2, -0.1], [1, 1, 1]], np.float32), 0.25)
    assert r["xq"].tolist() == [[127, 64, -32]]
    assert r["acc"].tolist() == [[95, 159]]
    assert r["y"][0, 0] == f32_nearest(Fraction(95, 4 * 127))
    assert r["y"][0, 1] == f32_nearest(Fraction(159, 4 * 127))

"""The identities the fused decode prologue (gemv.hip: code_bits,
chunk_absmax) uses to form the per-token int8 codes with fewer operations,
checked exhaustively over bf16 inputs in IEEE fp32 on the CPU.

"BitNet b1.58 in Production: 1-Bit LLMs and Energy Benchmarks", section
"The Mathematical Mechanism", item 2: code = RoundClip(x * 127 / a', -127,
127), a' = max |x| of the token (floored at 1e-8), round to nearest.  The
kernel forms the scale s = fl(127 / a') once and then
  * rounds by adding 1.5 * 2^23 to fl(x * s) and keeping the low byte of the
    sum's bit pattern, without a clamp;
  * takes max |x| as an unsigned maximum over bf16 bit patterns with the
    sign bit cleared.
Both are claimed exact for every finite input the token can hold.  These
tests compare them with the definition written out (rint with ties to even,
then the clamp) on every finite bf16 value and a spread of a'.
"""
import numpy as np

MAGIC = np.float32(12582912.0)  # 1.5 * 2^23


def all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    keep = np.isfinite(x)
    return bits[keep].astype(np.uint16), x[keep]


def code_by_definition(v):
    # RoundClip: nearest integer, ties to even (np.rint), then clamp
    return np.clip(np.rint(v), -127, 127).astype(np.int8)


def code_by_low_byte(v):
    s = (v + MAGIC).astype(np.float32)  # one fp32 rounding, ties to even
    return (s.view(np.uint32) & 0xFF).astype(np.uint8).view(np.int8)


def amax_values():
    _, x = all_finite_bf16()
    pos = np.unique(np.abs(x[x != 0]))
    rng = np.random.default_rng(7)
    picks = list(rng.choice(pos, 600, replace=False))
    # the floor, the extremes, and values around the powers of two
    picks += [np.float32(1e-8), pos[0], pos[-1], np.float32(1.0), np.float32(127.0), np.float32(3.0)]
    for e in (-30, -8, -1, 0, 1, 7, 20, 100):
        p = np.float32(2.0 ** e)
        picks += [p, np.nextafter(p, np.float32(0)), np.nextafter(p, np.float32(np.inf))]
    return np.array(picks, dtype=np.float32)


def test_low_byte_rounding_equals_roundclip():
    _, x = all_finite_bf16()
    checked = 0
    for amax in amax_values():
        a = max(np.float32(amax), np.float32(1e-8))  # a' = max(max|x|, 1e-8), as the method floors it
        s = np.float32(127.0) / np.float32(a)  # IEEE fp32 divide
        xs = x[np.abs(x) <= amax]  # the token's values: |x| <= max|x|
        v = (xs * s).astype(np.float32)  # fl(x * s)
        assert np.abs(v).max(initial=0) < 127.5  # so the clamp never binds
        got = code_by_low_byte(v)
        want = code_by_definition(v)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (a, xs[bad[:5]], got[bad[:5]], want[bad[:5]])
        checked += xs.size
    assert checked > 10_000_000


def test_low_byte_rounding_on_ties():
    # exact halves are rounded to even, as rint does
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 125.5], dtype=np.float32)
    assert list(code_by_low_byte(v)) == [0, 2, 2, 0, -2, -2, 126, -126, 126]
    assert list(code_by_low_byte(v)) == list(code_by_definition(v))


def test_magnitude_order_of_sign_cleared_bf16_patterns():
    bits, x = all_finite_bf16()
    mag_bits = bits & np.uint16(0x7FFF)
    order = np.argsort(mag_bits, kind="stable")
    assert np.all(np.diff(np.abs(x[order])) >= 0)
    # so the maximum pattern is the pattern of the maximum magnitude, token by token
    rng = np.random.default_rng(3)
    for _ in range(200):
        idx = rng.integers(0, bits.size, size=int(rng.integers(1, 64)))
        assert np.abs(x[idx]).max() == (mag_bits[idx].max().astype(np.uint32) << 16).view(np.float32)

"""Pins for the oracle's E4M3 decode and encode (CPU only).

The encoder is checked against an independent brute-force search over the
254 finite E4M3 values (exact rational distances for the special points,
fp64 distances for random samples), against hand-derived encodings in
tests/golden/e4m3_encode_unit_scale.txt, and against the format's closed
forms. The format: "Kernel-Level Optimisations for LLM Inference and
Training", section "Quantisation kernels" (E4M3: four exponent bits, three
mantissa bits), in the variant whose largest finite value is 448.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from conftest import parse_value, read_golden
from oracle import e4m3_decode, e4m3_encode, e4m3_value_table


def _hand_value(code):
    """Positive code -> exact value, written independently of the oracle:
    (8 + m) * 2^(E - 10) for E > 0, m * 2^-9 for E = 0."""
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return Fraction(m, 512)
    return Fraction(8 + m) * Fraction(2) ** (e - 10)


HAND = [_hand_value(c) for c in range(0x7F)]  # 0x7F is NaN


def brute_encode(v):
    """Nearest E4M3 code by exhaustive search with exact distances; ties to
    the even code; |v| > 448 saturates; sign bit copied from v."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = min(Fraction(abs(v)), Fraction(448))
    best, best_d = None, None
    for code, val in enumerate(HAND):
        d = abs(a - val)
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return sign | best


def brute_encode_f64(v):
    """Vectorised nearest search with fp64 distances (exact near the
    winning candidates for fp32 inputs); ties between neighbours go to the
    even code."""
    v = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v).astype(np.float64), 448.0)
    cand = np.array([float(x) for x in HAND])
    out = np.empty(v.shape, dtype=np.uint8)
    for i0 in range(0, v.size, 100_000):
        aa = a[i0:i0 + 100_000]
        d = np.abs(aa[:, None] - cand[None, :])
        i = d.argmin(axis=1)
        j = np.minimum(i + 1, len(cand) - 1)
        r = np.arange(len(aa))
        tie = (d[r, j] == d[r, i]) & (j != i)
        pick = np.where(tie & (i % 2 == 1), j, i)
        out[i0:i0 + 100_000] = pick
    return out | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def test_decode_table_closed_forms():
    t = e4m3_value_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0x3F] == 1.875
    assert t[0x00] == 0.0 and math.copysign(1, t[0x80]) < 0
    # Independent formula agrees on every finite positive code.
    for c in range(0x7F):
        assert Fraction(t[c]) == HAND[c]
        assert t[c | 0x80] == -t[c]
    # Positive codes are strictly increasing in value.
    assert np.all(np.diff(t[:0x7F]) > 0)


def test_decode_encode_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_encode_golden_hand_derived():
    rows = read_golden("e4m3_encode_unit_scale.txt")
    assert len(rows) >= 20
    for row in rows:
        v = np.float32(parse_value(row[0]))
        want = int(row[1], 16)
        got = int(e4m3_encode(np.array([v]))[0])
        assert got == want, (row, hex(got))
        assert brute_encode(float(v)) == want, row


def _special_points():
    pos = [float(x) for x in HAND]
    pts = list(pos)
    mids = [(pos[i] + pos[i + 1]) / 2 for i in range(len(pos) - 1)] + [464.0]
    pts += mids
    f = np.array(mids, dtype=np.float32)
    pts += list(np.nextafter(f, np.float32(np.inf)).astype(float))
    pts += list(np.nextafter(f, np.float32(0)).astype(float))
    pts += [447.99997, 448.00003, 463.99997, 464.00003, 1e30, 2.0 ** -149, 2.0 ** -126]
    allp = pts + [-p for p in pts] + [0.0, -0.0]
    return np.array(allp, dtype=np.float32)


def test_encode_matches_bruteforce_on_grid_midpoints_and_neighbours():
    pts = _special_points()
    got = e4m3_encode(pts)
    for v, g in zip(pts, got):
        assert int(g) == brute_encode(float(v)), (float(v), hex(int(g)))


def test_encode_matches_bruteforce_random():
    rng = np.random.default_rng(7)
    uni = rng.uniform(-464, 464, size=1_000_000).astype(np.float32)
    # Random bit patterns with magnitude up to 464: uniform over exponents, so
    # the subnormal and small-normal ranges are well covered.
    bits = rng.integers(0, 0x43E80001, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    bits |= (rng.integers(0, 2, size=bits.size, dtype=np.uint32) << np.uint32(31))
    logu = bits.view(np.float32)
    for v in (uni, logu):
        assert np.array_equal(e4m3_encode(v), brute_encode_f64(v))


def test_encode_saturates_and_keeps_sign():
    v = np.array([448.0, 500.0, 1e38, -1e38, -448.0, 3.4e38], dtype=np.float32)
    assert list(e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7E]
    tiny = np.array([-1e-30, -2.0 ** -11, 1e-30, -0.0, 0.0], dtype=np.float32)
    assert list(e4m3_encode(tiny)) == [0x80, 0x80, 0x00, 0x80, 0x00]


def test_mutant_tie_rule_is_caught(monkeypatch):
    """A planted mistake in the oracle (ties away from zero instead of to even)
    must fail the hand-derived pins."""
    import oracle.fp8bs_oracle as o

    real_rint = np.rint

    def away(x):
        return np.where(np.abs(x - np.trunc(x)) == 0.5, np.trunc(x) + np.sign(x), real_rint(x))

    monkeypatch.setattr(o.np, "rint", away)
    try:
        bad = int(o.e4m3_encode(np.array([np.float32(2.125)]))[0])
    finally:
        monkeypatch.setattr(o.np, "rint", real_rint)
    assert bad != 0x40


@pytest.mark.slow
def test_encode_matches_bruteforce_random_large():
    rng = np.random.default_rng(8)
    bits = rng.integers(0, 0x43E80001, size=10_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    assert np.array_equal(e4m3_encode(v), brute_encode_f64(v))

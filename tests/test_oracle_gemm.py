"""Pins for the oracle's fp64 GEMM and the tolerance check (CPU only).

Y[m][n] = sum over 128-wide K blocks of (exact block dot product of decoded
codes) x (activation scale x weight scale), the weight scale taken from the
128 x 128 block holding (n, k) ("A 23% faster GPU kernel, and a model that
did not move", section "Why this shape is hard").
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import (e4m3_decode, gemm_fused_ref, gemm_ref, quantize_act_ref,
                    quantize_weight_ref, tolerance_report, unquantized_gemm_ref,
                    within_tolerance)
from workloads import WORKLOADS, bf16_from_f32, f32_from_bf16, step_order


def _rand_codes(rng, shape):
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8)
    c |= (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)
    return c


def _rand_scales(rng, shape):
    return (rng.uniform(0.5, 2.0, size=shape) * 2.0 ** rng.integers(-12, 4, size=shape)).astype(np.float32)


def _exact(xq, xs, wq, ws):
    """The definition in exact rational arithmetic."""
    m, k = xq.shape
    n = wq.shape[0]
    xd = [[Fraction(float(v)) for v in row] for row in e4m3_decode(xq)]
    wd = [[Fraction(float(v)) for v in row] for row in e4m3_decode(wq)]
    out = [[Fraction(0)] * n for _ in range(m)]
    blocks = []
    for i in range(m):
        for j in range(n):
            tot = Fraction(0)
            per = []
            for kb in range(k // 128):
                p = sum(xd[i][t] * wd[j][t] for t in range(128 * kb, 128 * kb + 128))
                term = p * Fraction(float(xs[i, kb])) * Fraction(float(ws[j // 128, kb]))
                per.append(term)
                tot += term
            out[i][j] = tot
            blocks.append(per)
    return out, blocks


@pytest.mark.parametrize("m,n,k", [(1, 128, 128), (2, 256, 256), (1, 256, 384)])
def test_gemm_matches_exact_rational(m, n, k):
    rng = np.random.default_rng(1000 + m + n + k)
    xq, wq = _rand_codes(rng, (m, k)), _rand_codes(rng, (n, k))
    xs, ws = _rand_scales(rng, (m, k // 128)), _rand_scales(rng, (n // 128, k // 128))
    y = gemm_ref(xq, xs, wq, ws)
    exact, blocks = _exact(xq, xs, wq, ws)
    for i in range(m):
        for j in range(n):
            per = blocks[i * n + j]
            if k == 128:
                # one block: the product of an exact sum and an exact scale
                # product, rounded once
                assert y[i, j] == float(exact[i][j])
            else:
                bound = 2.0 ** -52 * sum(abs(float(t)) for t in per) * len(per)
                assert abs(y[i, j] - float(exact[i][j])) <= bound


def test_gemm_one_hot_weight_closed_form():
    """W[n][k] = c at k == n, else 0: the diagonal blocks have amax c, their
    codes are 448 there, the off-diagonal blocks have scale 0; so
    Y[m][n] = xs[m, n/128] * ws[n/128, n/128] * dec(xq[m, n]) * 448."""
    m, n, k = 3, 256, 256
    w = np.zeros((n, k), dtype=np.float32)
    w[np.arange(n), np.arange(n)] = np.float32(0.37)
    wb = bf16_from_f32(w)
    wq, ws = quantize_weight_ref(wb)
    assert ws[0, 1] == 0 and ws[1, 0] == 0
    x = bf16_from_f32(np.random.default_rng(9).standard_normal((m, k)).astype(np.float32))
    xq, xs = quantize_act_ref(x)
    y = gemm_ref(xq, xs, wq, ws)
    for i in range(m):
        for j in range(n):
            want = (float(xs[i, j // 128]) * float(ws[j // 128, j // 128])
                    * e4m3_decode(xq[i, j]) * 448.0)
            assert y[i, j] == want


def test_gemm_constant_weight_closed_form():
    """W = c everywhere: every weight code is 448, so
    Y[m][n] = sum_kb xs[m,kb] * ws * 448 * (sum of the block's decoded codes)."""
    m, n, k = 2, 128, 384
    wb = bf16_from_f32(np.full((n, k), 0.125, dtype=np.float32))
    wq, ws = quantize_weight_ref(wb)
    assert np.all(wq == 0x7E)
    x = bf16_from_f32(np.random.default_rng(10).standard_normal((m, k)).astype(np.float32))
    xq, xs = quantize_act_ref(x)
    y = gemm_ref(xq, xs, wq, ws)
    for i in range(m):
        want = 0.0
        for kb in range(3):
            blk = e4m3_decode(xq[i, 128 * kb:128 * kb + 128]).sum()
            want += float(xs[i, kb]) * float(ws[0, kb]) * 448.0 * blk
        assert np.allclose(y[i], want, rtol=1e-15, atol=0)


def test_gemm_chunking_does_not_change_results():
    rng = np.random.default_rng(11)
    xq, wq = _rand_codes(rng, (4, 512)), _rand_codes(rng, (640, 512))
    xs, ws = _rand_scales(rng, (4, 4)), _rand_scales(rng, (5, 4))
    assert np.array_equal(gemm_ref(xq, xs, wq, ws, n_chunk=128), gemm_ref(xq, xs, wq, ws))


def test_quantized_gemm_close_to_unquantized_on_tiny_workload():
    """Sanity of scale direction and indexing on the tiny workload: the
    quantization error of the FP8 result against the plain bf16 product is a
    few percent of rms, not O(1)."""
    wl = WORKLOADS["tiny"]
    w, x = wl.weight(), wl.act()
    wq, ws = quantize_weight_ref(w)
    ref = gemm_fused_ref(x, wq, ws)
    plain = unquantized_gemm_ref(x, w)
    rel = np.sqrt(np.mean((ref - plain) ** 2) / np.mean(plain ** 2))
    assert rel < 0.08, rel


def test_tolerance_check_accepts_rounding_and_rejects_planted_errors():
    rng = np.random.default_rng(12)
    ref = rng.standard_normal((8, 512)) * 3
    ok = bf16_from_f32(ref.astype(np.float32))
    assert within_tolerance(ok, ref)
    bad = bf16_from_f32((ref * (1 + 2.0 ** -5)).astype(np.float32))
    assert not within_tolerance(bad, ref)
    sign = ref.copy()
    sign[3, 7] *= -1
    assert not within_tolerance(bf16_from_f32(sign.astype(np.float32)), ref)
    nan = ok.copy()
    nan[0, 0] = 0x7FC0
    assert tolerance_report(nan, ref)["finite"] is False


def test_bf16_generator_is_round_to_nearest_even():
    """Pin the input generator's fp32 -> bf16 rounding against the exact
    nearest bf16 (ties to even mantissa) on 10^6 values."""
    rng = np.random.default_rng(13)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    b = bf16_from_f32(f)
    lo = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    hi = lo + np.uint16(1)
    vlo = f32_from_bf16(lo).astype(np.float64)
    vhi = f32_from_bf16(hi).astype(np.float64)
    x = f.astype(np.float64)
    dlo, dhi = np.abs(x - vlo), np.abs(x - vhi)
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    assert np.array_equal(b, want)
    # ties: exactly half-way patterns
    t = np.array([0x3F808000, 0x3F818000, 0xBF808000], dtype=np.uint32).view(np.float32)
    assert list(bf16_from_f32(t)) == [0x3F80, 0x3F82, 0xBF80]


def test_step_mix_order_is_stable():
    from collections import Counter
    c = Counter(step_order())
    assert c == {"square": 60, "mlp_up": 59, "mlp_down": 63, "vocab": 74}


def test_workload_generators_are_seeded_and_shaped():
    wl = WORKLOADS["tiny"]
    assert np.array_equal(wl.weight(), wl.weight())
    x = wl.act()
    assert x.shape == (8, 1024) and x.dtype == np.uint16
    xf = f32_from_bf16(x)
    big = np.abs(xf).max(axis=0) > 15  # the 4 outlier columns (x20)
    assert big.sum() == 4
    assert np.array_equal(WORKLOADS["square"].act(1), WORKLOADS["square"].act()[:1])
    assert WORKLOADS["mlp_up"].n_outlier == 51 and WORKLOADS["mlp_down"].n_outlier == 174
    assert WORKLOADS["square"].algorithmic_bytes(8) == 26_384_640
    assert WORKLOADS["vocab"].algorithmic_bytes(16) == 1_279_818_880

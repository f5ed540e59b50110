"""Pins for the oracle's block quantizers (CPU only).

Scale = fl32(amax / 448), code = encode(fl32(x / scale)), one scale per
128 x 128 weight block ("A 23% faster GPU kernel, and a model that did not
move", section "Why this shape is hard"; "The profiler said the kernel ran
zero times", section "The output layer, which did run") and, as the reading
taken for the activations, one per row per 128 columns.
"""
import numpy as np

from conftest import read_golden
from oracle import (bf16_bits_to_f32, e4m3_decode, e4m3_encode, quantize_act_ref,
                    quantize_blocks, quantize_weight_ref)
from workloads import bf16_from_f32, f32_from_bf16


def _bf16(vals):
    return bf16_from_f32(np.asarray(vals, dtype=np.float32))


def test_pow2_block_amax_one_hand_derived():
    """tests/golden/quant_pow2_amax1.txt: codes of 2^-j in a block with amax 1,
    and scales for several amax values, all derived by hand."""
    rows = read_golden("quant_pow2_amax1.txt")
    scales = [r for r in rows if r[0] == "scale"]
    codes = [r for r in rows if r[0] != "scale"]
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, 0] = 1.0
    for j, _ in codes:
        x[0, 1 + int(j)] = 2.0 ** -int(j)
    q, s = quantize_act_ref(_bf16(x))
    assert s.view(np.uint32)[0, 0] == 0x3B124925
    for j, want in codes:
        assert q[0, 1 + int(j)] == int(want, 16), (j, hex(q[0, 1 + int(j)]))
    assert q[0, 0] == 0x7E
    for _, amax, bits in scales:
        xx = np.zeros((1, 128), dtype=np.float32)
        xx[0, 5] = float(amax)
        _, ss = quantize_act_ref(_bf16(xx))
        assert ss.view(np.uint32)[0, 0] == int(bits, 16), (amax, hex(ss.view(np.uint32)[0, 0]))


def test_inverse_scale_reading_differs_at_pin():
    """Multiplying by fl32(448 / amax) instead of dividing by the stored scale
    would give the exact tie 3.5 * 2^-9 at x = 2^-16 in an amax-1 block, hence
    code 0x04; the pin above requires 0x03."""
    inv = np.float32(448.0) / np.float32(1.0)
    via_inv = e4m3_encode(np.array([np.float32(2.0 ** -16) * inv]))[0]
    s = np.float32(1.0) / np.float32(448.0)
    via_div = e4m3_encode(np.array([np.float32(2.0 ** -16) / s]))[0]
    assert via_div == 0x03 and via_inv == 0x04


def test_weight_block_layout_closed_form():
    """A 256 x 384 weight whose block (i, j) holds e4m3 grid values times
    2^(i + 2j) and whose amax is 448 * 2^(i + 2j): each scale is exactly
    2^(i + 2j), stored at [i][j], and the codes are the grid values' codes."""
    rng = np.random.default_rng(3)
    grid_codes = rng.integers(0, 0x7E, size=(256, 384)).astype(np.uint8)
    grid_codes |= (rng.integers(0, 2, size=grid_codes.shape, dtype=np.uint8) << 7)
    vals = e4m3_decode(grid_codes)
    for i in range(2):
        for j in range(3):
            blk = (slice(128 * i, 128 * i + 128), slice(128 * j, 128 * j + 128))
            vals[blk] *= 2.0 ** (i + 2 * j)
            grid_codes[128 * i + 7, 128 * j + 9] = 0x7E
            vals[128 * i + 7, 128 * j + 9] = 448.0 * 2.0 ** (i + 2 * j)
    w = _bf16(vals)  # grid values times powers of two are exact in bf16
    assert np.array_equal(f32_from_bf16(w).astype(np.float64), vals)
    q, s = quantize_weight_ref(w)
    assert s.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            assert s[i, j] == np.float32(2.0 ** (i + 2 * j))
    assert np.array_equal(q, grid_codes)


def test_zero_block_and_signed_zero():
    x = np.zeros((2, 256), dtype=np.float32)
    x[0, :128:2] = -0.0
    x[1, 128] = 3.0
    q, s = quantize_act_ref(_bf16(x))
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert np.all(q[0, :128:2] == 0x80) and np.all(q[0, 1:128:2] == 0x00)
    assert q[1, 128] == 0x7E and np.all(q[1, 129:] == 0)


def test_activation_rows_are_independent():
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((4, 384)).astype(np.float32))
    q, s = quantize_act_ref(x)
    for r in range(4):
        qr, sr = quantize_act_ref(x[r:r + 1])
        assert np.array_equal(qr[0], q[r]) and np.array_equal(sr[0], s[r])
    assert s.shape == (4, 3)


def test_every_nonzero_block_reaches_448():
    """The element of largest magnitude always encodes to +-448: fl32(amax/s)
    is within one fp32 ulp of 448, and with the smallest possible (subnormal)
    scales still within 1/256 of it, nearer to 448 than to 416."""
    rng = np.random.default_rng(5)
    exps = rng.uniform(-30, 30, size=20000)
    amax = (10.0 ** exps).astype(np.float32)
    # the bf16 rounding keeps amax a bf16 value, as it is for real inputs
    amax = f32_from_bf16(bf16_from_f32(amax))
    tiny = f32_from_bf16(np.arange(1, 4096, dtype=np.uint16))  # bf16 subnormals and up
    amax = np.concatenate([amax, tiny])
    x = np.zeros((amax.size, 128), dtype=np.float32)
    x[:, 0] = amax
    x[:, 1] = -amax * np.float32(0.5)
    x[:, 2] = amax * np.float32(0.999)
    q, s = quantize_blocks(x, 1, 128)
    assert np.all(q[:, 0] == 0x7E)
    assert np.all(s[:, 0] > 0)


def test_half_ulp_invariant_on_random_blocks():
    """dequantize(quantize(x)) is within half an E4M3 ulp of the fp32 quotient
    (equality only on ties, then with an even code), and within
    s * half_ulp + 2^-24 |x| of x itself."""
    rng = np.random.default_rng(6)
    w = rng.standard_normal((256, 512)).astype(np.float32) * np.float32(0.02)
    w[:, rng.choice(512, 5, replace=False)] *= 20
    w[:3, :7] = 0
    wb = _bf16(w)
    x = bf16_bits_to_f32(wb)
    for br, bc, qfun in ((128, 128, quantize_weight_ref), (1, 128, quantize_act_ref)):
        q, s = qfun(wb)
        sf = np.repeat(np.repeat(s, br, axis=0), bc, axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            quo = np.where(sf > 0, x / sf, 0).astype(np.float32).astype(np.float64)
        dec = e4m3_decode(q)
        a = np.abs(quo)
        binade = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        ulp = 2.0 ** (np.maximum(binade, -6) - 3)
        err = np.abs(quo - dec)
        assert np.all(err <= ulp / 2)
        tie = err == ulp / 2
        assert np.all((q[tie] & 1) == 0)
        xerr = np.abs(x.astype(np.float64) - sf * dec)
        assert np.all(xerr <= sf * ulp / 2 + 2.0 ** -24 * np.abs(x))

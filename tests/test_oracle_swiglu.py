"""Pins for the oracle's MLP epilogue (CPU only): the one-step fp64 -> bf16
rounding, silu, the gate/up layout of SwiGLU and the re-quantization of h.

SwiGLU is fused onto the up/gate projection ("Kernel-Level Optimisations for
LLM Inference and Training", section "Scheduling decides the shapes your
kernels see", its paragraph on fusion); its definition is the published
gated unit h = silu(gate) * up, silu(g) = g * sigmoid(g) (Shazeer, "GLU
Variants Improve Transformer", 2020).
"""
import math

import numpy as np
import scipy.special

from oracle import (bf16_bits_from_f64, bf16_bits_to_f32, e4m3_decode, quantize_act_ref,
                    silu_ref, swiglu_quant_ref, swiglu_ref)
from workloads import bf16_from_f32


def _finite_positive_bf16():
    """Every finite positive bf16 value (patterns 0x0001 .. 0x7F7F), ascending."""
    bits = np.arange(1, 0x7F80, dtype=np.uint16)
    return bits, bf16_bits_to_f32(bits).astype(np.float64)


def test_bf16_rounding_keeps_every_bf16_value():
    bits, vals = _finite_positive_bf16()
    assert np.array_equal(bf16_bits_from_f64(vals), bits)
    assert np.array_equal(bf16_bits_from_f64(-vals), bits | np.uint16(0x8000))
    z = bf16_bits_from_f64(np.array([0.0, -0.0]))
    assert z.tolist() == [0x0000, 0x8000]


def test_bf16_rounding_midpoints_go_to_even():
    """Exact midpoints between neighbouring bf16 values (subnormal, normal and
    across each power of two) round to the even pattern; a hair either side
    rounds to the nearer value."""
    bits, vals = _finite_positive_bf16()
    lo, hi = vals[:-1], vals[1:]
    mid = (lo + hi) / 2                                    # exact in fp64
    want = np.where(bits[:-1] % 2 == 0, bits[:-1], bits[1:])
    assert np.array_equal(bf16_bits_from_f64(mid), want)
    eps = (hi - lo) * 2.0 ** -20
    assert np.array_equal(bf16_bits_from_f64(mid - eps), bits[:-1])
    assert np.array_equal(bf16_bits_from_f64(mid + eps), bits[1:])


def test_bf16_rounding_overflow_and_underflow():
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127                  # 0x7F7F
    half_ulp = 2.0 ** 119
    got = bf16_bits_from_f64(np.array([top + half_ulp * 0.999, top + half_ulp, 1e39,
                                       2.0 ** -134, 2.0 ** -134 * 1.0001, -(2.0 ** -140)]))
    # the tie at top + half ulp goes to the even neighbour 2^128, i.e. infinity
    assert got.tolist() == [0x7F7F, 0x7F80, 0x7F80, 0x0000, 0x0001, 0x8000]


def test_bf16_rounding_matches_independent_fp32_rounding():
    """For fp32 inputs, one rounding from the fp64 value equals the input
    generator's own fp32 -> bf16 rounding (an independent integer routine)."""
    rng = np.random.default_rng(5)
    f = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),
        rng.integers(0, 0x7F7FFFFF, 200_000, dtype=np.uint32).view(np.float32),
    ])
    assert np.array_equal(bf16_bits_from_f64(f.astype(np.float64)), bf16_from_f32(f))


def test_silu_closed_forms():
    """sigmoid(ln k) = k / (k + 1), so silu(ln k) = ln(k) k / (k + 1);
    silu(0) = 0; silu(-g) = silu(g) - g; silu(g) -> g for large g and to a
    zero of g's sign for very negative g."""
    for k in (3.0, 1.0 / 3.0, 7.0, 0.25, 99.0):
        g = math.log(k)
        assert abs(silu_ref(np.array([g]))[0] - g * k / (k + 1)) <= 4e-16 * abs(g) + 1e-300
    assert silu_ref(np.array([0.0]))[0] == 0.0
    g = np.random.default_rng(6).standard_normal(10_000) * 6
    assert np.allclose(silu_ref(-g), silu_ref(g) - g, rtol=0, atol=4e-15 * (1 + np.abs(g)).max())
    assert silu_ref(np.array([40.0]))[0] == 40.0
    far = silu_ref(np.array([-800.0]))[0]
    assert far == 0.0 and math.copysign(1.0, far) < 0


def test_silu_matches_library_sigmoid():
    g = np.random.default_rng(7).standard_normal(100_000) * 8
    ref = g * scipy.special.expit(g)
    assert np.allclose(silu_ref(g), ref, rtol=1e-14, atol=1e-300)


def _y(gate, up):
    return np.concatenate([bf16_from_f32(np.asarray(gate, np.float32)),
                           bf16_from_f32(np.asarray(up, np.float32))], axis=1)


def test_swiglu_gate_first_then_up():
    """gate = 2, up = 3 gives 3 silu(2) = 6 sigmoid(2). Swapped halves would
    give 2 silu(3); dropping silu's factor g would give 3 sigmoid(2)."""
    y = _y(np.full((1, 128), 2.0), np.full((1, 128), 3.0))
    h = swiglu_ref(y)
    want = 6.0 * scipy.special.expit(2.0)
    assert np.allclose(h, want, rtol=1e-15)
    assert abs(want - 2.0 * 3.0 * scipy.special.expit(3.0)) > 0.1
    assert abs(want - 3.0 * scipy.special.expit(2.0)) > 1.0


def test_swiglu_columns_pair_up_one_to_one():
    """One-hot rows: only column j of the gate and column j of the up half
    are nonzero, so only h[:, j] is nonzero (sigmoid(1) = 1 / (1 + 1/e))."""
    m, inter = 3, 256
    gate = np.zeros((m, inter), np.float32)
    up = np.zeros((m, inter), np.float32)
    cols = [5, 130, 255]
    for r, j in enumerate(cols):
        gate[r, j] = 1.0
        up[r, j] = 1.0
    h = swiglu_ref(_y(gate, up))
    for r, j in enumerate(cols):
        row = h[r].copy()
        assert abs(row[j] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
        row[j] = 0.0
        assert not row.any()


def test_swiglu_quant_is_bf16_then_activation_cast():
    """The re-quantized h has one scale per row per 128 columns, every
    nonzero block holds a +-448 code, and each dequantized value is within
    half an E4M3 step of the bf16 h."""
    rng = np.random.default_rng(8)
    m, inter = 4, 512
    y = bf16_from_f32((rng.standard_normal((m, 2 * inter)) * 3).astype(np.float32))
    hb, codes, scales = swiglu_quant_ref(y)
    assert hb.shape == (m, inter) and codes.shape == (m, inter) and scales.shape == (m, 4)
    h = bf16_bits_to_f32(hb).astype(np.float64)
    assert np.array_equal(hb, bf16_bits_from_f64(swiglu_ref(y)))
    c2, s2 = quantize_act_ref(hb)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    blocks = codes.reshape(m, 4, 128)
    assert np.all(((blocks & 0x7F) == 0x7E).any(axis=2))
    deq = e4m3_decode(codes).reshape(m, 4, 128) * scales.astype(np.float64)[:, :, None]
    q = np.abs(h.reshape(m, 4, 128)) / scales.astype(np.float64)[:, :, None]
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(q, 2.0 ** -10))), -6) - 3)
    err = np.abs(deq - h.reshape(m, 4, 128))
    assert np.all(err <= 0.5 * step * scales[:, :, None] * (1 + 2.0 ** -20) + 1e-30)

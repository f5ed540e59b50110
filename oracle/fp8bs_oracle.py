"""Plain CPU oracle for the FP8 (E4M3) 128x128 block-scaled decode GEMM.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
test suite, the smoke check and the bench's CPU-baseline leg may import it.
It shares no code with the HIP path (no kernels, headers, tables or helpers)
and imports nothing from it.

What it computes, and where the pages say so:

* FP8 E4M3 element format -- four exponent bits, three mantissa bits
  ("Kernel-Level Optimisations for LLM Inference and Training", section
  "Quantisation kernels"). The variant is the one whose largest finite value
  is 448: exponent bias 7, subnormals at exponent field 0, no infinities, and
  NaN only at exponent and mantissa fields all ones (codes 0x7F, 0xFF).
* One fp32 scale per 128 x 128 block of the weight ("A 23% faster GPU
  kernel, and a model that did not move", section "Why this shape is hard";
  "The profiler said the kernel ran zero times", section "The output layer,
  which did run", where the output layer is converted the same way).
* Inputs of the multiply cast to FP8 on every call ("The profiler said the
  kernel ran zero times", section "What the trace showed": the cast shows up
  as its own share of the step). The pages do not give the activation
  granularity; the reading used here is one scale per row per 128 columns,
  aligned with the weight's K blocks.
* A block's scale is its largest magnitude divided by 448, computed as an
  IEEE fp32 division; each element is divided (fp32, round to nearest even)
  by that scale and then rounded to the nearest E4M3 value with ties to the
  even mantissa, saturating at +-448 and keeping the sign of zero. An all-zero
  block gets scale 0 and codes that keep the sign of each zero.
* The GEMM Y[m][n] = sum over K blocks of (block dot product of the decoded
  codes) x (activation scale x weight scale), evaluated in fp64. Each block dot
  product is exact in fp64 in any summation order (every product is a multiple
  of 2^-18 below 2^18 in magnitude, so 128 of them need at most 43 significant
  bits), and the product of two fp32 scales is exact in fp64; only the running
  sum over blocks rounds.

The reference result is kept in fp64 and never rounded to bf16.

MLP epilogue (the step after the up/gate projection):

* SwiGLU fused onto the multiply's output, and the 1 x 128 FP8 cast of its
  result that feeds the down projection ("Kernel-Level Optimisations for LLM
  Inference and Training", section "Scheduling decides the shapes your
  kernels see", its paragraph on fusion; the cast's cost as in "The profiler
  said the kernel ran zero times", section "What the trace showed"). The
  pages name SwiGLU without defining it; the definition used is the
  published gated unit (Shazeer, "GLU Variants Improve Transformer", 2020):
  h = silu(gate) * up, silu(g) = g * sigmoid(g) = g / (1 + e^-g).
* Readings the pages leave open: the fused up/gate output holds the gate in
  its first n/2 columns and the up projection in the last n/2; gate and up
  are the GEMM's bf16 outputs; h is rounded once to bf16 (the element type
  an unfused SwiGLU step would hand on) and then cast with the activation
  rule above. Here h is evaluated in fp64 and rounded to bf16 in one step.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "E4M3_MAX",
    "BLOCK",
    "e4m3_value_table",
    "e4m3_decode",
    "e4m3_encode",
    "bf16_bits_to_f32",
    "quantize_blocks",
    "quantize_weight_ref",
    "quantize_act_ref",
    "gemm_ref",
    "gemm_fused_ref",
    "tolerance_report",
    "within_tolerance",
    "unquantized_gemm_ref",
    "bf16_bits_from_f64",
    "silu_ref",
    "swiglu_ref",
    "swiglu_quant_ref",
]

E4M3_MAX = 448.0
BLOCK = 128


# ---------------------------------------------------------------------------
# E4M3 format ("Kernel-Level Optimisations...", section "Quantisation kernels")
# ---------------------------------------------------------------------------

def e4m3_value_table() -> np.ndarray:
    """Value of every one of the 256 codes, in fp64 (NaN at 0x7F and 0xFF).

    Bit layout: sign = bit 7, exponent field E = bits 6..3, mantissa m = bits
    2..0. E = 0 encodes m * 2^-9 (subnormals, and zero); otherwise the value is
    (1 + m/8) * 2^(E - 7).
    """
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_value_table()
# Positive finite codes 0x00..0x7E have strictly increasing values.
_POS_VALUES = _TABLE[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode uint8 codes to fp64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Encode fp32 values to E4M3 codes.

    Round to nearest, ties to the even mantissa; magnitudes above 448
    saturate to 448; the sign bit of the input is kept (so negative values
    that round to zero give 0x80). Inputs are finite.

    Method: in the binade [2^e, 2^(e+1)) the E4M3 grid step is 2^(e-3), and
    below 2^-6 it is the subnormal step 2^-9. Scaling |v| by the inverse step
    (a power of two, so exact in fp64) and rounding half-to-even to an integer
    gives the nearest grid point; a result that rounds up to 2^(e+1) is the
    first value of the next binade and is still on the grid.
    """
    v = np.asarray(v, dtype=np.float32)
    sign = np.signbit(v)
    a = np.minimum(np.abs(v).astype(np.float64), E4M3_MAX)
    _, e = np.frexp(a)                       # a = f * 2^e, f in [0.5, 1)
    step_exp = np.maximum(e - 1, -6) - 3     # log2 of the grid step
    n = np.rint(np.ldexp(a, -step_exp))      # np.rint rounds half to even
    val = np.ldexp(n, step_exp)
    code = np.searchsorted(_POS_VALUES, val).astype(np.uint8)
    if not np.array_equal(_POS_VALUES[np.minimum(code, 0x7E)], val):
        raise AssertionError("e4m3_encode: rounded value not on the E4M3 grid")
    return code | np.where(sign, np.uint8(0x80), np.uint8(0))


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to fp32 values (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Block quantization ("A 23% faster GPU kernel...", section "Why this shape is
# hard"; "The profiler said the kernel ran zero times", section "The output
# layer, which did run")
# ---------------------------------------------------------------------------

def quantize_blocks(x: np.ndarray, br: int, bc: int):
    """Quantize an fp32 matrix in blocks of br rows x bc columns.

    Returns (codes uint8 of x's shape, scales fp32 [rows/br][cols/bc]).
    scale = fl32(amax / 448); code = encode(fl32(x / scale)); an all-zero block
    has scale 0 and each code keeps its element's sign.
    """
    x = np.asarray(x, dtype=np.float32)
    r, c = x.shape
    if r % br or c % bc:
        raise ValueError("shape must be a multiple of the block shape")
    blocks = x.reshape(r // br, br, c // bc, bc)
    amax = np.abs(blocks).max(axis=(1, 3))                       # fp32, exact
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)     # IEEE fp32 division
    s4 = scale[:, None, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (blocks / s4).astype(np.float32)                     # IEEE fp32 division
    zero_block = np.broadcast_to(s4 == 0, blocks.shape)
    # In an all-zero block every element is +-0: keep its sign, value 0.
    q = np.where(zero_block, blocks, q)
    codes = e4m3_encode(q).reshape(r, c)
    return codes, scale


def quantize_weight_ref(w_bf16: np.ndarray):
    """W[n][k] bf16 bits -> (codes uint8 [n][k], scales fp32 [n/128][k/128])."""
    return quantize_blocks(bf16_bits_to_f32(w_bf16), BLOCK, BLOCK)


def quantize_act_ref(x_bf16: np.ndarray):
    """X[m][k] bf16 bits -> (codes uint8 [m][k], scales fp32 [m][k/128]).

    One scale per row per 128 columns (the reading stated in the module
    docstring)."""
    return quantize_blocks(bf16_bits_to_f32(x_bf16), 1, BLOCK)


# ---------------------------------------------------------------------------
# GEMM in fp64
# ---------------------------------------------------------------------------

def gemm_ref(xq: np.ndarray, xs: np.ndarray, wq: np.ndarray, ws: np.ndarray,
             n_chunk: int = 8192) -> np.ndarray:
    """Y[m][n] in fp64 from activation codes/scales and weight codes/scales.

    For each K block kb in ascending order:
        P = sum over the block's 128 k of dec(xq[m,k]) * dec(wq[n,k])   (exact)
        acc += P * (xs[m,kb] * ws[n//128, kb])                          (fp64)
    Rows of W are processed in chunks of ``n_chunk`` to bound memory.
    """
    xq = np.asarray(xq, dtype=np.uint8)
    wq = np.asarray(wq, dtype=np.uint8)
    m, k = xq.shape
    n, k2 = wq.shape
    if k != k2 or k % BLOCK or n % BLOCK:
        raise ValueError("bad shapes")
    kb_count = k // BLOCK
    xs = np.asarray(xs, dtype=np.float32).astype(np.float64)      # [m][kb]
    ws = np.asarray(ws, dtype=np.float32).astype(np.float64)      # [n/128][kb]
    xd = e4m3_decode(xq).reshape(m, kb_count, BLOCK)
    out = np.empty((m, n), dtype=np.float64)
    n_chunk = max(BLOCK, (n_chunk // BLOCK) * BLOCK)
    for n0 in range(0, n, n_chunk):
        n1 = min(n, n0 + n_chunk)
        wd = e4m3_decode(wq[n0:n1]).reshape(n1 - n0, kb_count, BLOCK)
        wsc = np.repeat(ws[n0 // BLOCK:n1 // BLOCK], BLOCK, axis=0)  # [n1-n0][kb]
        acc = np.zeros((m, n1 - n0), dtype=np.float64)
        for kb in range(kb_count):
            p = xd[:, kb, :] @ wd[:, kb, :].T                         # exact block sums
            acc += p * (xs[:, kb][:, None] * wsc[:, kb][None, :])
        out[:, n0:n1] = acc
    return out


def gemm_fused_ref(x_bf16: np.ndarray, wq: np.ndarray, ws: np.ndarray,
                   n_chunk: int = 8192) -> np.ndarray:
    """Cast X per row per 128 columns, then the fp64 GEMM."""
    xq, xs = quantize_act_ref(x_bf16)
    return gemm_ref(xq, xs, wq, ws, n_chunk=n_chunk)


def unquantized_gemm_ref(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """X . W^T in fp64 from the bf16 operands, no quantization (used only to
    report quantization error, never for pass/fail)."""
    x = bf16_bits_to_f32(x_bf16).astype(np.float64)
    w = bf16_bits_to_f32(w_bf16).astype(np.float64)
    return x @ w.T


# ---------------------------------------------------------------------------
# Output comparison
# ---------------------------------------------------------------------------

def tolerance_report(y_bf16: np.ndarray, ref: np.ndarray,
                     rel: float = 2.0 ** -7, abs_rms: float = 1e-3,
                     rms: float | None = None) -> dict:
    """Compare bf16 GEMM output bits with the fp64 reference.

    Bound per element: |y - ref| <= rel * |ref| + abs_rms * rms(ref), where
    rms(ref) is over the whole output (or given, for sampled checks).
    """
    y = bf16_bits_to_f32(y_bf16).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(y - ref)
    bound = rel * np.abs(ref) + abs_rms * rms
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0),
                     np.where(err > 0, np.inf, 0.0))
    return {
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_ratio": float(ratio.max()) if ratio.size else 0.0,
        "n_bad": int((err > bound).sum()),
        "rms_ref": rms,
        "finite": bool(np.all(np.isfinite(y))),
    }


def within_tolerance(y_bf16: np.ndarray, ref: np.ndarray, **kw) -> bool:
    r = tolerance_report(y_bf16, ref, **kw)
    return r["finite"] and r["n_bad"] == 0


# ---------------------------------------------------------------------------
# MLP epilogue: SwiGLU and the re-quantization of its output
# ---------------------------------------------------------------------------

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_bits_from_f64(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 in one step (nearest, ties to even mantissa);
    returns uint16 bit patterns.

    bf16 keeps 8 significant bits with fp32's exponent range: a value whose
    leading bit has weight 2^e is rounded to a multiple of 2^(e-7), and values
    below 2^-126 to multiples of 2^-133 (subnormals). Magnitudes that round
    past the largest finite value become infinity; zero keeps its sign.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                      # a = f * 2^e, 0.5 <= f < 1 (e = 0 for a = 0)
    qexp = np.maximum(e.astype(np.int64) - 8, -133)
    r = np.rint(np.ldexp(a, -qexp))         # exact scaling; rint rounds ties to even
    mag = np.ldexp(r, qexp)
    mag = np.where(mag > BF16_MAX, np.inf, mag)
    out = np.copysign(mag, v).astype(np.float32)   # exact: bf16 values are fp32 values
    return (out.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def silu_ref(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + e^-g) in fp64 (e^-g overflows to inf for very
    negative g, giving a zero with the sign of g)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ref(y_bf16: np.ndarray) -> np.ndarray:
    """h[m][j] = silu(gate[m][j]) * up[m][j] in fp64, from the bf16 bits of
    the up/gate output y[m][2I]: gate = y[:, :I], up = y[:, I:]."""
    y = np.asarray(y_bf16, dtype=np.uint16)
    m, n2 = y.shape
    if n2 % 2:
        raise ValueError("the up/gate output must have an even number of columns")
    inter = n2 // 2
    yf = bf16_bits_to_f32(y).astype(np.float64)
    return silu_ref(yf[:, :inter]) * yf[:, inter:]


def swiglu_quant_ref(y_bf16: np.ndarray):
    """y[m][2I] bf16 bits -> (h bf16 bits [m][I], codes uint8 [m][I], scales
    fp32 [m][I/128]): SwiGLU, one rounding to bf16, then the 1 x 128 cast."""
    hb = bf16_bits_from_f64(swiglu_ref(y_bf16))
    codes, scales = quantize_act_ref(hb)
    return hb, codes, scales

// Device helpers shared by every kernel of the library (gfx950 only).
//
// The quantization rule implemented here: per block, scale = fl32(amax/448)
// and code = RNE_e4m3(fl32(x/scale)), with the E4M3 variant whose largest
// finite value is 448 ("Kernel-Level Optimisations for LLM Inference and
// Training", section "Quantisation kernels"), one scale per 128x128 weight
// block ("The profiler said the kernel ran zero times", section "The output
// layer, which did run") and one per row per 128 columns for activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

constexpr int BLK = 128;          // block edge along K (and along N for weights)
constexpr int ACT_STRIDE = 144;   // LDS bytes per staged activation block row (128 + 16 pad)

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 ---

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return bf16_rne(a) | (bf16_rne(b) << 16);
}

// ---------------------------------------------------------------- E4M3 ---

// Integer software encoder: nearest E4M3 value, ties to even mantissa,
// magnitudes >= 448 saturate, the sign bit is copied.
__device__ __forceinline__ uint32_t e4m3_encode_sw(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;              // |v| >= 448
  if (a >= 0x3C800000u) {                                 // |v| >= 2^-6: normal E4M3
    // round the fp32 pattern to 3 fraction bits (bit 20 is the kept LSB)
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t code = ((r >> 23) - 120u) << 3 | ((r >> 20) & 7u);
    return sign | (code > 0x7Eu ? 0x7Eu : code);
  }
  // subnormal E4M3 grid: multiples of 2^-9; |v| * 512 is exact and < 8
  const float t = __builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | (uint32_t)t;                              // t == 8 gives 0x08 = 2^-6
}

// Hardware conversion (v_cvt_pk_fp8_f32, OCP E4M3 on gfx950) of four values.
__device__ __forceinline__ uint32_t e4m3x4_hw(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3x4_sw(float a, float b, float c, float d) {
  return e4m3_encode_sw(a) | e4m3_encode_sw(b) << 8 | e4m3_encode_sw(c) << 16 |
         e4m3_encode_sw(d) << 24;
}

#ifndef FP8BS_ENCODER_SW
#define FP8BS_ENCODER_SW 0
#endif

// The encoder every quantizer uses.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
#if FP8BS_ENCODER_SW
  return e4m3x4_sw(a, b, c, d);
#else
  return e4m3x4_hw(a, b, c, d);
#endif
}

// Decode the four codes of w (K order: byte 0 first) to fp32.
__device__ __forceinline__ void e4m3x4_decode(uint32_t w, float* out) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo.x;
  out[1] = lo.y;
  out[2] = hi.x;
  out[3] = hi.y;
}

// ----------------------------------------------------------- quotients ---

// Below this block amax the fast quotient's exactness argument (all
// intermediates normal, remainder exact) is not made; use IEEE division.
constexpr float FAST_QUOTIENT_MIN_AMAX = 0x1p-60f;

// Replace x[i] by fl32(x[i] / s) for a block with largest magnitude `amax`
// and scale s = fl32(amax / 448). For amax >= 2^-60 the quotient comes from
// the correctly rounded reciprocal r = fl32(1/s): q0 = fl32(x r), then one
// correction with the exact remainder, taken negated, e' = s q0 - x (a fused
// multiply-add): q = fl32(q0 - e' r). For bf16 x and bf16 amax this equals
// the correctly rounded quotient (checked exhaustively over all mantissa
// pairs and exponent gaps; the result is scale invariant while every
// intermediate is normal, which amax >= 2^-60 guarantees for every x whose
// code is not 0). Taking the remainder negated keeps the sign of a zero x:
// for x = -0, e' = (-0) + (+0) = +0 and q = (-0) + (-0) = -0. An all-zero
// block (amax == 0) leaves x unchanged (signed zeros, codes 0x00 / 0x80).
template <int N>
__device__ __forceinline__ void block_quotients(float (&x)[N], float amax, float s) {
  if (amax >= FAST_QUOTIENT_MIN_AMAX) {
    const float r = 1.0f / s;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float q0 = x[i] * r;
      const float en = __builtin_fmaf(s, q0, -x[i]);
      x[i] = __builtin_fmaf(-en, r, q0);
    }
  } else if (amax > 0.0f) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] / s;
  }
}

// Load from memory that no kernel writes while it runs (block scales):
// through the constant address space, so uniform indices become scalar
// loads that do not queue behind the vector weight loads.
template <typename T>
__device__ __forceinline__ T load_invariant(const T* p, size_t i) {
  typedef const __attribute__((address_space(4))) T* cptr;
  return ((cptr)(uintptr_t)p)[i];
}

// 16-byte load of streamed weight data, read once per GEMM: marked
// non-temporal so the caches do not keep it. On gfx950 this lifts the
// achievable read rate of large weight streams by ~15%.
__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, then meets the other waves. Unlike __syncthreads() it does not
// wait for outstanding global loads, so weight prefetches stay in flight
// across it. The memory clobber keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// --------------------------------------------------------- lane shuffles ---

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_ROR8 = 0x128;      // rotate each 16-lane row by 8

__device__ __forceinline__ float quad_max(float v) {
  v = __builtin_fmaxf(v, dpp_f<DPP_QUAD_XOR1>(v));
  v = __builtin_fmaxf(v, dpp_f<DPP_QUAD_XOR2>(v));
  return v;
}

// Sum over the 8 lanes of each aligned group of 8; every lane gets the same
// bits (each step adds a pair in an order-independent way).
__device__ __forceinline__ float octet_sum(float v) {
  v = v + dpp_f<DPP_QUAD_XOR1>(v);
  v = v + dpp_f<DPP_QUAD_XOR2>(v);
  v = v + dpp_f<DPP_ROW_HALF_MIRROR>(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o));
  return v;
}

// -------------------------------------------------- activation block cast ---

// One quarter (32 values) of a 1x128 activation block: xw holds 16 dwords =
// 32 bf16 in K order. Unpacks them to x and returns their largest magnitude.
__device__ __forceinline__ float quarter_unpack(const uint4 (&xw)[4], float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {xw[i].x, xw[i].y, xw[i].z, xw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[8 * i + 2 * j] = bf16_lo(w[j]);
      x[8 * i + 2 * j + 1] = bf16_hi(w[j]);
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(x[i]));
  return am;
}

// Codes (8 dwords = 32 codes in K order) of a quarter whose block has
// largest magnitude am; returns the block scale fl32(am / 448).
__device__ __forceinline__ float quarter_codes(float (&x)[32], float am, uint32_t (&codes)[8]) {
  const float s = am / 448.0f;
  block_quotients(x, am, s);
#pragma unroll
  for (int i = 0; i < 8; ++i) codes[i] = e4m3x4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  return s;
}

// Cast one quarter of a 1x128 activation block. The four quarters of a
// block must sit in the four lanes of one DPP quad, quarter q in lane q of
// the quad; the block amax is reduced across the quad.
// Returns the block scale (identical in the four lanes).
__device__ __forceinline__ float cast_quarter(const uint4 (&xw)[4], uint32_t (&codes)[8]) {
  float x[32];
  float am = quarter_unpack(xw, x);
  am = quad_max(am);
  return quarter_codes(x, am, codes);
}

// The same cast with the four quarters of a block in lanes l, l^16, l^32,
// l^48 (quarter l/16: the K layout of an MFMA operand). The block amax is the
// same maximum and each code the same per-element arithmetic, so scale and
// codes equal cast_quarter's bit for bit. The quotients and codes are formed
// 8 values at a time, which keeps few registers live in kernels that hold
// many operands.
__device__ __forceinline__ float cast_quarter_cols(const uint4 (&xw)[4], uint32_t (&codes)[8]) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {xw[i].x, xw[i].y, xw[i].z, xw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(bf16_lo(w[j])),
                                               __builtin_fabsf(bf16_hi(w[j]))));
  }
  am = __builtin_fmaxf(am, __shfl_xor(am, 16));
  am = __builtin_fmaxf(am, __shfl_xor(am, 32));
  const float s = am / 448.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w[4] = {xw[i].x, xw[i].y, xw[i].z, xw[i].w};
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(w[j]);
      x[2 * j + 1] = bf16_hi(w[j]);
    }
    block_quotients(x, am, s);
    codes[2 * i] = e4m3x4(x[0], x[1], x[2], x[3]);
    codes[2 * i + 1] = e4m3x4(x[4], x[5], x[6], x[7]);
    __builtin_amdgcn_sched_barrier(0);
  }
  return s;
}

// ----------------------------------------------------- SwiGLU epilogue ---

// fp64 -> bf16 bits in one rounding (nearest, ties to the even mantissa):
// a value whose leading bit has weight 2^e keeps the multiple of 2^(e-7)
// nearest to it, values below 2^-126 the nearest multiple of 2^-133
// (subnormals); magnitudes that round past the largest finite bf16 become
// infinity, and zero keeps its sign. Integer rounding on the fp64 pattern
// for the normal range, an exact power-of-two scaling and rint below it.
__device__ __forceinline__ uint32_t bf16_rne_f64(double v) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
  const uint64_t a = bits & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return sign | 0x7FC0u;   // NaN
  if (a >= 0x3810000000000000ull) {                        // |v| >= 2^-126
    // drop 45 of the 52 fraction bits; a carry moves into the exponent
    const uint64_t r = a + ((1ull << 44) - 1ull) + ((a >> 45) & 1ull);
    const int64_t e = (int64_t)(r >> 52) - 1023 + 127;     // biased bf16 exponent
    if (e >= 255) return sign | 0x7F80u;
    return sign | (uint32_t)(e << 7) | (uint32_t)((r >> 45) & 0x7Fu);
  }
  // |v| < 2^-126: the scaled value is exact and below 128; 128 itself is
  // the pattern of the smallest normal, 2^-126
  const double t = __builtin_rint(__longlong_as_double((long long)a) * 0x1p133);
  return sign | (uint32_t)t;
}

// h = silu(g) * u for one (gate, up) pair of bf16 values, rounded once to
// bf16: silu(g) = g / (1 + e^-g) (the gated unit of Shazeer, "GLU Variants
// Improve Transformer"). Evaluated in fp64: e^-g overflows only below
// g = -709, where silu(g) * u lies far below the smallest bf16, so the
// quotient g / inf = -0 gives the right bf16 zero; for every other bf16 g
// the intermediates stay normal fp64 values (fp32 evaluation would lose
// e^g to subnormals or overflow for g below about -87). No contraction
// into fused multiply-adds, so every kernel that applies it gives the same
// bits.
__device__ __forceinline__ uint32_t swiglu_one(float g, float u) {
#pragma clang fp contract(off)
  const double gd = (double)g;
  const double h = gd / (1.0 + exp(-gd)) * (double)u;
  return bf16_rne_f64(h);
}

// The pair of (gate, up) values packed as bf16 in one dword each.
__device__ __forceinline__ uint32_t swiglu_pair(uint32_t g, uint32_t u) {
  return swiglu_one(bf16_lo(g), bf16_lo(u)) | (swiglu_one(bf16_hi(g), bf16_hi(u)) << 16);
}

// The SwiGLU step and the 1x128 cast for one activation row of one 128-column
// block, by one wave: lane l holds gate and up columns 2l, 2l+1 (one dword of
// bf16 pairs each). The block amax is reduced over the wave; scale and codes
// follow the activation rule (the same quotient and encoder as cast_quarter).
// Writes codes 2l, 2l+1 to hq_row (the block's 128 codes) and, from lane 0,
// the scale to *hs.
__device__ __forceinline__ void swiglu_cast_wave(uint32_t gw, uint32_t uw, int l,
                                                 uint8_t* hq_row, float* hs) {
  const uint32_t hw = swiglu_pair(gw, uw);
  float x[2] = {bf16_lo(hw), bf16_hi(hw)};
  const float am = wave_max(__builtin_fmaxf(__builtin_fabsf(x[0]), __builtin_fabsf(x[1])));
  const float sc = am / 448.0f;
  block_quotients(x, am, sc);
  const uint32_t codes = e4m3x4(x[0], x[1], 0.0f, 0.0f);
  *reinterpret_cast<uint16_t*>(hq_row + 2 * l) = (uint16_t)codes;
  if (l == 0) *hs = sc;
}

// 32 pairs: g, u hold 16 dwords (32 bf16) each in column order; h gets 16 dwords.
__device__ __forceinline__ void swiglu_quarter(const uint32_t (&g)[16], const uint32_t (&u)[16],
                                               uint4 (&h)[4]) {
  uint32_t hw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) hw[i] = swiglu_pair(g[i], u[i]);
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = make_uint4(hw[4 * j], hw[4 * j + 1], hw[4 * j + 2], hw[4 * j + 3]);
}

}  // namespace fp8bs

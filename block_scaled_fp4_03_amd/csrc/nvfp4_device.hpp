// Device-side number formats and math shared by the gfx950 kernels.
//
// NVFP4: E2M1 element codes (sign bit 3, magnitudes {0,0.5,1,1.5,2,3,4,6}),
// one E4M3 (FN) scale per 16 elements, one float32 global scale per tensor in
// the dequantisation direction.  Every float step below is a single IEEE
// float32 operation; the library is compiled with -ffp-contract=off so no
// multiply-add is fused behind our back, which keeps the quantised codes,
// routing weights and combine results identical on every run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// E2M1 encode: magnitude index of a = |v| >= 0, round to nearest with ties to
// the even index, saturating at index 7 (6.0).  Each comparison adds one when
// a passes the boundary between two neighbouring magnitudes; a tie stays on
// the even side, so boundaries below an odd index use '>' and boundaries
// below an even index use '>='.
__device__ __forceinline__ uint32_t e2m1_index(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

// E4M3 (FN) code of a finite s >= 0: round to nearest-even on a 3-bit
// mantissa, saturate at 448 (code 0x7E); never NaN.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (s >= 448.0f) return 0x7Eu;                 // 448..464 rounds to 448; above saturates
  const uint32_t u = __float_as_uint(s);
  const int e = (int)(u >> 23) - 127;
  if (e < -6) {
    // E4M3 subnormals are m * 2^-9; s * 512 is exact, rint is ties-to-even,
    // and m == 8 is the smallest normal (code 0x08) as it should be.
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  // Normal: round the float32 mantissa to 3 bits, ties to even.  A carry out
  // of the mantissa bumps the exponent, which the bit arithmetic does for us.
  const uint32_t lsb = (u >> 20) & 1u;
  const uint32_t r = u + 0x7FFFFu + lsb;
  const uint32_t code = ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// E4M3 (FN) value of a non-negative code; exact.  gfx950 converts OCP E4M3
// natively (checked over all 256 codes).
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// Scale code of a block whose largest magnitude is bamax, with the
// reciprocal r that maps its elements onto the E2M1 grid; `zero` when the
// scale decodes to 0 (then every code of the block is 0x0).  Each step is
// one IEEE float32 operation, in this order.
__device__ __forceinline__ uint32_t block_scale(float bamax, float gs, float& r, bool& zero) {
  const float d = 6.0f * gs;
  const float s = bamax / d;
  const uint32_t sq = e4m3_encode(s);
  const float sf = e4m3_decode(sq);
  zero = sf == 0.0f;
  r = zero ? 0.0f : 1.0f / (sf * gs);
  return sq;
}

// E2M1 code of x in a block with reciprocal r: the sign bit of x plus the
// magnitude nearest to |x * r|.
__device__ __forceinline__ uint32_t e2m1_code(float x, float r, bool zero) {
  if (zero) return 0u;
  const float v = x * r;
  return e2m1_index(__builtin_fabsf(v)) | ((__float_as_uint(x) >> 28) & 8u);
}

// E2M1 codes of the 2P values x[0..2P) of one block with reciprocal r, value
// i in nibble i: the code e2m1_code gives for each.  gfx950's packed
// conversion (scale 1) rounds exactly like e2m1_code on every float32 that is
// not a NaN, sign included (checked over all 2^32 patterns), so for a finite
// r > 0 a pair costs two multiplies and one conversion; x * r can be a NaN
// only when r is not such a number (sf * gs underflowed, or a global scale
// that is not positive), and those blocks take the comparison encoder.
template <int P>
__device__ __forceinline__ uint32_t e2m1_pack(const float* x, float r, bool zero) {
  static_assert(P >= 1 && P <= 4, "one to four pairs per word");
  if (zero) return 0u;
  uint32_t w = 0u;
  if (r > 0.0f && r < __builtin_inff()) {
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] * r, x[1] * r, 1.0f, 0);
    if constexpr (P > 1) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] * r, x[3] * r, 1.0f, 1);
    if constexpr (P > 2) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] * r, x[5] * r, 1.0f, 2);
    if constexpr (P > 3) w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] * r, x[7] * r, 1.0f, 3);
    return w;
  }
#pragma unroll
  for (int i = 0; i < 2 * P; ++i) w |= e2m1_code(x[i], r, false) << (4 * i);
  return w;
}

// Quantise one 16-element block.  x: 16 finite floats.  Returns the scale code
// and writes the 16 packed codes (element 2i in the low nibble) as two words.
__device__ __forceinline__ uint32_t quantize_block16(const float (&x)[16], float gs,
                                                     uint32_t& lo, uint32_t& hi) {
  float bamax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bamax = __builtin_fmaxf(bamax, __builtin_fabsf(x[i]));
  float r;
  bool zero;
  const uint32_t sq = block_scale(bamax, gs, r, zero);
  lo = e2m1_pack<4>(x, r, zero);
  hi = e2m1_pack<4>(x + 8, r, zero);
  return sq;
}

// ---------------------------------------------------------------------------
// float32 exponential for SiLU and the routing softmax (Cody & Waite, 1980):
// n = rint(x*log2 e); r = (x - n*L_hi) - n*L_lo with L_hi = 355/512 (exact
// products for |n| < 2^15) and L_lo = ln 2 - L_hi; p = sum_{j<=8} r^j/j! by
// Horner; result p * 2^n.  x > 88 gives +Inf, x < -80 gives 0, so finite
// non-zero results are normal floats.
__device__ __forceinline__ float exp_f32(float x) {
  if (x > 88.0f) return __builtin_inff();
  if (x < -80.0f) return 0.0f;
  const float kLog2e = 0x1.715476p+0f;    // nearest float to 1/ln 2
  const float kLnHi = 0x1.63p-1f;        // 355/512
  const float kLnLo = -0x1.bd0106p-13f;  // ln 2 - 355/512, to float
  const float n = __builtin_rintf(x * kLog2e);
  float r = x - n * kLnHi;
  r = r - n * kLnLo;
  // 1/j! for j = 8..0, each rounded to float
  float p = 0x1.a01a02p-16f;                     // 1/8!
  p = p * r + 0x1.a01a02p-13f;                   // 1/7!
  p = p * r + 0x1.6c16c2p-10f;                   // 1/6!
  p = p * r + 0x1.111112p-7f;                    // 1/5!
  p = p * r + 0x1.555556p-5f;                    // 1/4!
  p = p * r + 0x1.555556p-3f;                    // 1/3!
  p = p * r + 0.5f;                                    // 1/2!
  p = p * r + 1.0f;                                    // 1/1!
  p = p * r + 1.0f;                                    // 1/0!
  return __builtin_ldexpf(p, (int)n);
}

// SiLU(g) * u with exp_f32, one IEEE op per step.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = exp_f32(-g);
  const float den = 1.0f + e;
  const float s = g / den;
  return s * u;
}

// ---------------------------------------------------------------------------
// bf16 <-> float (round to nearest-even; inputs are finite).  gfx950
// converts with v_cvt_pk_bf16_f32, two values per instruction; an in-bounds
// check over every finite float32 bit pattern (subnormals included) found it
// equal to round-to-nearest-even by integer arithmetic, (u + 0x7FFF +
// ((u >> 16) & 1)) >> 16, in all of them.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t bf16_from_float(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values as one word, a in the low half
__device__ __forceinline__ uint32_t bf16x2_from_float(float a, float b) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// Load 16 consecutive elements (bf16 or f32) as floats.  p must be 16-byte
// aligned.
template <bool kBf16>
__device__ __forceinline__ void load16(const void* p, float (&x)[16]) {
  if constexpr (kBf16) {
    const uint4* q = (const uint4*)p;
    const uint4 a = q[0], b = q[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* q = (const float4*)p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = q[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  }
}

// ---------------------------------------------------------------------------
// Dequantisation for the matrix cores: eight E2M1 codes (one 32-bit word,
// element 0 in the low nibble) times their block scale, as eight f16 values.
// The gfx950 convert instruction takes only the exponent of its scale
// operand, so it is used with scale 1 (exact E2M1 -> f16) and the E4M3 block
// scale is applied with a packed f16 multiply.  e2m1 * e4m3 has at most five
// significant bits and lies in [2^-10, 2688], so the f16 product is exact.
__device__ __forceinline__ half8_t dequant8(uint32_t codes, half2_t sf2) {
  half8_t r;
  const half2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sf2;
  const half2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sf2;
  const half2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sf2;
  const half2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sf2;
  r[0] = v0[0]; r[1] = v0[1]; r[2] = v1[0]; r[3] = v1[1];
  r[4] = v2[0]; r[5] = v2[1]; r[6] = v3[0]; r[7] = v3[1];
  return r;
}

// Two E2M1 codes (byte `sel` of `codes`) times their block scale, as f16;
// the pieces dequant8 is made of, for code that spreads them between other
// instructions.  `sel` must fold to a constant.
__device__ __forceinline__ half2_t dequant_pair(uint32_t codes, int sel, half2_t sf2) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * sf2;
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * sf2;
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * sf2;
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * sf2;
  }
}

// E4M3 scale code -> the f16 pair (sf, sf) for dequant8.
__device__ __forceinline__ half2_t scale_pair(uint32_t code) {
  const _Float16 h = (_Float16)e4m3_decode(code);     // exact: E4M3 values fit f16
  half2_t r;
  r[0] = h;
  r[1] = h;
  return r;
}

// The 16 dequantised values e2m1(code) * e4m3(scale) of a block (without
// the global scale) as f16, written as 32 contiguous bytes.  Exact: the
// product has at most five significant bits and lies in [2^-10, 2688].
__device__ __forceinline__ void store_dq16(void* dst, uint32_t lo, uint32_t hi, uint32_t scale_code) {
  const half2_t sf2 = scale_pair(scale_code);
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  u32x4v a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(uint32_t, dequant_pair(lo, i, sf2));
    b[i] = __builtin_bit_cast(uint32_t, dequant_pair(hi, i, sf2));
  }
  ((u32x4v*)dst)[0] = a;
  ((u32x4v*)dst)[1] = b;
}

// Value of an E2M1 code times a decoded block scale, as f16 (exact: at most
// five significant bits, magnitude in [2^-10, 2688]).
__device__ __forceinline__ uint16_t dq_f16(uint32_t code, float sf) {
  // magnitude index i: 0 -> 0, 1 -> 0.5, i >= 2 -> 2^(i/2 - 1) * (1 + (i & 1) / 2)
  const uint32_t i = code & 7u;
  const float m = i >= 2u ? __uint_as_float(((126u + (i >> 1)) << 23) | ((i & 1u) << 22)) : (i == 1u ? 0.5f : 0.0f);
  float v = m * sf;
  v = (code & 8u) ? -v : v;
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

}  // namespace nvfp4

// Shared device helpers for the gfx950 kernels: element types, conversions,
// MFMA fragment wrappers, wave reductions and the Philox4x32-10 generator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// ---------------------------------------------------------------------------- element types

// bfloat16 kept as its raw 16 bits.
struct bf16 {
  uint16_t v;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return __uint_as_float(uint32_t(x.v) << 16); }

// binary32 -> bfloat16, round to nearest even; NaN stays a (quiet) NaN.
// gfx950 converts in hardware (v_cvt_pk_bf16_f32, two values per
// instruction); checked against the integer round-to-nearest-even rule
// (add 0x7fff plus the lowest kept bit, truncate; NaN -> quiet NaN) on all
// 2^32 inputs, denormals included, with no difference.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ bf16 f32_to_bf16(float f) {
  return bf16{__builtin_bit_cast(uint16_t, (__bf16)f)};
}
// (lo, hi) -> one word holding bf16(lo) in bits 0..15 and bf16(hi) in 16..31
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float f) { return f32_to_bf16(f); }

// Round a binary32 value to the storage precision of T and back.
template <typename T> __device__ __forceinline__ float round_to(float f) {
  return to_f32(from_f32<T>(f));
}

// OCP E4M3FN code -> bfloat16 bits (exact: 3 mantissa bits fit in 7).
// Normal codes map exponent e (bias 7) to e + 120 (bias 127); subnormal codes
// (exponent field 0) encode m * 2^-9 and are rebuilt from their integer m.
// The NaN codes (S.1111.111) map to a bf16 NaN.
__device__ __forceinline__ uint16_t e4m3_to_bf16_bits(uint32_t c) {
  uint32_t s = (c & 0x80u) << 8;
  uint32_t em = c & 0x7fu;
  uint32_t normal = (em << 4) + (120u << 7);
  uint32_t sub = __float_as_uint(float(em) * 0x1p-9f) >> 16;   // exact for em < 8
  uint32_t r = (em >= 8u) ? normal : sub;
  if (em == 0x7fu) r = 0x7fc0u;
  return uint16_t(s | r);
}

// ---------------------------------------------------------------------------- vector types

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8 OCP E4M3FN codes (bytes of c, low first) -> 8 bf16 values, exact: the
// gfx950 packed conversion with scale 1 (checked against e4m3_to_bf16_bits
// for all 65536 byte pairs on the device).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 c) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true));
  return r;
}

// 8 E2M1 codes (the nibbles of w, lowest first: OCP MX FP4, 1 sign, 2
// exponent bits with bias 1, 1 mantissa bit) times the E8M0 block scale
// 2^(e8 - 127) -> 8 bf16 values, by the gfx950 packed FP4 -> BF16 conversion
// with an fp32 scale.  Exact for scale codes 1 .. 254 while the products stay
// in bf16's normal range (an E2M1 value has 2 significant bits); code 0
// yields zeros (the quantizer gives it only to all-zero blocks).
__device__ __forceinline__ u32x4 e2m1x8_to_bf16x8(uint32_t w, uint32_t e8) {
  const float sc = __uint_as_float(e8 << 23);
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return r;
}

// ---------------------------------------------------------------------------- MFMA

// D = A(16x32) * B(32x16) + C on one wave; lane l supplies row/col (l % 16)
// and k-slots 8*(l/16)..8*(l/16)+7 of its operand; D lane l holds column
// (l % 16), rows 4*(l/16)+0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// fp32 variant: A(16x4) * B(4x16); lane l supplies row/col (l % 16), k-slot l/16.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------- wave helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------- LM-head partials

// Online-softmax summary of a set of logits z of one row: m = max z,
// s = sum e^(z-m), t = sum e^(z-m)(z-m), sec = second largest z, idx = lowest
// column holding the max (INT_MAX: empty set).  The row's entropy is
// ln(s) - t/s.
struct LmPart {
  float m, s, t, sec;
  int idx;
};

__device__ __forceinline__ LmPart lm_empty_part() {
  LmPart p;
  p.m = -INFINITY;
  p.s = 0.f;
  p.t = 0.f;
  p.sec = -INFINITY;
  p.idx = 0x7fffffff;
  return p;
}

// Summary of the union of two disjoint column sets; equal maxima keep the
// lower index and make the second max equal to the max.
__device__ __forceinline__ LmPart lm_combine(LmPart a, LmPart b) {
  if (b.idx == 0x7fffffff) return a;
  if (a.idx == 0x7fffffff) return b;
  LmPart r;
  const float M = fmaxf(a.m, b.m);
  const float ea = __expf(a.m - M), eb = __expf(b.m - M);
  r.s = a.s * ea + b.s * eb;
  r.t = ea * (a.t + (a.m - M) * a.s) + eb * (b.t + (b.m - M) * b.s);
  r.m = M;
  if (a.m > b.m) {
    r.idx = a.idx;
    r.sec = fmaxf(a.sec, b.m);
  } else if (b.m > a.m) {
    r.idx = b.idx;
    r.sec = fmaxf(b.sec, a.m);
  } else {
    r.idx = min(a.idx, b.idx);
    r.sec = a.m;
  }
  return r;
}

__device__ __forceinline__ LmPart lm_shfl_xor(const LmPart& a, int o) {
  LmPart r;
  r.m = __shfl_xor(a.m, o, 64);
  r.s = __shfl_xor(a.s, o, 64);
  r.t = __shfl_xor(a.t, o, 64);
  r.sec = __shfl_xor(a.sec, o, 64);
  r.idx = __shfl_xor(a.idx, o, 64);
  return r;
}

// ---------------------------------------------------------------------------- Philox4x32-10

// Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011):
// ten rounds; each multiplies words 0 and 2 by M0/M1, mixes the product
// halves with words 1 and 3 and the round key; the key advances by W0/W1.
struct u32x4s {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4s philox4x32_10(u32x4s c, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    uint32_t hi0 = __umulhi(M0, c.x), lo0 = M0 * c.x;
    uint32_t hi1 = __umulhi(M1, c.z), lo1 = M1 * c.z;
    c = u32x4s{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

// Token draw for a canvas position: word 0 of counter (pos, tag, canvas, block).
__device__ __forceinline__ uint32_t canvas_draw(uint64_t seed, uint32_t pos, uint32_t tag,
                                                uint32_t canvas, uint32_t block, uint32_t vocab) {
  u32x4s r = philox4x32_10(u32x4s{pos, tag, canvas, block}, uint32_t(seed), uint32_t(seed >> 32));
  return vocab ? r.x % vocab : r.x;
}

}  // namespace dg

// codec.hpp -- device-side FP8 element codec for gfx950 (CDNA4).
//
// The operation is the FP8 cache path of the KV-cache quantization textbook
// (section 10.4.5): write cast_fp8(x / s), read cast_float(code) * s, with the
// OCP E4M3fn / E5M2 formats named in the vLLM FP8 KV-cache guide's
// kv_cache_dtype table.  Encoding saturates (|q| beyond max and +-Inf give
// +-max), rounds to nearest even, keeps NaN as NaN, keeps the sign of zero and
// produces subnormal codes.
//
// gfx950 converts natively between fp32 and OCP fp8/bf8 (v_cvt_pk_fp8_f32,
// v_cvt_pk_bf8_f32, round-to-nearest-even) and from fp8/bf8 to f32, f16 and
// bf16 (v_cvt_pk_f32_fp8, v_cvt_scalef32_pk_{f16,bf16}_{fp8,bf8}).  The only
// extra work the encoder needs is the saturating clamp, which must let NaN
// through: v_med3 alone would turn NaN into a finite value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// E4M3 / E5M2: OCP FP8.  INT8: symmetric 8-bit integers, clip(round(x/s),
// -127, 127) (the KV-cache quantization textbook's write rule, 10.4.2).
enum Fmt : int { E4M3 = 0, E5M2 = 1, INT8 = 2 };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Calls f(FmtTag<F>{}) for the runtime format (a template argument inside f).
template <int F>
struct FmtTag {
  static constexpr int value = F;
};
template <typename Fn>
__host__ inline void dispatch_fmt(int fmt, Fn&& f) {
  if (fmt == E4M3) f(FmtTag<E4M3>{});
  else if (fmt == E5M2) f(FmtTag<E5M2>{});
  else f(FmtTag<INT8>{});
}

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<E4M3> {
  static constexpr float kMax = 448.0f;
};
template <>
struct FmtTraits<E5M2> {
  static constexpr float kMax = 57344.0f;
};
template <>
struct FmtTraits<INT8> {
  static constexpr float kMax = 127.0f;
};

// ---------------------------------------------------------------- INT8
// code = two's complement byte of clip(round-half-even(x), -127, 127); a NaN
// quotient gives 0 and +-Inf clip to +-127 (there is no NaN or Inf code).
__device__ __forceinline__ uint32_t i8_code(float x) {
  float r = __builtin_amdgcn_fmed3f(__builtin_rintf(x), -127.0f, 127.0f);  // v_rndne_f32
  r = (x != x) ? 0.0f : r;
  return (uint32_t)(int)r & 0xffu;
}
// two signed codes (bytes 2 HI, 2 HI + 1 of w) -> f16x2, exact: the byte
// with its sign bit flipped is b + 128, placed as the low mantissa bits of
// the f16 1024.0 (bits 0x64xx) it reads 1152 + b; one packed subtract.
template <bool HI>
__device__ __forceinline__ f16x2 i8x2_to_f16(uint32_t w) {
  const uint32_t x = (HI ? (w >> 16) : w) ^ 0x8080u;
  const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u);  // [x0,64,x1,64]
  return __builtin_bit_cast(f16x2, bits) - f16x2{(_Float16)1152.0f, (_Float16)1152.0f};
}

// Saturating clamp that keeps NaN: med3 clamps finite values and +-Inf.
__device__ __forceinline__ float clamp_keep_nan(float x, float m) {
  float y = __builtin_amdgcn_fmed3f(x, -m, m);
  return (x != x) ? x : y;
}

// Two fp32 values -> two codes in the low 16 bits (a in byte 0, b in byte 1).
template <int FMT>
__device__ __forceinline__ uint32_t enc2(float a, float b) {
  if constexpr (FMT == INT8) return i8_code(a) | (i8_code(b) << 8);
  const float m = FmtTraits<FMT>::kMax;
  a = clamp_keep_nan(a, m);
  b = clamp_keep_nan(b, m);
  if constexpr (FMT == E4M3)
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  else
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
}

// Four fp32 values -> four codes packed little-endian in one dword.
template <int FMT>
__device__ __forceinline__ uint32_t enc4(float a, float b, float c, float d) {
  if constexpr (FMT == INT8)
    return i8_code(a) | (i8_code(b) << 8) | (i8_code(c) << 16) | (i8_code(d) << 24);
  const float m = FmtTraits<FMT>::kMax;
  a = clamp_keep_nan(a, m);
  b = clamp_keep_nan(b, m);
  c = clamp_keep_nan(c, m);
  d = clamp_keep_nan(d, m);
  int w;
  if constexpr (FMT == E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// Two codes (bytes 2*hi, 2*hi+1 of w) -> exact fp32 values.
template <int FMT, bool HI>
__device__ __forceinline__ f32x2 dec2_f32(uint32_t w) {
  if constexpr (FMT == INT8) {
    const uint32_t x = w ^ 0x80808080u;  // unsigned byte = code + 128
    return HI ? f32x2{(float)((x >> 16) & 0xffu) - 128.0f, (float)(x >> 24) - 128.0f}
              : f32x2{(float)(x & 0xffu) - 128.0f, (float)((x >> 8) & 0xffu) - 128.0f};
  } else if constexpr (FMT == E4M3)
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  else
    return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, HI);
}

// Two codes -> two exact bf16 values (every E4M3 and E5M2 value is a bf16 value).
template <int FMT, bool HI>
__device__ __forceinline__ bf16x2 dec2_bf16(uint32_t w) {
  if constexpr (FMT == INT8) {
    // |code| <= 128 has at most 8 significant bits: the fp32 value's top half
    // is the exact bf16
    const f32x2 f = dec2_f32<INT8, HI>(w);
    return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(__float_as_uint(f.y),
                                                            __float_as_uint(f.x), 0x07060302u));
  } else if constexpr (FMT == E4M3)
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
  else
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w, 1.0f, HI);
}

// Two codes -> two exact f16 values (every E4M3 and E5M2 value is an f16 value).
template <int FMT, bool HI>
__device__ __forceinline__ f16x2 dec2_f16(uint32_t w) {
  if constexpr (FMT == INT8)
    return i8x2_to_f16<HI>(w);
  else if constexpr (FMT == E4M3)
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI);
  else
    return __builtin_amdgcn_cvt_scalef32_pk_f16_bf8((int)w, 1.0f, HI);
}

// ---------------------------------------------------------------- quotient
// fl32(x / s) for a positive, finite, normal scale s whose reciprocal is
// normal too, given rs = fl32(1 / s).
//
// q0 = fl32(x * rs) is within an ulp of x / s; its remainder
// e = x - s * q0 is exact in one FMA, and q0 + e * rs rounded once is the
// correctly rounded quotient (Markstein's correction step, IBM J. Res. Dev.
// 34(1), 1990).  Three cases fall outside the theorem and are routed around
// it: |q0| >= 2^16 (including Inf and overflow), where every later step
// saturates to the format's max anyway and q0 is kept; NaN input, kept by the
// same select; and the sign of zero, restored from x.  Quotients below 2^-126
// may be off by an ulp there, but every such value encodes to a signed zero in
// both formats.  The library's tests compare this against an fp64 division
// over every bf16 input for each scale they use.
__device__ __forceinline__ float quotient(float x, float s, float rs) {
  float q0 = x * rs;
  float e = __builtin_fmaf(-q0, s, x);
  float q1 = __builtin_fmaf(e, rs, q0);
  q1 = (__builtin_fabsf(q0) < 65536.0f) ? q1 : q0;
  return __builtin_copysignf(q1, x);
}

// Correctly rounded reciprocal of the scale (computed once per thread).
__device__ __forceinline__ float recip_rn(float s) { return __fdiv_rn(1.0f, s); }

// A quantization scale prepared for the quotient above, for any positive
// finite s below 2^126 (every calibrated scale; subnormal ones included).  A
// scale below 2^-100 (calibration gives one only for a tensor whose amax is
// below about 2^-91) has a reciprocal at or beyond the fp32 range, so it is
// taken as s' = s 2^64 and the dividend as x' = x 2^64: both products are
// exact powers-of-two scalings, x' / s' = x / s, and x' overflows only where
// x / s saturates the format anyway.
struct Divisor {
  float s, rs, pre;
};
__device__ __forceinline__ Divisor make_divisor(float s) {
  Divisor d;
  d.pre = s < 0x1p-100f ? 0x1p64f : 1.0f;
  d.s = s * d.pre;
  d.rs = recip_rn(d.s);
  return d;
}
__device__ __forceinline__ float quotient(float x, const Divisor& d) {
  return quotient(x * d.pre, d.s, d.rs);
}

// The FP8 encoders' argument: fl32(x / s) clamped to +-max with NaN kept, the
// same value as clamp_keep_nan(quotient(x, d), max) in fewer operations (8).
// Where |x / s| >= 2^16 every later step saturates, so the first estimate is
// clamped to +-2^16 before the correction step instead of being selected
// after it: an infinite x then stays infinite (not NaN) through the
// correction and clamps to +-max; below 2^16 the estimate is untouched and the
// arithmetic is the quotient's.  NaN is restored from x at the end (the clamps
// drop it).  PRE: the divisor carries the 2^64 prescale of tiny scales (a
// caller whose scales are all at or above 2^-100 passes false and saves one
// multiply per value).
template <int FMT, bool PRE>
__device__ __forceinline__ float fp8_arg(float x, const Divisor& d) {
  const float xs = PRE ? x * d.pre : x;
  const float q0 = __builtin_amdgcn_fmed3f(xs * d.rs, -65536.0f, 65536.0f);
  const float e = __builtin_fmaf(-q0, d.s, xs);
  const float q1 = __builtin_copysignf(__builtin_fmaf(e, d.rs, q0), xs);
  constexpr float m = FmtTraits<FMT>::kMax;
  const float c = __builtin_amdgcn_fmed3f(q1, -m, m);
  return xs != xs ? xs : c;
}

// Four already clamped (or NaN) values -> four FP8 codes, little-endian.
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  int w;
  if constexpr (FMT == E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

// bf16 bit patterns packed two per dword -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept as a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace kvq

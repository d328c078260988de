// attn_common.hpp -- helpers shared by the attention kernels (decode over the
// FP8 / INT8 cache and decode over the 2-bit cache): constants of the log2-domain
// online softmax, DPP row reductions, streaming loads and MFMA operand types.
#pragma once

#include "codec.hpp"

namespace kvq {
namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max over the 16 lanes of a row (lanes 16i .. 16i+15); every lane gets it
__device__ __forceinline__ float max16(float x) {
  x = __builtin_fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = __builtin_fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = __builtin_fmaxf(x, dpp<0x141>(x));  // row_half_mirror
  x = __builtin_fmaxf(x, dpp<0x140>(x));  // row_mirror
  return x;
}

// 8 codes (two dwords) -> 8 exact bf16 / f16 values, assembled as one 128-bit
// value so the converts land directly in the MFMA operand registers
template <int FMT>
__device__ __forceinline__ bf16x8 codes_to_bf16x8(uint32_t a, uint32_t b) {
  const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, dec2_bf16<FMT, false>(a)),
                             __builtin_bit_cast(uint32_t, dec2_bf16<FMT, true>(a)),
                             __builtin_bit_cast(uint32_t, dec2_bf16<FMT, false>(b)),
                             __builtin_bit_cast(uint32_t, dec2_bf16<FMT, true>(b)));
  return __builtin_bit_cast(bf16x8, u);
}
template <int FMT>
__device__ __forceinline__ f16x8 codes_to_f16x8(uint32_t a, uint32_t b) {
  const uint4 u = make_uint4(__builtin_bit_cast(uint32_t, dec2_f16<FMT, false>(a)),
                             __builtin_bit_cast(uint32_t, dec2_f16<FMT, true>(a)),
                             __builtin_bit_cast(uint32_t, dec2_f16<FMT, false>(b)),
                             __builtin_bit_cast(uint32_t, dec2_f16<FMT, true>(b)));
  return __builtin_bit_cast(f16x8, u);
}

// word w of a uint4 held in registers (w folds to a constant once unrolled;
// a pointer cast instead can keep the array in scratch memory)
__device__ __forceinline__ uint32_t& u4word(uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}
__device__ __forceinline__ uint32_t u4word(const uint4& v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

// Cache loads are nontemporal: every cache byte is read once per call, so
// the loads stream through L2 instead of allocating in it.
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load8(const uint8_t* p) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

__device__ __forceinline__ int64_t clamp_block(int64_t blk, int64_t num_blocks) {
  return blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
}
}  // namespace
}  // namespace kvq

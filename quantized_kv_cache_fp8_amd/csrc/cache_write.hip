// cache_write.hip -- quantize-on-write of K and V into the paged FP8 cache.
//
// The write rule of the KV-cache quantization textbook (section 10.4.2,
// Kq = Q(K / sK), stored with sK) in its FP8 form (section 10.4.5,
// cast_fp8(K / sK)), placed through a slot mapping into the paged layout
// (slot -> block slot/bs, offset slot%bs):
//   K tiles are token-major  [num_blocks][Hkv][bs][dh]
//   V tiles are channel-major [num_blocks][Hkv][dh][bs]
// Both attention kernels contract V over tokens, so a channel-major V tile
// hands every matrix-core operand a contiguous run of tokens; the transpose
// is paid here, once per byte, in registers.
//
// Each thread owns four consecutive tokens x four consecutive channels of one
// KV head, for both K and V (consecutive threads take consecutive channel
// quads, so the bf16 loads are coalesced rows).  K codes go out as one dword
// per token.  When the four tokens occupy four consecutive, 4-aligned slots
// (the normal case: tokens of one sequence written in order) the 4x4 V code
// block is transposed with v_perm_b32 and goes out as one dword per channel;
// otherwise each V code is stored as a byte.  Per-head scales and their
// correctly rounded reciprocals are staged once per workgroup in LDS.
#include "codec.hpp"
#include "launch.hpp"

namespace kvq {

constexpr int kMaxHeadsLds = 256;
constexpr int kBs = 16;  // tokens per cache block

template <int FMT>
__device__ __forceinline__ uint32_t quant4(uint2 w, float s, float rs) {
  return enc4<FMT>(quotient(bf16lo(w.x), s, rs), quotient(bf16hi(w.x), s, rs),
                   quotient(bf16lo(w.y), s, rs), quotient(bf16hi(w.y), s, rs));
}

template <int FMT>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t T, int Hkv,
    int dh_shift, uint32_t units, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, int64_t num_slots,
    const float* __restrict__ ks, const float* __restrict__ vs, int per_head) {
  __shared__ float s_k[kMaxHeadsLds], r_k[kMaxHeadsLds], s_v[kMaxHeadsLds], r_v[kMaxHeadsLds];
  const int nh = per_head ? Hkv : 1;
  for (int i = threadIdx.x; i < nh; i += blockDim.x) {
    const float a = ks[i], b = vs[i];
    s_k[i] = a;
    r_k[i] = recip_rn(a);
    s_v[i] = b;
    r_v[i] = recip_rn(b);
  }
  __syncthreads();
  const int dh = 1 << dh_shift;
  const int cq_shift = dh_shift - 2;  // channel quads per row = dh / 4
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t cq = u & ((1u << cq_shift) - 1);
    const uint32_t rest = u >> cq_shift;  // tq * Hkv + h
    const uint32_t tq = rest / (uint32_t)Hkv;
    const int h = (int)(rest - tq * (uint32_t)Hkv);
    const int hs = per_head ? h : 0;
    const float sk = s_k[hs], rk = r_k[hs], sv = s_v[hs], rv = r_v[hs];
    const int64_t t0 = (int64_t)tq * 4;
    int64_t slot[4];
    uint2 wk[4], wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + j;
      slot[j] = t < T ? slot_mapping[t] : -1;
      if (slot[j] >= num_slots) slot[j] = -1;  // out of the pool: skipped like padding
      if (slot[j] >= 0) {
        const size_t src = ((size_t)t * Hkv + h) * dh + cq * 4;
        wk[j] = *reinterpret_cast<const uint2*>(k + src);
        wv[j] = *reinterpret_cast<const uint2*>(v + src);
      }
    }
    uint32_t cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (slot[j] < 0) continue;
      const int64_t blk = slot[j] >> 4, off = slot[j] & (kBs - 1);
      const size_t kt = ((size_t)(blk * Hkv + h) * kBs + off) * dh + cq * 4;
      *reinterpret_cast<uint32_t*>(kc + kt) = quant4<FMT>(wk[j], sk, rk);
      cv[j] = quant4<FMT>(wv[j], sv, rv);
    }
    const bool run4 = slot[0] >= 0 && (slot[0] & 3) == 0 && slot[1] == slot[0] + 1 &&
                      slot[2] == slot[0] + 2 && slot[3] == slot[0] + 3;
    if (run4) {
      // rows cv[j] = token j, bytes = channels 4cq..4cq+3 -> one dword per channel
      const uint32_t t0l = __builtin_amdgcn_perm(cv[1], cv[0], 0x05010400u);  // a0 b0 a1 b1
      const uint32_t t1l = __builtin_amdgcn_perm(cv[1], cv[0], 0x07030602u);  // a2 b2 a3 b3
      const uint32_t t2l = __builtin_amdgcn_perm(cv[3], cv[2], 0x05010400u);  // c0 d0 c1 d1
      const uint32_t t3l = __builtin_amdgcn_perm(cv[3], cv[2], 0x07030602u);  // c2 d2 c3 d3
      const int64_t blk = slot[0] >> 4, off = slot[0] & (kBs - 1);
      uint8_t* dst = vc + ((size_t)(blk * Hkv + h) * dh + cq * 4) * kBs + off;
      *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(t2l, t0l, 0x05040100u);
      *reinterpret_cast<uint32_t*>(dst + kBs) = __builtin_amdgcn_perm(t2l, t0l, 0x07060302u);
      *reinterpret_cast<uint32_t*>(dst + 2 * kBs) = __builtin_amdgcn_perm(t3l, t1l, 0x05040100u);
      *reinterpret_cast<uint32_t*>(dst + 3 * kBs) = __builtin_amdgcn_perm(t3l, t1l, 0x07060302u);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (slot[j] < 0) continue;
        const int64_t blk = slot[j] >> 4, off = slot[j] & (kBs - 1);
        uint8_t* dst = vc + ((size_t)(blk * Hkv + h) * dh + cq * 4) * kBs + off;
        dst[0] = (uint8_t)cv[j];
        dst[kBs] = (uint8_t)(cv[j] >> 8);
        dst[2 * kBs] = (uint8_t)(cv[j] >> 16);
        dst[3 * kBs] = (uint8_t)(cv[j] >> 24);
      }
    }
  }
}

hipError_t launch_cache_write(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                              const int64_t* slot, uint8_t* kc, uint8_t* vc, int64_t num_blocks,
                              const float* ks, const float* vs, int fmt, int per_head,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  int dh_shift = 0;
  while ((1 << dh_shift) < dh) ++dh_shift;
  const uint32_t units = (uint32_t)(((T + 3) / 4) * Hkv * (dh / 4));
  int64_t want = ((int64_t)units + 255) / 256;
  int64_t cap = (int64_t)device_cu_count() * 16;
  int grid = (int)(want < cap ? want : cap);
  const int64_t num_slots = num_blocks * kBs;
  if (fmt == E4M3)
    cache_write_kernel<E4M3><<<grid, 256, 0, s>>>(k, v, T, Hkv, dh_shift, units, slot, kc, vc,
                                                   num_slots, ks, vs, per_head);
  else
    cache_write_kernel<E5M2><<<grid, 256, 0, s>>>(k, v, T, Hkv, dh_shift, units, slot, kc, vc,
                                                   num_slots, ks, vs, per_head);
  return hipGetLastError();
}

}  // namespace kvq

// cache_write.hip -- quantize-on-write of K and V into the paged FP8 cache.
//
// The write rule of the KV-cache quantization textbook (section 10.4.2,
// Kq = Q(K / sK), stored with sK) in its FP8 form (section 10.4.5,
// cast_fp8(K / sK)), placed through a slot mapping into the paged layout
// uint8 [num_blocks][Hkv][bs][dh] (token slot -> block slot/bs, offset slot%bs).
//
// Pure streaming kernel: each thread owns one 16-byte chunk (8 channels) of
// one (token, head) row of K and the same chunk of V, so both loads are
// in flight together; consecutive threads cover consecutive chunks, so reads
// are fully coalesced and every (token, head) row becomes one contiguous
// dh-byte run in its cache tile.  Per-head scales and their correctly rounded
// reciprocals are staged once per workgroup in LDS.
#include "codec.hpp"
#include "launch.hpp"

namespace kvq {

constexpr int kMaxHeadsLds = 256;

template <int FMT>
__device__ __forceinline__ uint2 quant8(uint4 w, float s, float rs) {
  uint2 o;
  o.x = enc4<FMT>(quotient(bf16lo(w.x), s, rs), quotient(bf16hi(w.x), s, rs),
                  quotient(bf16lo(w.y), s, rs), quotient(bf16hi(w.y), s, rs));
  o.y = enc4<FMT>(quotient(bf16lo(w.z), s, rs), quotient(bf16hi(w.z), s, rs),
                  quotient(bf16lo(w.w), s, rs), quotient(bf16hi(w.w), s, rs));
  return o;
}

template <int FMT>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint32_t units, int Hkv,
    int cpr_shift, const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, int64_t num_slots, const float* __restrict__ ks,
    const float* __restrict__ vs, int per_head) {
  __shared__ float s_k[kMaxHeadsLds], r_k[kMaxHeadsLds], s_v[kMaxHeadsLds], r_v[kMaxHeadsLds];
  const int nh = per_head ? Hkv : 1;
  for (int i = threadIdx.x; i < nh; i += blockDim.x) {
    float a = ks[i], b = vs[i];
    s_k[i] = a;
    r_k[i] = recip_rn(a);
    s_v[i] = b;
    r_v[i] = recip_rn(b);
  }
  __syncthreads();
  const int cpr = 1 << cpr_shift;  // 16-byte chunks per (token, head) row
  const int dh = cpr * 8;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < units; u += stride) {
    const uint32_t c = u & (cpr - 1);
    const uint32_t row = u >> cpr_shift;  // t * Hkv + h
    const uint32_t t = row / (uint32_t)Hkv;
    const int h = (int)(row - t * (uint32_t)Hkv);
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots) continue;
    const size_t src = (size_t)row * dh + c * 8;
    uint4 wk = *reinterpret_cast<const uint4*>(k + src);
    uint4 wv = *reinterpret_cast<const uint4*>(v + src);
    const int hs = per_head ? h : 0;
    const int64_t blk = slot >> 4, off = slot & 15;  // bs == 16
    const size_t dst = (size_t)(((blk * Hkv + h) * 16 + off) * dh) + c * 8;
    *reinterpret_cast<uint2*>(kc + dst) = quant8<FMT>(wk, s_k[hs], r_k[hs]);
    *reinterpret_cast<uint2*>(vc + dst) = quant8<FMT>(wv, s_v[hs], r_v[hs]);
  }
}

hipError_t launch_cache_write(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                              const int64_t* slot, uint8_t* kc, uint8_t* vc, int64_t num_blocks,
                              const float* ks, const float* vs, int fmt, int per_head,
                              hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int cpr = dh >> 3;
  int cpr_shift = 0;
  while ((1 << cpr_shift) < cpr) ++cpr_shift;
  const uint32_t units = (uint32_t)(T * Hkv * cpr);
  int64_t want = ((int64_t)units + 255) / 256;
  int64_t cap = (int64_t)device_cu_count() * 16;
  int grid = (int)(want < cap ? want : cap);
  const int64_t num_slots = num_blocks * 16;
  if (fmt == E4M3)
    cache_write_kernel<E4M3><<<grid, 256, 0, s>>>(k, v, units, Hkv, cpr_shift, slot, kc, vc,
                                                   num_slots, ks, vs, per_head);
  else
    cache_write_kernel<E5M2><<<grid, 256, 0, s>>>(k, v, units, Hkv, cpr_shift, slot, kc, vc,
                                                   num_slots, ks, vs, per_head);
  return hipGetLastError();
}

}  // namespace kvq

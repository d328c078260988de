// calibrate.hip -- amax reduction and scale derivation.
//
// Per-tensor or per-head scale calibration (KV-cache quantization textbook,
// section 10.4.3 granularity table; vLLM FP8 KV-cache guide, scale shapes and
// scale sources): amax = max |x| over the set, scale = amax / fmax.
//
// Design: |x| of a bf16 value is its bit pattern with the sign cleared, and
// for non-negative floats the integer order of the bit patterns is the
// numeric order (NaN patterns sort above +Inf).  So the whole reduction is an
// exact, order-free integer max: packed 16-bit max in registers, a workgroup
// max per head through LDS atomics and one global atomicMax per (workgroup,
// head) on the fp32 image (bf16 bits << 16).  Three launches on the
// caller's stream: clear (unless accumulating), reduce, finalize.
#include "codec.hpp"
#include "launch.hpp"

namespace kvq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// up to two tensors per launch (K and V calibrated together share every
// launch); tensor j's arrays are amax[j] / scale[j]
struct CalibArrays {
  uint32_t* amax[2];
  float* scale[2];
};

__global__ void amax_clear_kernel(CalibArrays a, int n, int ntensors) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n * ntensors) a.amax[i / n][i % n] = 0u;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

static int64_t gcd64(int64_t a, int64_t b) {
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return a;
}

// Packed |x| max over one 16-byte chunk (8 bf16) -> a pair of u16 maxima.
__device__ __forceinline__ u16x2 absmax8(uint4 w) {
  const uint32_t m = 0x7fff7fffu;
  u16x2 a = __builtin_bit_cast(u16x2, w.x & m), b = __builtin_bit_cast(u16x2, w.y & m);
  u16x2 c = __builtin_bit_cast(u16x2, w.z & m), d = __builtin_bit_cast(u16x2, w.w & m);
  return __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                   __builtin_elementwise_max(c, d));
}

// grid (gx), 256 threads: a flat grid-stride scan over the tensor's 16-byte
// chunks (8 bf16), consecutive threads on consecutive chunks, so every wave
// reads 1 KB of contiguous memory per load.  The stride is a multiple of the
// chunks per token (H * dh / 8), so each thread always lands on the same head
// h = (chunk / (dh / 8)) % H and keeps one running max; the heads are then
// reduced in LDS, one atomicMax per (workgroup, slot).
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x,
                                                   int64_t nchunks, int H, int dh, int per_head,
                                                   int64_t stride, uint32_t* __restrict__ amax) {
  __shared__ uint32_t red[256];  // per head (per_head) or one slot
  const int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = dh >> 3;  // chunks per (token, head) row
  const int h = (int)((c0 / cpr) % H);
  for (int i = threadIdx.x; i < 256; i += 256) red[i] = 0u;
  const uint4* src = reinterpret_cast<const uint4*>(x);
  u16x2 acc = {0, 0};
  int64_t c = c0;
  // four chunks in flight per thread
  for (; c + 3 * stride < nchunks; c += 4 * stride) {
    const uint4 w0 = src[c], w1 = src[c + stride], w2 = src[c + 2 * stride],
                w3 = src[c + 3 * stride];
    acc = __builtin_elementwise_max(
        acc, __builtin_elementwise_max(__builtin_elementwise_max(absmax8(w0), absmax8(w1)),
                                       __builtin_elementwise_max(absmax8(w2), absmax8(w3))));
  }
  for (; c < nchunks; c += stride) acc = __builtin_elementwise_max(acc, absmax8(src[c]));
  const uint32_t m = umax(acc.x, acc.y);
  if (per_head && H > 256) {  // more heads than LDS slots: straight to memory
    if (m) atomicMax(amax + h, m << 16);
    return;
  }
  __syncthreads();
  if (m) atomicMax(&red[per_head ? h : 0], m);  // LDS atomic: workgroup-local
  __syncthreads();
  const int nslot = per_head ? H : 1;
  for (int i = threadIdx.x; i < nslot; i += 256)
    if (red[i]) atomicMax(amax + i, red[i] << 16);
}

// The same reduction with each workgroup on one contiguous range of the
// tensor (a plain streaming read, like a copy's): the tensor is cut into units
// of 256 J chunks, J = lcm(chunks per token, 256) / 256 in {1, 2, 4}, and
// workgroup w scans units [w U / G, (w + 1) U / G).  Thread t reads chunks
// t + 256 j of each unit, whose head ((t + 256 j) / cpr) % H is the same in
// every unit since a unit holds whole tokens; it keeps one running max per j.
// kUnitsPerStep units are read per step (that many J loads in flight per
// thread), with nontemporal loads: every byte is read once.  One workgroup
// per CU, each streaming one long range with eight loads in flight per
// thread, reads fastest: 43.3 us per 269 MB tensor against 53.7 us with 8
// workgroups per CU and four loads in flight (45.8 us at 2 per CU, 52.4 us at
// 1 per CU with four loads; sixteen loads time as eight).
constexpr int kUnitsPerStep = 8;

template <int J>
__global__ __launch_bounds__(256) void amax_contig_kernel(const uint16_t* __restrict__ x0,
                                                          const uint16_t* __restrict__ x1,
                                                          int64_t nchunks, int64_t nunits,
                                                          int H, int dh, int per_head,
                                                          CalibArrays arr, uint32_t gpt) {
  __shared__ uint32_t red[256];
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  // gpt workgroups per tensor: the first gpt scan x0, the next gpt x1
  const uint32_t tj = blockIdx.x / gpt, wb = blockIdx.x - tj * gpt;
  const uint16_t* __restrict__ x = tj ? x1 : x0;
  uint32_t* __restrict__ amax = arr.amax[tj];
  const int t = threadIdx.x;
  red[t] = 0u;
  const int cpr = dh >> 3;
  const int64_t u0 = nunits * wb / gpt, u1 = nunits * (wb + 1) / gpt;
  const u32x4* src = reinterpret_cast<const u32x4*>(x);
  u16x2 acc[J];
#pragma unroll
  for (int j = 0; j < J; ++j) acc[j] = u16x2{0, 0};
  auto chunk = [&](int64_t u, int j) { return u * (256 * J) + 256 * j + t; };
  auto absmax8v = [&](u32x4 v) { return absmax8(make_uint4(v.x, v.y, v.z, v.w)); };
  int64_t u = u0;
  // whole units strictly inside the tensor, kUnitsPerStep at a time
  const int64_t full = nchunks / (256 * J);  // units lying entirely inside the tensor
  const int64_t uf = u1 < full ? u1 : full;
  for (; u + kUnitsPerStep - 1 < uf; u += kUnitsPerStep) {
    u32x4 w[kUnitsPerStep][J];
#pragma unroll
    for (int k = 0; k < kUnitsPerStep; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j) w[k][j] = __builtin_nontemporal_load(src + chunk(u + k, j));
#pragma unroll
    for (int k = 0; k < kUnitsPerStep; ++k)
#pragma unroll
      for (int j = 0; j < J; ++j) acc[j] = __builtin_elementwise_max(acc[j], absmax8v(w[k][j]));
  }
  for (; u < u1; ++u)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t c = chunk(u, j);
      if (c < nchunks) acc[j] = __builtin_elementwise_max(acc[j], absmax8v(src[c]));
    }
  __syncthreads();  // red[] cleared
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint32_t m = umax(acc[j].x, acc[j].y);
    const int h = per_head ? ((t + 256 * j) / cpr) % H : 0;
    if (m) atomicMax(&red[h], m);  // LDS atomic: workgroup-local
  }
  __syncthreads();
  const int nslot = per_head ? H : 1;
  for (int i = t; i < nslot; i += 256)
    if (red[i]) atomicMax(amax + i, red[i] << 16);
}

template <int FMT>
__global__ void scale_finalize_kernel(CalibArrays arr, int n, int ntensors) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n * ntensors) return;
  float* __restrict__ scale = arr.scale[i / n];
  const uint32_t* __restrict__ amax = arr.amax[i / n];
  i %= n;
  float a = __uint_as_float(amax[i]);
  // finite and > 0 -> correctly rounded amax / fmax; otherwise 1.0
  bool ok = a > 0.0f && a <= 3.4028234663852886e38f;
  scale[i] = ok ? __fdiv_rn(a, FmtTraits<FMT>::kMax) : 1.0f;
}

// x[j], amax_io[j], scale_out[j] for j < ntensors (1 or 2): every tensor has
// the shape [T][H][dh]; three launches in all (clear unless accumulating,
// reduce, finalize)
hipError_t launch_calibrate_n(const uint16_t* const* x, int ntensors, int64_t T, int H, int dh,
                              int fmt, int per_head, float* const* amax_io,
                              float* const* scale_out, int accumulate, hipStream_t s) {
  const int n = per_head ? H : 1;
  CalibArrays arr;
  for (int j = 0; j < 2; ++j) {
    const int jj = j < ntensors ? j : 0;
    arr.amax[j] = reinterpret_cast<uint32_t*>(amax_io[jj]);
    arr.scale[j] = scale_out[jj];
  }
  if (!accumulate)
    amax_clear_kernel<<<(n * ntensors + 255) / 256, 256, 0, s>>>(arr, n, ntensors);
  if (T > 0) {
    const int64_t nchunks = T * H * (dh >> 3);
    const int64_t cpt = (int64_t)H * (dh >> 3);  // chunks per token: the stride's unit
    const int64_t lcm = cpt % 256 == 0 ? cpt : cpt * 256 / gcd64(cpt, 256);
    const int J = (int)(lcm / 256);
    if ((J == 1 || J == 2 || J == 4) && (!per_head || H <= 256)) {
      // contiguous ranges: one workgroup per CU in all, at least one step of
      // units each
      const int64_t nunits = (nchunks + 256 * J - 1) / (256 * J);
      int64_t g = (int64_t)device_cu_count() / ntensors;
      if (g > (nunits + kUnitsPerStep - 1) / kUnitsPerStep)
        g = (nunits + kUnitsPerStep - 1) / kUnitsPerStep;
      if (g < 1) g = 1;
      const uint16_t* x1 = ntensors > 1 ? x[1] : x[0];
      const uint32_t grid = (uint32_t)(g * ntensors);
      if (J == 1)
        amax_contig_kernel<1><<<grid, 256, 0, s>>>(x[0], x1, nchunks, nunits, H, dh, per_head,
                                                   arr, (uint32_t)g);
      else if (J == 2)
        amax_contig_kernel<2><<<grid, 256, 0, s>>>(x[0], x1, nchunks, nunits, H, dh, per_head,
                                                   arr, (uint32_t)g);
      else
        amax_contig_kernel<4><<<grid, 256, 0, s>>>(x[0], x1, nchunks, nunits, H, dh, per_head,
                                                   arr, (uint32_t)g);
    } else {
      // about 8 workgroups per CU, the grid's thread count a multiple of cpt
      int64_t threads = (int64_t)device_cu_count() * 8 * 256;
      threads = (threads + lcm - 1) / lcm * lcm;
      const int64_t need = (nchunks + 255) / 256 * 256;
      if (threads > need) threads = (need + lcm - 1) / lcm * lcm;
      for (int j = 0; j < ntensors; ++j)
        amax_kernel<<<(uint32_t)(threads / 256), 256, 0, s>>>(x[j], nchunks, H, dh, per_head,
                                                              threads, arr.amax[j]);
    }
  }
  dispatch_fmt(fmt, [&](auto f) {
    scale_finalize_kernel<decltype(f)::value>
        <<<(n * ntensors + 255) / 256, 256, 0, s>>>(arr, n, ntensors);
  });
  return hipGetLastError();
}

hipError_t launch_calibrate(const uint16_t* x, int64_t T, int H, int dh, int fmt, int per_head,
                            float* amax_io, float* scale_out, int accumulate, hipStream_t s) {
  return launch_calibrate_n(&x, 1, T, H, dh, fmt, per_head, &amax_io, &scale_out, accumulate, s);
}

}  // namespace kvq

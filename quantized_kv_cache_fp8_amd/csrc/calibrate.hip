// calibrate.hip -- amax reduction and scale derivation.
//
// Per-tensor or per-head scale calibration (KV-cache quantization textbook,
// section 10.4.3 granularity table; vLLM FP8 KV-cache guide, scale shapes and
// scale sources): amax = max |x| over the set, scale = amax / fmax.
//
// Design: |x| of a bf16 value is its bit pattern with the sign cleared, and
// for non-negative floats the integer order of the bit patterns is the
// numeric order (NaN patterns sort above +Inf).  So the whole reduction is an
// exact, order-free integer max: packed 16-bit max in registers, a wave max
// through DPP, a workgroup max through LDS and one global atomicMax per
// workgroup on the fp32 image (bf16 bits << 16).  Three launches on the
// caller's stream: clear (unless accumulating), reduce, finalize.
#include "codec.hpp"
#include "launch.hpp"

namespace kvq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__global__ void amax_clear_kernel(uint32_t* amax, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) amax[i] = 0u;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Packed |x| max over one 16-byte chunk (8 bf16) -> a pair of u16 maxima.
__device__ __forceinline__ u16x2 absmax8(uint4 w) {
  const uint32_t m = 0x7fff7fffu;
  u16x2 a = __builtin_bit_cast(u16x2, w.x & m), b = __builtin_bit_cast(u16x2, w.y & m);
  u16x2 c = __builtin_bit_cast(u16x2, w.z & m), d = __builtin_bit_cast(u16x2, w.w & m);
  return __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                   __builtin_elementwise_max(c, d));
}

// grid (gx, H); 256 threads.  Workgroup (x, h) scans rows t = x*rpi + r, ...
// of head h.  A row (t, h) is dh contiguous bf16 = dh/8 16-byte chunks.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                   int H, int dh, int per_head,
                                                   uint32_t* __restrict__ amax) {
  __shared__ uint32_t red[4];
  const int h = blockIdx.y;
  const int cpr = dh >> 3;             // chunks per row
  const int rpi = 256 / cpr;           // rows per workgroup step
  const int r = threadIdx.x / cpr, c = threadIdx.x % cpr;
  u16x2 acc = {0, 0};
  if (r < rpi) {
    const int64_t step = (int64_t)gridDim.x * rpi;
    int64_t t = (int64_t)blockIdx.x * rpi + r;
    // two rows in flight per thread
    for (; t + step < T; t += 2 * step) {
      uint4 w0 = *reinterpret_cast<const uint4*>(x + ((t * H + h) * dh + c * 8));
      uint4 w1 = *reinterpret_cast<const uint4*>(x + (((t + step) * H + h) * dh + c * 8));
      acc = __builtin_elementwise_max(acc, __builtin_elementwise_max(absmax8(w0), absmax8(w1)));
    }
    if (t < T) {
      uint4 w0 = *reinterpret_cast<const uint4*>(x + ((t * H + h) * dh + c * 8));
      acc = __builtin_elementwise_max(acc, absmax8(w0));
    }
  }
  uint32_t m = umax(acc.x, acc.y);
  // wave max (64 lanes)
  for (int off = 32; off >= 1; off >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = umax(umax(red[0], red[1]), umax(red[2], red[3]));
    if (m) atomicMax(amax + (per_head ? h : 0), m << 16);
  }
}

template <int FMT>
__global__ void scale_finalize_kernel(const uint32_t* __restrict__ amax, float* __restrict__ scale,
                                      int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float a = __uint_as_float(amax[i]);
  // finite and > 0 -> correctly rounded amax / fmax; otherwise 1.0
  bool ok = a > 0.0f && a <= 3.4028234663852886e38f;
  scale[i] = ok ? __fdiv_rn(a, FmtTraits<FMT>::kMax) : 1.0f;
}

hipError_t launch_calibrate(const uint16_t* x, int64_t T, int H, int dh, int fmt, int per_head,
                            float* amax_io, float* scale_out, int accumulate, hipStream_t s) {
  const int n = per_head ? H : 1;
  uint32_t* amax = reinterpret_cast<uint32_t*>(amax_io);
  if (!accumulate) amax_clear_kernel<<<(n + 255) / 256, 256, 0, s>>>(amax, n);
  if (T > 0) {
    const int rpi = 256 / (dh >> 3);
    int64_t rows_wg = (T + rpi - 1) / rpi;  // workgroups that would each take one step
    int64_t target = (int64_t)device_cu_count() * 8 / H;
    if (target < 1) target = 1;
    int gx = (int)(rows_wg < target ? rows_wg : target);
    amax_kernel<<<dim3(gx, H), 256, 0, s>>>(x, T, H, dh, per_head, amax);
  }
  dispatch_fmt(fmt, [&](auto f) {
    scale_finalize_kernel<decltype(f)::value><<<(n + 255) / 256, 256, 0, s>>>(amax, scale_out, n);
  });
  return hipGetLastError();
}

}  // namespace kvq

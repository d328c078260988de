// codec_kernels.hip -- standalone element encode / decode over flat arrays.
// These run exactly the device codec that the cache kernels inline
// (codec.hpp), so an exhaustive sweep through them checks that codec.
#include "codec.hpp"
#include "launch.hpp"

namespace kvq {

template <int FMT>
__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ x, int64_t n,
                                                     uint8_t* __restrict__ out) {
  // four elements per thread per step; the ragged tail is handled per element
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      float4 v = *reinterpret_cast<const float4*>(x + i);
      *reinterpret_cast<uint32_t*>(out + i) = enc4<FMT>(v.x, v.y, v.z, v.w);
    } else {
      for (int64_t j = i; j < n; ++j) out[j] = (uint8_t)enc2<FMT>(x[j], 0.0f);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void decode_kernel(const uint8_t* __restrict__ c, int64_t n,
                                                     float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 4;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n; i += stride) {
    if (i + 4 <= n) {
      uint32_t w = *reinterpret_cast<const uint32_t*>(c + i);
      f32x2 a = dec2_f32<FMT, false>(w), b = dec2_f32<FMT, true>(w);
      *reinterpret_cast<float4*>(out + i) = make_float4(a.x, a.y, b.x, b.y);
    } else {
      for (int64_t j = i; j < n; ++j) out[j] = dec2_f32<FMT, false>((uint32_t)c[j]).x;
    }
  }
}

static int flat_grid(int64_t n) {
  int64_t want = (n + 1023) / 1024;
  int64_t cap = (int64_t)device_cu_count() * 16;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

hipError_t launch_fp8_encode(int fmt, const float* x, int64_t n, uint8_t* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  dispatch_fmt(fmt, [&](auto f) {
    encode_kernel<decltype(f)::value><<<flat_grid(n), 256, 0, s>>>(x, n, out);
  });
  return hipGetLastError();
}

hipError_t launch_fp8_decode(int fmt, const uint8_t* c, int64_t n, float* out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  dispatch_fmt(fmt, [&](auto f) {
    decode_kernel<decltype(f)::value><<<flat_grid(n), 256, 0, s>>>(c, n, out);
  });
  return hipGetLastError();
}

}  // namespace kvq

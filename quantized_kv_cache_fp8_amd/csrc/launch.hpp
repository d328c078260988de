// launch.hpp -- host-side launchers shared between the C ABI layer (api.hip)
// and the kernel translation units.  Arguments have been validated by the
// caller; each launcher only sizes the grid and enqueues kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

// Compute units of the current device (cached per device).
int device_cu_count();

hipError_t launch_fp8_encode(int fmt, const float* x, int64_t n, uint8_t* out, hipStream_t s);
hipError_t launch_fp8_decode(int fmt, const uint8_t* c, int64_t n, float* out, hipStream_t s);

hipError_t launch_calibrate(const uint16_t* x, int64_t T, int H, int dh, int fmt, int per_head,
                            float* amax_io, float* scale_out, int accumulate, hipStream_t s);
// the same for ntensors (1 or 2) tensors of one shape, sharing every launch
hipError_t launch_calibrate_n(const uint16_t* const* x, int ntensors, int64_t T, int H, int dh,
                              int fmt, int per_head, float* const* amax_io,
                              float* const* scale_out, int accumulate, hipStream_t s);

hipError_t launch_cache_write(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                              const int64_t* slot, uint8_t* kc, uint8_t* vc, int64_t num_blocks,
                              const float* ks, const float* vs, int fmt, int per_head,
                              hipStream_t s, int64_t bstride = 0);

// bstride: bytes from one cache block to the next in k_cache and in v_cache
// (0 = the natural Hkv * 16 * dh; larger = pages padded to a common size).

// Quantize-on-write with one fp16 scale per (token, KV head) for K and for V,
// computed from the row's own amax; ksc/vsc are [num_blocks][Hkv][16] caches.
hipError_t launch_cache_write_token(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv,
                                    int dh, const int64_t* slot, uint8_t* kc, uint8_t* vc,
                                    uint16_t* ksc, uint16_t* vsc, int64_t num_blocks, int fmt,
                                    hipStream_t s, int64_t bstride = 0);

// Split-K decode geometry, shared by the workspace query and the launch.
struct DecodePlan {
  int part_blocks;  // cache blocks per split
  int nsplit;       // splits per sequence
  size_t ws_bytes;  // workspace bytes
};
DecodePlan decode_plan(int B, int Hq, int dh, int max_context_len, int bs);

hipError_t launch_decode(void* out, int out_bf16, const uint16_t* q, const uint8_t* kc,
                         const uint8_t* vc, int64_t num_blocks, const int32_t* bt,
                         int max_blocks, const int32_t* ctx, int B, int Hq, int Hkv, int dh,
                         int max_ctx, const float* ks, const float* vs, int fmt, int per_head,
                         float softmax_scale, const DecodePlan& plan, void* ws, hipStream_t s,
                         const uint16_t* ksc = nullptr, const uint16_t* vsc = nullptr,
                         int64_t bstride = 0, const uint16_t* k_new = nullptr,
                         const uint16_t* v_new = nullptr, uint8_t* kc_w = nullptr,
                         uint8_t* vc_w = nullptr);

// Bytes of the device-resident scratch array the allocation-free decode
// entry point keeps its split partials in (one array per GPU).
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
// That array's device address on the current device, looked up once per
// device (null if the lookup fails).
void* decode_static_scratch();

// Log-sum-exp merge of split partials ([B][Hq][nsplit] (m, l) pairs and dh
// partial sums) into out, times vs (null: 1).  part_blocks > 0: sequence b's
// first ceil(ctx / (16 part_blocks)) splits are merged; 0: all nsplit are.
void launch_decode_combine(void* out, int out_bf16, const float* ml, const float* acc,
                           const int32_t* ctx, int B, int Hq, int Hkv, int dh, int max_ctx,
                           const float* vs, int per_head, int part_blocks, int nsplit,
                           hipStream_t s);

// KIVI-style 2-bit cache (dh = 128, 32-token blocks, 3072-byte tiles).
hipError_t launch_kivi_quantize(const uint16_t* k, const uint16_t* v, int64_t n_groups, int Hkv,
                                const int32_t* group_blocks, uint8_t* cache, int64_t num_blocks,
                                hipStream_t s);
struct KiviPlan {
  int groups_per_split;  // 32-token groups per quantized split
  int nsplit;            // splits per sequence: the residual's, then the quantized ones
  size_t ws_bytes;       // workspace bytes
};
KiviPlan kivi_decode_plan(int B, int Hq, int Hkv, int max_groups);
hipError_t launch_kivi_decode(void* out, int out_bf16, const uint16_t* q, const uint8_t* cache,
                              int64_t num_blocks, const int32_t* bt, int max_blocks,
                              const int32_t* quant_groups, int max_groups, const uint16_t* res_k,
                              const uint16_t* res_v, const int32_t* res_lens, int R, int B,
                              int Hq, int Hkv, float softmax_scale, const KiviPlan& plan,
                              void* ws, hipStream_t s);

hipError_t launch_prefill(void* out, int out_bf16, const uint16_t* q, const int32_t* cu,
                          int max_q_len, const float* qs, int q_per_head, const uint8_t* kc,
                          const uint8_t* vc, int64_t num_blocks, const int32_t* bt,
                          int max_blocks, const int32_t* ctx, int B, int Hq, int Hkv, int dh,
                          const float* ks, const float* vs, int fmt, int kv_per_head,
                          float softmax_scale, hipStream_t s, int64_t bstride = 0);

}  // namespace kvq

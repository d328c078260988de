// api.hip -- the extern "C" entry points declared in include/kvq.h.
//
// Every entry point validates its arguments on the host before any HIP call
// (so invalid calls are cheap, deterministic and touch no device state), then
// hands a launch to the kernel translation units.  Status mapping:
// hipErrorNoDevice / wrong architecture -> KVQ_ERR_DEVICE, any other launch
// error -> KVQ_ERR_LAUNCH.
#include <string.h>

#include <mutex>

#include "../../include/kvq.h"
#include "launch.hpp"

namespace kvq {

namespace {
constexpr int kMaxDevices = 64;
int g_cu[kMaxDevices];
std::once_flag g_once[kMaxDevices];
}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  std::call_once(g_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    g_cu[dev] = n;
  });
  return g_cu[dev];
}

static kvq_status map_err(hipError_t e) {
  if (e == hipSuccess) return KVQ_OK;
  if (e == hipErrorNoDevice || e == hipErrorInvalidDevice || e == hipErrorNoBinaryForGpu ||
      e == hipErrorInvalidDeviceFunction)
    return KVQ_ERR_DEVICE;
  return KVQ_ERR_LAUNCH;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
static bool fmt_ok(int f) {
  return f == KVQ_FMT_E4M3 || f == KVQ_FMT_E5M2 || f == KVQ_FMT_INT8;
}
static bool gran_ok(int g) { return g == KVQ_SCALE_TENSOR || g == KVQ_SCALE_HEAD; }
static bool out_ok(int o) { return o == KVQ_OUT_F32 || o == KVQ_OUT_BF16; }
static bool dh_ok(int dh) { return dh == 64 || dh == 128; }

}  // namespace kvq

using namespace kvq;

extern "C" {

const char* kvq_strerror(int st) {
  switch (st) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "a required pointer is NULL";
    case KVQ_ERR_SHAPE: return "invalid or inconsistent sizes";
    case KVQ_ERR_UNSUPPORTED: return "unsupported value (dh, block size, group size, format, "
                                     "granularity, output type or alignment)";
    case KVQ_ERR_WORKSPACE: return "decode workspace too small";
    case KVQ_ERR_LAUNCH: return "HIP kernel launch failed";
    case KVQ_ERR_DEVICE: return "no usable gfx950 HIP device";
    case KVQ_ERR_SCRATCH: return "the call needs more split-partial bytes than the library's "
                                 "static scratch array holds (KVQ_STATIC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

uint64_t kvq_kv_cache_bytes(int L, int B, int Hkv, int64_t S, int dh, int bits_per_elem) {
  if (L < 0 || B < 0 || Hkv < 0 || S < 0 || dh < 0 || bits_per_elem < 0) return 0;
  return 2ull * (uint64_t)L * (uint64_t)B * (uint64_t)Hkv * (uint64_t)S * (uint64_t)dh *
         (uint64_t)bits_per_elem / 8ull;
}

kvq_status kvq_fp8_encode(int fmt, const float* x, int64_t n, uint8_t* out,
                          kvq_stream stream) {
  if (!fmt_ok(fmt)) return KVQ_ERR_UNSUPPORTED;
  if (n < 0) return KVQ_ERR_SHAPE;
  if (n == 0) return KVQ_OK;
  if (!x || !out) return KVQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out, 4)) return KVQ_ERR_UNSUPPORTED;
  return map_err(launch_fp8_encode(fmt, x, n, out, (hipStream_t)stream));
}

kvq_status kvq_fp8_decode(int fmt, const uint8_t* codes, int64_t n, float* out,
                          kvq_stream stream) {
  if (!fmt_ok(fmt)) return KVQ_ERR_UNSUPPORTED;
  if (n < 0) return KVQ_ERR_SHAPE;
  if (n == 0) return KVQ_OK;
  if (!codes || !out) return KVQ_ERR_NULL;
  if (!aligned(codes, 4) || !aligned(out, 16)) return KVQ_ERR_UNSUPPORTED;
  return map_err(launch_fp8_decode(fmt, codes, n, out, (hipStream_t)stream));
}

kvq_status kvq_calibrate_scales(const void* x_bf16, int64_t T, int H, int dh, int fmt,
                                int gran, float* amax_io, float* scale_out, int accumulate,
                                kvq_stream stream) {
  if (!fmt_ok(fmt) || !gran_ok(gran)) return KVQ_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || H > 65535 || dh < 8 || dh % 8 || dh > 2048) return KVQ_ERR_SHAPE;
  if (!amax_io || !scale_out || (T > 0 && !x_bf16)) return KVQ_ERR_NULL;
  if (T > 0 && !aligned(x_bf16, 16)) return KVQ_ERR_UNSUPPORTED;
  return map_err(launch_calibrate((const uint16_t*)x_bf16, T, H, dh, fmt,
                                  gran == KVQ_SCALE_HEAD, amax_io, scale_out, accumulate,
                                  (hipStream_t)stream));
}

kvq_status kvq_calibrate_scales_kv(const void* k_bf16, const void* v_bf16, int64_t T, int H,
                                   int dh, int fmt, int gran, float* k_amax_io, float* v_amax_io,
                                   float* k_scale_out, float* v_scale_out, int accumulate,
                                   kvq_stream stream) {
  if (!fmt_ok(fmt) || !gran_ok(gran)) return KVQ_ERR_UNSUPPORTED;
  if (T < 0 || H < 1 || H > 65535 || dh < 8 || dh % 8 || dh > 2048) return KVQ_ERR_SHAPE;
  if (!k_amax_io || !v_amax_io || !k_scale_out || !v_scale_out) return KVQ_ERR_NULL;
  if (T > 0 && (!k_bf16 || !v_bf16)) return KVQ_ERR_NULL;
  if (T > 0 && (!aligned(k_bf16, 16) || !aligned(v_bf16, 16))) return KVQ_ERR_UNSUPPORTED;
  const uint16_t* x[2] = {(const uint16_t*)k_bf16, (const uint16_t*)v_bf16};
  float* amax[2] = {k_amax_io, v_amax_io};
  float* scale[2] = {k_scale_out, v_scale_out};
  return map_err(launch_calibrate_n(x, 2, T, H, dh, fmt, gran == KVQ_SCALE_HEAD, amax, scale,
                                    accumulate, (hipStream_t)stream));
}

// block_stride: validated against the natural Hkv * bs * dh after the sizes
static kvq_status check_stride(int64_t block_stride, int Hkv, int bs, int dh) {
  if (block_stride < (int64_t)Hkv * bs * dh) return KVQ_ERR_SHAPE;
  if (block_stride % 16) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status kvq_cache_write(const void* k_bf16, const void* v_bf16, int64_t T, int Hkv, int dh,
                           const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                           int64_t num_blocks, int bs, const float* k_scale,
                           const float* v_scale, int fmt, int gran,
                           kvq_stream stream) {
  return kvq_cache_write_paged(k_bf16, v_bf16, T, Hkv, dh, slot_mapping, k_cache, v_cache,
                               num_blocks, bs, (int64_t)Hkv * bs * dh, k_scale, v_scale, fmt,
                               gran, stream);
}

kvq_status kvq_cache_write_paged(const void* k_bf16, const void* v_bf16, int64_t T, int Hkv,
                                 int dh, const int64_t* slot_mapping, uint8_t* k_cache,
                                 uint8_t* v_cache, int64_t num_blocks, int bs,
                                 int64_t block_stride, const float* k_scale,
                                 const float* v_scale, int fmt, int gran,
                                 kvq_stream stream) {
  if (!fmt_ok(fmt) || !gran_ok(gran)) return KVQ_ERR_UNSUPPORTED;
  if (T < 0 || Hkv < 1 || num_blocks < 1) return KVQ_ERR_SHAPE;
  if (!dh_ok(dh) || bs != 16 || Hkv > 256) return KVQ_ERR_UNSUPPORTED;
  const kvq_status sst = check_stride(block_stride, Hkv, bs, dh);
  if (sst != KVQ_OK) return sst;
  if ((uint64_t)T * (uint64_t)Hkv * (uint64_t)(dh / 8) >= (1ull << 32)) return KVQ_ERR_SHAPE;
  if (!k_cache || !v_cache || !k_scale || !v_scale) return KVQ_ERR_NULL;
  if (T == 0) return KVQ_OK;
  if (!k_bf16 || !v_bf16 || !slot_mapping) return KVQ_ERR_NULL;
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 8) || !aligned(slot_mapping, 8))
    return KVQ_ERR_UNSUPPORTED;
  return map_err(launch_cache_write((const uint16_t*)k_bf16, (const uint16_t*)v_bf16, T, Hkv, dh,
                                    slot_mapping, k_cache, v_cache, num_blocks, k_scale, v_scale,
                                    fmt, gran == KVQ_SCALE_HEAD, (hipStream_t)stream,
                                    block_stride));
}

size_t kvq_decode_workspace_size(int B, int Hq, int dh, int max_context_len, int bs) {
  return decode_plan(B, Hq, dh, max_context_len, bs).ws_bytes;
}

static kvq_status check_attn_common(const void* out, int out_dtype, const void* q,
                                    const uint8_t* kc, const uint8_t* vc, int64_t num_blocks,
                                    const int32_t* bt, int max_blocks, const int32_t* ctx, int B,
                                    int Hq, int Hkv, int dh, int bs, const void* ks,
                                    const void* vs, int fmt, int gran) {
  if (!fmt_ok(fmt) || !gran_ok(gran) || !out_ok(out_dtype)) return KVQ_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1) return KVQ_ERR_SHAPE;
  if (Hq % Hkv) return KVQ_ERR_SHAPE;
  if (!dh_ok(dh) || bs != 16 || Hq / Hkv > 16 || B > 65535) return KVQ_ERR_UNSUPPORTED;
  if (!out || !q || !kc || !vc || !bt || !ctx || !ks || !vs) return KVQ_ERR_NULL;
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16))
    return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

static kvq_status check_decode_ws(const DecodePlan& plan, int max_context_len, int max_blocks,
                                  int bs, const void* workspace, size_t ws_bytes) {
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks * bs)
    return KVQ_ERR_SHAPE;
  if (plan.nsplit > 65535) return KVQ_ERR_UNSUPPORTED;
  if (!workspace) return KVQ_ERR_NULL;
  if (ws_bytes < plan.ws_bytes) return KVQ_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status kvq_decode_attn(void* out, int out_dtype, const void* q_bf16,
                           const uint8_t* k_cache, const uint8_t* v_cache, int64_t num_blocks,
                           const int32_t* block_tables, int max_blocks,
                           const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                           int max_context_len, const float* k_scale, const float* v_scale,
                           int fmt, int gran, float softmax_scale, void* workspace,
                           size_t ws_bytes, kvq_stream stream) {
  return kvq_decode_attn_paged(out, out_dtype, q_bf16, k_cache, v_cache, num_blocks, block_tables,
                               max_blocks, context_lens, B, Hq, Hkv, dh, bs,
                               (int64_t)Hkv * bs * dh, max_context_len, k_scale, v_scale, fmt,
                               gran, softmax_scale, workspace, ws_bytes, stream);
}

kvq_status kvq_decode_attn_paged(void* out, int out_dtype, const void* q_bf16,
                                 const uint8_t* k_cache, const uint8_t* v_cache,
                                 int64_t num_blocks, const int32_t* block_tables, int max_blocks,
                                 const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                                 int bs, int64_t block_stride, int max_context_len,
                                 const float* k_scale, const float* v_scale, int fmt,
                                 int gran, float softmax_scale, void* workspace,
                                 size_t ws_bytes, kvq_stream stream) {
  kvq_status st = check_attn_common(out, out_dtype, q_bf16, k_cache, v_cache, num_blocks,
                                    block_tables, max_blocks, context_lens, B, Hq, Hkv, dh, bs,
                                    k_scale, v_scale, fmt, gran);
  if (st != KVQ_OK) return st;
  st = check_stride(block_stride, Hkv, bs, dh);
  if (st != KVQ_OK) return st;
  const DecodePlan plan = decode_plan(B, Hq, dh, max_context_len, bs);
  st = check_decode_ws(plan, max_context_len, max_blocks, bs, workspace, ws_bytes);
  if (st != KVQ_OK) return st;
  return map_err(launch_decode(out, out_dtype == KVQ_OUT_BF16, (const uint16_t*)q_bf16, k_cache,
                               v_cache, num_blocks, block_tables, max_blocks, context_lens, B, Hq,
                               Hkv, dh, max_context_len, k_scale, v_scale, fmt,
                               gran == KVQ_SCALE_HEAD, softmax_scale, plan, workspace,
                               (hipStream_t)stream, nullptr, nullptr, block_stride));
}

// Validation of the append calls up to the workspace (sizes, pointers, the
// split plan's bounds); fills plan.
static kvq_status check_append(const void* out, int out_dtype, const void* q, const void* k_new,
                               const void* v_new, const uint8_t* kc, const uint8_t* vc,
                               int64_t num_blocks, const int32_t* bt, int max_blocks,
                               const int32_t* ctx, int B, int Hq, int Hkv, int dh, int bs,
                               int max_context_len, const float* ks, const float* vs, int fmt,
                               int gran, DecodePlan* plan) {
  kvq_status st = check_attn_common(out, out_dtype, q, kc, vc, num_blocks, bt, max_blocks, ctx,
                                    B, Hq, Hkv, dh, bs, ks, vs, fmt, gran);
  if (st != KVQ_OK) return st;
  if (!k_new || !v_new) return KVQ_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return KVQ_ERR_UNSUPPORTED;
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks * bs)
    return KVQ_ERR_SHAPE;
  *plan = decode_plan(B, Hq, dh, max_context_len, bs);
  if (plan->nsplit > 65535) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

static_assert(KVQ_STATIC_SCRATCH_BYTES == kStaticScratchBytes,
              "the header's scratch size must be the array's");

kvq_status kvq_decode_attn_append_noalloc(void* out, int out_dtype, const void* q_bf16,
                                          const void* k_new_bf16, const void* v_new_bf16,
                                          uint8_t* k_cache, uint8_t* v_cache, int64_t num_blocks,
                                          const int32_t* block_tables, int max_blocks,
                                          const int32_t* context_lens, int B, int Hq, int Hkv,
                                          int dh, int bs, int max_context_len,
                                          const float* k_scale, const float* v_scale,
                                          int fmt, int gran, float softmax_scale,
                                          kvq_stream stream) {
  DecodePlan plan;
  kvq_status st = check_append(out, out_dtype, q_bf16, k_new_bf16, v_new_bf16, k_cache, v_cache,
                               num_blocks, block_tables, max_blocks, context_lens, B, Hq, Hkv,
                               dh, bs, max_context_len, k_scale, v_scale, fmt, gran, &plan);
  if (st != KVQ_OK) return st;
  if (plan.ws_bytes > kStaticScratchBytes) return KVQ_ERR_SCRATCH;
  void* ws = decode_static_scratch();  // the array's address on this device
  if (!ws) return KVQ_ERR_DEVICE;
  return map_err(launch_decode(out, out_dtype == KVQ_OUT_BF16, (const uint16_t*)q_bf16, k_cache,
                               v_cache, num_blocks, block_tables, max_blocks, context_lens, B, Hq,
                               Hkv, dh, max_context_len, k_scale, v_scale, fmt,
                               gran == KVQ_SCALE_HEAD, softmax_scale, plan, ws,
                               (hipStream_t)stream, nullptr, nullptr, 0,
                               (const uint16_t*)k_new_bf16, (const uint16_t*)v_new_bf16, k_cache,
                               v_cache));
}

kvq_status kvq_decode_attn_append(void* out, int out_dtype, const void* q_bf16,
                                  const void* k_new_bf16, const void* v_new_bf16,
                                  uint8_t* k_cache, uint8_t* v_cache, int64_t num_blocks,
                                  const int32_t* block_tables, int max_blocks,
                                  const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                                  int bs, int max_context_len, const float* k_scale,
                                  const float* v_scale, int fmt, int gran,
                                  float softmax_scale, void* workspace, size_t ws_bytes,
                                  kvq_stream stream) {
  DecodePlan plan;
  kvq_status st = check_append(out, out_dtype, q_bf16, k_new_bf16, v_new_bf16, k_cache, v_cache,
                               num_blocks, block_tables, max_blocks, context_lens, B, Hq, Hkv,
                               dh, bs, max_context_len, k_scale, v_scale, fmt, gran, &plan);
  if (st != KVQ_OK) return st;
  st = check_decode_ws(plan, max_context_len, max_blocks, bs, workspace, ws_bytes);
  if (st != KVQ_OK) return st;
  return map_err(launch_decode(out, out_dtype == KVQ_OUT_BF16, (const uint16_t*)q_bf16, k_cache,
                               v_cache, num_blocks, block_tables, max_blocks, context_lens, B, Hq,
                               Hkv, dh, max_context_len, k_scale, v_scale, fmt,
                               gran == KVQ_SCALE_HEAD, softmax_scale, plan, workspace,
                               (hipStream_t)stream, nullptr, nullptr, 0,
                               (const uint16_t*)k_new_bf16, (const uint16_t*)v_new_bf16, k_cache,
                               v_cache));
}

kvq_status kvq_cache_write_token_scales(const void* k_bf16, const void* v_bf16, int64_t T,
                                        int Hkv, int dh, const int64_t* slot_mapping,
                                        uint8_t* k_cache, uint8_t* v_cache,
                                        uint16_t* k_scale_cache, uint16_t* v_scale_cache,
                                        int64_t num_blocks, int bs, int fmt,
                                        kvq_stream stream) {
  if (!fmt_ok(fmt)) return KVQ_ERR_UNSUPPORTED;
  if (T < 0 || Hkv < 1 || num_blocks < 1) return KVQ_ERR_SHAPE;
  if (!dh_ok(dh) || bs != 16 || Hkv > 256) return KVQ_ERR_UNSUPPORTED;
  if ((uint64_t)T * (uint64_t)Hkv * (uint64_t)(dh / 16) + 256 >= (1ull << 32))
    return KVQ_ERR_SHAPE;
  if (!k_cache || !v_cache || !k_scale_cache || !v_scale_cache) return KVQ_ERR_NULL;
  if (T == 0) return KVQ_OK;
  if (!k_bf16 || !v_bf16 || !slot_mapping) return KVQ_ERR_NULL;
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(k_scale_cache, 2) || !aligned(v_scale_cache, 2) ||
      !aligned(slot_mapping, 8))
    return KVQ_ERR_UNSUPPORTED;
  return map_err(launch_cache_write_token((const uint16_t*)k_bf16, (const uint16_t*)v_bf16, T,
                                          Hkv, dh, slot_mapping, k_cache, v_cache,
                                          k_scale_cache, v_scale_cache, num_blocks, fmt,
                                          (hipStream_t)stream));
}

kvq_status kvq_decode_attn_token_scales(void* out, int out_dtype, const void* q_bf16,
                                        const uint8_t* k_cache, const uint8_t* v_cache,
                                        const uint16_t* k_scale_cache,
                                        const uint16_t* v_scale_cache, int64_t num_blocks,
                                        const int32_t* block_tables, int max_blocks,
                                        const int32_t* context_lens, int B, int Hq, int Hkv,
                                        int dh, int bs, int max_context_len, int fmt,
                                        float softmax_scale, void* workspace, size_t ws_bytes,
                                        kvq_stream stream) {
  kvq_status st = check_attn_common(out, out_dtype, q_bf16, k_cache, v_cache, num_blocks,
                                    block_tables, max_blocks, context_lens, B, Hq, Hkv, dh, bs,
                                    k_scale_cache, v_scale_cache, fmt, KVQ_SCALE_TENSOR);
  if (st != KVQ_OK) return st;
  if (Hq / Hkv > 4) return KVQ_ERR_UNSUPPORTED;
  if (!aligned(k_scale_cache, 2) || !aligned(v_scale_cache, 2)) return KVQ_ERR_UNSUPPORTED;
  const DecodePlan plan = decode_plan(B, Hq, dh, max_context_len, bs);
  st = check_decode_ws(plan, max_context_len, max_blocks, bs, workspace, ws_bytes);
  if (st != KVQ_OK) return st;
  return map_err(launch_decode(out, out_dtype == KVQ_OUT_BF16, (const uint16_t*)q_bf16, k_cache,
                               v_cache, num_blocks, block_tables, max_blocks, context_lens, B, Hq,
                               Hkv, dh, max_context_len, nullptr, nullptr, fmt, 0, softmax_scale,
                               plan, workspace, (hipStream_t)stream, k_scale_cache,
                               v_scale_cache));
}

kvq_status kvq_kivi_quantize(const void* k_bf16, const void* v_bf16, int64_t n_groups, int Hkv,
                             int dh, const int32_t* group_blocks, uint8_t* kivi_cache,
                             int64_t num_blocks, kvq_stream stream) {
  if (n_groups < 0 || Hkv < 1 || num_blocks < 1) return KVQ_ERR_SHAPE;
  if (dh != 128) return KVQ_ERR_UNSUPPORTED;
  if ((uint64_t)n_groups * (uint64_t)Hkv >= (1ull << 31)) return KVQ_ERR_SHAPE;
  if (!kivi_cache) return KVQ_ERR_NULL;
  if (n_groups == 0) return KVQ_OK;
  if (!k_bf16 || !v_bf16 || !group_blocks) return KVQ_ERR_NULL;
  if (!aligned(k_bf16, 16) || !aligned(v_bf16, 16) || !aligned(kivi_cache, 16) ||
      !aligned(group_blocks, 4))
    return KVQ_ERR_UNSUPPORTED;
  return map_err(launch_kivi_quantize((const uint16_t*)k_bf16, (const uint16_t*)v_bf16, n_groups,
                                      Hkv, group_blocks, kivi_cache, num_blocks,
                                      (hipStream_t)stream));
}

size_t kvq_kivi_decode_workspace_size(int B, int Hq, int Hkv, int max_groups) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || max_groups < 0) return 0;
  return kivi_decode_plan(B, Hq, Hkv, max_groups).ws_bytes;
}

kvq_status kvq_kivi_decode_attn(void* out, int out_dtype, const void* q_bf16,
                                const uint8_t* kivi_cache, int64_t num_blocks,
                                const int32_t* block_tables, int max_blocks,
                                const int32_t* quant_groups, int max_groups,
                                const void* res_k_bf16, const void* res_v_bf16,
                                const int32_t* res_lens, int R, int B, int Hq, int Hkv, int dh,
                                float softmax_scale, void* workspace, size_t ws_bytes,
                                kvq_stream stream) {
  if (!out_ok(out_dtype)) return KVQ_ERR_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || num_blocks < 1 || max_blocks < 1 || R < 1)
    return KVQ_ERR_SHAPE;
  if (Hq % Hkv || max_groups < 0 || max_groups > max_blocks) return KVQ_ERR_SHAPE;
  if (dh != 128 || Hq / Hkv > 4 || R > 256 || B > 65535 || Hkv > 65535)
    return KVQ_ERR_UNSUPPORTED;
  if (!out || !q_bf16 || !kivi_cache || !block_tables || !quant_groups || !res_k_bf16 ||
      !res_v_bf16 || !res_lens || !workspace)
    return KVQ_ERR_NULL;
  if (!aligned(out, 16) || !aligned(q_bf16, 16) || !aligned(kivi_cache, 16) ||
      !aligned(res_k_bf16, 16) || !aligned(res_v_bf16, 16) || !aligned(workspace, 16))
    return KVQ_ERR_UNSUPPORTED;
  const KiviPlan plan = kivi_decode_plan(B, Hq, Hkv, max_groups);
  if (plan.nsplit > 65535) return KVQ_ERR_UNSUPPORTED;
  if (ws_bytes < plan.ws_bytes) return KVQ_ERR_WORKSPACE;
  return map_err(launch_kivi_decode(out, out_dtype == KVQ_OUT_BF16, (const uint16_t*)q_bf16,
                                    kivi_cache, num_blocks, block_tables, max_blocks,
                                    quant_groups, max_groups, (const uint16_t*)res_k_bf16,
                                    (const uint16_t*)res_v_bf16, res_lens, R, B, Hq, Hkv,
                                    softmax_scale, plan, workspace, (hipStream_t)stream));
}

kvq_status kvq_prefill_attn(void* out, int out_dtype, const void* q_bf16,
                            const int32_t* cu_seqlens_q, int max_q_len, const float* q_scale,
                            int q_gran, const uint8_t* k_cache, const uint8_t* v_cache,
                            int64_t num_blocks, const int32_t* block_tables, int max_blocks,
                            const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                            const float* k_scale, const float* v_scale, int fmt,
                            int kv_gran, float softmax_scale, kvq_stream stream) {
  return kvq_prefill_attn_paged(out, out_dtype, q_bf16, cu_seqlens_q, max_q_len, q_scale, q_gran,
                                k_cache, v_cache, num_blocks, block_tables, max_blocks,
                                context_lens, B, Hq, Hkv, dh, bs, (int64_t)Hkv * bs * dh, k_scale,
                                v_scale, fmt, kv_gran, softmax_scale, stream);
}

kvq_status kvq_prefill_attn_paged(void* out, int out_dtype, const void* q_bf16,
                                  const int32_t* cu_seqlens_q, int max_q_len,
                                  const float* q_scale, int q_gran, const uint8_t* k_cache,
                                  const uint8_t* v_cache, int64_t num_blocks,
                                  const int32_t* block_tables, int max_blocks,
                                  const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                                  int bs, int64_t block_stride, const float* k_scale,
                                  const float* v_scale, int fmt, int kv_gran,
                                  float softmax_scale, kvq_stream stream) {
  kvq_status st = check_attn_common(out, out_dtype, q_bf16, k_cache, v_cache, num_blocks,
                                    block_tables, max_blocks, context_lens, B, Hq, Hkv, dh, bs,
                                    k_scale, v_scale, fmt, kv_gran);
  if (st != KVQ_OK) return st;
  st = check_stride(block_stride, Hkv, bs, dh);
  if (st != KVQ_OK) return st;
  if (fmt == KVQ_FMT_INT8) return KVQ_ERR_UNSUPPORTED;  // FP8-domain path: FP8 caches only
  if (!gran_ok(q_gran)) return KVQ_ERR_UNSUPPORTED;
  if (max_q_len < 0) return KVQ_ERR_SHAPE;
  if (!cu_seqlens_q || !q_scale) return KVQ_ERR_NULL;
  if (max_q_len == 0) return KVQ_OK;
  return map_err(launch_prefill(out, out_dtype == KVQ_OUT_BF16, (const uint16_t*)q_bf16,
                                cu_seqlens_q, max_q_len, q_scale, q_gran == KVQ_SCALE_HEAD,
                                k_cache, v_cache, num_blocks, block_tables, max_blocks,
                                context_lens, B, Hq, Hkv, dh, k_scale, v_scale, fmt,
                                kv_gran == KVQ_SCALE_HEAD, softmax_scale, (hipStream_t)stream,
                                block_stride));
}

// ---------------------------------------------------------------- skip-layers
int kvq_layer_index(const char* prefix) {
  if (!prefix) return -1;
  int found = -1, count = 0;
  const char* p = prefix;
  while (true) {
    const char* e = p;
    while (*e && *e != '.') ++e;
    bool digits = e > p;
    long v = 0;
    for (const char* c = p; c < e; ++c) {
      if (*c < '0' || *c > '9' || v > 100000000L) {
        digits = false;
        break;
      }
      v = v * 10 + (*c - '0');
    }
    if (digits) {
      ++count;
      found = (int)v;
    }
    if (!*e) break;
    p = e + 1;
  }
  return count == 1 ? found : -1;
}

int kvq_layer_skipped(int layer_index, int is_sliding_window, const char* const* skip_list,
                      int n_skip) {
  if (!skip_list || n_skip <= 0) return 0;
  char idx[16];
  int n = 0;
  if (layer_index >= 0) {  // decimal text of the index
    char rev[16];
    int v = layer_index;
    do {
      rev[n++] = (char)('0' + v % 10);
      v /= 10;
    } while (v && n < 15);
    for (int i = 0; i < n; ++i) idx[i] = rev[n - 1 - i];
  }
  idx[n] = 0;
  for (int i = 0; i < n_skip; ++i) {
    const char* s = skip_list[i];
    if (!s) continue;
    if (is_sliding_window && strcmp(s, "sliding_window") == 0) return 1;
    if (n > 0 && strcmp(s, idx) == 0) return 1;
  }
  return 0;
}

uint64_t kvq_page_bytes(int Hkv, int dh, int bs, int bits_per_elem) {
  if (Hkv < 0 || dh < 0 || bs < 0 || bits_per_elem < 0) return 0;
  return 2ull * (uint64_t)Hkv * (uint64_t)dh * (uint64_t)bs * (uint64_t)bits_per_elem / 8ull;
}

uint64_t kvq_common_page_bytes(const int* layer_bits, int L, int Hkv, int dh, int bs) {
  if (!layer_bits || L < 1) return 0;
  uint64_t p = 0;
  for (int l = 0; l < L; ++l) {
    const uint64_t b = kvq_page_bytes(Hkv, dh, bs, layer_bits[l]);
    p = b > p ? b : p;
  }
  return (p + 15) / 16 * 16;
}

}  // extern "C"

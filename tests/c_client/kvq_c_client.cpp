// A C++ client of the kvq C ABI: plain HIP device buffers, no Python and no
// torch.  Through libkvq it calibrates per-head scales, writes a paged cache
// and runs a decode step, plain and with each sequence's newest token appended
// in the same call.  Each result is checked against the C oracle (liborc):
//   - amax and scales bit-exact;
//   - cache bytes bit-exact (slots no token writes keep their NaN fill);
//   - attention within 2e-3 of the oracle, max |o - r| / max |r| over the
//     output and over every (sequence, head) row;
//   - the appended step's cache and output identical to write-then-decode.
// It also checks two host-side refusals, made before any device work.
// Usage: kvq_c_client [fmt], fmt 0 (E4M3, default), 1 (E5M2) or 2 (INT8).
// Exit status 0 when every check passes, 1 otherwise, 2 when no GPU is usable.
// This is test code: it links the oracle, which the library never does.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kvq.h"

extern "C" {  // the oracle's C entry points (oracle/kvq_oracle.c)
void orc_calibrate(const uint16_t* x, int64_t T, int H, int dh, int fmt, int gran,
                   float* amax_out, float* scale_out);
void orc_cache_write(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                     const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                     int64_t num_blocks, int bs, const float* k_scale, const float* v_scale,
                     int fmt, int gran);
void orc_decode_attn(double* out, const uint16_t* q, const uint8_t* k_cache,
                     const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                     const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                     const float* k_scale, const float* v_scale, int fmt, int gran,
                     float softmax_scale);
}

namespace {

int g_failures = 0;

void expect(bool ok, const char* what) {
  std::printf("%s: %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++g_failures;
}

#define HIP_OK(call)                                                               \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__,      \
                  __LINE__);                                                       \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

#define KVQ_OK_CALL(call)                                                          \
  do {                                                                             \
    kvq_status s_ = (call);                                                        \
    if (s_ != KVQ_OK) {                                                            \
      std::printf("kvq error %s at %s:%d\n", kvq_strerror(s_), __FILE__, __LINE__); \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

// Seeded inputs: splitmix64, a counter-based generator (Steele, Lea and Flood,
// "Fast splittable pseudorandom number generators", 2014).
struct SplitMix {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }  // [0, 1)
};

uint16_t to_bf16(float x) {  // round to nearest even (finite inputs)
  uint32_t b;
  std::memcpy(&b, &x, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

template <class T>
T* dev_copy(const std::vector<T>& h) {
  T* d = nullptr;
  HIP_OK(hipMalloc(&d, h.size() * sizeof(T)));
  HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}

template <class T>
std::vector<T> host_copy(const T* d, size_t n) {
  std::vector<T> h(n);
  HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

// max |o - r| / max |r| over everything, and the worst of the same per row
void attn_errors(const std::vector<float>& o, const std::vector<double>& r, int rows, int dh,
                 double* global, double* worst_row) {
  double num = 0.0, den = 0.0;
  *worst_row = 0.0;
  for (int i = 0; i < rows; ++i) {
    double rn = 0.0, rd = 0.0;
    for (int d = 0; d < dh; ++d) {
      const double e = std::fabs((double)o[(size_t)i * dh + d] - r[(size_t)i * dh + d]);
      const double a = std::fabs(r[(size_t)i * dh + d]);
      rn = e > rn ? e : rn;
      rd = a > rd ? a : rd;
    }
    num = rn > num ? rn : num;
    den = rd > den ? rd : den;
    const double rel = rd > 0.0 ? rn / rd : (rn > 0.0 ? INFINITY : 0.0);
    *worst_row = rel > *worst_row ? rel : *worst_row;
  }
  *global = den > 0.0 ? num / den : num;
}

}  // namespace

int main(int argc, char** argv) {
  const int fmt = argc > 1 ? std::atoi(argv[1]) : KVQ_FMT_E4M3;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    std::printf("no HIP device\n");
    return 2;
  }
  const int gran = KVQ_SCALE_HEAD;
  // a small GQA layer: 3 sequences (one token, one block boundary past 256,
  // a long one), 8 query heads over 2 KV heads, dh = 128, 16-token blocks
  const int B = 3, Hq = 8, Hkv = 2, dh = 128, bs = 16;
  const std::vector<int32_t> ctx = {1, 300, 1000};
  std::vector<int> nblk(B);
  int nb_used = 0, max_blocks = 1, max_ctx = 0;
  for (int b = 0; b < B; ++b) {
    nblk[b] = (ctx[b] + bs - 1) / bs;
    nb_used += nblk[b];
    max_blocks = nblk[b] > max_blocks ? nblk[b] : max_blocks;
    max_ctx = ctx[b] > max_ctx ? ctx[b] : max_ctx;
  }
  const int num_blocks = nb_used + 1;  // one spare block fills unused table entries

  SplitMix g{20260};
  // shuffled block ids (Fisher-Yates), handed to the sequences in order
  std::vector<int32_t> perm(num_blocks);
  for (int i = 0; i < num_blocks; ++i) perm[i] = i;
  for (int i = num_blocks - 1; i > 0; --i) {
    const int j = (int)(g.next() % (uint64_t)(i + 1));
    const int32_t t = perm[i];
    perm[i] = perm[j];
    perm[j] = t;
  }
  std::vector<int32_t> bt((size_t)B * max_blocks, perm[num_blocks - 1]);
  for (int b = 0, o = 0; b < B; ++b)
    for (int i = 0; i < nblk[b]; ++i) bt[(size_t)b * max_blocks + i] = perm[o++];

  // tokens in sequence order, each to its position's slot
  int64_t T = 0;
  for (int b = 0; b < B; ++b) T += ctx[b];
  std::vector<int64_t> slots(T), last(B);
  for (int b = 0, t = 0; b < B; ++b)
    for (int p = 0; p < ctx[b]; ++p, ++t) {
      slots[t] = (int64_t)bt[(size_t)b * max_blocks + p / bs] * bs + p % bs;
      last[b] = t;
    }
  // K with two outlier channels, per-head magnitudes from 0.5 to 8
  const double head_mult[Hkv] = {0.5, 8.0};
  std::vector<uint16_t> k((size_t)T * Hkv * dh), v(k.size()), q((size_t)B * Hq * dh);
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < Hkv; ++h)
      for (int d = 0; d < dh; ++d) {
        const size_t i = ((size_t)t * Hkv + h) * dh + d;
        const double out = (d == 7 || d == 90) ? 8.0 : 1.0;
        k[i] = to_bf16((float)((2.0 * g.uniform() - 1.0) * 2.0 * head_mult[h] * out));
        v[i] = to_bf16((float)((2.0 * g.uniform() - 1.0) * 2.0 * head_mult[Hkv - 1 - h]));
      }
  for (auto& x : q) x = to_bf16((float)(2.0 * g.uniform() - 1.0));

  // ---- device buffers: plain pointers and sizes across the boundary
  uint16_t *d_k = dev_copy(k), *d_v = dev_copy(v), *d_q = dev_copy(q);
  int64_t* d_slots = dev_copy(slots);
  int32_t *d_bt = dev_copy(bt), *d_ctx = dev_copy(ctx);
  float *d_kamax, *d_vamax, *d_ks, *d_vs, *d_out, *d_out2;
  HIP_OK(hipMalloc(&d_kamax, Hkv * sizeof(float)));
  HIP_OK(hipMalloc(&d_vamax, Hkv * sizeof(float)));
  HIP_OK(hipMalloc(&d_ks, Hkv * sizeof(float)));
  HIP_OK(hipMalloc(&d_vs, Hkv * sizeof(float)));
  const size_t n_out = (size_t)B * Hq * dh;
  HIP_OK(hipMalloc(&d_out, n_out * sizeof(float)));
  HIP_OK(hipMalloc(&d_out2, n_out * sizeof(float)));
  const size_t cache_bytes = (size_t)num_blocks * Hkv * bs * dh;
  uint8_t *d_kc, *d_vc;
  HIP_OK(hipMalloc(&d_kc, cache_bytes));
  HIP_OK(hipMalloc(&d_vc, cache_bytes));
  const uint8_t kFill = 0x7F;  // a NaN code in E4M3 and E5M2 (127 in INT8)
  HIP_OK(hipMemset(d_kc, kFill, cache_bytes));
  HIP_OK(hipMemset(d_vc, kFill, cache_bytes));
  const size_t ws_bytes = kvq_decode_workspace_size(B, Hq, dh, max_ctx, bs);
  void* d_ws = nullptr;
  HIP_OK(hipMalloc(&d_ws, ws_bytes));

  // ---- calibrate, write, decode
  KVQ_OK_CALL(kvq_calibrate_scales_kv(d_k, d_v, T, Hkv, dh, fmt, gran, d_kamax, d_vamax, d_ks,
                                      d_vs, 0, nullptr));
  KVQ_OK_CALL(kvq_cache_write(d_k, d_v, T, Hkv, dh, d_slots, d_kc, d_vc, num_blocks, bs, d_ks,
                              d_vs, fmt, gran, nullptr));
  KVQ_OK_CALL(kvq_decode_attn(d_out, KVQ_OUT_F32, d_q, d_kc, d_vc, num_blocks, d_bt, max_blocks,
                              d_ctx, B, Hq, Hkv, dh, bs, max_ctx, d_ks, d_vs, fmt, gran, 0.0f,
                              d_ws, ws_bytes, nullptr));
  HIP_OK(hipDeviceSynchronize());
  const auto kamax = host_copy(d_kamax, Hkv), vamax = host_copy(d_vamax, Hkv);
  const auto ks = host_copy(d_ks, Hkv), vs = host_copy(d_vs, Hkv);
  const auto kc = host_copy(d_kc, cache_bytes), vc = host_copy(d_vc, cache_bytes);
  const auto out = host_copy(d_out, n_out);

  // ---- the oracle on the same inputs
  std::vector<float> r_kamax(Hkv), r_vamax(Hkv), r_ks(Hkv), r_vs(Hkv);
  orc_calibrate(k.data(), T, Hkv, dh, fmt, gran, r_kamax.data(), r_ks.data());
  orc_calibrate(v.data(), T, Hkv, dh, fmt, gran, r_vamax.data(), r_vs.data());
  expect(std::memcmp(kamax.data(), r_kamax.data(), Hkv * 4) == 0 &&
             std::memcmp(vamax.data(), r_vamax.data(), Hkv * 4) == 0,
         "amax bit-exact");
  expect(std::memcmp(ks.data(), r_ks.data(), Hkv * 4) == 0 &&
             std::memcmp(vs.data(), r_vs.data(), Hkv * 4) == 0,
         "scales bit-exact");
  std::vector<uint8_t> r_kc(cache_bytes, kFill), r_vc(cache_bytes, kFill);
  orc_cache_write(k.data(), v.data(), T, Hkv, dh, slots.data(), r_kc.data(), r_vc.data(),
                  num_blocks, bs, r_ks.data(), r_vs.data(), fmt, gran);
  expect(kc == r_kc && vc == r_vc, "cache bytes bit-exact");
  std::vector<double> ref(n_out);
  orc_decode_attn(ref.data(), q.data(), r_kc.data(), r_vc.data(), bt.data(), max_blocks,
                  ctx.data(), B, Hq, Hkv, dh, bs, r_ks.data(), r_vs.data(), fmt, gran, 0.0f);
  double e = 0.0, er = 0.0;
  attn_errors(out, ref, B * Hq, dh, &e, &er);
  std::printf("decode: global rel err %.3e, worst row %.3e\n", e, er);
  expect(e <= 2e-3 && er <= 2e-3, "decode within 2e-3 of the oracle, globally and per row");

  // ---- the same step with each sequence's newest token appended in the call
  std::vector<int64_t> old_slots = slots;
  std::vector<uint16_t> k_new((size_t)B * Hkv * dh), v_new(k_new.size());
  for (int b = 0; b < B; ++b) {
    old_slots[last[b]] = -1;  // written by the append call instead
    std::memcpy(&k_new[(size_t)b * Hkv * dh], &k[(size_t)last[b] * Hkv * dh], Hkv * dh * 2);
    std::memcpy(&v_new[(size_t)b * Hkv * dh], &v[(size_t)last[b] * Hkv * dh], Hkv * dh * 2);
  }
  int64_t* d_old = dev_copy(old_slots);
  uint16_t *d_kn = dev_copy(k_new), *d_vn = dev_copy(v_new);
  HIP_OK(hipMemset(d_kc, kFill, cache_bytes));
  HIP_OK(hipMemset(d_vc, kFill, cache_bytes));
  KVQ_OK_CALL(kvq_cache_write(d_k, d_v, T, Hkv, dh, d_old, d_kc, d_vc, num_blocks, bs, d_ks,
                              d_vs, fmt, gran, nullptr));
  KVQ_OK_CALL(kvq_decode_attn_append(d_out2, KVQ_OUT_F32, d_q, d_kn, d_vn, d_kc, d_vc,
                                     num_blocks, d_bt, max_blocks, d_ctx, B, Hq, Hkv, dh, bs,
                                     max_ctx, d_ks, d_vs, fmt, gran, 0.0f, d_ws, ws_bytes,
                                     nullptr));
  HIP_OK(hipDeviceSynchronize());
  const auto kc2 = host_copy(d_kc, cache_bytes), vc2 = host_copy(d_vc, cache_bytes);
  const auto out2 = host_copy(d_out2, n_out);
  expect(kc2 == r_kc && vc2 == r_vc, "append: cache bytes bit-exact");
  expect(std::memcmp(out2.data(), out.data(), n_out * 4) == 0,
         "append: output identical to write-then-decode");

  // ---- refusals made on the host, before any device work
  expect(kvq_decode_attn(d_out, KVQ_OUT_F32, d_q, d_kc, d_vc, num_blocks, d_bt, max_blocks,
                         d_ctx, B, Hq, Hkv, dh, bs, max_ctx, d_ks, d_vs, fmt, gran, 0.0f, d_ws,
                         ws_bytes - 1, nullptr) == KVQ_ERR_WORKSPACE,
         "a workspace one byte short is refused");
  expect(kvq_cache_write(d_k, d_v, T, Hkv, 96, d_slots, d_kc, d_vc, num_blocks, bs, d_ks, d_vs,
                         fmt, gran, nullptr) == KVQ_ERR_UNSUPPORTED,
         "dh = 96 is refused");

  for (void* p : {(void*)d_k, (void*)d_v, (void*)d_q, (void*)d_slots, (void*)d_bt, (void*)d_ctx,
                  (void*)d_kamax, (void*)d_vamax, (void*)d_ks, (void*)d_vs, (void*)d_out,
                  (void*)d_out2, (void*)d_kc, (void*)d_vc, d_ws, (void*)d_old, (void*)d_kn,
                  (void*)d_vn})
    HIP_OK(hipFree(p));
  std::printf("%s (fmt %d, %d failure%s)\n", g_failures ? "FAILED" : "all checks passed", fmt,
              g_failures, g_failures == 1 ? "" : "s");
  return g_failures ? 1 : 0;
}

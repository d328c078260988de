// kivi.hip -- KIVI-style asymmetric 2-bit KV cache: batch quantization of
// whole token groups and split-K decode over the 2-bit cache plus a bf16
// residual of the newest tokens.
//
// What is computed (the KV-cache quantization textbook, section 10.4.4: K is
// grouped per channel over G tokens, V per token over groups of channels, the
// newest tokens stay unquantized in a high-precision residual):
//   per set of 32 values (K: one channel of a 32-token group; V: one 32-channel
//   group of one token)
//     s = fl16(min(fl32(fl32(max - min) / 3), 65504)), z = fl16(clamp(min))
//     code = clip(round-half-even(fl32(fl32(x - z) / s)), 0, 3)  (0 if s == 0)
//     x_hat = code * s + z
//   a set holding an Inf or NaN stores s = z = 0.
//
// Cache layout (dh = 128): the quantized part is paged in 32-token blocks, one
// K group per block; tile (block, head) is 3072 bytes:
//   [0, 1024)     K codes: lane L = 16 g4 + c16 of the decode kernel owns bytes
//                 16 L .. 16 L + 15: for token half th (token 16 th + c16) two
//                 dwords, dword j / 2 holding the codes of channels
//                 32 j + 8 g4 + i (i = 0..7) for j = 2 (j / 2), 2 (j / 2) + 1 at
//                 bit 8 (i / 2) + 4 (i % 2) + 2 (j % 2)
//   [1024, 1280)  K scales, fp16 per channel;  [1280, 1536) K zeros
//   [1536, 2560)  V codes: lane L (channel L and 64 + L) owns 16 bytes; dword
//                 (hc, w) holds channel 64 hc + L, tokens 16 w .. 16 w + 15,
//                 token 16 w + 4 sl + u at bit 8 (2 (sl % 2) + u / 2) +
//                 4 (u % 2) + 2 (sl / 2)
//   [2560, 3072)  V (scale, zero) fp16 pairs, [token][channel group]
// With these orders every 2-bit field is a nibble-aligned pair: masking a
// dword with 0x33333333 (or shifting it right by 2 first) leaves eight 4-bit
// fields whose FP4 (E2M1) value is code / 2, and v_cvt_scalef32_pk_f16_fp4
// with scale 2 turns two of them into the exact f16 codes, in MFMA operand
// order.
//
// Decode (one query per sequence, groups of at most 4 query heads per KV
// head): grid (1 + splits, Hkv, B).  Split 0 attends the residual in fp32 on
// the vector units; split s >= 1 owns quantized groups, one 32-token group
// per wave step:
//   Q K^T: K_hat = s_c code + z_c per channel, so
//     q . k_hat_t = sum_c (q_c s_c) code_tc + sum_c q_c z_c:
//   A' = q s against the exact codes on v_mfma_f32_16x16x32_f16, A' carried
//   as two f16 terms (hi = fl16(q s), lo = fl16(q s - hi), staged through
//   LDS) because the two sums cancel for outlier channels (z ~ -1.5 range) and
//   a single f16 rounding of q s would show in the scores; the accumulator is
//   seeded with q . z from the same instruction (A = q in f16, B = z).
//   P V: V_hat = code s_t + z_t per token and channel group, dequantized to
//   f16 with one packed FMA per two values, on v_mfma_f32_4x4x4_16b_f16 (lane =
//   output channel), as the FP8 decode does.
// Splits write (m, l, acc) partials for every split (empty ones included); the
// shared combine kernel merges them.
#include "attn_common.hpp"
#include "launch.hpp"

namespace kvq {

// Waves per SIMD of the decode split kernel (94 VGPRs at 5; 6 spills)
constexpr int kKiviWavesPerSimd = 5;

namespace {
constexpr int kG = 32;       // tokens per K group and per cache block; channels per V group
constexpr int kDH = 128;     // head dimension of the 2-bit cache
constexpr int kTile = 3072;  // bytes per (block, head) tile
constexpr int kKs = 1024, kKz = 1280, kVc = 1536, kVm = 2560;  // tile regions
constexpr float kLazyTauK = 8.0f;  // lazy running max (p <= 2^8, safe in f16)

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}
__device__ __forceinline__ float f16_val(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// (s, z) of a set from its min and max (finite = no Inf or NaN in the set)
__device__ __forceinline__ uint32_t kivi_sz(float mn, float mx, bool finite) {
  if (!finite) return 0;
  const float range = mx - mn;
  const float s = __builtin_fminf(__fdiv_rn(range, 3.0f), 65504.0f);
  const float z = __builtin_amdgcn_fmed3f(mn, -65504.0f, 65504.0f);
  return (uint32_t)f16_bits(s) | ((uint32_t)f16_bits(z) << 16);
}

// 2-bit code of x for a set's (s, z); rs = fl32(1 / s)
__device__ __forceinline__ uint32_t kivi_code(float x, float s, float rs, float z) {
  float q = quotient(x - z, s, rs);
  q = __builtin_amdgcn_fmed3f(__builtin_rintf(q), 0.0f, 3.0f);
  q = s > 0.0f ? q : 0.0f;
  return (uint32_t)q;
}

// eight nibble-aligned 2-bit codes (masked dword) -> eight exact f16 codes
__device__ __forceinline__ f16x8 codes8(uint32_t x) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 0);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 1);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 2);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 3);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// two of them (byte sel of x) -> two exact f16 codes; sel folds to a constant
__device__ __forceinline__ f16x2 codes2(uint32_t x, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x, 2.0f, 3);
  }
}
__device__ __forceinline__ uint32_t lo2(uint32_t w) { return w & 0x33333333u; }
__device__ __forceinline__ uint32_t hi2(uint32_t w) { return (w >> 2) & 0x33333333u; }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}
}  // namespace

// ---------------------------------------------------------------- quantize
// grid (n_groups * Hkv), 256 threads: one 32-token group of one KV head.  The
// group's K and V go to LDS as fp32; threads 0..127 take one K channel each
// (32 tokens), threads 128..255 one (token, channel group) of V; the codes
// are then packed into the tile's dwords, one K and one V dword per thread.
__global__ __launch_bounds__(256) void kivi_quantize_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int Hkv,
    const int32_t* __restrict__ group_blocks, int64_t num_blocks, uint8_t* __restrict__ cache) {
  // K, V values as their bf16 bits (exact; rows padded to 130 elements so
  // the per-token V reductions fall in distinct banks)
  __shared__ uint16_t xs[2][kG][kDH + 2];
  __shared__ uint8_t cs[2][kG][kDH];    // K, V codes
  const int g = (int)(blockIdx.x / (uint32_t)Hkv);
  const int h = (int)(blockIdx.x - (uint32_t)g * (uint32_t)Hkv);
  const int64_t blk = group_blocks[g];
  if (blk < 0 || blk >= num_blocks) return;  // the whole workgroup leaves together
  uint8_t* tile = cache + ((size_t)blk * Hkv + h) * kTile;
  const int tid = threadIdx.x;
  {
    const int t = tid >> 3, q = tid & 7;  // token, 16-channel piece
    const size_t src = (((size_t)g * kG + t) * Hkv + h) * kDH + 16 * q;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint16_t* x = m ? v : k;
      const uint4 a = *reinterpret_cast<const uint4*>(x + src);
      const uint4 b = *reinterpret_cast<const uint4*>(x + src + 8);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<uint32_t*>(&xs[m][t][16 * q + 2 * i]) = w[i];
    }
  }
  __syncthreads();
  {
    const bool isk = tid < kDH;
    const int c = tid, t = (tid - kDH) >> 2, gc = (tid - kDH) & 3;
    float mn = __builtin_inff(), mx = -__builtin_inff();
    bool fin = true;
    for (int i = 0; i < kG; ++i) {
      const float x = __uint_as_float((uint32_t)(isk ? xs[0][i][c] : xs[1][t][32 * gc + i]) << 16);
      fin = fin && __builtin_isfinite(x);
      mn = __builtin_fminf(mn, x);
      mx = __builtin_fmaxf(mx, x);
    }
    const uint32_t sz = kivi_sz(mn, mx, fin);
    const float s = f16_val(sz & 0xffffu), z = f16_val(sz >> 16);
    const float rs = s > 0.0f ? recip_rn(s) : 0.0f;
    if (isk) {
      reinterpret_cast<uint16_t*>(tile + kKs)[c] = (uint16_t)(sz & 0xffffu);
      reinterpret_cast<uint16_t*>(tile + kKz)[c] = (uint16_t)(sz >> 16);
      for (int i = 0; i < kG; ++i)
        cs[0][i][c] = (uint8_t)kivi_code(__uint_as_float((uint32_t)xs[0][i][c] << 16), s, rs, z);
    } else {
      reinterpret_cast<uint32_t*>(tile + kVm)[tid - kDH] = sz;  // at 16 t + 4 gc
      for (int i = 0; i < kG; ++i)
        cs[1][t][32 * gc + i] =
            (uint8_t)kivi_code(__uint_as_float((uint32_t)xs[1][t][32 * gc + i] << 16), s, rs, z);
    }
  }
  __syncthreads();
  {
    // K dword tid: lane L = tid / 4, token half th, dword j / 2 = wj
    const int L = tid >> 2, th = (tid >> 1) & 1, wj = tid & 1;
    const int t = 16 * th + (L & 15), c0 = 8 * (L >> 4);
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int ii = 0; ii < 2; ++ii)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          w |= (uint32_t)cs[0][t][32 * (2 * wj + jj) + c0 + 2 * e + ii] << (8 * e + 4 * ii + 2 * jj);
    reinterpret_cast<uint32_t*>(tile)[tid] = w;
  }
  {
    // V dword tid: channel 64 hc + L, tokens 16 w' .. 16 w' + 15
    const int L = tid >> 2, hc = (tid >> 1) & 1, wt = tid & 1;
    const int c = 64 * hc + L;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int uu = 0; uu < 2; ++uu)
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const int u = 2 * (e & 1) + uu, sl = 2 * ss + (e >> 1);
          w |= (uint32_t)cs[1][16 * wt + 4 * sl + u][c] << (8 * e + 4 * uu + 2 * ss);
        }
    reinterpret_cast<uint32_t*>(tile + kVc)[tid] = w;
  }
}

// ---------------------------------------------------------------- decode
namespace {
// dynamic LDS: per wave [P 4 x 32 f16][A' hi 4 x 128 f16][A' lo 4 x 128 f16]
// [z 128 f16][V s 4 x 32 f16][V z 4 x 32 f16], then the workgroup's q rows in
// f16 [4][128] and the wave-merge buffers (the residual split reuses the space
// for its q rows and scores)
constexpr int kWaveLds = 256 + 1024 + 1024 + 256 + 256 + 256;
constexpr int kMaxResidual = 256;
size_t kivi_lds_bytes(int NH) {
  const size_t a = 4 * kWaveLds + 1024 + 2 * 4 * 16 * sizeof(float) +
                   (size_t)4 * NH * kDH * sizeof(float);
  const size_t r = (size_t)4 * kDH * sizeof(float) + (size_t)4 * kMaxResidual * sizeof(float);
  return a > r ? a : r;
}
}  // namespace

// Split 0: the residual tokens (bf16, token-major [R][128]) in fp32 on the
// vector units; wave w owns head w of the group.
__device__ void kivi_residual_split(const uint16_t* __restrict__ q, const uint16_t* __restrict__ rk,
                                    const uint16_t* __restrict__ rv, int r, int NH, int b, int Hq,
                                    int hq0, float zc, int nsplit, float* __restrict__ ws_ml,
                                    float* __restrict__ ws_acc, uint8_t* smem) {
  float* qs = reinterpret_cast<float*>(smem);   // [4][128]
  float* sc = qs + 4 * kDH;                     // [4][kMaxResidual]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < NH * kDH; i += 256)
    qs[i] = bf16_to_f32(q[((size_t)b * Hq + hq0 + i / kDH) * kDH + i % kDH]);
  __syncthreads();
  if (wave >= NH) return;  // no barrier follows
  const float* qh = qs + wave * kDH;
  float m = -__builtin_inff();
  for (int t = lane; t < r; t += 64) {
    const uint4* row = reinterpret_cast<const uint4*>(rk + (size_t)t * kDH);
    float acc = 0.0f;
#pragma unroll 4
    for (int i = 0; i < kDH / 8; ++i) {
      const uint4 w = row[i];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(qh[8 * i + 2 * e], __uint_as_float(u[e] << 16), acc);
        acc = __builtin_fmaf(qh[8 * i + 2 * e + 1], __uint_as_float(u[e] & 0xffff0000u), acc);
      }
    }
    const float zt = acc * zc;
    sc[wave * kMaxResidual + t] = zt;
    m = __builtin_fmaxf(m, zt);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o));
  float l = 0.0f;
  for (int t = lane; t < r; t += 64) {
    const float p = __builtin_amdgcn_exp2f(sc[wave * kMaxResidual + t] - m);
    sc[wave * kMaxResidual + t] = p;
    l += p;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  // P V: lane owns channels 2 lane, 2 lane + 1 (each token row is one 256-byte load)
  float a0 = 0.0f, a1 = 0.0f;
  for (int t = 0; t < r; ++t) {
    const float p = sc[wave * kMaxResidual + t];
    const uint32_t w = reinterpret_cast<const uint32_t*>(rv + (size_t)t * kDH)[lane];
    a0 = __builtin_fmaf(p, __uint_as_float(w << 16), a0);
    a1 = __builtin_fmaf(p, __uint_as_float(w & 0xffff0000u), a1);
  }
  const size_t ridx = ((size_t)b * Hq + hq0 + wave) * nsplit;  // split 0
  reinterpret_cast<float2*>(ws_acc + ridx * kDH)[lane] = make_float2(a0, a1);
  if (lane == 0) {
    ws_ml[ridx * 2 + 0] = r > 0 ? m : kNegBig;
    ws_ml[ridx * 2 + 1] = l;
  }
}

template <int NPW>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kKiviWavesPerSimd, kKiviWavesPerSimd))) void
kivi_decode_split_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache,
                         int64_t num_blocks, const int32_t* __restrict__ bt, int max_blocks,
                         const int32_t* __restrict__ quant_groups, int max_groups,
                         const uint16_t* __restrict__ res_k, const uint16_t* __restrict__ res_v,
                         const int32_t* __restrict__ res_lens, int R, int Hq, int Hkv,
                         int rph_shift, float sm_scale, int nsplit, float* __restrict__ ws_ml,
                         float* __restrict__ ws_acc) {
  constexpr int PG = 4 * NPW;  // groups per split
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int NH = Hq / Hkv;  // <= 4: one workgroup serves all query heads of its KV head
  const int hq0 = h * NH;
  const float zc = sm_scale * kLog2e;

  if (split == 0) {
    int r = res_lens[b];
    r = r < 0 ? 0 : (r > R ? R : r);
    const size_t off = ((size_t)b * Hkv + h) * R * kDH;
    kivi_residual_split(q, res_k + off, res_v + off, r, NH, b, Hq, hq0, zc, nsplit, ws_ml,
                        ws_acc, smem);
    return;
  }

  int ng = quant_groups[b];
  ng = ng < 0 ? 0 : (ng > max_groups ? max_groups : ng);
  const int g0 = (split - 1) * PG;
  const int ngs = ng - g0 < PG ? ng - g0 : PG;  // groups of this split (may be <= 0)
  if (ngs <= 0) {  // past the sequence's groups: an empty partial
    for (int o = threadIdx.x; o < NH * kDH; o += 256) {
      const size_t ridx = ((size_t)b * Hq + hq0 + o / kDH) * nsplit + split;
      ws_acc[ridx * kDH + o % kDH] = 0.0f;
      if (o % kDH == 0) {
        ws_ml[ridx * 2 + 0] = kNegBig;
        ws_ml[ridx * 2 + 1] = 0.0f;
      }
    }
    return;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int rph_mask = (1 << rph_shift) - 1;
  const int head_a = c16 >> rph_shift;  // A row of the S tile
  const int head_s = (4 * g4) >> rph_shift;  // S rows of this lane
  const bool pub = ((4 * g4) & rph_mask) == 0 && head_s < NH;
  const int head_p = lane & 3;  // A row of the P V tile (rows >= NH read zeros)

  uint8_t* wl_base = smem + wave * kWaveLds;
  _Float16* ptr = reinterpret_cast<_Float16*>(wl_base);          // P [4][32]
  _Float16* aq = reinterpret_cast<_Float16*>(wl_base + 256);     // A' hi [4][128]
  _Float16* al = reinterpret_cast<_Float16*>(wl_base + 1280);    // A' lo [4][128]
  _Float16* zb = reinterpret_cast<_Float16*>(wl_base + 2304);    // K zeros [128]
  uint16_t* vsS = reinterpret_cast<uint16_t*>(wl_base + 2560);   // V scales [4][32]
  uint16_t* vsZ = reinterpret_cast<uint16_t*>(wl_base + 2816);   // V zeros [4][32]
  _Float16* qsh = reinterpret_cast<_Float16*>(smem + 4 * kWaveLds);  // q rows [4][128]
  float* wm = reinterpret_cast<float*>(smem + 4 * kWaveLds + 1024);
  float* wlsum = wm + 4 * 16;
  float* wo = wlsum + 4 * 16;  // [4][NH][128]

  // q operands: the workgroup's q rows in f16 in LDS (A of the bias product,
  // rows of heads >= NH zero) and the two channels 2 lane, 2 lane + 1 of every
  // head (fp32) for A' = q s
  for (int i = tid; i < 4 * kDH; i += 256) {
    const int hh = i / kDH;
    qsh[i] = hh < NH ? (_Float16)bf16_to_f32(q[((size_t)b * Hq + hq0 + hh) * kDH + i % kDH])
                     : (_Float16)0.0f;
  }
  float qa[4][2];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    qa[hh][0] = qa[hh][1] = 0.0f;
    if (hh < NH) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(
          q + ((size_t)b * Hq + hq0 + hh) * kDH)[lane];
      qa[hh][0] = __uint_as_float(w << 16);
      qa[hh][1] = __uint_as_float(w & 0xffff0000u);
    }
  }

  struct Regs {
    uint4 kc, vc;
    uint32_t ks, kz;
    uint2 vm;
  };
  // this wave's groups are wave + 4 k, k < NPW; their block ids come in one
  // vector load (lane k holds group wave + 4 k's id, clamped to the split's
  // last group), waited for here, before the loop
  const int32_t* btab = bt + (size_t)b * max_blocks + g0;
  int idv = 0;
  if (lane < NPW) {
    const int gl = wave + 4 * lane;
    idv = btab[gl < ngs ? gl : ngs - 1];
  }
  asm volatile("" ::"v"(idv));
  const int nb_last = num_blocks - 1 < 0x7fffffff ? (int)(num_blocks - 1) : 0x7fffffff;
  auto load = [&](Regs& x, int k) {
    int blk = __builtin_amdgcn_readlane(idv, k);
    blk = blk < 0 ? 0 : (blk > nb_last ? nb_last : blk);
    const uint8_t* tile = cache + ((size_t)blk * Hkv + h) * kTile;
    x.kc = load16(tile + 16 * lane);
    x.ks = *reinterpret_cast<const uint32_t*>(tile + kKs + 4 * lane);
    x.kz = *reinterpret_cast<const uint32_t*>(tile + kKz + 4 * lane);
    x.vc = load16(tile + kVc + 16 * lane);
    x.vm = load8(tile + kVm + 8 * lane);
  };

  // rows of heads >= NH in P, A' hi and A' lo stay zero (their products land in
  // output rows nobody reads, so the operand loads need no masking)
  for (int i = lane; i < (256 + 2048) / 16; i += 64)
    reinterpret_cast<uint4*>(wl_base)[i] = make_uint4(0, 0, 0, 0);
  // group 0's loads go out before the barrier (so they are issued ahead of
  // group 1's, and in flight while the q rows are staged)
  Regs r[2];
  load(r[0], 0);
  __syncthreads();  // the q rows are read by every wave

  float m_run = kNegBig, l_part = 0.0f;
  f32x4 O[2];
  O[0] = O[1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto step = [&](const Regs& cur, bool live) {
    // ---- stage A' = q s, the K zeros and the V (s, z) of this group in LDS
    {
      const f16x2 s2 = __builtin_bit_cast(f16x2, cur.ks);
      const float s0 = (float)s2[0], s1 = (float)s2[1];
      // (rows of heads >= NH have q = 0 and stay zero; writing them anyway
      // keeps the scale load out of a branch, where it would be issued late)
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float x0 = qa[hh][0] * s0, x1 = qa[hh][1] * s1;
        const f16x2 hi = f16x2{(_Float16)x0, (_Float16)x1};
        reinterpret_cast<f16x2*>(aq + hh * kDH)[lane] = hi;
        reinterpret_cast<f16x2*>(al + hh * kDH)[lane] =
            f16x2{(_Float16)(x0 - (float)hi[0]), (_Float16)(x1 - (float)hi[1])};
      }
      reinterpret_cast<uint32_t*>(zb)[lane] = cur.kz;
      const int t = lane >> 1, ga = 2 * (lane & 1);
      vsS[ga * kG + t] = (uint16_t)(cur.vm.x & 0xffffu);
      vsZ[ga * kG + t] = (uint16_t)(cur.vm.x >> 16);
      vsS[(ga + 1) * kG + t] = (uint16_t)(cur.vm.y & 0xffffu);
      vsZ[(ga + 1) * kG + t] = (uint16_t)(cur.vm.y >> 16);
    }
    // ---- S = (q s) codes + q z for both 16-token halves
    f32x4 Cb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x8 zop = *reinterpret_cast<const f16x8*>(zb + 32 * j + 8 * g4);
      const f16x8 qop = *reinterpret_cast<const f16x8*>(qsh + head_a * kDH + 32 * j + 8 * g4);
      Cb = __builtin_amdgcn_mfma_f32_16x16x32_f16(qop, zop, Cb, 0, 0, 0);
    }
    f32x4 S0 = Cb, S1 = Cb;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ao = head_a * kDH + 32 * j + 8 * g4;
      const f16x8 ahi = *reinterpret_cast<const f16x8*>(aq + ao);
      const f16x8 alo = *reinterpret_cast<const f16x8*>(al + ao);
      // token half 0 in kc.x / kc.y, half 1 in kc.z / kc.w; dword j / 2, field j % 2
      const uint32_t w0 = j < 2 ? cur.kc.x : cur.kc.y, w1 = j < 2 ? cur.kc.z : cur.kc.w;
      const f16x8 b0 = codes8((j & 1) ? hi2(w0) : lo2(w0));
      const f16x8 b1 = codes8((j & 1) ? hi2(w1) : lo2(w1));
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b0, S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, b1, S1, 0, 0, 0);
      S0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b0, S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, b1, S1, 0, 0, 0);
    }
    // a group past the split's end (live false) has every score at -inf: it
    // adds nothing (its tile is a real one, so its values are finite)
    const float zt[2] = {live ? S0[0] * zc : -__builtin_inff(),
                         live ? S1[0] * zc : -__builtin_inff()};
    // ---- online softmax (lazy max, wave-uniform rare rescale)
    const bool need = __builtin_fmaxf(zt[0], zt[1]) > m_run + kLazyTauK;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mt = max16(__builtin_fmaxf(zt[0], zt[1]));
      const bool up = mt > m_run + kLazyTauK;
      const float f = up ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
      m_run = up ? mt : m_run;
      l_part *= f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < NH) {
          const float fr = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), (4 * r) << rph_shift));
          O[0][r] *= fr;
          O[1][r] *= fr;
        }
      }
    }
    const float p0 = __builtin_amdgcn_exp2f(zt[0] - m_run);
    const float p1 = __builtin_amdgcn_exp2f(zt[1] - m_run);
    l_part += p0 + p1;
    if (pub) {
      ptr[head_s * kG + c16] = (_Float16)p0;
      ptr[head_s * kG + 16 + c16] = (_Float16)p1;
    }
    // ---- O += P V_hat: 8 steps of 4 tokens x 2 halves of 64 channels

#pragma unroll
    for (int t8 = 0; t8 < 4; ++t8) {  // 8 tokens: two MFMA steps per half
      const f16x8 p8 = *reinterpret_cast<const f16x8*>(ptr + head_p * kG + 8 * t8);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int gc = 2 * c + (lane >> 5);  // channel group of channel 64 c + lane
        const uint4 s8 = *reinterpret_cast<const uint4*>(vsS + gc * kG + 8 * t8);
        const uint4 z8 = *reinterpret_cast<const uint4*>(vsZ + gc * kG + 8 * t8);
        const uint32_t word = c ? (t8 < 2 ? cur.vc.z : cur.vc.w) : (t8 < 2 ? cur.vc.x : cur.vc.y);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int tq = 2 * t8 + st, sl = tq & 3;
          const uint32_t x = (sl >> 1) ? hi2(word) : lo2(word);
          const f16x2 c01 = codes2(x, 2 * (sl & 1));
          const f16x2 c23 = codes2(x, 2 * (sl & 1) + 1);
          const uint32_t sa = st ? s8.z : s8.x, sb = st ? s8.w : s8.y;
          const uint32_t za = st ? z8.z : z8.x, zb2 = st ? z8.w : z8.y;
          const f16x2 v01 = __builtin_elementwise_fma(c01, __builtin_bit_cast(f16x2, sa),
                                                      __builtin_bit_cast(f16x2, za));
          const f16x2 v23 = __builtin_elementwise_fma(c23, __builtin_bit_cast(f16x2, sb),
                                                      __builtin_bit_cast(f16x2, zb2));
          const f16x4 a = st ? f16x4{p8[4], p8[5], p8[6], p8[7]}
                             : f16x4{p8[0], p8[1], p8[2], p8[3]};
          O[c] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, f16x4{v01[0], v01[1], v23[0], v23[1]},
                                                   O[c], 0, 0, 0);
        }
      }
    }
  };

  // two register sets in turn, the loop fully unrolled: group k + 1's loads
  // are in flight while group k is processed.  Loads and steps are
  // unconditional (a group past the split's last one re-reads that group's
  // tile and contributes nothing), so no load is moved into a branch and each
  // wait for a group's registers leaves the next group's loads in flight.
#pragma unroll
  for (int k = 0; k < NPW; ++k) {
    if (k + 1 < NPW) load(r[(k + 1) & 1], k + 1);
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the step
    step(r[k & 1], wave + 4 * k < ngs);
  }

  // ---- merge the 4 waves through LDS and write the split's partial
  float x = l_part;
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  if (pub && c16 == 0) {
    wm[wave * 16 + head_s] = m_run;
    wlsum[wave * 16 + head_s] = x;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < NH) {
      wo[(wave * NH + r) * kDH + lane] = O[0][r];
      wo[(wave * NH + r) * kDH + 64 + lane] = O[1][r];
    }
  __syncthreads();
  for (int o = tid; o < NH * kDH; o += 256) {
    const int row = o / kDH, d = o - row * kDH;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = __builtin_fmaxf(M, wm[w * 16 + row]);
    float a = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w * 16 + row] - M);
      a += f * wo[(w * NH + row) * kDH + d];
      L += f * wlsum[w * 16 + row];
    }
    const size_t ridx = ((size_t)b * Hq + hq0 + row) * nsplit + split;
    ws_acc[ridx * kDH + d] = a;
    if (d == 0) {
      ws_ml[ridx * 2 + 0] = M;
      ws_ml[ridx * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------- launchers
// Workgroups the quantized splits should at least give (the split shrinks,
// from 32 groups down to 4, until they do).  About one round of resident
// workgroups (5 per CU): fewer, longer workgroups amortize each one's start
// (q staging, the block ids, the first group's latency).  On 8 x 16384 tokens
// 32-group splits (1088 workgroups) measured 34.1-37.0 us against 35.5-40.5
// for 16-group ones (2112), in five alternating rounds on one box.
constexpr int kKiviMinWgs = 1024;

KiviPlan kivi_decode_plan(int B, int Hq, int Hkv, int max_groups) {
  KiviPlan p{};
  int PG = 32;
  while (PG > 4 && (int64_t)B * Hkv * ((max_groups + PG - 1) / PG) < kKiviMinWgs) PG >>= 1;
  p.groups_per_split = PG;
  p.nsplit = 1 + (max_groups + PG - 1) / PG;
  // The workspace holds the most splits any max_groups up to this one plans
  // (a smaller max_groups can take a smaller split and so more of them), so a
  // workspace sized for the largest serves every call.  With fill quantized
  // splits per sequence filling the chip, 4-group splits run up to 8 (fill - 1)
  // groups, ceil(max_groups / 4) of them; no larger split size ever plans more
  // than 2 (fill - 1).
  const int64_t fill = (kKiviMinWgs + (int64_t)B * Hkv - 1) / ((int64_t)B * Hkv);
  int64_t ws_q = (max_groups + PG - 1) / PG;
  const int64_t short_q = (max_groups + 3) / 4 < 2 * (fill - 1) ? (max_groups + 3) / 4 : 2 * (fill - 1);
  if (short_q > ws_q) ws_q = short_q;
  p.ws_bytes = (size_t)B * Hq * (size_t)(1 + ws_q) * (2 + kDH) * sizeof(float);
  return p;
}

hipError_t launch_kivi_quantize(const uint16_t* k, const uint16_t* v, int64_t n_groups, int Hkv,
                                const int32_t* group_blocks, uint8_t* cache, int64_t num_blocks,
                                hipStream_t s) {
  if (n_groups == 0) return hipSuccess;
  kivi_quantize_kernel<<<(uint32_t)(n_groups * Hkv), 256, 0, s>>>(k, v, Hkv, group_blocks,
                                                                   num_blocks, cache);
  return hipGetLastError();
}

hipError_t launch_kivi_decode(void* out, int out_bf16, const uint16_t* q, const uint8_t* cache,
                              int64_t num_blocks, const int32_t* bt, int max_blocks,
                              const int32_t* quant_groups, int max_groups, const uint16_t* res_k,
                              const uint16_t* res_v, const int32_t* res_lens, int R, int B,
                              int Hq, int Hkv, float softmax_scale, const KiviPlan& plan,
                              void* ws, hipStream_t s) {
  const int NH = Hq / Hkv;
  int nhp_shift = 0;
  while ((1 << nhp_shift) < NH) ++nhp_shift;
  const int rph_shift = 4 - nhp_shift;
  float* ml = reinterpret_cast<float*>(ws);
  float* acc = ml + (size_t)B * Hq * plan.nsplit * 2;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / __builtin_sqrtf((float)kDH);
  const dim3 grid(plan.nsplit, Hkv, B);
  const size_t lds = kivi_lds_bytes(NH);
#define KVQ_KIVI(N)                                                                             \
  kivi_decode_split_kernel<N><<<grid, 256, lds, s>>>(q, cache, num_blocks, bt, max_blocks,       \
                                                     quant_groups, max_groups, res_k, res_v,     \
                                                     res_lens, R, Hq, Hkv, rph_shift, sm,        \
                                                     plan.nsplit, ml, acc)
  switch (plan.groups_per_split) {
    case 32: KVQ_KIVI(8); break;
    case 16: KVQ_KIVI(4); break;
    case 8: KVQ_KIVI(2); break;
    default: KVQ_KIVI(1); break;
  }
#undef KVQ_KIVI
  launch_decode_combine(out, out_bf16, ml, acc, nullptr, B, Hq, Hkv, kDH, 0, nullptr, 0, 0,
                        plan.nsplit, s);
  return hipGetLastError();
}

}  // namespace kvq

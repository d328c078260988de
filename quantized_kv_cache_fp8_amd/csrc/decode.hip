// decode.hip -- split-K paged decode attention over the FP8 cache, with the
// dequantization fused in.
//
// Computes, per sequence b and query head hq (KV head h = hq / G):
//   z_j = (q . k_hat_j) / sqrt(dh),  P = softmax(z),  o = sum_j P_j v_hat_j
// with k_hat = sK * cast_float(K8), v_hat = sV * cast_float(V8): the attention
// equation and the fused dequant + attention path of the KV-cache quantization
// textbook (section 10.4.2), on the FP8 storage of section 10.4.5.  No
// dequantized copy of the cache exists anywhere: codes go from HBM into
// registers and are converted there.
//
// Work decomposition (flash-decoding):
//   grid = (nsplit, Hq / GT, B); a workgroup of 4 waves owns one split of
//   part_blocks cache blocks of one sequence and GT query heads that share one
//   KV head (GT = 4 for the usual GQA group of 4).  Wave w takes blocks
//   w, w+4, ... of the split.
// Per cache block (16 tokens, one (block, head) tile = 16*dh contiguous bytes)
// a wave issues two coalesced loads of K and two of V (lane l holds dh/8
// bytes of token l/8 and of token 8 + l/8), so every byte is read from HBM
// exactly once and reused in registers by all GT query heads:
//   * q.k: codes -> bf16 pairs (exact, v_cvt_scalef32_pk_bf16_*), v_dot2 with
//     the bf16 query (exact products, fp32 accumulation), then a sum over the
//     8 lanes of a token by DPP (quad_perm, quad_perm, row_half_mirror);
//   * online softmax per lane in the log2 domain, with the running max only
//     raised when a score exceeds it by more than 2^8 (p stays <= 256), so the
//     accumulator rescale is rare;
//   * p.v: each lane pairs the codes of its two tokens channel by channel
//     (v_perm_b32), converts to f16 pairs (exact) and accumulates
//     p_a*v_a + p_b*v_b with v_dot2_f32_f16 (p rounded to f16, 11 bits).
// The split's partial (m, l, o) is merged across the 8 token lanes, across the
// 4 waves through LDS, and written to the workspace; a second kernel merges
// the splits (log-sum-exp) and applies sV.
#include "codec.hpp"
#include "launch.hpp"

namespace kvq {

constexpr int kBlockSize = 16;   // tokens per cache block
constexpr float kLazyTau = 8.0f; // log2 headroom before the running max moves
constexpr float kLog2e = 1.4426950408889634f;
// Running maxima start finite, so exp2(-inf - m) = 0 for masked keys and no
// merge ever forms -inf - (-inf).
constexpr float kNegBig = -1.0e30f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes of each half-row (lanes 8i .. 8i+7); every lane gets it.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x;
}

template <int DPL>
struct Chunk;  // DPL bytes of one token row held by one lane
template <>
struct Chunk<16> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const uint8_t* p) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
};
template <>
struct Chunk<8> {
  uint32_t w[2];
  __device__ __forceinline__ void load(const uint8_t* p) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  }
};

template <int DPL>
struct Tile {  // one lane's share of one block: tokens (l/8) and (8 + l/8), K and V
  Chunk<DPL> k0, k1, v0, v1;
};

template <int FMT, int DH, int GT>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
    const uint8_t* __restrict__ vc, int64_t num_blocks, const int32_t* __restrict__ bt,
    int max_blocks, const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int max_ctx,
    const float* __restrict__ ks, int per_head, float sm_scale, int part_blocks, int nsplit,
    float* __restrict__ ws_ml, float* __restrict__ ws_acc) {
  constexpr int DPL = DH / 8;  // bytes of a token row per lane
  constexpr int NW = DPL / 4;  // dwords per lane per token
  const int split = blockIdx.x, grp = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int gpk = G / GT;  // workgroups per KV head
  const int h = grp / gpk;
  const int hq0 = h * G + (grp - h * gpk) * GT;

  int ctx = ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
  const int tok0 = split * part_blocks * kBlockSize;
  if (tok0 >= ctx) return;  // nothing of this sequence lies in this split
  const int nblk_left = (ctx - tok0 + kBlockSize - 1) / kBlockSize;
  const int nblk = nblk_left < part_blocks ? nblk_left : part_blocks;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = lane >> 3, dl = lane & 7;

  // query rows of the GT heads, this lane's DPL channels, as bf16 pairs
  bf16x2 qv[GT][DPL / 2];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const uint16_t* qp = q + ((size_t)b * Hq + hq0 + g) * DH + dl * DPL;
#pragma unroll
    for (int j = 0; j < DPL / 8; ++j) {
      uint4 w = *reinterpret_cast<const uint4*>(qp + j * 8);
      qv[g][4 * j + 0] = __builtin_bit_cast(bf16x2, w.x);
      qv[g][4 * j + 1] = __builtin_bit_cast(bf16x2, w.y);
      qv[g][4 * j + 2] = __builtin_bit_cast(bf16x2, w.z);
      qv[g][4 * j + 3] = __builtin_bit_cast(bf16x2, w.w);
    }
  }
  // z (log2 domain) = (q . k_code) * sK / sqrt(dh) * log2(e)
  const float zc = sm_scale * ks[per_head ? h : 0] * kLog2e;

  float m[GT], l[GT], acc[GT][DPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = kNegBig;
    l[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < DPL; ++d) acc[g][d] = 0.0f;
  }

  const int32_t* btab = bt + (size_t)b * max_blocks + (size_t)split * part_blocks;
  const size_t tile_stride = (size_t)kBlockSize * DH;  // bytes per (block, head) tile
  auto load_tile = [&](int i, Tile<DPL>& t) {
    int64_t blk = btab[i];
    blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    const size_t base = ((size_t)blk * Hkv + h) * tile_stride + (size_t)lane * DPL;
    t.k0.load(kc + base);
    t.k1.load(kc + base + 8 * DH);
    t.v0.load(vc + base);
    t.v1.load(vc + base + 8 * DH);
  };

  Tile<DPL> cur, nxt;
  int i = wave;
  if (i < nblk) load_tile(i, cur);
  for (; i < nblk; i += 4) {
    if (i + 4 < nblk) load_tile(i + 4, nxt);
    const int tokb = tok0 + i * kBlockSize;
    const bool ok0 = tokb + kg < ctx, ok1 = tokb + 8 + kg < ctx;

    // ---- scores of this lane's two tokens for the GT heads
    float z0[GT], z1[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) { z0[g] = 0.0f; z1[g] = 0.0f; }
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const bf16x2 a_lo = dec2_bf16<FMT, false>(cur.k0.w[w]);
      const bf16x2 a_hi = dec2_bf16<FMT, true>(cur.k0.w[w]);
      const bf16x2 b_lo = dec2_bf16<FMT, false>(cur.k1.w[w]);
      const bf16x2 b_hi = dec2_bf16<FMT, true>(cur.k1.w[w]);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        z0[g] = __builtin_amdgcn_fdot2_f32_bf16(qv[g][2 * w], a_lo, z0[g], false);
        z0[g] = __builtin_amdgcn_fdot2_f32_bf16(qv[g][2 * w + 1], a_hi, z0[g], false);
        z1[g] = __builtin_amdgcn_fdot2_f32_bf16(qv[g][2 * w], b_lo, z1[g], false);
        z1[g] = __builtin_amdgcn_fdot2_f32_bf16(qv[g][2 * w + 1], b_hi, z1[g], false);
      }
    }
    f16x2 ph[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float s0 = ok0 ? sum8(z0[g]) * zc : -__builtin_inff();
      float s1 = ok1 ? sum8(z1[g]) * zc : -__builtin_inff();
      const float smax = __builtin_fmaxf(s0, s1);
      if (smax > m[g] + kLazyTau) {  // raise the running max, rescale (rare)
        const float f = __builtin_amdgcn_exp2f(m[g] - smax);
        l[g] *= f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) acc[g][d] *= f;
        m[g] = smax;
      }
      const float p0 = __builtin_amdgcn_exp2f(s0 - m[g]);
      const float p1 = __builtin_amdgcn_exp2f(s1 - m[g]);
      l[g] += p0 + p1;
      ph[g] = f16x2{(_Float16)p0, (_Float16)p1};
    }

    // ---- p . v: channel-wise pairs (token a, token b) against (p_a, p_b)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t x = cur.v0.w[w], y = cur.v1.w[w];
      const uint32_t lo = __builtin_amdgcn_perm(x, y, 0x01050004u);  // x0 y0 x1 y1
      const uint32_t hi = __builtin_amdgcn_perm(x, y, 0x03070206u);  // x2 y2 x3 y3
      const f16x2 c0 = dec2_f16<FMT, false>(lo), c1 = dec2_f16<FMT, true>(lo);
      const f16x2 c2 = dec2_f16<FMT, false>(hi), c3 = dec2_f16<FMT, true>(hi);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        acc[g][4 * w + 0] = __builtin_amdgcn_fdot2(ph[g], c0, acc[g][4 * w + 0], false);
        acc[g][4 * w + 1] = __builtin_amdgcn_fdot2(ph[g], c1, acc[g][4 * w + 1], false);
        acc[g][4 * w + 2] = __builtin_amdgcn_fdot2(ph[g], c2, acc[g][4 * w + 2], false);
        acc[g][4 * w + 3] = __builtin_amdgcn_fdot2(ph[g], c3, acc[g][4 * w + 3], false);
      }
    }
    cur = nxt;
  }

  // ---- merge the 8 token lanes that share a channel chunk (xor 8, 16, 32)
#pragma unroll
  for (int off = 8; off <= 32; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = __builtin_fmaxf(m[g], mo);
      const float fa = __builtin_amdgcn_exp2f(m[g] - mn);
      const float fb = __builtin_amdgcn_exp2f(mo - mn);
      l[g] = l[g] * fa + lo * fb;
#pragma unroll
      for (int d = 0; d < DPL; ++d) {
        const float ao = __shfl_xor(acc[g][d], off);
        acc[g][d] = acc[g][d] * fa + ao * fb;
      }
      m[g] = mn;
    }
  }

  // ---- merge the 4 waves through LDS and write the split's partial
  __shared__ float s_m[4][GT], s_l[4][GT];
  __shared__ float s_acc[4][GT][DH];
  if (kg == 0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int d = 0; d < DPL; ++d) s_acc[wave][g][dl * DPL + d] = acc[g][d];
      if (dl == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < GT * DH; o += 256) {
    const int g = o / DH, d = o - g * DH;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = __builtin_fmaxf(M, s_m[w][g]);
    float a = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][g] - M);
      a += f * s_acc[w][g][d];
      L += f * s_l[w][g];
    }
    const size_t row = ((size_t)b * Hq + hq0 + g) * nsplit + split;
    ws_acc[row * DH + d] = a;
    if (d == 0) {
      ws_ml[row * 2 + 0] = M;
      ws_ml[row * 2 + 1] = L;
    }
  }
}

// grid (Hq, B), DH threads: merge the valid splits of one (b, hq) row.
template <int DH, bool BF16>
__global__ __launch_bounds__(DH) void decode_combine_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int max_ctx,
    const float* __restrict__ vs, int per_head, int part_blocks, int nsplit) {
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int ctx = ctx_lens[b];
  ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
  const int span = part_blocks * kBlockSize;
  const int nvalid = (ctx + span - 1) / span;
  const size_t row0 = ((size_t)b * Hq + hq) * nsplit;
  float M = kNegBig;
  for (int s = 0; s < nvalid; ++s) M = __builtin_fmaxf(M, ws_ml[(row0 + s) * 2]);
  float L = 0.0f, a = 0.0f;
  for (int s = 0; s < nvalid; ++s) {
    const float f = __builtin_amdgcn_exp2f(ws_ml[(row0 + s) * 2] - M);
    L += f * ws_ml[(row0 + s) * 2 + 1];
    a += f * ws_acc[(row0 + s) * DH + d];
  }
  const int h = hq / (Hq / Hkv);
  const float r = L > 0.0f ? a / L * vs[per_head ? h : 0] : 0.0f;
  const size_t o = ((size_t)b * Hq + hq) * DH + d;
  if constexpr (BF16)
    reinterpret_cast<uint16_t*>(out)[o] = (uint16_t)f32_to_bf16_rne(r);
  else
    reinterpret_cast<float*>(out)[o] = r;
}

DecodePlan decode_plan(int B, int Hq, int dh, int max_context_len, int bs) {
  DecodePlan p{0, 0, 0};
  if (B < 1 || Hq < 1 || dh < 1 || bs < 1 || max_context_len < 0) return p;
  const int64_t nb = ((int64_t)max_context_len + bs - 1) / bs;
  const int64_t groups = (int64_t)B * (Hq >= 4 ? Hq / 4 : 1);
  int P = 32;
  // shrink the split until the grid has enough workgroups to fill the chip
  while (P > 4 && groups * ((nb + P - 1) / P) < 2048) P >>= 1;
  p.part_blocks = P;
  p.nsplit = (int)(nb > 0 ? (nb + P - 1) / P : 1);
  p.ws_bytes = (size_t)B * Hq * p.nsplit * (2 + dh) * sizeof(float);
  return p;
}

template <int FMT, int DH, int GT>
static void launch_split(dim3 grid, hipStream_t s, const uint16_t* q, const uint8_t* kc,
                         const uint8_t* vc, int64_t num_blocks, const int32_t* bt,
                         int max_blocks, const int32_t* ctx, int Hq, int Hkv, int max_ctx,
                         const float* ks, int per_head, float sm, const DecodePlan& plan,
                         float* ml, float* acc) {
  decode_split_kernel<FMT, DH, GT><<<grid, 256, 0, s>>>(q, kc, vc, num_blocks, bt, max_blocks, ctx,
                                                        Hq, Hkv, max_ctx, ks, per_head, sm,
                                                        plan.part_blocks, plan.nsplit, ml, acc);
}

template <int FMT, int DH>
static void launch_split_gt(int GT, dim3 grid, hipStream_t s, const uint16_t* q,
                            const uint8_t* kc, const uint8_t* vc, int64_t num_blocks,
                            const int32_t* bt, int max_blocks, const int32_t* ctx, int Hq, int Hkv,
                            int max_ctx, const float* ks, int per_head, float sm,
                            const DecodePlan& plan, float* ml, float* acc) {
  if (GT == 4)
    launch_split<FMT, DH, 4>(grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq, Hkv,
                             max_ctx, ks, per_head, sm, plan, ml, acc);
  else if (GT == 2)
    launch_split<FMT, DH, 2>(grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq, Hkv,
                             max_ctx, ks, per_head, sm, plan, ml, acc);
  else
    launch_split<FMT, DH, 1>(grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq, Hkv,
                             max_ctx, ks, per_head, sm, plan, ml, acc);
}

hipError_t launch_decode(void* out, int out_bf16, const uint16_t* q, const uint8_t* kc,
                         const uint8_t* vc, int64_t num_blocks, const int32_t* bt,
                         int max_blocks, const int32_t* ctx, int B, int Hq, int Hkv, int dh,
                         int max_ctx, const float* ks, const float* vs, int fmt, int per_head,
                         float softmax_scale, const DecodePlan& plan, void* ws, hipStream_t s) {
  const int G = Hq / Hkv;
  const int GT = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  float* ml = reinterpret_cast<float*>(ws);
  float* acc = ml + (size_t)B * Hq * plan.nsplit * 2;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / __builtin_sqrtf((float)dh);
  dim3 grid(plan.nsplit, Hq / GT, B);
  if (max_ctx > 0) {
    if (fmt == E4M3) {
      if (dh == 128)
        launch_split_gt<E4M3, 128>(GT, grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq,
                                   Hkv, max_ctx, ks, per_head, sm, plan, ml, acc);
      else
        launch_split_gt<E4M3, 64>(GT, grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq,
                                  Hkv, max_ctx, ks, per_head, sm, plan, ml, acc);
    } else {
      if (dh == 128)
        launch_split_gt<E5M2, 128>(GT, grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq,
                                   Hkv, max_ctx, ks, per_head, sm, plan, ml, acc);
      else
        launch_split_gt<E5M2, 64>(GT, grid, s, q, kc, vc, num_blocks, bt, max_blocks, ctx, Hq,
                                  Hkv, max_ctx, ks, per_head, sm, plan, ml, acc);
    }
  }
  dim3 cgrid(Hq, B);
  if (dh == 128) {
    if (out_bf16)
      decode_combine_kernel<128, true><<<cgrid, 128, 0, s>>>(out, ml, acc, ctx, Hq, Hkv, max_ctx, vs,
                                                             per_head, plan.part_blocks, plan.nsplit);
    else
      decode_combine_kernel<128, false><<<cgrid, 128, 0, s>>>(out, ml, acc, ctx, Hq, Hkv, max_ctx,
                                                              vs, per_head, plan.part_blocks,
                                                              plan.nsplit);
  } else {
    if (out_bf16)
      decode_combine_kernel<64, true><<<cgrid, 64, 0, s>>>(out, ml, acc, ctx, Hq, Hkv, max_ctx, vs,
                                                           per_head, plan.part_blocks, plan.nsplit);
    else
      decode_combine_kernel<64, false><<<cgrid, 64, 0, s>>>(out, ml, acc, ctx, Hq, Hkv, max_ctx, vs,
                                                            per_head, plan.part_blocks, plan.nsplit);
  }
  return hipGetLastError();
}

}  // namespace kvq

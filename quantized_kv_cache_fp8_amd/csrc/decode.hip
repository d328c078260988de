// decode.hip -- split-K paged decode attention over the FP8 cache, with the
// dequantization fused in.
//
// Computes, per sequence b and query head hq (KV head h = hq / G):
//   z_j = (q . k_hat_j) / sqrt(dh),  P = softmax(z),  o = sum_j P_j v_hat_j
// with k_hat = sK * cast_float(K8) and v_hat = sV * cast_float(V8): the
// attention equation and the fused dequant + attention path of the KV-cache
// quantization textbook (section 10.4.2) on the FP8 storage of section
// 10.4.5.  No dequantized copy of the cache exists anywhere: codes go from HBM
// into registers, are converted there (exactly: every E4M3/E5M2 value is a
// bf16 and an f16 value) and feed the matrix cores.
//
// Work decomposition (flash-decoding): grid = (Hq / NH, nsplit, B), head
// groups fastest.  A workgroup of 4 waves owns one split (part_blocks cache
// blocks of 16 tokens) of one sequence and the NH <= 16 query heads that share
// one KV head, so every K/V byte is read from HBM once and serves all NH
// heads.  Wave w takes
// block pairs w, w + 4, ... of the split, one pair (32 tokens) per step:
//
//   S = Q K^T on v_mfma_f32_16x16x32_bf16: A = the NH query rows (bf16, rows
//     NH..15 zero), B = the 16 tokens of a block (codes -> bf16 in registers;
//     each lane holds 32 code bytes of one token).
//   online softmax per row in the log2 domain, the running max raised lazily;
//     the S tile and the O tile map rows to lanes the same way, so rescaling
//     is lane-local.
//   O += P V on v_mfma_f32_16x16x32_f16: A = P of the pair (transposed
//     through a 1 KB per-wave LDS scratch), B = V from the channel-major tile
//     (each lane holds the 8 contiguous token bytes of one channel, -> f16).
//
// The next pair's keys are loaded as soon as the current keys are consumed and
// its values as soon as the current values are; registers are not doubled.  The
// 4 waves' (m, l, O) are merged through LDS and the split's partial goes to
// the workspace; a second kernel merges the splits (log-sum-exp), applies sV.
//
// Q K^T stays on bf16 (not FP8) matrix cores on purpose: the FP8 MFMA's
// internal accumulation keeps only about 16 bits relative to the largest
// product, which at decode-sized logits (tens in log2 units) is visible in
// the output, whereas bf16 products accumulate in full fp32.
#include <mutex>

#include "attn_common.hpp"
#include "launch.hpp"

namespace kvq {

// Tuning constants (each measured against its alternatives on the
// Llama-3-8B-shaped layer):
// query heads per combine workgroup (when it divides Hq)
constexpr int kCombineHeadsPerWg = 4;
// split sizes (cache blocks per workgroup), largest first: the plan takes the
// first that still gives the grid enough workgroups to fill the chip, so
// smaller splits are taken only for short contexts or small batches.  A split
// kernel instance covers 8 N blocks (4 waves, N block pairs each), and one is
// built for each of these sizes.
constexpr int kSplitBlocks[] = {40, 32, 16, 8};
// workgroups a plan aims for (about 1.6 rounds of resident workgroups)
constexpr int64_t kFillWgs = 2048;
// waves per SIMD of the generic split kernel: its whole state (Q operand, one
// block pair of codes, the O tile) fits in 128 registers
constexpr int kWavesPerSimd = 4;
// ... of the kernel for groups of at most 4 heads, and of its
// per-token-head-scale variant (114 registers at 4 waves; held to 94 for 5
// waves it spills nothing but times the same, 52.1 against 52.2 us on the
// Llama-shaped layer, so the allocator keeps its room)
constexpr int kG4WavesPerSimd = 5;
constexpr int kTsWavesPerSimd = 4;
// waves per workgroup of the kernel for groups of at most 4 heads
constexpr int kG4Waves = 4;

namespace {
constexpr int kBlockSize = 16;  // tokens per cache block
}  // namespace

// dynamic LDS bytes for one workgroup: per-wave P transpose scratch
// [4][16 rows][32 tokens] f16, then the wave-merge buffers.
static size_t decode_lds_bytes(int NH, int dh) {
  return 4 * 16 * 32 * sizeof(_Float16) + 2 * 4 * 16 * sizeof(float) +
         (size_t)4 * NH * dh * sizeof(float) + 2 * (size_t)dh;  // + appended token's codes
}
static size_t decode_g4_lds_bytes(int NH, int dh) {
  constexpr int NW = kG4Waves;
  return NW * 16 * 32 * sizeof(_Float16) + 2 * NW * 16 * sizeof(float) +
         (size_t)NW * NH * dh * sizeof(float) + 2 * (size_t)dh;  // + appended token's codes
}

// Lazy running max: it only moves when a score exceeds it by more than 2^8,
// so p = exp2(z - m) <= 256 (safe in f16) and accumulator rescales are rare.
constexpr float kLazyTau = 8.0f;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Channel slot i (0 or 1) of lane group g4: 16 contiguous channels at
// 16 g4 + i * DH / 2, present when g4 < DH / 32 (dh = 64 uses two groups).
template <int DH>
__device__ __forceinline__ bool chan_group_live(int g4) { return g4 < DH / 32; }

// Rows of the 16-row MFMA tiles are given to query heads in runs of
// RPH = 16 / NHp rows per head (NHp = NH rounded up to a power of two), so
// S and O rows come out replicated per head.  A lane holding S rows
// 4 g4 .. 4 g4 + 3 then holds HPL = max(1, NHp / 4) distinct heads, and the
// softmax is computed once per (head, token) rather than once per row.
template <int HPL>
struct LaneHeads {
  static constexpr int kStride = 4 / HPL;  // S register of distinct head i: r = i * kStride
};

// Append (decode step with the new token fused in): if this workgroup's split
// holds position ctx - 1, quantize that token's K and V for head h (the write
// kernels' codec arithmetic) into pw [2][DH] in LDS, store them into the cache
// when `writer` (one workgroup per KV head), and return the block pair,
// block and offset at which the caller patches them into its registers.
// Every thread of the workgroup calls it (it holds a barrier).
template <int FMT, int DH, int NT = 256>
__device__ __forceinline__ void append_prologue(
    int ctx, int tok0, int nblk, const int32_t* __restrict__ btab, int64_t num_blocks,
    int64_t bstride, int h, int Hkv, int b, bool writer, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const float* __restrict__ ks,
    const float* __restrict__ vs, int per_head, uint8_t* kc_w, uint8_t* vc_w, uint8_t* pw,
    int& p_new, int& e_new, int& off_new) {
  const int bi = (ctx - 1 - tok0) / kBlockSize;  // tok0 < ctx, so bi >= 0
  if (bi >= nblk) return;                        // the same for the whole workgroup
  const int tid = threadIdx.x;
  const size_t tile = (size_t)kBlockSize * DH;
  p_new = bi >> 1;
  e_new = bi & 1;
  off_new = (ctx - 1) & (kBlockSize - 1);
  // the block id goes out with the token's values (it does not depend on
  // them), so the store below waits for one memory round trip, not two
  const int64_t raw = btab[bi];
  for (int i = tid; i < 2 * DH; i += NT) {
    const bool isv = i >= DH;
    const int d = isv ? i - DH : i;
    const uint16_t x = (isv ? v_new : k_new)[((size_t)b * Hkv + h) * DH + d];
    const float qv = quotient(__uint_as_float((uint32_t)x << 16),
                              make_divisor((isv ? vs : ks)[per_head ? h : 0]));
    pw[i] = (uint8_t)(enc2<FMT>(qv, qv) & 0xffu);
  }
  __syncthreads();
  if (writer && raw >= 0 && raw < num_blocks) {
    uint8_t* kt = kc_w + (size_t)raw * bstride + (size_t)h * tile;
    uint8_t* vt = vc_w + (size_t)raw * bstride + (size_t)h * tile;
    if (tid < DH / 16)
      *reinterpret_cast<uint4*>(kt + tid * 256 + off_new * 16) =
          *reinterpret_cast<const uint4*>(pw + 16 * tid);
    // V codes from the second wave on (the first stores K), or from every
    // thread when the workgroup has one wave
    const int v0 = NT > 64 ? 64 : 0;
    for (int i = tid - v0; i >= 0 && i < DH; i += NT - v0)
      vt[i * kBlockSize + off_new] = pw[DH + i];
  }
}

template <int FMT, int DH, int NPW, int HPL, bool APPEND>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd))) void
decode_split_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
                    const uint8_t* __restrict__ vc, int64_t num_blocks, int64_t bstride,
                    const int32_t* __restrict__ bt, int max_blocks,
                    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int NH, int rph_shift,
                    int max_ctx, const float* __restrict__ ks, int per_head, float sm_scale,
                    int nsplit, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
                    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
                    uint8_t* kc_w, uint8_t* vc_w, const float* __restrict__ vs) {
  constexpr int NV = DH / 16;   // f16 MFMAs per block pair (16 channels each)
  constexpr int PB = 8 * NPW;   // blocks per split: 4 waves x NPW pairs x 2
  constexpr int HALF = DH / 2;
  constexpr int RS = LaneHeads<HPL>::kStride;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int split = blockIdx.y;
  const int grp = blockIdx.x, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int gpk = G / NH;
  const int h = grp / gpk;
  const int hq0 = h * G + (grp - h * gpk) * NH;

  // a context beyond the host bound is attended up to the bound; the append
  // then neither writes nor attends the new token (its true slot lies past
  // what this launch covers)
  const int ctx_raw = ctx_lens[b];
  const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > max_ctx ? max_ctx : ctx_raw);
  const int tok0 = split * PB * kBlockSize;
  if (tok0 >= ctx) return;  // nothing of this sequence lies in this split
  const int nblk_left = (ctx - tok0 + kBlockSize - 1) / kBlockSize;
  const int nblk = nblk_left < PB ? nblk_left : PB;
  const int npair = (nblk + 1) >> 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int rph_mask = (1 << rph_shift) - 1;
  // A operands (Q for S, P for O): row c16 carries head c16 / RPH
  const int head_a = c16 >> rph_shift;
  const bool head_a_real = head_a < NH;
  const bool chan_live = chan_group_live<DH>(g4);
  _Float16* ptr = reinterpret_cast<_Float16*>(smem) + wave * 16 * 32;  // this wave's P scratch
  float* wm = reinterpret_cast<float*>(smem + 4 * 16 * 32 * sizeof(_Float16));
  float* wl = wm + 4 * 16;
  float* wo = wl + 4 * 16;  // [4][NH][DH]
  const int32_t* btab = bt + (size_t)b * max_blocks + (size_t)split * PB;
  const size_t tile = (size_t)kBlockSize * DH;  // bytes per (block, head) tile
  const int eb = g4 >> 1, tk = 8 * (g4 & 1);   // V: this lane's block in a pair, token half

  // distinct heads of this lane's S / O rows, and whether this lane group is
  // the first copy of each (the one that publishes P and the results)
  int head_l[HPL];
  bool pub_l[HPL];
#pragma unroll
  for (int i = 0; i < HPL; ++i) {
    const int row = 4 * g4 + i * RS;
    head_l[i] = row >> rph_shift;
    pub_l[i] = (row & rph_mask) == 0 && head_l[i] < NH;
  }

  // A block pair (2 blocks of 16 tokens).  K: lane holds the 32 code bytes of
  // token c16 in channel slots 16 g4 + [0,16) and DH/2 + 16 g4 + [0,16) (K
  // tiles are [DH/16 chunks][16 tokens][16 channels]).
  // V: lane holds tokens tk .. tk + 7 of block eb for channel 16 n + c16.
  // Blocks past the split's end re-read its last block; their scores are
  // masked and their values zeroed, so nothing outside the table is read.
  i32x8 kr[2];
  uint2 vr[NV];
  auto block_src = [&](int bi) {
    bi = bi < nblk ? bi : nblk - 1;
    return (size_t)clamp_block(btab[bi], num_blocks) * bstride + (size_t)h * tile;
  };
  auto load_k = [&](int p, i32x8 (&kr)[2]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kr[e] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (chan_live) {
        // chunks g4 and DH/32 + g4 (channels 16 g4 + [0,16) and DH/2 + 16 g4 + [0,16))
        // of token c16: each of the two loads covers 16 tokens x 4 chunks, i.e.
        // DH/32 KB of contiguous tile
        const uint8_t* src = kc + block_src(2 * p + e) + g4 * 256 + c16 * 16;
        const uint4 a0 = load16(src);
        const uint4 a1 = load16(src + HALF * 16);
        kr[e] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      }
    }
  };
  auto load_v = [&](int p, uint2 (&vr)[NV]) {
    const uint8_t* src = vc + block_src(2 * p + eb) + c16 * kBlockSize + tk;
#pragma unroll
    for (int n = 0; n < NV; ++n) vr[n] = load8(src + 16 * n * kBlockSize);
  };

  // A operand of S = Q K^T (bf16, exact): query head_a in the channel slots
  // of the K operand: j = 2 i + c covers channels 16 g4 + i * DH/2 + 8 c + 0..7.
  // Q is loaded first and waited for before the loop (the empty asm uses its
  // registers) while the first pair's K and V stay in flight, so no load
  // issued before the loop is still pending at its head.
  uint4 qw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qw[j] = make_uint4(0, 0, 0, 0);
    if (head_a_real && chan_live)
      qw[j] = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + hq0 + head_a) * DH +
                                              16 * g4 + (j >> 1) * HALF + 8 * (j & 1));
  }
  int p = wave;
  if (p < npair) {
    load_k(p, kr);
    load_v(p, vr);
  }
  bf16x8 qop[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    asm volatile("" ::"v"(qw[j].x), "v"(qw[j].y), "v"(qw[j].z), "v"(qw[j].w));
    qop[j] = __builtin_bit_cast(bf16x8, qw[j]);
  }
  // ---- append: the new token (position ctx - 1) of this sequence
  int p_new = -1, e_new = 0, off_new = 0;
  uint8_t* pw = reinterpret_cast<uint8_t*>(wo + 4 * NH * DH);  // [2][DH]: K codes, V codes
  const uint8_t* patch = pw;
  if constexpr (APPEND)
    if (ctx_raw <= max_ctx)
      append_prologue<FMT, DH>(ctx, tok0, nblk, btab, num_blocks, bstride, h, Hkv, b,
                             grp == h * gpk, k_new, v_new, ks, vs, per_head, kc_w, vc_w, pw,
                             p_new, e_new, off_new);
  const float zc = sm_scale * ks[per_head ? h : 0] * kLog2e;

  // running state per distinct head (identical across the 16 lanes of a group)
  float m_run[HPL], l_part[HPL];
#pragma unroll
  for (int i = 0; i < HPL; ++i) {
    m_run[i] = kNegBig;
    l_part[i] = 0.0f;  // this lane's token share of the row sum
  }
  f32x4 O[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) O[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // one block pair: S, online softmax, P V (kr / vr hold the pair's codes)
  // (with `pre` the wave's next pair is loaded as registers free up)
  auto pair_step = [&](int p, i32x8 (&kr)[2], uint2 (&vr)[NV], bool pre)
      __attribute__((always_inline)) {
    // ---- S for both blocks on bf16 matrix cores (codes -> bf16 is exact):
    //      lane holds head head_l[i] for token c16 of block e
    if constexpr (APPEND) {
      if (p == p_new && c16 == off_new && chan_live) {  // the appended token's K codes
        const uint4 a0 = *reinterpret_cast<const uint4*>(patch + 16 * g4);
        const uint4 a1 = *reinterpret_cast<const uint4*>(patch + HALF + 16 * g4);
        const i32x8 kn = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                               (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        if (e_new == 0) kr[0] = kn; else kr[1] = kn;
      }
    }
    float z[2][HPL];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      f32x4 S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qop[j], codes_to_bf16x8<FMT>((uint32_t)kr[e][2 * j], (uint32_t)kr[e][2 * j + 1]), S,
            0, 0, 0);
      const bool valid = tok0 + (2 * p + e) * kBlockSize + c16 < ctx;
#pragma unroll
      for (int i = 0; i < HPL; ++i) z[e][i] = valid ? S[i * RS] * zc : -__builtin_inff();
    }
    // this pair's K registers are free: the next pair's keys load during the
    // softmax and P V below
    if (pre) load_k(p + 4, kr);
    // ---- online softmax per head.  Each lane tests its own scores against
    //      the running max; only when one exceeds it by more than tau does the
    //      wave take the (rare, wave-uniform) branch that finds the exact
    //      maxima of the 16-lane groups and rescales.  The O tile maps rows to
    //      lanes as the S tile does, so the rescale is lane-local.
    bool need = false;
#pragma unroll
    for (int i = 0; i < HPL; ++i)
      need |= __builtin_fmaxf(z[0][i], z[1][i]) > m_run[i] + kLazyTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
      for (int i = 0; i < HPL; ++i) {
        const float mt = max16(__builtin_fmaxf(z[0][i], z[1][i]));
        const bool up = mt > m_run[i] + kLazyTau;
        const float f = up ? __builtin_amdgcn_exp2f(m_run[i] - mt) : 1.0f;
        m_run[i] = up ? mt : m_run[i];
        l_part[i] *= f;
#pragma unroll
        for (int n = 0; n < NV; ++n)
#pragma unroll
          for (int r = i * RS; r < (i + 1) * RS; ++r) O[n][r] *= f;
      }
    }
#pragma unroll
    for (int i = 0; i < HPL; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(z[0][i] - m_run[i]);
      const float p1 = __builtin_amdgcn_exp2f(z[1][i] - m_run[i]);
      l_part[i] += p0 + p1;
      if (pub_l[i]) {
        ptr[head_l[i] * 32 + c16] = (_Float16)p0;
        ptr[head_l[i] * 32 + 16 + c16] = (_Float16)p1;
      }
    }
    // ---- P V on f16 matrix cores: A = P of head head_a, tokens 8 g4 .. 8 g4 + 7.
    //      Value codes of tokens past the context (the tail of the last block,
    //      or a re-read block) may hold anything, NaN included: zero them,
    //      since their zero weights would not cancel a NaN.
    if constexpr (APPEND) {
      // the appended token's V codes: byte off_new - tk of this lane's 8-token run
      if (p == p_new && eb == e_new && off_new >= tk && off_new < tk + 8) {
        const int sh = 8 * ((off_new - tk) & 3);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
          const uint32_t code = patch[DH + 16 * n + c16];
          if (off_new - tk < 4) vr[n].x = (vr[n].x & ~(0xffu << sh)) | (code << sh);
          else vr[n].y = (vr[n].y & ~(0xffu << sh)) | (code << sh);
        }
      }
    }
    if (2 * p + 2 > nblk_left || tok0 + (2 * p + 2) * kBlockSize > ctx) {
      const int left = ctx - (tok0 + (2 * p + eb) * kBlockSize + tk);
      const uint64_t keep = left >= 8 ? ~0ull : (left <= 0 ? 0ull : (1ull << (8 * left)) - 1);
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        vr[n].x &= (uint32_t)keep;
        vr[n].y &= (uint32_t)(keep >> 32);
      }
    }
    f16x8 pop = {};
    if (head_a_real) pop = *reinterpret_cast<const f16x8*>(ptr + head_a * 32 + 8 * g4);
#pragma unroll
    for (int n = 0; n < NV; ++n)
      O[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, codes_to_f16x8<FMT>(vr[n].x, vr[n].y),
                                                    O[n], 0, 0, 0);
    if (pre) load_v(p + 4, vr);  // V registers are free now
    };

  // the last pair runs without loads, so inside the loop both prefetches
  // always happen and a pair's K wait never covers its V codes too
#pragma unroll 1
  for (; p + 4 < npair; p += 4) pair_step(p, kr, vr, true);
  if (p < npair) pair_step(p, kr, vr, false);

  // ---- merge the 4 waves through LDS and write the split's partial
#pragma unroll
  for (int i = 0; i < HPL; ++i) {
    float x = l_part[i];
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    if (pub_l[i]) {
      const int hh = head_l[i];
      if (c16 == 0) {
        wm[wave * 16 + hh] = m_run[i];
        wl[wave * 16 + hh] = x;
      }
#pragma unroll
      for (int n = 0; n < NV; ++n) wo[(wave * NH + hh) * DH + 16 * n + c16] = O[n][i * RS];
    }
  }
  __syncthreads();
  for (int o = tid; o < NH * DH; o += 256) {
    const int row = o / DH, d = o - row * DH;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = __builtin_fmaxf(M, wm[w * 16 + row]);
    float a = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w * 16 + row] - M);
      a += f * wo[(w * NH + row) * DH + d];
      L += f * wl[w * 16 + row];
    }
    const size_t ridx = ((size_t)b * Hq + hq0 + row) * nsplit + split;
    ws_acc[ridx * DH + d] = a;
    if (d == 0) {
      ws_ml[ridx * 2 + 0] = M;
      ws_ml[ridx * 2 + 1] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// Groups of at most 4 query heads (G <= 4: the Llama-3 shape has G = 4).
// Q K^T and the softmax are as above (one distinct head per lane, rows
// replicated).  P V runs on v_mfma_f32_4x4x4_16b_f16 instead: 16 independent
// 4x4x4 products per instruction, where D[r][c] = sum_k A[r][k] B[k][c] with
// A row r in lane 4 blk + r, B and D column c in lane 4 blk + c and D's rows in
// that lane's 4 registers.  So lane l owns channel l (and 64 + l) of the
// output, for all 4 heads at once (8 accumulator registers, not 32):
//   A = P[head l % 4][4 tokens], B = V[4 tokens][channel l] (4 code bytes of
//   the channel's row in the channel-major tile),
// and each lane loads its channel's 16 token bytes per block: one 64-lane load
// is 1 KB of contiguous tile.
// MODE 0: scales per tensor or per head; 1: per-token-head fp16 scales (TS);
// 2: append -- the workgroup whose split holds position ctx - 1 quantizes the
// new token (k_new / v_new), writes its codes to the cache and patches them
// into its own K / V registers, so no workgroup reads that slot from memory.
template <int FMT, int DH, int NPW, int MODE>
__global__ __launch_bounds__(64 * kG4Waves)
__attribute__((amdgpu_waves_per_eu(MODE == 1 ? kTsWavesPerSimd
                                                : kG4WavesPerSimd,
                                    MODE == 1 ? kTsWavesPerSimd
                                                : kG4WavesPerSimd)))
void
decode_split_g4_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kc,
                       const uint8_t* __restrict__ vc, int64_t num_blocks, int64_t bstride,
                       const int32_t* __restrict__ bt, int max_blocks,
                       const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int NH,
                       int rph_shift, int max_ctx, const float* __restrict__ ks, int per_head,
                       float sm_scale, int nsplit, float* __restrict__ ws_ml,
                       float* __restrict__ ws_acc, const uint16_t* __restrict__ ksc,
                       const uint16_t* __restrict__ vsc, const uint16_t* __restrict__ k_new,
                       const uint16_t* __restrict__ v_new, uint8_t* kc_w, uint8_t* vc_w,
                       const float* __restrict__ vs) {
  constexpr bool TS = MODE == 1, APPEND = MODE == 2;
  typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
  constexpr int NW = kG4Waves;  // waves per workgroup
  constexpr int PB = 2 * NW * NPW;      // blocks per split: NW waves x NPW pairs x 2
  constexpr int HALF = DH / 2;
  constexpr int NC = DH / 64;     // 64-channel halves of the output
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int split = blockIdx.y;
  const int grp = blockIdx.x, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int gpk = G / NH;
  const int h = grp / gpk;
  const int hq0 = h * G + (grp - h * gpk) * NH;

  // a context beyond the host bound is attended up to the bound; the append
  // then neither writes nor attends the new token (its true slot lies past
  // what this launch covers)
  const int ctx_raw = ctx_lens[b];
  const int ctx = ctx_raw < 0 ? 0 : (ctx_raw > max_ctx ? max_ctx : ctx_raw);
  const int tok0 = split * PB * kBlockSize;
  if (tok0 >= ctx) return;  // nothing of this sequence lies in this split
  const int nblk_left = (ctx - tok0 + kBlockSize - 1) / kBlockSize;
  const int nblk = nblk_left < PB ? nblk_left : PB;
  const int npair = (nblk + 1) >> 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int rph_mask = (1 << rph_shift) - 1;
  const int head_a = c16 >> rph_shift;  // Q row of S's A operand
  const bool head_a_real = head_a < NH;
  const bool chan_live = chan_group_live<DH>(g4);
  // this lane's head in the S tile, and whether its lane group publishes P
  const int head_s = (4 * g4) >> rph_shift;
  const bool pub = ((4 * g4) & rph_mask) == 0 && head_s < NH;
  // P V: A row of this lane (head lane % 4), and the lane that holds head r's
  // running state in the S layout (first lane of its first lane group)
  const int head_p = lane & 3;
  // LDS (decode_g4_lds_bytes): per wave P scratch [16][32] f16, then the
  // waves' m and l [NW][16] and O [NW][NH][DH], then the appended token's codes
  _Float16* ptr = reinterpret_cast<_Float16*>(smem) + wave * 16 * 32;  // this wave's P scratch
  float* wm = reinterpret_cast<float*>(smem + NW * 16 * 32 * sizeof(_Float16));
  float* wl = wm + NW * 16;
  float* wo = wl + NW * 16;  // [NW][NH][DH]
  const int32_t* btab = bt + (size_t)b * max_blocks + (size_t)split * PB;
  const size_t tile = (size_t)kBlockSize * DH;  // bytes per (block, head) tile

  i32x8 kr[2];
  uint4 vq[2][NC];  // [block of the pair][half]: 16 token codes of channel 64 half + lane
  uint32_t tsc[2];  // fp16 scales of token c16 of each block, sK | sV << 16 (TS)
  auto block_id = [&](int bi) {
    bi = bi < nblk ? bi : nblk - 1;
    return (size_t)clamp_block(btab[bi], num_blocks);
  };
  auto load_k = [&](int p) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      kr[e] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (chan_live) {
        const uint8_t* src = kc + block_id(2 * p + e) * bstride + h * tile + g4 * 256 + c16 * 16;
        const uint4 a0 = load16(src);
        const uint4 a1 = load16(src + HALF * 16);
        kr[e] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      }
      if constexpr (TS) {  // scale caches are [num_blocks][Hkv][16], never padded
        const size_t si = (block_id(2 * p + e) * Hkv + h) * kBlockSize + c16;
        tsc[e] = (uint32_t)ksc[si] | ((uint32_t)vsc[si] << 16);
      }
    }
  };
  auto load_v = [&](int p) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint8_t* src = vc + block_id(2 * p + e) * bstride + h * tile + lane * kBlockSize;
#pragma unroll
      for (int c = 0; c < NC; ++c) vq[e][c] = load16(src + c * 64 * kBlockSize);
    }
  };

  // Q first, then the first pair's K and V.  Q is waited for before the loop
  // (the empty asm uses its registers) while K and V stay in flight: a load
  // issued before the loop and first used inside it would otherwise make that
  // use wait for every outstanding load, in every iteration.
  uint4 qw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qw[j] = make_uint4(0, 0, 0, 0);
    if (head_a_real && chan_live)
      qw[j] = *reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + hq0 + head_a) * DH +
                                              16 * g4 + (j >> 1) * HALF + 8 * (j & 1));
  }
  int p = wave;
  if (p < npair) {
    load_k(p);
    load_v(p);
  }
  bf16x8 qop[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    asm volatile("" ::"v"(qw[j].x), "v"(qw[j].y), "v"(qw[j].z), "v"(qw[j].w));
    qop[j] = __builtin_bit_cast(bf16x8, qw[j]);
  }
  // ---- append: the new token (position ctx - 1) of this sequence
  int p_new = -1, e_new = 0, off_new = 0;
  uint8_t* pw = reinterpret_cast<uint8_t*>(wo + NW * NH * DH);  // [2][DH]: K codes, V codes
  const uint8_t* patch = pw;
  if constexpr (APPEND)
    if (ctx_raw <= max_ctx)
      append_prologue<FMT, DH, 64 * NW>(ctx, tok0, nblk, btab, num_blocks, bstride, h, Hkv, b,
                             grp == h * gpk, k_new, v_new, ks, vs, per_head, kc_w, vc_w, pw,
                             p_new, e_new, off_new);

  // with per-token-head scales sK multiplies each score and log2 sV is added
  // to the exponent that forms P (the row sum l keeps the exponent without it)
  const float zc = sm_scale * (TS ? 1.0f : ks[per_head ? h : 0]) * kLog2e;

  float m_run = kNegBig, l_part = 0.0f;  // this lane's head (S layout)
  f32x4 O[NC];                           // O[c][r]: head r, channel 64 c + lane
#pragma unroll
  for (int c = 0; c < NC; ++c) O[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // One block pair: S, online softmax, P V.  With `pre` the next pair of this
  // wave is loaded as registers free up.  The last pair runs as a separate
  // step without loads, so inside the loop both prefetches always happen and
  // the wait for a pair's K codes never has to cover its V codes too.
  auto pair_step = [&](int p, bool pre) __attribute__((always_inline)) {
    // ---- S for both blocks (bf16 matrix cores, rows replicated per head)
    if constexpr (APPEND) {
      if (p == p_new && c16 == off_new && chan_live) {  // the appended token's K codes
        const uint4 a0 = *reinterpret_cast<const uint4*>(patch + 16 * g4);
        const uint4 a1 = *reinterpret_cast<const uint4*>(patch + HALF + 16 * g4);
        const i32x8 kn = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                               (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        if (e_new == 0) kr[0] = kn; else kr[1] = kn;
      }
    }
    float z[2], zp[2];  // log2-domain score; exponent of P (z + log2 sV with TS)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      f32x4 S = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            qop[j], codes_to_bf16x8<FMT>((uint32_t)kr[e][2 * j], (uint32_t)kr[e][2 * j + 1]), S,
            0, 0, 0);
      const bool valid = tok0 + (2 * p + e) * kBlockSize + c16 < ctx;
      if constexpr (TS) {
        const f16x2 sc = __builtin_bit_cast(f16x2, tsc[e]);
        z[e] = valid ? S[0] * zc * (float)sc[0] : -__builtin_inff();
        zp[e] = valid ? z[e] + __builtin_amdgcn_logf((float)sc[1]) : -__builtin_inff();
      } else {
        z[e] = valid ? S[0] * zc : -__builtin_inff();
        zp[e] = z[e];
      }
    }
    if (pre) load_k(p + NW);  // K registers are free
    // ---- online softmax (lazy max, wave-uniform rare rescale)
    const bool need = __builtin_fmaxf(zp[0], zp[1]) > m_run + kLazyTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mt = max16(__builtin_fmaxf(zp[0], zp[1]));
      const bool up = mt > m_run + kLazyTau;
      const float f = up ? __builtin_amdgcn_exp2f(m_run - mt) : 1.0f;
      m_run = up ? mt : m_run;
      l_part *= f;
      // head r's factor sits in lane (4 r) << rph_shift (first lane of its group)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r < NH) {
          const float fr = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), (4 * r) << rph_shift));
#pragma unroll
          for (int c = 0; c < NC; ++c) O[c][r] *= fr;
        }
      }
    }
    const float p0 = __builtin_amdgcn_exp2f(zp[0] - m_run);
    const float p1 = __builtin_amdgcn_exp2f(zp[1] - m_run);
    if constexpr (TS)
      l_part += __builtin_amdgcn_exp2f(z[0] - m_run) + __builtin_amdgcn_exp2f(z[1] - m_run);
    else
      l_part += p0 + p1;
    if (pub) {
      ptr[head_s * 32 + c16] = (_Float16)p0;
      ptr[head_s * 32 + 16 + c16] = (_Float16)p1;
    }
    // ---- value codes of slots past the context may hold anything (NaN
    //      included) and their zero weights would not cancel a NaN: zero them
    if (tok0 + (2 * p + 2) * kBlockSize > ctx) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int left = ctx - (tok0 + (2 * p + e) * kBlockSize);  // tokens inside the context
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int n = left - 4 * w;
          const uint32_t keep = n >= 4 ? 0xffffffffu : (n <= 0 ? 0u : (1u << (8 * n)) - 1);
#pragma unroll
          for (int c = 0; c < NC; ++c) u4word(vq[e][c], w) &= keep;
        }
      }
    }
    if constexpr (APPEND) {
      if (p == p_new) {  // the appended token's V codes: byte off_new of each channel's run
        const int wi = off_new >> 2, sh = 8 * (off_new & 3);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint32_t code = patch[DH + 64 * c + lane];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if (e != e_new) continue;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              uint32_t& d = u4word(vq[e][c], w);
              if (w == wi) d = (d & ~(0xffu << sh)) | (code << sh);
            }
          }
        }
      }
    }
    // ---- P V: 8 groups of 4 tokens x NC halves of 64 channels
    f16x8 pa[4] = {};
    if (head_p < NH) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = *reinterpret_cast<const f16x8*>(ptr + head_p * 32 + 8 * i);
    }
#pragma unroll
    for (int tq = 0; tq < 8; ++tq) {
      const f16x8 p8 = pa[tq >> 1];
      const f16x4 a = (tq & 1) ? f16x4{p8[4], p8[5], p8[6], p8[7]}
                               : f16x4{p8[0], p8[1], p8[2], p8[3]};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t codes = u4word(vq[tq >> 2][c], tq & 3);
        const f16x2 lo = dec2_f16<FMT, false>(codes), hi = dec2_f16<FMT, true>(codes);
        const f16x4 bv = {lo[0], lo[1], hi[0], hi[1]};
        O[c] = __builtin_amdgcn_mfma_f32_4x4x4f16(a, bv, O[c], 0, 0, 0);
      }
    }
    if (pre) load_v(p + NW);  // V registers are free
  };
#pragma unroll 1
  for (; p + NW < npair; p += NW) pair_step(p, true);
  if (p < npair) pair_step(p, false);

  // ---- merge the NW waves through LDS and write the split's partial
  float x = l_part;
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  if (pub && c16 == 0) {
    wm[wave * 16 + head_s] = m_run;
    wl[wave * 16 + head_s] = x;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (r < NH)
#pragma unroll
      for (int c = 0; c < NC; ++c) wo[(wave * NH + r) * DH + 64 * c + lane] = O[c][r];
  __syncthreads();
  for (int o = tid; o < NH * DH; o += 64 * NW) {
    const int row = o / DH, d = o - row * DH;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = __builtin_fmaxf(M, wm[w * 16 + row]);
    float a = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w * 16 + row] - M);
      a += f * wo[(w * NH + row) * DH + d];
      L += f * wl[w * 16 + row];
    }
    const size_t ridx = ((size_t)b * Hq + hq0 + row) * nsplit + split;
    ws_acc[ridx * DH + d] = a;
    if (d == 0) {
      ws_ml[ridx * 2 + 0] = M;
      ws_ml[ridx * 2 + 1] = L;
    }
  }
}

// grid (Hq / HPW, B), DH x HPW threads: merge the valid splits of HPW
// (b, hq) rows, one per thread row, one channel per thread (launched with one
// row per workgroup, for head counts the 4-channel kernel below does not take).
// Splits are taken 16 at a time, every load of a batch issued together (the
// (m, l) pairs are the same for all threads of the row: broadcast loads), and
// merged by log-sum-exp with a running maximum, so a typical row costs one
// round trip to memory and needs no LDS or barrier.
template <int DH, bool BF16, int HPW>
__global__ __launch_bounds__(DH * HPW) void decode_combine_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int max_ctx,
    const float* __restrict__ vs, int per_head, int part_blocks, int nsplit) {
  constexpr int kBatch = 16;
  const int hq = blockIdx.x * HPW + threadIdx.y, b = blockIdx.y, d = threadIdx.x;
  int nvalid = nsplit;  // part_blocks == 0: every split holds a partial (maybe empty)
  if (part_blocks > 0) {
    int ctx = ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
    const int span = part_blocks * kBlockSize;
    nvalid = (ctx + span - 1) / span;
  }
  const size_t row0 = ((size_t)b * Hq + hq) * nsplit;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  float M = kNegBig, L = 0.0f, a = 0.0f;
  for (int s0 = 0; s0 < nvalid; s0 += kBatch) {
    const int n = nvalid - s0 < kBatch ? nvalid - s0 : kBatch;
    float2 p[kBatch];
    float o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      p[j] = make_float2(kNegBig, 0.0f);
      o[j] = 0.0f;
      if (j < n) {
        p[j] = ml[row0 + s0 + j];
        o[j] = ws_acc[(row0 + s0 + j) * DH + d];
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mn = __builtin_fmaxf(Mn, p[j].x);
    const float f = __builtin_amdgcn_exp2f(M - Mn);
    L *= f;
    a *= f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = __builtin_amdgcn_exp2f(p[j].x - Mn);  // 0 for the padding entries
      L += w * p[j].y;
      a += w * o[j];
    }
    M = Mn;
  }
  const int h = hq / (Hq / Hkv);
  const float sv = vs ? vs[per_head ? h : 0] : 1.0f;  // null: sV already folded into P
  const float r = L > 0.0f ? a / L * sv : 0.0f;
  const size_t oi = ((size_t)b * Hq + hq) * DH + d;
  if constexpr (BF16)
    reinterpret_cast<uint16_t*>(out)[oi] = (uint16_t)f32_to_bf16_rne(r);
  else
    reinterpret_cast<float*>(out)[oi] = r;
}

// The same merge with each thread on 4 adjacent channels (16-byte partial
// loads and output stores): DH / 4 threads per row, HPW rows per workgroup,
// used whenever HPW divides Hq (the one-channel kernel above, one row per
// workgroup, serves the other head counts).  It needs the partials 16-byte
// aligned, i.e. an even B * Hq * nsplit (the (m, l) pairs come first), which
// an even HPW dividing Hq guarantees.  On the Llama-shaped layer it took 49.5 against
// 50.0 us per step for the one-channel merge, and 92.7 against 93.3 us on
// 32 x 8192 tokens (best of seven alternating rounds; 1, 2, 8 or 16 rows per
// workgroup were slower than 4).
template <int DH, bool BF16, int HPW>
__global__ __launch_bounds__(DH / 4 * HPW) void decode_combine4_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int max_ctx,
    const float* __restrict__ vs, int per_head, int part_blocks, int nsplit) {
  constexpr int kBatch = 16;
  const int hq = blockIdx.x * HPW + threadIdx.y, b = blockIdx.y, d4 = threadIdx.x;
  int nvalid = nsplit;  // part_blocks == 0: every split holds a partial (maybe empty)
  if (part_blocks > 0) {
    int ctx = ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
    const int span = part_blocks * kBlockSize;
    nvalid = (ctx + span - 1) / span;
  }
  const size_t row0 = ((size_t)b * Hq + hq) * nsplit;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  float M = kNegBig, L = 0.0f;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < nvalid; s0 += kBatch) {
    const int n = nvalid - s0 < kBatch ? nvalid - s0 : kBatch;
    float2 p[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      p[j] = make_float2(kNegBig, 0.0f);
      o[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (j < n) {
        p[j] = ml[row0 + s0 + j];
        o[j] = reinterpret_cast<const float4*>(ws_acc + (row0 + s0 + j) * DH)[d4];
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mn = __builtin_fmaxf(Mn, p[j].x);
    const float f = __builtin_amdgcn_exp2f(M - Mn);
    L *= f;
    a.x *= f;
    a.y *= f;
    a.z *= f;
    a.w *= f;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = __builtin_amdgcn_exp2f(p[j].x - Mn);  // 0 for the padding entries
      L += w * p[j].y;
      a.x += w * o[j].x;
      a.y += w * o[j].y;
      a.z += w * o[j].z;
      a.w += w * o[j].w;
    }
    M = Mn;
  }
  const int h = hq / (Hq / Hkv);
  const float sv = vs ? vs[per_head ? h : 0] : 1.0f;  // null: sV already folded into P
  const float r = L > 0.0f ? sv / L : 0.0f;
  const size_t oi = ((size_t)b * Hq + hq) * (DH / 4) + d4;
  if constexpr (BF16) {
    uint2 w;
    w.x = f32_to_bf16_rne(a.x * r) | (f32_to_bf16_rne(a.y * r) << 16);
    w.y = f32_to_bf16_rne(a.z * r) | (f32_to_bf16_rne(a.w * r) << 16);
    reinterpret_cast<uint2*>(out)[oi] = w;
  } else {
    reinterpret_cast<float4*>(out)[oi] = make_float4(a.x * r, a.y * r, a.z * r, a.w * r);
  }
}

// ---------------------------------------------------------------- static scratch
// Split partials of kvq_decode_attn_append_noalloc, for callers that cannot
// allocate: a file-scope device array (each GPU the library runs on holds its
// own copy until the process ends).  Host code never passes the array's name
// to a kernel -- on the host it only stands in for the device symbol -- but
// the address hipGetSymbolAddress returns for the current device.  Its
// contents need no initialisation: every partial the combine reads is written
// by the split kernel of the same call.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
void* g_scratch_ptr[kMaxScratchDevices];
std::once_flag g_scratch_once[kMaxScratchDevices];
}  // namespace

void* decode_static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
  });
  return g_scratch_ptr[dev];
}

// Rows with more than 16 splits (long contexts): grid (Hq, B), DH x kSL
// threads per (b, hq) row.  Split lane j of the block merges splits j, j + kSL,
// ... -- at most 16 of them in one batch for up to 16 kSL splits -- with every
// load of a batch issued together, and the kSL lanes' (M, L, a) are merged
// through LDS, so a row of up to 64 splits costs one round trip to memory
// instead of four.
constexpr int kSL = 4;
template <int DH, bool BF16>
__global__ __launch_bounds__(DH * kSL) void decode_combine_lanes_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int max_ctx,
    const float* __restrict__ vs, int per_head, int part_blocks, int nsplit) {
  constexpr int kBatch = 16;
  __shared__ float s_m[kSL], s_l[kSL][DH], s_a[kSL][DH];
  const int hq = blockIdx.x, b = blockIdx.y, d = threadIdx.x, j = threadIdx.y;
  int nvalid = nsplit;
  if (part_blocks > 0) {
    int ctx = ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
    const int span = part_blocks * kBlockSize;
    nvalid = (ctx + span - 1) / span;
  }
  const size_t row0 = ((size_t)b * Hq + hq) * nsplit;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  float M = kNegBig, L = 0.0f, a = 0.0f;
  for (int s0 = j; s0 < nvalid; s0 += kSL * kBatch) {
    float2 p[kBatch];
    float o[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int sp = s0 + i * kSL;
      p[i] = make_float2(kNegBig, 0.0f);
      o[i] = 0.0f;
      if (sp < nvalid) {
        p[i] = ml[row0 + sp];
        o[i] = ws_acc[(row0 + sp) * DH + d];
      }
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) Mn = __builtin_fmaxf(Mn, p[i].x);
    const float f = __builtin_amdgcn_exp2f(M - Mn);
    L *= f;
    a *= f;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = __builtin_amdgcn_exp2f(p[i].x - Mn);  // 0 for the padding entries
      L += w * p[i].y;
      a += w * o[i];
    }
    M = Mn;
  }
  if (d == 0) s_m[j] = M;
  s_l[j][d] = L;
  s_a[j][d] = a;
  __syncthreads();
  if (j != 0) return;
  float Mt = kNegBig;
#pragma unroll
  for (int i = 0; i < kSL; ++i) Mt = __builtin_fmaxf(Mt, s_m[i]);
  float Lt = 0.0f, at = 0.0f;
#pragma unroll
  for (int i = 0; i < kSL; ++i) {
    const float w = __builtin_amdgcn_exp2f(s_m[i] - Mt);
    Lt += w * s_l[i][d];
    at += w * s_a[i][d];
  }
  const int h = hq / (Hq / Hkv);
  const float sv = vs ? vs[per_head ? h : 0] : 1.0f;  // null: sV already folded into P
  const float r = Lt > 0.0f ? at / Lt * sv : 0.0f;
  const size_t oi = ((size_t)b * Hq + hq) * DH + d;
  if constexpr (BF16)
    reinterpret_cast<uint16_t*>(out)[oi] = (uint16_t)f32_to_bf16_rne(r);
  else
    reinterpret_cast<float*>(out)[oi] = r;
}

// The lanes merge with each thread on 4 adjacent channels (16-byte partial
// loads and output stores): DH / 4 x kSL threads per (b, hq) row.  It needs
// an even B * Hq * nsplit, which keeps the partials 16-byte aligned; the
// one-channel kernel above takes the other cases.  64 splits of 4 x 32768
// tokens: 48.7 against 49.2 us per step; 5 ragged sequences up to 32768
// tokens: 32.9 against 33.3 us; the KIVI decode 31.9 against 32.7 us (best of
// seven, seven and five alternating rounds).
template <int DH, bool BF16>
__global__ __launch_bounds__(DH / 4 * kSL) void decode_combine_lanes4_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ ctx_lens, int Hq, int Hkv, int max_ctx,
    const float* __restrict__ vs, int per_head, int part_blocks, int nsplit) {
  constexpr int kBatch = 16;
  __shared__ float s_m[kSL], s_l[kSL];
  __shared__ float4 s_a[kSL][DH / 4];
  const int hq = blockIdx.x, b = blockIdx.y, d4 = threadIdx.x, j = threadIdx.y;
  int nvalid = nsplit;  // part_blocks == 0: every split holds a partial (maybe empty)
  if (part_blocks > 0) {
    int ctx = ctx_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > max_ctx ? max_ctx : ctx);
    const int span = part_blocks * kBlockSize;
    nvalid = (ctx + span - 1) / span;
  }
  const size_t row0 = ((size_t)b * Hq + hq) * nsplit;
  const float2* ml = reinterpret_cast<const float2*>(ws_ml);
  float M = kNegBig, L = 0.0f;
  float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = j; s0 < nvalid; s0 += kSL * kBatch) {
    float2 p[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int sp = s0 + i * kSL;
      p[i] = make_float2(kNegBig, 0.0f);
      o[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (sp < nvalid) {
        p[i] = ml[row0 + sp];
        o[i] = reinterpret_cast<const float4*>(ws_acc + (row0 + sp) * DH)[d4];
      }
    }
    float Mn = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) Mn = __builtin_fmaxf(Mn, p[i].x);
    const float f = __builtin_amdgcn_exp2f(M - Mn);
    L *= f;
    a.x *= f;
    a.y *= f;
    a.z *= f;
    a.w *= f;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = __builtin_amdgcn_exp2f(p[i].x - Mn);  // 0 for the padding entries
      L += w * p[i].y;
      a.x += w * o[i].x;
      a.y += w * o[i].y;
      a.z += w * o[i].z;
      a.w += w * o[i].w;
    }
    M = Mn;
  }
  if (d4 == 0) {
    s_m[j] = M;
    s_l[j] = L;
  }
  s_a[j][d4] = a;
  __syncthreads();
  if (j != 0) return;
  float Mt = kNegBig;
#pragma unroll
  for (int i = 0; i < kSL; ++i) Mt = __builtin_fmaxf(Mt, s_m[i]);
  float Lt = 0.0f;
  float4 at = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
  for (int i = 0; i < kSL; ++i) {
    const float w = __builtin_amdgcn_exp2f(s_m[i] - Mt);
    const float4 x = s_a[i][d4];
    Lt += w * s_l[i];
    at.x += w * x.x;
    at.y += w * x.y;
    at.z += w * x.z;
    at.w += w * x.w;
  }
  const int h = hq / (Hq / Hkv);
  const float sv = vs ? vs[per_head ? h : 0] : 1.0f;  // null: sV already folded into P
  const float r = Lt > 0.0f ? sv / Lt : 0.0f;
  const size_t oi = ((size_t)b * Hq + hq) * (DH / 4) + d4;
  if constexpr (BF16) {
    uint2 w2;
    w2.x = f32_to_bf16_rne(at.x * r) | (f32_to_bf16_rne(at.y * r) << 16);
    w2.y = f32_to_bf16_rne(at.z * r) | (f32_to_bf16_rne(at.w * r) << 16);
    reinterpret_cast<uint2*>(out)[oi] = w2;
  } else {
    reinterpret_cast<float4*>(out)[oi] = make_float4(at.x * r, at.y * r, at.z * r, at.w * r);
  }
}

static int heads_per_group(int G) {
  // largest divisor of G that fits the 16 rows of one MFMA tile
  for (int n = G < 16 ? G : 16; n >= 1; --n)
    if (G % n == 0) return n;
  return 1;
}

DecodePlan decode_plan(int B, int Hq, int dh, int max_context_len, int bs) {
  DecodePlan p{0, 0, 0};
  if (B < 1 || Hq < 1 || dh < 1 || bs < 1 || max_context_len < 0) return p;
  const int64_t nb = ((int64_t)max_context_len + bs - 1) / bs;
  const int64_t groups = (int64_t)B * (Hq >= 4 ? Hq / 4 : 1);
  // splits per sequence that give the grid kFillWgs workgroups
  const int64_t fill = (kFillWgs + groups - 1) / groups;
  // the largest split that still fills the chip (8 blocks if none does).
  // 40-block splits first: 49.9 against 50.4 us per step for 32 on the
  // Llama-shaped layer (ragged contexts up to 8192), 93.2 against 94.5 us on
  // 32 x 8192 tokens (best of seven alternating rounds); 48 and 56 blocks gain
  // less on the ragged layer, 24 loses everywhere.
  int P = 8;
  for (int c : kSplitBlocks)
    if ((nb + c - 1) / c >= fill) {
      P = c;
      break;
    }
  p.part_blocks = P;
  p.nsplit = (int)(nb > 0 ? (nb + P - 1) / P : 1);
  // The workspace holds the most splits any max_context_len up to this one
  // plans, so a workspace sized for the longest context serves every shorter
  // call: a shorter context can take a smaller split and so more splits.
  // Below the 16-block threshold, 16 (fill - 1) blocks, the plan takes 8-block
  // splits, ceil(nb / 8) of them; above it no plan exceeds 2 (fill - 1) splits
  // save its own (a 16-block plan stops at 32 (fill - 1) blocks, a 32-block
  // plan at 40 (fill - 1)).
  int64_t ws_splits = p.nsplit;
  const int64_t short_splits = (nb + 7) / 8 < 2 * (fill - 1) ? (nb + 7) / 8 : 2 * (fill - 1);
  if (short_splits > ws_splits) ws_splits = short_splits;
  p.ws_bytes = (size_t)B * Hq * (size_t)ws_splits * (2 + dh) * sizeof(float);
  return p;
}

hipError_t launch_decode(void* out, int out_bf16, const uint16_t* q, const uint8_t* kc,
                         const uint8_t* vc, int64_t num_blocks, const int32_t* bt,
                         int max_blocks, const int32_t* ctx, int B, int Hq, int Hkv, int dh,
                         int max_ctx, const float* ks, const float* vs, int fmt, int per_head,
                         float softmax_scale, const DecodePlan& plan, void* ws, hipStream_t s,
                         const uint16_t* ksc, const uint16_t* vsc, int64_t bstride,
                         const uint16_t* k_new, const uint16_t* v_new, uint8_t* kc_w,
                         uint8_t* vc_w) {
  const bool ts = ksc != nullptr;  // per-token-head fp16 scales (groups of <= 4 heads only)
  const bool app = k_new != nullptr;  // fused append (groups of <= 4 heads only)
  if (bstride <= 0) bstride = (int64_t)Hkv * kBlockSize * dh;
  const int G = Hq / Hkv;
  const int NH = heads_per_group(G);
  float* ml = reinterpret_cast<float*>(ws);
  float* acc = ml + (size_t)B * Hq * plan.nsplit * 2;
  const float sm = softmax_scale > 0.0f ? softmax_scale : 1.0f / __builtin_sqrtf((float)dh);
  const dim3 grid(Hq / NH, plan.nsplit, B);  // head groups of one split dispatch together
  const size_t lds = decode_lds_bytes(NH, dh);
  int nhp_shift = 0;
  while ((1 << nhp_shift) < NH) ++nhp_shift;  // NHp = 2^nhp_shift >= NH
  const int rph_shift = 4 - nhp_shift;         // RPH = 16 / NHp rows per head
  if (max_ctx > 0) {
#define KVQ_SPLIT(F, D, N, HP)                                                              \
  do {                                                                                      \
    if (app)                                                                                \
      decode_split_kernel<F, D, N, HP, true><<<grid, 256, lds, s>>>(                         \
          q, kc, vc, num_blocks, bstride, bt, max_blocks, ctx, Hq, Hkv, NH, rph_shift,       \
          max_ctx, ks, per_head, sm, plan.nsplit, ml, acc, k_new, v_new, kc_w, vc_w, vs);    \
    else                                                                                    \
      decode_split_kernel<F, D, N, HP, false><<<grid, 256, lds, s>>>(                        \
          q, kc, vc, num_blocks, bstride, bt, max_blocks, ctx, Hq, Hkv, NH, rph_shift,       \
          max_ctx, ks, per_head, sm, plan.nsplit, ml, acc, k_new, v_new, kc_w, vc_w, vs);    \
  } while (0)
#define KVQ_SPLIT_G4(F, D, N, M)                                                           \
  decode_split_g4_kernel<F, D, N * 4 / kG4Waves, M>                                   \
      <<<grid, 64 * kG4Waves, decode_g4_lds_bytes(NH, dh), s>>>(                    \
      q, kc, vc, num_blocks, bstride, bt, max_blocks, ctx, Hq, Hkv, NH, rph_shift, max_ctx, ks, \
      per_head, sm, plan.nsplit, ml, acc, ksc, vsc, k_new, v_new, kc_w, vc_w, vs)
#define KVQ_SPLIT_HP(F, D, N)                                     \
  do {                                                            \
    if (ts) KVQ_SPLIT_G4(F, D, N, 1);                             \
    else if (nhp_shift <= 2 && app) KVQ_SPLIT_G4(F, D, N, 2);     \
    else if (nhp_shift <= 2) KVQ_SPLIT_G4(F, D, N, 0);            \
    else if (nhp_shift == 3) KVQ_SPLIT(F, D, N, 2);               \
    else KVQ_SPLIT(F, D, N, 4);                                   \
  } while (0)
#define KVQ_SPLIT_NP(F, D)                                    \
  do {                                                        \
    if (plan.part_blocks == 40) KVQ_SPLIT_HP(F, D, 5);        \
    else if (plan.part_blocks == 32) KVQ_SPLIT_HP(F, D, 4);   \
    else if (plan.part_blocks == 16) KVQ_SPLIT_HP(F, D, 2);   \
    else KVQ_SPLIT_HP(F, D, 1);                               \
  } while (0)
    // any other split size would cover only part of each split
    if (plan.part_blocks != 8 && plan.part_blocks != 16 && plan.part_blocks != 32 &&
        plan.part_blocks != 40)
      return hipErrorInvalidValue;
    dispatch_fmt(fmt, [&](auto f) {
      constexpr int F = decltype(f)::value;
      if (dh == 128) KVQ_SPLIT_NP(F, 128); else KVQ_SPLIT_NP(F, 64);
    });
#undef KVQ_SPLIT_NP
#undef KVQ_SPLIT_HP
#undef KVQ_SPLIT_G4
#undef KVQ_SPLIT
  }
  launch_decode_combine(out, out_bf16, ml, acc, ctx, B, Hq, Hkv, dh, max_ctx, ts ? nullptr : vs,
                        per_head, plan.part_blocks, plan.nsplit, s);
  return hipGetLastError();
}

void launch_decode_combine(void* out, int out_bf16, const float* ml, const float* acc,
                           const int32_t* ctx, int B, int Hq, int Hkv, int dh, int max_ctx,
                           const float* vs, int per_head, int part_blocks, int nsplit,
                           hipStream_t s) {
  constexpr int kHpw = kCombineHeadsPerWg;
  const bool wide = kHpw > 1 && Hq % kHpw == 0;
  const bool lanes = nsplit > 16;  // rows of more than one batch of splits
  // The 4-channel merge loads the partials 16 bytes at a time.  They start
  // 8 x B x Hq x nsplit bytes into the 16-byte aligned workspace, and a
  // multiple of kHpw (even) for Hq keeps that offset a multiple of 16.
  static_assert(kCombineHeadsPerWg % 2 == 0, "the 4-channel merge needs an even head count");
  const bool even = ((int64_t)B * Hq * nsplit) % 2 == 0;  // 16-byte aligned partials
#define KVQ_COMBINE(D, BF)                                                                     \
  do {                                                                                         \
    if (lanes && even)                                                                         \
      decode_combine_lanes4_kernel<D, BF><<<dim3(Hq, B), dim3(D / 4, kSL), 0, s>>>(             \
          out, ml, acc, ctx, Hq, Hkv, max_ctx, vs, per_head, part_blocks, nsplit);             \
    else if (lanes)                                                                            \
      decode_combine_lanes_kernel<D, BF><<<dim3(Hq, B), dim3(D, kSL), 0, s>>>(                  \
          out, ml, acc, ctx, Hq, Hkv, max_ctx, vs, per_head, part_blocks, nsplit);             \
    else if (wide)                                                                             \
      decode_combine4_kernel<D, BF, kHpw><<<dim3(Hq / kHpw, B), dim3(D / 4, kHpw), 0, s>>>(    \
          out, ml, acc, ctx, Hq, Hkv, max_ctx, vs, per_head, part_blocks, nsplit);             \
    else                                                                                       \
      decode_combine_kernel<D, BF, 1><<<dim3(Hq, B), D, 0, s>>>(                               \
          out, ml, acc, ctx, Hq, Hkv, max_ctx, vs, per_head, part_blocks, nsplit);             \
  } while (0)
  if (dh == 128) {
    if (out_bf16) KVQ_COMBINE(128, true); else KVQ_COMBINE(128, false);
  } else {
    if (out_bf16) KVQ_COMBINE(64, true); else KVQ_COMBINE(64, false);
  }
#undef KVQ_COMBINE
}

}  // namespace kvq

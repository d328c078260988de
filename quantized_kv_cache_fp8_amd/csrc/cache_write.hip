// cache_write.hip -- quantize-on-write of K and V into the paged FP8 cache.
//
// The write rule of the KV-cache quantization textbook (section 10.4.2,
// Kq = Q(K / sK), stored with sK) in its FP8 form (section 10.4.5,
// cast_fp8(K / sK)), placed through a slot mapping into the paged layout
// (slot -> block slot/bs, offset slot%bs):
//   K tiles [num_blocks][Hkv][dh/16][bs][16]: 16-channel chunks, token-major
//     inside a chunk (what the attention kernels' K loads want: 16 tokens x
//     4 chunks = 1 KB of contiguous bytes per 64-lane load)
//   V tiles are channel-major [num_blocks][Hkv][dh][bs]
// Both attention kernels contract V over tokens, so a channel-major V tile
// hands every matrix-core operand a contiguous run of tokens; the transpose
// is paid here, once per byte.
//
// A workgroup owns a chunk of 64 consecutive tokens of one KV head.
//   1. The chunk's slots go to LDS; wave 0 marks the start of every run of
//      tokens whose slots are consecutive inside one aligned group of four
//      slots ("quad"), with the run's length (1..4).
//   2. Every thread quantizes 4 tokens x 4 channels (dh 64) or 4 tokens x 8
//      channels (dh 128, one 16-byte bf16 load per token row) of K and V;
//      the lanes of a token row are consecutive, and the loads are issued
//      before step 1's barrier, since they do not depend on the slots.  K codes are parked
//      in an LDS tile [64 tokens][dh]; the 4x4 V code block is transposed
//      with v_perm_b32 and parked in an LDS tile [dh][64 tokens].
//   3. K: for each valid token and 16-channel chunk one thread stores the 16
//      code bytes (consecutive threads take consecutive tokens, so a block's
//      chunk row of 16 tokens goes out as 256 contiguous bytes).  V: a block
//      whose 16 tokens all lie in the chunk with consecutive slots (the
//      normal case for tokens of a sequence written in order) goes out as one
//      16-byte store per channel row; for each remaining run and channel one
//      thread stores the run's codes: one dword when the run fills its quad,
//      single bytes otherwise (a decode step's one new token per sequence,
//      the ends of a chunk or of a sequence).
// Tokens with a negative slot, or a slot outside the pool, are skipped.
// Writes of at most 512 tokens (a decode step) take a one-pass kernel instead.
#include "codec.hpp"
#include "launch.hpp"

#include <type_traits>

namespace kvq {

constexpr int kBs = 16;     // tokens per cache block
constexpr int kChunk = 64;  // tokens per workgroup (one wave marks the runs)
constexpr int kRowDw = kChunk / 4 + 1;  // LDS V-tile row: 16 dwords of codes + 1 pad
// Writes of at most this many tokens take a one-pass kernel (no LDS, no barrier).
constexpr int64_t kShortWrite = 512;

// Loads of the bf16 K and V rows are nontemporal: every input byte is read
// once, so the loads stream through L2 instead of allocating in it (142-151
// vs 166-172 us for the full headline context, 809 MB, in three alternating
// rounds; nontemporal stores of the codes gained nothing).
typedef unsigned u32x4n __attribute__((ext_vector_type(4)));
typedef unsigned u32x2n __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_nt16(const uint16_t* p) {
  const u32x4n v = __builtin_nontemporal_load(reinterpret_cast<const u32x4n*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt8(const uint16_t* p) {
  const u32x2n v = __builtin_nontemporal_load(reinterpret_cast<const u32x2n*>(p));
  return make_uint2(v.x, v.y);
}

// four bf16 values -> four codes; PRE as in fp8_arg (INT8 takes the general
// quotient and its own clip)
template <int FMT, bool PRE = true>
__device__ __forceinline__ uint32_t quant4(uint2 w, const Divisor& d) {
  if constexpr (FMT == INT8) {
    return enc4<FMT>(quotient(bf16lo(w.x), d), quotient(bf16hi(w.x), d),
                     quotient(bf16lo(w.y), d), quotient(bf16hi(w.y), d));
  } else {
    return cvt4<FMT>(fp8_arg<FMT, PRE>(bf16lo(w.x), d), fp8_arg<FMT, PRE>(bf16hi(w.x), d),
                     fp8_arg<FMT, PRE>(bf16lo(w.y), d), fp8_arg<FMT, PRE>(bf16hi(w.y), d));
  }
}

// Per-token-head scales (one fp16 scale per (token, head) for K and for V,
// stored beside the codes in [num_blocks][Hkv][bs] scale caches).  The lanes
// that share a (token, head) row -- aligned consecutive lanes, each holding a
// few channels -- reduce the row's amax over |x| bit patterns (an exact
// integer max in which NaN patterns sort above +Inf), derive
//   s = fl16(clamp(fl32(amax / fmax), 2^-24, 65504))   (1.0 for amax 0, Inf, NaN)
// and quantize their channels with it.  Long writes take the LDS-staged kernel
// below with TS set (a row is DH / 4 lanes of 4 channels); short ones take
// cache_write_token_kernel (a row is DH / 16 lanes of 16 channels).

// largest |x| bit pattern (sign cleared) among 8 bf16 values
__device__ __forceinline__ uint32_t absmax_bits8(uint4 w) {
  const uint32_t v[4] = {w.x & 0x7fff7fffu, w.y & 0x7fff7fffu, w.z & 0x7fff7fffu,
                         w.w & 0x7fff7fffu};
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = v[i] & 0xffffu, hi = v[i] >> 16;
    r = lo > r ? lo : r;
    r = hi > r ? hi : r;
  }
  return r;
}

// largest |x| bit pattern among 4 bf16 values
__device__ __forceinline__ uint32_t absmax_bits4(uint2 w) {
  const uint32_t a = w.x & 0x7fff7fffu, b = w.y & 0x7fff7fffu;
  const uint32_t m0 = (a & 0xffffu) > (a >> 16) ? (a & 0xffffu) : (a >> 16);
  const uint32_t m1 = (b & 0xffffu) > (b >> 16) ? (b & 0xffffu) : (b >> 16);
  return m0 > m1 ? m0 : m1;
}

template <int FMT>
__device__ __forceinline__ uint16_t scale16_from_amax_bits(uint32_t abits) {
  if (abits == 0 || abits >= 0x7f80u) return 0x3C00;  // 0, Inf or NaN -> 1.0
  float s = __fdiv_rn(__uint_as_float(abits << 16), FmtTraits<FMT>::kMax);
  s = __builtin_amdgcn_fmed3f(s, 0x1p-24f, 65504.0f);
  return __builtin_bit_cast(uint16_t, (_Float16)s);  // round to nearest even
}

template <int FMT, int DH, bool TS>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t T, int Hkv,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    int64_t num_slots, int64_t bstride, const float* __restrict__ ks,
    const float* __restrict__ vs, int per_head, uint16_t* __restrict__ ksc,
    uint16_t* __restrict__ vsc) {
  constexpr int kCq = DH / 4;  // channel quads per token row
  __shared__ int64_t s_slot[kChunk];
  __shared__ uint32_t s_run[kChunk];  // token index | run length << 8, compacted
  __shared__ int s_nrun;
  __shared__ uint8_t s_fblk[kChunk / kBs];  // chunk index of each whole block's first token
  __shared__ int s_nfb;
  __shared__ uint32_t s_vt[DH * kRowDw];
  constexpr int kKRow = DH / 4 + 4;  // LDS K-tile row (dwords): DH codes + 16 B pad
  __shared__ __attribute__((aligned(16))) uint32_t s_kt[kChunk * kKRow];
  __shared__ uint16_t s_sc[2][kChunk];  // per-token-head scales of the chunk (TS)

  const int h = (int)(blockIdx.x % (uint32_t)Hkv);
  const int64_t t0 = (int64_t)(blockIdx.x / (uint32_t)Hkv) * kChunk;
  const int tid = threadIdx.x;
  // the bf16 loads do not depend on the slots: issue them first so both
  // latencies overlap (tokens past T read nothing)
  constexpr int kJobs = (kChunk / 4) * kCq / 256;  // 4x4 jobs per thread
  // with two jobs a thread takes channel quads 2 c and 2 c + 1 of token quad
  // tq (one 16-byte load per token row); with one, quad c of token quad tq
  constexpr int kRowLanes = kCq / kJobs;  // lanes holding one token row
  const int co = tid % kRowLanes, tqs = tid / kRowLanes;
  auto job_cq = [&](int jb) { return kJobs * co + jb; };
  uint2 wk[kJobs][4], wv[kJobs][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t t = t0 + 4 * tqs + j;
#pragma unroll
    for (int jb = 0; jb < kJobs; ++jb) wk[jb][j] = wv[jb][j] = make_uint2(0, 0);
    if (t < T) {
      const size_t src = ((size_t)t * Hkv + h) * DH + co * 4 * kJobs;
      if constexpr (kJobs == 2) {
        const uint4 a = load_nt16(k + src);
        const uint4 b = load_nt16(v + src);
        wk[0][j] = make_uint2(a.x, a.y);
        wk[1][j] = make_uint2(a.z, a.w);
        wv[0][j] = make_uint2(b.x, b.y);
        wv[1][j] = make_uint2(b.z, b.w);
      } else {
        wk[0][j] = load_nt8(k + src);
        wv[0][j] = load_nt8(v + src);
      }
    }
  }
  static_assert(kJobs == 1 || kJobs == 2, "one or two jobs per thread");
  if (tid < kChunk) {
    const int64_t t = t0 + tid;
    int64_t s = t < T ? slot_mapping[t] : -1;
    if (s >= num_slots) s = -1;  // out of the pool: skipped like padding
    s_slot[tid] = s < 0 ? -1 : s;
  }
  __syncthreads();

  if (tid < kChunk) {  // wave 0: whole blocks, then runs inside one quad
    const int64_t s = s_slot[tid];
    // a whole block: 16 tokens of this chunk with consecutive slots from a
    // block's first slot
    bool fb = s >= 0 && (s & (kBs - 1)) == 0 && tid + kBs <= kChunk;
    for (int j = 1; fb && j < kBs; ++j) fb = s_slot[tid + j] == s + j;
    const uint64_t fbm = __builtin_amdgcn_ballot_w64(fb);
    const int off = (int)(s & (kBs - 1));
    const bool in_full = s >= 0 && tid >= off && ((fbm >> (tid - off)) & 1) &&
                         s_slot[tid - off] == s - off;
    if (fb) s_fblk[__builtin_popcountll(fbm & ((1ull << tid) - 1))] = (uint8_t)tid;
    if (tid == 0) s_nfb = __builtin_popcountll(fbm);
    const int q = (int)(s & 3);
    const bool cont = tid > 0 && q != 0 && s >= 0 && s_slot[tid - 1] == s - 1;
    const bool start = s >= 0 && !cont && !in_full;
    int n = 1;
    while (start && n < 4 - q && tid + n < kChunk && s_slot[tid + n] == s + n) ++n;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(start);
    if (start) {
      const int pos = __builtin_popcountll(mask & ((1ull << tid) - 1));
      s_run[pos] = (uint32_t)tid | ((uint32_t)n << 8);
    }
    if (tid == 0) s_nrun = __builtin_popcountll(mask);
  }

  float sk = 1.0f, sv = 1.0f;
  if constexpr (!TS) {
    sk = ks[per_head ? h : 0];
    sv = vs[per_head ? h : 0];
  }
  const Divisor dk0 = make_divisor(sk), dv0 = make_divisor(sv);
  // the tiny-scale prescale is decided per workgroup (per-token scales may
  // need it anywhere)
  auto quantize = [&](auto pre_tag) {
    constexpr bool PRE = decltype(pre_tag)::value;
    Divisor dk = dk0, dv = dv0;
    // per-token-head scales: the kRowLanes aligned consecutive lanes of token
    // 4 tq + j hold its row (all of the thread's jobs)
    Divisor tdk[4], tdv[4];
    if constexpr (TS) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t ak = 0, av = 0;
#pragma unroll
        for (int jb = 0; jb < kJobs; ++jb) {
          const uint32_t xk = absmax_bits4(wk[jb][j]), xv = absmax_bits4(wv[jb][j]);
          ak = ak > xk ? ak : xk;
          av = av > xv ? av : xv;
        }
#pragma unroll
        for (int o = 1; o < kRowLanes; o <<= 1) {
          const uint32_t xk = __shfl_xor(ak, o), xv = __shfl_xor(av, o);
          ak = ak > xk ? ak : xk;
          av = av > xv ? av : xv;
        }
        const uint16_t k16 = scale16_from_amax_bits<FMT>(ak);
        const uint16_t v16 = scale16_from_amax_bits<FMT>(av);
        if (co == 0) {
          s_sc[0][4 * tqs + j] = k16;
          s_sc[1][4 * tqs + j] = v16;
        }
        tdk[j] = make_divisor((float)__builtin_bit_cast(_Float16, k16));
        tdv[j] = make_divisor((float)__builtin_bit_cast(_Float16, v16));
      }
    }
#pragma unroll
    for (int jb = 0; jb < kJobs; ++jb) {
      const int cq = job_cq(jb), tq = tqs;
      uint32_t cv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (TS) {
          dk = tdk[j];
          dv = tdv[j];
        }
        cv[j] = quant4<FMT, PRE>(wv[jb][j], dv);
        s_kt[(4 * tq + j) * kKRow + cq] = quant4<FMT, PRE>(wk[jb][j], dk);
      }
      // rows cv[j] = token j, bytes = channels 4cq..4cq+3 -> one dword per channel
      const uint32_t t0l = __builtin_amdgcn_perm(cv[1], cv[0], 0x05010400u);  // a0 b0 a1 b1
      const uint32_t t1l = __builtin_amdgcn_perm(cv[1], cv[0], 0x07030602u);  // a2 b2 a3 b3
      const uint32_t t2l = __builtin_amdgcn_perm(cv[3], cv[2], 0x05010400u);  // c0 d0 c1 d1
      const uint32_t t3l = __builtin_amdgcn_perm(cv[3], cv[2], 0x07030602u);  // c2 d2 c3 d3
      uint32_t* row = s_vt + (4 * cq) * kRowDw + tq;
      row[0] = __builtin_amdgcn_perm(t2l, t0l, 0x05040100u);
      row[kRowDw] = __builtin_amdgcn_perm(t2l, t0l, 0x07060302u);
      row[2 * kRowDw] = __builtin_amdgcn_perm(t3l, t1l, 0x05040100u);
      row[3 * kRowDw] = __builtin_amdgcn_perm(t3l, t1l, 0x07060302u);
    }
  };
  if (TS || dk0.pre != 1.0f || dv0.pre != 1.0f)
    quantize(std::integral_constant<bool, true>{});
  else
    quantize(std::integral_constant<bool, false>{});
  __syncthreads();

  if constexpr (TS) {
    if (tid < kChunk && s_slot[tid] >= 0) {
      const int64_t sl = s_slot[tid];
      const size_t i = (size_t)((sl >> 4) * Hkv + h) * kBs + (sl & (kBs - 1));
      ksc[i] = s_sc[0][tid];
      vsc[i] = s_sc[1][tid];
    }
  }
  // K: 16 code bytes per (token, chunk); tokens fastest across threads
  for (int job = tid; job < kChunk * (DH / 16); job += 256) {
    const int t = job % kChunk, q = job / kChunk;
    const int64_t s = s_slot[t];
    if (s < 0) continue;
    const uint4 w = *reinterpret_cast<const uint4*>(s_kt + t * kKRow + 4 * q);
    *reinterpret_cast<uint4*>(kc + (size_t)(s >> 4) * bstride + (size_t)h * kBs * DH +
                              q * (kBs * 16) + (s & (kBs - 1)) * 16) = w;
  }

  // V of whole blocks: one 16-byte store per channel row
  const int nfb = s_nfb;
  for (int job = tid; job < nfb * DH; job += 256) {
    const int c = job % DH;
    const int i = s_fblk[job / DH];
    const int64_t s = s_slot[i];
    const uint32_t* row = s_vt + c * kRowDw + (i >> 2);
    const uint32_t sh = (uint32_t)(i & 3);
    const uint4 w = make_uint4(__builtin_amdgcn_alignbyte(row[1], row[0], sh),
                               __builtin_amdgcn_alignbyte(row[2], row[1], sh),
                               __builtin_amdgcn_alignbyte(row[3], row[2], sh),
                               __builtin_amdgcn_alignbyte(row[4], row[3], sh));
    *reinterpret_cast<uint4*>(vc + (size_t)(s >> 4) * bstride + ((size_t)h * DH + c) * kBs) = w;
  }
  const int nrun = s_nrun;
  for (int job = tid; job < nrun * DH; job += 256) {
    const int c = job % DH;
    const uint32_t e = s_run[job / DH];
    const int i = (int)(e & 0xff), n = (int)(e >> 8);
    const int64_t s = s_slot[i];
    // codes of tokens i..i+3 of channel c (bytes past the run are ignored)
    const uint32_t* row = s_vt + c * kRowDw + (i >> 2);
    const uint32_t w = __builtin_amdgcn_alignbyte(row[1], row[0], (uint32_t)(i & 3));
    uint8_t* dst = vc + (size_t)(s >> 4) * bstride + ((size_t)h * DH + c) * kBs + (s & (kBs - 1));
    if (n == 4) {
      *reinterpret_cast<uint32_t*>(dst) = w;  // a full quad starts 4-aligned
    } else {
      for (int b = 0; b < n; ++b) dst[b] = (uint8_t)(w >> (8 * b));
    }
  }
}

// Short writes (a decode step's new tokens, one per sequence, each in its own
// block): one thread per (token, head, 16-channel chunk) loads its slot and
// its 16 K and V values together, quantizes them and stores 16 K bytes and 16
// single V bytes -- one memory round trip, no LDS, no barrier.
template <int FMT, int DH>
__global__ __launch_bounds__(256) void cache_write_short_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint32_t units, int Hkv,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    int64_t num_slots, int64_t bstride, const float* __restrict__ ks,
    const float* __restrict__ vs, int per_head) {
  constexpr int kNc = DH / 16;  // chunks per token row
  const uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const uint32_t q = u % kNc, th = u / kNc;  // th = t * Hkv + h
  const uint32_t t = th / (uint32_t)Hkv;
  const int h = (int)(th - t * (uint32_t)Hkv);
  const size_t src = (size_t)th * DH + q * 16;
  const uint4 k0 = *reinterpret_cast<const uint4*>(k + src);
  const uint4 k1 = *reinterpret_cast<const uint4*>(k + src + 8);
  const uint4 v0 = *reinterpret_cast<const uint4*>(v + src);
  const uint4 v1 = *reinterpret_cast<const uint4*>(v + src + 8);
  const int64_t s = slot_mapping[t];
  if (s < 0 || s >= num_slots) return;  // padding or out of the pool: skipped
  const Divisor dk = make_divisor(ks[per_head ? h : 0]), dv = make_divisor(vs[per_head ? h : 0]);
  const uint4 kq = make_uint4(quant4<FMT>(make_uint2(k0.x, k0.y), dk),
                              quant4<FMT>(make_uint2(k0.z, k0.w), dk),
                              quant4<FMT>(make_uint2(k1.x, k1.y), dk),
                              quant4<FMT>(make_uint2(k1.z, k1.w), dk));
  const uint32_t vq[4] = {quant4<FMT>(make_uint2(v0.x, v0.y), dv),
                          quant4<FMT>(make_uint2(v0.z, v0.w), dv),
                          quant4<FMT>(make_uint2(v1.x, v1.y), dv),
                          quant4<FMT>(make_uint2(v1.z, v1.w), dv)};
  const size_t tile = (size_t)(s >> 4) * bstride + (size_t)h * kBs * DH;
  const int off = (int)(s & (kBs - 1));
  *reinterpret_cast<uint4*>(kc + tile + q * (kBs * 16) + off * 16) = kq;
  uint8_t* vd = vc + tile + (size_t)q * 16 * kBs + off;  // channel 16 q, token off
#pragma unroll
  for (int c = 0; c < 16; ++c) vd[c * kBs] = (uint8_t)(vq[c >> 2] >> (8 * (c & 3)));
}

template <int FMT, int DH>
__global__ __launch_bounds__(256) void cache_write_token_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint32_t units, int Hkv,
    const int64_t* __restrict__ slot_mapping, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
    uint16_t* __restrict__ ksc, uint16_t* __restrict__ vsc, int64_t num_slots, int64_t bstride) {
  constexpr int kNc = DH / 16;  // lanes per (token, head) row
  const uint32_t u = blockIdx.x * blockDim.x + threadIdx.x;
  const bool live = u < units;  // every lane takes part in the row reductions
  const uint32_t uu = live ? u : units - 1;
  const uint32_t q = uu % kNc, th = uu / kNc;
  const uint32_t t = th / (uint32_t)Hkv;
  const int h = (int)(th - t * (uint32_t)Hkv);
  const size_t src = (size_t)th * DH + q * 16;
  const uint4 k0 = *reinterpret_cast<const uint4*>(k + src);
  const uint4 k1 = *reinterpret_cast<const uint4*>(k + src + 8);
  const uint4 v0 = *reinterpret_cast<const uint4*>(v + src);
  const uint4 v1 = *reinterpret_cast<const uint4*>(v + src + 8);
  const int64_t s = slot_mapping[t];
  uint32_t ak = absmax_bits8(k0), ak1 = absmax_bits8(k1);
  uint32_t av = absmax_bits8(v0), av1 = absmax_bits8(v1);
  ak = ak > ak1 ? ak : ak1;
  av = av > av1 ? av : av1;
#pragma unroll
  for (int o = 1; o < kNc; o <<= 1) {  // rows are kNc aligned consecutive lanes
    const uint32_t xk = __shfl_xor(ak, o), xv = __shfl_xor(av, o);
    ak = ak > xk ? ak : xk;
    av = av > xv ? av : xv;
  }
  if (!live || s < 0 || s >= num_slots) return;  // padding or out of the pool: skipped
  const uint16_t sk16 = scale16_from_amax_bits<FMT>(ak), sv16 = scale16_from_amax_bits<FMT>(av);
  const Divisor dk = make_divisor((float)__builtin_bit_cast(_Float16, sk16));
  const Divisor dv = make_divisor((float)__builtin_bit_cast(_Float16, sv16));
  const uint4 kq = make_uint4(quant4<FMT>(make_uint2(k0.x, k0.y), dk),
                              quant4<FMT>(make_uint2(k0.z, k0.w), dk),
                              quant4<FMT>(make_uint2(k1.x, k1.y), dk),
                              quant4<FMT>(make_uint2(k1.z, k1.w), dk));
  const uint32_t vq[4] = {quant4<FMT>(make_uint2(v0.x, v0.y), dv),
                          quant4<FMT>(make_uint2(v0.z, v0.w), dv),
                          quant4<FMT>(make_uint2(v1.x, v1.y), dv),
                          quant4<FMT>(make_uint2(v1.z, v1.w), dv)};
  const size_t row = (size_t)((s >> 4) * Hkv + h);  // scale caches are not padded
  const size_t tile = (size_t)(s >> 4) * bstride + (size_t)h * kBs * DH;
  const int off = (int)(s & (kBs - 1));
  *reinterpret_cast<uint4*>(kc + tile + q * (kBs * 16) + off * 16) = kq;
  uint8_t* vd = vc + tile + (size_t)q * 16 * kBs + off;
#pragma unroll
  for (int c = 0; c < 16; ++c) vd[c * kBs] = (uint8_t)(vq[c >> 2] >> (8 * (c & 3)));
  if (q == 0) {
    ksc[row * kBs + off] = sk16;
    vsc[row * kBs + off] = sv16;
  }
}

hipError_t launch_cache_write_token(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv,
                                    int dh, const int64_t* slot, uint8_t* kc, uint8_t* vc,
                                    uint16_t* ksc, uint16_t* vsc, int64_t num_blocks, int fmt,
                                    hipStream_t s, int64_t bstride) {
  if (bstride <= 0) bstride = (int64_t)Hkv * kBs * dh;
  if (T == 0) return hipSuccess;
  const int64_t num_slots = num_blocks * kBs;
  const uint32_t units = (uint32_t)(T * Hkv * (dh / 16));
  const uint32_t grid = (uint32_t)(((T + kChunk - 1) / kChunk) * Hkv);
  dispatch_fmt(fmt, [&](auto f) {
    constexpr int F = decltype(f)::value;
    if (T > kShortWrite) {  // the LDS-staged kernel, one scale per token row
      if (dh == 128)
        cache_write_kernel<F, 128, true><<<grid, 256, 0, s>>>(
            k, v, T, Hkv, slot, kc, vc, num_slots, bstride, nullptr, nullptr, 0, ksc, vsc);
      else
        cache_write_kernel<F, 64, true><<<grid, 256, 0, s>>>(
            k, v, T, Hkv, slot, kc, vc, num_slots, bstride, nullptr, nullptr, 0, ksc, vsc);
    } else if (dh == 128) {
      cache_write_token_kernel<F, 128><<<(units + 255) / 256, 256, 0, s>>>(
          k, v, units, Hkv, slot, kc, vc, ksc, vsc, num_slots, bstride);
    } else {
      cache_write_token_kernel<F, 64><<<(units + 255) / 256, 256, 0, s>>>(
          k, v, units, Hkv, slot, kc, vc, ksc, vsc, num_slots, bstride);
    }
  });
  return hipGetLastError();
}


template <int FMT, int DH>
void launch_write(int64_t T, int Hkv, const uint16_t* k, const uint16_t* v, const int64_t* slot,
                  uint8_t* kc, uint8_t* vc, int64_t num_slots, int64_t bstride, const float* ks,
                  const float* vs, int per_head, hipStream_t s) {
  if (T <= kShortWrite) {
    const uint32_t units = (uint32_t)(T * Hkv * (DH / 16));
    cache_write_short_kernel<FMT, DH><<<(units + 255) / 256, 256, 0, s>>>(
        k, v, units, Hkv, slot, kc, vc, num_slots, bstride, ks, vs, per_head);
    return;
  }
  const uint32_t grid = (uint32_t)(((T + kChunk - 1) / kChunk) * Hkv);
  cache_write_kernel<FMT, DH, false><<<grid, 256, 0, s>>>(
      k, v, T, Hkv, slot, kc, vc, num_slots, bstride, ks, vs, per_head, nullptr, nullptr);
}

hipError_t launch_cache_write(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                              const int64_t* slot, uint8_t* kc, uint8_t* vc, int64_t num_blocks,
                              const float* ks, const float* vs, int fmt, int per_head,
                              hipStream_t s, int64_t bstride) {
  if (T == 0) return hipSuccess;
  const int64_t num_slots = num_blocks * kBs;
  if (bstride <= 0) bstride = (int64_t)Hkv * kBs * dh;
  dispatch_fmt(fmt, [&](auto f) {
    constexpr int F = decltype(f)::value;
    if (dh == 128)
      launch_write<F, 128>(T, Hkv, k, v, slot, kc, vc, num_slots, bstride, ks, vs, per_head, s);
    else
      launch_write<F, 64>(T, Hkv, k, v, slot, kc, vc, num_slots, bstride, ks, vs, per_head, s);
  });
  return hipGetLastError();
}

}  // namespace kvq

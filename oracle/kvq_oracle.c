/*
 * kvq_oracle.c -- reference CPU oracle for the FP8 paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow definition that the
 * GPU library is checked against.  Only the test-suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it.  It shares no source, header,
 * table or helper with the HIP library, and the library never calls it.
 *
 * Everything is written from the definitions on the pages:
 *   [T]  "10.4 KV Cache 量化: INT8 基础、KIVI 2-bit、FP8 KV" (KV-cache quantization
 *        textbook chapter), sections 10.4.1 - 10.4.5.
 *   [G]  "vLLM FP8 量化 KV Cache 完整指南" (vLLM FP8 KV-cache guide), sections on
 *        kv_cache_dtype formats, the two scale granularities and scale sources.
 * plus the OCP 8-bit floating point specification for the bit layouts of
 * E4M3 ("fn": no infinities, one NaN mantissa) and E5M2 (IEEE-like).
 *
 * Floating point is fp64 unless a step is defined in fp32 (the quantize
 * quotient and the scale, which the cache stores as fp32).
 *
 * Readings of points the pages leave open (numbered as in the design notes):
 *   R1 quantize divides by the scale (not multiply by a reciprocal);
 *   R2 rounding is round-to-nearest, ties to even;
 *   R3 out-of-range and +-Inf saturate to +-max, NaN stays NaN, -0 keeps its
 *      sign, subnormal codes are produced (no flush to zero);
 *   R4 scale = amax/fmax in fp32, 1.0 if amax is 0 or not finite;
 *   R5 query head hq reads KV head hq / (Hq/Hkv);
 *   R7 decode has no mask; prefill is causal at absolute positions;
 *   zero-length context gives an all-zero output row;
 *   symmetric INT8 (format 2): clip(round-half-even(fl32(x / s)), -127, 127),
 *   NaN -> 0, +-Inf -> +-127, scale = amax / 127.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops below use (1 without OpenMP): reported next to
 * the oracle's timing. */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

#define ORC_FMT_E4M3 0
#define ORC_FMT_E5M2 1
#define ORC_FMT_INT8 2 /* symmetric INT8 (textbook 10.4.2 write rule) */
#define ORC_GRAN_TENSOR 0
#define ORC_GRAN_HEAD 1

/* ---- format parameters (OCP FP8): mantissa bits, exponent bias, max ---- */

static int fmt_mbits(int fmt) { return fmt == ORC_FMT_E4M3 ? 3 : 2; }
static int fmt_bias(int fmt) { return fmt == ORC_FMT_E4M3 ? 7 : 15; }

double orc_fp8_max(int fmt) {
  /* E4M3fn: exponent field 15, mantissa 110b -> 1.75 * 2^8.
   * E5M2:   exponent field 30, mantissa 11b  -> 1.75 * 2^15.
   * INT8:   the clip bound of the symmetric write rule, 127. */
  if (fmt == ORC_FMT_INT8) return 127.0;
  return fmt == ORC_FMT_E4M3 ? 1.75 * 256.0 : 1.75 * 32768.0;
}

/* ---- symmetric INT8 (textbook 10.4.2): Kq = clip(round(K / sK), -127, 127),
 * read back as K_hat = sK * Kq.  The quotient arrives as fp32 (as for FP8);
 * round is to nearest with ties to even (R2); a NaN quotient gives code 0 and
 * +-Inf clip to +-127 (there is no NaN or Inf code).  The code is the two's
 * complement byte of Kq. ---- */

static uint8_t int8_encode(float x) {
  if (isnan(x)) return 0;
  double r = rint((double)x); /* default rounding mode: ties to even */
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (uint8_t)(int8_t)r;
}

/* ---- decode: code -> exact value (textbook 10.4.5: cast_float(Kfp8); for
 * INT8 the signed integer itself) ---- */

double orc_fp8_decode(int fmt, uint8_t code) {
  if (fmt == ORC_FMT_INT8) return (double)(int8_t)code;
  int s = code >> 7;
  int mb = fmt_mbits(fmt);
  int bias = fmt_bias(fmt);
  int e = (code & 0x7f) >> mb;
  int m = code & ((1 << mb) - 1);
  double v;
  if (fmt == ORC_FMT_E4M3) {
    if (e == 15 && m == 7) return NAN; /* the only NaN mantissa; no Inf */
  } else {
    if (e == 31) return m == 0 ? (s ? -INFINITY : INFINITY) : NAN;
  }
  if (e == 0)
    v = ldexp((double)m, 1 - bias - mb); /* subnormal: m * 2^(1-bias-mb) */
  else
    v = ldexp(1.0 + (double)m / (double)(1 << mb), e - bias);
  return s ? -v : v;
}

/* ---- encode: fp32 -> code, saturating round-to-nearest-even (R2, R3) ----
 * |x| is rounded onto the target grid as if the exponent were unbounded
 * above (quantum 2^(e-mb) in binade e, 2^(emin-mb) below the normal range),
 * then anything above max saturates.  All arithmetic is exact in fp64. */

uint8_t orc_fp8_encode(int fmt, float x) {
  if (fmt == ORC_FMT_INT8) return int8_encode(x);
  int mb = fmt_mbits(fmt);
  int bias = fmt_bias(fmt);
  int emin = 1 - bias;
  double fmax = orc_fp8_max(fmt);
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs((double)x);
  if (isnan(x)) return (uint8_t)(sign | 0x7f); /* 0x7f is NaN in both formats */
  if (isinf(x) || a > fmax) {
    /* saturate: encode max */
  } else {
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5,1) -> binade e2-1 */
    int binade = e2 - 1;
    if (binade < emin) binade = emin;
    double quantum = ldexp(1.0, binade - mb);
    double n = rint(a / quantum); /* exact quotient; rint = ties-to-even */
    double r = n * quantum;
    if (r <= fmax) {
      if (r == 0.0) return sign;
      int er;
      frexp(r, &er);
      int be = er - 1;
      if (be < emin) { /* subnormal code: value = mant * 2^(emin-mb) */
        int mant = (int)(r / ldexp(1.0, emin - mb));
        return (uint8_t)(sign | mant);
      }
      int mant = (int)((r / ldexp(1.0, be) - 1.0) * (double)(1 << mb));
      int efield = be + bias;
      return (uint8_t)(sign | (efield << mb) | mant);
    }
  }
  /* +-max */
  {
    int efield = fmt == ORC_FMT_E4M3 ? 15 : 30;
    int mant = fmt == ORC_FMT_E4M3 ? 6 : 3;
    return (uint8_t)(sign | (efield << mb) | mant);
  }
}

void orc_fp8_encode_many(int fmt, const float* x, uint8_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(fmt, x[i]);
}

void orc_fp8_decode_all(int fmt, double* out256) {
  for (int c = 0; c < 256; ++c) out256[c] = orc_fp8_decode(fmt, (uint8_t)c);
}

/* ---- bf16 and the quantize step (textbook 10.4.5: cast_fp8(K / sK)) ---- */

float orc_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* fl32(x / s): the fp64 quotient of two fp32 values, rounded once more to
 * fp32, equals the correctly rounded fp32 quotient (53 >= 2*24 + 2). */
float orc_quotient(float x, float s) { return (float)((double)x / (double)s); }

uint8_t orc_quantize(int fmt, uint16_t x_bf16, float s) {
  return orc_fp8_encode(fmt, orc_quotient(orc_bf16_to_f32(x_bf16), s));
}

void orc_quantize_many(int fmt, const uint16_t* x, int64_t n, float s, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = orc_quantize(fmt, x[i], s);
}

/* ---- scale calibration (textbook 10.4.3 granularity table; guide's scale
 * shapes [1] / [num_heads] / [num_kv_heads]) ----
 * amax = max |x| over the granularity set (NaN anywhere in the set gives NaN);
 * scale = fl32(amax / fmax) when amax is finite and > 0, else 1.0 (R4, the
 * guide's default scale when no calibration is done). */

float orc_scale_from_amax(int fmt, float amax) {
  if (!(amax > 0.0f) || isinf(amax)) return 1.0f;
  return (float)((double)amax / orc_fp8_max(fmt));
}

void orc_calibrate(const uint16_t* x, int64_t T, int H, int dh, int fmt, int gran,
                   float* amax_out, float* scale_out) {
  int nset = gran == ORC_GRAN_HEAD ? H : 1;
  double* amax = (double*)calloc((size_t)nset, sizeof(double));
  int* saw_nan = (int*)calloc((size_t)nset, sizeof(int));
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      int g = gran == ORC_GRAN_HEAD ? h : 0; /* the set this row belongs to */
      for (int d = 0; d < dh; ++d) {
        double v = fabs((double)orc_bf16_to_f32(x[(t * H + h) * dh + d]));
        if (isnan(v)) saw_nan[g] = 1;
        else if (v > amax[g]) amax[g] = v;
      }
    }
  for (int g = 0; g < nset; ++g) {
    amax_out[g] = saw_nan[g] ? NAN : (float)amax[g]; /* |bf16| is exact in fp32 */
    scale_out[g] = orc_scale_from_amax(fmt, amax_out[g]);
  }
  free(amax);
  free(saw_nan);
}

/* ---- paged quantize-write ----
 * For every token t with 0 <= slot_mapping[t] < num_blocks * bs, every KV head
 * h and channel d, with blk = slot / bs and off = slot % bs:
 *   K code -> k_cache[blk][h][d / 16][off][d % 16]  (tile [dh/16][bs][16]:
 *             16-channel chunks, token-major inside a chunk)
 *   V code -> v_cache[blk][h][d][off]               (channel-major tile [dh][bs])
 * each code = quantize(x[t][h][d], s[h or 0]).  The two tile orders are this
 * library's layout (the pages fix only that FP8 caches are raw bytes); the K
 * order needs dh to be a multiple of 16. */

static int64_t k_index(int64_t blk, int h, int off, int d, int Hkv, int bs, int dh) {
  return (((blk * Hkv + h) * (dh / 16) + d / 16) * bs + off) * 16 + d % 16;
}
static int64_t v_index(int64_t blk, int h, int off, int d, int Hkv, int bs, int dh) {
  return ((blk * Hkv + h) * dh + d) * bs + off;
}

void orc_cache_write(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                     const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                     int64_t num_blocks, int bs, const float* k_scale, const float* v_scale,
                     int fmt, int gran) {
  /* tokens are independent (distinct slots), so they may be written in parallel */
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * bs) continue; /* padding or out-of-range: skipped */
    int64_t blk = slot / bs, off = slot % bs;
    for (int h = 0; h < Hkv; ++h) {
      float sk = k_scale[gran == ORC_GRAN_HEAD ? h : 0];
      float sv = v_scale[gran == ORC_GRAN_HEAD ? h : 0];
      for (int d = 0; d < dh; ++d) {
        int64_t src = (t * Hkv + h) * dh + d;
        k_cache[k_index(blk, h, (int)off, d, Hkv, bs, dh)] = orc_quantize(fmt, k[src], sk);
        v_cache[v_index(blk, h, (int)off, d, Hkv, bs, dh)] = orc_quantize(fmt, v[src], sv);
      }
    }
  }
}

/* ---- dequantized read: x_hat = s * cast_float(code) (textbook 10.4.2/10.4.5) ---- */

static double deq_k(const uint8_t* cache, int64_t blk, int h, int off, int d, int Hkv, int bs,
                    int dh, double s, int fmt) {
  return s * orc_fp8_decode(fmt, cache[k_index(blk, h, off, d, Hkv, bs, dh)]);
}
static double deq_v(const uint8_t* cache, int64_t blk, int h, int off, int d, int Hkv, int bs,
                    int dh, double s, int fmt) {
  return s * orc_fp8_decode(fmt, cache[v_index(blk, h, off, d, Hkv, bs, dh)]);
}

/* Attention of one query vector q[dh] (fp64) over keys 0..nkeys-1 of one
 * sequence's paged cache (textbook 10.4.2: P = softmax(Q K^T / sqrt(dh) + mask),
 * O = P V), all in fp64; writes o[dh]. */
/* fp16 bits -> exact value (IEEE binary16: 5 exponent bits, bias 15). */
double orc_f16_to_double(uint16_t b) {
  int s = b >> 15, e = (b >> 10) & 31, m = b & 1023;
  double v;
  if (e == 31) v = m ? NAN : INFINITY;
  else if (e == 0) v = ldexp((double)m, -24);
  else v = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

/* scale of one (block, head, offset) slot: the uniform scale, or the slot's
 * fp16 per-token scale when a scale cache is given */
static double slot_scale(const uint16_t* sc, double s, int64_t blk, int h, int off, int Hkv,
                         int bs) {
  return sc ? orc_f16_to_double(sc[(blk * Hkv + h) * bs + off]) : s;
}

static void attend_one_ts(double* o, const double* q, int nkeys, const uint8_t* k_cache,
                          const uint8_t* v_cache, const uint16_t* ksc, const uint16_t* vsc,
                          const int32_t* btab, int h, int Hkv, int bs, int dh, double sk,
                          double sv, int fmt, double sm_scale);

static void attend_one(double* o, const double* q, int nkeys, const uint8_t* k_cache,
                       const uint8_t* v_cache, const int32_t* btab, int h, int Hkv, int bs,
                       int dh, double sk, double sv, int fmt, double sm_scale) {
  attend_one_ts(o, q, nkeys, k_cache, v_cache, NULL, NULL, btab, h, Hkv, bs, dh, sk, sv, fmt,
                sm_scale);
}

static void attend_one_ts(double* o, const double* q, int nkeys, const uint8_t* k_cache,
                          const uint8_t* v_cache, const uint16_t* ksc, const uint16_t* vsc,
                          const int32_t* btab, int h, int Hkv, int bs, int dh, double sk,
                          double sv, int fmt, double sm_scale) {
  for (int d = 0; d < dh; ++d) o[d] = 0.0;
  if (nkeys <= 0) return;
  double* z = (double*)malloc(sizeof(double) * (size_t)nkeys);
  double zmax = -INFINITY;
  for (int j = 0; j < nkeys; ++j) {
    int64_t blk = btab[j / bs];
    int off = j % bs;
    double acc = 0.0;
    double skj = slot_scale(ksc, sk, blk, h, off, Hkv, bs);
    for (int d = 0; d < dh; ++d) acc += q[d] * deq_k(k_cache, blk, h, off, d, Hkv, bs, dh, skj, fmt);
    z[j] = acc * sm_scale;
    if (z[j] > zmax) zmax = z[j];
  }
  double l = 0.0;
  for (int j = 0; j < nkeys; ++j) {
    z[j] = exp(z[j] - zmax);
    l += z[j];
  }
  for (int j = 0; j < nkeys; ++j) {
    int64_t blk = btab[j / bs];
    int off = j % bs;
    double p = z[j] / l;
    double svj = slot_scale(vsc, sv, blk, h, off, Hkv, bs);
    for (int d = 0; d < dh; ++d) o[d] += p * deq_v(v_cache, blk, h, off, d, Hkv, bs, dh, svj, fmt);
  }
  free(z);
}

static double default_scale(float softmax_scale, int dh) {
  return softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / sqrt((double)dh);
}

/* Decode: one query token per sequence, the last position, already written;
 * it attends to every cached key 0..context_lens[b]-1 (no mask, R7).
 * q: bf16 [B][Hq][dh]; out: fp64 [B][Hq][dh]. */
void orc_decode_attn(double* out, const uint16_t* q, const uint8_t* k_cache,
                     const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                     const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                     const float* k_scale, const float* v_scale, int fmt, int gran,
                     float softmax_scale) {
  int G = Hq / Hkv;
  double sm = default_scale(softmax_scale, dh);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int hq = 0; hq < Hq; ++hq) {
      int h = hq / G;
      double qd[512];
      for (int d = 0; d < dh; ++d) qd[d] = (double)orc_bf16_to_f32(q[((int64_t)b * Hq + hq) * dh + d]);
      double sk = k_scale[gran == ORC_GRAN_HEAD ? h : 0];
      double sv = v_scale[gran == ORC_GRAN_HEAD ? h : 0];
      attend_one(out + ((int64_t)b * Hq + hq) * dh, qd, context_lens[b], k_cache, v_cache,
                 block_tables + (int64_t)b * max_blocks, h, Hkv, bs, dh, sk, sv, fmt, sm);
    }
}

/* Decode for an explicit list of (b, hq) rows only (bounded CPU baseline and
 * sampled checks at full size).  rows: int32 pairs [n][2]; out: fp64 [n][dh]. */
void orc_decode_rows(double* out, const int32_t* rows, int n, const uint16_t* q,
                     const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* block_tables,
                     int max_blocks, const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                     int bs, const float* k_scale, const float* v_scale, int fmt, int gran,
                     float softmax_scale) {
  (void)B;
  int G = Hq / Hkv;
  double sm = default_scale(softmax_scale, dh);
#pragma omp parallel for schedule(dynamic)
  for (int i = 0; i < n; ++i) {
    int b = rows[2 * i], hq = rows[2 * i + 1];
    int h = hq / G;
    double qd[512];
    for (int d = 0; d < dh; ++d) qd[d] = (double)orc_bf16_to_f32(q[((int64_t)b * Hq + hq) * dh + d]);
    double sk = k_scale[gran == ORC_GRAN_HEAD ? h : 0];
    double sv = v_scale[gran == ORC_GRAN_HEAD ? h : 0];
    attend_one(out + (int64_t)i * dh, qd, context_lens[b], k_cache, v_cache,
               block_tables + (int64_t)b * max_blocks, h, Hkv, bs, dh, sk, sv, fmt, sm);
  }
}

/* Prefill of a chunk on top of a cached prefix, with Q quantized to E4M3 as
 * in the FP8-domain attention path the pages describe (the guide's FA3 note;
 * textbook 10.4.5): q_hat = s_q * cast_float(cast_fp8(q / s_q)).
 * Sequence b owns query rows cu_seqlens[b] .. cu_seqlens[b+1]-1; its row i
 * sits at absolute position context_lens[b] - qlen_b + i and attends keys
 * 0..position (causal mask, R7).  The chunk's own K/V must already be in the
 * cache.  P is kept exact (fp64).  out: fp64 [total_q][Hq][dh]. */
static void prefill_row(double* o, const uint16_t* q, const int32_t* cu_seqlens,
                        const float* q_scale, int q_gran, const uint8_t* k_cache,
                        const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                        const int32_t* context_lens, int b, int64_t row, int hq, int Hq, int Hkv,
                        int dh, int bs, const float* k_scale, const float* v_scale, int fmt,
                        int kv_gran, double sm) {
  int G = Hq / Hkv;
  int h = hq / G;
  int qlen = cu_seqlens[b + 1] - cu_seqlens[b];
  int64_t i = row - cu_seqlens[b];
  int64_t pos = (int64_t)context_lens[b] - qlen + i;
  float sq = q_scale[q_gran == ORC_GRAN_HEAD ? hq : 0];
  double qd[512];
  for (int d = 0; d < dh; ++d) {
    uint8_t c = orc_quantize(ORC_FMT_E4M3, q[(row * Hq + hq) * dh + d], sq);
    qd[d] = (double)sq * orc_fp8_decode(ORC_FMT_E4M3, c);
  }
  double sk = k_scale[kv_gran == ORC_GRAN_HEAD ? h : 0];
  double sv = v_scale[kv_gran == ORC_GRAN_HEAD ? h : 0];
  attend_one(o, qd, (int)(pos + 1), k_cache, v_cache, block_tables + (int64_t)b * max_blocks, h,
             Hkv, bs, dh, sk, sv, fmt, sm);
}

static int seq_of_row(const int32_t* cu_seqlens, int B, int64_t row) {
  int b = 0;
  while (b + 1 < B && cu_seqlens[b + 1] <= row) ++b;
  return b;
}

void orc_prefill_attn(double* out, const uint16_t* q, const int32_t* cu_seqlens,
                      const float* q_scale, int q_gran, const uint8_t* k_cache,
                      const uint8_t* v_cache, const int32_t* block_tables, int max_blocks,
                      const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                      const float* k_scale, const float* v_scale, int fmt, int kv_gran,
                      float softmax_scale) {
  int64_t total = cu_seqlens[B];
  double sm = default_scale(softmax_scale, dh);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t row = 0; row < total; ++row)
    for (int hq = 0; hq < Hq; ++hq) {
      int b = seq_of_row(cu_seqlens, B, row);
      prefill_row(out + (row * Hq + hq) * dh, q, cu_seqlens, q_scale, q_gran, k_cache, v_cache,
                  block_tables, max_blocks, context_lens, b, row, hq, Hq, Hkv, dh, bs, k_scale,
                  v_scale, fmt, kv_gran, sm);
    }
}

/* Prefill for an explicit list of (row, hq) pairs only.  out: fp64 [n][dh]. */
void orc_prefill_rows(double* out, const int64_t* rows, int n, const uint16_t* q,
                      const int32_t* cu_seqlens, const float* q_scale, int q_gran,
                      const uint8_t* k_cache, const uint8_t* v_cache, const int32_t* block_tables,
                      int max_blocks, const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                      int bs, const float* k_scale, const float* v_scale, int fmt, int kv_gran,
                      float softmax_scale) {
  double sm = default_scale(softmax_scale, dh);
#pragma omp parallel for schedule(dynamic)
  for (int i = 0; i < n; ++i) {
    int64_t row = rows[2 * i];
    int hq = (int)rows[2 * i + 1];
    int b = seq_of_row(cu_seqlens, B, row);
    prefill_row(out + (int64_t)i * dh, q, cu_seqlens, q_scale, q_gran, k_cache, v_cache,
                block_tables, max_blocks, context_lens, b, row, hq, Hq, Hkv, dh, bs, k_scale,
                v_scale, fmt, kv_gran, sm);
  }
}

/* Attention of explicit fp64 queries over an explicit fp64 K/V (no cache):
 * the plain softmax(q K^T * sm) V used to cross-check the paged paths.
 * q [nq][dh], k/v [nk][dh], out [nq][dh]; query i attends keys 0..nk-1, or
 * 0..(nk-nq+i) when causal. */
void orc_dense_attn(double* out, const double* q, const double* k, const double* v, int nq,
                    int nk, int dh, int causal, double sm) {
  for (int i = 0; i < nq; ++i) {
    int lim = causal ? nk - nq + i + 1 : nk;
    double zmax = -INFINITY, l = 0.0;
    double* z = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    for (int j = 0; j < lim; ++j) {
      double acc = 0.0;
      for (int d = 0; d < dh; ++d) acc += q[(int64_t)i * dh + d] * k[(int64_t)j * dh + d];
      z[j] = acc * sm;
      if (z[j] > zmax) zmax = z[j];
    }
    for (int d = 0; d < dh; ++d) out[(int64_t)i * dh + d] = 0.0;
    for (int j = 0; j < lim; ++j) {
      z[j] = exp(z[j] - zmax);
      l += z[j];
    }
    for (int j = 0; j < lim; ++j)
      for (int d = 0; d < dh; ++d) out[(int64_t)i * dh + d] += z[j] / l * v[(int64_t)j * dh + d];
    free(z);
  }
}

/* ---- memory arithmetic ----
 * textbook 10.4.1: M_KV = 2 * L * B * Hkv * S * dh * bytes_per_element, the
 * leading 2 counting K and V.  bits_per_elem may be below 8 (2-bit payload). */
/* ---- per-token-head scales (textbook 10.4.3: one scale per token along dh;
 * its metadata example keeps one FP16 scale per (token, head) for K and for
 * V).  Reading: s = fl16(clamp(fl32(amax / fmax), 2^-24, 65504)) with
 * round-to-nearest-even into fp16, 1.0 when amax is 0 or not finite; the
 * codes are then quantize(x, s) with that fp16 value.  Scale caches are fp16
 * [num_blocks][Hkv][bs], beside the code caches. ---- */

static uint16_t f16_bits_rne(double x) {
  /* x positive, in [2^-24, 65504]: round to the binary16 grid, ties to even */
  int e2;
  frexp(x, &e2);
  int be = e2 - 1;               /* x in [2^be, 2^(be+1)) */
  if (be < -14) be = -14;        /* subnormal range: quantum 2^-24 */
  double quantum = ldexp(1.0, be - 10);
  double r = rint(x / quantum) * quantum;
  /* encode r */
  if (r < ldexp(1.0, -14)) return (uint16_t)(r / ldexp(1.0, -24));
  int er;
  frexp(r, &er);
  int bexp = er - 1;
  int mant = (int)((r / ldexp(1.0, bexp) - 1.0) * 1024.0);
  return (uint16_t)(((bexp + 15) << 10) | mant);
}

uint16_t orc_scale16_from_amax(int fmt, float amax) {
  if (!(amax > 0.0f) || isinf(amax)) return 0x3C00; /* 1.0 */
  double s = (double)(float)((double)amax / orc_fp8_max(fmt)); /* fl32(amax / fmax) */
  if (s < ldexp(1.0, -24)) s = ldexp(1.0, -24);
  if (s > 65504.0) s = 65504.0;
  return f16_bits_rne(s);
}

void orc_cache_write_token(const uint16_t* k, const uint16_t* v, int64_t T, int Hkv, int dh,
                           const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                           uint16_t* k_scale_cache, uint16_t* v_scale_cache, int64_t num_blocks,
                           int bs, int fmt) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_blocks * bs) continue; /* padding or out-of-range: skipped */
    int64_t blk = slot / bs, off = slot % bs;
    for (int h = 0; h < Hkv; ++h) {
      const uint16_t* kr = k + (t * Hkv + h) * dh;
      const uint16_t* vr = v + (t * Hkv + h) * dh;
      float ak = 0.0f, av = 0.0f;
      int knan = 0, vnan = 0;
      for (int d = 0; d < dh; ++d) {
        float a = fabsf(orc_bf16_to_f32(kr[d])), b = fabsf(orc_bf16_to_f32(vr[d]));
        knan |= isnan(a);
        vnan |= isnan(b);
        if (a > ak) ak = a;
        if (b > av) av = b;
      }
      uint16_t sk16 = orc_scale16_from_amax(fmt, knan ? NAN : ak);
      uint16_t sv16 = orc_scale16_from_amax(fmt, vnan ? NAN : av);
      k_scale_cache[(blk * Hkv + h) * bs + off] = sk16;
      v_scale_cache[(blk * Hkv + h) * bs + off] = sv16;
      float sk = (float)orc_f16_to_double(sk16), sv = (float)orc_f16_to_double(sv16);
      for (int d = 0; d < dh; ++d) {
        k_cache[k_index(blk, h, (int)off, d, Hkv, bs, dh)] = orc_quantize(fmt, kr[d], sk);
        v_cache[v_index(blk, h, (int)off, d, Hkv, bs, dh)] = orc_quantize(fmt, vr[d], sv);
      }
    }
  }
}

/* Decode rows (b, hq) with per-token-head scales; as orc_decode_rows. */
void orc_decode_token_rows(double* out, const int32_t* rows, int n, const uint16_t* q,
                           const uint8_t* k_cache, const uint8_t* v_cache,
                           const uint16_t* k_scale_cache, const uint16_t* v_scale_cache,
                           const int32_t* block_tables, int max_blocks,
                           const int32_t* context_lens, int Hq, int Hkv, int dh, int bs, int fmt,
                           float softmax_scale) {
  int G = Hq / Hkv;
  double sm = default_scale(softmax_scale, dh);
#pragma omp parallel for schedule(dynamic)
  for (int i = 0; i < n; ++i) {
    int b = rows[2 * i], hq = rows[2 * i + 1];
    int h = hq / G;
    double qd[512];
    for (int d = 0; d < dh; ++d) qd[d] = (double)orc_bf16_to_f32(q[((int64_t)b * Hq + hq) * dh + d]);
    attend_one_ts(out + (int64_t)i * dh, qd, context_lens[b], k_cache, v_cache, k_scale_cache,
                  v_scale_cache, block_tables + (int64_t)b * max_blocks, h, Hkv, bs, dh, 1.0,
                  1.0, fmt, sm);
  }
}

uint64_t orc_kv_cache_bytes(int L, int B, int Hkv, int64_t S, int dh, int bits_per_elem) {
  uint64_t elems = 2ull * (uint64_t)L * (uint64_t)B * (uint64_t)Hkv * (uint64_t)S * (uint64_t)dh;
  return elems * (uint64_t)bits_per_elem / 8ull;
}

/* textbook 10.4.3: bytes one (token, head) costs for K and V together when each
 * of K and V carries its own per-token scale of scale_bytes. */
uint64_t orc_token_head_bytes(int dh, int bits_per_elem, int scale_bytes) {
  return 2ull * (uint64_t)dh * (uint64_t)bits_per_elem / 8ull + 2ull * (uint64_t)scale_bytes;
}

/* ---- KIVI-style asymmetric 2-bit KV (textbook 10.4.4: K grouped per channel
 * over G tokens, V per token over groups of channels; a high-precision residual
 * keeps the newest tokens unquantized).  The pages give the axes only; the
 * asymmetric codec is read as the plain min/max one:
 *   s = fl16(min(fl32(fl32(max - min) / 3), 65504)), z = fl16(clamp(min, +-65504))
 *   code = clip(round-half-even(fl32(fl32(x - z) / s)), 0, 3), or 0 when s == 0
 *   x_hat = code * s + z
 * over each set of 32 values (K: one channel of a 32-token group; V: one
 * 32-channel group of one token).  A set holding an Inf or NaN gets s = z = 0
 * (every code 0).  fp16 rounding is to nearest even.
 * Layout (this library's design; dh = 128): the quantized part is paged in
 * 32-token blocks, one K group per block, and each (block, head) tile is 3072
 * bytes: K codes [0, 1024), K scales (fp16, per channel) [1024, 1280), K zeros
 * [1280, 1536), V codes [1536, 2560), V (scale, zero) pairs per (token,
 * 32-channel group) [2560, 3072).  Code positions are given by kivi_k_pos and
 * kivi_v_pos below.  The residual holds the newest tokens in bf16, token-major
 * [B][Hkv][R][dh] for K and for V, oldest first. ---- */

#define KIVI_G 32
#define KIVI_DH 128
#define KIVI_TILE 3072

static uint16_t f16_bits_signed(double x) { /* |x| <= 65504, round to nearest even */
  if (x < 0) return (uint16_t)(0x8000u | f16_bits_rne(-x));
  return f16_bits_rne(x);
}

/* (s, z) fp16 bits of a set of n finite-or-not values */
static void kivi_params(const float* x, int n, uint16_t* s16, uint16_t* z16) {
  float mn = INFINITY, mx = -INFINITY;
  for (int i = 0; i < n; ++i) {
    if (!isfinite(x[i])) { *s16 = 0; *z16 = 0; return; }
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  float range = (float)((double)mx - (double)mn);   /* fl32(max - min) */
  float s = (float)((double)range / 3.0);           /* fl32(range / 3) */
  double sd = s > 65504.0f ? 65504.0 : (double)s;
  double zd = mn < -65504.0f ? -65504.0 : (mn > 65504.0f ? 65504.0 : (double)mn);
  *s16 = f16_bits_rne(sd);
  *z16 = f16_bits_signed(zd);
}

static uint8_t kivi_code(float x, uint16_t s16, uint16_t z16) {
  double s = orc_f16_to_double(s16);
  if (s == 0.0) return 0;
  float d = (float)((double)x - orc_f16_to_double(z16));  /* fl32(x - z) */
  float q = (float)((double)d / s);                       /* fl32(d / s) */
  double r = rint((double)q);
  if (r < 0.0) r = 0.0;
  if (r > 3.0) r = 3.0;
  return (uint8_t)r;
}

/* One set: its (s, z) and codes (for tests). */
void orc_kivi_group(const float* x, int n, uint16_t* s16, uint16_t* z16, uint8_t* codes) {
  kivi_params(x, n, s16, z16);
  for (int i = 0; i < n; ++i) codes[i] = kivi_code(x[i], *s16, *z16);
}

/* byte and bit offset of the code of token t (0..31), channel c (0..127) in a tile */
void orc_kivi_k_pos(int t, int c, int* byte, int* bit) {
  int th = t / 16, c16 = t % 16, j = c / 32, g4 = (c % 32) / 8, i = c % 8;
  int lane = 16 * g4 + c16;
  *byte = 16 * lane + 8 * th + 4 * (j / 2) + i / 2;
  *bit = 4 * (i % 2) + 2 * (j % 2);
}

void orc_kivi_v_pos(int t, int c, int* byte, int* bit) {
  int lane = c % 64, hc = c / 64, w = t / 16, sl = (t % 16) / 4, u = t % 4;
  *byte = 1536 + 16 * lane + 8 * hc + 4 * w + 2 * (sl % 2) + u / 2;
  *bit = 4 * (u % 2) + 2 * (sl / 2);
}

static void put_code(uint8_t* tile, int byte, int bit, uint8_t code) {
  tile[byte] = (uint8_t)((tile[byte] & ~(3u << bit)) | ((unsigned)code << bit));
}

static uint8_t get_code(const uint8_t* tile, int byte, int bit) {
  return (uint8_t)((tile[byte] >> bit) & 3u);
}

static void put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xff);
  p[1] = (uint8_t)(v >> 8);
}

static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* Quantize whole 32-token groups: k, v bf16 [n_groups * 32][Hkv][128]; group g
 * goes to block group_blocks[g] (skipped when outside [0, num_blocks)). */
void orc_kivi_quantize(const uint16_t* k, const uint16_t* v, int64_t n_groups, int Hkv,
                       const int32_t* group_blocks, uint8_t* cache, int64_t num_blocks) {
#pragma omp parallel for schedule(static)
  for (int64_t g = 0; g < n_groups; ++g) {
    int64_t blk = group_blocks[g];
    if (blk < 0 || blk >= num_blocks) continue;
    for (int h = 0; h < Hkv; ++h) {
      uint8_t* tile = cache + (blk * Hkv + h) * KIVI_TILE;
      float x[KIVI_G];
      uint16_t s16, z16;
      for (int c = 0; c < KIVI_DH; ++c) { /* K: one channel over the group's tokens */
        for (int t = 0; t < KIVI_G; ++t)
          x[t] = orc_bf16_to_f32(k[((g * KIVI_G + t) * Hkv + h) * KIVI_DH + c]);
        kivi_params(x, KIVI_G, &s16, &z16);
        put_u16(tile + 1024 + 2 * c, s16);
        put_u16(tile + 1280 + 2 * c, z16);
        for (int t = 0; t < KIVI_G; ++t) {
          int byte, bit;
          orc_kivi_k_pos(t, c, &byte, &bit);
          put_code(tile, byte, bit, kivi_code(x[t], s16, z16));
        }
      }
      for (int t = 0; t < KIVI_G; ++t) { /* V: one token over 32-channel groups */
        for (int gc = 0; gc < KIVI_DH / 32; ++gc) {
          for (int i = 0; i < 32; ++i)
            x[i] = orc_bf16_to_f32(v[((g * KIVI_G + t) * Hkv + h) * KIVI_DH + 32 * gc + i]);
          kivi_params(x, 32, &s16, &z16);
          put_u16(tile + 2560 + 16 * t + 4 * gc, s16);
          put_u16(tile + 2560 + 16 * t + 4 * gc + 2, z16);
          for (int i = 0; i < 32; ++i) {
            int byte, bit;
            orc_kivi_v_pos(t, 32 * gc + i, &byte, &bit);
            put_code(tile, byte, bit, kivi_code(x[i], s16, z16));
          }
        }
      }
    }
  }
}

/* Dequantized tile of one (block, head): k_hat, v_hat fp64 [32][128]. */
void orc_kivi_dequant_tile(const uint8_t* tile, double* kh, double* vh) {
  for (int c = 0; c < KIVI_DH; ++c) {
    double s = orc_f16_to_double(get_u16(tile + 1024 + 2 * c));
    double z = orc_f16_to_double(get_u16(tile + 1280 + 2 * c));
    for (int t = 0; t < KIVI_G; ++t) {
      int byte, bit;
      orc_kivi_k_pos(t, c, &byte, &bit);
      kh[t * KIVI_DH + c] = (double)get_code(tile, byte, bit) * s + z;
    }
  }
  for (int t = 0; t < KIVI_G; ++t) {
    for (int c = 0; c < KIVI_DH; ++c) {
      const uint8_t* m = tile + 2560 + 16 * t + 4 * (c / 32);
      double s = orc_f16_to_double(get_u16(m)), z = orc_f16_to_double(get_u16(m + 2));
      int byte, bit;
      orc_kivi_v_pos(t, c, &byte, &bit);
      vh[t * KIVI_DH + c] = (double)get_code(tile, byte, bit) * s + z;
    }
  }
}

/* Decode rows (b, hq) over a KIVI cache: the sequence's keys are its
 * quant_groups[b] quantized groups (block_tables[b][0..]) followed by its
 * res_lens[b] residual tokens, in position order; attention as textbook
 * 10.4.2 on the dequantized values.  out: fp64 [n][128]. */
void orc_kivi_decode_rows(double* out, const int32_t* rows, int n, const uint16_t* q,
                          const uint8_t* cache, const int32_t* block_tables, int max_blocks,
                          const int32_t* quant_groups, const uint16_t* res_k,
                          const uint16_t* res_v, const int32_t* res_lens, int R, int Hq, int Hkv,
                          float softmax_scale) {
  int G = Hq / Hkv;
  double sm = default_scale(softmax_scale, KIVI_DH);
#pragma omp parallel for schedule(dynamic)
  for (int i = 0; i < n; ++i) {
    int b = rows[2 * i], hq = rows[2 * i + 1], h = hq / G;
    int ng = quant_groups[b], nr = res_lens[b];
    int nk = ng * KIVI_G + nr;
    double* kk = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * KIVI_DH);
    double* vv = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1) * KIVI_DH);
    for (int g = 0; g < ng; ++g) {
      int64_t blk = block_tables[(int64_t)b * max_blocks + g];
      orc_kivi_dequant_tile(cache + (blk * Hkv + h) * KIVI_TILE, kk + (int64_t)g * KIVI_G * KIVI_DH,
                            vv + (int64_t)g * KIVI_G * KIVI_DH);
    }
    for (int r = 0; r < nr; ++r)
      for (int d = 0; d < KIVI_DH; ++d) {
        int64_t src = (((int64_t)b * Hkv + h) * R + r) * KIVI_DH + d;
        kk[((int64_t)ng * KIVI_G + r) * KIVI_DH + d] = orc_bf16_to_f32(res_k[src]);
        vv[((int64_t)ng * KIVI_G + r) * KIVI_DH + d] = orc_bf16_to_f32(res_v[src]);
      }
    double qd[KIVI_DH];
    for (int d = 0; d < KIVI_DH; ++d)
      qd[d] = (double)orc_bf16_to_f32(q[((int64_t)b * Hq + hq) * KIVI_DH + d]);
    if (nk > 0)
      orc_dense_attn(out + (int64_t)i * KIVI_DH, qd, kk, vv, 1, nk, KIVI_DH, 0, sm);
    else
      for (int d = 0; d < KIVI_DH; ++d) out[(int64_t)i * KIVI_DH + d] = 0.0;
    free(kk);
    free(vv);
  }
}

/*
 * kvq.h -- C ABI of the FP8 paged KV-cache library for AMD Instinct MI355X (gfx950).
 *
 * Keys and values are quantized as they are written into a paged cache of OCP
 * FP8 codes (E4M3fn or E5M2), with one fp32 scale per tensor or per KV head,
 * and attention reads that cache with the dequantization fused into the
 * kernel: no bf16/fp32 copy of the cache is ever written.
 *
 * What each call computes is defined on these pages:
 *   [T] "10.4 KV Cache 量化: INT8 基础、KIVI 2-bit、FP8 KV" (KV-cache
 *       quantization textbook chapter): 10.4.1 memory formula, 10.4.2 write /
 *       read / attention equations and the fused-dequant path, 10.4.3 scale
 *       granularity, 10.4.5 FP8 storage and compute types.
 *   [G] "vLLM FP8 量化 KV Cache 完整指南" (vLLM FP8 KV-cache guide): the
 *       kv_cache_dtype formats, per-tensor / per-attention-head scale shapes,
 *       scale sources (default 1.0), FP8 caches held as uint8 tensors, and the
 *       FP8-domain attention path that also quantizes Q.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Memory: every pointer argument is DEVICE memory on the current HIP device,
 *   allocated and owned by the caller.  The library allocates nothing and keeps
 *   no state except a cached copy of the device's compute-unit count.
 * - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Every call only enqueues work on that stream and returns; a
 *   status of KVQ_OK means the arguments were valid and the launches were
 *   accepted.  Faults inside a kernel surface at the caller's synchronize.
 * - Validation happens on the host before any HIP call, so a call with
 *   invalid arguments returns an error and touches no device memory.
 * - bf16 tensors are passed as void* holding IEEE bfloat16 bit patterns.
 * - Alignment: bf16 inputs, caches, attention outputs and the decode
 *   workspace must be 16-byte aligned, slot mappings 8-byte aligned (every
 *   torch allocation is); otherwise the call returns KVQ_ERR_UNSUPPORTED.
 * - Cache layout (this library's design; the pages fix only that FP8 caches
 *   are raw bytes): k_cache is uint8 [num_blocks][Hkv][dh/16][bs][16] (each
 *   tile is cut into 16-channel chunks, token-major inside a chunk: channel d
 *   of the token at offset o sits at byte (d/16)*bs*16 + o*16 + d%16 of its
 *   tile) and v_cache is uint8 [num_blocks][Hkv][dh][bs] (channel-major tiles).
 *   Token position j of sequence b lives in physical block
 *   block_tables[b][j / bs] at offset j % bs.  Each (block, head) tile is one
 *   contiguous bs*dh-byte run.  The K order lets one 64-lane load of the
 *   matrix-core operand (16 tokens x 4 chunks) cover 1 KB of contiguous
 *   memory; V is channel-major because P V contracts over tokens.
 * - GQA: query head hq reads KV head hq / (Hq / Hkv).
 * - Supported now: dh in {64, 128}; bs == 16; Hq % Hkv == 0; Hq/Hkv <= 16.
 * - Calls are reentrant; calls on the same stream run in order.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = -1,        /* a required pointer is NULL */
  KVQ_ERR_SHAPE = -2,       /* a size is negative, zero where it may not be, or inconsistent */
  KVQ_ERR_UNSUPPORTED = -3, /* a valid but unimplemented value (dh, bs, group size, enum) */
  KVQ_ERR_WORKSPACE = -4,   /* the decode workspace is smaller than kvq_decode_workspace_size */
  KVQ_ERR_LAUNCH = -5,      /* the HIP runtime refused a launch (hipGetLastError) */
  KVQ_ERR_DEVICE = -6,      /* no usable HIP device, or it is not gfx950 */
  KVQ_ERR_SCRATCH = -7      /* beyond the static scratch of kvq_decode_attn_append_noalloc */
} kvq_status;

/* Storage format of the cache codes ([G] kv_cache_dtype table: fp8 == fp8_e4m3,
 * fp8_e5m2).  OCP E4M3fn: bias 7, max 448, no Inf, NaN = S.1111.111.
 * OCP E5M2: bias 15, max 57344, IEEE-style Inf/NaN.
 * INT8: symmetric 8-bit integers, [T] 10.4.2's write rule
 *   code = clip(round(x / s), -127, 127) (ties to even; a NaN quotient gives 0,
 *   +-Inf clip to +-127), read back as s * code; "max" (for calibration) is
 *   127.  Calibration, the codec, quantize-write and decode attention take it;
 *   the FP8-domain prefill does not (KVQ_ERR_UNSUPPORTED). */
typedef enum { KVQ_FMT_E4M3 = 0, KVQ_FMT_E5M2 = 1, KVQ_FMT_INT8 = 2 } kvq_fmt;

/* Scale granularity ([T] 10.4.3 table; [G] shapes [1] vs [num_heads] /
 * [num_kv_heads]): one fp32 scale for the whole tensor, or one per head. */
typedef enum { KVQ_SCALE_TENSOR = 0, KVQ_SCALE_HEAD = 1 } kvq_gran;

/* Element type of attention outputs. */
typedef enum { KVQ_OUT_F32 = 0, KVQ_OUT_BF16 = 1 } kvq_out;

/* Entry points take these three as plain int parameters, so a value outside
 * the enumeration is a defined input that returns KVQ_ERR_UNSUPPORTED. */

typedef void* kvq_stream; /* hipStream_t */

/* Human-readable text for a status code (static storage, never NULL).  Takes
 * any int: a value that is no kvq_status gives "unknown status". */
const char* kvq_strerror(int status);

/* Bytes of a KV cache payload, [T] 10.4.1:
 *   M_KV = 2 * L * B * Hkv * S * dh * bits_per_elem / 8
 * (the 2 counts K and V; metadata, padding and scales are not included).
 * Pure host arithmetic; returns 0 if any argument is negative. */
uint64_t kvq_kv_cache_bytes(int L, int B, int Hkv, int64_t S, int dh, int bits_per_elem);

/* ---------------------------------------------------------------- codec
 * The element codec every kernel uses ([T] 10.4.5: cast_fp8 on write,
 * cast_float on read), exposed for callers and tests.
 *   kvq_fp8_encode: out[i] = saturating round-to-nearest-even code of x[i]
 *     (|x| beyond max and +-Inf give +-max; NaN gives a NaN code; -0 gives
 *     0x80; subnormal codes are produced).  x: fp32 [n], out: uint8 [n].
 *   kvq_fp8_decode: out[i] = exact fp32 value of code[i] (NaN codes give NaN,
 *     E5M2 Inf codes give +-Inf).  codes: uint8 [n], out: fp32 [n].
 * n == 0 is a no-op.  Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE (n < 0),
 * KVQ_ERR_UNSUPPORTED (fmt). */
kvq_status kvq_fp8_encode(int fmt, const float* x, int64_t n, uint8_t* out,
                          kvq_stream stream);
kvq_status kvq_fp8_decode(int fmt, const uint8_t* codes, int64_t n, float* out,
                          kvq_stream stream);

/* ---------------------------------------------------------------- calibration
 * Scale calibration ([T] 10.4.3 per-tensor / per-head; [G] scale shapes and
 * scale sources: scales fitted to the activation range, 1.0 without one).
 *   x: bf16 [T][H][dh].
 *   amax = max |x| over the whole tensor (gran == KVQ_SCALE_TENSOR, arrays of
 *     length 1) or over x[:, h, :] for each h (KVQ_SCALE_HEAD, length H).
 *     A NaN anywhere in a set makes that amax NaN.
 *   accumulate == 0: amax_io <- amax.  accumulate != 0: amax_io <- max(amax_io,
 *     amax), so calibration can continue over further batches.
 *   scale_out <- amax_io / fmax(fmt) correctly rounded in fp32 if that amax is
 *     finite and > 0, else 1.0.
 * T == 0 is allowed (amax of an empty set is 0).  amax_io and scale_out are
 * fp32 device arrays.  Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE (T < 0, H < 1,
 * dh < 1 or dh % 8), KVQ_ERR_UNSUPPORTED (fmt, gran). */
kvq_status kvq_calibrate_scales(const void* x_bf16, int64_t T, int H, int dh, int fmt,
                                int gran, float* amax_io, float* scale_out, int accumulate,
                                kvq_stream stream);

/* K and V calibrated together ([G] scale sources: k_scale and v_scale are
 * fitted from the K and V activations of the same layer): exactly
 *   kvq_calibrate_scales(k_bf16, ..., k_amax_io, k_scale_out, ...) and
 *   kvq_calibrate_scales(v_bf16, ..., v_amax_io, v_scale_out, ...)
 * (bit-identical results), with K and V of one shape [T][H][dh] sharing each
 * of the three launches (clear, reduce, finalize) instead of taking three each.
 * The four output arrays must not overlap.  Errors as kvq_calibrate_scales. */
kvq_status kvq_calibrate_scales_kv(const void* k_bf16, const void* v_bf16, int64_t T, int H,
                                   int dh, int fmt, int gran, float* k_amax_io, float* v_amax_io,
                                   float* k_scale_out, float* v_scale_out, int accumulate,
                                   kvq_stream stream);

/* ---------------------------------------------------------------- quantize-write
 * Quantize-on-write into the paged cache ([T] 10.4.2 write rule, 10.4.5
 * cast_fp8(K / sK)):
 *   for every token t with 0 <= slot_mapping[t] < num_blocks * bs, every KV
 *   head h and channel d:
 *     k_cache[slot / bs][h][d / 16][slot % bs][d % 16] = fp8(fl32(k[t][h][d] / sK))
 *     v_cache[slot / bs][h][d][slot % bs] = fp8(fl32(v[t][h][d] / sV))
 *   with s = scale[h] (KVQ_SCALE_HEAD) or scale[0] (KVQ_SCALE_TENSOR), the
 *   quotient correctly rounded to fp32 and fp8() the encoder above.  Tokens
 *   whose slot is negative (padding) or out of range are skipped; no other
 *   cache byte is touched; if two tokens name the same slot, which one lands
 *   is unspecified.  Scales must be positive finite fp32 values below
 *   2^126 (subnormal ones included); every scale kvq_calibrate_scales returns
 *   is one.  Other values give unspecified codes.
 *   k, v: bf16 [T][Hkv][dh]; slot_mapping: int64 [T].
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_cache_write(const void* k_bf16, const void* v_bf16, int64_t T, int Hkv, int dh,
                           const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                           int64_t num_blocks, int bs, const float* k_scale,
                           const float* v_scale, int fmt, int gran, kvq_stream stream);

/* ---------------------------------------------------------------- decode
 * Bytes of device workspace kvq_decode_attn needs for these sizes (split-K
 * partial results).  Returns 0 for invalid sizes.  The size never decreases as
 * max_context_len grows (B, Hq, dh and bs fixed), so a workspace sized for the
 * longest context serves every shorter call. */
size_t kvq_decode_workspace_size(int B, int Hq, int dh, int max_context_len, int bs);

/* Paged decode attention over the FP8 cache with the dequantization fused in
 * ([T] 10.4.2: P = softmax(Q K_hat^T / sqrt(dh)), O = P V_hat with
 * K_hat = sK * K8, V_hat = sV * V8; the fused path of the same section).
 *   q: bf16 [B][Hq][dh], one query per sequence: the newest token, whose own
 *     K/V must already be in the cache.  It attends to every cached position
 *     0 .. context_lens[b]-1 (no mask).
 *   block_tables: int32 [B][max_blocks]; context_lens: int32 [B], read on the
 *     device only.  max_context_len: host-side bound, >= every context_lens[b]
 *     (larger values are clamped to it) and <= max_blocks * bs.
 *   num_blocks: pool size; block ids outside [0, num_blocks) are clamped into
 *     it, so a corrupt table gives wrong numbers but never an out-of-bounds read.
 *   softmax_scale <= 0 means 1/sqrt(dh).
 *   out: [B][Hq][dh] fp32 or bf16 (round-to-nearest-even); a sequence with
 *     context length 0 gets an all-zero row.
 *   workspace: device buffer of >= kvq_decode_workspace_size(...) bytes; its
 *     contents need no initialisation and are overwritten.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE. */
kvq_status kvq_decode_attn(void* out, int out_dtype, const void* q_bf16,
                           const uint8_t* k_cache, const uint8_t* v_cache, int64_t num_blocks,
                           const int32_t* block_tables, int max_blocks,
                           const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                           int max_context_len, const float* k_scale, const float* v_scale,
                           int fmt, int gran, float softmax_scale, void* workspace,
                           size_t ws_bytes, kvq_stream stream);

/* ---------------------------------------------------------------- skip-layers, padded pages
 * Mixed quantized / unquantized layers ([G] kv_cache_dtype_skip_layers): the
 * listed layers keep the model's native dtype ("auto"), every other layer
 * uses the quantized cache; skipped layers still take part in the page
 * (block) alignment, the smaller pages being padded so that the mixed cache
 * lines up page by page.
 *
 * Reading of the skip rule: a layer is skipped when it is a sliding-window
 * layer and the list holds "sliding_window", or when the list holds its layer
 * index written in decimal ("0", "1", "23").  Returns 1 (skipped) or 0. */
int kvq_layer_skipped(int layer_index, int is_sliding_window, const char* const* skip_list,
                      int n_skip);

/* The layer index inside a module prefix such as "model.layers.12.self_attn":
 * the one dot-separated component made only of decimal digits; -1 when there
 * is none or more than one. */
int kvq_layer_index(const char* prefix);

/* Bytes of one page (one block of bs tokens, K and V, all KV heads) of a
 * layer whose cache stores bits_per_elem bits per element: 2 Hkv bs dh bits/8
 * (0 for negative arguments). */
uint64_t kvq_page_bytes(int Hkv, int dh, int bs, int bits_per_elem);

/* Reading of the page padding: every layer's pages are padded to the largest
 * natural page among the L layers (layer_bits[l] = 16 for a skipped bf16
 * layer, 8 for an FP8 / INT8 one), rounded up to 16 bytes.  0 for invalid
 * arguments. */
uint64_t kvq_common_page_bytes(const int* layer_bits, int L, int Hkv, int dh, int bs);

/* The quantized calls on a padded layout: block b of k_cache starts at byte
 * b * block_stride (likewise v_cache), block_stride >= Hkv * bs * dh and a
 * multiple of 16; inside a block the layout is the one above.  One page of a
 * mixed pool holds a layer's K block then its V block (k_cache = page base,
 * v_cache = page base + Hkv * bs * dh, block_stride = the common page size);
 * padding bytes are never read or written.  Otherwise identical to
 * kvq_cache_write / kvq_decode_attn / kvq_prefill_attn, which are these calls
 * with block_stride = Hkv * bs * dh.
 * Errors: as the unpadded calls; KVQ_ERR_SHAPE for a block_stride below
 * Hkv * bs * dh, KVQ_ERR_UNSUPPORTED when it is not a multiple of 16. */
kvq_status kvq_cache_write_paged(const void* k_bf16, const void* v_bf16, int64_t T, int Hkv,
                                 int dh, const int64_t* slot_mapping, uint8_t* k_cache,
                                 uint8_t* v_cache, int64_t num_blocks, int bs,
                                 int64_t block_stride, const float* k_scale,
                                 const float* v_scale, int fmt, int gran,
                                 kvq_stream stream);
kvq_status kvq_decode_attn_paged(void* out, int out_dtype, const void* q_bf16,
                                 const uint8_t* k_cache, const uint8_t* v_cache,
                                 int64_t num_blocks, const int32_t* block_tables, int max_blocks,
                                 const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                                 int bs, int64_t block_stride, int max_context_len,
                                 const float* k_scale, const float* v_scale, int fmt,
                                 int gran, float softmax_scale, void* workspace,
                                 size_t ws_bytes, kvq_stream stream);
kvq_status kvq_prefill_attn_paged(void* out, int out_dtype, const void* q_bf16,
                                  const int32_t* cu_seqlens_q, int max_q_len,
                                  const float* q_scale, int q_gran, const uint8_t* k_cache,
                                  const uint8_t* v_cache, int64_t num_blocks,
                                  const int32_t* block_tables, int max_blocks,
                                  const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                                  int bs, int64_t block_stride, const float* k_scale,
                                  const float* v_scale, int fmt, int kv_gran,
                                  float softmax_scale, kvq_stream stream);

/* ---------------------------------------------------------------- per-token-head scales
 * Finer scale granularity ([T] 10.4.3: one scale per token row along dh; its
 * metadata example keeps one FP16 scale for K and one for V per token and
 * head).  The scales live in caches paged like the codes:
 *   k_scale_cache, v_scale_cache: fp16 bit patterns, uint16 [num_blocks][Hkv][bs];
 *   the scale of the token at slot s and head h sits at [s / bs][h][s % bs].
 *
 * Quantize-on-write computing each row's own scale: for every token t with
 * 0 <= slot_mapping[t] < num_blocks * bs and every KV head h, with
 * amax = max_d |x[t][h][d]| (x = k, then v):
 *   s = fl16(clamp(fl32(amax / fmax(fmt)), 2^-24, 65504))  (round to nearest
 *       even; 1.0 if amax is 0 or the row holds an Inf or NaN)
 *   codes as kvq_cache_write with that s; the scale caches receive s.
 * Skipped tokens touch neither codes nor scales.  Any fmt; dh in {64, 128};
 * bs == 16.  The scale caches must be 2-byte aligned.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_cache_write_token_scales(const void* k_bf16, const void* v_bf16, int64_t T,
                                        int Hkv, int dh, const int64_t* slot_mapping,
                                        uint8_t* k_cache, uint8_t* v_cache,
                                        uint16_t* k_scale_cache, uint16_t* v_scale_cache,
                                        int64_t num_blocks, int bs, int fmt,
                                        kvq_stream stream);

/* Paged decode over a cache written by kvq_cache_write_token_scales: as
 * kvq_decode_attn with K_hat[j] = sK[j] * K8[j] and V_hat[j] = sV[j] * V8[j]
 * per cached position j ([T] 10.4.2 read rule at 10.4.3's per-token
 * granularity).  Only groups of at most 4 query heads per KV head
 * (Hq / Hkv <= 4) are supported; larger groups return KVQ_ERR_UNSUPPORTED.
 * The workspace is sized by kvq_decode_workspace_size as for kvq_decode_attn.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE. */
kvq_status kvq_decode_attn_token_scales(void* out, int out_dtype, const void* q_bf16,
                                        const uint8_t* k_cache, const uint8_t* v_cache,
                                        const uint16_t* k_scale_cache,
                                        const uint16_t* v_scale_cache, int64_t num_blocks,
                                        const int32_t* block_tables, int max_blocks,
                                        const int32_t* context_lens, int B, int Hq, int Hkv,
                                        int dh, int bs, int max_context_len, int fmt,
                                        float softmax_scale, void* workspace, size_t ws_bytes,
                                        kvq_stream stream);

/* ---------------------------------------------------------------- KIVI 2-bit
 * KIVI-style asymmetric 2-bit KV ([T] 10.4.4: K quantized per channel within
 * groups of G tokens, V per token within groups of channels; the newest
 * tokens stay unquantized in a high-precision residual and are compressed in
 * batches).  Here G = 32 tokens, V groups are 32 channels, dh = 128.  For each
 * set of 32 values (K: one channel of a 32-token group; V: one 32-channel
 * group of one token):
 *   s = fl16(min(fl32(fl32(max - min) / 3), 65504)), z = fl16(clamp(min, +-65504))
 *   code = clip(round-half-even(fl32(fl32(x - z) / s)), 0, 3)   (0 if s == 0)
 *   x_hat = code * s + z;  a set holding an Inf or NaN stores s = z = 0.
 * (fp16 rounding is to nearest even.)
 * kivi_cache: uint8 [num_blocks][Hkv][3072], one 32-token block (= one K group)
 *   per tile.  Tile bytes: [0, 1024) K codes, [1024, 1280) K scales and
 *   [1280, 1536) K zeros (fp16 per channel), [1536, 2560) V codes,
 *   [2560, 3072) V (scale, zero) fp16 pairs [token][channel group].  The code
 *   bit positions are this library's design (kivi.hip states them); the
 *   cache is only meant to be read by kvq_kivi_decode_attn.
 * Residual: res_k, res_v bf16 [B][Hkv][R][128], token-major; sequence b's
 *   res_lens[b] newest tokens, oldest first, follow its quantized groups.
 *
 * Quantize whole groups: k, v bf16 [n_groups * 32][Hkv][128]; tokens
 * 32 g .. 32 g + 31 form group g and go to block group_blocks[g] (int32
 * [n_groups]; a block outside [0, num_blocks) skips the group).  Only the
 * target tiles are written; two groups that name the same block leave that
 * tile's contents unspecified (each writes its tile piece by piece).
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED (dh != 128, alignment). */
kvq_status kvq_kivi_quantize(const void* k_bf16, const void* v_bf16, int64_t n_groups, int Hkv,
                             int dh, const int32_t* group_blocks, uint8_t* kivi_cache,
                             int64_t num_blocks, kvq_stream stream);

/* Bytes of device workspace kvq_kivi_decode_attn needs (0 for invalid sizes).
 * Never decreases as max_groups grows (B, Hq and Hkv fixed), so a workspace
 * sized for the largest max_groups serves every smaller call. */
size_t kvq_kivi_decode_workspace_size(int B, int Hq, int Hkv, int max_groups);

/* Decode attention over a KIVI cache ([T] 10.4.2 attention on the values
 * x_hat read back per 10.4.4's grouping): the query of sequence b attends its
 * quant_groups[b] quantized groups (blocks block_tables[b][0 .. quant_groups[b]-1],
 * positions 32 g .. 32 g + 31) and then its res_lens[b] residual tokens.
 *   q: bf16 [B][Hq][128]; out: [B][Hq][128] fp32 or bf16; Hq / Hkv <= 4.
 *   quant_groups, res_lens: int32 [B], read on the device, clamped to
 *     [0, max_groups] and [0, R]; max_groups <= max_blocks; 1 <= R <= 256.
 *   Block ids outside the pool are clamped into it.
 *   softmax_scale <= 0 means 1/sqrt(128).  A sequence with no tokens gets an
 *   all-zero row.
 * Precision: the quantized part runs on f16 matrix cores (q s, z, q and the
 * dequantized V in f16, P in f16, fp32 accumulation), so |q|, |K| and |V|
 * must lie within the fp16 range; the residual is attended in fp32.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED, KVQ_ERR_WORKSPACE. */
kvq_status kvq_kivi_decode_attn(void* out, int out_dtype, const void* q_bf16,
                                const uint8_t* kivi_cache, int64_t num_blocks,
                                const int32_t* block_tables, int max_blocks,
                                const int32_t* quant_groups, int max_groups,
                                const void* res_k_bf16, const void* res_v_bf16,
                                const int32_t* res_lens, int R, int B, int Hq, int Hkv, int dh,
                                float softmax_scale, void* workspace, size_t ws_bytes,
                                kvq_stream stream);

/* Decode with the step's new token appended: for every sequence b with
 * 1 <= context_lens[b] <= max_context_len the new token's K and V
 * (k_new, v_new: bf16 [B][Hkv][dh]) are quantized and written at position
 * context_lens[b] - 1, i.e. block block_tables[b][pos / bs], offset pos % bs
 * (skipped when that block id lies outside [0, num_blocks)), and the query
 * then attends positions 0 .. context_lens[b] - 1 as in kvq_decode_attn.
 * The result and the cache bytes equal kvq_cache_write of those tokens
 * followed by kvq_decode_attn; here one kernel does both ([T] 10.4.2 write
 * rule and attention of the same step), so no launch sits between them.
 * A sequence whose context_lens[b] exceeds max_context_len (a bound taken
 * before the lengths grew) attends its first max_context_len positions, as
 * kvq_decode_attn does, and its new token is neither written nor attended: no
 * cache byte of it changes.  k_new / v_new must be 16-byte aligned.
 * Errors: as kvq_decode_attn. */
kvq_status kvq_decode_attn_append(void* out, int out_dtype, const void* q_bf16,
                                  const void* k_new_bf16, const void* v_new_bf16,
                                  uint8_t* k_cache, uint8_t* v_cache, int64_t num_blocks,
                                  const int32_t* block_tables, int max_blocks,
                                  const int32_t* context_lens, int B, int Hq, int Hkv, int dh,
                                  int bs, int max_context_len, const float* k_scale,
                                  const float* v_scale, int fmt, int gran,
                                  float softmax_scale, void* workspace, size_t ws_bytes,
                                  kvq_stream stream);

/* Bytes of the device scratch array kvq_decode_attn_append_noalloc keeps its
 * split partials in (16 MiB; one array per GPU). */
#define KVQ_STATIC_SCRATCH_BYTES ((size_t)16 << 20)

/* kvq_decode_attn_append for callers that cannot allocate device memory --
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation: the same kernels and the same results, bit for bit, but the
 * split partials live in a file-scope device array of
 * KVQ_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends, so no workspace is passed and nothing is allocated
 * (no hipMalloc, no hipFree, no allocating library call).  The caller still
 * passes every input and output.  The array's address on a device is looked
 * up on the first call made with that device current.
 * Limit: calls whose kvq_decode_workspace_size(B, Hq, dh, max_context_len, bs)
 * exceeds KVQ_STATIC_SCRATCH_BYTES return KVQ_ERR_SCRATCH before any device
 * work (B = 32, Hq = 32, dh = 128, bs = 16 fits up to max_context_len = 19840).
 * Every call on a GPU shares that GPU's array, which keeps the last call's
 * contents (no call reads what another left there): calls that overlap in
 * time on one GPU -- on different streams, or from different threads -- race
 * and must be ordered by the caller.
 * Errors: as kvq_decode_attn_append without KVQ_ERR_WORKSPACE, plus
 * KVQ_ERR_SCRATCH; KVQ_ERR_DEVICE if the array's address cannot be found. */
kvq_status kvq_decode_attn_append_noalloc(void* out, int out_dtype, const void* q_bf16,
                                          const void* k_new_bf16, const void* v_new_bf16,
                                          uint8_t* k_cache, uint8_t* v_cache, int64_t num_blocks,
                                          const int32_t* block_tables, int max_blocks,
                                          const int32_t* context_lens, int B, int Hq, int Hkv,
                                          int dh, int bs, int max_context_len,
                                          const float* k_scale, const float* v_scale,
                                          int fmt, int gran, float softmax_scale,
                                          kvq_stream stream);

/* ---------------------------------------------------------------- prefill
 * Causal chunked prefill in the FP8 domain ([G] the FlashAttention-3 note:
 * attention computed on FP8 operands with Q quantized too; [T] 10.4.5 storage
 * vs compute type; [T] 10.4.2 attention with a mask):
 *   q: bf16 [total_q][Hq][dh], variable length: sequence b owns rows
 *     cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (int32 [B+1], cu_seqlens_q[0] = 0),
 *     read on the device only; max_q_len bounds every chunk length on the host
 *     (rows of a longer chunk past that bound are left unspecified).  An empty
 *     chunk (cu_seqlens_q[b+1] == cu_seqlens_q[b]) is allowed.
 *   Row i of sequence b is the token at absolute position
 *     context_lens[b] - qlen_b + i and attends keys 0..position (causal).  The
 *     chunk's own K/V must already be in the cache (kvq_cache_write).
 *     context_lens: int32 [B], read on the device, clamped to
 *     [0, max_blocks * bs]; a row whose position is negative (a context
 *     shorter than its chunk) sees no key and gets an all-zero row.
 *   Block ids outside [0, num_blocks) are clamped into the pool, as in decode.
 *   Q is quantized in-kernel to E4M3 with q_scale (q_gran: [1] or [Hq]):
 *     q_hat = s_q * fp8(fl32(q / s_q)); Q K^T runs on FP8 matrix cores with
 *     fp32 accumulation; P is fed to the P V product as two E4M3 terms,
 *     P_hi = fp8(F p) and P_lo = fp8(16 (F p - P_hi)) with F = 64 and the
 *     running max kept within 2 (log2) of the true one, recombined as
 *     (P_hi + P_lo / 16) / F, so the FP8 product keeps about 8 significant
 *     bits of P.
 *   out: [total_q][Hq][dh] fp32 or bf16.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_prefill_attn(void* out, int out_dtype, const void* q_bf16,
                            const int32_t* cu_seqlens_q, int max_q_len, const float* q_scale,
                            int q_gran, const uint8_t* k_cache, const uint8_t* v_cache,
                            int64_t num_blocks, const int32_t* block_tables, int max_blocks,
                            const int32_t* context_lens, int B, int Hq, int Hkv, int dh, int bs,
                            const float* k_scale, const float* v_scale, int fmt,
                            int kv_gran, float softmax_scale, kvq_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */

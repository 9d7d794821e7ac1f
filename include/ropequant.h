/*
 * libropequant - fused RoPE + block-FP8 steps around DeepSeek-V4-style
 * 512-dim attention heads, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "vLLM DeepSeek-V4 성능 최적화: Eager Break 시 Workspace 재사용 개선"
 *        (analysis of vLLM PR #49236): section 1 defines the fused q-norm/RoPE
 *        and kv-RoPE/quant/insert op with a caller-allocated q_out and lists its
 *        argument checks; section 2 gives its schema (outputs mutated, returns
 *        nothing), and names beside it the full-cache forms: q written in
 *        place (bf16) or to a separate FP8 tensor, kv into a contiguous,
 *        512-wide, token-strided cache.
 *   [P3] "vLLM, DeepSeek V4 모델의 저지연을 위한 RMSNorm과 라우터 GEMV 연산
 *        융합으로 성능 극대화" (analysis of vLLM PR #41263): section 5 gives the
 *        RMSNorm formula.
 *   [P4] "한 프로그램이 4개 head를 처리하게 하라: DeepSeek-V4 inverse RoPE +
 *        FP8 quant 커널 3.5배 가속기" (analysis of vLLM PR #63540): intro (the
 *        op sits before the wo_a projection), section 1 (heads grouped per
 *        wo_a group, scale column = head_in_group * 4 + block), section 2 (the
 *        GPT-J inverse rotation), section 3 (block-128 amax, UE8M0 packing),
 *        section 4 (the kernel's compile keys, among them `quantize`).
 *   [P5] "vLLM의 GLM5.2 성능 최적화: Triton 커널 융합을 통한 E2E Throughput
 *        향상" (analysis of vLLM PR #46862): section 1 (the fused indexer
 *        query kernel: rotate-half RoPE with a bf16 round trip, power-of-two
 *        scale, weight fold).
 *
 * Common conventions
 *   - Head vectors are 512 dims: dims 0..447 are not rotated, dims 448..511
 *     are rotated GPT-J style, in adjacent pairs (2k, 2k+1), k = 224..255.
 *   - cos_sin_cache is fp32 [max_pos, 64], row-major: row p holds cos in
 *     columns 0..31 and sin in columns 32..63; pair k uses column k-224 and
 *     32+k-224 of row positions[t].  It must be 16-byte aligned.
 *   - bf16 values are passed as their uint16_t bit patterns; e4m3 codes as
 *     uint8_t (OCP E4M3: bias 7, max 448, no infinities, 0x7F/0xFF NaN).
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees, synchronizes or keeps state; it is
 *     reentrant.  Work is enqueued on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and the call returns without waiting.
 *   - Launch shape: a fixed table picks the workgroup size from the size of
 *     the call alone (the analogue of [P4] section 4's program-count rule):
 *     calls of at least 16384 512-dim units (indexer: 16384 4-head items)
 *     use 256-thread workgroups, smaller calls 64.  Results never depend on
 *     the entry taken.
 *   - Return value: RQ_OK (0) or a negative RQ_ERR_* status.  On any error
 *     nothing is launched and no output byte is touched.  n_tokens == 0
 *     returns RQ_OK with no launch (pointers are then not inspected).
 *   - Device data is not read by the host.  Caller contract: positions in
 *     [0, max_pos); slots unique and below num_blocks * cache_block_size;
 *     input values finite (and |q| < 2^59 for qnorm_rope).  The kernels never
 *     access memory outside the described tensors even when the contract is
 *     broken: a unit whose position is out of range gets NaN scales (fp32
 *     NaN, or UE8M0 exponent bytes 0xFF), so every value it dequantizes to is
 *     NaN, its codes being unspecified; qnorm_rope writes such a head as bf16
 *     NaN (0x7FC0); and a slot outside [0, num_blocks * cache_block_size) is
 *     skipped.
 *   - Finite inputs can still rotate past the fp32 range (a GPT-J or
 *     rotate-half pair near the bf16 maximum).  The block holding such a
 *     value gets an infinite maximum and the IEEE results of the usual
 *     formulas: scale +inf (FP32; its other codes are signed zeros) or
 *     exponent byte 0xFF, the E8M0 NaN (UE8M0; its finite values scaled by
 *     2^-128), and for the indexer an infinite q_scale and folded weight.
 *     The code written for the infinite value itself is unspecified.
 *   - Strides are in elements of the tensor's own type unless "bytes" is said.
 *     Strides that place any element of a tensor more than 2^56 bytes from
 *     its base (or overflow 64-bit arithmetic on the way) return
 *     RQ_ERR_STRIDE: no device address space is that large.
 *   - Arithmetic: every fp32 step is an IEEE-754 basic operation rounded to
 *     nearest even, with no fused multiply-add; division and square root are
 *     correctly rounded; denormals are kept.
 */
#ifndef ROPEQUANT_H
#define ROPEQUANT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROPEQUANT_ABI_VERSION 3

enum {
  RQ_OK = 0,
  RQ_ERR_NULL = -1,   /* a required pointer is NULL */
  RQ_ERR_SHAPE = -2,  /* a size is out of range or inconsistent */
  RQ_ERR_STRIDE = -3, /* a stride is non-positive or lets outputs overlap */
  RQ_ERR_ALIGN = -4,  /* a pointer or stride breaks the required alignment */
  RQ_ERR_VALUE = -5,  /* a scalar argument (scale_fmt, eps) is invalid */
  RQ_ERR_HIP = -6     /* the HIP runtime refused the launch */
};

enum {
  RQ_SCALE_FP32 = 0,  /* one fp32 scale per 128-dim block: amax / 448 */
  RQ_SCALE_UE8M0 = 1  /* power-of-two scale, exponent byte per block */
};

/*
 * inv_rope_fp8_quant - inverse RoPE, then block-128 FP8 quantization, of the
 * attention output before the grouped wo_a projection ([P4] intro, sections
 * 1-3).  For every token t < n_tokens and head h < n_heads:
 *   x   = fp32(o[t, h, :])
 *   x'  = x with pairs k >= 224 rotated back:  e' = e*c + o*s,  o' = o*c - e*s
 *   m_b = max(max_{i in block b} |x'_i|, eps)            (b = 0..3)
 *   RQ_SCALE_FP32 : s_b = m_b / 448;  codes = e4m3_rne(x' * (1 / s_b))
 *   RQ_SCALE_UE8M0: k_b = smallest integer with 2^k_b >= m_b / 448;
 *                   codes = e4m3_rne(x' * 2^-k_b)
 * with g = h / heads_per_group, j = h % heads_per_group:
 *   out   [g*out_stride_group + t*out_stride_token + j*512 + d]  (bytes)
 *   FP32  scales (float*)   [g*sc_stride_group + t*sc_stride_token + (j*4+b)*sc_stride_block] = s_b
 *   UE8M0 scales (uint32_t*)[g*sc_stride_group + t*sc_stride_token + j*sc_stride_block]
 *         = sum_b (k_b + 127) << (8*b)      (block b in byte b)
 * Default (group-major, what wo_a consumes) layout: out [G, N, hpg*512] with
 * strides (N*hpg*512, hpg*512); FP32 scales [G, N, hpg*4] with strides
 * (N*hpg*4, hpg*4, 1); UE8M0 scales [G, N, hpg] with strides (N*hpg, hpg, 1).
 * Token-major [N, H, 512] is out strides (hpg*512, H*512).  Scales may also be
 * laid out MN-major for a GEMM that reads them per column (token fastest):
 * FP32 [G, hpg*4, N] is strides (hpg*4*N, 1, N); UE8M0 [G, hpg, N] is
 * (hpg*N, 1, N).
 *
 * o: bf16 [N, H, 512] with strides (o_stride_token, o_stride_head, 1); base
 *    16-byte aligned, strides positive multiples of 8.
 * positions: int64 [N].  eps: amax floor (>= 2^-116 as fp32; vLLM-style
 *    default 1e-10).  out: 16-byte aligned, strides positive multiples of 16,
 *    rows must not overlap.  scales: 4-byte aligned, positive strides, no two
 *    scales may share an address.  n_tokens * n_heads < 2^31.
 */
int inv_rope_fp8_quant(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                       const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                       int64_t n_tokens, int32_t n_heads, int32_t heads_per_group,
                       int32_t scale_fmt, double eps,
                       uint8_t* out, int64_t out_stride_group, int64_t out_stride_token,
                       void* scales, int64_t sc_stride_group, int64_t sc_stride_token,
                       int64_t sc_stride_block, void* stream);

/*
 * inv_rope_bf16 - the inverse RoPE of inv_rope_fp8_quant with the
 * quantization switched off ([P4] section 4 lists `quantize` among the
 * kernel's compile keys), for a wo_a projection that takes bf16:
 *   out[g*out_stride_group + t*out_stride_token + j*512 + d] = bf16_rne(x'_d)
 * with x', g, j as above (pass-through dims are thus copied bit for bit).
 * out: bf16, 16-byte aligned, strides (elements) positive multiples of 8,
 *   rows must not overlap.  Group-major [G, N, hpg*512] is strides
 *   (N*hpg*512, hpg*512); token-major [N, H, 512] is (hpg*512, H*512).
 *   out may be o itself only in that token-major form with o laid out
 *   [N, H, 512] (o_stride_head 512): each head then overwrites its own row;
 *   other aliasing returns RQ_ERR_STRIDE when out == o and is undefined
 *   otherwise.  A head whose position is out of range is written as bf16 NaN.
 */
int inv_rope_bf16(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                  const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                  int64_t n_tokens, int32_t n_heads, int32_t heads_per_group, uint16_t* out,
                  int64_t out_stride_group, int64_t out_stride_token, void* stream);

/*
 * qnorm_rope - per-head RMSNorm and forward RoPE of the queries, written into
 * a head-padded output whose pad heads are zero ([P1] section 1: q_out is
 * preallocated by the caller, every element is written so it may be
 * uninitialized, q_head_padded >= num_heads_q; [P3] section 5: RMSNorm).
 * For t < n_tokens, h < n_heads_q:
 *   x  = fp32(q_in[t, h, :])
 *   ss = sum of x_d^2 in a fixed order: 64 chunks of 8 consecutive dims, each
 *        summed left to right; then 6 butterfly rounds, chunk c adding chunk
 *        c xor k for k = 1, 2, 4, 8, 16, 32
 *   r  = 1 / sqrt(ss * (1/512) + eps)
 *   y  = (x * r) * w   (w = fp32(norm_weight), or y = x * r if norm_weight is NULL)
 *   y' = y with pairs k >= 224 rotated forward:  e' = e*c - o*s,  o' = o*c + e*s
 *   q_out[t, h, :] = bf16_rne(y')
 * and q_out[t, h, :] = +0 (0x0000) for n_heads_q <= h < q_head_padded.
 * q_in: bf16 [N, Hq, 512], strides (q_stride_token, q_stride_head, 1), base
 *   16-byte aligned, strides positive multiples of 8.  norm_weight: bf16
 *   [512] or NULL, 16-byte aligned.  q_out: bf16 [N, q_head_padded, 512]
 *   contiguous, 16-byte aligned.  eps: RMSNorm epsilon (> 0, fp32-finite).
 *   n_tokens * q_head_padded < 2^31.  In place ([P1] section 2's full-cache
 *   form): q_out may be q_in itself when q_head_padded == n_heads_q and q_in
 *   is contiguous; q_out == q_in with any other shape returns RQ_ERR_STRIDE.
 */
int qnorm_rope(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
               const uint16_t* norm_weight, const int64_t* positions,
               const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
               int32_t n_heads_q, int32_t q_head_padded, double eps, uint16_t* q_out,
               void* stream);

/*
 * qnorm_rope_fp8 - the q path written to a separate FP8 tensor ([P1] section
 * 2's full-cache form).  y' as in qnorm_rope, kept in fp32 (not rounded to
 * bf16), then block-128 quantized as in inv_rope_fp8_quant with quant_eps as
 * the amax floor; a pad head (n_heads_q <= h < q_head_padded) is a zero head
 * quantized the same way: codes +0, scales quant_eps / 448 (FP32) or the
 * power of two covering it (UE8M0).  With u = t * q_head_padded + h:
 *   q_fp8[u*512 + d]                                   (e4m3 [N, Hpad, 512])
 *   RQ_SCALE_FP32 : ((float*)q_scales)[u*4 + b] = s_b  (fp32 [N, Hpad, 4])
 *   RQ_SCALE_UE8M0: ((uint32_t*)q_scales)[u]           ([N, Hpad], packed as
 *                   in inv_rope_fp8_quant)
 * q_fp8 16-byte aligned; q_scales 4-byte aligned; quant_eps >= 2^-116 as
 * fp32.  A live head whose position is out of range gets NaN scales.  Other
 * arguments as in qnorm_rope.
 */
int qnorm_rope_fp8(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
                   const uint16_t* norm_weight, const int64_t* positions,
                   const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
                   int32_t n_heads_q, int32_t q_head_padded, double eps, int32_t scale_fmt,
                   double quant_eps, uint8_t* q_fp8, void* q_scales, void* stream);

/*
 * kv_rope_quant_insert - forward RoPE and block-128 FP8 quantization of the
 * shared 512-dim kv vector, inserted into a paged uint8 cache through
 * slot_mapping ([P1] section 1: k_cache [num_blocks, block_bytes] uint8,
 * slot_mapping [N] int64, cache_block_size, per-block stride).
 * For t < n_tokens with s = slot_mapping[t] >= 0:
 *   x' = forward RoPE of fp32(kv[t, :]); codes and block scales as in
 *        inv_rope_fp8_quant
 *   record = k_cache + (s / cache_block_size) * block_stride_bytes
 *                    + (s % cache_block_size) * 528
 *   record[0..511]   = the 512 e4m3 codes
 *   RQ_SCALE_FP32 : record[512..527] = s_0..s_3 as little-endian fp32
 *   RQ_SCALE_UE8M0: record[512..515] = exponent bytes k_b + 127 (block b at
 *                   byte 512+b), record[516..527] = 0
 * s < 0 skips the token (padding).  No other byte of k_cache is written.
 * kv: bf16 [N, 512], row stride kv_stride_token (positive multiple of 8),
 *   16-byte aligned.  k_cache: 16-byte aligned; block_stride_bytes a multiple
 *   of 16 and >= cache_block_size * 528; num_blocks * cache_block_size < 2^31.
 *   Slots must be unique (duplicates race).
 */
int kv_rope_quant_insert(const uint16_t* kv, int64_t kv_stride_token,
                         const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                         const int64_t* slot_mapping, int64_t n_tokens,
                         uint8_t* k_cache, int64_t num_blocks, int64_t block_stride_bytes,
                         int32_t cache_block_size, int32_t scale_fmt, double eps,
                         void* stream);

/*
 * kv_rope_insert_full - forward RoPE of kv into a contiguous token-strided
 * bf16 cache ([P1] section 2's full-cache form): for t < n_tokens with
 * s = slot_mapping[t] >= 0,
 *   cache[s * cache_stride_token + d] = bf16_rne(x'_d),  d < 512
 * x' as in kv_rope_quant_insert.  s < 0 skips the token; s >= num_slots is
 * skipped too (caller contract: slots unique and below num_slots).  No other
 * element is written; a token whose position is out of range gets a NaN row.
 * cache: bf16 [num_slots, cache_stride_token], 16-byte aligned;
 *   cache_stride_token >= 512 and a multiple of 8.  kv as in
 *   kv_rope_quant_insert.
 */
int kv_rope_insert_full(const uint16_t* kv, int64_t kv_stride_token,
                        const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                        const int64_t* slot_mapping, int64_t n_tokens, uint16_t* cache,
                        int64_t num_slots, int64_t cache_stride_token, void* stream);

/*
 * qnorm_rope_kv_rope_quant_insert - qnorm_rope and kv_rope_quant_insert in a
 * single launch, the op's own shape in [P1] section 1 (the `_out` form: q_out
 * and k_cache preallocated by the caller, nothing returned; section 2 gives
 * the schema).  Every argument means what it means in the two functions
 * above, the two share positions / cos_sin_cache / n_tokens, and the results
 * are bit-identical to calling both: eps is the RMSNorm epsilon, quant_eps the
 * kv amax floor (>= 2^-116 as fp32).  Validation is the union of both.
 */
int qnorm_rope_kv_rope_quant_insert(
    const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
    const uint16_t* norm_weight, const uint16_t* kv, int64_t kv_stride_token,
    const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
    const int64_t* slot_mapping, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
    double eps, uint16_t* q_out, uint8_t* k_cache, int64_t num_blocks,
    int64_t block_stride_bytes, int32_t cache_block_size, int32_t scale_fmt, double quant_eps,
    void* stream);

/*
 * qnorm_rope_kv_rope_insert_full and qnorm_rope_fp8_kv_rope_insert_full - the
 * full-cache forms of the fused op ([P1] section 2) in one launch: the q path
 * of qnorm_rope (q_out, in place allowed as there) or of qnorm_rope_fp8, and
 * the kv path of kv_rope_insert_full.  Bit-identical to the two separate
 * calls; validation is the union of both.
 */
int qnorm_rope_kv_rope_insert_full(
    const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
    const uint16_t* norm_weight, const uint16_t* kv, int64_t kv_stride_token,
    const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
    const int64_t* slot_mapping, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
    double eps, uint16_t* q_out, uint16_t* cache, int64_t num_slots, int64_t cache_stride_token,
    void* stream);

int qnorm_rope_fp8_kv_rope_insert_full(
    const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
    const uint16_t* norm_weight, const uint16_t* kv, int64_t kv_stride_token,
    const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
    const int64_t* slot_mapping, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
    double eps, int32_t scale_fmt, double quant_eps, uint8_t* q_fp8, void* q_scales,
    uint16_t* cache, int64_t num_slots, int64_t cache_stride_token, void* stream);

/*
 * indexer_q_rope_quant - the sparse-attention indexer's query path ([P5]
 * section 1): rotate-half RoPE, per-head power-of-two FP8 quantization, and
 * the scale folded into the per-head weights.  For t < n_tokens, h < n_heads
 * (128-dim heads):
 *   x   = fp32(q[t, h, :])
 *   for i < 32, c = cos_sin_cache[positions[t], i], s = ... [32 + i]:
 *     y_i = bf16_round(x_i * c - x_{i+32} * s)
 *     y_{i+32} = bf16_round(x_{i+32} * c + x_i * s)
 *   y_d = x_d for d = 64..127; bf16_round = round to bf16 (RNE) and back
 *   m   = max(max_d |y_d|, eps);  k = smallest integer with 2^k >= m / 448
 *   q_fp8[t, h, :]     = e4m3_rne(y * 2^-k)
 *   weights_out[t, h]  = ((weights[t, h] * 2^k) * softmax_scale) * head_scale
 * q: bf16 [N, H, 128], strides (q_stride_token, q_stride_head, 1), base
 *   16-byte aligned, strides multiples of 8.  weights / weights_out: fp32
 *   [N, H] with token strides w_stride_token / wo_stride_token (heads
 *   contiguous); weights_out may be weights itself (in place).  q_fp8: e4m3
 *   [N, H, 128] with byte strides (out_stride_token, out_stride_head), 8-byte
 *   aligned, multiples of 8, rows not overlapping.  softmax_scale, head_scale
 *   finite (as fp32); eps >= 2^-116 as fp32.  n_tokens * n_heads < 2^31;
 *   q_stride_head <= 2^28 and out_stride_head <= 2^30 (RQ_ERR_STRIDE
 *   otherwise).  A head whose position is out of range gets a NaN weight.
 */
int indexer_q_rope_quant(const uint16_t* q, int64_t q_stride_token, int64_t q_stride_head,
                         const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                         const float* weights, int64_t w_stride_token, int64_t n_tokens,
                         int32_t n_heads, double softmax_scale, double head_scale, double eps,
                         uint8_t* q_fp8, int64_t out_stride_token, int64_t out_stride_head,
                         float* weights_out, int64_t wo_stride_token, void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* ropequant_strerror(int status);

/* ROPEQUANT_ABI_VERSION of the loaded library. */
int ropequant_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ROPEQUANT_H */

/*
 * CPU oracle for the fused RoPE + block-FP8 hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, single-threaded
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the HIP library, and it never
 * reads anything the GPU produced.
 *
 * Sources (web pages; cited by title and section, never by line):
 *   [P1] "vLLM DeepSeek-V4 성능 최적화: Eager Break 시 Workspace 재사용 개선"
 *        (analysis of vLLM PR #49236) - sections 1 (the _out op and its
 *        argument checks) and 2 (the op schema, and the full-cache variants
 *        named beside it).
 *   [P3] "vLLM, DeepSeek V4 모델의 저지연을 위한 RMSNorm과 라우터 GEMV 연산
 *        융합으로 성능 극대화" (analysis of vLLM PR #41263) - section 5 (the
 *        RMSNorm formula).
 *   [P4] "한 프로그램이 4개 head를 처리하게 하라: DeepSeek-V4 inverse RoPE +
 *        FP8 quant 커널 3.5배 가속기" (analysis of vLLM PR #63540) - intro,
 *        section 1 (BLOCK_H and group addressing), section 2 (the register
 *        partner swap and the rotation formulas), section 3 (block amax,
 *        UE8M0 packing), section 4 (the kernel's compile keys, `quantize`
 *        among them).
 *   [P5] "vLLM의 GLM5.2 성능 최적화: Triton 커널 융합을 통한 E2E Throughput
 *        향상" (analysis of vLLM PR #46862) - section 1 (power-of-two scale).
 *
 * Arithmetic model: every floating-point step is one IEEE-754 binary32 basic
 * operation, round-to-nearest-even, with no fused multiply-add (the file is
 * compiled with -ffp-contract=off and without -march flags, so x86-64 SSE2
 * arithmetic is exact binary32).  Readings of points the pages leave open are
 * stated where they are used.
 *
 * Parity pins: every function here is pinned by the CPU test suite against
 * library routines (torch's bfloat16 / float8_e4m3fn casts), brute force,
 * fp64 closed forms and exact special cases.  None is "parity unpinned".
 */
/* no FMA contraction: the build passes -ffp-contract=off */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HEAD_DIM 512   /* [P4] intro: 512-dim heads */
#define NOPE_DIM 448   /* [P4] section 2: NoPE pairs pass through */
#define ROPE_DIM 64    /* last 64 dims are rotated */
#define HALF_ROPE 32   /* cos in columns 0..31, sin in 32..63 of a cache row */
#define QBLOCK 128     /* [P4] section 3: block of 128 elements per scale */
#define NBLOCK 4       /* blocks per head */
#define E4M3_MAX 448.0f
#define RECORD_BYTES 528 /* one cache slot: 512 codes + 16 bytes of scale */

/* status codes: same numeric meaning as the library's, defined here anew */
enum { ORC_OK = 0, ORC_ERR_NULL = -1, ORC_ERR_SHAPE = -2, ORC_ERR_STRIDE = -3,
       ORC_ERR_ALIGN = -4, ORC_ERR_VALUE = -5 };
enum { ORC_SCALE_FP32 = 0, ORC_SCALE_UE8M0 = 1 };

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ---------------------------------------------------------------- codecs */

/* bf16 -> fp32 is exact: the 16 bits are the top half of the fp32 word. */
float orc_bf16_to_f32(uint16_t h) { return float_of((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even (finite inputs).  Keep the top
 * 16 bits; the dropped 16 bits decide: above half rounds up, exactly half
 * rounds up only when the kept part is odd.  A carry out of the mantissa
 * correctly moves to the next binade. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u = bits_of(f);
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xFFFFu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

/* OCP 8-bit E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (M/8 * 2^-6); S.1111.111 is NaN; no
 * infinities.  Largest finite magnitude 1.75 * 2^8 = 448. */
float orc_e4m3_to_f32(uint8_t c) {
  int sign = c >> 7;
  int e = (c >> 3) & 15;
  int m = c & 7;
  float mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) mag = ldexpf((float)m, -9);            /* m/8 * 2^-6 */
  else mag = ldexpf((float)(8 + m), e - 7 - 3);      /* (1+m/8) * 2^(e-7) */
  return sign ? -mag : mag;
}

/* fp32 -> e4m3, round to nearest, ties to even mantissa.  Domain: finite
 * |v| <= 448 (callers clamp first), and NaN, which takes the format's NaN
 * code with its sign (S.1111.111).  The sign is kept for zero and for values
 * that round to zero.
 *
 * Method, straight from the format: find the spacing q of e4m3 values in the
 * binade of |v| (2^-9 below the smallest normal 2^-6, else 2^(e-3) for
 * 2^e <= |v| < 2^(e+1)); n = |v|/q is exact (power-of-two scaling); round n
 * to an integer, ties to even; rebuild the fields, carrying into the next
 * binade when n reaches 16 (or reaching the smallest normal when a subnormal
 * rounds up to 8). */
uint8_t orc_f32_to_e4m3(float v) {
  uint32_t sign = bits_of(v) >> 31;
  float a = fabsf(v);
  int e, subnormal;
  float n, fl, frac;
  uint32_t code;
  if (a != a) return (uint8_t)((sign << 7) | 0x7Fu);
  if (a == 0.0f) return (uint8_t)(sign << 7);
  if (a < ldexpf(1.0f, -6)) {
    subnormal = 1;
    e = -6;
    n = ldexpf(a, 9);
  } else {
    subnormal = 0;
    e = (int)((bits_of(a) >> 23) & 0xFF) - 127; /* a >= 2^-6 is an fp32 normal */
    n = ldexpf(a, 3 - e);                        /* in [8, 16) */
  }
  fl = floorf(n);
  frac = n - fl; /* exact: the fraction bits of n */
  if (frac > 0.5f || (frac == 0.5f && fmodf(fl, 2.0f) == 1.0f)) fl += 1.0f;
  if (subnormal) {
    if (fl >= 8.0f) code = 1u << 3;              /* 2^-6, the smallest normal */
    else code = (uint32_t)fl;                    /* exponent field 0 */
  } else {
    if (fl >= 16.0f) { fl = 8.0f; e += 1; }
    code = ((uint32_t)(e + 7) << 3) | ((uint32_t)fl - 8u);
  }
  return (uint8_t)((sign << 7) | code);
}

/* Smallest integer k with 2^k >= t, for finite t > 0 that is an fp32 normal.
 * Exact: the fp32 exponent of t, plus one when any mantissa bit is set.  (The
 * fp32 log2 route can round a value just above 2^k down to k.) */
int orc_pow2_ceil_exp(float t) {
  uint32_t u = bits_of(t);
  int k = (int)((u >> 23) & 0xFF) - 127;
  if (u & 0x7FFFFFu) k += 1;
  return k;
}

/* ------------------------------------------------------------ RoPE steps */

/* GPT-J interleaved RoPE on the last 64 dims of one 512-dim head.
 * Pairs (2k, 2k+1) for k = 224..255 rotate with c = row[k-224] and
 * s = row[32 + k-224]; pairs below 224 are copied unchanged.
 *   inverse ([P4] section 2, rotation by -theta):
 *     e' = e*c + o*s,  o' = o*c - e*s
 *   forward (rotation by +theta; its inverse is the above):
 *     e' = e*c - o*s,  o' = o*c + e*s
 * Each product is rounded, then the sum or difference is rounded. */
void orc_rope_head(const float* x, float* y, const float* cs_row, int inverse) {
  int k;
  for (k = 0; k < HEAD_DIM; ++k) y[k] = x[k];
  for (k = NOPE_DIM / 2; k < HEAD_DIM / 2; ++k) {
    float c = cs_row[k - NOPE_DIM / 2];
    float s = cs_row[HALF_ROPE + k - NOPE_DIM / 2];
    float e = x[2 * k], o = x[2 * k + 1];
    float ec = e * c, os = o * s, oc = o * c, es = e * s;
    if (inverse) {
      y[2 * k] = ec + os;
      y[2 * k + 1] = oc - es;
    } else {
      y[2 * k] = ec - os;
      y[2 * k + 1] = oc + es;
    }
  }
}

/* ------------------------------------------------------- block FP8 quant */

/* Quantize one 512-dim fp32 head in four blocks of 128 ([P4] section 3).
 *   m_b = max(max_i |x_i|, eps)
 *   FP32 scale:  s_b = m_b / 448;  inv = 1 / s_b;  v = x * inv
 *   UE8M0 scale: t = m_b / 448;  k = ceil(log2 t) exactly;  s_b = 2^k;
 *                v = x * 2^-k (exact)                 ([P4] section 3, [P5])
 *   v is clamped to [-448, 448], then encoded e4m3 RNE.
 * A block whose values overflowed fp32 (amax = +inf) follows the same
 * formulas in IEEE arithmetic: FP32 s = +inf and inv = 0; UE8M0 k = 128,
 * s = +inf, 2^-k = 2^-128 and exponent byte 0xFF.
 * Reading: the quotient x / s is taken as x * (1/s) with 1/s rounded once
 * per block; the pages do not show which form the kernel uses.
 * Outputs: codes[512]; scales_f32[4] (FP32 mode: s_b; UE8M0 mode: 2^k);
 * *ue8m0_word = exponent bytes k_b + 127, block b in byte b (UE8M0 mode). */
void orc_quant_head(const float* x, int scale_fmt, float eps, uint8_t* codes,
                    float* scales_f32, uint32_t* ue8m0_word) {
  int b, i;
  uint32_t word = 0;
  for (b = 0; b < NBLOCK; ++b) {
    const float* xb = x + b * QBLOCK;
    float m = 0.0f, mult, s;
    for (i = 0; i < QBLOCK; ++i) {
      float a = fabsf(xb[i]);
      if (a > m) m = a;
    }
    if (eps > m) m = eps;
    if (scale_fmt == ORC_SCALE_UE8M0) {
      float t = m / E4M3_MAX;
      int k = orc_pow2_ceil_exp(t);
      s = ldexpf(1.0f, k);
      mult = ldexpf(1.0f, -k);
      word |= (uint32_t)(k + 127) << (8 * b);
    } else {
      s = m / E4M3_MAX;
      mult = 1.0f / s;
    }
    if (scales_f32) scales_f32[b] = s;
    for (i = 0; i < QBLOCK; ++i) {
      float v = xb[i] * mult;
      if (v > E4M3_MAX) v = E4M3_MAX;
      if (v < -E4M3_MAX) v = -E4M3_MAX;
      codes[b * QBLOCK + i] = orc_f32_to_e4m3(v);
    }
  }
  if (ue8m0_word) *ue8m0_word = word;
}

/* ------------------------------------------------------------- RMSNorm */

/* Per-head RMSNorm over the 512 dims ([P3] section 5 formula:
 * y = x * rsqrt(mean(x^2) + eps) * w), read plainly in fp32:
 *   ss = x_0^2 + x_1^2 + ... + x_511^2, added left to right in index order,
 *        each square and each sum rounded;
 *   mean = ss / 512 (exact: a power of two);
 *   r = 1 / sqrt(mean + eps)  (correctly rounded sqrt, then divide);
 *   y_d = (x_d * r) * w_d, or x_d * r when there is no weight.
 * The pages fix no summation order; index order is the plain reading of
 * "mean(x^2)".  orc_rmsnorm_head_pairwise below differs only in that order. */
static void rms_apply(const float* x, const uint16_t* weight, float eps, float ss, float* y) {
  int d;
  float mean = ss / 512.0f;
  float r = 1.0f / sqrtf(mean + eps);
  for (d = 0; d < HEAD_DIM; ++d) {
    float v = x[d] * r;
    y[d] = weight ? v * orc_bf16_to_f32(weight[d]) : v;
  }
}

/* x_0^2 + x_1^2 + ... + x_{n-1}^2, added left to right */
static float sum_squares_index(const float* x, int n) {
  int d;
  float ss = x[0] * x[0];
  for (d = 1; d < n; ++d) ss = ss + x[d] * x[d];
  return ss;
}

void orc_rmsnorm_head(const float* x, const uint16_t* weight, float eps, float* y) {
  rms_apply(x, weight, eps, sum_squares_index(x, HEAD_DIM), y);
}

/* Sum of x_i^2 over [0, n) by pairwise summation: the sums of the two
 * halves [0, n/2) and [n/2, n), each found the same way, added; one term is
 * its square.  Every square and every sum is one fp32 rounding.  (The
 * recursive pairwise order analysed in N. J. Higham, "The accuracy of
 * floating point summation", SIAM J. Sci. Comput. 14(4), 1993.) */
static float sum_squares_pairwise(const float* x, int n) {
  if (n == 1) return x[0] * x[0];
  return sum_squares_pairwise(x, n / 2) + sum_squares_pairwise(x + n / 2, n - n / 2);
}

/* The same RMSNorm with the squares added by pairwise summation over the 512
 * dims.  Not the definition's order: a second standard rounding order of the
 * same sum, for tests that separate the summation order from every other
 * step. */
void orc_rmsnorm_head_pairwise(const float* x, const uint16_t* weight, float eps, float* y) {
  rms_apply(x, weight, eps, sum_squares_pairwise(x, HEAD_DIM), y);
}

/* sum_order argument of the q-path ops: ORC_SUM_INDEX is the definition */
enum { ORC_SUM_INDEX = 0, ORC_SUM_PAIRWISE = 1 };

/* The sum of squares RMSNorm uses, over n >= 1 values, in sum_order
 * (exported so that tests can pin each order's sums themselves: a change of
 * a few units in a sum near 2^24 can vanish in the rounded 1 / sqrt). */
float orc_sum_squares(const float* x, int32_t n, int32_t sum_order) {
  if (n < 1) return 0.0f;
  return sum_order == ORC_SUM_PAIRWISE ? sum_squares_pairwise(x, n) : sum_squares_index(x, n);
}

static void rmsnorm_by_order(const float* x, const uint16_t* weight, float eps, int32_t order,
                             float* y) {
  if (order == ORC_SUM_PAIRWISE) orc_rmsnorm_head_pairwise(x, weight, eps, y);
  else orc_rmsnorm_head(x, weight, eps, y);
}

/* ------------------------------------------------------ shared validation */

static int eps_ok(double eps) {
  float e = (float)eps;
  /* finite, and eps/448 must stay an fp32 normal so 1/s is finite */
  return isfinite(eps) && e >= ldexpf(1.0f, -116) && isfinite(e);
}

static int load_head(const uint16_t* src, float* x) {
  int d;
  for (d = 0; d < HEAD_DIM; ++d) x[d] = orc_bf16_to_f32(src[d]);
  return 0;
}

/* ------------------------------------------------- inv_rope_fp8_quant */

/* Attention output o[N, H, 512] bf16 -> inverse RoPE -> block FP8.
 * [P4] intro (the op before the wo_a projection), sections 1-3.
 * Output layout (reading of [P4] section 1, where a program's heads must share
 * one wo_a group and the scale column is head_in_group * 4 + block):
 *   codes  out[g*out_stride_group + t*out_stride_token + j*512 + d]   (bytes)
 *   FP32   scales[g*sg + t*st + (j*4 + b)*sb]                       (floats)
 *   UE8M0  scales[g*sg + t*st + j*sb]                        (uint32 words)
 * with g = h / heads_per_group, j = h % heads_per_group. */
int orc_inv_rope_fp8_quant(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                           const int64_t* positions, const float* cos_sin_cache,
                           int64_t max_pos, int64_t n_tokens, int32_t n_heads,
                           int32_t heads_per_group, int32_t scale_fmt, double eps,
                           uint8_t* out, int64_t out_stride_group, int64_t out_stride_token,
                           void* scales, int64_t sc_stride_group, int64_t sc_stride_token,
                           int64_t sc_stride_block) {
  int64_t t;
  int32_t h;
  float x[HEAD_DIM], y[HEAD_DIM], sf[NBLOCK];
  uint8_t codes[HEAD_DIM];
  uint32_t word;
  float epsf = (float)eps;
  if (n_tokens < 0 || n_heads <= 0 || heads_per_group <= 0 || max_pos <= 0) return ORC_ERR_SHAPE;
  if (n_heads % heads_per_group) return ORC_ERR_SHAPE;
  if (scale_fmt != ORC_SCALE_FP32 && scale_fmt != ORC_SCALE_UE8M0) return ORC_ERR_VALUE;
  if (!eps_ok(eps)) return ORC_ERR_VALUE;
  if (n_tokens == 0) return ORC_OK;
  if (!o || !positions || !cos_sin_cache || !out || !scales) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t)
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
  for (t = 0; t < n_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * ROPE_DIM;
    for (h = 0; h < n_heads; ++h) {
      int64_t g = h / heads_per_group, j = h % heads_per_group;
      int b, d;
      load_head(o + t * o_stride_token + (int64_t)h * o_stride_head, x);
      orc_rope_head(x, y, row, 1);
      orc_quant_head(y, scale_fmt, epsf, codes, sf, &word);
      for (d = 0; d < HEAD_DIM; ++d)
        out[g * out_stride_group + t * out_stride_token + j * HEAD_DIM + d] = codes[d];
      if (scale_fmt == ORC_SCALE_UE8M0) {
        uint32_t* sc = (uint32_t*)scales;
        sc[g * sc_stride_group + t * sc_stride_token + j * sc_stride_block] = word;
      } else {
        float* sc = (float*)scales;
        for (b = 0; b < NBLOCK; ++b)
          sc[g * sc_stride_group + t * sc_stride_token + (j * NBLOCK + b) * sc_stride_block] = sf[b];
      }
    }
  }
  return ORC_OK;
}

/* ----------------------------------------------------- inv_rope_bf16 */

/* The inverse RoPE alone, bf16 out: the IRQ kernel with its quantization
 * switched off ([P4] section 4 lists `quantize` as a compile-time key of the
 * kernel).  Reading: the same fp32 rotation as above, then one bf16 RNE
 * rounding per element (so the 448 pass-through dims come out as bit copies),
 * stored with the group addressing of the codes above, in elements:
 *   out[g*out_stride_group + t*out_stride_token + j*512 + d]. */
int orc_inv_rope_bf16(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                      const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                      int64_t n_tokens, int32_t n_heads, int32_t heads_per_group,
                      uint16_t* out, int64_t out_stride_group, int64_t out_stride_token) {
  int64_t t;
  int32_t h;
  float x[HEAD_DIM], y[HEAD_DIM];
  if (n_tokens < 0 || n_heads <= 0 || heads_per_group <= 0 || max_pos <= 0) return ORC_ERR_SHAPE;
  if (n_heads % heads_per_group) return ORC_ERR_SHAPE;
  if (n_tokens == 0) return ORC_OK;
  if (!o || !positions || !cos_sin_cache || !out) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t)
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
  for (t = 0; t < n_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * ROPE_DIM;
    for (h = 0; h < n_heads; ++h) {
      int64_t g = h / heads_per_group, j = h % heads_per_group;
      uint16_t* dst = out + g * out_stride_group + t * out_stride_token + j * HEAD_DIM;
      int d;
      load_head(o + t * o_stride_token + (int64_t)h * o_stride_head, x);
      orc_rope_head(x, y, row, 1);
      for (d = 0; d < HEAD_DIM; ++d) dst[d] = orc_f32_to_bf16(y[d]);
    }
  }
  return ORC_OK;
}

/* ---------------------------------------------------------- qnorm_rope */

/* q_in[N, Hq, 512] bf16 -> per-head RMSNorm -> forward RoPE -> bf16 RNE into
 * q_out[N, Hpad, 512] (contiguous); heads Hq..Hpad-1 are written as +0.
 * [P1] section 1 (q_out preallocated, every element written, pad zeroed,
 * q_head_padded >= num_heads_q); [P3] section 5 (RMSNorm).
 * Reading: fp32 throughout, one bf16 rounding at the end.
 * sum_order: ORC_SUM_INDEX (the RMSNorm definition) or ORC_SUM_PAIRWISE. */
int orc_qnorm_rope(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
                   const uint16_t* norm_weight, const int64_t* positions,
                   const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
                   int32_t n_heads_q, int32_t q_head_padded, double eps, uint16_t* q_out,
                   int32_t sum_order) {
  int64_t t;
  int32_t h;
  int d;
  float x[HEAD_DIM], y[HEAD_DIM], z[HEAD_DIM];
  float epsf = (float)eps;
  if (n_tokens < 0 || n_heads_q <= 0 || max_pos <= 0) return ORC_ERR_SHAPE;
  if (q_head_padded < n_heads_q) return ORC_ERR_SHAPE;
  if (!(eps > 0.0) || !isfinite(eps) || !(epsf > 0.0f)) return ORC_ERR_VALUE;
  if (sum_order != ORC_SUM_INDEX && sum_order != ORC_SUM_PAIRWISE) return ORC_ERR_VALUE;
  if (n_tokens == 0) return ORC_OK;
  if (!q_in || !positions || !cos_sin_cache || !q_out) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t)
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
  for (t = 0; t < n_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * ROPE_DIM;
    for (h = 0; h < q_head_padded; ++h) {
      uint16_t* dst = q_out + (t * q_head_padded + h) * HEAD_DIM;
      if (h >= n_heads_q) {
        for (d = 0; d < HEAD_DIM; ++d) dst[d] = 0;
        continue;
      }
      load_head(q_in + t * q_stride_token + (int64_t)h * q_stride_head, x);
      rmsnorm_by_order(x, norm_weight, epsf, sum_order, y);
      orc_rope_head(y, z, row, 0);
      for (d = 0; d < HEAD_DIM; ++d) dst[d] = orc_f32_to_bf16(z[d]);
    }
  }
  return ORC_OK;
}

/* The fp32 values the q paths round: RMSNorm (squares added in sum_order)
 * then forward RoPE, exactly as orc_qnorm_rope computes them before its bf16
 * rounding and orc_qnorm_rope_fp8 before its quantization; live heads only,
 * z[(t*Hq + h)*512 + d].  Tests use them to tell where a rounding decision
 * sits close to its boundary. */
int orc_qnorm_rope_f32(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
                       const uint16_t* norm_weight, const int64_t* positions,
                       const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
                       int32_t n_heads_q, double eps, float* z_out, int32_t sum_order) {
  int64_t t;
  int32_t h;
  float x[HEAD_DIM], y[HEAD_DIM];
  float epsf = (float)eps;
  if (n_tokens < 0 || n_heads_q <= 0 || max_pos <= 0) return ORC_ERR_SHAPE;
  if (!(eps > 0.0) || !isfinite(eps) || !(epsf > 0.0f)) return ORC_ERR_VALUE;
  if (sum_order != ORC_SUM_INDEX && sum_order != ORC_SUM_PAIRWISE) return ORC_ERR_VALUE;
  if (n_tokens == 0) return ORC_OK;
  if (!q_in || !positions || !cos_sin_cache || !z_out) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t)
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
  for (t = 0; t < n_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * ROPE_DIM;
    for (h = 0; h < n_heads_q; ++h) {
      load_head(q_in + t * q_stride_token + (int64_t)h * q_stride_head, x);
      rmsnorm_by_order(x, norm_weight, epsf, sum_order, y);
      orc_rope_head(y, z_out + (t * n_heads_q + h) * HEAD_DIM, row, 0);
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------ qnorm_rope_fp8 */

/* The q path into a separate FP8 tensor, one of the full-cache variants named
 * beside the op schema in [P1] section 2.  Readings (the pages give only the
 * variant's name): RMSNorm (its squares added in sum_order) and forward RoPE
 * exactly as in orc_qnorm_rope, in fp32; the fp32 head (not its bf16 rounding: the same fusion as the kv path)
 * goes through orc_quant_head; a pad head h in [Hq, Hpad) is a zero head
 * quantized the same way (codes +0, scales from eps).  Layout:
 *   codes   q_fp8[(t*Hpad + h)*512 + d]                          (bytes)
 *   FP32    q_scales[(t*Hpad + h)*4 + b]                         (floats)
 *   UE8M0   q_scales[t*Hpad + h]                          (uint32 words) */
int orc_qnorm_rope_fp8(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
                       const uint16_t* norm_weight, const int64_t* positions,
                       const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
                       int32_t n_heads_q, int32_t q_head_padded, double eps, int32_t scale_fmt,
                       double quant_eps, uint8_t* q_fp8, void* q_scales, int32_t sum_order) {
  int64_t t;
  int32_t h;
  int b;
  float x[HEAD_DIM], y[HEAD_DIM], z[HEAD_DIM], sf[NBLOCK];
  uint32_t word;
  float epsf = (float)eps, qepsf = (float)quant_eps;
  if (n_tokens < 0 || n_heads_q <= 0 || max_pos <= 0) return ORC_ERR_SHAPE;
  if (q_head_padded < n_heads_q) return ORC_ERR_SHAPE;
  if (!(eps > 0.0) || !isfinite(eps) || !(epsf > 0.0f)) return ORC_ERR_VALUE;
  if (scale_fmt != ORC_SCALE_FP32 && scale_fmt != ORC_SCALE_UE8M0) return ORC_ERR_VALUE;
  if (!eps_ok(quant_eps)) return ORC_ERR_VALUE;
  if (sum_order != ORC_SUM_INDEX && sum_order != ORC_SUM_PAIRWISE) return ORC_ERR_VALUE;
  if (n_tokens == 0) return ORC_OK;
  if (!q_in || !positions || !cos_sin_cache || !q_fp8 || !q_scales) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t)
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
  for (t = 0; t < n_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * ROPE_DIM;
    for (h = 0; h < q_head_padded; ++h) {
      int64_t u = t * q_head_padded + h;
      if (h < n_heads_q) {
        load_head(q_in + t * q_stride_token + (int64_t)h * q_stride_head, x);
        rmsnorm_by_order(x, norm_weight, epsf, sum_order, y);
        orc_rope_head(y, z, row, 0);
      } else {
        memset(z, 0, sizeof z);
      }
      orc_quant_head(z, scale_fmt, qepsf, q_fp8 + u * HEAD_DIM, sf, &word);
      if (scale_fmt == ORC_SCALE_UE8M0)
        ((uint32_t*)q_scales)[u] = word;
      else
        for (b = 0; b < NBLOCK; ++b) ((float*)q_scales)[u * NBLOCK + b] = sf[b];
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------- kv_rope_quant_insert */

/* kv[N, 512] bf16 -> forward RoPE -> block FP8 -> one 528-byte record in the
 * paged uint8 cache ([P1] section 1: k_cache [num_blocks, block_bytes] uint8,
 * slot_mapping [N] int64, cache_block_size, block stride).
 * Reading of the unprinted record layout: bytes 0..511 are the e4m3 codes;
 * bytes 512..527 hold the four block scales - FP32 mode: four little-endian
 * fp32 s_b; UE8M0 mode: the packed exponent word in bytes 512..515 and zeros
 * in 516..527.  Slot s maps to block s / bs, index s % bs, at byte offset
 * block*block_stride + index*528.  s < 0 means "skip this token".  Slots must
 * be unique (checked here).  No other byte is written. */
int orc_kv_rope_quant_insert(const uint16_t* kv, int64_t kv_stride_token,
                             const int64_t* positions, const float* cos_sin_cache,
                             int64_t max_pos, const int64_t* slot_mapping, int64_t n_tokens,
                             uint8_t* k_cache, int64_t num_blocks, int64_t block_stride_bytes,
                             int32_t cache_block_size, int32_t scale_fmt, double eps) {
  int64_t t, u;
  int b;
  float x[HEAD_DIM], y[HEAD_DIM], sf[NBLOCK];
  uint8_t codes[HEAD_DIM];
  uint32_t word;
  float epsf = (float)eps;
  if (n_tokens < 0 || max_pos <= 0 || num_blocks <= 0 || cache_block_size <= 0) return ORC_ERR_SHAPE;
  if (block_stride_bytes < (int64_t)cache_block_size * RECORD_BYTES) return ORC_ERR_STRIDE;
  if (scale_fmt != ORC_SCALE_FP32 && scale_fmt != ORC_SCALE_UE8M0) return ORC_ERR_VALUE;
  if (!eps_ok(eps)) return ORC_ERR_VALUE;
  if (n_tokens == 0) return ORC_OK;
  if (!kv || !positions || !cos_sin_cache || !slot_mapping || !k_cache) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t) {
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
    if (slot_mapping[t] >= num_blocks * (int64_t)cache_block_size) return ORC_ERR_VALUE;
    if (slot_mapping[t] >= 0)
      for (u = 0; u < t; ++u)
        if (slot_mapping[u] == slot_mapping[t]) return ORC_ERR_VALUE;
  }
  for (t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    uint8_t* rec;
    if (s < 0) continue;
    load_head(kv + t * kv_stride_token, x);
    orc_rope_head(x, y, cos_sin_cache + positions[t] * ROPE_DIM, 0);
    orc_quant_head(y, scale_fmt, epsf, codes, sf, &word);
    rec = k_cache + (s / cache_block_size) * block_stride_bytes +
          (s % cache_block_size) * RECORD_BYTES;
    memcpy(rec, codes, HEAD_DIM);
    if (scale_fmt == ORC_SCALE_UE8M0) {
      uint8_t tail[16] = {0};
      for (b = 0; b < 4; ++b) tail[b] = (uint8_t)(word >> (8 * b));
      memcpy(rec + HEAD_DIM, tail, 16);
    } else {
      for (b = 0; b < NBLOCK; ++b) memcpy(rec + HEAD_DIM + 4 * b, &sf[b], 4);
    }
  }
  return ORC_OK;
}

/* --------------------------------------------------- kv_rope_insert_full */

/* The kv path into a contiguous, token-strided cache, the other full-cache
 * variant named beside the op schema in [P1] section 2.  Readings (the pages
 * give only "512 wide" and "token strided"): the cache holds bf16 rows of 512
 * (no quantization, hence no scales), slot s owns the row at
 * cache + s*cache_stride_token (elements); forward RoPE as in
 * orc_kv_rope_quant_insert, then one bf16 RNE rounding.  s < 0 skips the
 * token; s >= num_slots and repeated slots are rejected; nothing else is
 * written. */
int orc_kv_rope_insert_full(const uint16_t* kv, int64_t kv_stride_token,
                            const int64_t* positions, const float* cos_sin_cache,
                            int64_t max_pos, const int64_t* slot_mapping, int64_t n_tokens,
                            uint16_t* cache, int64_t num_slots, int64_t cache_stride_token) {
  int64_t t, u;
  int d;
  float x[HEAD_DIM], y[HEAD_DIM];
  if (n_tokens < 0 || max_pos <= 0 || num_slots <= 0) return ORC_ERR_SHAPE;
  if (cache_stride_token < HEAD_DIM) return ORC_ERR_STRIDE;
  if (n_tokens == 0) return ORC_OK;
  if (!kv || !positions || !cos_sin_cache || !slot_mapping || !cache) return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t) {
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
    if (slot_mapping[t] >= num_slots) return ORC_ERR_VALUE;
    if (slot_mapping[t] >= 0)
      for (u = 0; u < t; ++u)
        if (slot_mapping[u] == slot_mapping[t]) return ORC_ERR_VALUE;
  }
  for (t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    load_head(kv + t * kv_stride_token, x);
    orc_rope_head(x, y, cos_sin_cache + positions[t] * ROPE_DIM, 0);
    for (d = 0; d < HEAD_DIM; ++d) cache[s * cache_stride_token + d] = orc_f32_to_bf16(y[d]);
  }
  return ORC_OK;
}

/* ------------------------------------------------ bulk codec entry points */
/* Array forms of the codecs above, for the codec pins (one call per array
 * instead of one per element). */
void orc_f32_to_e4m3_n(const float* v, uint8_t* c, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) c[i] = orc_f32_to_e4m3(v[i]);
}
void orc_f32_to_bf16_n(const float* v, uint16_t* h, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) h[i] = orc_f32_to_bf16(v[i]);
}
void orc_bf16_to_f32_n(const uint16_t* h, float* v, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) v[i] = orc_bf16_to_f32(h[i]);
}
void orc_pow2_ceil_exp_n(const float* t, int32_t* k, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) k[i] = orc_pow2_ceil_exp(t[i]);
}

/* ------------------------------------------------ indexer_q_rope_quant */

/* One 128-dim indexer query head ([P5] section 1):
 *   dims 0..63 get rotate-half ("NeoX") RoPE with pairs (i, i+32), i < 32,
 *   c = row[i], s = row[32+i]:
 *     r0 = x_i * c - x_{i+32} * s,   r1 = x_{i+32} * c + x_i * s
 *   and each rotated value is rounded to bf16 and back (as printed on the
 *   page for r0; r1 by the same rule); dims 64..127 pass through.
 *   m = max(max |y|, eps); t = m / 448; q_scale = 2^k with k the exact
 *   ceiling of log2 t ([P5] section 1: exp2(ceil(log2(amax / 448))));
 *   codes = e4m3_rne(clamp(y * 2^-k, +-448)) (the scaling is exact);
 *   w_out = ((w * q_scale) * softmax_scale) * head_scale, left to right as
 *   printed.  Readings: eps is an argument (the page reports a 1e-4 vs 1e-10
 *   discussion); head_scale, undefined on the page, is an argument. */
void orc_indexer_rope(const float* x, const float* cs_row, float* y) {
  int i;
  for (i = 0; i < 128; ++i) y[i] = x[i];
  for (i = 0; i < 32; ++i) {
    float c = cs_row[i], s = cs_row[32 + i];
    float x0 = x[i], x1 = x[i + 32];
    float a = x0 * c, b = x1 * s, d = x1 * c, e = x0 * s;
    y[i] = orc_bf16_to_f32(orc_f32_to_bf16(a - b));
    y[i + 32] = orc_bf16_to_f32(orc_f32_to_bf16(d + e));
  }
}

void orc_indexer_head(const float* x, const float* cs_row, float eps, float softmax_scale,
                      float head_scale, float w, uint8_t* codes, float* w_out, float* q_scale) {
  float y[128];
  float m = 0.0f;
  int i, k;
  orc_indexer_rope(x, cs_row, y);
  for (i = 0; i < 128; ++i) {
    float av = fabsf(y[i]);
    if (av > m) m = av;
  }
  if (eps > m) m = eps;
  k = orc_pow2_ceil_exp(m / E4M3_MAX);
  for (i = 0; i < 128; ++i) {
    float v = y[i] * ldexpf(1.0f, -k);
    if (v > E4M3_MAX) v = E4M3_MAX;
    if (v < -E4M3_MAX) v = -E4M3_MAX;
    codes[i] = orc_f32_to_e4m3(v);
  }
  *q_scale = ldexpf(1.0f, k);
  *w_out = ((w * *q_scale) * softmax_scale) * head_scale;
}

/* q[N, H, 128] bf16 -> q_fp8[N, H, 128] e4m3 (+ folded weights [N, H] fp32).
 * Strides: q in elements (token, head); q_fp8 in bytes (token, head); weights
 * and weights_out in elements per token (heads contiguous). */
int orc_indexer_q_rope_quant(const uint16_t* q, int64_t q_stride_token, int64_t q_stride_head,
                             const int64_t* positions, const float* cos_sin_cache,
                             int64_t max_pos, const float* weights, int64_t w_stride_token,
                             int64_t n_tokens, int32_t n_heads, double softmax_scale,
                             double head_scale, double eps, uint8_t* q_fp8,
                             int64_t out_stride_token, int64_t out_stride_head,
                             float* weights_out, int64_t wo_stride_token) {
  int64_t t;
  int32_t h;
  int d;
  float x[128], qs;
  if (n_tokens < 0 || n_heads <= 0 || max_pos <= 0) return ORC_ERR_SHAPE;
  if (!eps_ok(eps) || !isfinite(softmax_scale) || !isfinite(head_scale)) return ORC_ERR_VALUE;
  if (n_tokens == 0) return ORC_OK;
  if (!q || !positions || !cos_sin_cache || !weights || !q_fp8 || !weights_out)
    return ORC_ERR_NULL;
  for (t = 0; t < n_tokens; ++t)
    if (positions[t] < 0 || positions[t] >= max_pos) return ORC_ERR_VALUE;
  for (t = 0; t < n_tokens; ++t) {
    const float* row = cos_sin_cache + positions[t] * ROPE_DIM;
    for (h = 0; h < n_heads; ++h) {
      const uint16_t* src = q + t * q_stride_token + (int64_t)h * q_stride_head;
      for (d = 0; d < 128; ++d) x[d] = orc_bf16_to_f32(src[d]);
      orc_indexer_head(x, row, (float)eps, (float)softmax_scale, (float)head_scale,
                       weights[t * w_stride_token + h],
                       q_fp8 + t * out_stride_token + (int64_t)h * out_stride_head,
                       &weights_out[t * wo_stride_token + h], &qs);
    }
  }
  return ORC_OK;
}

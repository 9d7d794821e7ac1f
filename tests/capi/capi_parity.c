/*
 * The C ABI used from plain C: HIP runtime allocations, a stream of the
 * program's own, no Python and no torch.  Runs inv_rope_fp8_quant (both
 * scale formats), qnorm_rope and kv_rope_quant_insert through
 * libropequant.so on small ragged cases and compares every output with the
 * CPU oracle (libropequant_oracle.so, linked as test infrastructure), to the
 * parity bar: scales and untouched cache bytes bit for bit; e4m3 codes equal
 * except at most 1e-4 of them one adjacent code apart; qnorm_rope's bf16 rows
 * within one bf16 ulp of the oracle's RMSNorm definition (its squares summed
 * in index order) on at most 1e-3 of the elements, and bit for bit equal to
 * the oracle summing them by recursive pairwise summation.  Also
 * checks that a rejected call reports its status and launches nothing.
 *
 * Inputs come from a seeded xorshift generator in this file.  Prints one line
 * per case and "capi parity OK" at the end; exits 1 on any mismatch.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ropequant.h"

/* the oracle's entry points (oracle/oracle.c) */
int orc_inv_rope_fp8_quant(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                           const int64_t* positions, const float* cos_sin_cache,
                           int64_t max_pos, int64_t n_tokens, int32_t n_heads,
                           int32_t heads_per_group, int32_t scale_fmt, double eps,
                           uint8_t* out, int64_t out_stride_group, int64_t out_stride_token,
                           void* scales, int64_t sc_stride_group, int64_t sc_stride_token,
                           int64_t sc_stride_block);
int orc_qnorm_rope(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
                   const uint16_t* norm_weight, const int64_t* positions,
                   const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
                   int32_t n_heads_q, int32_t q_head_padded, double eps, uint16_t* q_out,
                   int32_t sum_order);
int orc_kv_rope_quant_insert(const uint16_t* kv, int64_t kv_stride_token,
                             const int64_t* positions, const float* cos_sin_cache,
                             int64_t max_pos, const int64_t* slot_mapping, int64_t n_tokens,
                             uint8_t* k_cache, int64_t num_blocks, int64_t block_stride_bytes,
                             int32_t cache_block_size, int32_t scale_fmt, double eps);

#define HIP_OK(x)                                                                     \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(2);                                                                        \
    }                                                                                 \
  } while (0)

static uint64_t rng_state;

static uint64_t next_u64(void) {
  uint64_t x = rng_state;
  x ^= x << 13;
  x ^= x >> 7;
  x ^= x << 17;
  return rng_state = x;
}

/* approximately N(0, std): sum of 4 uniforms, centred and scaled */
static float draw(float std) {
  double s = 0.0;
  for (int i = 0; i < 4; ++i) s += (double)(next_u64() >> 11) * 0x1p-53;
  return (float)((s - 2.0) * 1.7320508 * std);
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite) */
static uint16_t bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float* cos_sin_table(int64_t max_pos) {
  float* t = malloc((size_t)max_pos * 64 * sizeof(float));
  for (int64_t p = 0; p < max_pos; ++p)
    for (int i = 0; i < 32; ++i) {
      const double ang = (double)p * pow(10000.0, -2.0 * i / 64.0);
      t[p * 64 + i] = (float)cos(ang);
      t[p * 64 + 32 + i] = (float)sin(ang);
    }
  return t;
}

static void* to_dev(const void* h, size_t n) {
  void* d;
  HIP_OK(hipMalloc(&d, n ? n : 1));
  if (n) HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
  return d;
}

static int failures;

static void check_bytes(const char* what, const uint8_t* got, const uint8_t* exp, size_t n) {
  size_t bad = 0;
  for (size_t i = 0; i < n; ++i) bad += got[i] != exp[i];
  printf("[capi] %s: %zu/%zu bytes equal\n", what, n - bad, n);
  if (bad) ++failures;
}

/* bf16 bit patterns: equal, except at most max_frac of them one ulp apart
 * with the same sign */
static void check_bf16_ulp(const char* what, const uint16_t* got, const uint16_t* exp, size_t n,
                           double max_frac) {
  size_t diff = 0, far = 0;
  for (size_t i = 0; i < n; ++i) {
    if (got[i] == exp[i]) continue;
    ++diff;
    if ((got[i] >> 15) != (exp[i] >> 15) || abs((int)got[i] - (int)exp[i]) != 1) ++far;
  }
  printf("[capi] %s: %zu/%zu exact, %zu one ulp apart, %zu further\n", what, n - diff, n,
         diff - far, far);
  if (far || (double)diff > max_frac * (double)n) ++failures;
}

static void check_codes(const char* what, const uint8_t* got, const uint8_t* exp, size_t n) {
  size_t diff = 0, far = 0;
  for (size_t i = 0; i < n; ++i) {
    if (got[i] == exp[i]) continue;
    ++diff;
    const int same_sign = (got[i] >> 7) == (exp[i] >> 7);
    const int adjacent = abs((got[i] & 0x7F) - (exp[i] & 0x7F)) == 1;
    if (!(same_sign && adjacent)) ++far;
  }
  printf("[capi] %s: %zu/%zu codes exact, %zu differ\n", what, n - diff, n, diff);
  if (far || (double)diff > 1e-4 * (double)n) ++failures;
}

static void case_irq(hipStream_t stream, int32_t fmt) {
  const int64_t N = 37, max_pos = 65536;
  const int32_t H = 24, hpg = 8, G = H / hpg;
  const size_t n_o = (size_t)N * H * 512, n_out = (size_t)G * N * hpg * 512;
  const size_t n_sc = fmt == RQ_SCALE_FP32 ? (size_t)G * N * hpg * 4 : (size_t)G * N * hpg;
  uint16_t* o = malloc(n_o * 2);
  int64_t* pos = malloc(N * 8);
  for (size_t i = 0; i < n_o; ++i) o[i] = bf16(draw(1.0f));
  for (int64_t t = 0; t < N; ++t) pos[t] = (int64_t)(next_u64() % (uint64_t)max_pos);
  float* cs = cos_sin_table(max_pos);
  uint16_t* d_o = to_dev(o, n_o * 2);
  int64_t* d_pos = to_dev(pos, N * 8);
  float* d_cs = to_dev(cs, (size_t)max_pos * 256);
  uint8_t* d_out;
  void* d_sc;
  HIP_OK(hipMalloc((void**)&d_out, n_out));
  HIP_OK(hipMalloc(&d_sc, n_sc * 4));
  const int rc = inv_rope_fp8_quant(d_o, H * 512, 512, d_pos, d_cs, max_pos, N, H, hpg, fmt,
                                    1e-10, d_out, N * hpg * 512, hpg * 512, d_sc,
                                    fmt == RQ_SCALE_FP32 ? N * hpg * 4 : N * hpg,
                                    fmt == RQ_SCALE_FP32 ? hpg * 4 : hpg, 1, stream);
  if (rc != RQ_OK) {
    printf("[capi] inv_rope_fp8_quant: %s\n", ropequant_strerror(rc));
    ++failures;
    return;
  }
  HIP_OK(hipStreamSynchronize(stream));
  uint8_t* out = malloc(n_out);
  uint8_t* eout = malloc(n_out);
  uint32_t* sc = malloc(n_sc * 4);
  uint32_t* esc = malloc(n_sc * 4);
  HIP_OK(hipMemcpy(out, d_out, n_out, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(sc, d_sc, n_sc * 4, hipMemcpyDeviceToHost));
  if (orc_inv_rope_fp8_quant(o, H * 512, 512, pos, cs, max_pos, N, H, hpg, fmt, 1e-10, eout,
                             N * hpg * 512, hpg * 512, esc,
                             fmt == RQ_SCALE_FP32 ? N * hpg * 4 : N * hpg,
                             fmt == RQ_SCALE_FP32 ? hpg * 4 : hpg, 1) != 0) {
    printf("[capi] oracle refused the irq case\n");
    ++failures;
    return;
  }
  check_bytes(fmt == RQ_SCALE_FP32 ? "irq fp32 scales" : "irq ue8m0 scales", (uint8_t*)sc,
              (uint8_t*)esc, n_sc * 4);
  check_codes(fmt == RQ_SCALE_FP32 ? "irq fp32 codes" : "irq ue8m0 codes", out, eout, n_out);
  HIP_OK(hipFree(d_o));
  HIP_OK(hipFree(d_pos));
  HIP_OK(hipFree(d_cs));
  HIP_OK(hipFree(d_out));
  HIP_OK(hipFree(d_sc));
  free(o), free(pos), free(cs), free(out), free(eout), free(sc), free(esc);
}

static void case_qnr(hipStream_t stream) {
  const int64_t N = 19, max_pos = 4096;
  const int32_t Hq = 5, Hpad = 8;
  const size_t n_q = (size_t)N * Hq * 512, n_out = (size_t)N * Hpad * 512;
  uint16_t* q = malloc(n_q * 2);
  uint16_t w[512];
  int64_t* pos = malloc(N * 8);
  for (size_t i = 0; i < n_q; ++i) q[i] = bf16(draw(2.0f));
  for (int i = 0; i < 512; ++i) w[i] = bf16(0.5f + (float)((next_u64() >> 11) * 0x1p-53));
  for (int64_t t = 0; t < N; ++t) pos[t] = (int64_t)(next_u64() % (uint64_t)max_pos);
  float* cs = cos_sin_table(max_pos);
  uint16_t* d_q = to_dev(q, n_q * 2);
  uint16_t* d_w = to_dev(w, sizeof w);
  int64_t* d_pos = to_dev(pos, N * 8);
  float* d_cs = to_dev(cs, (size_t)max_pos * 256);
  uint16_t* d_out;
  HIP_OK(hipMalloc((void**)&d_out, n_out * 2));
  HIP_OK(hipMemset(d_out, 0xFF, n_out * 2));  /* pad heads must come back zero */
  const int rc = qnorm_rope(d_q, Hq * 512, 512, d_w, d_pos, d_cs, max_pos, N, Hq, Hpad, 1e-6,
                            d_out, stream);
  if (rc != RQ_OK) {
    printf("[capi] qnorm_rope: %s\n", ropequant_strerror(rc));
    ++failures;
    return;
  }
  HIP_OK(hipStreamSynchronize(stream));
  uint16_t* out = malloc(n_out * 2);
  uint16_t* eout = malloc(n_out * 2);
  HIP_OK(hipMemcpy(out, d_out, n_out * 2, hipMemcpyDeviceToHost));
  if (orc_qnorm_rope(q, Hq * 512, 512, w, pos, cs, max_pos, N, Hq, Hpad, 1e-6, eout, 0) != 0) {
    printf("[capi] oracle refused the qnorm_rope case\n");
    ++failures;
    return;
  }
  check_bf16_ulp("qnorm_rope bf16 rows vs index-order RMSNorm", out, eout, n_out, 1e-3);
  if (orc_qnorm_rope(q, Hq * 512, 512, w, pos, cs, max_pos, N, Hq, Hpad, 1e-6, eout, 1) != 0) {
    printf("[capi] oracle refused the qnorm_rope case\n");
    ++failures;
    return;
  }
  check_bytes("qnorm_rope bf16 rows vs pairwise-summed RMSNorm", (uint8_t*)out, (uint8_t*)eout,
              n_out * 2);
  HIP_OK(hipFree(d_q));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_pos));
  HIP_OK(hipFree(d_cs));
  HIP_OK(hipFree(d_out));
  free(q), free(pos), free(cs), free(out), free(eout);
}

static void case_kvi(void) {  /* on the NULL (default) stream */
  const int64_t N = 50, max_pos = 4096, nb = 8;
  const int32_t bs = 16;
  const int64_t stride = bs * 528 + 32, n_cache = nb * stride;
  uint16_t* kv = malloc((size_t)N * 512 * 2);
  int64_t* pos = malloc(N * 8);
  int64_t* slots = malloc(N * 8);
  int64_t perm[128];
  for (int i = 0; i < nb * bs; ++i) perm[i] = i;
  for (int i = nb * bs - 1; i > 0; --i) {  /* seeded Fisher-Yates */
    const int j = (int)(next_u64() % (uint64_t)(i + 1));
    const int64_t tmp = perm[i];
    perm[i] = perm[j];
    perm[j] = tmp;
  }
  for (int64_t t = 0; t < N; ++t) {
    slots[t] = t % 7 == 3 ? -1 : perm[t];  /* some tokens are skipped */
    pos[t] = (int64_t)(next_u64() % (uint64_t)max_pos);
  }
  for (int64_t i = 0; i < N * 512; ++i) kv[i] = bf16(draw(1.0f));
  float* cs = cos_sin_table(max_pos);
  uint16_t* d_kv = to_dev(kv, (size_t)N * 1024);
  int64_t* d_pos = to_dev(pos, N * 8);
  int64_t* d_slots = to_dev(slots, N * 8);
  float* d_cs = to_dev(cs, (size_t)max_pos * 256);
  uint8_t* d_cache;
  HIP_OK(hipMalloc((void**)&d_cache, n_cache));
  HIP_OK(hipMemset(d_cache, 0xAA, n_cache));
  const int rc = kv_rope_quant_insert(d_kv, 512, d_pos, d_cs, max_pos, d_slots, N, d_cache, nb,
                                      stride, bs, RQ_SCALE_FP32, 1e-10, NULL);  /* NULL stream */
  if (rc != RQ_OK) {
    printf("[capi] kv_rope_quant_insert: %s\n", ropequant_strerror(rc));
    ++failures;
    return;
  }
  HIP_OK(hipDeviceSynchronize());
  uint8_t* cache = malloc(n_cache);
  uint8_t* ecache = malloc(n_cache);
  memset(ecache, 0xAA, n_cache);
  HIP_OK(hipMemcpy(cache, d_cache, n_cache, hipMemcpyDeviceToHost));
  if (orc_kv_rope_quant_insert(kv, 512, pos, cs, max_pos, slots, N, ecache, nb, stride, bs,
                               0, 1e-10) != 0) {
    printf("[capi] oracle refused the kv case\n");
    ++failures;
    return;
  }
  /* codes of written records within the code bar; every other byte exact */
  uint8_t* is_code = calloc(n_cache, 1);
  for (int64_t t = 0; t < N; ++t)
    if (slots[t] >= 0) {
      const int64_t off = (slots[t] / bs) * stride + (slots[t] % bs) * 528;
      memset(is_code + off, 1, 512);
    }
  size_t nc = 0, nr = 0;
  uint8_t *gc = malloc(n_cache), *ec = malloc(n_cache), *gr = malloc(n_cache),
          *er = malloc(n_cache);
  for (int64_t i = 0; i < n_cache; ++i) {
    if (is_code[i]) gc[nc] = cache[i], ec[nc++] = ecache[i];
    else gr[nr] = cache[i], er[nr++] = ecache[i];
  }
  check_codes("kv_rope_quant_insert codes", gc, ec, nc);
  check_bytes("kv_rope_quant_insert scales, holes and gaps", gr, er, nr);
  HIP_OK(hipFree(d_kv));
  HIP_OK(hipFree(d_pos));
  HIP_OK(hipFree(d_slots));
  HIP_OK(hipFree(d_cs));
  HIP_OK(hipFree(d_cache));
  free(kv), free(pos), free(slots), free(cs), free(cache), free(ecache), free(is_code);
  free(gc), free(ec), free(gr), free(er);
}

static void case_rejected(hipStream_t stream) {
  /* heads_per_group 7 does not divide 24 heads: RQ_ERR_SHAPE, no launch, and
   * the output stays as it was */
  uint8_t* d_out;
  HIP_OK(hipMalloc((void**)&d_out, 4096));
  HIP_OK(hipMemset(d_out, 0x5A, 4096));
  const int rc = inv_rope_fp8_quant((const uint16_t*)d_out, 24 * 512, 512, (const int64_t*)d_out,
                                    (const float*)d_out, 16, 1, 24, 7, RQ_SCALE_FP32, 1e-10,
                                    d_out, 512, 512, d_out, 32, 32, 1, stream);
  HIP_OK(hipStreamSynchronize(stream));
  uint8_t back[4096];
  HIP_OK(hipMemcpy(back, d_out, sizeof back, hipMemcpyDeviceToHost));
  size_t touched = 0;
  for (size_t i = 0; i < sizeof back; ++i) touched += back[i] != 0x5A;
  printf("[capi] rejected call: status %d (%s), %zu bytes touched\n", rc, ropequant_strerror(rc),
         touched);
  if (rc != RQ_ERR_SHAPE || touched) ++failures;
  HIP_OK(hipFree(d_out));
}

int main(void) {
  rng_state = 0x9E3779B97F4A7C15ull;
  if (ropequant_abi_version() != ROPEQUANT_ABI_VERSION) {
    printf("[capi] ABI version %d, header %d\n", ropequant_abi_version(), ROPEQUANT_ABI_VERSION);
    return 1;
  }
  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  case_irq(stream, RQ_SCALE_FP32);
  case_irq(stream, RQ_SCALE_UE8M0);
  case_qnr(stream);
  case_kvi();
  case_rejected(stream);
  HIP_OK(hipStreamDestroy(stream));
  if (failures) {
    printf("capi parity FAILED (%d)\n", failures);
    return 1;
  }
  printf("capi parity OK\n");
  return 0;
}

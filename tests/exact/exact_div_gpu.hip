// GPU check of rope_fp8_quant_amd/csrc/exact_div.h, the header the kernels
// use: for every positive normal fp32 x,
//   div448(x)      == x / 448    (IEEE division), for x >= 2^-116;
//   recip_scale(x) == 1 / x,                       for x <  2^126.
// Prints the mismatch counts; exit status 0 iff both are zero.  Counters and
// the first mismatching inputs live in a 4-word device buffer (constant,
// in-bounds indices); the grid-stride loop cannot wrap (hi + stride < 2^32).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "../../rope_fp8_quant_amd/csrc/exact_div.h"

#define CHECK(x)                                                        \
  do {                                                                  \
    hipError_t e_ = (x);                                                \
    if (e_ != hipSuccess) {                                             \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 2;                                                         \
    }                                                                   \
  } while (0)

__global__ void check(unsigned long long* count, unsigned int* first) {
  const uint32_t lo = 0x00800000u, hi = 0x7F800000u;
  const uint32_t div_lo = 0x05800000u;  // 2^-116
  const uint32_t rcp_hi = 0x7E800000u;  // 2^126
  const uint32_t stride = gridDim.x * blockDim.x;
  unsigned long long c0 = 0, c1 = 0;
  for (uint32_t u = lo + blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += stride) {
    const float x = __uint_as_float(u);
    if (u >= div_lo && __float_as_uint(div448(x)) != __float_as_uint(x / 448.0f)) {
      ++c0;
      atomicMin(&first[0], u);
    }
    if (u < rcp_hi && __float_as_uint(recip_scale(x)) != __float_as_uint(1.0f / x)) {
      ++c1;
      atomicMin(&first[1], u);
    }
  }
  if (c0) atomicAdd(&count[0], c0);
  if (c1) atomicAdd(&count[1], c1);
}

int main() {
  unsigned long long* count;
  unsigned int* first;
  CHECK(hipMalloc(&count, 2 * sizeof(unsigned long long)));
  CHECK(hipMalloc(&first, 2 * sizeof(unsigned int)));
  CHECK(hipMemset(count, 0, 2 * sizeof(unsigned long long)));
  CHECK(hipMemset(first, 0xFF, 2 * sizeof(unsigned int)));
  check<<<4096, 256>>>(count, first);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  unsigned long long h[2];
  unsigned int f[2];
  CHECK(hipMemcpy(h, count, sizeof h, hipMemcpyDeviceToHost));
  CHECK(hipMemcpy(f, first, sizeof f, hipMemcpyDeviceToHost));
  printf("div448 (x >= 2^-116): %llu mismatches (first 0x%08x)\n", h[0], f[0]);
  printf("recip_scale (x < 2^126): %llu mismatches (first 0x%08x)\n", h[1], f[1]);
  return (h[0] || h[1]) ? 1 : 0;
}

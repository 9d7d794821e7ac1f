/*
 * Host check of the division form the kernels use for m / 448: for every
 * fp32 m from 2^-116 (the kernels' amax floor) to the largest finite one
 * (below about 2^-117 the quotient is subnormal and the 2^-6 step would round
 * a second time: outside the domain),
 *     q0 = RN(m * RN(1/7)),  q = RN(q0 + RN(m - 7 q0) ... ) via two FMAs,
 *     RN(m / 448) == q * 2^-6.
 * Written out here in C with fmaf; the GPU checker runs the kernels' own
 * header.  Exit status 0 iff there is no mismatch.  Splits the range over
 * argv[1] threads of work given as argv[2] (index) for parallel runs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  const uint32_t lo = 0x05800000u, hi = 0x7F800000u;  /* [2^-116, +inf) */
  const uint32_t parts = argc > 2 ? (uint32_t)atoi(argv[1]) : 1u;
  const uint32_t part = argc > 2 ? (uint32_t)atoi(argv[2]) : 0u;
  const uint32_t span = (hi - lo) / parts + 1u;
  const uint32_t a = lo + part * span;
  const uint32_t b = (hi - a) > span ? a + span : hi;
  const float c7 = 1.0f / 7.0f;
  uint64_t bad = 0;
  for (uint32_t u = a; u < b; ++u) {
    const float m = f_of(u);
    const float q0 = m * c7;
    const float q = fmaf(fmaf(-q0, 7.0f, m), c7, q0);
    const float got = q * 0x1p-6f;
    const float ref = m / 448.0f;
    if (u_of(got) != u_of(ref)) {
      if (bad < 5) printf("mismatch m=%a got=%a ref=%a\n", m, got, ref);
      ++bad;
    }
  }
  printf("div448 host: bits [0x%08x, 0x%08x): %llu mismatches\n", a, b, (unsigned long long)bad);
  return bad != 0;
}

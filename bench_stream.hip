// Streaming kernels for bench.py (measurement only; not part of libropequant's
// ABI).  They move bytes in the access patterns the library's kernels use,
// with no arithmetic, so that bench.py can report what this part's HBM
// sustains for each pattern beside what the kernels reach:
//   * stream_read     - one 1 KiB row per 16-byte-per-lane nontemporal load
//                       instruction, four rows per wave (the kernels' reads;
//                       the row index is clamped rather than branched on, so
//                       the four loads issue back to back);
//   * stream_write    - 1 KiB rows written with nontemporal, plain or
//                       sc1-policy (buffer) 16-byte stores, sixteen rows per
//                       wave (timed fastest of 4, 8 and 16);
//   * stream_irq      - inv_rope_fp8_quant's traffic per 512-dim unit: a 1 KiB
//                       row read, 512 bytes and one 16-byte scale group
//                       written, in 128-thread workgroups dealt to the XCDs
//                       in chunks of 64, with a round trip through LDS
//                       between the reads and the writes as the kernels make
//                       (without it the same bytes took 5% longer); four
//                       units per wave (the library's common structure) or
//                       two (inv_rope_fp8_quant's); each also with the rows
//                       read straight into LDS (global_load_lds_dwordx4);
//   * stream_rows_gm  - inv_rope_bf16's traffic per 512-dim unit: a 1 KiB row
//                       read and a 1 KiB row written, group-major as that
//                       op writes them ([G, tokens, hpg rows]), four units per
//                       wave in 256-thread workgroups dealt to the XCDs in
//                       chunks of 64, through LDS as above;
//   * stream_q        - the q paths' traffic per unit of a head-padded output:
//                       a 1 KiB row read for a live head (none for a pad
//                       head), then 1 KiB written (qnorm_rope's bf16 rows) or
//                       512 bytes and a 16-byte scale group (qnorm_rope_fp8),
//                       the rows with sc1 buffer stores as those kernels,
//                       four units per wave in 256-thread workgroups dealt to
//                       the XCDs in chunks of 16, through LDS;
//   * stream_empty    - a launch that does nothing: the fixed cost of one
//                       launch on a stream.
// Every kernel covers exactly `rows` rows; the host sizes the grid so that no
// wave reads or writes past them.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t* gptr_c;
typedef __attribute__((address_space(1))) u32x4_t* gptr;

// Workgroups dealt to the 8 XCDs in chunks of 2^chunk_log2 consecutive ones
// (a bijection on [0, gridDim.x); a tail shorter than 8 chunks keeps its
// order), the mapping the library's kernels use.
__device__ __forceinline__ uint32_t xcd_block(uint32_t chunk_log2) {
  const uint32_t nb = gridDim.x, b = blockIdx.x;
  const uint32_t full = (nb >> (chunk_log2 + 3)) << (chunk_log2 + 3);
  if (b >= full) return b;
  const uint32_t xcd = b & 7u, local = b >> 3;
  const uint32_t chunk = local >> chunk_log2, within = local & ((1u << chunk_log2) - 1u);
  return (((chunk << 3) + xcd) << chunk_log2) + within;
}

__device__ __forceinline__ uint32_t wave_id(uint32_t chunk_log2) {
  return __builtin_amdgcn_readfirstlane(xcd_block(chunk_log2) * (blockDim.x >> 6) +
                                        (threadIdx.x >> 6));
}

// Reads rows [4w, 4w + 4) of 1 KiB (a row past the end reads the last row
// again); a value is written to sink only when the XOR of everything read
// equals `never` (chosen by the host as a value the data cannot produce),
// which keeps the loads live.
__global__ __launch_bounds__(256) void stream_read(const uint8_t* src, uint64_t rows,
                                                   uint32_t never, uint32_t* sink) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t r0 = (uint64_t)wave_id(4) * 4;
  u32x4_t acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t r = r0 + k < rows ? r0 + k : rows - 1;
    acc ^= __builtin_nontemporal_load((gptr_c)(src + r * 1024 + 16 * lane));
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == never) sink[lane] = x;
}

// Writes rows [16w, 16w + 16).  POLICY: 0 nontemporal, 1 plain, 2 sc1
// through a buffer store on the row.
constexpr int kWriteRows = 16;

template <int POLICY>
__global__ __launch_bounds__(256) void stream_write(uint8_t* dst, uint64_t rows, uint32_t v) {
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t r0 = (uint64_t)wave_id(4) * kWriteRows;
  const u32x4_t w = {v, v ^ lane, v + lane, ~v};
#pragma unroll
  for (int k = 0; k < kWriteRows; ++k) {
    if (r0 + k >= rows) continue;
    uint8_t* row = dst + (r0 + k) * 1024;
    if (POLICY == 0) {
      __builtin_nontemporal_store(w, (gptr)(row + 16 * lane));
    } else if (POLICY == 1) {
      *(gptr)(row + 16 * lane) = w;
    } else {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, 0, 1024, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b128(w, rs, 16 * lane, 0, 16);
    }
  }
}

// Per unit u: read the 1 KiB row u of src; write 512 bytes at codes + 512 u
// (nontemporal) and 16 bytes at scales + 16 u (plain), as inv_rope_fp8_quant
// does with group-major outputs.  U units per wave (4, as the kernel, or 2);
// each store instruction writes two units' code rows, lanes 0..31 the even
// unit and lanes 32..63 the odd one, 16 bytes each.
//
// DIRECT: the rows go straight into the wave's LDS slice instead
// (global_load_lds_dwordx4, nontemporal: lane i's 16 bytes land at byte 16 i
// of the destination), with no VGPR staging and no LDS write instruction;
// the wait for those LDS writes is explicit, since the compiler does not
// order LDS reads after these loads by itself.
constexpr short kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0); expcnt, lgkmcnt left alone

template <int U, bool DIRECT>
__global__ __launch_bounds__(128) void stream_irq(const uint8_t* src, uint8_t* codes,
                                                  uint8_t* scales, uint64_t units) {
  extern __shared__ u32x4_t lds[];
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t u0 = (uint64_t)wave_id(6) * U;
  u32x4_t* slice = lds + 64 * U * (threadIdx.x >> 6);
  u32x4_t in[U];
  if (DIRECT) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint64_t u = u0 + k < units ? u0 + k : units - 1;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + u * 1024 + 16 * lane),
          (__attribute__((address_space(3))) void*)(slice + 64 * k), 16, 0, 2 /* nt */);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  } else {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint64_t u = u0 + k < units ? u0 + k : units - 1;
      in[k] = __builtin_nontemporal_load((gptr_c)(src + u * 1024 + 16 * lane));
    }
    // through the wave's U KiB of LDS and back, lanes permuted, as the
    // kernel's transpose does
#pragma unroll
    for (int k = 0; k < U; ++k) slice[64 * k + lane] = in[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
#pragma unroll
  for (int k = 0; k < U; ++k) in[k] = slice[64 * k + (lane ^ 5)];
  const uint32_t half = lane >> 5, j = lane & 31;
#pragma unroll
  for (int k = 0; k < U / 2; ++k) {
    const uint64_t u = u0 + 2 * k + half;
    // something from every row read, so no load is dead (the same for both
    // halves: a per-lane pick of the register array would cost hundreds of
    // selects)
    const u32x4_t w = in[2 * k] ^ in[2 * k + 1];
    if (u < units) __builtin_nontemporal_store(w, (gptr)(codes + u * 512 + 16 * j));
  }
  // unit k's scales from lane 16 k
  const uint32_t row = lane >> 4;
  if ((lane & 15) == 0 && row < (uint32_t)U && u0 + row < units) {
    u32x4_t s = in[0];
#pragma unroll
    for (int k = 1; k < U; ++k)
      if (row == (uint32_t)k) s = in[k];
    *(gptr)(scales + (u0 + row) * 16) = s;
  }
}

// Per unit u = (t, h) of `units` = tokens x 2^heads_log2: read the 1 KiB row
// u of src, write it (through LDS, lanes permuted) as row j of group
// g = h / 2^hpg_log2, token t of dst, group-major:
// dst + ((g * tokens + t) * 2^hpg_log2 + j) KiB.  (Powers of two, so that the
// index arithmetic is shifts: a division by a runtime value would cost more
// than the rest of the kernel.)
__global__ __launch_bounds__(256) void stream_rows_gm(const uint8_t* src, uint8_t* dst,
                                                      uint64_t units, uint32_t heads_log2,
                                                      uint32_t hpg_log2) {
  extern __shared__ u32x4_t lds[];
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t u0 = (uint64_t)wave_id(6) * 4;
  const uint64_t tokens = units >> heads_log2;
  u32x4_t in[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t u = u0 + k < units ? u0 + k : units - 1;
    in[k] = __builtin_nontemporal_load((gptr_c)(src + u * 1024 + 16 * lane));
  }
  u32x4_t* slice = lds + 256 * (threadIdx.x >> 6);
#pragma unroll
  for (int k = 0; k < 4; ++k) slice[64 * k + lane] = in[k];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int k = 0; k < 4; ++k) in[k] = slice[64 * k + (lane ^ 5)];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t u = u0 + k;
    if (u < units) {
      const uint64_t t = u >> heads_log2, h = u & ((1u << heads_log2) - 1u);
      const uint64_t row = (((h >> hpg_log2) * tokens + t) << hpg_log2) + (h & ((1u << hpg_log2) - 1u));
      __builtin_nontemporal_store(in[k], (gptr)(dst + row * 1024 + 16 * lane));
    }
  }
}

// Per unit u = (t, h) of `units` = tokens x 2^hpad_log2: a live head (h < hq)
// reads row t * hq + h of src; every unit writes out_bytes (1024, or 512 and
// 16 scale bytes) at dst + u * out_bytes (and scales + 16 u).
template <int OUT_BYTES>
__global__ __launch_bounds__(256) void stream_q(const uint8_t* src, uint8_t* dst, uint8_t* scales,
                                                uint64_t units, uint32_t hq, uint32_t hpad_log2) {
  extern __shared__ u32x4_t lds[];
  const uint32_t lane = threadIdx.x & 63;
  const uint64_t u0 = (uint64_t)wave_id(4) * 4;
  u32x4_t in[4] = {};
  bool live[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t u = u0 + k < units ? u0 + k : units - 1;
    const uint64_t t = u >> hpad_log2, h = u & ((1u << hpad_log2) - 1u);
    live[k] = h < hq;
    if (live[k]) in[k] = __builtin_nontemporal_load((gptr_c)(src + (t * hq + h) * 1024 + 16 * lane));
  }
  u32x4_t* slice = lds + 256 * (threadIdx.x >> 6);
#pragma unroll
  for (int k = 0; k < 4; ++k) slice[64 * k + lane] = in[k];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int k = 0; k < 4; ++k) in[k] = slice[64 * k + (lane ^ 5)];
  // the rows go out as the q kernels write them: buffer stores with the sc1
  // cache-policy bit
  if (OUT_BYTES == 1024) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (u0 + k < units) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(dst + (u0 + k) * 1024, 0, 1024, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(in[k], rs, 16 * lane, 0, 16);
      }
  } else {
    const uint32_t half = lane >> 5, j = lane & 31;
    // one resource over the wave's four 512-byte rows (a tail wave's missing
    // rows are never written: the guard below)
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(dst + u0 * 512, 0, 4 * 512, 0x00020000);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint64_t u = u0 + 2 * k + half;
      const u32x4_t w = in[2 * k] ^ in[2 * k + 1];  // as in stream_irq
      if (u < units) __builtin_amdgcn_raw_buffer_store_b128(w, rs, 512 * (2 * k + half) + 16 * j, 0, 16);
    }
    // unit k's scale group from lane 16 k
    const uint32_t row = lane >> 4;
    if ((lane & 15) == 0 && u0 + row < units) {
      u32x4_t sv = in[0];
#pragma unroll
      for (int k = 1; k < 4; ++k)
        if (row == (uint32_t)k) sv = in[k];
      *(gptr)(scales + (u0 + row) * 16) = sv;
    }
  }
}

__global__ void stream_empty() {}

int grid_for(uint64_t rows_or_units, uint32_t per_block) {
  return (int)((rows_or_units + per_block - 1) / per_block);
}

}  // namespace

extern "C" {

// Each returns 0, or -1 when the runtime refuses the launch (or the size is
// out of range for a 32-bit grid).
int bench_stream_read(const void* src, uint64_t rows, uint32_t never, void* sink, void* stream) {
  if (rows == 0 || rows > (1ull << 36)) return -1;
  hipLaunchKernelGGL(stream_read, dim3(grid_for(rows, 16)), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)src, rows, never, (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int bench_stream_write(void* dst, uint64_t rows, int policy, void* stream) {
  if (rows == 0 || rows > (1ull << 36) || policy < 0 || policy > 2) return -1;
  const dim3 g(grid_for(rows, 4 * kWriteRows)), b(256);
  const hipStream_t s = (hipStream_t)stream;
  if (policy == 0) hipLaunchKernelGGL(stream_write<0>, g, b, 0, s, (uint8_t*)dst, rows, 0x5A5Au);
  if (policy == 1) hipLaunchKernelGGL(stream_write<1>, g, b, 0, s, (uint8_t*)dst, rows, 0x5A5Au);
  if (policy == 2) hipLaunchKernelGGL(stream_write<2>, g, b, 0, s, (uint8_t*)dst, rows, 0x5A5Au);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// units_per_wave: 4 or 2, or either | kDirect for the direct-to-LDS reads
constexpr int kDirect = 0x100;

int bench_stream_irq(const void* src, void* codes, void* scales, uint64_t units,
                     int units_per_wave, void* stream) {
  if (units == 0 || units > (1ull << 36)) return -1;
  const hipStream_t s = (hipStream_t)stream;
  const uint8_t* in = (const uint8_t*)src;
  uint8_t *c = (uint8_t*)codes, *sc = (uint8_t*)scales;
  if (units_per_wave == 4)
    hipLaunchKernelGGL((stream_irq<4, false>), dim3(grid_for(units, 8)), dim3(128), 2 * 4096, s,
                       in, c, sc, units);
  else if (units_per_wave == 2)
    hipLaunchKernelGGL((stream_irq<2, false>), dim3(grid_for(units, 4)), dim3(128), 2 * 2048, s,
                       in, c, sc, units);
  else if (units_per_wave == (4 | kDirect))
    hipLaunchKernelGGL((stream_irq<4, true>), dim3(grid_for(units, 8)), dim3(128), 2 * 4096, s,
                       in, c, sc, units);
  else if (units_per_wave == (2 | kDirect))
    hipLaunchKernelGGL((stream_irq<2, true>), dim3(grid_for(units, 4)), dim3(128), 2 * 2048, s,
                       in, c, sc, units);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int bench_stream_rows_gm(const void* src, void* dst, uint64_t units, uint32_t heads,
                         uint32_t hpg, void* stream) {
  // heads and hpg powers of two, hpg <= heads
  if (units == 0 || units > (1ull << 36) || heads == 0 || hpg == 0 || (heads & (heads - 1)) ||
      (hpg & (hpg - 1)) || heads % hpg || units % heads)
    return -1;
  hipLaunchKernelGGL(stream_rows_gm, dim3(grid_for(units, 16)), dim3(256), 4 * 4096,
                     (hipStream_t)stream, (const uint8_t*)src, (uint8_t*)dst, units,
                     (uint32_t)__builtin_ctz(heads), (uint32_t)__builtin_ctz(hpg));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int bench_stream_q(const void* src, void* dst, void* scales, uint64_t units, uint32_t hq,
                   uint32_t hpad, int out_bytes, void* stream) {
  // hpad a power of two
  if (units == 0 || units > (1ull << 36) || hq == 0 || hpad < hq || (hpad & (hpad - 1)) ||
      units % hpad)
    return -1;
  const hipStream_t s = (hipStream_t)stream;
  const uint32_t hl = (uint32_t)__builtin_ctz(hpad);
  if (out_bytes == 1024)
    hipLaunchKernelGGL(stream_q<1024>, dim3(grid_for(units, 16)), dim3(256), 4 * 4096, s,
                       (const uint8_t*)src, (uint8_t*)dst, (uint8_t*)scales, units, hq, hl);
  else if (out_bytes == 512 && scales)
    hipLaunchKernelGGL(stream_q<512>, dim3(grid_for(units, 16)), dim3(256), 4 * 4096, s,
                       (const uint8_t*)src, (uint8_t*)dst, (uint8_t*)scales, units, hq, hl);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int bench_stream_empty(void* stream) {
  hipLaunchKernelGGL(stream_empty, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"

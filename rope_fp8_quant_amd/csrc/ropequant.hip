// libropequant: gfx950 kernels and the C ABI for the fused RoPE + block-FP8
// steps around 512-dim attention heads, and the sparse-attention indexer's
// 128-dim query path.
//
// Sources (web pages; cited by title and section):
//   [P1] "vLLM DeepSeek-V4 성능 최적화: Eager Break 시 Workspace 재사용 개선"
//        (analysis of vLLM PR #49236), section 1: the q-norm/RoPE + kv
//        RoPE/quant/insert op, its caller-allocated q_out and its checks;
//        section 2: the op schema and the full-cache forms beside it.
//   [P3] "vLLM, DeepSeek V4 모델의 저지연을 위한 RMSNorm과 라우터 GEMV 연산
//        융합으로 성능 극대화" (analysis of vLLM PR #41263), section 5: RMSNorm.
//   [P4] "한 프로그램이 4개 head를 처리하게 하라: DeepSeek-V4 inverse RoPE +
//        FP8 quant 커널 3.5배 가속기" (analysis of vLLM PR #63540): intro,
//        sections 1-4 (heads per program, partner kept in registers, block
//        amax, the compile keys and the launch shape by program count).
//   [P5] "vLLM의 GLM5.2 성능 최적화: Triton 커널 융합을 통한 E2E Throughput
//        향상" (analysis of vLLM PR #46862), section 1: the indexer query path.
//
// Work decomposition (the 512-dim kernels; the indexer's is described at
// its kernel)
//   A "unit" is one 512-dim head vector: (token, head) for inv_rope_* and
//   qnorm_rope*, a token for the kv paths.  One unit is handled by one 16-lane
//   DPP row of a wave64, so a wave holds 4 units and every cross-lane step
//   stays inside a row.  Lane L of the row (quad q = L >> 2, r = L & 3) owns
//   the four 8-dim chunks 16q + r + 4k (k = 0..3), i.e. dims
//   [128q + 8r + 32k, +8): all 32 of its dims lie in quant block q, so a
//   block's amax is a max over 32 registers and two quad DPP steps, and each
//   lane computes its block's scale once.  Every GPT-J pair (2i, 2i+1) sits
//   in one lane as the low/high halves of a bf16 dword, so the RoPE partner
//   never leaves its register ([P4] section 2's point, with no split/join at
//   all).  The rotated dims 448..511 are chunks k = 2, 3 of lanes 12..15.
//   The pages group heads per program so that a program never straddles a
//   wo_a group ([P4] section 1); here each row computes its own
//   (group, head-in-group) address, so a wave may mix groups or tokens and
//   ragged head counts need no special case.
//
// Arithmetic: IEEE binary32 basic operations, round to nearest even, no
// contraction (built with -ffp-contract=off); the square root is the
// compiler's correctly rounded one; m / 448 and 1 / s come from the exact
// FMA forms of exact_div.h; fp32 denormals are preserved.  Results therefore
// match an unfused fp32 evaluation bit for bit.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <cstring>

#include "ropequant.h"
#include "exact_div.h"

namespace {

constexpr int kHeadDim = 512;
constexpr int kRecordBytes = 528;  // one paged-cache slot: 512 codes + 16 scale bytes
constexpr float kE4m3Max = 448.0f;

// ------------------------------------------------------------ small helpers

// n / d for n < 2^31: q = (n * mul) >> shift with mul = ceil(2^(31+s) / d),
// s = ceil(log2 d).  With e = mul*d - 2^(31+s) < d the error term n*e/(d*2^(31+s))
// stays below 2^-s <= 1/d, so the floor is exact.
struct Magic {
  uint32_t mul;
  uint32_t shift;
};

__device__ __forceinline__ uint32_t magic_div(uint32_t n, Magic m) {
  return (uint32_t)(((uint64_t)n * m.mul) >> m.shift);
}

// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
// Renumber them so each XCD takes chunks of 2^chunk_log2 consecutive
// workgroups (chunk i of the grid goes to XCD i mod 8): neighbouring units
// share an XCD (and so their cos/sin rows share its L2) while all XCDs still
// sweep the tensors together.  The chunk size is a launch-table entry,
// measured per kernel (whole-range chunks, plain round-robin and sizes in
// between were timed).  A bijection on [0, gridDim.x): a tail shorter than
// 8 chunks keeps the plain order.
__device__ __forceinline__ uint32_t xcd_block_id(uint32_t chunk_log2) {
  const uint32_t nb = gridDim.x, b = blockIdx.x;
  const uint32_t full = (nb >> (chunk_log2 + 3)) << (chunk_log2 + 3);
  if (b >= full) return b;
  const uint32_t xcd = b & 7u, local = b >> 3;
  const uint32_t chunk = local >> chunk_log2, within = local & ((1u << chunk_log2) - 1u);
  return (((chunk << 3) + xcd) << chunk_log2) + within;
}

__device__ __forceinline__ float bf_lo(uint32_t w) {
  return (float)__builtin_bit_cast(__bf16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float bf_hi(uint32_t w) {
  return (float)__builtin_bit_cast(__bf16, (uint16_t)(w >> 16));
}

// DPP controls (row = 16 lanes)
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within the row
constexpr int kRowShl8 = 0x108;       // lane i <- lane i+8 within the row

// Every control used here either has a source lane for each lane or leaves
// the lanes without one at 0, so bound_ctrl (write 0) and an old value of 0
// agree; with bound_ctrl set the compiler needs no zeroed destination first.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// max(m, m of the lane CTRL names) for m >= 0 and not NaN, which every
// per-lane block maximum of NaN-free inputs is: such floats order like their
// bit patterns, and the integer max takes the DPP read as an operand where
// a float max would first quiet it.
template <int CTRL>
__device__ __forceinline__ float max_dpp_nonneg(float m) {
  const uint32_t u = __builtin_bit_cast(uint32_t, m);
  return __builtin_bit_cast(float, max(u, dpp_u32<CTRL>(u)));
}

// 2^k and 2^-k for the power-of-two (UE8M0) scales, k in [-126, 128].  A
// finite amax gives k <= 120 (t = amax / 448 < 2^120); k = 128 comes only
// from an amax that overflowed to +inf, where 2^k is +inf and 2^-k the
// subnormal 2^-128, as exact powers of two (so the codes of the block's
// finite values are still their exact scaling).
__device__ __forceinline__ float pow2_f32(int k) {
  return __builtin_bit_cast(float, (uint32_t)(k + 127) << 23);
}
__device__ __forceinline__ float pow2_neg_f32(int k) {
  return __builtin_bit_cast(float, k < 127 ? (uint32_t)(127 - k) << 23
                                           : 0x00400000u >> (k - 127));
}

// The lane's 32 values: x[k][e] is dim lane_dim0 + 32k + e.
struct Vals {
  float x[4][8];
};

__device__ __forceinline__ int lane_dim0(int L) { return 128 * (L >> 2) + 8 * (L & 3); }

__device__ __forceinline__ void unpack_bf16(const uint4 (&w)[4], Vals& v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t d[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v.x[k][2 * i] = bf_lo(d[i]);
      v.x[k][2 * i + 1] = bf_hi(d[i]);
    }
  }
}

// ---- staging: contiguous HBM reads, then the per-lane layout through LDS
//
// Each wave owns 4 KiB of LDS: one 1 KiB row per unit.  A wave first reads
// its 4 units' rows with 16-byte nontemporal loads whose 64 lanes cover one
// whole 1 KiB row per instruction (full cache lines per instruction, which
// is what lets the streaming reads run near the HBM peak), writes them to
// LDS, and each 16-lane row then reads back its unit's 4 chunks per lane.
// 16-byte slot s of a unit row is stored at LDS slot s ^ (((s >> 4) & 3) << 2):
// the 16 lanes of a row then read 16 different bank groups for each of
// their 4 reads, and the writes stay conflict-free too.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t* global_u32x4_ptr;

// 16-byte nontemporal load from global memory (the explicit address space
// keeps it a global_load rather than a flat one).
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((global_u32x4_ptr)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Wave-uniform read of an input that no kernel writes while this one runs
// (token positions, slot ids).  Through the constant address space it is
// always a scalar load, whatever shape the surrounding control flow takes.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// 16-byte nontemporal store: the output rows are not read again by this
// kernel, and for whole 1 KiB rows it measured faster than a plain store.
__device__ __forceinline__ void store_nt(uint8_t* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (__attribute__((address_space(1))) u32x4_t*)p);
}

__device__ __forceinline__ void wave_lds_sync() {
  // LDS operations of one wave complete in issue order; these keep the
  // compiler from moving the reads above the writes.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// rows[k] = first element of unit k's 512-dim bf16 row (wave-uniform; the
// kernels substitute a row they do read for any slot without a unit, so the
// four loads are unconditional).  issue_rows starts the four 1 KiB reads;
// transpose_rows parks them in LDS and hands lane L of row q, in w[m], the
// 8 bf16 of dims lane_dim0(L) + 32m of unit q.
__device__ __forceinline__ void issue_rows(const uint16_t* const (&rows)[4], int lane,
                                           uint4 (&raw)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) raw[k] = load_nt(reinterpret_cast<const uint4*>(rows[k]) + lane);
}

__device__ __forceinline__ void transpose_rows(uint4* lds_wave, const uint4 (&raw)[4], int lane,
                                               uint4 (&w)[4]) {
  const int wslot = lane ^ (((lane >> 4) & 3) << 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) lds_wave[64 * k + wslot] = raw[k];
  wave_lds_sync();
  const int q = lane >> 4, L = lane & 15, b = L >> 2, r = L & 3;
  // slot 16b + r + 4m lives at 16b + r + 4(m ^ b)
#pragma unroll
  for (int m = 0; m < 4; ++m) w[m] = lds_wave[64 * q + 16 * b + r + 4 * (m ^ b)];
}

// cos/sin for the lane's rotated pairs (lanes 12..15 only): c[0] = cos of
// the 4 pairs in chunk k=2, c[1] = cos for k=3; s[] the matching sin.
struct RopeCS {
  float4 c[2];
  float4 s[2];
};

__device__ __forceinline__ void load_cs(const float* row, int r, RopeCS& cs) {
  const float4* p = reinterpret_cast<const float4*>(row);
  cs.c[0] = p[r];       // cos[4r .. 4r+3]
  cs.c[1] = p[4 + r];   // cos[16+4r ..]
  cs.s[0] = p[8 + r];   // sin[4r ..]      (column 32 + ...)
  cs.s[1] = p[12 + r];  // sin[16+4r ..]
}

// GPT-J rotation of the lane's chunks 2 and 3 (dims 448..511 on lanes 12..15).
//   INVERSE: e' = e*c + o*s,  o' = o*c - e*s   ([P4] section 2)
//   forward: e' = e*c - o*s,  o' = o*c + e*s
template <bool INVERSE>
__device__ __forceinline__ void rope_lane(Vals& v, const RopeCS& cs) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const float cv[4] = {cs.c[kk].x, cs.c[kk].y, cs.c[kk].z, cs.c[kk].w};
    const float sv[4] = {cs.s[kk].x, cs.s[kk].y, cs.s[kk].z, cs.s[kk].w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float e = v.x[2 + kk][2 * p], o = v.x[2 + kk][2 * p + 1];
      const float ec = e * cv[p], os = o * sv[p], oc = o * cv[p], es = e * sv[p];
      if (INVERSE) {
        v.x[2 + kk][2 * p] = ec + os;
        v.x[2 + kk][2 * p + 1] = oc - es;
      } else {
        v.x[2 + kk][2 * p] = ec - os;
        v.x[2 + kk][2 * p + 1] = oc + es;
      }
    }
  }
}

// The scale of a block whose absolute maximum is m ([P4] section 3): m is
// floored at eps; FP32 mode gives scale = m/448 and the multiplier 1/scale,
// both correctly rounded; UE8M0 gives scale = 2^k for the smallest k with
// m/448 <= 2^k, the multiplier 2^-k and the exponent byte k+127.  An
// infinite m (a rotated pair past the fp32 range) gives scale +inf with
// multiplier 0 (FP32), or k = 128 (UE8M0).
template <int FMT>
__device__ __forceinline__ void block_scale(float m, float eps, float& scale, float& mult,
                                            uint32_t& ebyte) {
  m = __builtin_fmaxf(m, eps);
  if (FMT == RQ_SCALE_UE8M0) {
    const float t = m < __builtin_inff() ? div448(m) : m;
    const uint32_t u = __builtin_bit_cast(uint32_t, t);
    const int kexp = (int)((u >> 23) & 0xFFu) - 127 + ((u & 0x7FFFFFu) ? 1 : 0);
    scale = pow2_f32(kexp);
    mult = pow2_neg_f32(kexp);
    ebyte = (uint32_t)(kexp + 127);
  } else {
    const bool finite = m < __builtin_inff();
    scale = finite ? div448(m) : m;
    mult = finite ? recip_scale(scale) : 0.0f;
    ebyte = 0;
  }
}

// Block quantization of the lane's 32 values ([P4] section 3).  The 4 lanes
// of a quad share block q.  Returns the block's scale value (FP32 mode:
// m/448; UE8M0: 2^k) and the exponent byte k+127 (UE8M0), and the codes as
// 8 dwords (chunk k -> codes[2k], codes[2k+1]).
template <int FMT>
__device__ __forceinline__ void quantize_lane(const Vals& v, float eps, float& scale,
                                              uint32_t& ebyte, uint32_t (&codes)[8]) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v.x[k][e]));
  m = max_dpp_nonneg<kQuadSwap1>(m);
  m = max_dpp_nonneg<kQuadSwap2>(m);
  float mult;
  block_scale<FMT>(m, eps, scale, mult, ebyte);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // No clamp is needed before the convert: |x * mult| <= 448 * (1 + 2^-24)^3
      // < 448.0001 (two roundings of the scale, one of the product), and the
      // convert rounds to nearest even, giving 448 for every value up to 464.
      float q[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = v.x[k][4 * h + e] * mult;
      // bytes 2..3 of the first result are overwritten by the second convert,
      // so any register serves as its "old" operand
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], __builtin_bit_cast(int, q[0]), false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], w, true);
      codes[2 * k + h] = (uint32_t)w;
    }
  }
}

// OR of the four blocks' exponent bytes into one word (block q in byte q).
// Within a quad the byte is uniform, so the two mirrors act as xor-4 / xor-8.
__device__ __forceinline__ uint32_t pack_ue8m0(uint32_t ebyte, int q) {
  uint32_t w = ebyte << (8 * q);
  w |= dpp_u32<kRowHalfMirror>(w);
  w |= dpp_u32<kRowMirror>(w);
  return w;
}

// Output forms of a kernel's 512-dim results: block FP8 with fp32 or UE8M0
// scales (the RQ_SCALE_* values), or plain bf16 (no quantization).
constexpr int kOutBf16 = 2;

// The lane's 32 values rounded to bf16 (RNE), chunk m in outv[m]: the
// layout the bf16 row store below takes.
__device__ __forceinline__ void pack_bf16(const Vals& v, uint4 (&outv)[4]) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t o4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 f = {v.x[k][2 * i], v.x[k][2 * i + 1]};
      o4[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    outv[k] = make_uint4(o4[0], o4[1], o4[2], o4[3]);
  }
}

// Stores of the wave's four 512-dim results, staged back through LDS so
// that every store instruction writes whole rows.  dst[k] is unit k's
// destination; it is written only when ok[k] (wave-uniform) is set.
//
// bf16: lane L of row q holds, in outv[m], dims lane_dim0(L) + 32m of unit q.
// Through LDS with the input side's slot swizzle, each store then writes one
// unit's contiguous 1 KiB.  POL picks the store's cache policy:
//   kStoreNt  - nontemporal (inv_rope_bf16's rows and the kv bf16 cache);
//   kStoreSc1 - the sc1 policy bit, through a buffer store on a resource
//               spanning the unit's row (qnorm_rope's q_out, which is half
//               pad heads: 1.7% faster there, slower for inv_rope_bf16).
constexpr int kStoreNt = 0;
constexpr int kStoreSc1 = 16;  // the buffer-store cache-policy operand's sc1 bit

template <int POL>
__device__ __forceinline__ void store_rows_bf16(uint4* lds_wave, const uint4 (&outv)[4], int lane,
                                                uint8_t* const (&dst)[4],
                                                const bool (&ok)[4]) {
  const int q = lane >> 4, L = lane & 15, b = L >> 2, r = L & 3;
  wave_lds_sync();  // the transpose reads are done before the slice is reused
#pragma unroll
  for (int m = 0; m < 4; ++m) lds_wave[64 * q + 16 * b + r + 4 * (m ^ b)] = outv[m];
  wave_lds_sync();
  const int rslot = lane ^ (((lane >> 4) & 3) << 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (!ok[k]) continue;
    const uint4 v = lds_wave[64 * k + rslot];
    if (POL == kStoreNt) {
      store_nt(dst[k] + 16 * lane, v);
    } else {
      // dst[k] is wave-uniform, so the resource lives in scalar registers.
      // It spans exactly the 1 KiB row (stride 0, 1024 bytes; flags word:
      // 32-bit data format, the raw-buffer setting on this architecture).
      const __amdgpu_buffer_rsrc_t row =
          __builtin_amdgcn_make_buffer_rsrc(dst[k], 0, 1024, 0x00020000);
      const u32x4_t w = {v.x, v.y, v.z, v.w};
      __builtin_amdgcn_raw_buffer_store_b128(w, row, 16 * lane, 0, POL);
    }
  }
}

// e4m3 codes (chunk m in codes[2m], codes[2m+1]): each store writes one
// unit's 512 contiguous bytes.  8-byte granule G of unit q sits in LDS at
// G ^ ((((G >> 4) & 3) ^ (q & 1)) << 2), which keeps both the per-lane writes
// and the row reads free of bank conflicts.  Lanes 0..31 store units 0 and 2,
// lanes 32..63 units 1 and 3 (constant indices throughout, so the base
// pointers stay in scalar registers).  Unit k is stored when
// unit0 + k < units (a tail wave past the last unit stores nothing).  POL:
//   kStoreNt  - nontemporal stores (inv_rope_fp8_quant).  Timed with each
//               launch on buffers the previous launches have not touched, as
//               in a model, they beat plain stores by 6%.  Relaunched on the
//               same output, plain stores win instead: they overwrite lines
//               the last launch left in the last-level cache.
//   kStoreSc1 - the sc1 policy bit, through buffer stores on one resource
//               over the four rows, which must be consecutive 512-byte rows
//               from dst[0] (the q path's FP8 output): 2.2% faster there.
template <int POL>
__device__ __forceinline__ void store_rows_fp8(uint4* lds_wave, const uint32_t (&codes)[8],
                                               int lane, uint8_t* const (&dst)[4],
                                               uint32_t unit0, uint32_t units) {
  const int q = lane >> 4, L = lane & 15, blk = L >> 2, r = L & 3;
  wave_lds_sync();  // the transpose reads are done before the slice is reused
  uint2* lds8 = reinterpret_cast<uint2*>(lds_wave);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int G = 16 * blk + r + 4 * m;
    lds8[64 * q + (G ^ (((blk ^ (q & 1)) & 3) << 2))] = make_uint2(codes[2 * m], codes[2 * m + 1]);
  }
  wave_lds_sync();
  const int half = lane >> 5, j16 = lane & 31;
  const int G0 = 2 * j16;
  const int sw = (G0 >> 4) & 3;
  const uint4 c01 = *reinterpret_cast<const uint4*>(lds8 + 64 * half + (G0 ^ ((sw ^ half) << 2)));
  const uint4 c23 =
      *reinterpret_cast<const uint4*>(lds8 + 64 * (2 + half) + (G0 ^ ((sw ^ half) << 2)));
  if (POL == kStoreNt) {
    uint8_t* const base01 = half ? dst[1] : dst[0];
    uint8_t* const base23 = half ? dst[3] : dst[2];
    if (unit0 + half < units) store_nt(base01 + 16 * j16, c01);
    if (unit0 + 2 + half < units) store_nt(base23 + 16 * j16, c23);
  } else {
    // rows k at dst[0] + 512k; the resource spans the four (a tail wave's
    // missing rows are never written: the guards below)
    const __amdgpu_buffer_rsrc_t rows =
        __builtin_amdgcn_make_buffer_rsrc(dst[0], 0, 4 * kHeadDim, 0x00020000);
    const u32x4_t w01 = {c01.x, c01.y, c01.z, c01.w}, w23 = {c23.x, c23.y, c23.z, c23.w};
    if (unit0 + half < units)
      __builtin_amdgcn_raw_buffer_store_b128(w01, rows, kHeadDim * half + 16 * j16, 0, POL);
    if (unit0 + 2 + half < units)
      __builtin_amdgcn_raw_buffer_store_b128(w23, rows, kHeadDim * (2 + half) + 16 * j16, 0,
                                             POL);
  }
}

// Launch shape, filled in by the host: every params struct starts with it.
struct LaunchHdr {
  uint32_t wpb_log2;    // log2(waves per workgroup)
  uint32_t chunk_log2;  // log2(workgroups per XCD chunk)
};

// Wave index in the grid, made wave-uniform (so row addresses live in SGPRs).
__device__ __forceinline__ uint32_t wave_index(const LaunchHdr& h) {
  return __builtin_amdgcn_readfirstlane((xcd_block_id(h.chunk_log2) << h.wpb_log2) +
                                        (threadIdx.x >> 6));
}

// --------------------------------------------------------------- kernels

struct IrqParams {
  LaunchHdr hdr;
  const uint16_t* o;
  int64_t o_st, o_sh;
  const int64_t* positions;
  const float* cs;
  int64_t max_pos;
  uint32_t units;  // n_tokens * n_heads
  Magic div_heads, div_hpg;
  uint32_t n_heads, hpg;
  float eps;
  uint8_t* out;
  int64_t out_sg, out_st;
  void* scales;
  int64_t sc_sg, sc_st, sc_sb;
  uint32_t sc_vec4;  // FP32 scales of a head contiguous and 16-byte aligned
};

// Row q of the wave picks its value out of the four wave-uniform ones.
// (Two levels of selects on the bits of q; the four values are passed
// separately so they stay in registers.)
template <typename T>
__device__ __forceinline__ T pick_row(int q, T v0, T v1, T v2, T v3) {
  const bool odd = (q & 1) != 0, high = (q & 2) != 0;
  const T lo = odd ? v1 : v0;
  const T hi = odd ? v3 : v2;
  return high ? hi : lo;
}
#define PICK_ROW(q, a) pick_row((q), (a)[0], (a)[1], (a)[2], (a)[3])

// inv_rope_bf16: the rotation only, bf16 rows in inv_rope_fp8_quant's
// group-major places (quantization off).  Four units per wave, in the common
// structure: a 16-lane row per unit, its 32 dims per lane through the LDS
// transpose, the rows staged back through LDS for whole-row stores.  (The
// two-unit structure of irq_kernel below measured 0.5% slower here.)
__global__ __launch_bounds__(256) void irb_kernel(IrqParams p) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, L = lane & 15, r = L & 3;
  const uint32_t unit0 = wave_index(p.hdr) * 4u;
  uint4* lds_wave = lds + 256 * (threadIdx.x >> 6);
  // The wave's four units, all wave-uniform (scalar registers and loads).
  // A tail wave repeats its last unit in the missing slots: every read stays
  // inside the tensors, and slots without a unit store nothing.
  const uint16_t* rows[4];
  const float* csk[4];
  int64_t posk[4];
  uint32_t badk[4];
  uint8_t* outk[4];
  bool ok[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = min(unit0 + k, p.units - 1u);
    const uint32_t t = magic_div(u, p.div_heads);
    const uint32_t h = u - t * p.n_heads;
    const uint32_t g = magic_div(h, p.div_hpg);
    const uint32_t j = h - g * p.hpg;
    rows[k] = p.o + (int64_t)t * p.o_st + (int64_t)h * p.o_sh;
    posk[k] = load_uniform(p.positions + t);
    outk[k] = p.out + (int64_t)g * p.out_sg + (int64_t)t * p.out_st + (int64_t)j * 2 * kHeadDim;
    ok[k] = unit0 + k < p.units;
  }
  uint4 raw[4], w[4];
  issue_rows(rows, lane, raw);
  // (positions are used only after the row reads are on their way, so the
  // four scalar loads overlap them instead of running one after another)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool bad = posk[k] < 0 || posk[k] >= p.max_pos;
    badk[k] = bad;
    csk[k] = p.cs + (bad ? 0 : posk[k]) * 64;
  }
  // every lane reads its unit's cos/sin (cached; only lanes 12..15 use it):
  // unconditional loads keep the memory counters' order fixed
  RopeCS cs;
  load_cs(PICK_ROW(q, csk), r, cs);
  transpose_rows(lds_wave, raw, lane, w);

  Vals v;
  unpack_bf16(w, v);
  if (L >= 12) rope_lane<true>(v, cs);
  // a unit whose position is outside the table is written as NaN
  uint4 outv[4];
  pack_bf16(v, outv);
  if (PICK_ROW(q, badk) != 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      outv[k] = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  }
  store_rows_bf16<kStoreNt>(lds_wave, outv, lane, outk, ok);
}

// inv_rope_fp8_quant, two units per wave: lanes 32h .. 32h+31 work on unit h
// of the wave.  Within a half, lane L = 8b + r holds the 8-dim chunks 16b + r
// and 16b + 8 + r of its unit, so quant block b is the aligned 8-lane group
// b (three DPP steps for its maximum) and the rotated dims 448..511 are the
// second chunks of group 3, one chunk (4 GPT-J pairs, 4r .. 4r+3) per lane.
// Each unit's 1 KiB row is read by one 16-byte-per-lane load and reaches
// those lanes through the wave's 2 KiB of LDS; 16-byte slot s sits at
// s ^ (((s >> 4) & 1) << 3), and 8-byte code granule G at
// G ^ (((G >> 5) & 1) << 3), which keeps every LDS access free of bank
// conflicts.  One store instruction writes both units' 512-byte code rows
// (lanes 0..31 unit 0, 32..63 unit 1).
//
// Why two units per wave: the same bytes streamed with no arithmetic took
// 120.9 us with 2 KiB per wave against 126.0 us with 4 KiB for the 16384 x 32
// workload on MI355X.  The four-unit form of this kernel (a 16-lane row per
// unit) ran at the latter; this one, in 256-thread workgroups dealt to the
// XCDs in chunks of 64, runs at 122.5-123.0 us, and 2-3% faster on the
// irregular and larger launches.  Waves of one unit, or two in a layout
// without the transpose, were slower than both: their rotation and scale
// work falls on fewer lanes.
template <int FMT>
__global__ __launch_bounds__(256) void irq_kernel(IrqParams p) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, L = lane & 31, b = L >> 3, r = L & 7;
  const uint32_t unit0 = wave_index(p.hdr) * 2u;
  uint4* lds_wave = lds + 128 * (threadIdx.x >> 6);
  const uint16_t* rows[2];
  const float* csk[2];
  int64_t posk[2];
  uint32_t badk[2];
  uint8_t* outk[2];
  uint8_t* sck[2];
  bool ok[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t u = min(unit0 + k, p.units - 1u);
    const uint32_t t = magic_div(u, p.div_heads);
    const uint32_t hh = u - t * p.n_heads;
    const uint32_t g = magic_div(hh, p.div_hpg);
    const uint32_t j = hh - g * p.hpg;
    rows[k] = p.o + (int64_t)t * p.o_st + (int64_t)hh * p.o_sh;
    posk[k] = load_uniform(p.positions + t);
    outk[k] = p.out + (int64_t)g * p.out_sg + (int64_t)t * p.out_st + (int64_t)j * kHeadDim;
    const int64_t first = (int64_t)g * p.sc_sg + (int64_t)t * p.sc_st +
                          (int64_t)(FMT == RQ_SCALE_UE8M0 ? j : 4 * j) * p.sc_sb;
    sck[k] = static_cast<uint8_t*>(p.scales) + 4 * first;
    ok[k] = unit0 + k < p.units;
  }
  uint4 raw[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) raw[k] = load_nt(reinterpret_cast<const uint4*>(rows[k]) + lane);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bool bad = posk[k] < 0 || posk[k] >= p.max_pos;
    badk[k] = bad;
    csk[k] = p.cs + (bad ? 0 : posk[k]) * 64;
  }
  // cos / sin of the lane's 4 pairs 4r .. 4r+3 (used by group 3 only; read
  // by every lane, cached)
  const float4* csrow = reinterpret_cast<const float4*>(h ? csk[1] : csk[0]);
  const float4 c4 = csrow[r], s4 = csrow[8 + r];
  const bool row_bad = (h ? badk[1] : badk[0]) != 0;

  // transpose: slot s of unit k at 64k + (s ^ (((s >> 4) & 1) << 3))
#pragma unroll
  for (int k = 0; k < 2; ++k) lds_wave[64 * k + (lane ^ (((lane >> 4) & 1) << 3))] = raw[k];
  wave_lds_sync();
  const int c0 = 16 * b + r, c1 = 16 * b + 8 + r;
  const uint4 w0 = lds_wave[64 * h + (c0 ^ (((c0 >> 4) & 1) << 3))];
  const uint4 w1 = lds_wave[64 * h + (c1 ^ (((c1 >> 4) & 1) << 3))];

  float x[2][8];
  {
    const uint32_t d0[4] = {w0.x, w0.y, w0.z, w0.w}, d1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[0][2 * i] = bf_lo(d0[i]);
      x[0][2 * i + 1] = bf_hi(d0[i]);
      x[1][2 * i] = bf_lo(d1[i]);
      x[1][2 * i + 1] = bf_hi(d1[i]);
    }
  }
  if (b == 3) {
    // inverse GPT-J rotation ([P4] section 2): e' = e*c + o*s, o' = o*c - e*s
    const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = x[1][2 * i], o = x[1][2 * i + 1];
      const float ec = e * cv[i], os = o * sv[i], oc = o * cv[i], es = e * sv[i];
      x[1][2 * i] = ec + os;
      x[1][2 * i + 1] = oc - es;
    }
  }
  wave_lds_sync();  // the transpose reads are done before the slice is reused

  {
    // block amax over the 8-lane group ([P4] section 3)
    float m = 0.0f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(x[cc][e]));
    m = max_dpp_nonneg<kQuadSwap1>(m);
    m = max_dpp_nonneg<kQuadSwap2>(m);
    m = max_dpp_nonneg<kRowHalfMirror>(m);
    float scale, mult;
    uint32_t ebyte;
    block_scale<FMT>(m, p.eps, scale, mult, ebyte);
    // No clamp before the convert: |x * mult| <= 448 * (1 + 2^-24)^3, and
    // the convert rounds to nearest even, giving 448 up to 464.
    uint2* lds8 = reinterpret_cast<uint2*>(lds_wave);
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      uint32_t code[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float q0 = x[cc][4 * hf] * mult, q1 = x[cc][4 * hf + 1] * mult;
        const float q2 = x[cc][4 * hf + 2] * mult, q3 = x[cc][4 * hf + 3] * mult;
        // bytes 2..3 of the first convert are overwritten by the second
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, __builtin_bit_cast(int, q0), false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, wd, true);
        code[hf] = (uint32_t)wd;
      }
      const int G = cc ? c1 : c0;  // 8-byte granule of the unit's code row
      lds8[64 * h + (G ^ (((G >> 5) & 1) << 3))] = make_uint2(code[0], code[1]);
    }

    // scales.  A unit whose position is outside the table gets NaN scales.
    // Block b's value is uniform over group b.  Lane 32h gathers its unit's
    // four (group 1 through a DPP row shift, groups 2 and 3 from lane
    // 32h + 16 through ds_bpermute) and writes them with one 16-byte store
    // when they are contiguous and aligned; else the first lane of each
    // group writes its own (MN-major layouts).
    uint8_t* const sc = h ? sck[1] : sck[0];
    const bool sc_ok = h ? ok[1] : ok[0];
    if (FMT == RQ_SCALE_UE8M0) {
      uint32_t wd = ebyte << (8 * b);
      wd |= dpp_u32<kRowMirror>(wd);  // the row's other group
      const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane + 16) & 63), (int)wd);
      if (L == 0 && sc_ok) *reinterpret_cast<uint32_t*>(sc) = row_bad ? 0xFFFFFFFFu : (wd | hi);
    } else {
      const float sv = row_bad ? __builtin_nanf("") : scale;
      if (p.sc_vec4) {
        const uint32_t s0 = __builtin_bit_cast(uint32_t, sv);
        const uint32_t s1 = dpp_u32<kRowShl8>(s0);
        const uint32_t s2 = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane + 16) & 63), (int)s0);
        const uint32_t s3 = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane + 16) & 63), (int)s1);
        if (L == 0 && sc_ok) *reinterpret_cast<uint4*>(sc) = make_uint4(s0, s1, s2, s3);
      } else if (r == 0 && sc_ok) {
        reinterpret_cast<float*>(sc)[(int64_t)b * p.sc_sb] = sv;
      }
    }
    wave_lds_sync();
    // codes: lane (h, j) stores bytes 16j .. 16j+15 of unit h's row; one
    // instruction writes both units' rows (two half-wave stores through
    // scalar bases measured 1.2% slower)
    const int G0 = 2 * L;
    const uint4 cw = *reinterpret_cast<const uint4*>(lds8 + 64 * h + (G0 ^ (((G0 >> 5) & 1) << 3)));
    if (h ? ok[1] : ok[0]) store_nt((h ? outk[1] : outk[0]) + 16 * L, cw);
  }
}

// inv_rope_fp8_quant for a few tokens: one head per wave, so that a wave's
// own instruction latency, which sets the time of a call this small, covers
// one head instead of two.  Lane l holds dims 8l .. 8l+7 (one 16-byte load,
// no LDS); quant block b is the lanes of DPP row b, its maximum four DPP
// steps; the rotated dims 448..511 are lanes 56..63, GPT-J pairs
// 4(l - 56) .. 4(l - 56) + 3.  Every value is computed by irq_kernel's
// operations in its order (inverse rotation [P4] section 2, block scale and
// codes [P4] section 3), so both kernels write the same bits.  Lane l stores
// codes 8l .. 8l+7 of the head's row; the first lane gathers the four block
// scales (readlane) and stores them as irq_kernel does.
template <int FMT>
__global__ __launch_bounds__(256) void irq1_kernel(IrqParams p) {
  const int lane = threadIdx.x & 63;
  const uint32_t u =
      __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
  if (u >= p.units) return;
  const uint32_t t = magic_div(u, p.div_heads);
  const uint32_t hh = u - t * p.n_heads;
  const uint32_t g = magic_div(hh, p.div_hpg);
  const uint32_t j = hh - g * p.hpg;
  const int64_t pos = load_uniform(p.positions + t);
  const uint4 raw =
      reinterpret_cast<const uint4*>(p.o + (int64_t)t * p.o_st + (int64_t)hh * p.o_sh)[lane];
  const bool bad = pos < 0 || pos >= p.max_pos;
  // cos / sin of the lane's pairs (lanes 56..63; the others read a row they
  // do not use)
  const float4* csrow = reinterpret_cast<const float4*>(p.cs + (bad ? 0 : pos) * 64);
  const int pr = lane >= 56 ? lane - 56 : (lane & 7);
  const float4 c4 = csrow[pr], s4 = csrow[8 + pr];
  float x[8];
  const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf_lo(d[i]);
    x[2 * i + 1] = bf_hi(d[i]);
  }
  if (lane >= 56) {  // inverse GPT-J rotation: e' = e*c + o*s, o' = o*c - e*s
    const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = x[2 * i], o = x[2 * i + 1];
      const float ec = e * cv[i], os = o * sv[i], oc = o * cv[i], es = e * sv[i];
      x[2 * i] = ec + os;
      x[2 * i + 1] = oc - es;
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(x[e]));
  m = max_dpp_nonneg<kQuadSwap1>(m);
  m = max_dpp_nonneg<kQuadSwap2>(m);
  m = max_dpp_nonneg<kRowHalfMirror>(m);
  m = max_dpp_nonneg<kRowMirror>(m);
  float scale, mult;
  uint32_t ebyte;
  block_scale<FMT>(m, p.eps, scale, mult, ebyte);
  uint32_t code[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float q0 = x[4 * hf] * mult, q1 = x[4 * hf + 1] * mult;
    const float q2 = x[4 * hf + 2] * mult, q3 = x[4 * hf + 3] * mult;
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, __builtin_bit_cast(int, q0), false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, wd, true);
    code[hf] = (uint32_t)wd;
  }
  uint8_t* const row = p.out + (int64_t)g * p.out_sg + (int64_t)t * p.out_st + (int64_t)j * kHeadDim;
  reinterpret_cast<uint2*>(row)[lane] = make_uint2(code[0], code[1]);
  // scales of the head; a position outside the table gives NaN scales
  const int64_t first = (int64_t)g * p.sc_sg + (int64_t)t * p.sc_st +
                        (int64_t)(FMT == RQ_SCALE_UE8M0 ? j : 4 * j) * p.sc_sb;
  uint8_t* const sc = static_cast<uint8_t*>(p.scales) + 4 * first;
  if (FMT == RQ_SCALE_UE8M0) {
    const uint32_t wd = ebyte << (8 * (lane >> 4));
    const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)wd, 0) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wd, 16) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wd, 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wd, 48);
    if (lane == 0) *reinterpret_cast<uint32_t*>(sc) = bad ? 0xFFFFFFFFu : word;
  } else {
    const float sv = bad ? __builtin_nanf("") : scale;
    if (p.sc_vec4) {
      const int sb = __builtin_bit_cast(int, sv);
      const uint4 s4v = make_uint4((uint32_t)__builtin_amdgcn_readlane(sb, 0),
                                   (uint32_t)__builtin_amdgcn_readlane(sb, 16),
                                   (uint32_t)__builtin_amdgcn_readlane(sb, 32),
                                   (uint32_t)__builtin_amdgcn_readlane(sb, 48));
      if (lane == 0) *reinterpret_cast<uint4*>(sc) = s4v;
    } else if ((lane & 15) == 0) {
      reinterpret_cast<float*>(sc)[(int64_t)(lane >> 4) * p.sc_sb] = sv;
    }
  }
}

struct QnrParams {
  LaunchHdr hdr;
  const uint16_t* q;
  int64_t q_st, q_sh;
  const uint16_t* weight;
  const int64_t* positions;
  const float* cs;
  int64_t max_pos;
  uint32_t units;  // n_tokens * q_head_padded
  Magic div_hpad;
  uint32_t hq, hpad;
  float eps;
  uint16_t* q_out;   // bf16 form: [N, Hpad, 512]
  uint8_t* q_fp8;    // FP8 form: codes [N, Hpad, 512] ...
  void* q_scales;    // ... and scales [N, Hpad, 4] fp32 or [N, Hpad] UE8M0 words
  float quant_eps;
  float pad_scale;     // a zero head's block scale: quant_eps / 448, or its UE8M0 power of two
  uint32_t pad_ebyte;  // a zero head's UE8M0 exponent byte
};

// RMSNorm of the lane's row ([P3] section 5), v <- (v * r) * w, in two
// steps.  rms_inv: r = 1 / sqrt(mean(v^2) + eps), the sum of squares by
// pairwise summation over the 512 dims (recursive halving: each half-range's
// sum added to the other's, down to single squares).  Every level of that
// tree is a pairing the lane layout already holds: dims 8c .. 8c+7 of chunk
// c = 16b + 4k + r sit in one lane (levels 1-3, in registers); chunks c and
// c^1, c^2 are lanes r^1, r^2 of the quad (levels 4-5, DPP); c^4, c^8 are
// this lane's k^1, k^2 (levels 6-7); c^16, c^32 the quads b^1, b^2 (levels
// 8-9, DPP).  Each lane ends with the same bits, as fp32 addition commutes.
__device__ __forceinline__ float rms_inv(const Vals& v, float eps) {
  float ps[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float sq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] = v.x[k][e] * v.x[k][e];
    ps[k] = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) ps[k] = ps[k] + dpp_f32<kQuadSwap1>(ps[k]);
#pragma unroll
  for (int k = 0; k < 4; ++k) ps[k] = ps[k] + dpp_f32<kQuadSwap2>(ps[k]);
  float ss = (ps[0] + ps[1]) + (ps[2] + ps[3]);
  ss = ss + dpp_f32<kRowHalfMirror>(ss);
  ss = ss + dpp_f32<kRowMirror>(ss);
  const float mean = ss * (1.0f / 512.0f);
  // 1 / sqrt, each correctly rounded: sqrtf is the compiler's exact square
  // root; the reciprocal of its result (a normal below 2^64, as the argument
  // is at least the smallest positive fp32) is recip_scale, exact there
  return recip_scale(sqrtf(mean + eps));
}

// v <- (v * rs) * w with the lane's weight chunks already in registers
// (HAS_WEIGHT), or v <- v * rs.
template <bool HAS_WEIGHT>
__device__ __forceinline__ void rmsnorm_lane(Vals& v, const uint4 (&wt)[4], float eps) {
  const float rs = rms_inv(v, eps);
  if (HAS_WEIGHT) {
    Vals wv;
    unpack_bf16(wt, wv);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) v.x[k][e] = (v.x[k][e] * rs) * wv.x[k][e];
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) v.x[k][e] = v.x[k][e] * rs;
  }
}

// The same, reading the lane's weight chunks (cached) only here, pair by pair:
// fewer registers live across the kernel, for the heavier FP8 form.
template <bool HAS_WEIGHT>
__device__ __forceinline__ void rmsnorm_lane_late_weight(Vals& v, const uint16_t* wrow,
                                                         float eps) {
  const float rs = rms_inv(v, eps);
  if (HAS_WEIGHT) {
    const uint4* wp = reinterpret_cast<const uint4*>(wrow);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint4 wk = wp[4 * k];
      const uint32_t d[4] = {wk.x, wk.y, wk.z, wk.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v.x[k][2 * i] = (v.x[k][2 * i] * rs) * bf_lo(d[i]);
        v.x[k][2 * i + 1] = (v.x[k][2 * i + 1] * rs) * bf_hi(d[i]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) v.x[k][e] = v.x[k][e] * rs;
  }
}

// The wave with grid-wide index `wave` handles units 4*wave .. 4*wave+3.
// OUT: kOutBf16 (q_out) or RQ_SCALE_FP32 / RQ_SCALE_UE8M0 (q_fp8 + q_scales).
template <bool HAS_WEIGHT, int OUT>
__device__ __forceinline__ void qnr_body(const QnrParams& p, uint32_t wave, uint4* lds_wave) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, L = lane & 15;
  const uint32_t unit0 = wave * 4u;
  const uint16_t* rows[4];
  uint32_t livek[4];
  int64_t posk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t u = min(unit0 + k, p.units - 1u);
    const uint32_t t = magic_div(u, p.div_hpad);
    const uint32_t h = u - t * p.hpad;
    livek[k] = (unit0 + k < p.units && h < p.hq) ? 1u : 0u;
    rows[k] = p.q + (int64_t)t * p.q_st + (int64_t)min(h, p.hq - 1u) * p.q_sh;
    posk[k] = load_uniform(p.positions + t);
  }
  // A wave of pad heads only reads nothing (its rows in LDS are never used).
  uint4 raw[4] = {}, w[4];
  if (livek[0] | livek[1] | livek[2] | livek[3]) issue_rows(rows, lane, raw);

  const bool live = PICK_ROW(q, livek) != 0;
  const int64_t pos = PICK_ROW(q, posk);
  const bool bad = pos < 0 || pos >= p.max_pos;
  const bool rope = L >= 12;
  const int d0 = lane_dim0(L);
  // bf16 form: weight and cos/sin are read by every lane (cached) before the
  // transpose, so their latency hides behind it (unconditional loads keep the
  // memory counters' order fixed).  The FP8 form, which holds more registers,
  // reads them where they are used: it measured faster with the higher
  // occupancy that buys, the bf16 form slower.
  const float* csrow = p.cs + (bad ? 0 : pos) * 64;
  uint4 wt[4];
  RopeCS cs;
  if constexpr (OUT == kOutBf16) {
    if (HAS_WEIGHT) {
      const uint4* wp = reinterpret_cast<const uint4*>(p.weight + d0);
#pragma unroll
      for (int k = 0; k < 4; ++k) wt[k] = wp[4 * k];
    }
    load_cs(csrow, L & 3, cs);
  }
  transpose_rows(lds_wave, raw, lane, w);

  uint8_t* dst[4];
  bool ok[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ok[k] = unit0 + k < p.units;
    dst[k] = OUT == kOutBf16
                 ? reinterpret_cast<uint8_t*>(p.q_out + (int64_t)(unit0 + k) * kHeadDim)
                 : p.q_fp8 + (int64_t)(unit0 + k) * kHeadDim;
  }

  if constexpr (OUT == kOutBf16) {
    uint4 outv[4];
    if (live) {
      Vals v;
      unpack_bf16(w, v);
      rmsnorm_lane<HAS_WEIGHT>(v, wt, p.eps);
      if (rope) rope_lane<false>(v, cs);
      pack_bf16(v, outv);
      if (bad) {  // position outside the table: the head is written as NaN
#pragma unroll
        for (int k = 0; k < 4; ++k)
          outv[k] = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
      }
    } else {  // pad head (or no unit): exact +0 ([P1] section 1)
#pragma unroll
      for (int k = 0; k < 4; ++k) outv[k] = make_uint4(0u, 0u, 0u, 0u);
    }
    store_rows_bf16<kStoreSc1>(lds_wave, outv, lane, dst, ok);
  } else {
    // A pad head is a zero head, quantized like any other: codes +0 and the
    // scales of a block whose amax is quant_eps, which the host computed with
    // the same fp32 operations.  Only live heads run the arithmetic.
    float scale = p.pad_scale;
    uint32_t ebyte = p.pad_ebyte, codes[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if (live) {
      Vals v;
      unpack_bf16(w, v);
      rmsnorm_lane_late_weight<HAS_WEIGHT>(v, HAS_WEIGHT ? p.weight + d0 : nullptr, p.eps);
      load_cs(csrow, L & 3, cs);
      if (rope) rope_lane<false>(v, cs);
      quantize_lane<OUT>(v, p.quant_eps, scale, ebyte, codes);
    }
    // scales of unit u at u*4 floats (FP32) or word u (UE8M0); a live head of
    // a token whose position is outside the table gets NaN scales
    if (unit0 + q < p.units) {
      const bool poison = live && bad;
      const int64_t u = unit0 + q;
      const int blk = L >> 2;
      if (OUT == RQ_SCALE_UE8M0) {
        const uint32_t word = pack_ue8m0(ebyte, blk);
        if (L == 0) static_cast<uint32_t*>(p.q_scales)[u] = poison ? 0xFFFFFFFFu : word;
      } else if ((L & 3) == 0) {
        static_cast<float*>(p.q_scales)[4 * u + blk] = poison ? __builtin_nanf("") : scale;
      }
    }
    store_rows_fp8<kStoreSc1>(lds_wave, codes, lane, dst, unit0, p.units);
  }
}

template <bool HAS_WEIGHT, int OUT>
__global__ __launch_bounds__(256) void qnr_kernel(QnrParams p) {
  extern __shared__ uint4 lds[];
  qnr_body<HAS_WEIGHT, OUT>(p, wave_index(p.hdr), lds + 256 * (threadIdx.x >> 6));
}

// qnorm_rope (bf16 q_out) for a few tokens: one head per wave, so that a
// wave's own instruction latency, which sets the time of a call this small,
// covers one head instead of four (108 VALU instructions per wave against
// qnr_kernel's 387).  Lane l holds dims 8l .. 8l+7, read by one 16-byte load
// and written by one 16-byte store: no LDS.  The sum of squares is the same
// pairwise tree as rms_inv's: dims 8l .. 8l+7 in the lane (levels 1-3), then
// lanes l ^ 1, l ^ 2 (quad DPP), the row halves and rows of 16 (row mirrors,
// on values already uniform over the quads and halves), then l ^ 16 and
// l ^ 32 (ds_bpermute); every lane ends with the same bits.  The rotated dims
// 448..511 are lanes 56..63, GPT-J pairs 4(l - 56) .. 4(l - 56) + 3.  Every
// other operation is qnr_body's, in its order, so the two kernels write the
// same bits ([P3] section 5 RMSNorm, then forward RoPE, bf16 RNE; pad heads
// +0 [P1] section 1).
template <bool HAS_WEIGHT>
__device__ __forceinline__ void qnr1_body(const QnrParams& p, uint32_t u) {
  const int lane = threadIdx.x & 63;
  const uint32_t t = magic_div(u, p.div_hpad);
  const uint32_t h = u - t * p.hpad;
  uint4 outw = make_uint4(0u, 0u, 0u, 0u);  // pad head: +0
  if (h < p.hq) {
    const int64_t pos = load_uniform(p.positions + t);
    const uint4 raw =
        reinterpret_cast<const uint4*>(p.q + (int64_t)t * p.q_st + (int64_t)h * p.q_sh)[lane];
    uint4 wt = make_uint4(0u, 0u, 0u, 0u);
    if (HAS_WEIGHT) wt = reinterpret_cast<const uint4*>(p.weight)[lane];
    const bool bad = pos < 0 || pos >= p.max_pos;
    // cos / sin of the lane's pairs (lanes 56..63; the others read a row
    // they do not use)
    const float4* csrow = reinterpret_cast<const float4*>(p.cs + (bad ? 0 : pos) * 64);
    const int pr = lane >= 56 ? lane - 56 : (lane & 7);
    const float4 c4 = csrow[pr], s4 = csrow[8 + pr];
    float x[8];
    const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf_lo(d[i]);
      x[2 * i + 1] = bf_hi(d[i]);
    }
    float sq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sq[e] = x[e] * x[e];
    float ss = ((sq[0] + sq[1]) + (sq[2] + sq[3])) + ((sq[4] + sq[5]) + (sq[6] + sq[7]));
    ss = ss + dpp_f32<kQuadSwap1>(ss);
    ss = ss + dpp_f32<kQuadSwap2>(ss);
    ss = ss + dpp_f32<kRowHalfMirror>(ss);
    ss = ss + dpp_f32<kRowMirror>(ss);
    ss = ss + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                            4 * (lane ^ 16), __builtin_bit_cast(int, ss)));
    ss = ss + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                            4 * (lane ^ 32), __builtin_bit_cast(int, ss)));
    const float mean = ss * (1.0f / 512.0f);
    const float rs = recip_scale(sqrtf(mean + p.eps));  // as rms_inv
    if (HAS_WEIGHT) {
      const uint32_t wd[4] = {wt.x, wt.y, wt.z, wt.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = (x[2 * i] * rs) * bf_lo(wd[i]);
        x[2 * i + 1] = (x[2 * i + 1] * rs) * bf_hi(wd[i]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = x[e] * rs;
    }
    if (lane >= 56) {  // forward GPT-J rotation, as rope_lane<false>
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = x[2 * i], o = x[2 * i + 1];
        const float ec = e * cv[i], os = o * sv[i], oc = o * cv[i], es = e * sv[i];
        x[2 * i] = ec - os;
        x[2 * i + 1] = oc + es;
      }
    }
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    uint32_t o4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 f = {x[2 * i], x[2 * i + 1]};
      o4[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
    }
    // a position outside the table: the head is written as NaN
    outw = bad ? make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u)
               : make_uint4(o4[0], o4[1], o4[2], o4[3]);
  }
  reinterpret_cast<uint4*>(p.q_out + (int64_t)u * kHeadDim)[lane] = outw;
}

// Wave index of the one-head-per-wave kernels (no XCD dealing: their
// launches are a few hundred waves), made wave-uniform.
__device__ __forceinline__ uint32_t flat_wave_index() {
  return __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
}

template <bool HAS_WEIGHT>
__global__ __launch_bounds__(256) void qnr1_kernel(QnrParams p) {
  const uint32_t u = flat_wave_index();
  if (u < p.units) qnr1_body<HAS_WEIGHT>(p, u);
}

struct KviParams {
  LaunchHdr hdr;
  const uint16_t* kv;
  int64_t kv_st;
  const int64_t* positions;
  const float* cs;
  int64_t max_pos;
  const int64_t* slots;
  uint32_t n_tokens;
  int64_t num_slots;
  Magic div_bs;
  uint32_t bs;
  uint8_t* cache;
  int64_t block_stride;  // bytes: between blocks (records), or between rows (bf16 cache)
  float eps;
};

// kv_rope_insert_full and the full-cache fused forms: the wave with
// grid-wide index `wave` rotates tokens 4*wave .. 4*wave+3 and writes each as
// a bf16 row of the token-strided cache (slot s at cache + s * block_stride
// bytes).  Two tokens per wave measured slower here from 8192 tokens on.
__device__ __forceinline__ void kvf_body(const KviParams& p, uint32_t wave, uint4* lds_wave) {
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, L = lane & 15, r = L & 3;
  const uint32_t t0 = wave * 4u;
  const uint16_t* rows[4];
  const float* csk[4];
  int64_t posk[4];
  uint32_t badk[4];
  uint8_t* reck[4];  // the token's row, or nullptr: nothing to write
  int64_t slotk[4];
  // The slot and position loads are issued first and the row reads right
  // after, with nothing in between that waits for the former (the scheduling
  // barriers keep it so); the cos/sin reads, which need the positions, go out
  // before the slot arithmetic.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t t = min(t0 + k, p.n_tokens - 1u);
    rows[k] = p.kv + (int64_t)t * p.kv_st;
    slotk[k] = load_uniform(p.slots + t);
    posk[k] = load_uniform(p.positions + t);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 raw[4], w[4];
  issue_rows(rows, lane, raw);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool bad = posk[k] < 0 || posk[k] >= p.max_pos;
    badk[k] = bad;
    csk[k] = p.cs + (bad ? 0 : posk[k]) * 64;
  }
  RopeCS cs;
  load_cs(PICK_ROW(q, csk), r, cs);  // every lane, unconditionally (cached)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (t0 + k >= p.n_tokens) slotk[k] = -1;
    // else: padding token, or no such slot
    reck[k] = slotk[k] >= 0 && slotk[k] < p.num_slots ? p.cache + slotk[k] * p.block_stride
                                                       : nullptr;
  }
  transpose_rows(lds_wave, raw, lane, w);

  Vals v;
  unpack_bf16(w, v);
  if (L >= 12) rope_lane<false>(v, cs);
  uint4 outv[4];
  pack_bf16(v, outv);
  if (PICK_ROW(q, badk) != 0) {  // position outside the table: a NaN row
#pragma unroll
    for (int k = 0; k < 4; ++k)
      outv[k] = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  }
  bool ok[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) ok[k] = reck[k] != nullptr;
  store_rows_bf16<kStoreNt>(lds_wave, outv, lane, reck, ok);
}

__global__ __launch_bounds__(256) void kvf_kernel(KviParams p) {
  extern __shared__ uint4 lds[];
  kvf_body(p, wave_index(p.hdr), lds + 256 * (threadIdx.x >> 6));
}

// kv_rope_quant_insert standalone, two tokens per wave: the lane layout of
// irq_kernel (token h on lanes 32h .. 32h+31, lane 8b + r holding chunks
// 16b + r and 16b + 8 + r, quant block b on 8-lane group b), the forward
// rotation, and each token's 528-byte record written as 33 16-byte granules:
// the codes by lanes 32h .. 32h+31 through LDS, the scale tail by lane 32h.
// With four tokens per wave these launches ran 2-7% slower.  The fused kernel
// runs the same body for its kv waves.  NT: the record stores are
// nontemporal.  Records land at the caller's slots, scattered over the
// cache, and share their first and last 128-byte lines with records written
// at other times or not at all; from 4096 tokens on, nontemporal stores
// measured 7-20% faster, below that plain ones up to 4% faster (the host
// picks by token count).
template <int FMT, bool NT>
__device__ __forceinline__ void kvi2_body(const KviParams& p, uint32_t wave, uint4* lds_wave) {
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, L = lane & 31, b = L >> 3, r = L & 7;
  const uint32_t t0 = wave * 2u;
  const uint16_t* rows[2];
  const float* csk[2];
  int64_t posk[2], slotk[2];
  uint32_t badk[2];
  uint8_t* reck[2];  // the token's record, or nullptr: nothing to write
  // load order as in kvf_body: slots and positions, rows, then cos/sin
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t t = min(t0 + k, p.n_tokens - 1u);
    rows[k] = p.kv + (int64_t)t * p.kv_st;
    slotk[k] = load_uniform(p.slots + t);
    posk[k] = load_uniform(p.positions + t);
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 raw[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) raw[k] = load_nt(reinterpret_cast<const uint4*>(rows[k]) + lane);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const bool bad = posk[k] < 0 || posk[k] >= p.max_pos;
    badk[k] = bad;
    csk[k] = p.cs + (bad ? 0 : posk[k]) * 64;
  }
  const float4* csrow = reinterpret_cast<const float4*>(h ? csk[1] : csk[0]);
  const float4 c4 = csrow[r], s4 = csrow[8 + r];
  const bool row_bad = (h ? badk[1] : badk[0]) != 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    if (t0 + k >= p.n_tokens) slotk[k] = -1;
    reck[k] = nullptr;
    if (slotk[k] >= 0 && slotk[k] < p.num_slots) {  // else: padding token, or no such slot
      const uint32_t blk_i = magic_div((uint32_t)slotk[k], p.div_bs);
      const uint32_t idx = (uint32_t)slotk[k] - blk_i * p.bs;
      reck[k] = p.cache + (int64_t)blk_i * p.block_stride + (int64_t)idx * kRecordBytes;
    }
  }

  // transpose: slot s of token k at 64k + (s ^ (((s >> 4) & 1) << 3))
#pragma unroll
  for (int k = 0; k < 2; ++k) lds_wave[64 * k + (lane ^ (((lane >> 4) & 1) << 3))] = raw[k];
  wave_lds_sync();
  const int c0 = 16 * b + r, c1 = 16 * b + 8 + r;
  const uint4 w0 = lds_wave[64 * h + (c0 ^ (((c0 >> 4) & 1) << 3))];
  const uint4 w1 = lds_wave[64 * h + (c1 ^ (((c1 >> 4) & 1) << 3))];
  float x[2][8];
  {
    const uint32_t d0[4] = {w0.x, w0.y, w0.z, w0.w}, d1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[0][2 * i] = bf_lo(d0[i]);
      x[0][2 * i + 1] = bf_hi(d0[i]);
      x[1][2 * i] = bf_lo(d1[i]);
      x[1][2 * i + 1] = bf_hi(d1[i]);
    }
  }
  if (b == 3) {
    // forward GPT-J rotation: e' = e*c - o*s, o' = o*c + e*s
    const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = x[1][2 * i], o = x[1][2 * i + 1];
      const float ec = e * cv[i], os = o * sv[i], oc = o * cv[i], es = e * sv[i];
      x[1][2 * i] = ec - os;
      x[1][2 * i + 1] = oc + es;
    }
  }
  wave_lds_sync();  // the transpose reads are done before the slice is reused
  float m = 0.0f;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(x[cc][e]));
  m = max_dpp_nonneg<kQuadSwap1>(m);
  m = max_dpp_nonneg<kQuadSwap2>(m);
  m = max_dpp_nonneg<kRowHalfMirror>(m);
  float scale, mult;
  uint32_t ebyte;
  block_scale<FMT>(m, p.eps, scale, mult, ebyte);
  uint2* lds8 = reinterpret_cast<uint2*>(lds_wave);
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    uint32_t code[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float q0 = x[cc][4 * hf] * mult, q1 = x[cc][4 * hf + 1] * mult;
      const float q2 = x[cc][4 * hf + 2] * mult, q3 = x[cc][4 * hf + 3] * mult;
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, __builtin_bit_cast(int, q0), false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, wd, true);
      code[hf] = (uint32_t)wd;
    }
    const int G = cc ? c1 : c0;
    lds8[64 * h + (G ^ (((G >> 5) & 1) << 3))] = make_uint2(code[0], code[1]);
  }
  // the record's scale tail, gathered into lane 32h (a token whose position
  // is outside the table gets NaN scales)
  uint4 tail;
  if (FMT == RQ_SCALE_UE8M0) {
    uint32_t wd = ebyte << (8 * b);
    wd |= dpp_u32<kRowMirror>(wd);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane + 16) & 63), (int)wd);
    tail = make_uint4(row_bad ? 0xFFFFFFFFu : (wd | hi), 0u, 0u, 0u);
  } else {
    const uint32_t s0 = row_bad ? 0x7FC00000u : __builtin_bit_cast(uint32_t, scale);
    const uint32_t s1 = dpp_u32<kRowShl8>(s0);
    const uint32_t s2 = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane + 16) & 63), (int)s0);
    const uint32_t s3 = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * ((lane + 16) & 63), (int)s1);
    tail = make_uint4(s0, s1, s2, s3);
  }
  wave_lds_sync();
  const int G0 = 2 * L;
  const uint4 cw = *reinterpret_cast<const uint4*>(lds8 + 64 * h + (G0 ^ (((G0 >> 5) & 1) << 3)));
  uint8_t* const rec = h ? reck[1] : reck[0];
  if (rec) {
    if (NT) {
      store_nt(rec + 16 * L, cw);
      if (L == 0) store_nt(rec + kHeadDim, tail);
    } else {
      *reinterpret_cast<uint4*>(rec + 16 * L) = cw;
      if (L == 0) *reinterpret_cast<uint4*>(rec + kHeadDim) = tail;
    }
  }
}

template <int FMT, bool NT>
__global__ __launch_bounds__(256) void kvi2_kernel(KviParams p) {
  extern __shared__ uint4 lds[];
  kvi2_body<FMT, NT>(p, wave_index(p.hdr), lds + 128 * (threadIdx.x >> 6));
}

// kv_rope_quant_insert for a few tokens: one token per wave, the layout of
// irq1_kernel (lane l holds dims 8l .. 8l+7, quant block b = DPP row b, the
// rotated dims on lanes 56..63) with kvi2_body's operations in its order:
// forward RoPE, block scale and codes ([P4] sections 2-3), and the 528-byte
// record at the token's slot [P1] section 1 (codes 8l .. 8l+7 from lane l,
// the 16-byte scale tail from the first lane; plain stores: a decode step
// reads the cache right after).  A slot outside the cache, or negative,
// writes nothing; a position outside the table gives NaN scales.
template <int FMT>
__device__ __forceinline__ void kvi1_body(const KviParams& p, uint32_t t) {
  const int lane = threadIdx.x & 63;
  const int64_t slot = load_uniform(p.slots + t);
  const int64_t pos = load_uniform(p.positions + t);
  const uint4 raw = reinterpret_cast<const uint4*>(p.kv + (int64_t)t * p.kv_st)[lane];
  const bool bad = pos < 0 || pos >= p.max_pos;
  const float4* csrow = reinterpret_cast<const float4*>(p.cs + (bad ? 0 : pos) * 64);
  const int pr = lane >= 56 ? lane - 56 : (lane & 7);
  const float4 c4 = csrow[pr], s4 = csrow[8 + pr];
  float x[8];
  const uint32_t d[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf_lo(d[i]);
    x[2 * i + 1] = bf_hi(d[i]);
  }
  if (lane >= 56) {  // forward GPT-J rotation: e' = e*c - o*s, o' = o*c + e*s
    const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = x[2 * i], o = x[2 * i + 1];
      const float ec = e * cv[i], os = o * sv[i], oc = o * cv[i], es = e * sv[i];
      x[2 * i] = ec - os;
      x[2 * i + 1] = oc + es;
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(x[e]));
  m = max_dpp_nonneg<kQuadSwap1>(m);
  m = max_dpp_nonneg<kQuadSwap2>(m);
  m = max_dpp_nonneg<kRowHalfMirror>(m);
  m = max_dpp_nonneg<kRowMirror>(m);
  float scale, mult;
  uint32_t ebyte;
  block_scale<FMT>(m, p.eps, scale, mult, ebyte);
  uint32_t code[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float q0 = x[4 * hf] * mult, q1 = x[4 * hf + 1] * mult;
    const float q2 = x[4 * hf + 2] * mult, q3 = x[4 * hf + 3] * mult;
    int wd = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, __builtin_bit_cast(int, q0), false);
    wd = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, wd, true);
    code[hf] = (uint32_t)wd;
  }
  uint4 tail;
  if (FMT == RQ_SCALE_UE8M0) {
    const uint32_t wd = ebyte << (8 * (lane >> 4));
    const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)wd, 0) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wd, 16) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wd, 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)wd, 48);
    tail = make_uint4(bad ? 0xFFFFFFFFu : word, 0u, 0u, 0u);
  } else {
    const int sb = bad ? 0x7FC00000 : __builtin_bit_cast(int, scale);
    tail = make_uint4((uint32_t)__builtin_amdgcn_readlane(sb, 0),
                      (uint32_t)__builtin_amdgcn_readlane(sb, 16),
                      (uint32_t)__builtin_amdgcn_readlane(sb, 32),
                      (uint32_t)__builtin_amdgcn_readlane(sb, 48));
  }
  if (slot < 0 || slot >= p.num_slots) return;  // padding token, or no such slot
  const uint32_t blk_i = magic_div((uint32_t)slot, p.div_bs);
  const uint32_t idx = (uint32_t)slot - blk_i * p.bs;
  uint8_t* const rec = p.cache + (int64_t)blk_i * p.block_stride + (int64_t)idx * kRecordBytes;
  reinterpret_cast<uint2*>(rec)[lane] = make_uint2(code[0], code[1]);
  if (lane == 0) *reinterpret_cast<uint4*>(rec + kHeadDim) = tail;
}

template <int FMT>
__global__ __launch_bounds__(256) void kvi1_kernel(KviParams p) {
  const uint32_t t = flat_wave_index();
  if (t < p.n_tokens) kvi1_body<FMT>(p, t);
}

// The q path and the kv path in one launch ([P1] section 1: the op
// normalizes and rotates q and inserts the rotated kv in a single kernel;
// section 2 names the full-cache forms: q as bf16 (in place) or FP8, kv into
// a token-strided cache).  Waves [0, q_waves) run the q path, the rest the kv
// path; the branch is per wave, and every wave has its own LDS slice.
struct FusedParams {
  LaunchHdr hdr;
  QnrParams q;
  KviParams k;
  uint32_t q_waves;
};

// s_waitcnt vmcnt(0), the other counters left at their maximum (gfx9 encoding)
constexpr int kWaitVmcnt0 = 0x0F70;

template <bool HAS_WEIGHT, int QOUT, int KOUT>
__global__ __launch_bounds__(256) void fused_qnr_kvi_kernel(FusedParams p) {
  extern __shared__ uint4 lds[];
  uint4* lds_wave = lds + 256 * (threadIdx.x >> 6);
  const uint32_t w = wave_index(p.hdr);
  if (w >= p.q_waves) {
    if constexpr (KOUT == kOutBf16) kvf_body(p.k, w - p.q_waves, lds_wave);
    else kvi2_body<KOUT, true>(p.k, w - p.q_waves, lds_wave);
    // The compiler lays the two paths out one after the other; with the kv
    // stores drained here, the q path's loads keep their per-load waits.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  } else {
    qnr_body<HAS_WEIGHT, QOUT>(p.q, w, lds_wave);
  }
}

// qnorm_rope_kv_rope_quant_insert for a few tokens: the decode kernels' one
// head (q) or one token (kv) per wave, q waves first.  The two paths share
// nothing but the positions, so each wave runs one body.
template <bool HAS_WEIGHT, int KFMT>
__global__ __launch_bounds__(256) void fused1_kernel(FusedParams p) {
  const uint32_t w = flat_wave_index();
  if (w < p.q.units) {
    qnr1_body<HAS_WEIGHT>(p.q, w);
  } else if (w - p.q.units < p.k.n_tokens) {
    kvi1_body<KFMT>(p.k, w - p.q.units);
  }
}

// ---------------------------------------------------- indexer query path

// A wave takes four work items, each 4 consecutive heads of one token (a
// token's last item may hold fewer): 16 heads of 128 dims.  The item's token,
// position, cos/sin row and base addresses are wave-uniform and live in
// scalar registers.  Each load instruction reads one item's four 256-byte
// head rows, 16 bytes per lane (1 KiB, contiguous when the heads are), and an
// LDS transpose hands lane (row i, L) the 8-dim chunks 8s + {0, 32, 64, 96}
// of head L >> 2 of item i (s = L & 3).  Every rotate-half pair (j, j + 32)
// then sits in one lane, every lane rotates 8 pairs, and a head's amax is a
// quad max.  The codes go back through LDS so that each store instruction
// writes two items' 512-byte code rows, 16 bytes per lane.  (An earlier
// layout, one head per 16-lane row with 8-byte loads and two items per wave,
// kept 2 KiB in flight per wave and streamed at 6.0 TB/s for large launches;
// this one streams at 7.1 TB/s.)
struct IdxParams {
  LaunchHdr hdr;
  const uint16_t* q;
  int64_t q_st, q_sh;
  const int64_t* positions;
  const float* cs;
  int64_t max_pos;
  const float* w;
  int64_t w_st;
  uint32_t items;  // n_tokens * quads
  Magic div_quads;
  uint32_t quads, n_heads;  // quads = ceil(n_heads / 4)
  float softmax_scale, head_scale, eps;
  uint8_t* out;
  int64_t out_st, out_sh;
  float* wo;
  int64_t wo_st;
  uint32_t out16;  // code rows 16-byte aligned (base and both strides)
};

// LDS slots (16 bytes) of item i: head row hh, 16-byte granule g at
// 64 i + 16 hh + (g ^ 4 (hh & 1)), so the lanes of a read group hit distinct
// banks.  Codes: head hh's 8-byte piece at byte 32 c + 8 s of its 128-byte
// row is kept at 512 i + 128 hh + ((32 c + 8 s) ^ 32 (hh & 3)).
__global__ __launch_bounds__(256) void idx_kernel(IdxParams p) {
  extern __shared__ uint4 lds[];
  const int lane = threadIdx.x & 63;
  const int row = lane >> 4, L = lane & 15, hh = L >> 2, sub = L & 3;
  uint4* lds_wave = lds + 256 * (threadIdx.x >> 6);
  const uint32_t item0 = wave_index(p.hdr) * 4u;
  // The wave's four items, wave-uniform.  A slot past the last item repeats
  // the last item, and a head past the token's last reads the item's first
  // head: every read stays inside q, and neither stores anything.
  // Load order: the positions (scalar), the q rows, then the cos/sin rows
  // and the head weights; the scheduling barriers keep the compiler from
  // waiting for the positions before the row reads are issued.
  uint32_t tk[4], h0k[4], nvk[4];
  const uint8_t* qk[4];
  int64_t posk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t it = min(item0 + k, p.items - 1u);
    const uint32_t t = magic_div(it, p.div_quads);
    tk[k] = t;
    h0k[k] = 4u * (it - t * p.quads);
    nvk[k] = (item0 + k < p.items) ? min(4u, p.n_heads - h0k[k]) : 0u;
    qk[k] = reinterpret_cast<const uint8_t*>(p.q + (int64_t)t * p.q_st + (int64_t)h0k[k] * p.q_sh);
    posk[k] = load_uniform(p.positions + t);
  }
  __builtin_amdgcn_sched_barrier(0);
  // Reads: instruction k, lane L' -> head L' >> 4 of item k, granule L' & 15.
  const uint32_t lhead = (uint32_t)lane >> 4;
  uint4 raw[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t nv = max(nvk[k], 1u);
    const uint32_t off = (lhead < nv ? lhead * (uint32_t)p.q_sh * 2u : 0u) + 16u * (lane & 15);
    raw[k] = load_nt(qk[k] + off);
  }
  __builtin_amdgcn_sched_barrier(0);
  // The weight of the lane's head, read now so that its latency overlaps the
  // q reads' instead of following the arithmetic (every lane reads; a head
  // past the token's last reads the token's last head and stores nothing).
  const uint32_t nv = PICK_ROW(row, nvk);
  const bool wlane = sub == 0 && (uint32_t)hh < nv;
  const uint32_t wt_tok = PICK_ROW(row, tk), wt_head = PICK_ROW(row, h0k) + (uint32_t)hh;
  const float wv = p.w[(int64_t)wt_tok * p.w_st + min(wt_head, p.n_heads - 1u)];
  const float* csk[4];
  uint32_t badk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bool bad = posk[k] < 0 || posk[k] >= p.max_pos;
    badk[k] = bad;
    csk[k] = p.cs + (bad ? 0 : posk[k]) * 64;
  }
  // cos / sin of the lane's 8 pairs: columns 8s .. 8s + 7 of its item's row
  const float4* csrow = reinterpret_cast<const float4*>(PICK_ROW(row, csk));
  const float4 c0 = csrow[2 * sub], c1 = csrow[2 * sub + 1];
  const float4 s0 = csrow[8 + 2 * sub], s1 = csrow[8 + 2 * sub + 1];
  // transpose through LDS
  const int wslot = lane ^ (((lane >> 4) & 1) << 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) lds_wave[64 * k + wslot] = raw[k];
  wave_lds_sync();
  uint4 w[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) w[c] = lds_wave[64 * row + 16 * hh + 4 * (c ^ (hh & 1)) + sub];

  // rotate-half on chunks 0 (dims 8s + j) and 1 (dims 32 + 8s + j), each
  // result rounded to bf16 and back; chunks 2, 3 pass through
  const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  float x[4][8];
  {
    const uint32_t e4[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
    const uint32_t o4[4] = {w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e = (j & 1) ? bf_hi(e4[j >> 1]) : bf_lo(e4[j >> 1]);
      const float o = (j & 1) ? bf_hi(o4[j >> 1]) : bf_lo(o4[j >> 1]);
      const float a = e * cv[j], b = o * sv[j], d = o * cv[j], f = e * sv[j];
      x[0][j] = (float)(__bf16)(a - b);
      x[1][j] = (float)(__bf16)(d + f);
    }
    const uint32_t p2[4] = {w[2].x, w[2].y, w[2].z, w[2].w};
    const uint32_t p3[4] = {w[3].x, w[3].y, w[3].z, w[3].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2][2 * j] = bf_lo(p2[j]);
      x[2][2 * j + 1] = bf_hi(p2[j]);
      x[3][2 * j] = bf_lo(p3[j]);
      x[3][2 * j + 1] = bf_hi(p3[j]);
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(x[c][j]));
  m = max_dpp_nonneg<kQuadSwap1>(m);
  m = max_dpp_nonneg<kQuadSwap2>(m);
  m = __builtin_fmaxf(m, p.eps);
  const uint32_t tb = __builtin_bit_cast(uint32_t, m < __builtin_inff() ? div448(m) : m);
  const int kexp = (int)((tb >> 23) & 0xFFu) - 127 + ((tb & 0x7FFFFFu) ? 1 : 0);
  const float qs = pow2_f32(kexp);
  const float mult = pow2_neg_f32(kexp);
  uint32_t code[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const float a0 = x[c][4 * hf] * mult, a1 = x[c][4 * hf + 1] * mult;
      const float a2 = x[c][4 * hf + 2] * mult, a3 = x[c][4 * hf + 3] * mult;
      int wd = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, __builtin_bit_cast(int, a0), false);
      wd = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, wd, true);
      code[2 * c + hf] = (uint32_t)wd;
    }
  }
  // folded weight of the lane's head
  if (wlane) {
    const float fold = ((wv * qs) * p.softmax_scale) * p.head_scale;
    p.wo[(int64_t)wt_tok * p.wo_st + wt_head] = PICK_ROW(row, badk) ? __builtin_nanf("") : fold;
  }
  // codes through LDS (the transpose reads are done before the slice is reused)
  wave_lds_sync();
  uint2* lds8 = reinterpret_cast<uint2*>(lds_wave);
#pragma unroll
  for (int c = 0; c < 4; ++c)
    lds8[64 * row + 16 * hh + ((4 * c + sub) ^ (4 * (hh & 3)))] =
        make_uint2(code[2 * c], code[2 * c + 1]);
  wave_lds_sync();
  // store instruction j: lanes 0..31 item 2j, lanes 32..63 item 2j + 1; lane
  // granule g = lane & 31 is head g >> 3, bytes 16 (g & 7) of its code row
  const uint32_t g = (uint32_t)lane & 31u, sh = g >> 3, gg = g & 7u;
  const int half = lane >> 5;
  const uint4* lds16 = reinterpret_cast<const uint4*>(lds_wave);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k0 = 2 * j, k1 = 2 * j + 1;  // the instruction's two items
    const uint4 v = lds16[32 * (k0 + half) + 8 * sh + 2 * ((gg >> 1) ^ (sh & 3)) + (gg & 1)];
    const uint32_t nvi = half ? nvk[k1] : nvk[k0];
    uint8_t* const base = half ? p.out + (int64_t)tk[k1] * p.out_st + (int64_t)h0k[k1] * p.out_sh
                               : p.out + (int64_t)tk[k0] * p.out_st + (int64_t)h0k[k0] * p.out_sh;
    if (sh < nvi) {
      uint8_t* const dst = base + (int64_t)sh * p.out_sh + 16 * gg;
      if (p.out16) {
        store_nt(dst, v);
      } else {  // 8-byte aligned rows
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(1))) u32x2_t* gptr2;
        __builtin_nontemporal_store(u32x2_t{v.x, v.y}, (gptr2)dst);
        __builtin_nontemporal_store(u32x2_t{v.z, v.w}, (gptr2)(dst + 8));
      }
    }
  }
}

// ------------------------------------------------------------ host side

Magic make_magic(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << (31 + s)) + d - 1) / d;
  return Magic{(uint32_t)m, 31u + s};
}

// Per-kernel launch shape, timed on MI355X: the XCD chunk size (log2
// workgroups) and the workgroup size for many units.
struct LaunchShape {
  uint32_t chunk_log2;
  int prefill_threads;
};

// Launch table: the analogue of [P4] section 4's program-count rule.  Many
// units (prefill): the kernel's prefill workgroup size (256 threads for
// every kernel now), plenty of workgroups per CU.  Few units (decode):
// 64-thread workgroups, one wave each, so the work spreads over as many CUs
// as possible; inv_rope_fp8_quant and qnorm_rope switch to their
// one-head-per-wave kernels there instead (launch_one_head).  Results do not
// depend on the choice.
int pick_block_threads(uint32_t units, int prefill_threads) {
  return units >= 16384u ? prefill_threads : 64;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool eps_quant_ok(double eps) {
  // finite and at least 2^-116 as fp32, so eps/448 stays normal and 1/s finite
  if (!(eps == eps) || eps > 3.0e38 || eps < 0) return false;
  const float e = (float)eps;
  return e >= 0x1p-116f;
}

// Non-overlap of an index space sum_i n_i * s_i (+ row of `row` contiguous
// elements): with dims of extent > 1 sorted by stride, each stride must exceed
// the span of all inner dims.  Sufficient (not necessary) for disjointness.
bool no_overlap(int nd, const int64_t* n, const int64_t* s, int64_t row) {
  int64_t ns[4], ss[4];
  int m = 0;
  for (int i = 0; i < nd; ++i)
    if (n[i] > 1) { ns[m] = n[i]; ss[m] = s[i]; ++m; }
  for (int i = 1; i < m; ++i)  // insertion sort by stride
    for (int k = i; k > 0 && ss[k] < ss[k - 1]; --k) {
      int64_t tn = ns[k]; ns[k] = ns[k - 1]; ns[k - 1] = tn;
      int64_t ts = ss[k]; ss[k] = ss[k - 1]; ss[k - 1] = ts;
    }
  int64_t span = row;  // elements covered by the inner dims so far
  for (int i = 0; i < m; ++i) {
    if (ss[i] < span) return false;
    int64_t t;
    if (__builtin_mul_overflow(ns[i] - 1, ss[i], &t) || __builtin_add_overflow(t, span, &span))
      return false;
  }
  return true;
}

// A tensor of `nd` dims (extent n[i], stride s[i] >= 1, in elements of `elem`
// bytes) over rows of `row` contiguous elements stays within 2^56 bytes of
// its base, computed without overflow.  No device address space is that
// large, so strides that fail this cannot describe a real tensor (and would
// wrap the kernels' 64-bit address arithmetic).
bool extent_ok(int nd, const int64_t* n, const int64_t* s, int64_t row, int64_t elem) {
  int64_t last = row;
  for (int i = 0; i < nd; ++i) {
    if (n[i] <= 1) continue;
    int64_t t;
    if (__builtin_mul_overflow(n[i] - 1, s[i], &t) || __builtin_add_overflow(t, last, &last))
      return false;
  }
  int64_t bytes;
  return !__builtin_mul_overflow(last, elem, &bytes) && bytes <= (int64_t(1) << 56);
}

// Every params struct starts with a LaunchHdr, filled in here.
// `units` counts the kernel's work units (512-dim heads; the indexer's
// 4-head items), `units_per_wave` how many one wave takes (4, or 2 for
// inv_rope_fp8_quant).  Each wave gets 1 KiB of LDS per unit.
int launch(const void* fn, uint32_t units, LaunchShape shape, void* params,
           hipStream_t stream, uint32_t units_per_wave = 4) {
  const int threads = pick_block_threads(units, shape.prefill_threads);
  LaunchHdr* hdr = static_cast<LaunchHdr*>(params);
  hdr->wpb_log2 = threads == 256 ? 2u : threads == 128 ? 1u : 0u;
  hdr->chunk_log2 = shape.chunk_log2;
  const uint32_t per_block = (uint32_t)threads / 64u * units_per_wave;
  const uint32_t blocks = (units + per_block - 1) / per_block;
  void* args[] = {params};
  const size_t lds_bytes = (size_t)(threads / 64) * 1024 * units_per_wave;
  const hipError_t e =
      hipLaunchKernel(fn, dim3(blocks), dim3((uint32_t)threads), args, lds_bytes, stream);
  return e == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

// Timed with every launch on buffers that earlier launches have not touched.
constexpr LaunchShape kIrqShape{6, 256};  // FP8 codes, two units per wave
constexpr LaunchShape kIrbShape{6, 256};  // bf16 rows
constexpr LaunchShape kQnrShape{4, 256};  // bf16 q_out
constexpr uint32_t kQnrOneHeadUnits = 2048;  // qnorm_rope: one head per wave up to here
constexpr uint32_t kIrqOneHeadUnits = 16383;  // inv_rope_fp8_quant: below the prefill entry
constexpr uint32_t kOneHeadSmallUnits = 512;  // ... in 64-thread workgroups up to here (waves)
constexpr LaunchShape kQf8Shape{4, 256};  // FP8 q_out
constexpr LaunchShape kFusedShape{4, 256};
constexpr LaunchShape kKviShape{4, 256};
constexpr uint32_t kKviOneTokenTokens = 2048;  // kv_rope_quant_insert: one token per wave
constexpr uint32_t kKviNtTokens = 4096;  // kv_rope_quant_insert: nontemporal record stores from here
constexpr LaunchShape kIdxShape{4, 256};

// The launch-table entry for few heads (decode): a one-head-per-wave kernel
// (qnr1_kernel, irq1_kernel, kvi1_kernel, fused1_kernel), in 64-thread
// workgroups up to 512 waves (they spread over the most CUs) and 256-thread
// ones above.  Per call in a HIP graph on MI355X:
//   qnorm_rope, 32 heads padded to 128: 1.94 against 2.50 us (four heads per
//   wave) at 1 token, 2.26 against 2.65 at 16; from 32 tokens on, the
//   thousands of single-head waves (most of them pad heads) cost more to
//   launch than they save, and the four-head kernel takes over;
//   inv_rope_fp8_quant, 32 heads: 1.93 against 2.09 us (two heads per wave)
//   at 1 token, 2.62 against 2.78 at 128, 5.35 against 5.77 at 511, so it
//   takes every call below the prefill entry;
//   kv_rope_quant_insert (kvi1_kernel, one token per wave): 1.67 against
//   1.74 us (two tokens per wave) at 1 token, 2.04 against 2.19 at 1024; it
//   takes calls of up to 2048 tokens, below the size where the records'
//   stores turn nontemporal;
//   qnorm_rope_kv_rope_quant_insert (fused1_kernel) with the q path's entry:
//   1.94 against 2.63 us at 1 token, 2.31 against 3.02 at 16.
int launch_one_head(const void* fn, void* params, uint32_t units, void* stream) {
  const uint32_t threads = units <= kOneHeadSmallUnits ? 64u : 256u;
  const uint32_t per_block = threads / 64u;
  void* args[] = {params};
  const hipError_t e = hipLaunchKernel(fn, dim3((units + per_block - 1u) / per_block),
                                       dim3(threads), args, 0, (hipStream_t)stream);
  return e == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

bool finite_f32(double v) {
  const float f = (float)v;
  return v == v && f == f && f - f == 0.0f;
}

}  // namespace

extern "C" {

int ropequant_abi_version(void) { return ROPEQUANT_ABI_VERSION; }

const char* ropequant_strerror(int status) {
  switch (status) {
    case RQ_OK: return "ok";
    case RQ_ERR_NULL: return "a required pointer is NULL";
    case RQ_ERR_SHAPE: return "a size is out of range or inconsistent";
    case RQ_ERR_STRIDE: return "a stride is non-positive or lets outputs overlap";
    case RQ_ERR_ALIGN: return "a pointer or stride breaks the required alignment";
    case RQ_ERR_VALUE: return "a scalar argument (scale_fmt, eps) is invalid";
    case RQ_ERR_HIP: return "the HIP runtime refused the launch";
    default: return "unknown status";
  }
}

int inv_rope_fp8_quant(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                       const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                       int64_t n_tokens, int32_t n_heads, int32_t heads_per_group,
                       int32_t scale_fmt, double eps, uint8_t* out, int64_t out_stride_group,
                       int64_t out_stride_token, void* scales, int64_t sc_stride_group,
                       int64_t sc_stride_token, int64_t sc_stride_block, void* stream) {
  if (n_tokens < 0 || n_heads < 1 || heads_per_group < 1 || max_pos < 1) return RQ_ERR_SHAPE;
  if (n_heads % heads_per_group) return RQ_ERR_SHAPE;
  if ((int64_t)n_tokens * n_heads >= (int64_t(1) << 31)) return RQ_ERR_SHAPE;
  if (scale_fmt != RQ_SCALE_FP32 && scale_fmt != RQ_SCALE_UE8M0) return RQ_ERR_VALUE;
  if (!eps_quant_ok(eps)) return RQ_ERR_VALUE;
  if (n_tokens == 0) return RQ_OK;
  if (!o || !positions || !cos_sin_cache || !out || !scales) return RQ_ERR_NULL;
  if (o_stride_token < 1 || o_stride_head < 1 || out_stride_group < 1 || out_stride_token < 1 ||
      sc_stride_group < 1 || sc_stride_token < 1 || sc_stride_block < 1)
    return RQ_ERR_STRIDE;
  if (!aligned(o, 16) || (o_stride_token % 8) || (o_stride_head % 8) || !aligned(positions, 8) ||
      !aligned(cos_sin_cache, 16) || !aligned(out, 16) || (out_stride_group % 16) ||
      (out_stride_token % 16) || !aligned(scales, 4))
    return RQ_ERR_ALIGN;
  const int64_t G = n_heads / heads_per_group;
  {
    const int64_t n[2] = {n_tokens, n_heads}, s[2] = {o_stride_token, o_stride_head};
    if (!extent_ok(2, n, s, kHeadDim, 2)) return RQ_ERR_STRIDE;
  }
  {
    const int64_t n[2] = {G, n_tokens}, s[2] = {out_stride_group, out_stride_token};
    const int64_t row = (int64_t)heads_per_group * kHeadDim;
    if (!no_overlap(2, n, s, row) || !extent_ok(2, n, s, row, 1)) return RQ_ERR_STRIDE;
  }
  {
    const int64_t per = scale_fmt == RQ_SCALE_FP32 ? (int64_t)heads_per_group * 4 : heads_per_group;
    const int64_t n[3] = {G, n_tokens, per}, s[3] = {sc_stride_group, sc_stride_token, sc_stride_block};
    if (!no_overlap(3, n, s, 1) || !extent_ok(3, n, s, 1, 4)) return RQ_ERR_STRIDE;
  }
  IrqParams p;
  p.o = o; p.o_st = o_stride_token; p.o_sh = o_stride_head;
  p.positions = positions; p.cs = cos_sin_cache; p.max_pos = max_pos;
  p.units = (uint32_t)(n_tokens * n_heads);
  p.div_heads = make_magic((uint32_t)n_heads);
  p.div_hpg = make_magic((uint32_t)heads_per_group);
  p.n_heads = (uint32_t)n_heads; p.hpg = (uint32_t)heads_per_group;
  p.eps = (float)eps;
  p.out = out; p.out_sg = out_stride_group; p.out_st = out_stride_token;
  p.scales = scales; p.sc_sg = sc_stride_group; p.sc_st = sc_stride_token; p.sc_sb = sc_stride_block;
  p.sc_vec4 = scale_fmt == RQ_SCALE_FP32 && sc_stride_block == 1 && sc_stride_group % 4 == 0 &&
              sc_stride_token % 4 == 0 && aligned(scales, 16);
  if (p.units <= kIrqOneHeadUnits) {
    const void* fn1 = scale_fmt == RQ_SCALE_UE8M0 ? (const void*)irq1_kernel<RQ_SCALE_UE8M0>
                                                  : (const void*)irq1_kernel<RQ_SCALE_FP32>;
    return launch_one_head(fn1, &p, p.units, stream);
  }
  const void* fn = scale_fmt == RQ_SCALE_UE8M0 ? (const void*)irq_kernel<RQ_SCALE_UE8M0>
                                               : (const void*)irq_kernel<RQ_SCALE_FP32>;
  return launch(fn, p.units, kIrqShape, &p, (hipStream_t)stream, 2);
}

int inv_rope_bf16(const uint16_t* o, int64_t o_stride_token, int64_t o_stride_head,
                  const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                  int64_t n_tokens, int32_t n_heads, int32_t heads_per_group, uint16_t* out,
                  int64_t out_stride_group, int64_t out_stride_token, void* stream) {
  if (n_tokens < 0 || n_heads < 1 || heads_per_group < 1 || max_pos < 1) return RQ_ERR_SHAPE;
  if (n_heads % heads_per_group) return RQ_ERR_SHAPE;
  if ((int64_t)n_tokens * n_heads >= (int64_t(1) << 31)) return RQ_ERR_SHAPE;
  if (n_tokens == 0) return RQ_OK;
  if (!o || !positions || !cos_sin_cache || !out) return RQ_ERR_NULL;
  if (o_stride_token < 1 || o_stride_head < 1 || out_stride_group < 1 || out_stride_token < 1)
    return RQ_ERR_STRIDE;
  if (!aligned(o, 16) || (o_stride_token % 8) || (o_stride_head % 8) || !aligned(positions, 8) ||
      !aligned(cos_sin_cache, 16) || !aligned(out, 16) || (out_stride_group % 8) ||
      (out_stride_token % 8))
    return RQ_ERR_ALIGN;
  const int64_t G = n_heads / heads_per_group;
  {
    const int64_t n[2] = {n_tokens, n_heads}, s[2] = {o_stride_token, o_stride_head};
    if (!extent_ok(2, n, s, kHeadDim, 2)) return RQ_ERR_STRIDE;
  }
  {
    const int64_t n[2] = {G, n_tokens}, s[2] = {out_stride_group, out_stride_token};
    const int64_t row = (int64_t)heads_per_group * kHeadDim;
    if (!no_overlap(2, n, s, row) || !extent_ok(2, n, s, row, 2)) return RQ_ERR_STRIDE;
  }
  // in place only when every head's output lands on its own input row
  if (out == o && !(o_stride_head == kHeadDim && out_stride_token == o_stride_token &&
                    out_stride_group == (int64_t)heads_per_group * kHeadDim))
    return RQ_ERR_STRIDE;
  IrqParams p;
  p.o = o; p.o_st = o_stride_token; p.o_sh = o_stride_head;
  p.positions = positions; p.cs = cos_sin_cache; p.max_pos = max_pos;
  p.units = (uint32_t)(n_tokens * n_heads);
  p.div_heads = make_magic((uint32_t)n_heads);
  p.div_hpg = make_magic((uint32_t)heads_per_group);
  p.n_heads = (uint32_t)n_heads; p.hpg = (uint32_t)heads_per_group;
  p.eps = 0.0f;
  p.out = reinterpret_cast<uint8_t*>(out);
  p.out_sg = 2 * out_stride_group; p.out_st = 2 * out_stride_token;  // bytes in the kernel
  p.scales = nullptr; p.sc_sg = p.sc_st = p.sc_sb = 0; p.sc_vec4 = 0;
  return launch((const void*)irb_kernel, p.units, kIrbShape, &p,
                (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Validation and parameter set-up shared by the standalone and the fused
// entry points.  RQ_OK with `empty` set means there is nothing to launch.
// qout: kOutBf16 (q_out) or a scale format (q_fp8 + q_scales, quant_eps).
int prep_qnr(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
             const uint16_t* norm_weight, const int64_t* positions, const float* cos_sin_cache,
             int64_t max_pos, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
             double eps, int qout, uint16_t* q_out, uint8_t* q_fp8, void* q_scales,
             double quant_eps, QnrParams& p, bool& empty) {
  empty = true;
  const bool bf16 = qout == kOutBf16;
  if (n_tokens < 0 || n_heads_q < 1 || max_pos < 1) return RQ_ERR_SHAPE;
  if (q_head_padded < n_heads_q) return RQ_ERR_SHAPE;  // [P1] section 1 check
  if ((int64_t)n_tokens * q_head_padded >= (int64_t(1) << 31)) return RQ_ERR_SHAPE;
  if (!(eps > 0.0) || !((float)eps > 0.0f) || !((float)eps <= 3.0e38f)) return RQ_ERR_VALUE;
  if (!bf16 && !eps_quant_ok(quant_eps)) return RQ_ERR_VALUE;
  if (n_tokens == 0) return RQ_OK;
  if (!q_in || !positions || !cos_sin_cache) return RQ_ERR_NULL;
  if (bf16 ? !q_out : (!q_fp8 || !q_scales)) return RQ_ERR_NULL;
  if (q_stride_token < 1 || q_stride_head < 1) return RQ_ERR_STRIDE;
  {
    const int64_t n[2] = {n_tokens, n_heads_q}, s[2] = {q_stride_token, q_stride_head};
    if (!extent_ok(2, n, s, kHeadDim, 2)) return RQ_ERR_STRIDE;
  }
  if (!aligned(q_in, 16) || (q_stride_token % 8) || (q_stride_head % 8) ||
      !aligned(positions, 8) || !aligned(cos_sin_cache, 16) ||
      (norm_weight && !aligned(norm_weight, 16)))
    return RQ_ERR_ALIGN;
  if (bf16 ? !aligned(q_out, 16) : (!aligned(q_fp8, 16) || !aligned(q_scales, 4)))
    return RQ_ERR_ALIGN;
  // in place only when every head's output lands on its own input row
  if (bf16 && q_out == q_in &&
      !(q_head_padded == n_heads_q && q_stride_head == kHeadDim &&
        q_stride_token == (int64_t)n_heads_q * kHeadDim))
    return RQ_ERR_STRIDE;
  p.q = q_in; p.q_st = q_stride_token; p.q_sh = q_stride_head;
  p.weight = norm_weight; p.positions = positions; p.cs = cos_sin_cache; p.max_pos = max_pos;
  p.units = (uint32_t)(n_tokens * q_head_padded);
  p.div_hpad = make_magic((uint32_t)q_head_padded);
  p.hq = (uint32_t)n_heads_q; p.hpad = (uint32_t)q_head_padded;
  p.eps = (float)eps;
  p.q_out = bf16 ? q_out : nullptr;
  p.q_fp8 = bf16 ? nullptr : q_fp8;
  p.q_scales = bf16 ? nullptr : q_scales;
  p.quant_eps = bf16 ? 0.0f : (float)quant_eps;
  // a zero head's scale, by quantize_lane's own steps (fp32 division, exact
  // power-of-two rounding); host fp32 arithmetic is IEEE round-to-nearest
  p.pad_scale = 0.0f;
  p.pad_ebyte = 0u;
  if (!bf16) {
    const float t = p.quant_eps / kE4m3Max;
    if (qout == RQ_SCALE_UE8M0) {
      uint32_t u;
      std::memcpy(&u, &t, 4);
      const int kexp = (int)((u >> 23) & 0xFFu) - 127 + ((u & 0x7FFFFFu) ? 1 : 0);
      const uint32_t sb = (uint32_t)(kexp + 127) << 23;
      std::memcpy(&p.pad_scale, &sb, 4);
      p.pad_ebyte = (uint32_t)(kexp + 127);
    } else {
      p.pad_scale = t;
    }
  }
  empty = false;
  return RQ_OK;
}

int prep_kvi(const uint16_t* kv, int64_t kv_stride_token, const int64_t* positions,
             const float* cos_sin_cache, int64_t max_pos, const int64_t* slot_mapping,
             int64_t n_tokens, uint8_t* k_cache, int64_t num_blocks, int64_t block_stride_bytes,
             int32_t cache_block_size, int32_t scale_fmt, double eps, KviParams& p,
             bool& empty) {
  empty = true;
  if (n_tokens < 0 || max_pos < 1 || num_blocks < 1 || cache_block_size < 1) return RQ_ERR_SHAPE;
  if (n_tokens >= (int64_t(1) << 27)) return RQ_ERR_SHAPE;
  if (num_blocks * (int64_t)cache_block_size >= (int64_t(1) << 31)) return RQ_ERR_SHAPE;
  if (block_stride_bytes < (int64_t)cache_block_size * kRecordBytes) return RQ_ERR_STRIDE;
  if (scale_fmt != RQ_SCALE_FP32 && scale_fmt != RQ_SCALE_UE8M0) return RQ_ERR_VALUE;
  if (!eps_quant_ok(eps)) return RQ_ERR_VALUE;
  if (n_tokens == 0) return RQ_OK;
  if (!kv || !positions || !cos_sin_cache || !slot_mapping || !k_cache) return RQ_ERR_NULL;
  if (kv_stride_token < 1) return RQ_ERR_STRIDE;
  if (!extent_ok(1, &n_tokens, &kv_stride_token, kHeadDim, 2) ||
      !extent_ok(1, &num_blocks, &block_stride_bytes, (int64_t)cache_block_size * kRecordBytes, 1))
    return RQ_ERR_STRIDE;
  if (!aligned(kv, 16) || (kv_stride_token % 8) || !aligned(positions, 8) ||
      !aligned(cos_sin_cache, 16) || !aligned(slot_mapping, 8) || !aligned(k_cache, 16) ||
      (block_stride_bytes % 16))
    return RQ_ERR_ALIGN;
  p.kv = kv; p.kv_st = kv_stride_token; p.positions = positions; p.cs = cos_sin_cache;
  p.max_pos = max_pos; p.slots = slot_mapping; p.n_tokens = (uint32_t)n_tokens;
  p.num_slots = num_blocks * (int64_t)cache_block_size;
  p.div_bs = make_magic((uint32_t)cache_block_size); p.bs = (uint32_t)cache_block_size;
  p.cache = k_cache; p.block_stride = block_stride_bytes; p.eps = (float)eps;
  empty = false;
  return RQ_OK;
}

// The kv path into the token-strided bf16 cache: slot s owns the 512
// elements at cache + s * cache_stride_token.
int prep_kvf(const uint16_t* kv, int64_t kv_stride_token, const int64_t* positions,
             const float* cos_sin_cache, int64_t max_pos, const int64_t* slot_mapping,
             int64_t n_tokens, uint16_t* cache, int64_t num_slots, int64_t cache_stride_token,
             KviParams& p, bool& empty) {
  empty = true;
  if (n_tokens < 0 || max_pos < 1 || num_slots < 1) return RQ_ERR_SHAPE;
  if (n_tokens >= (int64_t(1) << 27)) return RQ_ERR_SHAPE;
  if (cache_stride_token < kHeadDim) return RQ_ERR_STRIDE;
  if (num_slots > (int64_t(1) << 62) / cache_stride_token) return RQ_ERR_SHAPE;
  if (n_tokens == 0) return RQ_OK;
  if (!kv || !positions || !cos_sin_cache || !slot_mapping || !cache) return RQ_ERR_NULL;
  if (kv_stride_token < 1) return RQ_ERR_STRIDE;
  if (!extent_ok(1, &n_tokens, &kv_stride_token, kHeadDim, 2) ||
      !extent_ok(1, &num_slots, &cache_stride_token, kHeadDim, 2))
    return RQ_ERR_STRIDE;
  if (!aligned(kv, 16) || (kv_stride_token % 8) || !aligned(positions, 8) ||
      !aligned(cos_sin_cache, 16) || !aligned(slot_mapping, 8) || !aligned(cache, 16) ||
      (cache_stride_token % 8))
    return RQ_ERR_ALIGN;
  p.kv = kv; p.kv_st = kv_stride_token; p.positions = positions; p.cs = cos_sin_cache;
  p.max_pos = max_pos; p.slots = slot_mapping; p.n_tokens = (uint32_t)n_tokens;
  p.num_slots = num_slots;
  p.div_bs = make_magic(1u); p.bs = 1u;  // unused by the bf16 form
  p.cache = reinterpret_cast<uint8_t*>(cache);
  p.block_stride = 2 * cache_stride_token;  // bytes in the kernel
  p.eps = 0.0f;
  empty = false;
  return RQ_OK;
}

template <int QOUT>
const void* qnr_fn(bool has_weight) {
  return has_weight ? (const void*)qnr_kernel<true, QOUT> : (const void*)qnr_kernel<false, QOUT>;
}

template <int QOUT, int KOUT>
const void* fused_fn(bool has_weight) {
  return has_weight ? (const void*)fused_qnr_kvi_kernel<true, QOUT, KOUT>
                    : (const void*)fused_qnr_kvi_kernel<false, QOUT, KOUT>;
}

// One grid for both paths: q waves first, then kv waves of
// `kv_tokens_per_wave` tokens (2 for the paged FP8 cache, 4 for the bf16
// one).  `launch` sizes grids in 16-lane rows, 4 per wave.
int launch_fused(const void* fn, FusedParams& p, void* stream, uint32_t kv_tokens_per_wave) {
  p.q_waves = (p.q.units + 3u) / 4u;
  const uint32_t kv_waves = (p.k.n_tokens + kv_tokens_per_wave - 1u) / kv_tokens_per_wave;
  return launch(fn, 4u * (p.q_waves + kv_waves), kFusedShape, &p, (hipStream_t)stream);
}

}  // namespace

extern "C" {

int qnorm_rope(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
               const uint16_t* norm_weight, const int64_t* positions,
               const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
               int32_t n_heads_q, int32_t q_head_padded, double eps, uint16_t* q_out,
               void* stream) {
  QnrParams p;
  bool empty;
  const int rc = prep_qnr(q_in, q_stride_token, q_stride_head, norm_weight, positions,
                          cos_sin_cache, max_pos, n_tokens, n_heads_q, q_head_padded, eps,
                          kOutBf16, q_out, nullptr, nullptr, 0.0, p, empty);
  if (rc != RQ_OK || empty) return rc;
  if (p.units <= kQnrOneHeadUnits)
    return launch_one_head(norm_weight != nullptr ? (const void*)qnr1_kernel<true>
                                                  : (const void*)qnr1_kernel<false>,
                           &p, p.units, stream);
  return launch(qnr_fn<kOutBf16>(norm_weight != nullptr), p.units, kQnrShape, &p,
                (hipStream_t)stream);
}

int qnorm_rope_fp8(const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
                   const uint16_t* norm_weight, const int64_t* positions,
                   const float* cos_sin_cache, int64_t max_pos, int64_t n_tokens,
                   int32_t n_heads_q, int32_t q_head_padded, double eps, int32_t scale_fmt,
                   double quant_eps, uint8_t* q_fp8, void* q_scales, void* stream) {
  if (scale_fmt != RQ_SCALE_FP32 && scale_fmt != RQ_SCALE_UE8M0) return RQ_ERR_VALUE;
  QnrParams p;
  bool empty;
  const int rc = prep_qnr(q_in, q_stride_token, q_stride_head, norm_weight, positions,
                          cos_sin_cache, max_pos, n_tokens, n_heads_q, q_head_padded, eps,
                          scale_fmt, nullptr, q_fp8, q_scales, quant_eps, p, empty);
  if (rc != RQ_OK || empty) return rc;
  const bool w = norm_weight != nullptr;
  const void* fn = scale_fmt == RQ_SCALE_UE8M0 ? qnr_fn<RQ_SCALE_UE8M0>(w)
                                               : qnr_fn<RQ_SCALE_FP32>(w);
  return launch(fn, p.units, kQf8Shape, &p, (hipStream_t)stream);
}

int kv_rope_quant_insert(const uint16_t* kv, int64_t kv_stride_token, const int64_t* positions,
                         const float* cos_sin_cache, int64_t max_pos,
                         const int64_t* slot_mapping, int64_t n_tokens, uint8_t* k_cache,
                         int64_t num_blocks, int64_t block_stride_bytes,
                         int32_t cache_block_size, int32_t scale_fmt, double eps,
                         void* stream) {
  KviParams p;
  bool empty;
  const int rc = prep_kvi(kv, kv_stride_token, positions, cos_sin_cache, max_pos, slot_mapping,
                          n_tokens, k_cache, num_blocks, block_stride_bytes, cache_block_size,
                          scale_fmt, eps, p, empty);
  if (rc != RQ_OK || empty) return rc;
  if (p.n_tokens <= kKviOneTokenTokens)
    return launch_one_head(scale_fmt == RQ_SCALE_UE8M0 ? (const void*)kvi1_kernel<RQ_SCALE_UE8M0>
                                                       : (const void*)kvi1_kernel<RQ_SCALE_FP32>,
                           &p, p.n_tokens, stream);
  const bool nt = p.n_tokens >= kKviNtTokens;
  const void* fn = scale_fmt == RQ_SCALE_UE8M0
                       ? (nt ? (const void*)kvi2_kernel<RQ_SCALE_UE8M0, true>
                             : (const void*)kvi2_kernel<RQ_SCALE_UE8M0, false>)
                       : (nt ? (const void*)kvi2_kernel<RQ_SCALE_FP32, true>
                             : (const void*)kvi2_kernel<RQ_SCALE_FP32, false>);
  return launch(fn, p.n_tokens, kKviShape, &p, (hipStream_t)stream, 2);
}

int kv_rope_insert_full(const uint16_t* kv, int64_t kv_stride_token, const int64_t* positions,
                        const float* cos_sin_cache, int64_t max_pos,
                        const int64_t* slot_mapping, int64_t n_tokens, uint16_t* cache,
                        int64_t num_slots, int64_t cache_stride_token, void* stream) {
  KviParams p;
  bool empty;
  const int rc = prep_kvf(kv, kv_stride_token, positions, cos_sin_cache, max_pos, slot_mapping,
                          n_tokens, cache, num_slots, cache_stride_token, p, empty);
  if (rc != RQ_OK || empty) return rc;
  return launch((const void*)kvf_kernel, p.n_tokens, kKviShape, &p,
                (hipStream_t)stream);
}

int qnorm_rope_kv_rope_quant_insert(
    const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
    const uint16_t* norm_weight, const uint16_t* kv, int64_t kv_stride_token,
    const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
    const int64_t* slot_mapping, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
    double eps, uint16_t* q_out, uint8_t* k_cache, int64_t num_blocks,
    int64_t block_stride_bytes, int32_t cache_block_size, int32_t scale_fmt, double quant_eps,
    void* stream) {
  FusedParams p;
  bool eq, ek;
  int rc = prep_qnr(q_in, q_stride_token, q_stride_head, norm_weight, positions, cos_sin_cache,
                    max_pos, n_tokens, n_heads_q, q_head_padded, eps, kOutBf16, q_out, nullptr,
                    nullptr, 0.0, p.q, eq);
  if (rc != RQ_OK) return rc;
  rc = prep_kvi(kv, kv_stride_token, positions, cos_sin_cache, max_pos, slot_mapping, n_tokens,
                k_cache, num_blocks, block_stride_bytes, cache_block_size, scale_fmt, quant_eps,
                p.k, ek);
  if (rc != RQ_OK || eq) return rc;  // both are empty exactly when n_tokens == 0
  const bool w = norm_weight != nullptr;
  if (p.q.units <= kQnrOneHeadUnits) {
    const bool ue = scale_fmt == RQ_SCALE_UE8M0;
    const void* fn1 = w ? (ue ? (const void*)fused1_kernel<true, RQ_SCALE_UE8M0>
                              : (const void*)fused1_kernel<true, RQ_SCALE_FP32>)
                        : (ue ? (const void*)fused1_kernel<false, RQ_SCALE_UE8M0>
                              : (const void*)fused1_kernel<false, RQ_SCALE_FP32>);
    return launch_one_head(fn1, &p, p.q.units + p.k.n_tokens, stream);
  }
  const void* fn = scale_fmt == RQ_SCALE_UE8M0 ? fused_fn<kOutBf16, RQ_SCALE_UE8M0>(w)
                                               : fused_fn<kOutBf16, RQ_SCALE_FP32>(w);
  return launch_fused(fn, p, stream, 2);
}

int qnorm_rope_kv_rope_insert_full(
    const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
    const uint16_t* norm_weight, const uint16_t* kv, int64_t kv_stride_token,
    const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
    const int64_t* slot_mapping, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
    double eps, uint16_t* q_out, uint16_t* cache, int64_t num_slots, int64_t cache_stride_token,
    void* stream) {
  FusedParams p;
  bool eq, ek;
  int rc = prep_qnr(q_in, q_stride_token, q_stride_head, norm_weight, positions, cos_sin_cache,
                    max_pos, n_tokens, n_heads_q, q_head_padded, eps, kOutBf16, q_out, nullptr,
                    nullptr, 0.0, p.q, eq);
  if (rc != RQ_OK) return rc;
  rc = prep_kvf(kv, kv_stride_token, positions, cos_sin_cache, max_pos, slot_mapping, n_tokens,
                cache, num_slots, cache_stride_token, p.k, ek);
  if (rc != RQ_OK || eq) return rc;
  return launch_fused(fused_fn<kOutBf16, kOutBf16>(norm_weight != nullptr), p, stream, 4);
}

int qnorm_rope_fp8_kv_rope_insert_full(
    const uint16_t* q_in, int64_t q_stride_token, int64_t q_stride_head,
    const uint16_t* norm_weight, const uint16_t* kv, int64_t kv_stride_token,
    const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
    const int64_t* slot_mapping, int64_t n_tokens, int32_t n_heads_q, int32_t q_head_padded,
    double eps, int32_t scale_fmt, double quant_eps, uint8_t* q_fp8, void* q_scales,
    uint16_t* cache, int64_t num_slots, int64_t cache_stride_token, void* stream) {
  if (scale_fmt != RQ_SCALE_FP32 && scale_fmt != RQ_SCALE_UE8M0) return RQ_ERR_VALUE;
  FusedParams p;
  bool eq, ek;
  int rc = prep_qnr(q_in, q_stride_token, q_stride_head, norm_weight, positions, cos_sin_cache,
                    max_pos, n_tokens, n_heads_q, q_head_padded, eps, scale_fmt, nullptr, q_fp8,
                    q_scales, quant_eps, p.q, eq);
  if (rc != RQ_OK) return rc;
  rc = prep_kvf(kv, kv_stride_token, positions, cos_sin_cache, max_pos, slot_mapping, n_tokens,
                cache, num_slots, cache_stride_token, p.k, ek);
  if (rc != RQ_OK || eq) return rc;
  const bool w = norm_weight != nullptr;
  const void* fn = scale_fmt == RQ_SCALE_UE8M0 ? fused_fn<RQ_SCALE_UE8M0, kOutBf16>(w)
                                               : fused_fn<RQ_SCALE_FP32, kOutBf16>(w);
  return launch_fused(fn, p, stream, 4);
}

int indexer_q_rope_quant(const uint16_t* q, int64_t q_stride_token, int64_t q_stride_head,
                         const int64_t* positions, const float* cos_sin_cache, int64_t max_pos,
                         const float* weights, int64_t w_stride_token, int64_t n_tokens,
                         int32_t n_heads, double softmax_scale, double head_scale, double eps,
                         uint8_t* q_fp8, int64_t out_stride_token, int64_t out_stride_head,
                         float* weights_out, int64_t wo_stride_token, void* stream) {
  if (n_tokens < 0 || n_heads < 1 || max_pos < 1) return RQ_ERR_SHAPE;
  if ((int64_t)n_tokens * n_heads >= (int64_t(1) << 31)) return RQ_ERR_SHAPE;
  if (!eps_quant_ok(eps) || !finite_f32(softmax_scale) || !finite_f32(head_scale))
    return RQ_ERR_VALUE;
  if (n_tokens == 0) return RQ_OK;
  if (!q || !positions || !cos_sin_cache || !weights || !q_fp8 || !weights_out)
    return RQ_ERR_NULL;
  if (q_stride_token < 1 || q_stride_head < 1 || w_stride_token < 1 || out_stride_token < 1 ||
      out_stride_head < 1 || wo_stride_token < 1)
    return RQ_ERR_STRIDE;
  if (!aligned(q, 16) || (q_stride_token % 8) || (q_stride_head % 8) || !aligned(positions, 8) ||
      !aligned(cos_sin_cache, 16) || !aligned(weights, 4) || !aligned(q_fp8, 8) ||
      (out_stride_token % 8) || (out_stride_head % 8) || !aligned(weights_out, 4))
    return RQ_ERR_ALIGN;
  {
    const int64_t n[2] = {n_tokens, n_heads}, st[2] = {out_stride_token, out_stride_head};
    if (!no_overlap(2, n, st, 128) || !extent_ok(2, n, st, 128, 1)) return RQ_ERR_STRIDE;
    const int64_t sw[2] = {wo_stride_token, 1};
    if (!no_overlap(2, n, sw, 1) || !extent_ok(1, &n_tokens, &wo_stride_token, n_heads, 4))
      return RQ_ERR_STRIDE;
    const int64_t sq[2] = {q_stride_token, q_stride_head};
    if (!extent_ok(2, n, sq, 128, 2) || !extent_ok(1, &n_tokens, &w_stride_token, n_heads, 4))
      return RQ_ERR_STRIDE;
  }
  // per-lane offsets inside a 4-head item are kept in 32 bits
  if (q_stride_head > (int64_t(1) << 28) || out_stride_head > (int64_t(1) << 30))
    return RQ_ERR_STRIDE;
  IdxParams p;
  p.q = q; p.q_st = q_stride_token; p.q_sh = q_stride_head;
  p.positions = positions; p.cs = cos_sin_cache; p.max_pos = max_pos;
  p.w = weights; p.w_st = w_stride_token;
  p.quads = (uint32_t)((n_heads + 3) / 4);
  p.items = (uint32_t)(n_tokens * p.quads);
  p.div_quads = make_magic(p.quads); p.n_heads = (uint32_t)n_heads;
  p.softmax_scale = (float)softmax_scale; p.head_scale = (float)head_scale; p.eps = (float)eps;
  p.out = q_fp8; p.out_st = out_stride_token; p.out_sh = out_stride_head;
  p.wo = weights_out; p.wo_st = wo_stride_token;
  p.out16 = aligned(q_fp8, 16) && out_stride_token % 16 == 0 && out_stride_head % 16 == 0;
  // one item per 16-lane row, four per wave
  const uint32_t rows = 4u * ((p.items + 3u) / 4u);
  return launch((const void*)idx_kernel, rows, kIdxShape, &p, (hipStream_t)stream);
}

}  // extern "C"

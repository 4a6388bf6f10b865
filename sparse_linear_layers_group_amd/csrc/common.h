// common.h -- device-side helpers shared by the gfx950 kernels of the
// BitLinear library.  Host code includes it only for the format constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// ---------------------------------------------------------------------
// Packed ternary format ("code plus index"), per 8-group of one row:
//   bits [0,4)      nonzero bitmap of positions 0..3
//   bits [4,4+S)    sign bits (1 = negative); the i-th nonzero of the low
//                   half at 4+i, the i-th nonzero of the high half at
//                   4+S-1-i
//   bits [4+S,8+S)  nonzero bitmap of positions 4..7
// so the low half decodes from field bits [0,8) and the high half from
// field bits [S, S+8), each an 8-bit key of (bitmap, 4 sign bits).
// A block holds the 16 fields of one row and one 128-wide k block, field
// g at bit g*(8+S), 2*(8+S) bytes.  Blocks are stored by slot
//   ((row/16) * (k/128) + kb) * 16 + row%16
// so the 64 blocks a wavefront reads for 16 rows x 512 k are contiguous.
// ---------------------------------------------------------------------
constexpr int kBlockK = 128;
constexpr int kTileRows = 16;
constexpr int kStripRows = 64;  // rows of a packed superblock

// Packed layout: rows in strips of 64; the superblock of (strip, k block)
// holds 64 chunks of 2(8+S) bytes.  Chunk c = r + 16q carries, as field
// f = 4i + 2h + e, the 8-group 8h + 2q + e of strip row 16i + r, so chunk c
// is exactly the A operand lane c needs for the 8 MFMAs (row tile i, k half
// h) of one superblock.
// Forward epilogue Y = acc * gamma * s_t: gamma * s_t is formed in binary64
// and rounded once to binary32, then the product is rounded once more
// (relative error below 2^-22; acc is exact in binary32 up to 2^24).  The
// decode and prefill kernels share it, so they give identical outputs.
__device__ __forceinline__ float out_scale(double gamma, float s_t) {
  return (float)(gamma * (double)s_t);
}
__device__ __forceinline__ float out_value(int32_t acc, float gs) { return (float)acc * gs; }

__host__ __device__ constexpr int field_row(int c, int f) { return 16 * (f >> 2) + (c & 15); }
__host__ __device__ constexpr int field_group(int c, int f) {
  return 8 * ((f >> 1) & 1) + 2 * (c >> 4) + (f & 1);
}

__host__ __device__ constexpr int block_bytes(int S) { return 2 * (8 + S); }

// sign slots per 8-group for a supported n:m, else -1 (an even count at
// least the nonzeros an 8-group can hold, so a chunk is whole 32-bit words:
// 3:8 shares the 4-slot layout of 4:8 and 2:4)
__host__ __device__ constexpr int s_of(int n, int m) {
  return (m == 8 && n == 8) ? 8 : (m == 8 && n == 6) ? 6 : (m == 8 && n == 4) ? 4
       : (m == 4 && n == 2) ? 4 : (m == 8 && n == 3) ? 4 : (m == 8 && n == 2) ? 2 : -1;
}

// bf16 helpers ---------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// MFMA operand types ---------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));

// four binary32 outputs as bf16 (nearest, ties to even), packed for one
// 8-byte store
__device__ __forceinline__ u32x2 bf16x4(v4f y) {
  return u32x2{(uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16),
               (uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16)};
}

// explicit global-address-space accesses: pointers that arrive through
// memory (e.g. from a plan) would otherwise become flat accesses, which also
// count against the LDS counter and force extra waits
template <class T>
__device__ __forceinline__ T ld_global(const T* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
template <class T>
__device__ __forceinline__ void st_global(T* p, T v) {
  *(__attribute__((address_space(1))) T*)(p) = v;
}
// a store that streams past the caches (non-temporal): for large outputs
// that no later access in the kernel reads
template <class T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  __builtin_nontemporal_store(v, (__attribute__((address_space(1))) T*)(p));
}

// Device-scope integer atomics through global-address-space pointers: on a
// generic pointer they would be FLAT operations, which may touch LDS, and a
// pending FLAT operation makes every later wait drain all outstanding
// loads.
template <class T>
__device__ __forceinline__ void atomic_add_global(T* p, T v) {
  __hip_atomic_fetch_add((__attribute__((address_space(1))) T*)(p), v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T atomic_fetch_add_global(T* p, T v) {
  return __hip_atomic_fetch_add((__attribute__((address_space(1))) T*)(p), v, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T atomic_exchange_global(T* p, T v) {
  return __hip_atomic_exchange((__attribute__((address_space(1))) T*)(p), v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// 64-bit load at agent scope: served coherently for the whole device (not
// from a CU's possibly stale L1), for data another workgroup published
__device__ __forceinline__ unsigned long long ld_agent_u64(const unsigned long long* p) {
  return __hip_atomic_load((const __attribute__((address_space(1))) unsigned long long*)(p),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 64-bit store at agent scope: written through to where every XCD reads
// it.  A plain store may stay in the writing XCD's L2 (the L2s of the XCDs
// are not kept coherent with each other within a kernel), where a
// workgroup on another XCD would not see it.
__device__ __forceinline__ void st_agent_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store((__attribute__((address_space(1))) unsigned long long*)(p), v,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every memory operation this wavefront issued has completed.
// Partial sums that meet across workgroups go only through device-scope
// atomics, which are performed at the device's coherence point; once they
// have completed, a later atomic (a ticket) is ordered after them.  This
// gives that order without the L2 write-back an agent-scope fence implies
// (which, per wavefront, would cost far more than the whole contraction).
__device__ __forceinline__ void wait_memory_ops() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// wave-level reductions ------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// funnel shift: bits [sh, sh+32) of the 64-bit value (hi:lo)
__device__ __forceinline__ uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t sh) {
  return __builtin_amdgcn_alignbit(hi, lo, sh);
}

// int8x4 codes of one half-group from its 8-bit key.
// half 0: key = bitmap(4) | signs(4) << 4, i-th nonzero's sign at bit 4+i
// half 1: key = signs(4) | bitmap(4) << 4, i-th nonzero's sign at bit 3-i
__host__ __device__ constexpr uint32_t half_codes(uint32_t key, uint32_t half) {
  const uint32_t bm = half ? (key >> 4) : (key & 15u);
  const uint32_t sg = half ? (key & 15u) : (key >> 4);
  uint32_t out = 0, rank = 0;
  for (int p = 0; p < 4; ++p) {
    if ((bm >> p) & 1u) {
      const uint32_t bit = half ? (3u - rank) : rank;
      out |= (((sg >> bit) & 1u) ? 0xffu : 0x01u) << (8 * p);
      ++rank;
    }
  }
  return out;
}

// The 512 table entries, entry key * 2 + half, built at compile time and
// held in device memory: a kernel fills its LDS copies with plain loads.
struct HalfCodeTable {
  uint32_t v[512];
};
constexpr HalfCodeTable make_half_code_table() {
  HalfCodeTable t{};
  for (uint32_t e = 0; e < 512; ++e) t.v[e] = half_codes(e >> 1, e & 1u);
  return t;
}
__device__ constexpr HalfCodeTable kHalfCodeTable = make_half_code_table();
static_assert(make_half_code_table().v[2 * 0x1f + 0] == 0x010101ffu, "low half: bitmap 1111, sign of nonzero 0");

// Decode groups [G0, G0+NG) of one packed block held in registers w[0..kW]
// (w[kW] = 0): emit(g, lo, hi) receives the int8x4 codes of positions 0..3
// and 4..7 of group g.  lut[key] is the low-half table, lut[256+key] the
// high-half table.  Offsets are compile-time, so w stays in registers.
template <int S, int G0, int NG, class Lut, class Emit>
__device__ __forceinline__ void decode_groups(const uint32_t* w, Lut lut, Emit emit) {
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    constexpr int kField = 8 + S;
    const int off = (G0 + gg) * kField, offh = off + S;
    const uint32_t klo = funnel(w[(off >> 5) + 1], w[off >> 5], off & 31) & 0xffu;
    const uint32_t khi = funnel(w[(offh >> 5) + 1], w[offh >> 5], offh & 31) & 0xffu;
    emit(G0 + gg, lut(klo, 0), lut(khi, 1));
  }
}

}  // namespace bl

// quant.hip -- weight and activation quantisation kernels (gfx950).
//
//  mask_gamma_kernel  : N:M mask from latent |W| plus exact partial |W|
//                       sums, one per workgroup;
//  gamma_finalize_kernel: adds the partials, rounds once to binary64 and
//                       writes gamma.
//  ternary_pack_kernel: masked ternary codes -> packed bitmap+sign blocks
//                       (and/or plain int8 codes).
//  act_quant_kernel   : per-token absmax int8 activations.
//
// Sparse-BitNet explainer article §三/§五/§六 (dynamic N:M mask from the
// full-precision weights, quantise before sparsifying); BitNet b1.58 2B4T
// article §一 (absmean ternary weights, 8-bit activations).
#include "common.h"
#include "launch.h"

namespace bl {

// ---------------------------------------------------------------------
// Exact sum of |W|.  A finite bf16 magnitude is sig * 2^(max(E,1) - 134)
// with E the 8-bit exponent field and sig = (E ? 128 : 0) + fraction.
// Two fixed-point windows cover |W| in [2^-41, 2): E in [kHiLo, kHiLo+21)
// adds sig << (E - kHiLo) to a 64-bit integer in units of 2^(kHiLo-134),
// E in [kLoLo, kHiLo) adds sig << (E - kLoLo) to a second one in units of
// 2^(kLoLo-134).  Any other nonzero magnitude adds sig into an exponent
// bin of its workgroup (in LDS).  Integer addition is associative, so the
// result does not depend on scheduling.
// ---------------------------------------------------------------------
constexpr int kHiLo = 107;
constexpr int kLoLo = 86;
constexpr int kWin = 21;  // sig << 20 < 2^28: eight of them fit in 32 bits

struct MaskPart {
  unsigned long long hi, lo;  // window sums
  uint32_t binned;            // nonzero: this workgroup wrote its 256 bins
  uint32_t pad[3];
};
static_assert(sizeof(MaskPart) == 32, "mask partial record");

// keys: |h| (15 bits) above a 3-bit code that ranks a lower index higher;
// all keys of a group are distinct and a larger key ranks first.
__device__ __forceinline__ uint32_t rank_key(uint32_t h, int j) {
  return ((h & 0x7fffu) << 3) | (uint32_t)(7 - j);
}

__device__ __forceinline__ void cswap(uint32_t& a, uint32_t& b) {
  uint32_t lo = min(a, b), hi = max(a, b);
  a = lo;
  b = hi;
}

// mask bits of one 8-group (w = 8 bf16, element j in bits 16j..16j+15 of
// the four words) for the pattern N:M
template <int N, int M>
__device__ __forceinline__ uint32_t group_mask(const uint32_t w[4]) {
  if (N == M) return 0xffu;
  uint32_t key[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) key[j] = rank_key((w[j >> 1] >> (16 * (j & 1))) & 0xffffu, j);
  uint32_t tau_lo, tau_hi;  // a key is kept iff it exceeds its half's / group's tau
  if (M == 4) {
    // 2:4 -- per half of four, drop the two smallest keys
    uint32_t t[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t p0 = min(key[4 * h], key[4 * h + 1]), P0 = max(key[4 * h], key[4 * h + 1]);
      uint32_t p1 = min(key[4 * h + 2], key[4 * h + 3]), P1 = max(key[4 * h + 2], key[4 * h + 3]);
      t[h] = min(max(p0, p1), min(P0, P1));  // second smallest of four
    }
    tau_lo = t[0];
    tau_hi = t[1];
  } else if (N == 6) {
    // 6:8 -- tau = second smallest of eight
    uint32_t p[4], P[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = min(key[2 * i], key[2 * i + 1]);
      P[i] = max(key[2 * i], key[2 * i + 1]);
    }
    uint32_t q1 = min(p[0], p[1]), q2 = min(max(p[0], p[1]), min(P[0], P[1]));
    uint32_t r1 = min(p[2], p[3]), r2 = min(max(p[2], p[3]), min(P[2], P[3]));
    tau_lo = tau_hi = min(max(q1, r1), min(q2, r2));
  } else {
    // general N of 8: sort (Batcher odd-even merge network, 19 swaps),
    // tau = (8-N)-th smallest
    uint32_t s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = key[j];
    cswap(s[0], s[1]); cswap(s[2], s[3]); cswap(s[4], s[5]); cswap(s[6], s[7]);
    cswap(s[0], s[2]); cswap(s[1], s[3]); cswap(s[4], s[6]); cswap(s[5], s[7]);
    cswap(s[1], s[2]); cswap(s[5], s[6]);
    cswap(s[0], s[4]); cswap(s[1], s[5]); cswap(s[2], s[6]); cswap(s[3], s[7]);
    cswap(s[2], s[4]); cswap(s[3], s[5]);
    cswap(s[1], s[2]); cswap(s[3], s[4]); cswap(s[5], s[6]);
    tau_lo = tau_hi = s[7 - N];
  }
  uint32_t bits = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t tau = (j < 4) ? tau_lo : tau_hi;
    bits |= ((tau - key[j]) >> 31) << j;  // key > tau (keys < 2^18)
  }
  return bits;
}

// exact |W| accumulation of one 8-group into the two window sums
template <bool MASKED>
__device__ __forceinline__ void group_abs_sum(const uint32_t w[4], uint32_t keep,
                                              unsigned long long& hi, unsigned long long& lo,
                                              unsigned long long* bins, uint32_t& binned) {
  uint32_t sh_sum = 0, sl_sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t a = (w[j >> 1] >> (16 * (j & 1))) & 0x7fffu;
    if (MASKED && !((keep >> j) & 1u)) a = 0;
    const uint32_t e = a >> 7;
    const uint32_t sig = (a & 0x7fu) | (e ? 0x80u : 0u);
    const uint32_t sh = e - (uint32_t)kHiLo, sl = e - (uint32_t)kLoLo;
    const bool in_h = sh < (uint32_t)kWin, in_l = sl < (uint32_t)kWin;
    sh_sum += in_h ? (sig << sh) : 0u;
    sl_sum += in_l ? (sig << sl) : 0u;
    if (!in_h && !in_l && a != 0u) {
      atomicAdd(&bins[e], (unsigned long long)sig);
      binned = 1;
    }
  }
  hi += sh_sum;
  lo += sl_sum;
}

// 320-bit unsigned integer in 32-bit limbs, units of 2^-133; limb indices
// are compile-time after unrolling, so the value stays in registers
struct Big {
  uint32_t limb[10];
};

// b += v * 2^shift
__device__ __forceinline__ void big_add(Big& b, unsigned long long v, int shift) {
  const int li = shift >> 5, bo = shift & 31;
  const uint32_t p0 = (uint32_t)(v << bo);
  const uint32_t p1 = bo ? (uint32_t)(v >> (32 - bo)) : (uint32_t)(v >> 32);
  const uint32_t p2 = bo ? (uint32_t)(v >> (64 - bo)) : 0u;
  unsigned long long carry = 0;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i < li) continue;
    const uint32_t add = i == li ? p0 : i == li + 1 ? p1 : i == li + 2 ? p2 : 0u;
    const unsigned long long t = (unsigned long long)b.limb[i] + add + carry;
    b.limb[i] = (uint32_t)t;
    carry = t >> 32;
  }
}

// nearest binary64 (ties to even) of b * 2^-133: the top 64 bits, with
// every lower nonzero bit folded into the last one (a sticky bit far below
// the rounding position), converted by one correctly rounded u64 -> f64
// conversion; the final power-of-two scaling is exact
__device__ double big_round(const Big& b) {
  int ti = -1;
#pragma unroll
  for (int i = 0; i < 10; ++i)
    if (b.limb[i]) ti = i;
  if (ti < 0) return 0.0;
  uint32_t x2 = 0, x1 = 0, x0 = 0, sticky = 0;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i == ti) x2 = b.limb[i];
    if (i == ti - 1) x1 = b.limb[i];
    if (i == ti - 2) x0 = b.limb[i];
    if (i < ti - 2) sticky |= b.limb[i];
  }
  const int lz = __clz(x2);
  const unsigned long long top = ((unsigned long long)x2 << 32) | x1;
  unsigned long long m = lz ? (top << lz) | (x0 >> (32 - lz)) : top;
  sticky |= lz ? (x0 << lz) : x0;
  m |= sticky ? 1ull : 0ull;
  // b = m * 2^(32 (ti - 2) + 32 - lz) (up to the sticky bit)
  return ldexp((double)m, 32 * (ti - 2) + 32 - lz - 133);
}

// Kernel 1: mask bytes of every 8-group and the workgroup's exact partial
// sums.  Workgroup b covers the contiguous 8-groups [b*per, (b+1)*per);
// every load instruction of a wavefront reads 1 KiB of consecutive
// weights.
template <int N, int M, bool MASKED>
__global__ __launch_bounds__(256) void mask_gamma_kernel(const uint4* __restrict__ W,
                                                        int64_t ngroups, int64_t per,
                                                        uint8_t* __restrict__ mask,
                                                        char* __restrict__ ws) {
  __shared__ unsigned long long bins[256];
  __shared__ unsigned long long part[2][4];
  __shared__ uint32_t any_binned;
  bins[threadIdx.x] = 0ull;
  if (threadIdx.x == 0) any_binned = 0;
  __syncthreads();
  unsigned long long hi = 0, lo = 0;
  uint32_t binned = 0;
  const int64_t g_begin = (int64_t)blockIdx.x * per;
  const int64_t g_end = g_begin + per < ngroups ? g_begin + per : ngroups;
  for (int64_t c0 = g_begin; c0 < g_end; c0 += kMaskGroupsPerPass) {
    uint4 v[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t grp = c0 + 256 * g + threadIdx.x;
      v[g] = grp < g_end ? W[grp] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t grp = c0 + 256 * g + threadIdx.x;
      if (grp >= g_end) break;
      const uint32_t w[4] = {v[g].x, v[g].y, v[g].z, v[g].w};
      const uint32_t keep = group_mask<N, M>(w);
      mask[grp] = (uint8_t)keep;
      group_abs_sum<MASKED>(w, keep, hi, lo, bins, binned);
    }
  }
  hi = wave_sum_u64(hi);
  lo = wave_sum_u64(lo);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    part[0][wave] = hi;
    part[1][wave] = lo;
  }
  if (binned) any_binned = 1;
  __syncthreads();
  MaskPart* rec = reinterpret_cast<MaskPart*>(ws) + blockIdx.x;
  if (threadIdx.x == 0) {
    MaskPart r;
    r.hi = part[0][0] + part[0][1] + part[0][2] + part[0][3];
    r.lo = part[1][0] + part[1][1] + part[1][2] + part[1][3];
    r.binned = any_binned;
    r.pad[0] = r.pad[1] = r.pad[2] = 0;
    *rec = r;
  }
  if (any_binned) {
    unsigned long long* out =
        reinterpret_cast<unsigned long long*>(ws + (size_t)gridDim.x * sizeof(MaskPart)) +
        (size_t)blockIdx.x * 256;
    out[threadIdx.x] = bins[threadIdx.x];
  }
}

// Kernel 2 (one workgroup of 256): gamma = (sum of the partials) / count,
// the sum rounded once to binary64.
__global__ __launch_bounds__(256) void gamma_finalize_kernel(const char* __restrict__ ws,
                                                             int nblocks, double* __restrict__ gamma,
                                                             double count) {
  __shared__ unsigned long long part[2][4];
  __shared__ unsigned long long bins[256];
  __shared__ uint32_t any_binned;
  if (threadIdx.x == 0) any_binned = 0;
  const MaskPart* rec = reinterpret_cast<const MaskPart*>(ws);
  unsigned long long hi = 0, lo = 0;
  uint32_t binned = 0;
  for (int b = threadIdx.x; b < nblocks; b += 256) {
    hi += rec[b].hi;
    lo += rec[b].lo;
    binned |= rec[b].binned;
  }
  hi = wave_sum_u64(hi);
  lo = wave_sum_u64(lo);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();  // any_binned initialised
  if (lane == 0) {
    part[0][wave] = hi;
    part[1][wave] = lo;
  }
  if (binned) any_binned = 1;
  __syncthreads();
  unsigned long long bin = 0;
  if (any_binned) {
    const unsigned long long* all =
        reinterpret_cast<const unsigned long long*>(ws + (size_t)nblocks * sizeof(MaskPart));
    for (int b = 0; b < nblocks; ++b)
      if (rec[b].binned) bin += all[(size_t)b * 256 + threadIdx.x];
  }
  bins[threadIdx.x] = bin;
  __syncthreads();
  if (threadIdx.x != 0) return;
  Big big;
#pragma unroll
  for (int i = 0; i < 10; ++i) big.limb[i] = 0;
  big_add(big, part[0][0] + part[0][1] + part[0][2] + part[0][3], kHiLo - 1);
  big_add(big, part[1][0] + part[1][1] + part[1][2] + part[1][3], kLoLo - 1);
  if (any_binned)
    for (int e = 0; e < 256; ++e)
      if (bins[e]) big_add(big, bins[e], e > 0 ? e - 1 : 0);
  *gamma = big_round(big) / count;
}

// ---------------------------------------------------------------------
// Ternary codes and packing.  The code of W is sign(W) where the mask
// keeps it and 2|W| > gamma.  Since bf16 magnitudes are ordered like their
// 15-bit patterns, that test is |h| >= thr for the smallest pattern thr
// whose value v has 2v > gamma, i.e. v > gamma/2 (halving is exact in
// binary64): one past the largest bf16 <= gamma/2, which is the top half of
// gamma/2 rounded toward zero to binary32 (every bf16 value is a binary32
// value, so the next bf16 up exceeds gamma/2).  Past the largest finite
// bf16 the infinity pattern is the threshold.
// ---------------------------------------------------------------------
__device__ uint32_t code_threshold(double g) {
  if (!(g > 0.0)) return 0x10000u;  // no entry qualifies
  const uint32_t b = __float_as_uint(__double2float_rz(0.5 * g)) >> 16;  // largest bf16 <= g/2
  return b + 1u > 0x7f80u ? 0x7f80u : b + 1u;
}

// field (8+S bits) and int8 codes (two words, positions 0..3 / 4..7) of one
// 8-group: w = 8 bf16 values, keep = the group's mask byte
template <int S>
__device__ __forceinline__ uint32_t group_field(const uint4& v, uint32_t keep, uint32_t thr,
                                                uint32_t& lo, uint32_t& hi) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t nz = 0, neg = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t h = (w[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    uint32_t on = ((keep >> j) & 1u) & ((h & 0x7fffu) >= thr ? 1u : 0u);
    nz |= on << j;
    neg |= (on & (h >> 15)) << j;
  }
  // signs: low half from the bottom, high half from the top
  uint32_t sign = 0;
  int nlo = 0, nhi = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if ((nz >> p) & 1u) { sign |= ((neg >> p) & 1u) << nlo; ++nlo; }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    if ((nz >> (4 + p)) & 1u) { sign |= ((neg >> (4 + p)) & 1u) << (S - 1 - nhi); ++nhi; }
  }
  lo = 0;
  hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t cl = ((nz >> j) & 1u) ? (((neg >> j) & 1u) ? 0xffu : 0x01u) : 0u;
    uint32_t ch = ((nz >> (4 + j)) & 1u) ? (((neg >> (4 + j)) & 1u) ? 0xffu : 0x01u) : 0u;
    lo |= cl << (8 * j);
    hi |= ch << (8 * j);
  }
  return (nz & 0xfu) | (sign << 4) | ((nz >> 4) << (4 + S));
}

// One thread per packed chunk: it gathers the 16 (row, group) fields the
// chunk holds (field_row / field_group), builds them from the latent
// weights, the mask and gamma, and writes the chunk with plain stores; the
// int8 codes of those groups go to wq when it is requested.  Padding rows
// of the last strip give zero fields.
template <int S, bool PACKED, bool WQ>
__global__ __launch_bounds__(256) void ternary_pack_kernel(const uint16_t* __restrict__ W,
                                                          const uint8_t* __restrict__ mask,
                                                          const double* __restrict__ gamma,
                                                          int64_t n_out, int64_t k,
                                                          uint32_t* __restrict__ packed,
                                                          int8_t* __restrict__ wq) {
  constexpr int kWords = block_bytes(S) / 4;
  constexpr int kField = 8 + S;
  const int64_t nkb = k / kBlockK;
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (chunk >= strips * nkb * kStripRows) return;
  const int64_t sb = chunk / kStripRows;  // superblock = strip * nkb + kb
  const int c = (int)(chunk - sb * kStripRows);
  const int64_t strip = sb / nkb, kb = sb - strip * nkb;
  const uint32_t thr = code_threshold(*gamma);

  uint32_t out[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) out[i] = 0;
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    const int64_t row = strip * kStripRows + field_row(c, f);
    const int grp = field_group(c, f);
    if (row >= n_out) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(W + row * k + kb * kBlockK + 8 * grp);
    const uint32_t keep = mask[row * (k / 8) + kb * 16 + grp];
    uint32_t lo, hi;
    const uint32_t field = group_field<S>(v, keep, thr, lo, hi);
    const int off = f * kField;
    out[off >> 5] |= field << (off & 31);
    if ((off & 31) + kField > 32) out[(off >> 5) + 1] |= field >> (32 - (off & 31));
    if (WQ) *reinterpret_cast<uint2*>(wq + row * k + kb * kBlockK + 8 * grp) = make_uint2(lo, hi);
  }
  if (PACKED) {
    uint32_t* dst = packed + chunk * kWords;
#pragma unroll
    for (int i = 0; i < kWords; ++i) dst[i] = out[i];
  }
}

// ---------------------------------------------------------------------
// Per-token absmax int8 activations.  One block per token.
// x_q = rint(127 x / a) with a correctly rounded binary32 division: 127 x
// is exact in binary32, and a quotient of two 8-bit-significand values that
// is not a half-integer sits at least ~2^-16 (relative) away from one, far
// beyond binary32 rounding, so rint(ties to even) of the rounded quotient
// equals round-half-even of the exact quotient.  |x_q| <= 127, so the clip
// to [-128, 127] never binds.  Optionally zeroes a workspace range.
// ---------------------------------------------------------------------
__device__ __forceinline__ uint2 quant8(const uint4& v, float a) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t q[2] = {0, 0};
  if (a > 0.f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
      const int qi = (int)rintf((127.0f * x) / a);
      q[j >> 2] |= ((uint32_t)qi & 0xffu) << (8 * (j & 3));
    }
  }
  return make_uint2(q[0], q[1]);
}

__device__ __forceinline__ float absmax8(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) a = fmaxf(a, fmaxf(fabsf(bf16_lo(w[j])), fabsf(bf16_hi(w[j]))));
  return a;
}

// One row of k values by a 256-thread block.  Rows up to 256 * 8 * kHeld
// values are read once and held in registers between the absmax and the
// quantisation; longer rows take a second pass over memory.
constexpr int kHeld = 4;  // 16-byte vectors held per thread (rows <= 8192)
__device__ __forceinline__ void quant_row(const uint16_t* __restrict__ X, int64_t k,
                                          int8_t* __restrict__ xq, float* __restrict__ scale,
                                          float* red) {
  const uint4* row = reinterpret_cast<const uint4*>(X);
  const int64_t nvec = k / 8;
  uint4 held[kHeld];
  float a = 0.f;
#pragma unroll
  for (int h = 0; h < kHeld; ++h) {
    const int64_t i = threadIdx.x + 256 * h;
    held[h] = i < nvec ? row[i] : make_uint4(0, 0, 0, 0);
    a = fmaxf(a, absmax8(held[h]));
  }
  for (int64_t i = threadIdx.x + 256 * kHeld; i < nvec; i += 256) a = fmaxf(a, absmax8(row[i]));
  a = wave_max(a);
  __syncthreads();  // red[] free from a previous row
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (threadIdx.x == 0) *scale = a / 127.0f;
  uint2* out = reinterpret_cast<uint2*>(xq);
#pragma unroll
  for (int h = 0; h < kHeld; ++h) {
    const int64_t i = threadIdx.x + 256 * h;
    if (i < nvec) out[i] = quant8(held[h], a);
  }
  for (int64_t i = threadIdx.x + 256 * kHeld; i < nvec; i += 256) out[i] = quant8(row[i], a);
}

__global__ __launch_bounds__(256) void act_quant_kernel(const uint16_t* __restrict__ X, int64_t k,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ scale,
                                                       uint32_t* __restrict__ zero_ws,
                                                       int64_t zero_words) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  quant_row(X + t * k, k, xq + t * k, scale + t, red);
  if (zero_ws) {
    for (int64_t i = t * blockDim.x + threadIdx.x; i < zero_words; i += (int64_t)gridDim.x * blockDim.x)
      zero_ws[i] = 0u;
  }
}

// grouped: every row descriptor of a decode plan, grid-stride
__global__ __launch_bounds__(256) void act_quant_group_kernel(const char* __restrict__ plan) {
  __shared__ float red[4];
  const GroupHeader* hdr = reinterpret_cast<const GroupHeader*>(plan);
  const RowDesc* rows = reinterpret_cast<const RowDesc*>(plan + group_rows_offset());
  const int64_t nrows = hdr->rows;
  // the first row descriptor is read together with the header (the row
  // region holds at least kActGroupBlocks zero-padded descriptors)
  RowDesc d = rows[blockIdx.x];
  // Workgroup b < kDecodeBlocks also reads the 16 wavefront records of
  // contraction workgroup b, which runs next on the same XCD (both grids
  // are dealt round-robin over the XCDs): the contraction then finds them
  // in that XCD's L2 instead of waiting for HBM before its first loads.
  constexpr int kStartVecs = kDecodeWavesPerBlock * (int)sizeof(WaveStart) / 16;
  const bool warm = blockIdx.x < kDecodeBlocks && threadIdx.x < kStartVecs;
  u32x4 ws = u32x4{0u, 0u, 0u, 0u};
  if (warm)
    ws = ld_global(reinterpret_cast<const u32x4*>(plan + group_waves_offset() +
                                                  (size_t)blockIdx.x * kDecodeWavesPerBlock * sizeof(WaveStart)) +
                   threadIdx.x);
  for (int64_t r = blockIdx.x; r < nrows; r += gridDim.x) {
    if (r != blockIdx.x) d = rows[r];
    quant_row(d.X, d.k, d.xq, d.scale, red);
  }
  if (warm) asm volatile("" : : "v"(ws.x));  // keeps the read
}

// ------------------------------------------------------------- launchers
template <int N, int M>
static hipError_t launch_mask(const uint16_t* W, int64_t n_out, int64_t k, int gamma_over,
                              uint8_t* mask, double* gamma, void* ws, hipStream_t s) {
  const int64_t ngroups = n_out * k / 8;
  const int64_t blocks = mask_blocks(n_out, k);
  int64_t per = (ngroups + blocks - 1) / blocks;
  per = (per + kMaskGroupsPerPass - 1) / kMaskGroupsPerPass * kMaskGroupsPerPass;
  char* w = reinterpret_cast<char*>(ws);
  const uint4* W4 = reinterpret_cast<const uint4*>(W);
  if (gamma_over == 0)
    mask_gamma_kernel<N, M, false><<<(unsigned)blocks, 256, 0, s>>>(W4, ngroups, per, mask, w);
  else
    mask_gamma_kernel<N, M, true><<<(unsigned)blocks, 256, 0, s>>>(W4, ngroups, per, mask, w);
  gamma_finalize_kernel<<<1, 256, 0, s>>>(w, (int)blocks, gamma, (double)(n_out * k));
  return hipGetLastError();
}

hipError_t launch_mask_gamma(const uint16_t* W, int64_t n_out, int64_t k, int n, int m,
                             int gamma_over, uint8_t* mask, double* gamma, void* ws,
                             hipStream_t s) {
  if (m == 8 && n == 8) return launch_mask<8, 8>(W, n_out, k, gamma_over, mask, gamma, ws, s);
  if (m == 8 && n == 6) return launch_mask<6, 8>(W, n_out, k, gamma_over, mask, gamma, ws, s);
  if (m == 8 && n == 4) return launch_mask<4, 8>(W, n_out, k, gamma_over, mask, gamma, ws, s);
  return launch_mask<2, 4>(W, n_out, k, gamma_over, mask, gamma, ws, s);
}

template <int S>
static hipError_t launch_tp(const uint16_t* W, const uint8_t* mask, const double* gamma,
                            int64_t n_out, int64_t k, void* packed, int8_t* wq, hipStream_t s) {
  const int64_t chunks = ((n_out + kStripRows - 1) / kStripRows) * kStripRows * (k / kBlockK);
  const unsigned blocks = (unsigned)((chunks + 255) / 256);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  if (packed && wq)
    ternary_pack_kernel<S, true, true><<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, p, wq);
  else if (packed)
    ternary_pack_kernel<S, true, false><<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, p, wq);
  else
    ternary_pack_kernel<S, false, true><<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, p, wq);
  return hipGetLastError();
}

hipError_t launch_ternary_pack(const uint16_t* W, const uint8_t* mask, const double* gamma,
                               int64_t n_out, int64_t k, int S, void* packed, int8_t* wq,
                               hipStream_t s) {
  if (S == 8) return launch_tp<8>(W, mask, gamma, n_out, k, packed, wq, s);
  if (S == 6) return launch_tp<6>(W, mask, gamma, n_out, k, packed, wq, s);
  return launch_tp<4>(W, mask, gamma, n_out, k, packed, wq, s);
}

hipError_t launch_act_quant_group(const void* plan, hipStream_t s) {
  act_quant_group_kernel<<<kActGroupBlocks, 256, 0, s>>>(reinterpret_cast<const char*>(plan));
  return hipGetLastError();
}

hipError_t launch_act_quant(const uint16_t* X, int64_t tokens, int64_t k, int8_t* xq,
                            float* scale, void* zero_ws, int64_t zero_bytes, hipStream_t s) {
  act_quant_kernel<<<(unsigned)tokens, 256, 0, s>>>(X, k, xq, scale,
                                                    reinterpret_cast<uint32_t*>(zero_ws),
                                                    zero_ws ? zero_bytes / 4 : 0);
  return hipGetLastError();
}

}  // namespace bl

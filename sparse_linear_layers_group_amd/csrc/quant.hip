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
#include "actq.h"
#include "common.h"
#include "launch.h"

namespace bl {

// ---------------------------------------------------------------------
// Exact sum of |W|.  A finite bf16 magnitude is sig * 2^(max(E,1) - 134)
// with E the 8-bit exponent field and sig = (E ? 128 : 0) + fraction.
// One fixed-point window covers |W| in [2^-59, 2): E in [kWinLo, 128)
// adds sig << (E - kWinLo) (< 2^60; eight of them < 2^63) to an integer
// in units of 2^(kWinLo-134).  A group whose eight magnitudes are all in
// the window and within 2^13 of each other (the common case) is summed in
// binary32, exactly; one with a wider spread takes the 64-bit window sum;
// a group holding a zero or any magnitude outside the window takes the
// exact per-element path, where every other nonzero magnitude adds sig
// into an exponent bin of its workgroup (in LDS).  Integer addition is
// associative, so the result does not depend on scheduling.
// ---------------------------------------------------------------------
constexpr int kWinLo = 75;
// rank keys (|h| << 3 | index code) bounding the window: a group is on
// the fast path iff its smallest key >= kKeyLo and its largest < kKeyHi
constexpr uint32_t kKeyLo = (uint32_t)kWinLo << 23;
constexpr uint32_t kKeyHi = 128u << 23;

struct MaskPart {
  unsigned long long hi, lo;  // window sum = hi * 2^32 + lo
  uint32_t binned;            // nonzero: this workgroup wrote its 256 bins
  uint32_t pad[3];
};
static_assert(sizeof(MaskPart) == 32, "mask partial record");

// keys: |h| (15 bits) in bits 16..30 above a 3-bit code (bits 0..2) that
// ranks a lower index higher; all keys of a group are distinct, a larger
// key ranks first, and bits 3..15 are zero, so 0x80 >> (key & 31) is the
// mask bit of the key's element (the mask keeps the shift defined; the
// shift instruction reads only those five bits anyway, so it costs
// nothing).
__device__ __forceinline__ uint32_t drop_bit(uint32_t key) { return 0x80u >> (key & 31u); }

__device__ __forceinline__ uint32_t min3(uint32_t a, uint32_t b, uint32_t c) { return min(min(a, b), c); }
__device__ __forceinline__ uint32_t max3(uint32_t a, uint32_t b, uint32_t c) { return max(max(a, b), c); }

__device__ __forceinline__ void cswap(uint32_t& a, uint32_t& b) {
  uint32_t lo = min(a, b), hi = max(a, b);
  a = lo;
  b = hi;
}

// mask bits of one 8-group (w = 8 bf16, element j in bits 16j..16j+15 of
// the four words) for the pattern N:M: every element but the M-N smallest
// keys of each group of M; kmin / kmax receive the smallest and largest
// rank key of the eight
template <int N, int M>
__device__ __forceinline__ uint32_t group_mask(const uint32_t w[4], uint32_t& kmin, uint32_t& kmax) {
  uint32_t key[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = w[i] & 0x7fff7fffu;
    key[2 * i] = (a << 16) | (uint32_t)(7 - 2 * i);
    key[2 * i + 1] = (a & 0xffff0000u) | (uint32_t)(6 - 2 * i);
  }
  if (N == M) {
    kmin = min(min3(key[0], key[1], key[2]), min3(key[3], key[4], min3(key[5], key[6], key[7])));
    kmax = max(max3(key[0], key[1], key[2]), max3(key[3], key[4], max3(key[5], key[6], key[7])));
    return 0xffu;
  }
  if (M == 4) {
    // 2:4 -- per half of four, drop the two smallest keys
    uint32_t drop = 0, lo[2], hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t p0 = min(key[4 * h], key[4 * h + 1]), P0 = max(key[4 * h], key[4 * h + 1]);
      uint32_t p1 = min(key[4 * h + 2], key[4 * h + 3]), P1 = max(key[4 * h + 2], key[4 * h + 3]);
      lo[h] = min(p0, p1);                   // smallest of four
      const uint32_t t = min3(max(p0, p1), P0, P1);  // second smallest of four
      hi[h] = max(P0, P1);
      drop |= drop_bit(lo[h]) | drop_bit(t);
    }
    kmin = min(lo[0], lo[1]);
    kmax = max(hi[0], hi[1]);
    return 0xffu & ~drop;
  } else if (N == 6) {
    // 6:8 -- drop the smallest and the second smallest of eight
    uint32_t p[4], P[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = min(key[2 * i], key[2 * i + 1]);
      P[i] = max(key[2 * i], key[2 * i + 1]);
    }
    const uint32_t q1 = min(p[0], p[1]), q2 = min3(max(p[0], p[1]), P[0], P[1]);
    const uint32_t r1 = min(p[2], p[3]), r2 = min3(max(p[2], p[3]), P[2], P[3]);
    kmin = min(q1, r1);
    const uint32_t second = min3(max(q1, r1), q2, r2);
    kmax = max(max3(P[0], P[1], P[2]), P[3]);
    return 0xffu ^ drop_bit(kmin) ^ drop_bit(second);
  } else {
    // general N of 8: sort (Batcher odd-even merge network, 19 swaps),
    // drop the 8-N smallest
    uint32_t s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = key[j];
    cswap(s[0], s[1]); cswap(s[2], s[3]); cswap(s[4], s[5]); cswap(s[6], s[7]);
    cswap(s[0], s[2]); cswap(s[1], s[3]); cswap(s[4], s[6]); cswap(s[5], s[7]);
    cswap(s[1], s[2]); cswap(s[5], s[6]);
    cswap(s[0], s[4]); cswap(s[1], s[5]); cswap(s[2], s[6]); cswap(s[3], s[7]);
    cswap(s[2], s[4]); cswap(s[3], s[5]);
    cswap(s[1], s[2]); cswap(s[3], s[4]); cswap(s[5], s[6]);
    uint32_t drop = 0;
#pragma unroll
    for (int j = 0; j < 8 - N; ++j) drop |= drop_bit(s[j]);
    kmin = s[0];
    kmax = s[7];
    return 0xffu & ~drop;
  }
}

// window sum of one 8-group whose eight magnitudes are nonzero, in the
// window and within 2^13 of each other (exponent fields at most 13 apart),
// as hi * 2^32 + lo: in units of the smallest one's last bit they are
// integers below 2^21, so every partial sum in binary32 is exact (below
// 2^24 of those units) and so is the total s < 16, a multiple of 2^-59;
// hi = floor(s 2^27), lo = frac(s 2^27) 2^32 (both conversions exact)
__device__ __forceinline__ void group_sum_f32(const uint32_t w[4], uint32_t& hi, uint32_t& lo) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += __builtin_fabsf(__uint_as_float(w[i] << 16));
    s += __builtin_fabsf(__uint_as_float(w[i] & 0xffff0000u));
  }
  const float t = s * 0x1p27f;
  hi = (uint32_t)t;
  lo = (uint32_t)(__builtin_amdgcn_fractf(t) * 0x1p32f);
}

// window sum of one 8-group whose eight magnitudes are all nonzero and in
// the window
__device__ __forceinline__ unsigned long long group_sum_window(const uint32_t w[4]) {
  unsigned long long s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = w[j >> 1] >> (16 * (j & 1));
    const uint32_t e = (h >> 7) & 0xffu;
    const uint32_t sig = (h & 0x7fu) | 0x80u;
    s += (unsigned long long)sig << (e - (uint32_t)kWinLo);
  }
  return s;
}

// exact per-element path: the window sum of the in-window magnitudes
// (kept ones only when MASKED); every other nonzero magnitude goes to its
// exponent bin
template <bool MASKED>
__device__ __forceinline__ unsigned long long group_sum_exact(const uint32_t w[4], uint32_t keep,
                                                              unsigned long long* bins,
                                                              uint32_t& binned) {
  unsigned long long s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint32_t a = (w[j >> 1] >> (16 * (j & 1))) & 0x7fffu;
    if (MASKED && !((keep >> j) & 1u)) a = 0;
    const uint32_t e = a >> 7;
    const uint32_t sig = (a & 0x7fu) | (e ? 0x80u : 0u);
    if (e >= (uint32_t)kWinLo && e < 128u) {
      s += (unsigned long long)sig << (e - (uint32_t)kWinLo);
    } else if (a != 0u) {
      atomicAdd(&bins[e], (unsigned long long)sig);
      binned = 1;
    }
  }
  return s;
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
// sums.  Workgroup b (of nb) covers the contiguous 8-groups [b*per,
// (b+1)*per); every load instruction of a wavefront reads 1 KiB of
// consecutive weights.  The body is shared by the single-layer kernel and
// the grouped one (which runs it for several (layer, b) in turn).
struct MaskShared {
  unsigned long long bins[256];
  unsigned long long part[2][4];
  uint32_t any_binned;
};
template <int N, int M, bool MASKED>
__device__ __forceinline__ void mask_gamma_body(const uint4* __restrict__ W, int64_t ngroups,
                                                int64_t per, uint8_t* __restrict__ mask,
                                                char* __restrict__ ws, int64_t b, int64_t nb,
                                                MaskShared& sh) {
  unsigned long long* bins = sh.bins;
  __syncthreads();  // the shared arrays are free (a previous body may have used them)
  bins[threadIdx.x] = 0ull;
  if (threadIdx.x == 0) sh.any_binned = 0;
  __syncthreads();
  unsigned long long hi = 0, lo = 0;
  uint32_t binned = 0;
  const int64_t g_begin = b * per;
  const int64_t g_end = g_begin + per < ngroups ? g_begin + per : ngroups;
  for (int64_t c0 = g_begin; c0 < g_end; c0 += kMaskGroupsPerPass) {
    uint4 v[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t grp = c0 + 256 * g + threadIdx.x;
      u32x4 x = u32x4{0u, 0u, 0u, 0u};
      if (grp < g_end) x = ld_global(reinterpret_cast<const u32x4*>(W + grp));
      v[g] = make_uint4(x[0], x[1], x[2], x[3]);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t grp = c0 + 256 * g + threadIdx.x;
      if (grp >= g_end) break;
      const uint32_t w[4] = {v[g].x, v[g].y, v[g].z, v[g].w};
      uint32_t kmin, kmax;
      const uint32_t keep = group_mask<N, M>(w, kmin, kmax);
      st_global(mask + grp, (uint8_t)keep);
      uint32_t ghi, glo;
      group_sum_f32(w, ghi, glo);
      const bool inwin = kmin >= kKeyLo && kmax < kKeyHi;
      if (MASKED || !inwin || (kmax >> 23) - (kmin >> 23) > 13u) {
        unsigned long long gs;
        if (!MASKED && inwin)
          gs = group_sum_window(w);
        else
          gs = group_sum_exact<MASKED>(w, keep, bins, binned);
        ghi = (uint32_t)(gs >> 32);
        glo = (uint32_t)gs;
      }
      lo += glo;
      hi += ghi;
    }
  }
  hi = wave_sum_u64(hi);
  lo = wave_sum_u64(lo);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    sh.part[0][wave] = hi;
    sh.part[1][wave] = lo;
  }
  if (binned) sh.any_binned = 1;
  __syncthreads();
  MaskPart* rec = reinterpret_cast<MaskPart*>(ws) + b;
  if (threadIdx.x == 0) {
    MaskPart r;
    r.hi = sh.part[0][0] + sh.part[0][1] + sh.part[0][2] + sh.part[0][3];
    r.lo = sh.part[1][0] + sh.part[1][1] + sh.part[1][2] + sh.part[1][3];
    r.binned = sh.any_binned;
    r.pad[0] = r.pad[1] = r.pad[2] = 0;
    *rec = r;
  }
  if (sh.any_binned) {
    unsigned long long* out =
        reinterpret_cast<unsigned long long*>(ws + (size_t)nb * sizeof(MaskPart)) + (size_t)b * 256;
    out[threadIdx.x] = bins[threadIdx.x];
  }
}

template <int N, int M, bool MASKED>
__global__ __launch_bounds__(256) void mask_gamma_kernel(const uint4* __restrict__ W,
                                                        int64_t ngroups, int64_t per,
                                                        uint8_t* __restrict__ mask,
                                                        char* __restrict__ ws) {
  __shared__ MaskShared sh;
  mask_gamma_body<N, M, MASKED>(W, ngroups, per, mask, ws, blockIdx.x, gridDim.x, sh);
}

// Kernel 2 (one workgroup of 256): gamma = (sum of the partials) / count,
// the sum rounded once to binary64.
__device__ __forceinline__ void gamma_finalize_body(const char* __restrict__ ws, int nblocks,
                                                    double* __restrict__ gamma, double count,
                                                    MaskShared& sh) {
  unsigned long long(&part)[2][4] = sh.part;
  unsigned long long* bins = sh.bins;
  uint32_t& any_binned = sh.any_binned;
  __syncthreads();  // the shared arrays are free (a previous body may have used them)
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
  if (threadIdx.x == 0) {  // (no early return: the grouped kernel loops over layers)
    Big big;
#pragma unroll
    for (int i = 0; i < 10; ++i) big.limb[i] = 0;
    big_add(big, part[0][0] + part[0][1] + part[0][2] + part[0][3], kWinLo - 1 + 32);
    big_add(big, part[1][0] + part[1][1] + part[1][2] + part[1][3], kWinLo - 1);
    if (any_binned)
      for (int e = 0; e < 256; ++e)
        if (bins[e]) big_add(big, bins[e], e > 0 ? e - 1 : 0);
    *gamma = big_round(big) / count;
  }
}

__global__ __launch_bounds__(256) void gamma_finalize_kernel(const char* __restrict__ ws,
                                                             int nblocks, double* __restrict__ gamma,
                                                             double count) {
  __shared__ MaskShared sh;
  gamma_finalize_body(ws, nblocks, gamma, count, sh);
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
__device__ __forceinline__ void ternary_pack_body(const uint16_t* __restrict__ W,
                                                  const uint8_t* __restrict__ mask,
                                                  const double* __restrict__ gamma,
                                                  int64_t n_out, int64_t k,
                                                  uint32_t* __restrict__ packed,
                                                  int8_t* __restrict__ wq, int64_t chunk) {
  constexpr int kWords = block_bytes(S) / 4;
  constexpr int kField = 8 + S;
  const int64_t nkb = k / kBlockK;
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
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

// Packed blocks only (no int8 codes): the same fields as ternary_pack_body
// with fewer instructions.  All sixteen group loads of a chunk are issued
// before any field is formed (rows past n_out read the last row and get
// keep = 0).  Per 8-group, with d = h - thr taken per 16-bit half, bit 15
// of d is (|h| < thr) xor sign(h); v_perm spreads bit 15 / 31 of each word
// into 0x00 / 0xff bytes and v_sad_u8 sums the selected bits, so the
// kept-nonzero and negative bit sets take a few word operations.  The sign
// bits are compacted through two 256-entry tables in LDS, indexed by
// (nonzero nibble, negative nibble) of each half of four:
//   lo[i] = nz | pext(neg, nz) << 4         (signs from the bottom)
//   hi[i] = rev4(pext(neg, nz)) | nz << 4   (signs from the top)
// so that field = lo[low half] | hi[high half] << S.
struct PackTables {
  uint8_t lo[256], hi[256];
};

__device__ __forceinline__ void build_pack_tables(PackTables& t) {
  const uint32_t i = threadIdx.x;  // blockDim.x == 256
  const uint32_t nz = i >> 4, neg = i & 15u;
  uint32_t p = 0, n = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if ((nz >> b) & 1u) {
      p |= ((neg >> b) & 1u) << n;
      ++n;
    }
  uint32_t r = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) r |= ((p >> b) & 1u) << (3 - b);
  t.lo[i] = (uint8_t)(nz | (p << 4));
  t.hi[i] = (uint8_t)(r | (nz << 4));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// bit j of the result = bit 15 (j even) or 31 (j odd) of word j / 2
__device__ __forceinline__ uint32_t gather_top_bits(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3) {
  const uint32_t lo = __builtin_amdgcn_perm(x1, x0, 0x0b0a0908u) & 0x08040201u;
  const uint32_t hi = __builtin_amdgcn_perm(x3, x2, 0x0b0a0908u) & 0x80402010u;
  return __builtin_amdgcn_sad_u8(hi, 0u, __builtin_amdgcn_sad_u8(lo, 0u, 0u));
}

__device__ __forceinline__ uint32_t sub_halves(uint32_t x, uint32_t thr2) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, x) - __builtin_bit_cast(u16x2, thr2));
}

template <int S>
__device__ __forceinline__ uint32_t fast_field(const u32x4& x, uint32_t keep, uint32_t thr2,
                                               const PackTables& t) {
  const uint32_t d8 = gather_top_bits(sub_halves(x[0], thr2), sub_halves(x[1], thr2),
                                      sub_halves(x[2], thr2), sub_halves(x[3], thr2));
  const uint32_t s8 = gather_top_bits(x[0], x[1], x[2], x[3]);
  const uint32_t nz = keep & ~(d8 ^ s8);  // kept and |h| >= thr
  const uint32_t neg = s8 & nz;
  const uint32_t ilo = ((nz << 4) & 0xf0u) | (neg & 0x0fu);
  const uint32_t ihi = (nz & 0xf0u) | (neg >> 4);
  return (uint32_t)t.lo[ilo] | ((uint32_t)t.hi[ihi] << S);
}

template <int S>
__device__ __forceinline__ void pack_fast_body(const uint16_t* __restrict__ W,
                                               const uint8_t* __restrict__ mask, uint32_t thr,
                                               int64_t n_out, int64_t k,
                                               uint32_t* __restrict__ packed, int64_t chunk,
                                               const PackTables& tab) {
  constexpr int kWords = block_bytes(S) / 4;
  constexpr int kField = 8 + S;
  const int64_t nkb = k / kBlockK;
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  if (chunk >= strips * nkb * kStripRows) return;
  const int64_t sb = chunk / kStripRows;  // superblock = strip * nkb + kb
  const int c = (int)(chunk - sb * kStripRows);
  const int64_t strip = sb / nkb, kb = sb - strip * nkb;
  const uint32_t thr2 = thr * 0x10001u;
  // field f: row 16 (f >> 2) + (c & 15) of the strip, group
  // 8 ((f >> 1) & 1) + 2 (c >> 4) + (f & 1) of the block (see field_row /
  // field_group): per row, groups 2 (c >> 4) + {0, 1, 8, 9}
  u32x4 v[16];
  uint32_t keep[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t row = strip * kStripRows + 16 * q + (c & 15);
    const bool ok = row < n_out;
    const int64_t r = ok ? row : n_out - 1;
    const uint16_t* wr = W + r * k + kb * kBlockK + 16 * (c >> 4);
    v[4 * q + 0] = ld_global(reinterpret_cast<const u32x4*>(wr));
    v[4 * q + 1] = ld_global(reinterpret_cast<const u32x4*>(wr + 8));
    v[4 * q + 2] = ld_global(reinterpret_cast<const u32x4*>(wr + 64));
    v[4 * q + 3] = ld_global(reinterpret_cast<const u32x4*>(wr + 72));
    const uint8_t* mr = mask + r * (k / 8) + kb * 16 + 2 * (c >> 4);
    const uint32_t m0 = ld_global(reinterpret_cast<const uint16_t*>(mr));
    const uint32_t m1 = ld_global(reinterpret_cast<const uint16_t*>(mr + 8));
    keep[2 * q] = ok ? m0 : 0u;
    keep[2 * q + 1] = ok ? m1 : 0u;
  }
  uint32_t out[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) out[i] = 0;
#pragma unroll
  for (int f = 0; f < 16; ++f) {
    const uint32_t kp = (keep[f >> 1] >> (8 * (f & 1))) & 0xffu;
    const uint32_t field = fast_field<S>(v[f], kp, thr2, tab);
    const int off = f * kField;
    out[off >> 5] |= field << (off & 31);
    if ((off & 31) + kField > 32) out[(off >> 5) + 1] |= field >> (32 - (off & 31));
  }
  uint32_t* dst = packed + chunk * kWords;
#pragma unroll
  for (int i = 0; i < kWords; ++i) st_global(dst + i, out[i]);
}

// code threshold as a 16-bit magnitude bound in [1, 0x8000] (0x8000: no
// magnitude qualifies)
__device__ __forceinline__ uint32_t code_threshold16(double g) {
  const uint32_t t = code_threshold(g);
  return t > 0x8000u ? 0x8000u : t;
}

template <int S>
__global__ __launch_bounds__(256) void pack_fast_kernel(const uint16_t* __restrict__ W,
                                                       const uint8_t* __restrict__ mask,
                                                       const double* __restrict__ gamma,
                                                       int64_t n_out, int64_t k,
                                                       uint32_t* __restrict__ packed) {
  __shared__ PackTables tab;
  build_pack_tables(tab);
  __syncthreads();
  pack_fast_body<S>(W, mask, code_threshold16(*gamma), n_out, k, packed,
                    (int64_t)blockIdx.x * blockDim.x + threadIdx.x, tab);
}

template <int S, bool PACKED, bool WQ>
__global__ __launch_bounds__(256) void ternary_pack_kernel(const uint16_t* __restrict__ W,
                                                          const uint8_t* __restrict__ mask,
                                                          const double* __restrict__ gamma,
                                                          int64_t n_out, int64_t k,
                                                          uint32_t* __restrict__ packed,
                                                          int8_t* __restrict__ wq) {
  ternary_pack_body<S, PACKED, WQ>(W, mask, gamma, n_out, k, packed, wq,
                                   (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// ---------------------------------------------------------------------
// 2:4 codes in the sparse-operand + index layout (the operand form of the
// gfx950 sparse int8 matrix instruction).  One thread per 32-byte chunk:
// chunk c = r + 16q of superblock (strip, kb) holds rows 16i + r of the
// strip over k = 128kb + 32q .. +31, per row tile i an index word (2 bits
// per element: the slot's position in its quad) and a value word (2 bits
// per element at bit 8(e%4) + 2(e/4): 0, 1 = +1, 3 = -1), element e =
// 2u + s for quad u, slot s.  A quad's slots: its two nonzero codes in
// position order; one nonzero at a: (0, 1) if a = 0, else (0, a) with the
// code in slot 1; none: (0, 1).  The codes are those of the dense format
// (kept by the mask and 2|W| > gamma); a quad with more than two kept
// nonzero codes (a mask that is not 2:4) keeps its first two.
// ---------------------------------------------------------------------
__device__ __forceinline__ void sp24_quad(uint32_t nz, uint32_t neg, int u, uint32_t& idx,
                                          uint32_t& val) {
  uint32_t p0 = 0, p1 = 1, c0 = 0, c1 = 0;
  if (nz) {
    const uint32_t a = __builtin_ctz(nz), rest = nz & (nz - 1);
    const uint32_t ca = ((neg >> a) & 1u) ? 3u : 1u;
    if (rest) {
      const uint32_t b = __builtin_ctz(rest);
      p0 = a; p1 = b; c0 = ca; c1 = ((neg >> b) & 1u) ? 3u : 1u;
    } else if (a == 0) {
      c0 = ca;
    } else {
      p1 = a; c1 = ca;
    }
  }
  const int e0 = 2 * u, e1 = 2 * u + 1;
  idx |= (p0 << (2 * e0)) | (p1 << (2 * e1));
  val |= (c0 << (8 * (e0 & 3) + 2 * (e0 >> 2))) | (c1 << (8 * (e1 & 3) + 2 * (e1 >> 2)));
}

__global__ __launch_bounds__(256) void pack_sp24_kernel(const uint16_t* __restrict__ W,
                                                       const uint8_t* __restrict__ mask,
                                                       const double* __restrict__ gamma,
                                                       int64_t n_out, int64_t k,
                                                       uint32_t* __restrict__ packed) {
  const int64_t chunk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nkb = k / kBlockK;
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  if (chunk >= strips * nkb * kStripRows) return;
  const int64_t sb = chunk / kStripRows;
  const int c = (int)(chunk - sb * kStripRows);
  const int64_t strip = sb / nkb, kb = sb - strip * nkb;
  const int r = c & 15, q = c >> 4;
  const uint32_t thr = code_threshold(*gamma);
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = strip * kStripRows + 16 * i + r;
    uint32_t idx = 0, val = 0;
    uint32_t nz = 0, neg = 0;  // 32 positions of the row's k slice
    if (row < n_out) {
      const uint16_t* w = W + row * k + kb * kBlockK + 32 * q;
      const uint32_t keep = *reinterpret_cast<const uint32_t*>(mask + row * (k / 8) + kb * 16 + 4 * q);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint4 v = reinterpret_cast<const uint4*>(w)[g];
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t h = (ws[j >> 1] >> (16 * (j & 1))) & 0xffffu;
          const uint32_t on = ((keep >> (8 * g + j)) & 1u) & ((h & 0x7fffu) >= thr ? 1u : 0u);
          nz |= on << (8 * g + j);
          neg |= (on & (h >> 15)) << (8 * g + j);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sp24_quad((nz >> (4 * u)) & 15u, (neg >> (4 * u)) & 15u, u, idx, val);
    out[2 * i] = idx;
    out[2 * i + 1] = val;
  }
  uint4* dst = reinterpret_cast<uint4*>(packed + chunk * 8);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

hipError_t launch_pack_sp24(const uint16_t* W, const uint8_t* mask, const double* gamma,
                            int64_t n_out, int64_t k, void* packed, hipStream_t s) {
  const unsigned blocks = (unsigned)pack_blocks(n_out, k);
  pack_sp24_kernel<<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, reinterpret_cast<uint32_t*>(packed));
  return hipGetLastError();
}

// ---------------------------------------------------------------------
// Grouped weight quantisation (several layers per launch).  Each launch
// has a fixed grid; workgroup g takes the plan's workgroups g, g + grid, ...
// and finds their layer in the plan's owner table.  Every workgroup of a
// launch runs the same number of loop trips give or take one, and the loop
// bound depends only on the plan, so every barrier inside is reached by the
// whole workgroup.
// ---------------------------------------------------------------------
template <int N, int M, bool MASKED>
__global__ __launch_bounds__(256) void mask_gamma_group_kernel(const char* __restrict__ plan) {
  __shared__ MaskShared sh;
  const QuantGroupHeader* h = reinterpret_cast<const QuantGroupHeader*>(plan);
  const QuantItemDesc* items = reinterpret_cast<const QuantItemDesc*>(plan + sizeof(QuantGroupHeader));
  const int32_t* owner = reinterpret_cast<const int32_t*>(plan + quant_owner_offset(h->count));
  // a plan made for another pattern or gamma mode: write nothing
  const int64_t total = (h->n == N && h->m == M && h->gamma_over == (MASKED ? 1 : 0)) ? h->mask_blocks : 0;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const QuantItemDesc& it = items[owner[b]];
    mask_gamma_body<N, M, MASKED>(reinterpret_cast<const uint4*>(it.W), it.ngroups, it.per,
                                  it.mask, it.ws, b - it.mblock0, it.nmblocks, sh);
  }
}

__global__ __launch_bounds__(256) void gamma_finalize_group_kernel(const char* __restrict__ plan, int n,
                                                                   int m, int gamma_over) {
  __shared__ MaskShared sh;
  const QuantGroupHeader* h = reinterpret_cast<const QuantGroupHeader*>(plan);
  const QuantItemDesc* items = reinterpret_cast<const QuantItemDesc*>(plan + sizeof(QuantGroupHeader));
  // a plan made for another pattern or gamma mode: the mask and pack
  // launches write nothing, and every item's gamma becomes a quiet NaN, so
  // the stale codes cannot pass unnoticed (every output formed with that
  // gamma is NaN)
  const bool match = h->n == n && h->m == m && h->gamma_over == gamma_over;
  for (int64_t i = blockIdx.x; i < h->count; i += gridDim.x) {
    const QuantItemDesc& it = items[i];
    if (match)
      gamma_finalize_body(it.ws, (int)it.nmblocks, it.gamma, (double)(it.n_out * it.k), sh);
    else if (threadIdx.x == 0)
      st_global(it.gamma, __builtin_nan(""));
  }
}

template <int S>
__global__ __launch_bounds__(256) void ternary_pack_group_kernel(const char* __restrict__ plan, int n,
                                                                 int m, int gamma_over) {
  __shared__ PackTables tab;
  build_pack_tables(tab);
  __syncthreads();
  const QuantGroupHeader* h = reinterpret_cast<const QuantGroupHeader*>(plan);
  const QuantItemDesc* items = reinterpret_cast<const QuantItemDesc*>(plan + sizeof(QuantGroupHeader));
  const int32_t* owner =
      reinterpret_cast<const int32_t*>(plan + quant_owner_offset(h->count)) + h->mask_blocks;
  // a plan made for another pattern or gamma mode: write nothing (its
  // packed buffers are sized for that pattern's sign slots)
  const int64_t total =
      (h->n == n && h->m == m && h->gamma_over == gamma_over && s_of(n, m) == S) ? h->pack_blocks : 0;
  for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
    const QuantItemDesc& it = items[owner[b]];
    pack_fast_body<S>(it.W, it.mask, code_threshold16(*it.gamma), it.n_out, it.k,
                      reinterpret_cast<uint32_t*>(it.packed), (b - it.pblock0) * 256 + threadIdx.x, tab);
  }
}

// ---------------------------------------------------------------------
// Per-token absmax int8 activations (quant8 / absmax8 in actq.h).  One
// block per token; optionally zeroes a workspace range.
// ---------------------------------------------------------------------
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

// ---------------------------------------------------------------------
// Latent-weight update.  The latent weights are kept in binary32 (the
// bf16 W the mask and codes read is derived from them): per element
// Wm = RN32(Wm - lr * dW) with one fused multiply-add, then W = the bf16
// nearest to Wm (ties to even).  Eight elements per thread and trip.
// ---------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void latent_update_kernel(float* __restrict__ Wm,
                                                           const float* __restrict__ dW,
                                                           int64_t n8, float lr,
                                                           uint16_t* __restrict__ W) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const f32x4 w0 = ld_global(reinterpret_cast<const f32x4*>(Wm) + 2 * i);
    const f32x4 w1 = ld_global(reinterpret_cast<const f32x4*>(Wm) + 2 * i + 1);
    const f32x4 g0 = ld_global(reinterpret_cast<const f32x4*>(dW) + 2 * i);
    const f32x4 g1 = ld_global(reinterpret_cast<const f32x4*>(dW) + 2 * i + 1);
    f32x4 r0, r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = __builtin_fmaf(-lr, g0[e], w0[e]);
      r1[e] = __builtin_fmaf(-lr, g1[e], w1[e]);
    }
    st_global(reinterpret_cast<f32x4*>(Wm) + 2 * i, r0);
    st_global(reinterpret_cast<f32x4*>(Wm) + 2 * i + 1, r1);
    u32x4 h;
    h[0] = bf16_rne(r0[0]) | (bf16_rne(r0[1]) << 16);
    h[1] = bf16_rne(r0[2]) | (bf16_rne(r0[3]) << 16);
    h[2] = bf16_rne(r1[0]) | (bf16_rne(r1[1]) << 16);
    h[3] = bf16_rne(r1[2]) | (bf16_rne(r1[3]) << 16);
    st_global(reinterpret_cast<u32x4*>(W) + i, h);
  }
}

// ---------------------------------------------------------------------
// Squared-ReLU gating (BitNet b1.58 2B4T article §一: squared ReLU in
// place of SwiGLU), fused with the down projection's activation
// quantisation.  One block per token; the bf16 values of h are held in
// registers (rows up to 256 * 8 * kGateHeld) between the absmax and the
// quantisation, longer rows recompute them from G and U.
// ---------------------------------------------------------------------
__device__ __forceinline__ uint32_t gate_h(float g, float u) {
  const float r = g > 0.f ? g : 0.f;
  const float r2 = r * r;
  return bf16_rne(r2 * u);
}

__device__ __forceinline__ uint4 gate_h8(const float* G, const float* U, int64_t v) {
  const f32x4 g0 = ld_global(reinterpret_cast<const f32x4*>(G) + 2 * v);
  const f32x4 g1 = ld_global(reinterpret_cast<const f32x4*>(G) + 2 * v + 1);
  const f32x4 u0 = ld_global(reinterpret_cast<const f32x4*>(U) + 2 * v);
  const f32x4 u1 = ld_global(reinterpret_cast<const f32x4*>(U) + 2 * v + 1);
  uint4 h;
  h.x = gate_h(g0[0], u0[0]) | (gate_h(g0[1], u0[1]) << 16);
  h.y = gate_h(g0[2], u0[2]) | (gate_h(g0[3], u0[3]) << 16);
  h.z = gate_h(g1[0], u1[0]) | (gate_h(g1[1], u1[1]) << 16);
  h.w = gate_h(g1[2], u1[2]) | (gate_h(g1[3], u1[3]) << 16);
  return h;
}

constexpr int kGateHeld = 4;
__global__ __launch_bounds__(256) void relu2_gate_kernel(const float* __restrict__ G,
                                                        const float* __restrict__ U, int64_t n,
                                                        uint16_t* __restrict__ H,
                                                        int8_t* __restrict__ xq,
                                                        float* __restrict__ scale) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const float* g = G + t * n;
  const float* u = U + t * n;
  const int64_t nvec = n / 8;
  uint4 held[kGateHeld];
  float a = 0.f;
#pragma unroll
  for (int h = 0; h < kGateHeld; ++h) {
    const int64_t i = threadIdx.x + 256 * h;
    held[h] = i < nvec ? gate_h8(g, u, i) : make_uint4(0, 0, 0, 0);
    if (i < nvec && H)
      st_global(reinterpret_cast<u32x4*>(H + t * n) + i, u32x4{held[h].x, held[h].y, held[h].z, held[h].w});
    a = fmaxf(a, absmax8(held[h]));
  }
  for (int64_t i = threadIdx.x + 256 * kGateHeld; i < nvec; i += 256) {
    const uint4 hv = gate_h8(g, u, i);
    if (H) st_global(reinterpret_cast<u32x4*>(H + t * n) + i, u32x4{hv.x, hv.y, hv.z, hv.w});
    a = fmaxf(a, absmax8(hv));
  }
  a = wave_max(a);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (threadIdx.x == 0) scale[t] = a / 127.0f;
  uint2* out = reinterpret_cast<uint2*>(xq + t * n);
#pragma unroll
  for (int h = 0; h < kGateHeld; ++h) {
    const int64_t i = threadIdx.x + 256 * h;
    if (i < nvec) out[i] = quant8(held[h], a);
  }
  for (int64_t i = threadIdx.x + 256 * kGateHeld; i < nvec; i += 256) out[i] = quant8(gate_h8(g, u, i), a);
}

__global__ __launch_bounds__(256) void relu2_gate_bwd_kernel(const float* __restrict__ dH,
                                                            const float* __restrict__ G,
                                                            const float* __restrict__ U, int64_t n8,
                                                            uint16_t* __restrict__ dG,
                                                            uint16_t* __restrict__ dU) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    uint32_t og[4], ou[4];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const f32x4 d = ld_global(reinterpret_cast<const f32x4*>(dH) + 2 * i + q);
      const f32x4 g = ld_global(reinterpret_cast<const f32x4*>(G) + 2 * i + q);
      const f32x4 u = ld_global(reinterpret_cast<const f32x4*>(U) + 2 * i + q);
      uint32_t bg[4], bu[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float r = g[e] > 0.f ? g[e] : 0.f;
        const float r2 = r * r;
        bu[e] = bf16_rne(d[e] * r2);
        const float du = d[e] * u[e];
        bg[e] = bf16_rne(du * (2.f * r));
      }
      og[2 * q] = bg[0] | (bg[1] << 16);
      og[2 * q + 1] = bg[2] | (bg[3] << 16);
      ou[2 * q] = bu[0] | (bu[1] << 16);
      ou[2 * q + 1] = bu[2] | (bu[3] << 16);
    }
    st_global(reinterpret_cast<u32x4*>(dG) + i, u32x4{og[0], og[1], og[2], og[3]});
    st_global(reinterpret_cast<u32x4*>(dU) + i, u32x4{ou[0], ou[1], ou[2], ou[3]});
  }
}

hipError_t launch_relu2_gate(const float* G, const float* U, int64_t tokens, int64_t n, uint16_t* H,
                             int8_t* xq, float* scale, hipStream_t s) {
  relu2_gate_kernel<<<(unsigned)tokens, 256, 0, s>>>(G, U, n, H, xq, scale);
  return hipGetLastError();
}

hipError_t launch_relu2_gate_bwd(const float* dH, const float* G, const float* U, int64_t count,
                                 uint16_t* dG, uint16_t* dU, hipStream_t s) {
  const int64_t n8 = count / 8;
  const int64_t blocks = (n8 + 255) / 256;
  relu2_gate_bwd_kernel<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(dH, G, U, n8, dG, dU);
  return hipGetLastError();
}

hipError_t launch_latent_update(float* Wm, const float* dW, int64_t count, float lr, uint16_t* W,
                                hipStream_t s) {
  const int64_t n8 = count / 8;
  const int64_t blocks = (n8 + 255) / 256;
  latent_update_kernel<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(Wm, dW, n8, lr, W);
  return hipGetLastError();
}

// ------------------------------------------------------------- launchers
template <int N, int M>
static hipError_t launch_mask(const uint16_t* W, int64_t n_out, int64_t k, int gamma_over,
                              uint8_t* mask, double* gamma, void* ws, hipStream_t s) {
  const int64_t ngroups = n_out * k / 8;
  const int64_t blocks = mask_blocks(n_out, k);
  const int64_t per = mask_groups_per_block(n_out, k);
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
  if (m == 8 && n == 3) return launch_mask<3, 8>(W, n_out, k, gamma_over, mask, gamma, ws, s);
  if (m == 8 && n == 2) return launch_mask<2, 8>(W, n_out, k, gamma_over, mask, gamma, ws, s);
  return launch_mask<2, 4>(W, n_out, k, gamma_over, mask, gamma, ws, s);
}

template <int S>
static hipError_t launch_tp(const uint16_t* W, const uint8_t* mask, const double* gamma,
                            int64_t n_out, int64_t k, void* packed, int8_t* wq, hipStream_t s) {
  const unsigned blocks = (unsigned)pack_blocks(n_out, k);
  uint32_t* p = reinterpret_cast<uint32_t*>(packed);
  if (packed && wq)
    ternary_pack_kernel<S, true, true><<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, p, wq);
  else if (packed)
    pack_fast_kernel<S><<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, p);
  else
    ternary_pack_kernel<S, false, true><<<blocks, 256, 0, s>>>(W, mask, gamma, n_out, k, p, wq);
  return hipGetLastError();
}

template <int N, int M>
static hipError_t launch_qg(const char* plan, int gamma_over, hipStream_t s) {
  if (gamma_over == 0)
    mask_gamma_group_kernel<N, M, false><<<kQuantGrid, 256, 0, s>>>(plan);
  else
    mask_gamma_group_kernel<N, M, true><<<kQuantGrid, 256, 0, s>>>(plan);
  gamma_finalize_group_kernel<<<kQuantGammaGrid, 256, 0, s>>>(plan, N, M, gamma_over);
  ternary_pack_group_kernel<s_of(N, M)><<<kQuantGrid, 256, 0, s>>>(plan, N, M, gamma_over);
  return hipGetLastError();
}

hipError_t launch_quant_group(const void* plan, int n, int m, int gamma_over, hipStream_t s) {
  const char* p = reinterpret_cast<const char*>(plan);
  if (m == 8 && n == 8) return launch_qg<8, 8>(p, gamma_over, s);
  if (m == 8 && n == 6) return launch_qg<6, 8>(p, gamma_over, s);
  if (m == 8 && n == 4) return launch_qg<4, 8>(p, gamma_over, s);
  if (m == 8 && n == 3) return launch_qg<3, 8>(p, gamma_over, s);
  if (m == 8 && n == 2) return launch_qg<2, 8>(p, gamma_over, s);
  return launch_qg<2, 4>(p, gamma_over, s);
}

hipError_t launch_ternary_pack(const uint16_t* W, const uint8_t* mask, const double* gamma,
                               int64_t n_out, int64_t k, int S, void* packed, int8_t* wq,
                               hipStream_t s) {
  if (S == 8) return launch_tp<8>(W, mask, gamma, n_out, k, packed, wq, s);
  if (S == 6) return launch_tp<6>(W, mask, gamma, n_out, k, packed, wq, s);
  if (S == 2) return launch_tp<2>(W, mask, gamma, n_out, k, packed, wq, s);
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

// gemv.hip -- decode-shaped BitLinear contraction (tokens <= 16) on gfx950.
//
// acc[t, r] = sum_c x_q[t, c] * code[r, c];  Y = acc * gamma * s_t.
// BitNet b1.58 2B4T article §四 describes the GPU recipe for ternary x int8:
// pack the ternary codes, stream them from HBM, unpack next to the compute
// and multiply with the int8 activations, to make the most of memory
// bandwidth.  This kernel keeps that shape for the bitmap+sign format and
// CDNA4:
//
//  * A wavefront owns a tile of 16 weight rows and walks k in 512-wide
//    super-tiles.  Lane l (row l%16, block l/16) loads the 2*(8+S) packed
//    bytes of one row's 128-wide k block; the 64 lanes read 64 consecutive
//    blocks, i.e. one contiguous span of the packed buffer.
//  * Each 8-group decodes from two 8-bit keys (low half: bitmap + first
//    four signs; high half: last four signs + bitmap) through two 256-entry
//    tables of int8x4 codes in LDS.  Every lane reads its own copy of the
//    tables (32 copies, one per bank) so the lookups are free of bank
//    conflicts.
//  * The codes go straight into v_mfma_i32_16x16x64_i8 as the A operand
//    (16 rows); the activations of up to 16 tokens are the B operand.  A and
//    B take the same k slice per lane group, so the dot product covers each
//    k exactly once.  int32 accumulation is exact.
//  * When a layer has too few row tiles to fill the chip, k is split into
//    ranges; partial sums meet in an int32 workspace by integer atomics
//    (order independent, hence bit-reproducible), and the last range to
//    finish a tile writes its outputs.
//  * The grouped kernel runs many such GEMVs (same token count and pattern)
//    from one device-resident plan in a single launch.
#include "common.h"
#include "launch.h"

namespace bl {

constexpr int kGemvThreads = 512;  // 8 wavefronts
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kLutCopies = 32;
constexpr int64_t kResidentWaves = 256 * 2 * kGemvWaves;  // 256 CUs x 2 blocks

__device__ __forceinline__ void fill_lut(uint32_t* lut) {
  for (int idx = threadIdx.x; idx < 512; idx += blockDim.x) {
    const uint32_t key = idx & 255, half = idx >> 8;
    const uint32_t v = half_codes(key, half);
    uint4* dst = reinterpret_cast<uint4*>(&lut[(key * 2 + half) * kLutCopies]);
#pragma unroll
    for (int c = 0; c < kLutCopies / 4; ++c) dst[c] = make_uint4(v, v, v, v);
  }
}

// partial dot products of one 16-row tile over super-tiles [st0, st1):
// returns acc of rows tile*16 + 4*(lane/16) + i for token lane%16
template <int S>
__device__ __forceinline__ v4i tile_dot(const uint32_t* __restrict__ packed,
                                        const int8_t* __restrict__ xq, int64_t tile, int64_t nkb,
                                        int64_t st0, int64_t st1, int64_t k, bool tok_ok,
                                        const uint32_t* lut_lane, int lane) {
  constexpr int kW = block_bytes(S) / 4;
  constexpr int kField = 8 + S;
  const int r16 = lane & 15, grp = lane >> 4;
  v4i c = {0, 0, 0, 0};
  for (int64_t st = st0; st < st1; ++st) {
    const int64_t kb = st * 4 + grp;
    const bool blk_ok = kb < nkb;
    uint32_t w[kW + 1];
#pragma unroll
    for (int i = 0; i <= kW; ++i) w[i] = 0;
    if (blk_ok) {
      const uint32_t* src = packed + ((tile * nkb + kb) * kTileRows + r16) * kW;
#pragma unroll
      for (int i = 0; i < kW; ++i) w[i] = src[i];
    }
    v4i b[8];
    if (blk_ok && tok_ok) {
      const v4i* xs = reinterpret_cast<const v4i*>(xq + (int64_t)r16 * k + kb * kBlockK);
#pragma unroll
      for (int m = 0; m < 8; ++m) b[m] = xs[m];
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) b[m] = v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      v4i a;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int off = (2 * m + q) * kField;
        const int offh = off + S;
        const uint32_t klo = funnel(w[(off >> 5) + 1], w[off >> 5], off & 31) & 0xffu;
        const uint32_t khi = funnel(w[(offh >> 5) + 1], w[offh >> 5], offh & 31) & 0xffu;
        a[2 * q] = (int)lut_lane[(klo * 2 + 0) * kLutCopies];
        a[2 * q + 1] = (int)lut_lane[(khi * 2 + 1) * kLutCopies];
      }
      c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[m], c, 0, 0, 0);
    }
  }
  return c;
}

__device__ __forceinline__ void store_tile(float* __restrict__ Y, int32_t* __restrict__ acc_out,
                                           const v4i& c, int64_t row0, int64_t n_out, int token,
                                           double g, double st) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + i;
    if (row < n_out) {
      Y[(int64_t)token * n_out + row] = (float)((double)c[i] * g * st);
      if (acc_out) acc_out[(int64_t)token * n_out + row] = c[i];
    }
  }
}

template <int S>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(
    const uint32_t* __restrict__ packed, const int8_t* __restrict__ xq,
    const float* __restrict__ scale, const double* __restrict__ gamma, float* __restrict__ Y,
    int32_t* __restrict__ acc_out, int32_t* __restrict__ partial, uint32_t* __restrict__ tickets,
    int tokens, int64_t k, int64_t n_out, int ksplit, int st_per_unit, int64_t units) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 2 * kLutCopies];
  fill_lut(lut);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;  // row of the A operand, token of the B operand
  const int grp = lane >> 4;  // which 128-wide block of the super-tile
  const uint32_t* lut_lane = lut + (lane & (kLutCopies - 1));
  const int64_t nkb = k / kBlockK;
  const int64_t nst = (nkb + 3) / 4;
  const double g = *gamma;
  const bool tok_ok = r16 < tokens;
  const double st = tok_ok ? (double)scale[r16] : 0.0;

  for (int64_t u = (int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6); u < units;
       u += (int64_t)gridDim.x * kGemvWaves) {
    const int64_t tile = u / ksplit;
    const int part = (int)(u - tile * ksplit);
    const int64_t st0 = (int64_t)part * st_per_unit;
    const int64_t st1 = min(st0 + st_per_unit, nst);
    const v4i c = tile_dot<S>(packed, xq, tile, nkb, st0, st1, k, tok_ok, lut_lane, lane);
    const int64_t row0 = tile * kTileRows + 4 * grp;
    if (ksplit == 1) {
      if (tok_ok) store_tile(Y, acc_out, c, row0, n_out, r16, g, st);
      continue;
    }
    if (tok_ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + i;
        if (row < n_out && c[i] != 0) atomicAdd(&partial[(int64_t)r16 * n_out + row], c[i]);
      }
    }
    __threadfence();
    uint32_t t = 0;
    if (lane == 0) t = atomicAdd(&tickets[tile], 1u);
    t = __shfl(t, 0, 64);
    if (t != (uint32_t)(ksplit - 1)) continue;
    // last range of this tile: collect the sums and leave the workspace
    // zeroed for the next call (no memset needed)
    __threadfence();
    if (tok_ok) {
      v4i tot;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = row0 + i;
        tot[i] = row < n_out ? atomicExch(&partial[(int64_t)r16 * n_out + row], 0) : 0;
      }
      store_tile(Y, acc_out, tot, row0, n_out, r16, g, st);
    }
    if (lane == 0) atomicExch(&tickets[tile], 0u);
  }
}

template <int S>
__global__ __launch_bounds__(kGemvThreads) void gemv_group_kernel(const char* __restrict__ plan) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 2 * kLutCopies];
  fill_lut(lut);
  __syncthreads();
  const GroupHeader* hdr = reinterpret_cast<const GroupHeader*>(plan);
  const GroupItem* items = reinterpret_cast<const GroupItem*>(plan + sizeof(GroupHeader));
  const uint32_t* units_tab =
      reinterpret_cast<const uint32_t*>(items + hdr->count) + hdr->rows;
  const int tokens = hdr->tokens;
  const int64_t units = hdr->units;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, grp = lane >> 4;
  const bool tok_ok = r16 < tokens;
  const uint32_t* lut_lane = lut + (lane & (kLutCopies - 1));
  for (int64_t u = (int64_t)blockIdx.x * kGemvWaves + (threadIdx.x >> 6); u < units;
       u += (int64_t)gridDim.x * kGemvWaves) {
    const uint32_t e = units_tab[u];
    const GroupItem it = items[e >> 16];
    const int64_t tile = e & 0xffffu;
    const int64_t nkb = it.k / kBlockK;
    const v4i c = tile_dot<S>(it.packed, it.xq, tile, nkb, 0, (nkb + 3) / 4, it.k, tok_ok, lut_lane, lane);
    if (tok_ok)
      store_tile(it.Y, nullptr, c, tile * kTileRows + 4 * grp, it.n_out, r16, *it.gamma,
                 (double)it.scale[r16]);
  }
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

GemvPlan plan_gemv(int64_t tokens, int64_t k, int64_t n_out) {
  GemvPlan p;
  const int64_t tiles = (n_out + kTileRows - 1) / kTileRows;
  const int64_t nst = (k / kBlockK + 3) / 4;
  int64_t ks = 1;
  if (tiles < kResidentWaves) ks = (kResidentWaves + tiles - 1) / tiles;
  if (ks > nst) ks = nst;
  if (ks < 1) ks = 1;
  const int64_t per = (nst + ks - 1) / ks;
  ks = (nst + per - 1) / per;
  p.ksplit = (int)ks;
  p.st_per_unit = (int)per;
  p.units = tiles * ks;
  p.ws_bytes = ks > 1 ? align256((size_t)tokens * n_out * 4) + align256((size_t)tiles * 4) : 0;
  return p;
}

size_t gemv_ws_bytes_max(int64_t tokens, int64_t k, int64_t n_out) {
  return plan_gemv(tokens, k, n_out).ws_bytes;
}

template <int S>
static hipError_t launch_gemv_s(const void* packed, const int8_t* xq, const float* scale,
                                const double* gamma, float* Y, int32_t* acc, void* ws, int tokens,
                                int64_t k, int64_t n_out, hipStream_t s) {
  const GemvPlan p = plan_gemv(tokens, k, n_out);
  int32_t* partial = nullptr;
  uint32_t* tickets = nullptr;
  if (p.ksplit > 1) {
    partial = reinterpret_cast<int32_t*>(ws);
    tickets = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) +
                                          align256((size_t)tokens * n_out * 4));
  }
  int64_t blocks = (p.units + kGemvWaves - 1) / kGemvWaves;
  if (blocks > 512) blocks = 512;
  gemv_kernel<S><<<(unsigned)blocks, kGemvThreads, 0, s>>>(
      reinterpret_cast<const uint32_t*>(packed), xq, scale, gamma, Y, acc, partial, tickets,
      tokens, k, n_out, p.ksplit, p.st_per_unit, p.units);
  return hipGetLastError();
}

hipError_t launch_gemv(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, int32_t* acc, void* ws, int tokens,
                       int64_t k, int64_t n_out, int S, hipStream_t s) {
  if (S == 8) return launch_gemv_s<8>(packed, xq, scale, gamma, Y, acc, ws, tokens, k, n_out, s);
  if (S == 6) return launch_gemv_s<6>(packed, xq, scale, gamma, Y, acc, ws, tokens, k, n_out, s);
  return launch_gemv_s<4>(packed, xq, scale, gamma, Y, acc, ws, tokens, k, n_out, s);
}

hipError_t launch_gemv_group(const void* plan, int S, hipStream_t s) {
  const char* p = reinterpret_cast<const char*>(plan);
  if (S == 8) gemv_group_kernel<8><<<512, kGemvThreads, 0, s>>>(p);
  else if (S == 6) gemv_group_kernel<6><<<512, kGemvThreads, 0, s>>>(p);
  else gemv_group_kernel<4><<<512, kGemvThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bl

// bwd.hip -- dual straight-through backward of BitLinear on gfx950.
//
// Sparse-BitNet article §三 and §六: the gradient passes straight through
// the ternary rounding and the N:M sparsification, and a masked weight
// still receives its gradient.
//   dX[t, c] = gamma * sum_r dY[t, r] * code[r, c]     (through the masked
//              ternary weights the forward used)
//   dW[r, c] = sum_t dY[t, r] * s_t * x_q[t, c]        (dense)
// Both run on v_mfma_f32_16x16x32_bf16 with binary32 accumulation.  codes
// and x_q are exact in bf16; dY * s_t is rounded to bf16 once.
//
// Tiles: 128 x 128 outputs per workgroup of 4 wavefronts (2 x 2, 64 x 64
// each), contraction step 64.  Operands whose contraction index is not the
// contiguous one in memory are transposed while staging into LDS.
#include "common.h"
#include "launch.h"

namespace bl {

constexpr int kP = 72;  // LDS row pitch in bf16 elements (64 + 8)

__device__ __forceinline__ uint16_t code_bf16(uint32_t byte) {
  // 0x01 -> +1.0, 0xff -> -1.0, 0 -> 0
  return byte == 0u ? (uint16_t)0 : (byte == 1u ? (uint16_t)0x3f80 : (uint16_t)0xbf80);
}

__device__ __forceinline__ void mma_tile(const uint16_t* As, const uint16_t* Bs, int wm, int wn,
                                         int lane, v4f c[4][4]) {
  const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    v8bf a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const v8bf*>(As + (wm * 64 + i * 16 + l16) * kP + kk * 32 + lg * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const v8bf*>(Bs + (wn * 64 + j * 16 + l16) * kP + kk * 32 + lg * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], c[i][j], 0, 0, 0);
  }
}

// dX tile: 128 tokens (blockIdx.y) x one 128-wide k block (blockIdx.x)
template <int S>
__global__ __launch_bounds__(256) void dx_kernel(const uint16_t* __restrict__ dY,
                                                const uint32_t* __restrict__ packed,
                                                const double* __restrict__ gamma,
                                                float* __restrict__ dX, int64_t tokens, int64_t k,
                                                int64_t n_out) {
  constexpr int kW = block_bytes(S) / 4;
  __shared__ __attribute__((aligned(16))) uint16_t As[128 * kP];  // [t][r]
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * kP];  // [c][r]
  __shared__ uint32_t lut[512];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  for (int idx = tid; idx < 512; idx += 256) lut[idx] = half_codes(idx & 255, idx >> 8);
  const int64_t m0 = (int64_t)blockIdx.y * 128;
  const int64_t kb = blockIdx.x;
  const int64_t nkb = k / kBlockK;

  v4f c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t r0 = 0; r0 < n_out; r0 += 64) {
    __syncthreads();
    {  // A: dY[m0 + t][r0 .. r0+63], thread: token tid/2, 32 r's
      const int t = tid >> 1, h = tid & 1;
      const int64_t tt = m0 + t;
      u32x4* dst = reinterpret_cast<u32x4*>(As + t * kP + h * 32);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + h * 32 + i * 8;
        const bool ok = tt < tokens && r < n_out;
        dst[i] = ok ? *reinterpret_cast<const u32x4*>(dY + tt * n_out + r) : u32x4{0u, 0u, 0u, 0u};
      }
    }
    {  // B: codes of rows r0 .. r0+63 (one packed superblock) for block
       // kb, written transposed [c][r]; wavefront w decodes fields
       // 4w..4w+3 of chunk `lane` (row tile w of the strip; padding rows
       // of the last strip hold zero codes)
      const int ch = lane;
      uint32_t w[kW + 1];
#pragma unroll
      for (int i = 0; i <= kW; ++i) w[i] = 0;
      {
        const uint32_t* src = packed + (((r0 / kStripRows) * nkb + kb) * kStripRows + ch) * kW;
#pragma unroll
        for (int i = 0; i < kW; ++i) w[i] = src[i];
      }
      auto lk = [&](uint32_t key, int half) { return lut[half * 256 + key]; };
      auto emit = [&](int f, uint32_t lo, uint32_t hi) {
        const int rr = field_row(ch, f), gi = field_group(ch, f);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          Bs[(gi * 8 + p) * kP + rr] = code_bf16((lo >> (8 * p)) & 0xffu);
          Bs[(gi * 8 + 4 + p) * kP + rr] = code_bf16((hi >> (8 * p)) & 0xffu);
        }
      };
      switch (wave) {
        case 0: decode_groups<S, 0, 4>(w, lk, emit); break;
        case 1: decode_groups<S, 4, 4>(w, lk, emit); break;
        case 2: decode_groups<S, 8, 4>(w, lk, emit); break;
        default: decode_groups<S, 12, 4>(w, lk, emit); break;
      }
    }
    __syncthreads();
    mma_tile(As, Bs, wm, wn, lane, c);
  }
  const double g = *gamma;
  const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = m0 + wm * 64 + i * 16 + 4 * lg + q;
      if (t >= tokens) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = kb * kBlockK + wn * 64 + j * 16 + l16;
        dX[t * k + col] = (float)((double)c[i][j][q] * g);
      }
    }
}

// dW tile: 128 weight rows (blockIdx.y) x 128 input columns (blockIdx.x)
__global__ __launch_bounds__(256) void dw_kernel(const uint16_t* __restrict__ dY,
                                                const int8_t* __restrict__ xq,
                                                const float* __restrict__ scale,
                                                float* __restrict__ dW, int64_t tokens, int64_t k,
                                                int64_t n_out) {
  __shared__ __attribute__((aligned(16))) uint16_t As[128 * kP];  // [r][t]
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * kP];  // [c][t]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t r0 = (int64_t)blockIdx.y * 128;
  const int64_t c0 = (int64_t)blockIdx.x * 128;

  v4f c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = 0; t0 < tokens; t0 += 64) {
    __syncthreads();
    const int t = tid >> 2, q = tid & 3;  // token, quarter (32 columns)
    const int64_t tt = t0 + t;
    {  // A: (dY[tt][r0 + ...] * s_tt) as bf16, transposed to [r][t]
      const float s = tt < tokens ? scale[tt] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + q * 32 + i * 8;
        const bool ok = tt < tokens && r < n_out;
        const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(dY + tt * n_out + r) : u32x4{0u, 0u, 0u, 0u};
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
          As[(q * 32 + i * 8 + e) * kP + t] = f32_to_bf16_rne(x * s);
        }
      }
    }
    {  // B: x_q[tt][c0 + ...] as bf16 (exact), transposed to [c][t]
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4 v = tt < tokens ? *reinterpret_cast<const u32x4*>(xq + tt * k + c0 + q * 32 + i * 16)
                                    : u32x4{0u, 0u, 0u, 0u};
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int8_t b = (int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
          Bs[(q * 32 + i * 16 + e) * kP + t] = f32_to_bf16_rne((float)b);
        }
      }
    }
    __syncthreads();
    mma_tile(As, Bs, wm, wn, lane, c);
  }
  const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = r0 + wm * 64 + i * 16 + 4 * lg + q;
      if (r >= n_out) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) dW[r * k + c0 + wn * 64 + j * 16 + l16] = c[i][j][q];
    }
}

template <int S>
static hipError_t launch_dx_s(const uint16_t* dY, const void* packed, const double* gamma, float* dX,
                              int64_t tokens, int64_t k, int64_t n_out, hipStream_t s) {
  dim3 grid((unsigned)(k / kBlockK), (unsigned)((tokens + 127) / 128));
  dx_kernel<S><<<grid, 256, 0, s>>>(dY, reinterpret_cast<const uint32_t*>(packed), gamma, dX,
                                    tokens, k, n_out);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dY, const void* packed, const double* gamma, float* dX,
                         int64_t tokens, int64_t k, int64_t n_out, int S, hipStream_t s) {
  if (S == 8) return launch_dx_s<8>(dY, packed, gamma, dX, tokens, k, n_out, s);
  if (S == 6) return launch_dx_s<6>(dY, packed, gamma, dX, tokens, k, n_out, s);
  return launch_dx_s<4>(dY, packed, gamma, dX, tokens, k, n_out, s);
}

hipError_t launch_bwd_dw(const uint16_t* dY, const int8_t* xq, const float* scale, float* dW,
                         int64_t tokens, int64_t k, int64_t n_out, hipStream_t s) {
  dim3 grid((unsigned)(k / 128), (unsigned)((n_out + 127) / 128));
  dw_kernel<<<grid, 256, 0, s>>>(dY, xq, scale, dW, tokens, k, n_out);
  return hipGetLastError();
}

}  // namespace bl

// gemm.hip -- prefill-shaped BitLinear contraction (many tokens) on gfx950.
//
// acc[t, r] = sum_c x_q[t, c] * code[r, c];  Y = acc * gamma * s_t.
// The ternary codes are decoded once per 128-wide k block into an LDS tile
// and reused by every token row of the workgroup, so the decode cost is
// amortised over the token dimension and the loop is bound by the int8
// matrix cores (v_mfma_i32_16x16x64_i8).  The pages' custom sparse operator
// (Sparse-BitNet article §四) gains from hardware 6:8 support on other
// hardware; gfx950 has no 6:8 matrix instruction, so the dense int8 MFMA
// multiplies the pruned zeros and the format only saves weight bytes.
//
// Tile: 128 tokens x 128 weight rows per workgroup of 4 wavefronts (2 x 2,
// 64 x 64 each, 4 x 4 MFMA tiles of 16 x 16), k step 128.
#include "common.h"
#include "launch.h"

namespace bl {

constexpr int kBM = 128, kBN = 128, kPitch = 144;  // LDS row pitch in bytes

template <int S>
__global__ __launch_bounds__(256) void gemm_kernel(const uint32_t* __restrict__ packed,
                                                  const int8_t* __restrict__ xq,
                                                  const float* __restrict__ scale,
                                                  const double* __restrict__ gamma,
                                                  float* __restrict__ Y,
                                                  int32_t* __restrict__ acc_out, int64_t tokens,
                                                  int64_t k, int64_t n_out) {
  constexpr int kW = block_bytes(S) / 4;
  __shared__ __attribute__((aligned(16))) int8_t As[kBM * kPitch];
  __shared__ __attribute__((aligned(16))) int8_t Bs[kBN * kPitch];
  __shared__ uint32_t lut[512];  // [half * 256 + key]

  const int tid = threadIdx.x;
  for (int idx = tid; idx < 512; idx += 256) lut[idx] = half_codes(idx & 255, idx >> 8);

  const int64_t m0 = (int64_t)blockIdx.y * kBM;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;
  const int64_t nkb = k / kBlockK;
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;

  // loader roles: A -- row tid/2, 64-byte half; B -- chunk tid%64 of
  // superblock (tid/64)%2 of the tile's two strips, fields 8*(tid/128) ..
  // +7 (wave-uniform, so field offsets are compile-time constants)
  const int ld_row = tid >> 1, ld_half = tid & 1;
  const int64_t a_tok = m0 + ld_row;
  const int b_sb = (tid >> 6) & 1, b_chunk = tid & 63, b_part = tid >> 7;
  const int64_t b_strip = n0 / kStripRows + b_sb;
  const bool b_ok = b_strip < strips;

  v4i c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4i{0, 0, 0, 0};

  for (int64_t kb = 0; kb < nkb; ++kb) {
    __syncthreads();  // previous tile fully consumed (and the table ready)
    // A tile: x_q[m0 .. m0+127][kb*128 .. +128]
    {
      const u32x4* src = reinterpret_cast<const u32x4*>(xq + a_tok * k + kb * kBlockK + ld_half * 64);
      u32x4* dst = reinterpret_cast<u32x4*>(As + ld_row * kPitch + ld_half * 64);
      const bool ok = a_tok < tokens;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = ok ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
    // B tile: codes of rows n0 .. n0+127 (two packed superblocks) for this
    // k block; each field lands at its (row, group) of the tile
    {
      uint32_t w[kW + 1];
#pragma unroll
      for (int i = 0; i <= kW; ++i) w[i] = 0;
      if (b_ok) {
        const uint32_t* src = packed + ((b_strip * nkb + kb) * kStripRows + b_chunk) * kW;
#pragma unroll
        for (int i = 0; i < kW; ++i) w[i] = src[i];
      }
      auto lk = [&](uint32_t key, int half) { return lut[half * 256 + key]; };
      auto emit = [&](int f, uint32_t lo, uint32_t hi) {
        const int row = b_sb * kStripRows + field_row(b_chunk, f);
        *reinterpret_cast<uint2*>(Bs + row * kPitch + 8 * field_group(b_chunk, f)) =
            make_uint2(lo, hi);
      };
      if (b_part == 0) decode_groups<S, 0, 8>(w, lk, emit);
      else decode_groups<S, 8, 8>(w, lk, emit);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      v4i a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const v4i*>(As + (wm * 64 + i * 16 + l16) * kPitch + kk * 64 + lg * 16);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const v4i*>(Bs + (wn * 64 + j * 16 + l16) * kPitch + kk * 64 + lg * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) c[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], c[i][j], 0, 0, 0);
    }
  }

  const double g = *gamma;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t t = m0 + wm * 64 + i * 16 + 4 * lg + q;
      if (t >= tokens) continue;
      const float gs = out_scale(g, scale[t]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t r = n0 + wn * 64 + j * 16 + l16;
        if (r < n_out) {
          Y[t * n_out + r] = out_value(c[i][j][q], gs);
          if (acc_out) acc_out[t * n_out + r] = c[i][j][q];
        }
      }
    }
  }
}

template <int S>
static hipError_t launch_gemm_s(const void* packed, const int8_t* xq, const float* scale,
                                const double* gamma, float* Y, int32_t* acc, int64_t tokens,
                                int64_t k, int64_t n_out, hipStream_t s) {
  dim3 grid((unsigned)((n_out + kBN - 1) / kBN), (unsigned)((tokens + kBM - 1) / kBM));
  gemm_kernel<S><<<grid, 256, 0, s>>>(reinterpret_cast<const uint32_t*>(packed), xq, scale, gamma,
                                      Y, acc, tokens, k, n_out);
  return hipGetLastError();
}

hipError_t launch_gemm(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, int32_t* acc, int64_t tokens, int64_t k,
                       int64_t n_out, int S, hipStream_t s) {
  if (S == 8) return launch_gemm_s<8>(packed, xq, scale, gamma, Y, acc, tokens, k, n_out, s);
  if (S == 6) return launch_gemm_s<6>(packed, xq, scale, gamma, Y, acc, tokens, k, n_out, s);
  return launch_gemm_s<4>(packed, xq, scale, gamma, Y, acc, tokens, k, n_out, s);
}

}  // namespace bl

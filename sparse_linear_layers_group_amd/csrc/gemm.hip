// gemm.hip -- prefill-shaped BitLinear contraction (many tokens) on gfx950.
//
// acc[t, r] = sum_c x_q[t, c] * code[r, c];  Y = acc * gamma * s_t.
// The ternary codes are decoded once per k step into an LDS tile and reused
// by every token of the workgroup, so the decode cost is amortised over the
// token dimension and the loop is bound by the int8 matrix cores
// (v_mfma_i32_16x16x64_i8).  The pages' custom sparse operator
// (Sparse-BitNet article §四) gains from hardware 6:8 support on other
// hardware; gfx950 has no 6:8 matrix instruction, so the dense int8 MFMA
// multiplies the pruned zeros and the format only saves weight bytes.
//
// Workgroup tile: 128 weight rows x BT tokens (BT = 256 or 128), 4
// wavefronts (2 along rows x 2 along tokens), each 64 rows x BT/2 tokens.
// The codes are the MFMA A operand and the activations the B operand, so
// each lane's results are 4 consecutive rows of one token: one 16-byte
// store.  k advances 64 at a time through double-buffered LDS tiles (rows
// padded to 80 bytes: the 16-byte operand reads of a quarter wavefront hit
// 16 distinct 4-bank groups).  While the MFMAs of step j run, the
// workgroup has the activations of step j+1 in flight and decodes its codes
// from packed chunks held in registers; one barrier per step.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace bl {

constexpr int kGBN = 128;       // weight rows per workgroup
constexpr int kGKS = 64;        // k per step
constexpr int kGPitch = 80;     // LDS row pitch in bytes
constexpr int kGLutCopies = 8;  // copies of the decode tables (fewer bank conflicts)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t g_rsrc(const void* p, int64_t bytes) {
  const int64_t b = bytes < 0x7fffffff ? bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)b, 0x00020000);
}

// decode fields F0, F0+1 of a chunk held in w[0..kW] (w[kW] = 0) into the
// code tile: field f is row 16*(f/4) + (c%16) of superblock sb, k bytes
// 16*(c/16) + 8*(f%2) of the step
template <int S, int F0>
__device__ __forceinline__ void decode_pair(const uint32_t* w, const uint32_t* lut_lane, int8_t* Cs,
                                            int sb, int c) {
  auto lk = [&](uint32_t key, int half) { return lut_lane[(key * 2 + half) * kGLutCopies]; };
  auto emit = [&](int f, uint32_t lo, uint32_t hi) {
    const int row = sb * kStripRows + 16 * (f >> 2) + (c & 15);
    *reinterpret_cast<uint2*>(Cs + row * kGPitch + 16 * (c >> 4) + 8 * (f & 1)) = make_uint2(lo, hi);
  };
  decode_groups<S, F0, 2>(w, lk, emit);
}

template <int S, int BT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint32_t* __restrict__ packed,
                                                  const int8_t* __restrict__ xq,
                                                  const float* __restrict__ scale,
                                                  const double* __restrict__ gamma,
                                                  float* __restrict__ Y,
                                                  int32_t* __restrict__ acc_out, int64_t tokens,
                                                  int64_t k, int64_t n_out) {
  constexpr int kW = block_bytes(S) / 4;
  constexpr int kTT = BT / 32;  // 16-token tiles per wavefront
  __shared__ __attribute__((aligned(16))) int8_t Xs[2][BT * kGPitch];
  __shared__ __attribute__((aligned(16))) int8_t Cs[2][kGBN * kGPitch];
  __shared__ __attribute__((aligned(16))) uint32_t lut[512 * kGLutCopies];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;  // wavefront: rows 64*wn.., tokens (BT/2)*wt..
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kGBN;
  const int64_t t0 = (int64_t)blockIdx.y * BT;
  const int64_t nkb = k / kBlockK;
  const int nks = (int)(k / kGKS);
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;

  for (int idx = tid; idx < 512 * kGLutCopies; idx += 256)
    lut[idx] = half_codes((idx / kGLutCopies) >> 1, (idx / kGLutCopies) & 1);
  const uint32_t* lut_lane = lut + (lane & (kGLutCopies - 1));

  // activations: thread -> token row (BT=256: one row, 64 bytes; BT=128:
  // half a row, 32 bytes) of the step
  constexpr int kXLoads = BT * kGKS / 16 / 256;  // 16-byte loads per thread
  const int x_row = BT == 256 ? tid : tid >> 1;
  const int x_col = BT == 256 ? 0 : 32 * (tid & 1);
  const __amdgpu_buffer_rsrc_t xr = g_rsrc(xq, tokens * k);
  const uint32_t x_off = (uint32_t)((t0 + x_row) * k + x_col);
  const bool x_ok = t0 + x_row < tokens;
  // codes: thread -> chunk c of superblock sb of the tile's two strips;
  // fields of row tiles 2*part, 2*part+1
  const int c_chunk = tid & 63, c_sb = (tid >> 6) & 1, c_part = tid >> 7;
  const __amdgpu_buffer_rsrc_t pr = g_rsrc(packed, strips * nkb * kStripRows * block_bytes(S));
  const int64_t c_strip = n0 / kStripRows + c_sb;
  const bool c_ok = c_strip < strips;

  // register rings: activations two steps ahead, packed chunks two k
  // blocks ahead (so global latency is covered by two steps of MFMAs)
  u32x4 xv[2][kXLoads];
  uint32_t w[2][kW + 1];
  w[0][kW] = 0;
  w[1][kW] = 0;
  auto load_x = [&](int ks, u32x4* dst) {
#pragma unroll
    for (int q = 0; q < kXLoads; ++q)
      dst[q] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, x_ok && ks < nks ? x_off + (uint32_t)(ks * kGKS + 16 * q) : 0x80000000u, 0, 0);
  };
  auto load_chunk = [&](int kb, uint32_t* dst) {
    const uint32_t o =
        c_ok && kb < nkb
            ? (uint32_t)(((c_strip * nkb + kb) * kStripRows + c_chunk) * block_bytes(S))
            : 0x80000000u;
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(pr, o, 0, 0);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    if constexpr (kW == 8) {
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(pr, o + 16, 0, 0);
      dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
    } else if constexpr (kW == 7) {
      typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 b = __builtin_amdgcn_raw_buffer_load_b96(pr, o + 16, 0, 0);
      dst[4] = b.x; dst[5] = b.y; dst[6] = b.z;
    } else {
      const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(pr, o + 16, 0, 0);
      dst[4] = b.x; dst[5] = b.y;
    }
  };
  auto store_x = [&](int p, const u32x4* src) {
#pragma unroll
    for (int q = 0; q < kXLoads; ++q)
      *reinterpret_cast<u32x4*>(&Xs[p][x_row * kGPitch + x_col + 16 * q]) = src[q];
  };
  // the codes of k half H of the chunk's 128-wide block
  auto decode = [&](auto half, const uint32_t* wc, int p) {
    constexpr int H = decltype(half)::value;
    int8_t* cs = Cs[p];
    if (c_part == 0) {
      decode_pair<S, 2 * H + 0>(wc, lut_lane, cs, c_sb, c_chunk);
      decode_pair<S, 2 * H + 4>(wc, lut_lane, cs, c_sb, c_chunk);
    } else {
      decode_pair<S, 2 * H + 8>(wc, lut_lane, cs, c_sb, c_chunk);
      decode_pair<S, 2 * H + 12>(wc, lut_lane, cs, c_sb, c_chunk);
    }
  };

  v4i c[kTT][4];
#pragma unroll
  for (int i = 0; i < kTT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4i{0, 0, 0, 0};

  // prologue: step 0 in LDS buffer 0, step 1 and k block 1 in flight
  load_x(0, xv[0]);
  load_chunk(0, w[0]);
  load_x(1, xv[1]);
  load_chunk(1, w[1]);
  __syncthreads();  // tables ready
  decode(std::integral_constant<int, 0>{}, w[0], 0);
  store_x(0, xv[0]);
  load_x(2, xv[0]);
  __syncthreads();

  // step ks (phase PH = ks % 4): MFMAs on LDS buffer ks%2; then step ks+1
  // goes into the other buffer from the registers loaded two steps ago,
  // and the loads for step ks+3 (and k block (ks+3)/2 + 1) are issued
  auto step = [&](auto phase, int ks) {
    constexpr int PH = decltype(phase)::value;
    constexpr int p = PH & 1;
    v4i a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[j] = *reinterpret_cast<const v4i*>(&Cs[p][(64 * wn + 16 * j + l16) * kGPitch + 16 * lg]);
#pragma unroll
    for (int i = 0; i < kTT; ++i) {
      const v4i b = *reinterpret_cast<const v4i*>(
          &Xs[p][((BT / 2) * wt + 16 * i + l16) * kGPitch + 16 * lg]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b, c[i][j], 0, 0, 0);
    }
    if (ks + 1 < nks) {
      // step ks+1 = half (PH+1)%2 of k block (ks+1)/2, held in w[((PH+1)/2)%2]
      decode(std::integral_constant<int, (PH + 1) & 1>{}, w[((PH + 1) >> 1) & 1], p ^ 1);
      store_x(p ^ 1, xv[(PH + 1) & 1]);
      load_x(ks + 3, xv[(PH + 1) & 1]);
      // k block (ks+1)/2 + 1 goes into the chunk slot freed by block (ks+1)/2 - 1
      if constexpr ((PH & 1) == 0) load_chunk((ks + 1) / 2 + 1, w[(((PH + 1) >> 1) + 1) & 1]);
    }
    __syncthreads();
  };
  for (int ks = 0; ks < nks; ks += 4) {
    step(std::integral_constant<int, 0>{}, ks);
    if (ks + 1 < nks) step(std::integral_constant<int, 1>{}, ks + 1);
    if (ks + 2 < nks) step(std::integral_constant<int, 2>{}, ks + 2);
    if (ks + 3 < nks) step(std::integral_constant<int, 3>{}, ks + 3);
  }

  // epilogue: lane holds rows n0 + 64*wn + 16*j + 4*lg + q of token
  // t0 + (BT/2)*wt + 16*i + l16
  const double g = *gamma;
#pragma unroll
  for (int i = 0; i < kTT; ++i) {
    const int64_t t = t0 + (BT / 2) * wt + 16 * i + l16;
    if (t >= tokens) continue;
    const float gs = out_scale(g, scale[t]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t r = n0 + 64 * wn + 16 * j + 4 * lg;
      float* y = Y + t * n_out + r;
      if (r + 4 <= n_out && (n_out & 3) == 0) {
        st_global(reinterpret_cast<v4f*>(y),
                  v4f{out_value(c[i][j][0], gs), out_value(c[i][j][1], gs),
                      out_value(c[i][j][2], gs), out_value(c[i][j][3], gs)});
        if (acc_out) st_global(reinterpret_cast<v4i*>(acc_out + t * n_out + r), c[i][j]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (r + q < n_out) {
            st_global(y + q, out_value(c[i][j][q], gs));
            if (acc_out) st_global(acc_out + t * n_out + r + q, (int32_t)c[i][j][q]);
          }
      }
    }
  }
}

template <int S>
static hipError_t launch_gemm_s(const void* packed, const int8_t* xq, const float* scale,
                                const double* gamma, float* Y, int32_t* acc, int64_t tokens,
                                int64_t k, int64_t n_out, hipStream_t s) {
  // 128-token tiles: two workgroups per CU (the 256-token tile needs more
  // registers than fit twice) hide each other's load and barrier latency
  const int64_t nb = (n_out + kGBN - 1) / kGBN;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  dim3 grid((unsigned)nb, (unsigned)((tokens + 127) / 128));
  gemm_kernel<S, 128><<<grid, 256, 0, s>>>(p, xq, scale, gamma, Y, acc, tokens, k, n_out);
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

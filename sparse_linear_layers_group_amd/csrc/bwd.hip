// bwd.hip -- dual straight-through backward of BitLinear on gfx950.
//
// Sparse-BitNet article §三 and §六: the gradient passes straight through
// the ternary rounding and the N:M sparsification, and a masked weight
// still receives its gradient.
//   dX[t, c] = gamma * sum_r dY[t, r] * code[r, c]     (through the masked
//              ternary weights the forward used)
//   dW[r, c] = sum_t dY[t, r] * s_t * x_q[t, c]        (dense)
// Both are one bf16 "NT" product C[m, n] = alpha * sum_k A[m, k] B[n, k]
// on v_mfma_f32_16x16x32_bf16 with binary32 accumulation, whose operands
// both run along the contraction index in memory:
//   dX: A = dY [tokens x n_out] as given, B = codes^T [k x n_out];
//   dW: A = (dY * s)^T [n_out x tokens], B = x_q^T [k x tokens].
// Prep kernels write the operands that are not in that form into the
// workspace: the codes decoded from the packed layout and transposed
// (exact in bf16), bf16(dY * s_t) transposed (rounded once), and x_q
// transposed (exact).  Every conversion happens once per element, so the
// product kernel is a plain copy-to-LDS and MFMA loop.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace bl {

__device__ __forceinline__ uint16_t code_bf16(uint32_t byte) {
  // 0x01 -> +1.0, 0xff -> -1.0, 0 -> 0
  return byte == 0u ? (uint16_t)0 : (byte == 1u ? (uint16_t)0x3f80 : (uint16_t)0xbf80);
}

// ------------------------------------------------------------- prep
// 64 x 64 transposes through LDS.  Source rows are the contraction index
// of the product (tokens); each thread loads 16 bytes of a source row and
// writes 16 bytes (8 consecutive source rows) of a destination row.
constexpr int kTP = 66;  // LDS pitch (bf16) of the 64 x 64 transpose tile

// dYsT[r][t] = bf16(dY[t][r] * s_t) for t < tokens, 0 for tokens <= t < tp
__global__ __launch_bounds__(256) void prep_dys_t_kernel(const uint16_t* __restrict__ dY,
                                                        const float* __restrict__ scale,
                                                        int64_t tokens, int64_t n_out, int64_t tp,
                                                        uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[64 * kTP];  // [t][r]
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 64, r0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p, t = q >> 3, r8 = 8 * (q & 7);
    const int64_t tt = t0 + t;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    float s = 0.f;
    if (tt < tokens && r0 + r8 < n_out) {  // n_out % 8 == 0: a run is all in or all out
      v = ld_global(reinterpret_cast<const u32x4*>(dY + tt * n_out + r0 + r8));
      s = scale[tt];
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
      tile[t * kTP + r8 + e] = f32_to_bf16_rne(x * s);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p, r = q >> 3, t8 = 8 * (q & 7);
    if (r0 + r >= n_out) continue;
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)tile[(t8 + 2 * e) * kTP + r] | ((uint32_t)tile[(t8 + 2 * e + 1) * kTP + r] << 16);
    st_global(reinterpret_cast<u32x4*>(out + (r0 + r) * tp + t0 + t8), u32x4{o[0], o[1], o[2], o[3]});
  }
}

// xbT[c][t] = bf16(x_q[t][c]) (exact) for t < tokens, 0 up to tp
__global__ __launch_bounds__(256) void prep_xq_t_kernel(const int8_t* __restrict__ xq,
                                                       int64_t tokens, int64_t k, int64_t tp,
                                                       uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[64 * kTP];  // [t][c]
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
  {
    const int t = tid >> 2, c16 = 16 * (tid & 3);
    const int64_t tt = t0 + t;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (tt < tokens) v = ld_global(reinterpret_cast<const u32x4*>(xq + tt * k + c0 + c16));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int8_t b = (int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xffu);
      tile[t * kTP + c16 + e] = f32_to_bf16_rne((float)b);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = tid + 256 * p, c = q >> 3, t8 = 8 * (q & 7);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)tile[(t8 + 2 * e) * kTP + c] | ((uint32_t)tile[(t8 + 2 * e + 1) * kTP + c] << 16);
    st_global(reinterpret_cast<u32x4*>(out + (c0 + c) * tp + t0 + t8), u32x4{o[0], o[1], o[2], o[3]});
  }
}

// codesT[c][r] = bf16(code[r][c]) for the rows of one packed superblock
// (64 rows x 128 columns) per workgroup of 64 threads; padding rows of
// the last strip are zero fields, so rows up to the strip end are written
// (the row pitch np = 64 * strips)
template <int S>
__global__ __launch_bounds__(64) void prep_codes_t_kernel(const uint32_t* __restrict__ packed,
                                                         int64_t nkb, int64_t np,
                                                         uint16_t* __restrict__ out) {
  constexpr int kW = block_bytes(S) / 4;
  __shared__ uint16_t tile[kBlockK * kTP];  // [c][r]
  __shared__ uint32_t lut[512];
  const int lane = threadIdx.x;
  for (int idx = lane; idx < 512; idx += 64)  // lut[half * 256 + key]
    lut[idx] = ld_global(&kHalfCodeTable.v[(idx & 255) * 2 + (idx >> 8)]);
  const int64_t sb = blockIdx.x;  // superblock = strip * nkb + kb
  const int64_t strip = sb / nkb, kb = sb - strip * nkb;
  uint32_t w[kW + 1];
  const uint32_t* src = packed + (sb * kStripRows + lane) * kW;
#pragma unroll
  for (int i = 0; i < kW; ++i) w[i] = ld_global(src + i);
  w[kW] = 0;
  __syncthreads();
  auto lk = [&](uint32_t key, int half) { return lut[half * 256 + key]; };
  auto emit = [&](int f, uint32_t lo, uint32_t hi) {
    const int rr = field_row(lane, f), gi = field_group(lane, f);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      tile[(gi * 8 + p) * kTP + rr] = code_bf16((lo >> (8 * p)) & 0xffu);
      tile[(gi * 8 + 4 + p) * kTP + rr] = code_bf16((hi >> (8 * p)) & 0xffu);
    }
  };
  decode_groups<S, 0, 16>(w, lk, emit);
  __syncthreads();
  // 128 columns x 64 rows: each thread writes 8 rows of 8 bf16 runs
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int q = lane + 64 * p, c = q >> 3, r8 = 8 * (q & 7);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = (uint32_t)tile[c * kTP + r8 + 2 * e] | ((uint32_t)tile[c * kTP + r8 + 2 * e + 1] << 16);
    st_global(reinterpret_cast<u32x4*>(out + (kb * kBlockK + c) * np + strip * kStripRows + r8),
              u32x4{o[0], o[1], o[2], o[3]});
  }
}

// ------------------------------------------------------------- product
// C[m][n] = alpha * sum_k A[m][k] * B[n][k], A/B bf16 row-major with row
// pitches lda/ldb (elements, multiples of 8), C binary32 [M][ldc].
// Workgroup tile 128 x 128, four wavefronts of 64 x 64 (4 x 4 MFMA
// tiles); k advances 64 at a time through double-buffered LDS tiles
// (rows padded to 80 bf16; of the pitches 64, 68, 72 and 80 this one
// measured fastest on MI355X, 64 slowest).  Global loads run two steps
// ahead in a register ring; one barrier per step.  k positions at or past
// K read as zero.  The output goes out with streaming stores.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, each with its
// own L2.  Workgroup b is mapped to the (b % 8)-th contiguous eighth of a
// grouped tile order (groups of kGroupM row tiles, column tiles within a
// group, row tiles fastest), so the workgroups an XCD runs at once cover a
// compact block of rows and columns and share their operand rows in that
// L2; with the plain row-major order every XCD read nearly all of both
// operands.
constexpr int kBP = 80;
constexpr int kGroupM = 8;

__global__ __launch_bounds__(256, 2) void gemm_nt_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    float* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K,
    const double* __restrict__ alpha, int64_t klen) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * kBP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * kBP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;
  const int64_t tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
  int64_t m0, n0;
  {
    const int64_t T = tiles_m * tiles_n, per = (T + 7) / 8;
    const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int64_t full = T - (per - 1) * 8;  // XCDs that get `per` tiles
    if (slot >= (xcd < full ? per : per - 1)) return;
    const int64_t t = xcd < full ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
    const int64_t g = t / (kGroupM * tiles_n), r = t - g * kGroupM * tiles_n;
    const int64_t gm = tiles_m - g * kGroupM < kGroupM ? tiles_m - g * kGroupM : kGroupM;
    m0 = (g * kGroupM + r % gm) * 128;
    n0 = (r / gm) * 128;
  }
  // k range of this workgroup's split (blockIdx.y): [k0, k0 + klen) of K;
  // a split writes its partial tile to plane blockIdx.y of C
  const int64_t k0 = (int64_t)blockIdx.y * klen;
  K = K - k0 < klen ? K - k0 : klen;
  C += (int64_t)blockIdx.y * M * ldc;
  const int64_t nks = (K + 63) / 64;

  // loads: piece q = tid + 256 p (p < 4) of each tile is row q/8, k
  // columns 8*(q%8) .. +8 of the step.  A register ring holds two steps in
  // flight, so a step's global loads have two steps of MFMAs to land.
  u32x4 ra[2][4], rb[2][4];
  // buffer loads: an offset past the range (kOOB) reads zeros, so rows
  // past M/N and k past K need no branches (operands stay below 2 GiB)
  const __amdgpu_buffer_rsrc_t ar =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(A), (short)0, (int)(M * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t br =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(B), (short)0, (int)(N * ldb * 2), 0x00020000);
  constexpr uint32_t kOOB = 0x80000000u;
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int q = tid + 256 * p, row = q >> 3, kc = 8 * (q & 7);
    a_off[p] = m0 + row < M ? (uint32_t)(((m0 + row) * lda + k0 + kc) * 2) : kOOB;
    b_off[p] = n0 + row < N ? (uint32_t)(((n0 + row) * ldb + k0 + kc) * 2) : kOOB;
  }
  auto load = [&](int64_t ks, u32x4* xa, u32x4* xb) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int kc = 8 * ((tid + 256 * p) & 7);
      const bool ka = ks * 64 + kc < K;
      const uint32_t ko = (uint32_t)(ks * 128);
      xa[p] = __builtin_amdgcn_raw_buffer_load_b128(ar, ka ? a_off[p] + ko : kOOB, 0, 0);
      xb[p] = __builtin_amdgcn_raw_buffer_load_b128(br, ka ? b_off[p] + ko : kOOB, 0, 0);
    }
  };
  auto store = [&](int st, const u32x4* xa, const u32x4* xb) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int q = tid + 256 * p, row = q >> 3, kc = 8 * (q & 7);
      *reinterpret_cast<u32x4*>(&As[st][row * kBP + kc]) = xa[p];
      *reinterpret_cast<u32x4*>(&Bs[st][row * kBP + kc]) = xb[p];
    }
  };

  v4f c[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // step ks (parity P): MFMAs from LDS stage P; in between, step ks+1
  // (registers ra/rb[P^1], loaded two steps ago) goes to stage P^1 and
  // those registers take the loads of step ks+3.  Loads past the last step
  // read zeros (k >= K) and their stores are never read.
  auto step = [&](auto parity, int64_t ks) {
    constexpr int P = decltype(parity)::value;
    // fragments of both k halves are read up front, so the second half's
    // LDS latency hides behind the first half's MFMAs
    v8bf a[2][4], b[2][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[kk][i] = *reinterpret_cast<const v8bf*>(&As[P][(wm * 64 + i * 16 + l16) * kBP + kk * 32 + lg * 8]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[kk][j] = *reinterpret_cast<const v8bf*>(&Bs[P][(wn * 64 + j * 16 + l16) * kBP + kk * 32 + lg * 8]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          c[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk][i], b[kk][j], c[i][j], 0, 0, 0);
      if (kk == 0) {
        store(P ^ 1, ra[P ^ 1], rb[P ^ 1]);
        load(ks + 3, ra[P ^ 1], rb[P ^ 1]);
      }
    }
    __syncthreads();
  };

  load(0, ra[0], rb[0]);
  load(1, ra[1], rb[1]);
  store(0, ra[0], rb[0]);
  load(2, ra[0], rb[0]);
  __syncthreads();
  int64_t ks = 0;
  for (; ks + 1 < nks; ks += 2) {
    step(std::integral_constant<int, 0>{}, ks);
    step(std::integral_constant<int, 1>{}, ks + 1);
  }
  if (ks < nks) step(std::integral_constant<int, 0>{}, ks);

  // lane holds C[m0 + 64wm + 16i + 4lg + q][n0 + 64wn + 16j + l16]
  const double g = alpha ? *alpha : 1.0;
  if (m0 + 128 <= M && n0 + 128 <= N) {  // whole tile in range: no checks
    float* cb = C + (m0 + wm * 64 + 4 * lg) * ldc + n0 + wn * 64 + l16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float* cr = cb + (int64_t)(i * 16 + q) * ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st_stream(cr + j * 16, alpha ? (float)((double)c[i][j][q] * g) : c[i][j][q]);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + wm * 64 + i * 16 + 4 * lg + q;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + l16;
        if (n < N) C[m * ldc + n] = alpha ? (float)((double)c[i][j][q] * g) : c[i][j][q];
      }
    }
}

// C = alpha * (sum of the split planes, in order), binary32 sums
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ P, int splits,
                                                       int64_t n4, const double* __restrict__ alpha,
                                                       float* __restrict__ C) {
  const double g = alpha ? *alpha : 1.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    v4f acc = ld_global(reinterpret_cast<const v4f*>(P) + i);
    for (int s = 1; s < splits; ++s) {
      const v4f v = ld_global(reinterpret_cast<const v4f*>(P) + (int64_t)s * n4 + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    if (alpha) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = (float)((double)acc[e] * g);
    }
    st_global(reinterpret_cast<v4f*>(C) + i, acc);
  }
}

// zero fill (dW when there are no tokens)
__global__ void zero_f32_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// ------------------------------------------------------------- launchers
// C has row pitch ldc = N when the product is split (the partial planes in
// `partials`, M * N floats each)
static hipError_t gemm_nt(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                          int64_t ldc, int64_t M, int64_t N, int64_t K, const double* alpha,
                          float* partials, hipStream_t s) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  const unsigned gx = (unsigned)((tiles + 7) / 8 * 8);
  const int splits = bwd_splits(M, N, K);
  if (splits == 1) {
    gemm_nt_bf16_kernel<<<gx, 256, 0, s>>>(A, lda, B, ldb, C, ldc, M, N, K, alpha, K);
    return hipGetLastError();
  }
  const int64_t klen = bwd_split_len(K, splits);
  const int used = (int)((K + klen - 1) / klen);
  gemm_nt_bf16_kernel<<<dim3(gx, (unsigned)used), 256, 0, s>>>(A, lda, B, ldb, partials, N, M, N, K,
                                                               nullptr, klen);
  const int64_t n4 = M * N / 4;
  const int64_t blocks = (n4 + 255) / 256;
  split_sum_kernel<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(partials, used, n4, alpha, C);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dY, const void* packed, const double* gamma, float* dX,
                         void* ws, int64_t tokens, int64_t k, int64_t n_out, int S, hipStream_t s) {
  const int64_t nkb = k / kBlockK, strips = (n_out + kStripRows - 1) / kStripRows;
  const int64_t np = strips * kStripRows;
  uint16_t* codes_t = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + bwd_codes_offset(tokens, k, n_out));
  const uint32_t* p = reinterpret_cast<const uint32_t*>(packed);
  const unsigned sbs = (unsigned)(strips * nkb);
  if (S == 8) prep_codes_t_kernel<8><<<sbs, 64, 0, s>>>(p, nkb, np, codes_t);
  else if (S == 6) prep_codes_t_kernel<6><<<sbs, 64, 0, s>>>(p, nkb, np, codes_t);
  else if (S == 2) prep_codes_t_kernel<2><<<sbs, 64, 0, s>>>(p, nkb, np, codes_t);
  else prep_codes_t_kernel<4><<<sbs, 64, 0, s>>>(p, nkb, np, codes_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dX [tokens x k] = gamma * dY [tokens x n_out] . codes^T [k x n_out]^T
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + bwd_partial_offset(tokens, k, n_out));
  return gemm_nt(dY, n_out, codes_t, np, dX, k, tokens, k, n_out, gamma, partials, s);
}

hipError_t launch_bwd_dw(const uint16_t* dY, const int8_t* xq, const float* scale, float* dW,
                         void* ws, int64_t tokens, int64_t k, int64_t n_out, hipStream_t s) {
  if (tokens == 0) {
    zero_f32_kernel<<<1024, 256, 0, s>>>(dW, n_out * k);
    return hipGetLastError();
  }
  const int64_t tp = bwd_tokens_padded(tokens);
  char* w = reinterpret_cast<char*>(ws);
  uint16_t* dys_t = reinterpret_cast<uint16_t*>(w + bwd_dys_offset(tokens, k, n_out));
  uint16_t* xq_t = reinterpret_cast<uint16_t*>(w + bwd_xq_offset(tokens, k, n_out));
  prep_dys_t_kernel<<<dim3((unsigned)(tp / 64), (unsigned)((n_out + 63) / 64)), 256, 0, s>>>(
      dY, scale, tokens, n_out, tp, dys_t);
  prep_xq_t_kernel<<<dim3((unsigned)(tp / 64), (unsigned)(k / 64)), 256, 0, s>>>(xq, tokens, k, tp,
                                                                              xq_t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dW [n_out x k] = (dY s)^T [n_out x tp] . x_q^T [k x tp]^T
  float* partials = reinterpret_cast<float*>(w + bwd_partial_offset(tokens, k, n_out));
  return gemm_nt(dys_t, tp, xq_t, tp, dW, k, n_out, k, tp, nullptr, partials, s);
}

}  // namespace bl

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
#include "bwd_group.h"
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <atomic>
#include <utility>
#include <vector>

#include <type_traits>

namespace bl {

// ------------------------------------------------------------- prep
// All operand conversions of one backward call run in one launch: a list
// of tasks (one matrix each), every workgroup of 256 threads takes one job
// of one task.  Jobs of a dY or x_q task are 64 x 64 transposes through
// LDS; jobs of a codes task are four packed superblocks, one per
// wavefront, transposed in registers.

// bf16 codes of one half-group from its 8-bit key: entry key * 2 + half
// holds positions 0..3 as two bf16 pairs (the int8 codes of half_codes
// with 0x01 -> +1.0 and 0xff -> -1.0, both exact)
struct HalfBf16Table {
  uint32_t v[1024];
};
constexpr uint32_t code_to_bf16(uint32_t byte) {
  return byte == 0u ? 0u : (byte == 1u ? 0x3f80u : 0xbf80u);
}
constexpr HalfBf16Table make_half_bf16_table() {
  HalfBf16Table t{};
  for (uint32_t e = 0; e < 512; ++e) {
    const uint32_t c = half_codes(e >> 1, e & 1u);
    t.v[2 * e] = code_to_bf16(c & 0xffu) | (code_to_bf16((c >> 8) & 0xffu) << 16);
    t.v[2 * e + 1] = code_to_bf16((c >> 16) & 0xffu) | (code_to_bf16(c >> 24) << 16);
  }
  return t;
}
__device__ constexpr HalfBf16Table kHalfBf16Table = make_half_bf16_table();
static_assert(make_half_bf16_table().v[2 * (2 * 0x1f + 0)] == 0x3f80bf80u,
              "low half, bitmap 1111, sign of nonzero 0: -1.0 then +1.0");

enum PrepKind : int32_t { kPrepCodes = 0, kPrepDys = 1, kPrepXq = 2 };

// One matrix of a prep launch.
//   codes: src = packed codes, rows = k blocks per strip, cols = strips,
//          pitch = np (rows of codes^T); jobs = ceil(superblocks / 4)
//   dys:   src = dY, scale = s_t, rows = tokens, cols = n_out, pitch = tp
//   xq:    src = x_q, rows = tokens, cols = k, pitch = tp
// dY and x_q jobs are (64-token block fastest, 64-column block) tiles.
struct PrepTask {
  const void* src;
  const float* scale;
  uint16_t* out;
  int64_t rows, cols, pitch;
  int32_t kind, jobs;
};
constexpr int kMaxPrep = 16;
struct PrepSet {
  PrepTask t[kMaxPrep];
  int32_t n;
};

// 64 x 64 transposes through LDS.  Source rows are the contraction index
// of the product (tokens); each thread loads 16 bytes of a source row and
// writes 16 bytes (8 consecutive source rows) of a destination row.
constexpr int kTP = 66;  // LDS pitch (bf16) of the 64 x 64 transpose tile

// dYsT[r][t] = bf16(dY[t][r] * s_t) for t < tokens, 0 for tokens <= t < tp
__device__ __forceinline__ void prep_dys_tile(const uint16_t* __restrict__ dY,
                                              const float* __restrict__ scale, int64_t tokens,
                                              int64_t n_out, int64_t tp, uint16_t* __restrict__ out,
                                              int64_t t0, int64_t r0, uint16_t* tile, int tid) {
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
__device__ __forceinline__ void prep_xq_tile(const int8_t* __restrict__ xq, int64_t tokens, int64_t k,
                                             int64_t tp, uint16_t* __restrict__ out, int64_t t0,
                                             int64_t c0, uint16_t* tile, int tid) {
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

// Lane exchanges inside groups of 8 lanes (data-parallel primitives: the
// partner's register value, lane j reading lane j ^ 1, j ^ 2 or j ^ 4)
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t lane_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ uint32_t lane_xor4(uint32_t v) {
  // lanes 0-3 and 8-11 of each row of 16 read lane + 4 (row_shl:4), lanes
  // 4-7 and 12-15 read lane - 4 (row_shr:4)
  const int a = __builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xf, 0x5, false);
  return (uint32_t)__builtin_amdgcn_update_dpp(a, (int)v, 0x114, 0xf, 0xa, false);
}
__device__ __forceinline__ uint32_t byte_perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 8 x 8 transpose of bf16 values across the 8 lanes j = lane & 7 of a
// group: in d[m], lane j holds elements 2m, 2m+1 of row j; out o[m], lane
// j holds element j of rows 2m, 2m+1.  Three exchange stages, each with
// the partner at lane distance 1, 2, 4.
__device__ __forceinline__ void transpose8_bf16(const uint32_t (&d)[4], uint32_t (&o)[4], int lane) {
  const int j = lane & 7;
  // stage 1: lane j holds rows (j & ~1, +1) of elements 2m + (j & 1)
  const uint32_t sel = (j & 1) ? 0x03020706u : 0x05040100u;
  uint32_t x[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) x[m] = byte_perm(lane_xor1(d[m]), d[m], sel);
  // stage 2: lane j holds rows (j & ~3) .. +3 of elements 2m + (j & 1),
  // m = b and b + 2 with b = bit 1 of j
  const bool b = (j >> 1) & 1;
  const uint32_t r0 = lane_xor2(b ? x[0] : x[1]), r1 = lane_xor2(b ? x[2] : x[3]);
  const uint32_t k0 = b ? x[1] : x[0], k1 = b ? x[3] : x[2];
  const uint32_t y[4] = {b ? r0 : k0, b ? k0 : r0, b ? r1 : k1, b ? k1 : r1};
  // stage 3: lane j holds rows 0..7 of element 2(2t + b) + (j & 1) = j,
  // t = bit 2 of j
  const bool t = (j >> 2) & 1;
  const uint32_t q0 = lane_xor4(t ? y[0] : y[2]), q1 = lane_xor4(t ? y[1] : y[3]);
  const uint32_t h0 = t ? y[2] : y[0], h1 = t ? y[3] : y[1];
  o[0] = t ? q0 : h0;
  o[1] = t ? q1 : h1;
  o[2] = t ? h0 : q0;
  o[3] = t ? h1 : q1;
}

// codesT[c][r] = bf16(code[r][c]) for one packed superblock (64 rows x 128
// columns) per wavefront.  Lane c decodes chunk c: field f holds 8-group g
// = field_group(c, f) of row field_row(c, f), so the 8 lanes of a group
// hold 8 consecutive rows of one 8-group; after the transpose lane j holds
// column 8g + j of those rows, one 16-byte store.  Padding rows of the last
// strip are zero fields, so rows up to the strip end are written (the row
// pitch np = 64 * strips).
template <int S>
__device__ __forceinline__ void prep_codes_sb(const uint32_t* __restrict__ packed, int64_t sb,
                                              int64_t nkb, int64_t np, uint16_t* __restrict__ out,
                                              const u32x2* lut, int lane) {
  constexpr int kW = block_bytes(S) / 4;
  const int64_t strip = sb / nkb, kb = sb - strip * nkb;
  uint32_t w[kW + 1];
  const uint32_t* src = packed + (sb * kStripRows + lane) * kW;
#pragma unroll
  for (int i = 0; i < kW; ++i) w[i] = ld_global(src + i);
  w[kW] = 0;
  uint16_t* dst = out + (kb * kBlockK + (lane & 7)) * np + strip * kStripRows + (lane & 8);
  auto lk = [&](uint32_t key, int half) { return lut[key * 2 + half]; };
  auto emit = [&](int f, u32x2 lo, u32x2 hi) {
    const uint32_t d[4] = {lo.x, lo.y, hi.x, hi.y};
    uint32_t o[4];
    transpose8_bf16(d, o, lane);
    st_global(reinterpret_cast<u32x4*>(dst + (int64_t)(8 * field_group(lane, f)) * np + 16 * (f >> 2)),
              u32x4{o[0], o[1], o[2], o[3]});
  };
  decode_groups<S, 0, 16>(w, lk, emit);
}

template <int S>
__global__ __launch_bounds__(256) void prep_group_kernel(PrepSet set) {
  __shared__ uint16_t tile[64 * kTP];
  __shared__ u32x2 lut[512];
  const int tid = threadIdx.x;
  int job = (int)blockIdx.x, ti = 0;
  while (ti + 1 < set.n && job >= set.t[ti].jobs) job -= set.t[ti].jobs, ++ti;
  const PrepTask& tk = set.t[ti];
  if (tk.kind == kPrepCodes) {
    reinterpret_cast<u32x4*>(lut)[tid] = ld_global(reinterpret_cast<const u32x4*>(kHalfBf16Table.v) + tid);
    __syncthreads();
    const int64_t sb = 4 * (int64_t)job + (tid >> 6);
    if (sb < tk.rows * tk.cols)
      prep_codes_sb<S>(reinterpret_cast<const uint32_t*>(tk.src), sb, tk.rows, tk.pitch, tk.out, lut,
                       tid & 63);
    return;
  }
  const int64_t bx = tk.pitch / 64, t0 = 64 * (job % bx), c0 = 64 * (job / bx);
  if (tk.kind == kPrepDys)
    prep_dys_tile(reinterpret_cast<const uint16_t*>(tk.src), tk.scale, tk.rows, tk.cols, tk.pitch, tk.out,
                  t0, c0, tile, tid);
  else
    prep_xq_tile(reinterpret_cast<const int8_t*>(tk.src), tk.rows, tk.cols, tk.pitch, tk.out, t0, c0,
                 tile, tid);
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

// One product of a launch: C[M][N] (row pitch ldc) = alpha * A B^T over a
// k range of klen (split launches: plane blockIdx.y of C).
struct NtProblem {
  const uint16_t* A;
  const uint16_t* B;
  float* C;
  const double* alpha;
  int64_t lda, ldb, ldc, M, N, K, klen;
  // gated epilogue (256-row kernel only): with G set, C is not written;
  // the squared-ReLU gating backward of C (as relu2_gate_bwd_kernel
  // computes it from a stored C) goes to dG and dU instead, G, U, dG, dU
  // laid out like C
  const float* G = nullptr;
  const float* U = nullptr;
  uint16_t* dG = nullptr;
  uint16_t* dU = nullptr;
};

// the products of one launch of the 256-row kernel (its tiles dealt over
// the XCDs problem by problem, in this order)
constexpr int kMaxNt = 16;
struct NtSet {
  NtProblem p[kMaxNt];
  int32_t n;
};

__host__ __device__ inline int64_t nt_tiles(const NtProblem& p) {
  return ((p.M + 127) / 128) * ((p.N + 127) / 128);
}

// XCD share of a problem's tiles: XCD x runs tiles [start, start + cnt)
__device__ __forceinline__ void xcd_share(int64_t T, int64_t x, int64_t& start, int64_t& cnt) {
  const int64_t per = (T + 7) / 8, full = T - (per - 1) * 8;  // XCDs that get `per` tiles
  cnt = T == 0 ? 0 : (x < full ? per : per - 1);
  start = T == 0 ? 0 : (x < full ? x * per : full * per + (x - full) * (per - 1));
}

// A launch runs one or two independent products (the dX and dW of a
// layer): the tiles of each are shared out over the 8 XCDs separately, so
// every XCD runs the same mix of the two (tiles of different k depth cost
// different times), the first problem's first within an XCD.  Two
// products in one launch fill the partly used last round of each with
// tiles of the other.
__global__ __launch_bounds__(256, 2) void gemm_nt_bf16_kernel(NtProblem p0, NtProblem p1) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * kBP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * kBP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;
  int64_t m0, n0, t;
  bool second;
  {
    const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    int64_t s0, c0, s1, c1;
    xcd_share(nt_tiles(p0), xcd, s0, c0);
    xcd_share(nt_tiles(p1), xcd, s1, c1);
    if (slot >= c0 + c1) return;
    second = slot >= c0;
    t = second ? s1 + slot - c0 : s0 + slot;
  }
  const NtProblem& pr = second ? p1 : p0;
  const uint16_t* __restrict__ A = pr.A;
  const uint16_t* __restrict__ B = pr.B;
  float* __restrict__ C = pr.C;
  const double* __restrict__ alpha = pr.alpha;
  const int64_t lda = pr.lda, ldb = pr.ldb, ldc = pr.ldc, M = pr.M, N = pr.N, klen = pr.klen;
  int64_t K = pr.K;
  {
    const int64_t tiles_m = (M + 127) / 128, tiles_n = (N + 127) / 128;
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

// ------------------------------------------- 256 x 128 and 256 x 256 tiles
// Large products run on 256-row tiles of wavefronts of 128 x 64 (8 x 4
// MFMA tiles each): 256 x 128 (four wavefronts, two workgroups per CU) or
// 256 x 256 (eight wavefronts, one per CU).  Each byte of an operand
// fragment read from LDS feeds 1.33 times the MFMA work of the 64 x 64
// wavefront tiles above, and each byte written into LDS 1.33 (256 x 128) or
// 2 (256 x 256) times: those tiles' fragment reads and tile writes need
// more LDS bandwidth than a CU has at the full MFMA rate.  (128 x 128
// wavefront tiles would read less still, but 256 accumulators per lane made
// the register allocator shuttle them between register files around every
// MFMA.)  The tiles stream through three LDS stages of 32 k filled by LDS
// DMA (buffer loads that write LDS directly, 16 bytes per lane, 1 KiB per
// wavefront instruction), issued two stages ahead.  In a stage each
// operand row's 64 bytes hold four 16-byte pieces, piece c of row r at
// position c ^ ((r >> 1) & 3): the eight lanes that read one 128-byte bank
// line at a time (rows r..r+7 of one k piece) then hit distinct banks, and
// a DMA instruction's 64 lanes still write 1 KiB in order (lane l writes
// row l / 4, position l % 4, and loads the piece that belongs there).
constexpr int kBigM = 256;
constexpr int kBigK = 32;                        // k per stage
constexpr int kBigABytes = kBigM * kBigK * 2;    // 16 KiB
template <int kWN>  // column wavefronts: tile N = 64 kWN, 2 kWN wavefronts
struct BigTile {
  static constexpr int N = 64 * kWN;
  static constexpr int kWaves = 2 * kWN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kStageBytes = kBigABytes + N * kBigK * 2;
  static constexpr int kAInstr = 16 / kWaves;    // A DMA instructions per wavefront and step
  static constexpr int kPerStep = kAInstr + 2;   // + two of B
};

template <int kWN>
__host__ __device__ inline int64_t nt_tiles_big(const NtProblem& p) {
  return ((p.M + kBigM - 1) / kBigM) * ((p.N + BigTile<kWN>::N - 1) / BigTile<kWN>::N);
}

// gfx950-only builtins sit in plain (non-template) functions: used directly
// in the kernel template, the host pass (which checks template bodies
// against its own target) dropped the kernel's launch stub
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, __attribute__((address_space(3))) void* dst,
                                          uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// wait until at most N vector memory operations of this wavefront are in
// flight (the waits below count LDS DMA themselves) and, with kLds, until
// its LDS reads have returned
template <int N, bool kLds = false>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((kLds ? 0 : 15) << 8));
}

// the three stages are separate arrays, each step's stage a compile-time
// choice: the compiler then sees that a step's fragment reads and the DMA
// in flight into the other stages touch different objects, and waits only
// for the DMA of the stage being read (with one array it waited for every
// DMA in flight before each read)
// (namespace-scope arrays: a function-local __shared__ array in a template
// made the host pass drop the kernel's launch stub)
__shared__ __attribute__((aligned(1024))) char g_big2_st0[BigTile<2>::kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_big2_st1[BigTile<2>::kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_big2_st2[BigTile<2>::kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_big4_st0[BigTile<4>::kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_big4_st1[BigTile<4>::kStageBytes];
__shared__ __attribute__((aligned(1024))) char g_big4_st2[BigTile<4>::kStageBytes];
template <int kWN, int P>
__device__ __forceinline__ char* big_stage() {
  static_assert(kWN == 2 || kWN == 4, "tile widths");
  if constexpr (kWN == 2) return P == 0 ? g_big2_st0 : P == 1 ? g_big2_st1 : g_big2_st2;
  else return P == 0 ? g_big4_st0 : P == 1 ? g_big4_st1 : g_big4_st2;
}

// (512 threads at most: two wavefronts per SIMD either way, so the
// register budget is the same; bounds that depend on kWN broke the host
// side's template deduction)
template <int kWN>
__global__ __launch_bounds__(512) void gemm_nt_bf16_big_kernel(NtSet set) {
  typedef BigTile<kWN> T;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef __attribute__((address_space(3))) void lds_void;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int l16 = lane & 15, lg = lane >> 4;
  int64_t m0, n0, t = 0;
  int which = -1;
  {
    // workgroup (XCD x, slot) takes the slot-th tile of XCD x's run: the XCD
    // shares of the problems one after the other
    const int64_t xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    int64_t before = 0;
    for (int i = 0; i < set.n; ++i) {
      int64_t s0, c0;
      xcd_share(nt_tiles_big<kWN>(set.p[i]), xcd, s0, c0);
      if (which < 0 && slot < before + c0) {
        which = i;
        t = s0 + slot - before;
      }
      before += c0;
    }
    if (which < 0) return;
  }
  const NtProblem& pr = set.p[which];
  const uint16_t* __restrict__ A = pr.A;
  const uint16_t* __restrict__ B = pr.B;
  float* __restrict__ C = pr.C;
  const double* __restrict__ alpha = pr.alpha;
  const int64_t lda = pr.lda, ldb = pr.ldb, ldc = pr.ldc, M = pr.M, N = pr.N, klen = pr.klen;
  int64_t K = pr.K;
  {
    const int64_t tiles_m = (M + kBigM - 1) / kBigM, tiles_n = (N + T::N - 1) / T::N;
    constexpr int64_t kG = 4;  // row tiles per group of the tile order
    const int64_t g = t / (kG * tiles_n), r = t - g * kG * tiles_n;
    const int64_t gm = tiles_m - g * kG < kG ? tiles_m - g * kG : kG;
    m0 = (g * kG + r % gm) * kBigM;
    n0 = (r / gm) * T::N;
  }
  const int64_t k0 = (int64_t)blockIdx.y * klen;
  K = K - k0 < klen ? K - k0 : klen;
  C += (int64_t)blockIdx.y * M * ldc;
  const int64_t nks = (K + kBigK - 1) / kBigK;

  const __amdgpu_buffer_rsrc_t ar = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A), (short)0, (int)(M * lda * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B), (short)0, (int)(N * ldb * 2), 0x00020000);
  constexpr uint32_t kOOB = 0x80000000u;
  // DMA: wavefront w fills A rows [16 kAInstr w, +16 kAInstr) and B rows
  // [32w, 32w + 32), 16 rows per instruction; lane l covers row l / 4 of
  // the instruction's 16 at position l % 4, i.e. logical piece kc / 8
  // below (the same for every instruction)
  const int kc = 8 * ((lane & 3) ^ ((lane >> 3) & 3));
  uint32_t a_off[T::kAInstr], b_off[2];
#pragma unroll
  for (int q = 0; q < T::kAInstr; ++q) {
    const int64_t row = 16 * (T::kAInstr * wave + q) + (lane >> 2);
    a_off[q] = m0 + row < M ? (uint32_t)(((m0 + row) * lda + k0 + kc) * 2) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t row = 32 * wave + 16 * q + (lane >> 2);
    b_off[q] = n0 + row < N ? (uint32_t)(((n0 + row) * ldb + k0 + kc) * 2) : kOOB;
  }
  // every step issues the same instructions per wavefront (past the last
  // step they read zeros into a stage nobody reads), so the waits below
  // can count them
  auto dma = [&](auto stage, int64_t ks) {
    constexpr int P = decltype(stage)::value;
    const bool kv = ks * kBigK + kc < K;
    const uint32_t ko = (uint32_t)(ks * kBigK * 2);
    lds_char* st = (lds_char*)big_stage<kWN, P>();
#pragma unroll
    for (int q = 0; q < T::kAInstr; ++q)
      lds_dma16(ar, (lds_void*)(st + 1024 * (T::kAInstr * wave + q)), kv ? a_off[q] + ko : kOOB);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      lds_dma16(br, (lds_void*)(st + kBigABytes + 1024 * (2 * wave + q)), kv ? b_off[q] + ko : kOOB);
  };

  v4f c[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  // fragment of MFMA row tile i / column tile j: row (or column) 16i + l16
  // of the wavefront's range, logical k piece lg
  const uint32_t frag = (uint32_t)(l16 * 64 + 16 * (lg ^ ((l16 >> 1) & 3)));
  const uint32_t a_base = (uint32_t)(wm * 128 * 64) + frag;
  const uint32_t b_base = (uint32_t)kBigABytes + (uint32_t)(wn * 64 * 64) + frag;

  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;
  typedef std::integral_constant<int, 2> S2;
  // step ks reads stage ks % 3 and refills stage (ks + 2) % 3 (last read in
  // step ks - 1) with step ks + 2
  auto step = [&](auto stage, int64_t ks) {
    constexpr int P = decltype(stage)::value;
    // this wavefront's part of step ks has landed and its reads of step
    // ks - 1 have returned, then everyone's has.  A plain barrier with
    // compiler-only fences: __syncthreads()'s workgroup release would wait
    // for every LDS DMA in flight (they write LDS), draining the steps ahead
    wait_vmcnt<T::kPerStep, true>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    dma(std::integral_constant<int, (P + 2) % 3>{}, ks + 2);
    const lds_char* st = (const lds_char*)big_stage<kWN, P>();
    v8bf a[8], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const __attribute__((address_space(3))) v8bf*>(st + b_base + j * 16 * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      a[i] = *reinterpret_cast<const __attribute__((address_space(3))) v8bf*>(st + a_base + i * 16 * 64);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        c[i][j] = mfma_bf16(a[i], b[j], c[i][j]);
  };

  dma(S0{}, 0);
  dma(S1{}, 1);
  int64_t ks = 0;
  for (; ks + 2 < nks; ks += 3) {
    step(S0{}, ks);
    step(S1{}, ks + 1);
    step(S2{}, ks + 2);
  }
  if (ks < nks) step(S0{}, ks);
  if (ks + 1 < nks) step(S1{}, ks + 1);
  wait_vmcnt<0>();  // no LDS DMA outlives the workgroup

  // lane holds C[m0 + 128wm + 16i + 4lg + q][n0 + 64wn + 16j + l16]
  const double g = alpha ? *alpha : 1.0;
  const bool scaled = alpha != nullptr;
  if (pr.G) {
    const float* __restrict__ G = pr.G;
    const float* __restrict__ U = pr.U;
    uint16_t* __restrict__ dG = pr.dG;
    uint16_t* __restrict__ dU = pr.dU;
    // software-pipelined over the MFMA row tiles: row tile i + 1's 32
    // loads issue before row tile i's stores (stores could alias them as
    // far as the compiler knows, so a load written after a store waits)
    float gv[2][4][4], uv[2][4][4];
    auto load = [&](int i, float (&gb)[4][4], float (&ub)[4][4]) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = m0 + wm * 128 + i * 16 + 4 * lg + q;
          const int64_t n = n0 + wn * 64 + j * 16 + l16;
          const bool in = m < M && n < N;
          const int64_t e = in ? m * ldc + n : 0;
          gb[q][j] = in ? ld_global(G + e) : 0.f;
          ub[q][j] = in ? ld_global(U + e) : 0.f;
        }
    };
    load(0, gv[0], uv[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 1 < 8) load(i + 1, gv[(i + 1) & 1], uv[(i + 1) & 1]);
      // lanes l16 and l16 ^ 1 hold neighbouring columns of the same four
      // rows: after one exchange the even lane stores rows 0 and 2 and the
      // odd lane rows 1 and 3, each as a 4-byte pair of columns (k is a
      // multiple of 128, so both columns of a pair are in range together)
      const bool odd = (l16 & 1) != 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t hu[4], hg[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float dh = scaled ? (float)((double)c[i][j][q] * g) : c[i][j][q];
          const float gq = gv[i & 1][q][j];
          const float r = gq > 0.f ? gq : 0.f;
          const float r2 = r * r;
          const float du = dh * uv[i & 1][q][j];
          hu[q] = f32_to_bf16_rne(dh * r2);
          hg[q] = f32_to_bf16_rne(du * (2.f * r));
        }
        const uint32_t pu0 = hu[0] | hu[1] << 16, pu1 = hu[2] | hu[3] << 16;
        const uint32_t pg0 = hg[0] | hg[1] << 16, pg1 = hg[2] | hg[3] << 16;
        const uint32_t xu0 = lane_xor1(pu0), xu1 = lane_xor1(pu1);
        const uint32_t xg0 = lane_xor1(pg0), xg1 = lane_xor1(pg1);
        const int64_t col = n0 + wn * 64 + j * 16 + (l16 & ~1);
        if (col >= N) continue;
        const int64_t ra = m0 + wm * 128 + i * 16 + 4 * lg + (odd ? 1 : 0);
        if (ra < M) {
          const int64_t e = ra * ldc + col;
          st_global(reinterpret_cast<uint32_t*>(dU + e),
                    odd ? (xu0 >> 16) | (pu0 & 0xffff0000u) : (pu0 & 0xffffu) | (xu0 << 16));
          st_global(reinterpret_cast<uint32_t*>(dG + e),
                    odd ? (xg0 >> 16) | (pg0 & 0xffff0000u) : (pg0 & 0xffffu) | (xg0 << 16));
        }
        if (ra + 2 < M) {
          const int64_t e = (ra + 2) * ldc + col;
          st_global(reinterpret_cast<uint32_t*>(dU + e),
                    odd ? (xu1 >> 16) | (pu1 & 0xffff0000u) : (pu1 & 0xffffu) | (xu1 << 16));
          st_global(reinterpret_cast<uint32_t*>(dG + e),
                    odd ? (xg1 >> 16) | (pg1 & 0xffff0000u) : (pg1 & 0xffffu) | (xg1 << 16));
        }
      }
    }
    return;
  }
  if (m0 + kBigM <= M && n0 + T::N <= N) {
    float* cb = C + (m0 + wm * 128 + 4 * lg) * ldc + n0 + wn * 64 + l16;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float* cr = cb + (int64_t)(i * 16 + q) * ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          st_stream(cr + j * 16, scaled ? (float)((double)c[i][j][q] * g) : c[i][j][q]);
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t m = m0 + wm * 128 + i * 16 + 4 * lg + q;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + wn * 64 + j * 16 + l16;
        if (n < N) C[m * ldc + n] = scaled ? (float)((double)c[i][j][q] * g) : c[i][j][q];
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
// A product with few tiles and a deep k range runs split along k: its
// planes go to `partials` (row pitch N, M * N floats each) and
// split_sum_kernel adds them in order into C.
static hipError_t gemm_nt_split(NtProblem p, float* partials, hipStream_t s) {
  const int splits = bwd_splits(p.M, p.N, p.K);
  const int64_t klen = bwd_split_len(p.K, splits);
  const int used = (int)((p.K + klen - 1) / klen);
  float* C = p.C;
  const double* alpha = p.alpha;
  p.C = partials;
  p.ldc = p.N;
  p.alpha = nullptr;
  p.klen = klen;
  NtProblem none = p;
  none.M = 0;  // no tiles
  const unsigned gx = (unsigned)((nt_tiles(p) + 7) / 8 * 8);
  gemm_nt_bf16_kernel<<<dim3(gx, (unsigned)used), 256, 0, s>>>(p, none);
  const int64_t n4 = p.M * p.N / 4;
  const int64_t blocks = (n4 + 255) / 256;
  split_sum_kernel<<<(unsigned)(blocks < 2048 ? blocks : 2048), 256, 0, s>>>(partials, used, n4, alpha, C);
  return hipGetLastError();
}

// Tiles of the products that are not split: 0 chooses per launch by the
// tile counts; 1, 2, 3 fix 128 x 128, 256 x 128 or 256 x 256
// (bitlinear_bwd_tiles).
static std::atomic<int> g_bwd_tiles{0};
int bwd_set_tiles(int tiles) {
  if (tiles < 0 || tiles > 3) return -1;
  g_bwd_tiles.store(tiles, std::memory_order_relaxed);
  return 0;
}
// The tile size with the shorter estimated time, in rounds of one XCD's
// 32 CUs (each XCD runs an eighth of every product).  256 x 256 tiles run
// one per CU and a round costs 1, a partly filled last round too; 256 x 128
// tiles run two per CU at ~1.18 per round (the same flops per CU at the
// lower rate the narrower tiles reach), except a last round that leaves
// every CU at most one tile, which costs ~0.6.  Ties (within 5%) go to
// 256 x 256.  E.g. a 4096 x 2560 dX with its 2560 x 2560 dW (260 large
// tiles: two rounds, the second nearly empty) takes 256 x 128; gate and up
// of the BitNet-2B4T block together (860 large tiles) take 256 x 256.
static int big_kind(const NtSet& set) {
  int64_t n3 = 0, n2 = 0;
  for (int i = 0; i < set.n; ++i) {
    n3 += (nt_tiles_big<4>(set.p[i]) + 7) / 8;
    n2 += (nt_tiles_big<2>(set.p[i]) + 7) / 8;
  }
  const double t3 = (double)((n3 + 31) / 32);
  const int64_t rem2 = n2 % 64;
  const double t2 = 1.18 * (double)(n2 / 64) + (rem2 == 0 ? 0.0 : rem2 <= 32 ? 0.6 : 1.18);
  return t2 < 0.95 * t3 ? 2 : 3;
}
static int bwd_tile_kind(const NtSet& set) {
  const int f = g_bwd_tiles.load(std::memory_order_relaxed);
  return f ? f : big_kind(set);
}
static hipError_t launch_big(const NtSet& set, int kind, hipStream_t s) {
  int64_t per = 0;
  if (kind == 3) {
    for (int i = 0; i < set.n; ++i) per += (nt_tiles_big<4>(set.p[i]) + 7) / 8;
    gemm_nt_bf16_big_kernel<4><<<(unsigned)(8 * per), BigTile<4>::kThreads, 0, s>>>(set);
  } else {
    for (int i = 0; i < set.n; ++i) per += (nt_tiles_big<2>(set.p[i]) + 7) / 8;
    gemm_nt_bf16_big_kernel<2><<<(unsigned)(8 * per), BigTile<2>::kThreads, 0, s>>>(set);
  }
  return hipGetLastError();
}

// The products that are not split run in one launch (a null `b` is no
// second product); split ones follow, one after the other (they share the
// partial planes).
static hipError_t gemm_nt_run(const NtProblem* a, const NtProblem* b, float* partials, hipStream_t s) {
  const NtProblem* whole[2] = {nullptr, nullptr};
  const NtProblem* split[2] = {nullptr, nullptr};
  int nw = 0, ns = 0;
  for (const NtProblem* p : {a, b}) {
    if (!p) continue;
    if (bwd_splits(p->M, p->N, p->K) > 1) split[ns++] = p;
    else whole[nw++] = p;
  }
  if (nw) {
    NtProblem p0 = *whole[0], p1 = p0;
    if (nw == 2) {
      p1 = *whole[1];
      if (p1.K > p0.K) std::swap(p0, p1);  // the deeper product first within each XCD
    } else {
      p1.M = 0;  // no tiles
    }
    NtSet set{};
    set.p[0] = p0;
    set.p[1] = p1;
    set.n = nw;
    const int kind = bwd_tile_kind(set);
    if (kind >= 2) {
      hipError_t e = launch_big(set, kind, s);
      if (e != hipSuccess) return e;
    } else {
      const int64_t per = (nt_tiles(p0) + 7) / 8 + (nt_tiles(p1) + 7) / 8;
      gemm_nt_bf16_kernel<<<(unsigned)(8 * per), 256, 0, s>>>(p0, p1);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int i = 0; i < ns; ++i) {
    hipError_t e = gemm_nt_split(*split[i], partials, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

// the prep tasks of one call, launched together (in chunks of kMaxPrep)
struct PrepList {
  std::vector<PrepTask> t;
  hipError_t launch(int S, hipStream_t s) const {
    for (size_t first = 0; first < t.size(); first += kMaxPrep) {
      PrepSet set{};
      set.n = (int32_t)std::min<size_t>(kMaxPrep, t.size() - first);
      int64_t jobs = 0;
      for (int i = 0; i < set.n; ++i) {
        set.t[i] = t[first + (size_t)i];
        jobs += set.t[i].jobs;
      }
      if (jobs == 0) continue;
      if (S == 8) prep_group_kernel<8><<<(unsigned)jobs, 256, 0, s>>>(set);
      else if (S == 6) prep_group_kernel<6><<<(unsigned)jobs, 256, 0, s>>>(set);
      else if (S == 2) prep_group_kernel<2><<<(unsigned)jobs, 256, 0, s>>>(set);
      else prep_group_kernel<4><<<(unsigned)jobs, 256, 0, s>>>(set);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
};

// dX operand: the codes decoded and transposed (codes^T [k x np])
static void prep_dx(PrepList& L, const void* packed, void* ws, int64_t tokens, int64_t k, int64_t n_out) {
  const int64_t nkb = k / kBlockK, strips = (n_out + kStripRows - 1) / kStripRows;
  uint16_t* codes_t = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + bwd_codes_offset(tokens, k, n_out));
  L.t.push_back(PrepTask{packed, nullptr, codes_t, nkb, strips, strips * kStripRows, kPrepCodes,
                         (int32_t)((strips * nkb + 3) / 4)});
}

// dX [tokens x k] = gamma * dY [tokens x n_out] . codes^T [k x n_out]^T
static NtProblem dx_problem(const uint16_t* dY, const double* gamma, float* dX, void* ws, int64_t tokens,
                            int64_t k, int64_t n_out) {
  const int64_t np = (n_out + kStripRows - 1) / kStripRows * kStripRows;
  const uint16_t* codes_t =
      reinterpret_cast<const uint16_t*>(reinterpret_cast<char*>(ws) + bwd_codes_offset(tokens, k, n_out));
  return NtProblem{dY, codes_t, dX, gamma, n_out, np, k, tokens, k, n_out, n_out};
}

// dW operands: bf16(dY * s)^T unless with_dys is false, x_q^T unless
// with_xq is false (the grouped call reuses another item's x_q^T when two
// items share x_q, and its phases split the two)
static void prep_dw(PrepList& L, const uint16_t* dY, const int8_t* xq, const float* scale, void* ws,
                    int64_t tokens, int64_t k, int64_t n_out, bool with_xq = true, bool with_dys = true) {
  const int64_t tp = bwd_tokens_padded(tokens);
  char* w = reinterpret_cast<char*>(ws);
  uint16_t* dys_t = reinterpret_cast<uint16_t*>(w + bwd_dys_offset(tokens, k, n_out));
  uint16_t* xq_t = reinterpret_cast<uint16_t*>(w + bwd_xq_offset(tokens, k, n_out));
  if (with_dys)
    L.t.push_back(PrepTask{dY, scale, dys_t, tokens, n_out, tp, kPrepDys, (int32_t)((tp / 64) * ((n_out + 63) / 64))});
  if (with_xq) L.t.push_back(PrepTask{xq, nullptr, xq_t, tokens, k, tp, kPrepXq, (int32_t)((tp / 64) * (k / 64))});
}

// dW [n_out x k] = (dY s)^T [n_out x tp] . x_q^T [k x tp]^T
static NtProblem dw_problem(float* dW, void* ws, int64_t tokens, int64_t k, int64_t n_out) {
  const int64_t tp = bwd_tokens_padded(tokens);
  char* w = reinterpret_cast<char*>(ws);
  return NtProblem{reinterpret_cast<const uint16_t*>(w + bwd_dys_offset(tokens, k, n_out)),
                   reinterpret_cast<const uint16_t*>(w + bwd_xq_offset(tokens, k, n_out)),
                   dW, nullptr, tp, tp, k, n_out, k, tp, tp};
}

hipError_t launch_bwd(const uint16_t* dY, const int8_t* xq, const float* scale, const void* packed,
                      const double* gamma, float* dX, float* dW, void* ws, int64_t tokens, int64_t k,
                      int64_t n_out, int S, hipStream_t s) {
  if (tokens == 0) {  // dX is empty; dW is all zeros
    if (dW) zero_f32_kernel<<<1024, 256, 0, s>>>(dW, n_out * k);
    return hipGetLastError();
  }
  PrepList L;
  if (dX) prep_dx(L, packed, ws, tokens, k, n_out);
  if (dW) prep_dw(L, dY, xq, scale, ws, tokens, k, n_out);
  hipError_t e = L.launch(S, s);
  if (e != hipSuccess) return e;
  NtProblem px{}, pw{};
  if (dX) px = dx_problem(dY, gamma, dX, ws, tokens, k, n_out);
  if (dW) pw = dw_problem(dW, ws, tokens, k, n_out);
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + bwd_partial_offset(tokens, k, n_out));
  return gemm_nt_run(dX ? &px : nullptr, dW ? &pw : nullptr, partials, s);
}

// The down projection's backward with the gating backward fused into its
// dX product: the dX tiles never reach memory; their epilogue forms dG and
// dU (the squared-ReLU gating backward of dX, as relu2_gate_bwd_kernel
// computes it), so results equal bitlinear_bwd followed by the gating
// backward bit for bit.  dX runs unsplit on the 256-row kernel (its
// epilogue holds the gating); dW as in launch_bwd.  tokens > 0.
hipError_t launch_bwd_gate(const uint16_t* dY, const int8_t* xq, const float* scale, const void* packed,
                           const double* gamma, const float* G, const float* U, uint16_t* dG, uint16_t* dU,
                           float* dW, void* ws, int64_t tokens, int64_t k, int64_t n_out, int S,
                           hipStream_t s) {
  PrepList L;
  prep_dx(L, packed, ws, tokens, k, n_out);
  if (dW) prep_dw(L, dY, xq, scale, ws, tokens, k, n_out);
  hipError_t e = L.launch(S, s);
  if (e != hipSuccess) return e;
  NtProblem px = dx_problem(dY, gamma, nullptr, ws, tokens, k, n_out);
  px.G = G;
  px.U = U;
  px.dG = dG;
  px.dU = dU;
  NtSet set{};
  set.p[0] = px;
  set.n = 1;
  NtProblem pw{};
  bool dw_split = false;
  if (dW) {
    pw = dw_problem(dW, ws, tokens, k, n_out);
    dw_split = bwd_splits(pw.M, pw.N, pw.K) > 1;
    if (!dw_split) {
      set.p[1] = pw;
      set.n = 2;
      if (pw.K > px.K) std::swap(set.p[0], set.p[1]);  // the deeper product first within each XCD
    }
  }
  const int f = g_bwd_tiles.load(std::memory_order_relaxed);
  e = launch_big(set, f >= 2 ? f : big_kind(set), s);  // 128 x 128 tiles have no gated epilogue
  if (e != hipSuccess) return e;
  if (dw_split) {
    float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + bwd_partial_offset(tokens, k, n_out));
    e = gemm_nt_split(pw, partials, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_group(const BwdItem* items, int count, int64_t tokens, int S, void* ws, int phase,
                            hipStream_t s) {
  // phase bit 0: the conversions that read only packed codes and x_q;
  // bit 1: the dY conversions and the products.  Both walk the items in
  // the same order, so every operand lands at the same place either way
  const bool first = (phase & 1) != 0, second = (phase & 2) != 0;
  std::vector<NtProblem> probs;
  // x_q^T already prepared in this call, by x_q pointer and k: layers fed
  // the same input (q, k, v; gate, up) share it
  struct XqT {
    const int8_t* xq;
    int64_t k;
    const uint16_t* t;
  };
  std::vector<XqT> done;
  PrepList L;
  char* w = reinterpret_cast<char*>(ws);
  for (int i = 0; i < count; ++i) {
    const BwdItem& it = items[i];
    if (it.dX) {
      if (first) prep_dx(L, it.packed, w, tokens, it.k, it.n_out);
      probs.push_back(dx_problem(it.dY, it.gamma, it.dX, w, tokens, it.k, it.n_out));
    }
    if (it.dW) {
      const XqT* seen = nullptr;
      for (const XqT& d : done)
        if (d.xq == it.xq && d.k == it.k) seen = &d;
      prep_dw(L, it.dY, it.xq, it.scale, w, tokens, it.k, it.n_out, first && seen == nullptr, second);
      NtProblem p = dw_problem(it.dW, w, tokens, it.k, it.n_out);
      if (seen) p.B = seen->t;
      else done.push_back(XqT{it.xq, it.k, p.B});
      probs.push_back(p);
    }
    w += bwd_group_item_bytes(tokens, it.k, it.n_out);
  }
  hipError_t pe = L.launch(S, s);
  if (pe != hipSuccess || !second) return pe;
  // deepest contraction first: within each XCD the longest tiles start
  // first and the short ones fill the end (a longest-first schedule)
  std::stable_sort(probs.begin(), probs.end(),
                   [](const NtProblem& a, const NtProblem& b) { return a.K > b.K; });
  for (size_t first = 0; first < probs.size(); first += kMaxNt) {
    NtSet set{};
    set.n = (int32_t)std::min<size_t>(kMaxNt, probs.size() - first);
    for (int i = 0; i < set.n; ++i) set.p[i] = probs[first + (size_t)i];
    const int f = g_bwd_tiles.load(std::memory_order_relaxed);
    hipError_t e = launch_big(set, f >= 2 ? f : big_kind(set), s);  // 128 x 128 tiles take two products only
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace bl

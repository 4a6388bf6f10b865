// gemm.hip -- prefill-shaped BitLinear contraction (many tokens) on gfx950.
//
// acc[t, r] = sum_c x_q[t, c] * code[r, c];  Y = acc * gamma * s_t.
// The pages' custom sparse operator (Sparse-BitNet article §四) gains from
// hardware 6:8 support on other hardware; gfx950 has no 6:8 matrix
// instruction, so the dense int8 MFMA (v_mfma_i32_16x16x64_i8) multiplies
// the pruned zeros and the format only saves weight bytes.
//
// Workgroup tile: four 64-row strips x BT tokens, one strip per wavefront.
// The packed layout stores, for each (strip, 128-wide k block), chunk c as
// exactly the A operands lane c needs for the 8 MFMAs of that block, so a
// wavefront loads its strip's chunks straight into registers and decodes
// them there (LDS tables, one lookup per half group): the codes never pass
// through LDS.  The activations of the tile are the B operands; the four
// wavefronts share them through a double-buffered LDS tile, written once
// per k block and read by every wavefront.  In that tile each B operand
// (16 tokens x 64 k) is one 1 KiB block, with the 16-byte pieces of a row
// XOR-swizzled so that the reads (a permutation within each quarter
// wavefront) and the writes (two tokens x eight pieces per quarter
// wavefront) both spread over all banks.  Per k block a wavefront issues
// the MFMAs of block kb while it decodes block kb+1, writes the activations
// of kb+1 and loads those of kb+3 and the chunk of kb+3 (a three-slot
// register ring for chunks); one barrier per k block.  With BT = 64 (the launched size) LDS stays at 48 KiB and
// registers at <= 168, so three workgroups share a CU; on MI355X that beat
// 128-token tiles at two per CU on every measured shape (more tiles for
// layers with few rows, shorter store bursts at the end of a round).
#include "common.h"
#include "gemm_group.h"
#include "launch.h"

#include <algorithm>
#include <type_traits>

namespace bl {

constexpr int kGStrips = 4;      // strips (wavefronts) per workgroup
constexpr int kGLutCopies = 16;  // table copies: lane l reads copy l % 16
constexpr uint32_t kGOOB = 0x80000000u;  // buffer offset past every range: loads give 0
constexpr int kMaxGemmLayers = 8;       // layers of one grouped prefill launch

__device__ __forceinline__ __amdgpu_buffer_rsrc_t g_rsrc(const void* p, int64_t bytes) {
  const int64_t b = bytes < 0x7fffffff ? bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)b, 0x00020000);
}

// position (in 16-byte units) of activation piece (token tt of the tile,
// 16-byte column c of the 128-wide k block) in one LDS stage: block
// (tt/16, c/4) of 64 pieces, inside it token tt%16 XOR-swizzled by column
__host__ __device__ constexpr int b_slot(int tt, int c) {
  return ((tt >> 4) * 2 + (c >> 2)) * 64 + (((tt & 15) ^ (2 * (c & 3) + 8 * (c >> 2))) + 16 * (c & 3));
}

// Split-k meeting and epilogue of one wavefront's 64-row x 16*kTT-token
// tile (shared by the dense and the sparse-operand kernels): with several
// parts, each part publishes its exact int32 tile (agent-scope stores: the
// reader may sit on another XCD) and takes the (tile, wavefront) ticket;
// the last part adds the others' tiles (agent-scope loads), writes Y and
// returns the ticket to zero.  Lane l holds rows 64*strip + 16i +
// 4*(l/16) + q of token t0 + 16j + l%16.
template <int kTT>
__device__ __forceinline__ void gemm_finish(v4i (&c)[kTT][4], bool live, int splits, int tile, int part,
                                            int wave, int lane, int64_t strip, int64_t t0,
                                            int64_t tokens, int64_t n_out,
                                            const double* __restrict__ gamma,
                                            const float* __restrict__ scale, float* __restrict__ Y,
                                            uint16_t* __restrict__ Yb, int32_t* __restrict__ acc_out,
                                            uint32_t* __restrict__ tickets,
                                            v4i* __restrict__ partials) {
  constexpr int BT = 16 * kTT;
  if (!live) return;
  if (splits > 1) {
    // publish this part's tile (agent-scope stores: the reader may sit on
    // another XCD), take the (tile, wavefront) ticket; the last part adds
    // the others' tiles (agent-scope loads) and writes Y, then returns the
    // ticket to zero
    constexpr int kTileV4 = kTT * 4 * 64;  // v4i per wavefront tile
    unsigned long long* own = reinterpret_cast<unsigned long long*>(
        partials + ((size_t)(tile * splits + part) * kGStrips + wave) * kTileV4);
#pragma unroll
    for (int j = 0; j < kTT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const size_t e = 2 * ((size_t)(j * 4 + i) * 64 + lane);
        st_agent_u64(own + e, (uint32_t)c[j][i][0] | ((unsigned long long)(uint32_t)c[j][i][1] << 32));
        st_agent_u64(own + e + 1, (uint32_t)c[j][i][2] | ((unsigned long long)(uint32_t)c[j][i][3] << 32));
      }
    wait_memory_ops();
    uint32_t t = 0;
    if (lane == 0) t = atomic_fetch_add_global(&tickets[tile * kGStrips + wave], 1u);
    t = __builtin_amdgcn_readfirstlane(t);
    if (t != (uint32_t)splits - 1) return;
    for (int z = 0; z < splits; ++z) {
      if (z == part) continue;
      const unsigned long long* other = reinterpret_cast<const unsigned long long*>(
          partials + ((size_t)(tile * splits + z) * kGStrips + wave) * kTileV4);
#pragma unroll
      for (int j = 0; j < kTT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const size_t e = 2 * ((size_t)(j * 4 + i) * 64 + lane);
          const unsigned long long lo = ld_agent_u64(other + e), hi = ld_agent_u64(other + e + 1);
          c[j][i] += v4i{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi,
                         (int)(uint32_t)(hi >> 32)};
        }
    }
    if (lane == 0) atomic_exchange_global(&tickets[tile * kGStrips + wave], 0u);
  }
  // epilogue: lane holds rows 64*strip + 16i + 4*(lane/16) + q of token
  // t0 + 16j + lane%16
  const double g = *gamma;
  const int64_t r0 = strip * kStripRows + 4 * (lane >> 4);
  if (t0 + BT <= tokens && strip * kStripRows + kStripRows <= n_out && (n_out & 3) == 0) {
    // whole tile in range: 16-byte (8-byte for bf16) stores, no per-element
    // checks; element offsets fit 32 bits (tokens * n_out < 2^31)
    const uint32_t base = (uint32_t)(t0 + (lane & 15)) * (uint32_t)n_out + (uint32_t)r0;
#pragma unroll
    for (int j = 0; j < kTT; ++j) {
      const float gs = out_scale(g, scale[t0 + 16 * j + (lane & 15)]);
      const uint32_t o = base + (uint32_t)(16 * j) * (uint32_t)n_out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4f y = v4f{out_value(c[j][i][0], gs), out_value(c[j][i][1], gs),
                          out_value(c[j][i][2], gs), out_value(c[j][i][3], gs)};
        if (Yb)
          st_stream(reinterpret_cast<u32x2*>(Yb + o + 16 * i), bf16x4(y));
        else
          st_stream(reinterpret_cast<v4f*>(Y + o + 16 * i), y);
        if (acc_out) st_global(reinterpret_cast<v4i*>(acc_out + o + 16 * i), c[j][i]);
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kTT; ++j) {
    const int64_t t = t0 + 16 * j + (lane & 15);
    if (t >= tokens) continue;
    const float gs = out_scale(g, scale[t]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + 16 * i;
      const int64_t e = t * n_out + r;
      if (r + 4 <= n_out && (n_out & 3) == 0) {
        const v4f y = v4f{out_value(c[j][i][0], gs), out_value(c[j][i][1], gs),
                          out_value(c[j][i][2], gs), out_value(c[j][i][3], gs)};
        if (Yb)
          st_global(reinterpret_cast<u32x2*>(Yb + e), bf16x4(y));
        else
          st_global(reinterpret_cast<v4f*>(Y + e), y);
        if (acc_out) st_global(reinterpret_cast<v4i*>(acc_out + e), c[j][i]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (r + q < n_out) {
            const float y = out_value(c[j][i][q], gs);
            if (Yb)
              st_global(Yb + e + q, f32_to_bf16_rne(y));
            else
              st_global(Y + e + q, y);
            if (acc_out) st_global(acc_out + e + q, (int32_t)c[j][i][q]);
          }
      }
    }
  }
}

// One launch covers the layers of a GemmSet: layers that read the same
// activations (x_q, s_t, tokens, k), each with its own codes, gamma and
// output.  Tiles are numbered token block by token block, and within one
// the row blocks of layer 0, then of layer 1, ..., so the workgroups an
// XCD runs together share activations whatever layer they belong to.  A
// single layer is a set of one (its tile order is then the plain one).
struct GemmLayer {
  const uint32_t* packed;
  const double* gamma;
  float* Y;
  uint16_t* Yb;
  int32_t* acc;
  int64_t n_out;
  int32_t row_blocks, first_rb;  // its row blocks; row blocks of the layers before it
};
struct GemmSet {
  GemmLayer l[kMaxGemmLayers];
  int32_t n, row_blocks;  // layers; row blocks of all layers (tiles per token block)
};

template <int S, int BT>
__global__ __launch_bounds__(256, BT == 128 ? 2 : 3) void gemm_kernel(GemmSet set,
                                                     const int8_t* __restrict__ xq,
                                                     const float* __restrict__ scale,
                                                     int64_t tokens, int64_t k,
                                                     int token_blocks, int splits,
                                                     uint32_t* __restrict__ tickets,
                                                     v4i* __restrict__ partials) {
  constexpr int kW = block_bytes(S) / 4;
  constexpr int kTT = BT / 16;           // 16-token tiles
  constexpr int kPieces = BT * 8 / 256;  // 16-byte activation pieces per thread per k block
  __shared__ __attribute__((aligned(16))) v4i Bs[2][kTT * 2 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t lut[512 * kGLutCopies];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; give
  // each XCD a contiguous run of (part, tile) indices (row blocks fastest),
  // so tiles that share activations share that XCD's L2.  The grid is a
  // multiple of 8.
  const int nblk = set.row_blocks * token_blocks;
  const int nwork = nblk * splits;
  const int per_xcd = (nwork + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int full = nwork - (per_xcd - 1) * 8;  // XCDs that get per_xcd items
  const int logical = xcd < full ? xcd * per_xcd + slot
                                 : full * per_xcd + (xcd - full) * (per_xcd - 1) + slot;
  if (slot >= (xcd < full ? per_xcd : per_xcd - 1)) return;
  const int part = logical / nblk, tile = logical - part * nblk;
  const int tb = tile / set.row_blocks, rball = tile - tb * set.row_blocks;
  int li = 0;
  while (li + 1 < set.n && rball >= set.l[li + 1].first_rb) ++li;
  const GemmLayer& L = set.l[li];
  const int rb = rball - L.first_rb;
  const uint32_t* __restrict__ packed = L.packed;
  const double* __restrict__ gamma = L.gamma;
  float* __restrict__ Y = L.Y;
  uint16_t* __restrict__ Yb = L.Yb;
  int32_t* __restrict__ acc_out = L.acc;
  const int64_t n_out = L.n_out;

  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  const int64_t strip = (int64_t)rb * kGStrips + wave;
  const int64_t t0 = (int64_t)tb * BT;
  const int nkb_all = (int)(k / kBlockK);
  // this part's k blocks [kb0, kb0 + nkb)
  const int kb0 = (int)((int64_t)part * nkb_all / splits);
  const int nkb = (int)((int64_t)(part + 1) * nkb_all / splits) - kb0;

  const uint32_t* lut_lane = lut + (lane & (kGLutCopies - 1));

  // activation pieces of this thread: piece q = tid + 256 r is token q/8,
  // 16-byte column q%8 of the k block
  const __amdgpu_buffer_rsrc_t xr = g_rsrc(xq, tokens * k);
  uint32_t x_off[kPieces];
  int x_slot[kPieces];
#pragma unroll
  for (int r = 0; r < kPieces; ++r) {
    const int q = tid + 256 * r, tt = q >> 3, c = q & 7;
    x_off[r] = t0 + tt < tokens ? (uint32_t)((t0 + tt) * k + 16 * c) : kGOOB;
    x_slot[r] = b_slot(tt, c);
  }
  // B operand of token tile j, k half h: lane l takes token 16j + l%16,
  // column l/16 + 4h
  int b_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) b_rd[h] = b_slot(lane & 15, (lane >> 4) + 4 * h);

  // Loads need no guards: a block index past the last one (the prologue
  // and the last blocks run ahead by up to three) either reads the next
  // strip's or token's data, which is never used, or lands past the end of
  // the buffer range (or at kGOOB + small), where buffer loads return zeros.
  const __amdgpu_buffer_rsrc_t pr =
      g_rsrc(packed, strips * nkb_all * kStripRows * block_bytes(S));
  const bool live = strip < strips;
  const uint32_t c_base =
      live ? (uint32_t)((strip * nkb_all * kStripRows + lane) * block_bytes(S)) : kGOOB;

  auto load_x = [&](int kb, u32x4* dst) {
#pragma unroll
    for (int r = 0; r < kPieces; ++r)
      dst[r] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off[r] + (uint32_t)((kb0 + kb) * kBlockK),
                                                     0, 0);
  };
  auto store_x = [&](int p, const u32x4* src) {
#pragma unroll
    for (int r = 0; r < kPieces; ++r) Bs[p][x_slot[r]] = (v4i)src[r];
  };
  auto load_chunk = [&](int kb, uint32_t* dst) {
    const uint32_t o = c_base + (uint32_t)(kb0 + kb) * (uint32_t)(kStripRows * block_bytes(S));
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(pr, o, 0, 0);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    if constexpr (kW == 8) {
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(pr, o + 16, 0, 0);
      dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
    } else if constexpr (kW == 7) {
      const u32x3 b = __builtin_amdgcn_raw_buffer_load_b96(pr, o + 16, 0, 0);
      dst[4] = b.x; dst[5] = b.y; dst[6] = b.z;
    } else if constexpr (kW == 6) {
      const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(pr, o + 16, 0, 0);
      dst[4] = b.x; dst[5] = b.y;
    } else {
      static_assert(kW == 5, "chunk size");
      dst[4] = __builtin_amdgcn_raw_buffer_load_b32(pr, o + 16, 0, 0);
    }
  };
  // one field of a chunk: the codes of field 4i + 2h + q go to lanes
  // 2q, 2q+1 of the A operand (row tile i, k half h)
  auto decode_field = [&](const uint32_t* w, int i, int h, int q, v4i& a) {
    constexpr int kField = 8 + S;
    const int off = (4 * i + 2 * h + q) * kField;
    const int offh = off + S;
    const uint32_t lo_next = (off >> 5) + 1 < kW ? w[(off >> 5) + 1] : 0u;
    const uint32_t hi_next = (offh >> 5) + 1 < kW ? w[(offh >> 5) + 1] : 0u;
    const uint32_t klo = funnel(lo_next, w[off >> 5], off & 31) & 0xffu;
    const uint32_t khi = funnel(hi_next, w[offh >> 5], offh & 31) & 0xffu;
    a[2 * q] = (int)lut_lane[(klo * 2 + 0) * kGLutCopies];
    a[2 * q + 1] = (int)lut_lane[(khi * 2 + 1) * kGLutCopies];
  };

  // accumulators c[j][i]: token tile j, row tile i
  v4i c[kTT][4];
#pragma unroll
  for (int j = 0; j < kTT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) c[j][i] = v4i{0, 0, 0, 0};

  u32x4 xv[2][kPieces];  // activations, two k blocks ahead of their LDS stage
  uint32_t w[3][kW];     // chunk ring: the chunk of k block kb sits in w[kb % 3]
  v4i a[8];              // A operands a[2i + h] (row tile i, k half h)

  // prologue: k block 0 in LDS stage 0 with its half 0 decoded; the
  // activations of blocks 1, 2 and the chunks of blocks 1, 2 in flight
  // tables: 16-byte runs of copies of the compile-time entries (key * 2 +
  // half) from device memory.  Their reads go out before the first blocks'
  // loads (loads complete in order, so behind those they would wait for
  // HBM); the LDS writes happen while those loads fly.
  constexpr int kRuns = 512 * kGLutCopies / 4 / 256;
  uint32_t tv[kRuns];
#pragma unroll
  for (int r = 0; r < kRuns; ++r)
    tv[r] = ld_global(&kHalfCodeTable.v[(tid + 256 * r) / (kGLutCopies / 4)]);
  load_x(0, xv[0]);
  load_chunk(0, w[0]);
  load_chunk(1, w[1]);
  load_chunk(2, w[2]);
  load_x(1, xv[1]);
#pragma unroll
  for (int r = 0; r < kRuns; ++r)
    reinterpret_cast<u32x4*>(lut)[tid + 256 * r] = u32x4{tv[r], tv[r], tv[r], tv[r]};
  store_x(0, xv[0]);
  load_x(2, xv[0]);
  __syncthreads();  // tables and stage 0 ready
#pragma unroll
  for (int f = 0; f < 8; ++f) decode_field(w[0], f >> 1, 0, f & 1, a[2 * (f >> 1)]);

  // One k half of the MFMAs of block kb (parity P) in kTT segments; segment
  // j issues the B operand read of segment j+1, the four MFMAs of token
  // tile j and side work side(j), and the compiler may not move work across
  // segments.  Half 0 runs alongside the decode of half 1 of the same
  // block; half 1 alongside the decode of half 0 of block kb+1, the LDS
  // write of block kb+1's activations and the loads for blocks kb+2/kb+3.
  auto half = [&](auto parity, auto hh, auto&& side) {
    constexpr int P = decltype(parity)::value;
    constexpr int H = decltype(hh)::value;
    v4i b = Bs[P][b_rd[H]];
#pragma unroll
    for (int j = 0; j < kTT; ++j) {
      v4i bn = b;
      if (j + 1 < kTT) bn = Bs[P][b_rd[H] + 128 * (j + 1)];
      else if (H == 0) bn = Bs[P][b_rd[1]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2 * i + H], b, c[j][i], 0, 0, 0);
      side(j);
      __builtin_amdgcn_sched_barrier(0);
      b = bn;
    }
  };
  // side work per segment: the 8 (row tile, field pair) decodes of a half
  // spread over the kTT segments
  static_assert(kTT == 8 || kTT == 4, "side work is laid out for 8 or 4 segments per half");
  constexpr int kPairs = 8 / kTT;
  // k block kb runs with LDS stage P = kb % 2 and chunk slot R = kb % 3.
  // The chunk of kb is decoded (its half 1) during half 0; its slot then
  // takes the load of chunk kb+3, so chunk loads have about three k blocks
  // to land.  Each load writes a fixed register set that nothing copies,
  // so the compiler needs no early wait for it.
  auto kblock = [&](auto parity, auto slot, int kb) {
    constexpr int P = decltype(parity)::value;
    constexpr int R = decltype(slot)::value;
    const uint32_t* wc = w[R];
    const uint32_t* wn = w[(R + 1) % 3];
    // past the last block the side work is harmless and branch-free: the
    // loads read zeros (out-of-range offsets), the decoded codes and the
    // other LDS stage are never used
    half(parity, std::integral_constant<int, 0>{}, [&](int j) {
#pragma unroll
      for (int u = 0; u < kPairs; ++u) {
        const int f = j * kPairs + u;
        decode_field(wc, f >> 1, 1, f & 1, a[2 * (f >> 1) + 1]);
      }
    });
    load_chunk(kb + 3, w[R]);
    half(parity, std::integral_constant<int, 1>{}, [&](int j) {
#pragma unroll
      for (int u = 0; u < kPairs; ++u) {
        const int f = j * kPairs + u;
        decode_field(wn, f >> 1, 0, f & 1, a[2 * (f >> 1)]);
      }
      if (j < kPieces) Bs[P ^ 1][x_slot[j]] = (v4i)xv[P ^ 1][j];
      if (j == kTT / 2) load_x(kb + 3, xv[P ^ 1]);
    });
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int kb = 0;
  for (; kb + 5 < nkb; kb += 6) {  // six blocks: both parities x three slots
    kblock(I0{}, I0{}, kb);
    kblock(I1{}, I1{}, kb + 1);
    kblock(I0{}, I2{}, kb + 2);
    kblock(I1{}, I0{}, kb + 3);
    kblock(I0{}, I1{}, kb + 4);
    kblock(I1{}, I2{}, kb + 5);
  }
  if (kb < nkb) kblock(I0{}, I0{}, kb);
  if (kb + 1 < nkb) kblock(I1{}, I1{}, kb + 1);
  if (kb + 2 < nkb) kblock(I0{}, I2{}, kb + 2);
  if (kb + 3 < nkb) kblock(I1{}, I0{}, kb + 3);
  if (kb + 4 < nkb) kblock(I0{}, I1{}, kb + 4);

  gemm_finish<kTT>(c, live, splits, tile, part, wave, lane, strip, t0, tokens, n_out, gamma, scale, Y,
                   Yb, acc_out, tickets, partials);
}

// ---------------------------------------------------------------------
// 2:4 on the sparse int8 matrix instruction.  gfx950's
// v_smfmac_i32_16x16x128_i8 multiplies a 16 x 128 operand that holds two
// nonzeros per four k -- the structured sparsity the Sparse-BitNet article
// (§七) points to in other vendors' sparse tensor cores -- stored as 16
// values per lane plus a 2-bit position per value, at twice the dense
// rate.  The weights come in the sparse-operand + index layout
// (launch_pack_sp24): lane c of a (strip, k block) superblock loads its
// 32-byte chunk, whose index words feed the instruction as they are and
// whose value words (2-bit codes) become int8 operands with one v_perm per
// four values.  Lane group q of an operand covers dense k [32q, 32q+32);
// its partner in the B operand is k [16q, 16q+16) and [64+16q, 64+16q+16)
// of the same lanes, i.e. the two B operands the dense kernel reads for its
// two k halves, so the activation tile and its reads are the dense
// kernel's.  Per k block a wavefront issues one sparse MFMA per (token
// tile, row tile) -- half the dense kernel's count -- while it decodes the
// next block's operands; chunks ride a four-slot register ring (the chunk
// of block kb in slot kb % 4, loaded four blocks ahead).
// ---------------------------------------------------------------------
__device__ __forceinline__ v4i sp24_values(uint32_t val) {
  // element e's code sits at bit 8(e%4) + 2(e/4): shifting by 2d brings the
  // codes of elements 4d..4d+3 to the low bits of the four bytes, and each
  // selects byte 0 (0x00), 1 (0x01) or 3 (0xff) of 0xff000100
  v4i a;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    a[d] = (int)__builtin_amdgcn_perm(0xff000100u, 0xff000100u, (val >> (2 * d)) & 0x03030303u);
  return a;
}

template <int BT>
__global__ __launch_bounds__(256, 2) void gemm_sp24_kernel(const uint32_t* __restrict__ packed,
                                                          const int8_t* __restrict__ xq,
                                                          const float* __restrict__ scale,
                                                          const double* __restrict__ gamma,
                                                          float* __restrict__ Y,
                                                          uint16_t* __restrict__ Yb,
                                                          int32_t* __restrict__ acc_out,
                                                          int64_t tokens, int64_t k, int64_t n_out,
                                                          int row_blocks, int token_blocks, int splits,
                                                          uint32_t* __restrict__ tickets,
                                                          v4i* __restrict__ partials) {
  constexpr int kTT = BT / 16;
  constexpr int kPieces = BT * 8 / 256;
  constexpr int kChunk = 32;  // bytes per lane per k block
  static_assert(kTT == 4, "one row tile of the next block is decoded per token-tile segment");
  __shared__ __attribute__((aligned(16))) v4i Bs[2][kTT * 2 * 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = row_blocks * token_blocks;
  const int nwork = nblk * splits;
  const int per_xcd = (nwork + 7) / 8;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int full = nwork - (per_xcd - 1) * 8;
  const int logical = xcd < full ? xcd * per_xcd + slot
                                 : full * per_xcd + (xcd - full) * (per_xcd - 1) + slot;
  if (slot >= (xcd < full ? per_xcd : per_xcd - 1)) return;
  const int part = logical / nblk, tile = logical - part * nblk;
  const int rb = tile % row_blocks, tb = tile / row_blocks;

  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  const int64_t strip = (int64_t)rb * kGStrips + wave;
  const int64_t t0 = (int64_t)tb * BT;
  const int nkb_all = (int)(k / kBlockK);
  const int kb0 = (int)((int64_t)part * nkb_all / splits);
  const int nkb = (int)((int64_t)(part + 1) * nkb_all / splits) - kb0;

  const __amdgpu_buffer_rsrc_t xr = g_rsrc(xq, tokens * k);
  uint32_t x_off[kPieces];
  int x_slot[kPieces];
#pragma unroll
  for (int r = 0; r < kPieces; ++r) {
    const int q = tid + 256 * r, tt = q >> 3, c = q & 7;
    x_off[r] = t0 + tt < tokens ? (uint32_t)((t0 + tt) * k + 16 * c) : kGOOB;
    x_slot[r] = b_slot(tt, c);
  }
  int b_rd[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) b_rd[h] = b_slot(lane & 15, (lane >> 4) + 4 * h);

  // out-of-range loads (blocks past the last, strips past the layer) read
  // zeros through the buffer range: no guards, no branches
  const __amdgpu_buffer_rsrc_t pr = g_rsrc(packed, strips * nkb_all * kStripRows * kChunk);
  const bool live = strip < strips;
  const uint32_t c_base = live ? (uint32_t)((strip * nkb_all * kStripRows + lane) * kChunk) : kGOOB;

  auto load_x = [&](int kb, u32x4* dst) {
#pragma unroll
    for (int r = 0; r < kPieces; ++r)
      dst[r] = __builtin_amdgcn_raw_buffer_load_b128(xr, x_off[r] + (uint32_t)((kb0 + kb) * kBlockK),
                                                     0, 0);
  };
  auto load_chunk = [&](int kb, uint32_t* dst) {
    const uint32_t o = c_base + (uint32_t)(kb0 + kb) * (uint32_t)(kStripRows * kChunk);
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(pr, o, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(pr, o + 16, 0, 0);
    dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
    dst[4] = b.x; dst[5] = b.y; dst[6] = b.z; dst[7] = b.w;
  };

  v4i c[kTT][4];
#pragma unroll
  for (int j = 0; j < kTT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) c[j][i] = v4i{0, 0, 0, 0};

  u32x4 xv[2][kPieces];
  uint32_t w[4][8];       // chunk ring: block kb in w[kb % 4]
  v4i a[2][4];            // operands of the current and the next block (set kb % 2)
  int ix[2][4];           // their index words

  load_x(0, xv[0]);
  load_chunk(0, w[0]);
  load_chunk(1, w[1]);
  load_chunk(2, w[2]);
  load_chunk(3, w[3]);
  load_x(1, xv[1]);
#pragma unroll
  for (int r = 0; r < kPieces; ++r) Bs[0][x_slot[r]] = (v4i)xv[0][r];
  load_x(2, xv[0]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[0][i] = sp24_values(w[0][2 * i + 1]);
    ix[0][i] = (int)w[0][2 * i];
  }

  // block kb: LDS stage and operand set P = kb % 2, chunk slot R = kb % 4
  auto kblock = [&](auto parity, auto ring, int kb) {
    constexpr int P = decltype(parity)::value;
    constexpr int R = decltype(ring)::value;
    load_chunk(kb + 4, w[R]);  // block kb's chunk was decoded during block kb-1
    const uint32_t* wn = w[(R + 1) % 4];
    v4i b0 = Bs[P][b_rd[0]], b1 = Bs[P][b_rd[1]];
#pragma unroll
    for (int j = 0; j < kTT; ++j) {
      v4i n0 = b0, n1 = b1;
      if (j + 1 < kTT) {
        n0 = Bs[P][b_rd[0] + 128 * (j + 1)];
        n1 = Bs[P][b_rd[1] + 128 * (j + 1)];
      }
      const v8i b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        c[j][i] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(a[P][i], b, c[j][i], ix[P][i], 0, 0);
      // side work: row tile j of the next block, this thread's activation
      // pieces of the next block into the other stage, the loads of kb+3
      a[P ^ 1][j] = sp24_values(wn[2 * j + 1]);
      ix[P ^ 1][j] = (int)wn[2 * j];
      if (j < kPieces) Bs[P ^ 1][x_slot[j]] = (v4i)xv[P ^ 1][j];
      if (j == kTT / 2) load_x(kb + 3, xv[P ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
      b0 = n0;
      b1 = n1;
    }
    __syncthreads();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int kb = 0;
  for (; kb + 3 < nkb; kb += 4) {
    kblock(I0{}, I0{}, kb);
    kblock(I1{}, I1{}, kb + 1);
    kblock(I0{}, I2{}, kb + 2);
    kblock(I1{}, I3{}, kb + 3);
  }
  if (kb < nkb) kblock(I0{}, I0{}, kb);
  if (kb + 1 < nkb) kblock(I1{}, I1{}, kb + 1);
  if (kb + 2 < nkb) kblock(I0{}, I2{}, kb + 2);

  gemm_finish<kTT>(c, live, splits, tile, part, wave, lane, strip, t0, tokens, n_out, gamma, scale, Y,
                   Yb, acc_out, tickets, partials);
}

hipError_t launch_gemm_sp24(const void* packed, const int8_t* xq, const float* scale,
                            const double* gamma, float* Y, int32_t* acc, void* ws, int64_t tokens,
                            int64_t k, int64_t n_out, hipStream_t s) {
  uint16_t* const Yb = nullptr;
  constexpr int BT = kGemmTileTokens;
  static_assert(kGemmTileRows == kGStrips * kStripRows, "tile rows");
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  const int row_blocks = (int)((strips + kGStrips - 1) / kGStrips);
  const int token_blocks = (int)((tokens + BT - 1) / BT);
  const int splits = gemm_splits(tokens, k, n_out);
  if (splits > 1 && !ws) return hipErrorInvalidValue;
  uint32_t* tickets = splits > 1 ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  v4i* partials = splits > 1 ? reinterpret_cast<v4i*>(reinterpret_cast<char*>(ws) +
                                                      gemm_ticket_bytes(tokens, n_out))
                             : nullptr;
  const int nwork = row_blocks * token_blocks * splits;
  gemm_sp24_kernel<BT><<<(unsigned)((nwork + 7) / 8 * 8), 256, 0, s>>>(
      reinterpret_cast<const uint32_t*>(packed), xq, scale, gamma, Y, Yb, acc, tokens, k, n_out,
      row_blocks, token_blocks, splits, tickets, partials);
  return hipGetLastError();
}

template <int S>
static hipError_t launch_gemm_s(const void* packed, const int8_t* xq, const float* scale,
                                const double* gamma, float* Y, uint16_t* Yb, int32_t* acc, void* ws,
                                int64_t tokens, int64_t k, int64_t n_out, hipStream_t s) {
  constexpr int BT = kGemmTileTokens;
  static_assert(kGemmTileRows == kGStrips * kStripRows, "tile rows");
  static_assert(BT == 64, "launch bounds assume three workgroups per CU");
  const int64_t strips = (n_out + kStripRows - 1) / kStripRows;
  const int row_blocks = (int)((strips + kGStrips - 1) / kGStrips);
  const int token_blocks = (int)((tokens + BT - 1) / BT);
  const int splits = gemm_splits(tokens, k, n_out);
  if (splits > 1 && !ws) return hipErrorInvalidValue;
  uint32_t* tickets = splits > 1 ? reinterpret_cast<uint32_t*>(ws) : nullptr;
  v4i* partials = splits > 1 ? reinterpret_cast<v4i*>(reinterpret_cast<char*>(ws) +
                                                      gemm_ticket_bytes(tokens, n_out))
                             : nullptr;
  const int nwork = row_blocks * token_blocks * splits;
  GemmSet set{};
  set.l[0] = GemmLayer{reinterpret_cast<const uint32_t*>(packed), gamma, Y, Yb, acc, n_out, row_blocks, 0};
  set.n = 1;
  set.row_blocks = row_blocks;
  gemm_kernel<S, BT><<<(unsigned)((nwork + 7) / 8 * 8), 256, 0, s>>>(set, xq, scale, tokens, k, token_blocks,
                                                                    splits, tickets, partials);
  return hipGetLastError();
}

// Layers that read the same activations, in launches of up to
// kMaxGemmLayers layers each, never split along k
template <int S>
static hipError_t launch_gemm_group_s(const GemmGroupLayer* layers, int count, const int8_t* xq,
                                      const float* scale, int64_t tokens, int64_t k, hipStream_t s) {
  constexpr int BT = kGemmTileTokens;
  const int token_blocks = (int)((tokens + BT - 1) / BT);
  for (int first = 0; first < count; first += kMaxGemmLayers) {
    GemmSet set{};
    set.n = std::min(kMaxGemmLayers, count - first);
    int rbs = 0;
    for (int i = 0; i < set.n; ++i) {
      const GemmGroupLayer& g = layers[first + i];
      const int64_t strips = (g.n_out + kStripRows - 1) / kStripRows;
      const int row_blocks = (int)((strips + kGStrips - 1) / kGStrips);
      set.l[i] = GemmLayer{reinterpret_cast<const uint32_t*>(g.packed), g.gamma, g.Y, g.Yb, g.acc, g.n_out,
                           row_blocks, rbs};
      rbs += row_blocks;
    }
    set.row_blocks = rbs;
    const int nwork = rbs * token_blocks;
    gemm_kernel<S, BT><<<(unsigned)((nwork + 7) / 8 * 8), 256, 0, s>>>(set, xq, scale, tokens, k, token_blocks,
                                                                      1, nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemm_group(const GemmGroupLayer* layers, int count, const int8_t* xq, const float* scale,
                             int64_t tokens, int64_t k, int S, hipStream_t s) {
  if (S == 8) return launch_gemm_group_s<8>(layers, count, xq, scale, tokens, k, s);
  if (S == 6) return launch_gemm_group_s<6>(layers, count, xq, scale, tokens, k, s);
  if (S == 2) return launch_gemm_group_s<2>(layers, count, xq, scale, tokens, k, s);
  return launch_gemm_group_s<4>(layers, count, xq, scale, tokens, k, s);
}

hipError_t launch_gemm(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, uint16_t* Yb, int32_t* acc, void* ws,
                       int64_t tokens, int64_t k, int64_t n_out, int S, hipStream_t s) {
  if (S == 8) return launch_gemm_s<8>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
  if (S == 6) return launch_gemm_s<6>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
  if (S == 2) return launch_gemm_s<2>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
  return launch_gemm_s<4>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
}

}  // namespace bl

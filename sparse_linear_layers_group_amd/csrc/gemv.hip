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

constexpr int kGemvThreads = 1024;  // 16 wavefronts, one block per CU
constexpr int kGemvWaves = kGemvThreads / 64;
constexpr int kLutCopies = 64;      // one table copy per LDS bank: lane l reads copy l
constexpr int64_t kResidentWaves = 256 * kGemvWaves;

// Tables in LDS: entry (key, half) of copy c at dword (key * 2 + half) * 64 + c
// (128 KB).  Lane l always reads copy l, i.e. bank l, so a wavefront's 64
// lookups never collide whatever the keys.  The fill first computes the 512
// distinct entries into a small table, then writes the big one linearly
// (consecutive lanes, consecutive 16-byte chunks: no bank conflicts).
__device__ __forceinline__ void fill_lut(uint32_t* lut, uint32_t* entries) {
  for (int idx = threadIdx.x; idx < 512; idx += blockDim.x)
    entries[idx] = half_codes(idx >> 1, idx & 1);  // entry index = key * 2 + half
  __syncthreads();
  constexpr int kChunks = 512 * kLutCopies / 4;  // 16-byte chunks
  for (int ch = threadIdx.x; ch < kChunks; ch += blockDim.x) {
    const uint32_t v = entries[ch / (kLutCopies / 4)];
    reinterpret_cast<uint4*>(lut)[ch] = make_uint4(v, v, v, v);
  }
}

// wavefront index within the block, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ---------------------------------------------------------------------
// Streaming loop.  A wavefront walks a contiguous range of units (16-row
// tiles, or k ranges of a tile) as one flat sequence of 512-wide
// super-tiles.  The loads of the next super-tile (packed codes and
// activations) are issued before the current one is decoded, across unit
// boundaries, so every wavefront keeps loads in flight while it computes.
// Loads go through buffer resources: a lane whose block or token is out of
// range gets an offset past the end of the buffer and reads zeros (no
// branches, no zero fills).
// ---------------------------------------------------------------------
constexpr uint32_t kOOB = 0x80000000u;  // beyond every buffer (all < 2^31 bytes)
constexpr int kDepth = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

struct Unit {
  __amdgpu_buffer_rsrc_t pk, xr;  // unit's packed blocks / item's activations
  int32_t nst;                    // super-tiles in the unit
  int32_t nkb;                    // k blocks from the unit's first column to the row end
  int32_t k;                      // x_q row stride
  int32_t x_col;                  // first k column of the unit
  // epilogue
  float* Y;
  const float* scale;
  const double* gamma;
  int64_t row0, n_out, tile;
};

template <int S>
struct Stage {
  uint32_t w[block_bytes(S) / 4];
  v4i b[8];
};

template <int S>
__device__ __forceinline__ void issue(Stage<S>& st, const Unit& u, int sti, bool live, int lane,
                                      int tokens) {
  constexpr int kBytes = block_bytes(S);
  const int r16 = lane & 15, grp = lane >> 4;
  const int kb = 4 * sti + grp;
  const bool blk = live && kb < u.nkb;
  const uint32_t po = blk ? (uint32_t)(sti * 64 + lane) * kBytes : kOOB;
  if constexpr (kBytes == 32) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(u.pk, po, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(u.pk, po + 16, 0, 0);
    st.w[0] = a.x; st.w[1] = a.y; st.w[2] = a.z; st.w[3] = a.w;
    st.w[4] = b.x; st.w[5] = b.y; st.w[6] = b.z; st.w[7] = b.w;
  } else if constexpr (kBytes == 28) {
    typedef unsigned int u32x3 __attribute__((ext_vector_type(3)));
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(u.pk, po, 0, 0);
    const u32x3 b = __builtin_amdgcn_raw_buffer_load_b96(u.pk, po + 16, 0, 0);
    st.w[0] = a.x; st.w[1] = a.y; st.w[2] = a.z; st.w[3] = a.w;
    st.w[4] = b.x; st.w[5] = b.y; st.w[6] = b.z;
  } else {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(u.pk, po, 0, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(u.pk, po + 16, 0, 0);
    st.w[0] = a.x; st.w[1] = a.y; st.w[2] = a.z; st.w[3] = a.w;
    st.w[4] = b.x; st.w[5] = b.y;
  }
  // B operand: the MFMA's output columns >= tokens are never stored, so
  // those lanes may hold anything -- they read token 0's row (a broadcast of
  // the same address, cheap for the address unit) instead of a masked load.
  // A block past the row end has all-zero codes, so its activations are
  // irrelevant too; those lanes read block 0.
  const uint32_t xo =
      (uint32_t)((r16 < tokens ? r16 : 0) * u.k) + (uint32_t)u.x_col + (uint32_t)(blk ? kb * kBlockK : 0);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(u.xr, xo + 16 * m, 0, 0);
    st.b[m] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
  }
}

template <int S>
__device__ __forceinline__ v4i decode_mma(const Stage<S>& st, v4i c, const uint32_t* lut_lane) {
  constexpr int kW = block_bytes(S) / 4;
  constexpr int kField = 8 + S;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    v4i a;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int off = (2 * m + q) * kField;
      const int offh = off + S;
      const uint32_t lo_hi = (off >> 5) + 1 < kW ? st.w[(off >> 5) + 1] : 0u;
      const uint32_t hi_hi = (offh >> 5) + 1 < kW ? st.w[(offh >> 5) + 1] : 0u;
      const uint32_t klo = funnel(lo_hi, st.w[off >> 5], off & 31) & 0xffu;
      const uint32_t khi = funnel(hi_hi, st.w[offh >> 5], offh & 31) & 0xffu;
      a[2 * q] = (int)lut_lane[(klo * 2 + 0) * kLutCopies];
      a[2 * q + 1] = (int)lut_lane[(khi * 2 + 1) * kLutCopies];
    }
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, st.b[m], c, 0, 0, 0);
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
      st_global(&Y[(int64_t)token * n_out + row], (float)((double)c[i] * g * st));
      if (acc_out) st_global(&acc_out[(int64_t)token * n_out + row], (int32_t)c[i]);
    }
  }
}

// Walk `count` units of `src` from cursor `first`.  A source policy has a
// cursor type Cur holding the current Unit (wave-uniform, in scalar
// registers), next(cur) to move a cursor to the following unit -- plain
// arithmetic except when a grouped plan changes item, which is rare -- and
// finish(unit, acc, ...) for the epilogue.  No memory is read per step, so
// no scalar-cache miss (whose counter the LDS lookups share) sits in the
// loop.
template <int S, class Src>
__device__ __forceinline__ void stream(const Src& src, const uint32_t* lut_lane, int lane,
                                       typename Src::Cur first, int64_t count) {
  if (count <= 0) return;
  const int tokens = src.tokens;
  // the load cursor runs kDepth-1 super-tiles ahead of the compute cursor
  typename Src::Cur L = first, C = first;
  int64_t lleft = count, cleft = count;
  int lst = 0, cst = 0;
  bool live = true;
  Stage<S> ring[kDepth];
  auto load_step = [&](Stage<S>& st) {
    issue<S>(st, L.u, lst, live, lane, tokens);
    if (++lst == L.u.nst) {
      lst = 0;
      if (--lleft == 0) live = false;
      else src.next(L);
    }
  };
#pragma unroll
  for (int s = 0; s < kDepth - 1; ++s) load_step(ring[s]);
  v4i c = {0, 0, 0, 0};
  // token scale and gamma are loaded when a unit starts, long before its
  // epilogue needs them: the epilogue never waits on a fresh load (which
  // would also drain the prefetched loads behind it)
  const int tok = lane & 15;
  float s_tok = tok < tokens ? ld_global(&C.u.scale[tok]) : 0.f;
  double g = ld_global(C.u.gamma);
  while (true) {
#pragma unroll
    for (int s = 0; s < kDepth; ++s) {
      load_step(ring[(s + kDepth - 1) % kDepth]);
      c = decode_mma<S>(ring[s], c, lut_lane);
      if (++cst == C.u.nst) {
        src.finish(C.u, c, lane, s_tok, g);
        c = v4i{0, 0, 0, 0};
        cst = 0;
        if (--cleft == 0) return;
        src.next(C);
        s_tok = tok < tokens ? ld_global(&C.u.scale[tok]) : 0.f;
        g = ld_global(C.u.gamma);
      }
    }
  }
}

// one GEMV, k optionally split into ranges of st_per_unit super-tiles
struct SingleSrc {
  const void* packed;
  const int8_t* xq;
  uint32_t x_bytes;
  const float* scale;
  const double* gamma;
  float* Y;
  int32_t* acc_out;
  int32_t* partial;
  uint32_t* tickets;
  int64_t units, n_out;
  int32_t k, nkb, nst, ksplit, st_per_unit, tokens, kbytes;

  struct Cur {
    Unit u;
    int64_t idx;
  };

  __device__ Unit unit(int64_t u) const {
    const int64_t tile = u / ksplit;
    const int part = (int)(u - tile * ksplit);
    const int st0 = part * st_per_unit;
    Unit r;
    r.nst = min(st_per_unit, nst - st0);
    r.pk = rsrc(reinterpret_cast<const char*>(packed) +
                    (size_t)((tile * nkb + 4 * st0) * kTileRows) * kbytes,
                (uint32_t)(r.nst * 64 * kbytes));
    r.xr = rsrc(xq, x_bytes);
    r.nkb = nkb - 4 * st0;
    r.k = k;
    r.x_col = 4 * st0 * kBlockK;
    r.Y = Y;
    r.scale = scale;
    r.gamma = gamma;
    r.row0 = tile * kTileRows;
    r.n_out = n_out;
    r.tile = tile;
    return r;
  }
  __device__ Cur start(int64_t u) const { return Cur{unit(u), u}; }
  __device__ void next(Cur& c) const {
    c.idx += 1;
    c.u = unit(c.idx);
  }

  __device__ void finish(const Unit& u, const v4i& c, int lane, float s_tok, double g) const {
    const int r16 = lane & 15, grp = lane >> 4;
    const bool tok_ok = r16 < tokens;
    const int64_t row0 = u.row0 + 4 * grp;
    const double st = (double)s_tok;
    if (ksplit == 1) {
      if (tok_ok) store_tile(Y, acc_out, c, row0, n_out, r16, g, st);
      return;
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
    if (lane == 0) t = atomicAdd(&tickets[u.tile], 1u);
    t = __shfl(t, 0, 64);
    if (t != (uint32_t)(ksplit - 1)) return;
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
    if (lane == 0) atomicExch(&tickets[u.tile], 0u);
  }
};

// many GEMVs from a device plan; units are the 16-row tiles of the items,
// in item order
template <int S>
struct GroupSrc {
  const GroupItem* items;
  int32_t count, tokens;

  struct Cur {
    Unit u;
    int32_t item, tiles;
    uint64_t tile_stride;  // packed bytes per 16-row tile
    const char* pk_base;   // packed blocks of the current tile
  };

  __device__ void load_item(Cur& c, int32_t item, int32_t tile) const {
    const GroupItem& it = items[item];
    const int32_t k = (int32_t)it.k;
    const int32_t nkb = k / kBlockK;
    const int64_t n_out = it.n_out;
    c.item = item;
    c.tiles = (int32_t)((n_out + kTileRows - 1) / kTileRows);
    c.tile_stride = (uint64_t)nkb * kTileRows * block_bytes(S);
    c.pk_base = reinterpret_cast<const char*>(it.packed) + (uint64_t)tile * c.tile_stride;
    c.u.nst = (nkb + 3) / 4;
    c.u.pk = rsrc(c.pk_base, (uint32_t)(c.u.nst * 64 * block_bytes(S)));
    c.u.xr = rsrc(it.xq, (uint32_t)(tokens * k));
    c.u.nkb = nkb;
    c.u.k = k;
    c.u.x_col = 0;
    c.u.Y = it.Y;
    c.u.scale = it.scale;
    c.u.gamma = it.gamma;
    c.u.row0 = (int64_t)tile * kTileRows;
    c.u.n_out = n_out;
    c.u.tile = tile;
  }
  __device__ Cur start(int32_t item, int32_t tile) const {
    Cur c;
    load_item(c, item, tile);
    return c;
  }
  __device__ void next(Cur& c) const {
    if (c.u.tile + 1 < c.tiles) {  // same item: arithmetic only
      c.u.tile += 1;
      c.u.row0 += kTileRows;
      c.pk_base += c.tile_stride;
      c.u.pk = rsrc(c.pk_base, (uint32_t)(c.u.nst * 64 * block_bytes(S)));
    } else if (c.item + 1 < count) {
      load_item(c, c.item + 1, 0);
    }
  }

  __device__ void finish(const Unit& u, const v4i& c, int lane, float s_tok, double g) const {
    const int r16 = lane & 15, grp = lane >> 4;
    if (r16 < tokens) store_tile(u.Y, nullptr, c, u.row0 + 4 * grp, u.n_out, r16, g, (double)s_tok);
  }
};

template <int S>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(SingleSrc src) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 2 * kLutCopies];
  __shared__ uint32_t entries[512];
  fill_lut(lut, entries);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  // contiguous, equal ranges of units per wavefront
  const int64_t nw = (int64_t)gridDim.x * kGemvWaves;
  const int64_t w = (int64_t)blockIdx.x * kGemvWaves + wave_id();
  const int64_t u0 = src.units * w / nw, u1 = src.units * (w + 1) / nw;
  if (u0 < u1) stream<S>(src, lut + lane, lane, src.start(u0), u1 - u0);
}

template <int S>
__global__ __launch_bounds__(kGemvThreads) void gemv_group_kernel(const char* __restrict__ plan) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 2 * kLutCopies];
  __shared__ uint32_t entries[512];
  fill_lut(lut, entries);
  __syncthreads();
  const GroupHeader* hdr = reinterpret_cast<const GroupHeader*>(plan);
  GroupSrc<S> src;
  src.items = reinterpret_cast<const GroupItem*>(plan + sizeof(GroupHeader));
  src.count = hdr->count;
  src.tokens = hdr->tokens;
  const WaveStart* starts =
      reinterpret_cast<const WaveStart*>(plan + group_starts_offset(hdr->count, hdr->rows));
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * kGemvWaves + wave_id();
  const WaveStart a = starts[w], b = starts[w + 1];
  if (a.unit < b.unit) stream<S>(src, lut + lane, lane, src.start(a.item, a.tile), b.unit - a.unit);
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
  SingleSrc src;
  const int64_t nkb = k / kBlockK;
  src.packed = packed;
  src.xq = xq;
  src.x_bytes = (uint32_t)(tokens * k);
  src.scale = scale;
  src.gamma = gamma;
  src.Y = Y;
  src.acc_out = acc;
  src.partial = nullptr;
  src.tickets = nullptr;
  if (p.ksplit > 1) {
    src.partial = reinterpret_cast<int32_t*>(ws);
    src.tickets = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(ws) +
                                              align256((size_t)tokens * n_out * 4));
  }
  src.units = p.units;
  src.n_out = n_out;
  src.k = (int32_t)k;
  src.nkb = (int32_t)nkb;
  src.nst = (int32_t)((nkb + 3) / 4);
  src.ksplit = p.ksplit;
  src.st_per_unit = p.st_per_unit;
  src.tokens = tokens;
  src.kbytes = block_bytes(S);
  int64_t blocks = (p.units + kGemvWaves - 1) / kGemvWaves;
  if (blocks > 256) blocks = 256;
  gemv_kernel<S><<<(unsigned)blocks, kGemvThreads, 0, s>>>(src);
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
  if (S == 8) gemv_group_kernel<8><<<kGroupBlocks, kGemvThreads, 0, s>>>(p);
  else if (S == 6) gemv_group_kernel<6><<<kGroupBlocks, kGemvThreads, 0, s>>>(p);
  else gemv_group_kernel<4><<<kGroupBlocks, kGemvThreads, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace bl

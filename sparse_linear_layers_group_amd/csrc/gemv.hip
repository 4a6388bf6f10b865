// gemv.hip -- decode-shaped BitLinear contraction (tokens <= 16) on gfx950.
//
// acc[t, r] = sum_c x_q[t, c] * code[r, c];  Y = acc * gamma * s_t.
// BitNet b1.58 2B4T article §四 describes the GPU recipe for ternary x int8:
// pack the ternary codes, stream them from HBM, unpack next to the compute
// and multiply with the int8 activations, to make the most of memory
// bandwidth.  This kernel keeps that shape for the bitmap+sign format and
// CDNA4:
//
//  * A step is one packed superblock: 64 weight rows x one 128-wide k block.
//    Lane c loads chunk c -- the 2(8+S) bytes holding exactly the groups its
//    A operands need -- so a wavefront's 64 loads are one contiguous span.
//  * Each 8-group decodes from two 8-bit keys (low half: bitmap + first
//    four signs; high half: last four signs + bitmap) through two 256-entry
//    tables of int8x4 codes in LDS.  Lane l reads copy l % 32 of the tables
//    (32 copies), so the lookups of a half wavefront never conflict.
//  * The codes go straight into v_mfma_i32_16x16x64_i8 as the A operand
//    (row tile i, k half h); the B operand is the 16 activation bytes of
//    token l%16 at k slice l/16 of that half -- two 16-byte loads per step
//    serve all four row tiles and any token count.  int32 accumulation is
//    exact.
//  * Loads run kDepth-1 steps ahead of the decode (a register ring), across
//    strip and item boundaries.
//  * Each workgroup runs a list of steps, cut into 16 equal contiguous
//    ranges, one per wavefront, so every wavefront streams the same number
//    of bytes whatever the layer shapes.  Whole strips are written as they
//    finish; a strip cut between wavefronts is summed in LDS (over the
//    then-dead code tables) by its first wavefront once all are done.  A
//    strip cut between workgroups -- only single calls with too few strips
//    to fill the chip -- meets in an int32 workspace through integer
//    atomics (order independent, hence bit-reproducible); the last
//    workgroup to contribute writes it and leaves the workspace zeroed.
//  * The grouped kernel runs many GEMVs (same token count and pattern) from
//    one device-resident plan in a single launch; the plan gives every
//    workgroup whole strips, packed on the host for equal step counts.
#include "actq.h"
#include "common.h"
#include "launch.h"

namespace bl {

constexpr int kGemvThreads = 1024;  // 16 wavefronts, one workgroup per CU
constexpr int kGemvWaves = kGemvThreads / 64;
static_assert(kGemvWaves == kDecodeWavesPerBlock, "wavefronts per workgroup");
constexpr int kLutCopies = kDecodeLutCopies;  // lane l reads copy l % 32
constexpr int kDepth = 3;       // register ring: steps in flight + 1
constexpr int kSlotDwords = 16 * kStripRows;  // one wavefront's cut-strip sums [token][row]

// Tables in LDS: entry (key, half) of copy c at dword (key * 2 + half) * 32 + c
// (64 KB).  Lane l always reads copy l % 32, i.e. bank l % 32, so the
// lookups of each half wavefront never collide whatever the keys (64 copies
// measured no faster on MI355X and took twice the LDS and fill time).  The
// fill reads
// the 512 entries from the compile-time table in device memory and writes
// the big one linearly (consecutive lanes, consecutive 16-byte chunks: no
// conflicts).  The reads are issued before the first steps' loads: loads
// complete in order, and a table read queued behind them would wait for
// HBM (measured: ~3 us from entry to the filled tables that way).
constexpr int kLutChunks = 512 * kLutCopies / 4;  // 16-byte chunks
static_assert(kLutChunks % kGemvThreads == 0, "every thread fills the same count");
struct LutVals {
  uint32_t v[kLutChunks / kGemvThreads];
};
__device__ __forceinline__ LutVals load_lut() {
  LutVals t;
#pragma unroll
  for (int r = 0; r < kLutChunks / kGemvThreads; ++r)
    t.v[r] = ld_global(&kHalfCodeTable.v[(threadIdx.x + kGemvThreads * r) / (kLutCopies / 4)]);
  return t;
}
__device__ __forceinline__ void write_lut(uint32_t* lut, const LutVals& t) {
#pragma unroll
  for (int r = 0; r < kLutChunks / kGemvThreads; ++r)
    reinterpret_cast<uint4*>(lut)[threadIdx.x + kGemvThreads * r] = make_uint4(t.v[r], t.v[r], t.v[r], t.v[r]);
}
static_assert(kGemvWaves * kSlotDwords <= 256 * 2 * kLutCopies, "cut-strip slots fit the tables");

// wavefront index within the block, as a wave-uniform (scalar) value
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Loads go through buffer resources: a lane past the end of the range gets
// an offset beyond the buffer and reads zeros (no branches, no zero fills).
constexpr uint32_t kOOB = 0x80000000u;  // beyond every buffer (all < 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// what a wavefront needs of the strip it streams (wave-uniform, scalar
// registers)
struct StripView {
  __amdgpu_buffer_rsrc_t pk, xr;  // the strip's superblocks / the item's activations
  int32_t k, nkb, row0;
  int64_t n_out;
  float* Y;
  uint16_t* Yb;  // bf16 outputs instead of Y when not null
  int32_t* acc;  // optional int32 sums
  uint32_t x_lds, s_lds;  // fused runs: LDS byte offsets of the item's codes and scales
  const float* scale;
  const double* gamma;
};

template <int S>
__device__ __forceinline__ StripView make_strip(const char* strip_packed, const int8_t* xq,
                                                int tokens, int32_t k, int64_t n_out,
                                                int32_t row0) {
  StripView v;
  v.k = k;
  v.nkb = k / kBlockK;
  v.row0 = row0;
  v.n_out = n_out;
  v.pk = rsrc(strip_packed, (uint32_t)(v.nkb * kStripRows * block_bytes(S)));
  v.xr = rsrc(xq, (uint32_t)(tokens * k));
  return v;
}

// position in a workgroup's list; sid numbers the strips of the list
struct Cursor {
  StripView sv;
  int32_t kb, sid;
};

// One step in flight: packed words, the B operand, and -- for the first
// step of a strip -- the strip's token scale and gamma.  Those two small
// loads ride with that step, and the compute cursor takes them when it
// decodes it, so a strip's epilogue never waits on a later load (which
// would also drain the steps loaded behind it: loads complete in order).
template <int S>
struct Stage {
  uint32_t w[block_bytes(S) / 4];
  v4i b[2];
  float sc;
  double gm;
};

// kLdsX: the activations come from the workgroup's LDS copy (fused runs),
// read when the step is decoded (lds_operands), not here: the first steps
// are issued before the copy exists
template <int S, bool kLdsX>
__device__ __forceinline__ void issue(Stage<S>& st, const Cursor& cur, bool live, int lane,
                                      int tokens) {
  constexpr int kBytes = block_bytes(S);
  const uint32_t po = live ? ((uint32_t)cur.kb * kStripRows + (uint32_t)lane) * kBytes : kOOB;
  uint32_t* w = st.w;
  if constexpr (kBytes == 32) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(cur.sv.pk, po, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(cur.sv.pk, po + 16, 0, 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else if constexpr (kBytes == 28) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(cur.sv.pk, po, 0, 0);
    const u32x3 b = __builtin_amdgcn_raw_buffer_load_b96(cur.sv.pk, po + 16, 0, 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z;
  } else if constexpr (kBytes == 24) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(cur.sv.pk, po, 0, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(cur.sv.pk, po + 16, 0, 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y;
  } else {
    static_assert(kBytes == 20, "chunk size");
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(cur.sv.pk, po, 0, 0);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = __builtin_amdgcn_raw_buffer_load_b32(cur.sv.pk, po + 16, 0, 0);
  }
  // B operand of k half h: token t = lane%16, k slice lane/16.  Columns
  // t >= tokens are never stored, so those lanes read token 0 (in range).
  if constexpr (!kLdsX) {
    const int t = lane & 15, g = lane >> 4;
    const uint32_t xo = (uint32_t)((t < tokens ? t : 0) * cur.sv.k + cur.kb * kBlockK + 16 * g);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(cur.sv.xr, xo + 64 * h, 0, 0);
      st.b[h] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    }
  }
}

// A zero the compiler cannot see through.  Each strip's first stage loads
// its own copy of the strip's scales: merged with an earlier stage's
// identical load, the stage's registers became a copy of that one, and the
// copy waited for every load in flight.
__device__ __forceinline__ uint32_t opaque_zero() {
  uint32_t z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// Fused runs: the B operands of the step the compute cursor is at, and its
// strip's token scale, from the LDS copy
template <int S>
__device__ __forceinline__ void lds_operands(Stage<S>& st, const Cursor& cur, int lane, int tokens,
                                             const char* lds_x) {
  typedef __attribute__((address_space(3))) char lds_char;
  const int t = lane & 15, g = lane >> 4;
  const int tt = t < tokens ? t : 0;
  const uint32_t xo = cur.sv.x_lds + (uint32_t)(tt * cur.sv.k + cur.kb * kBlockK + 16 * g);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    st.b[h] = *reinterpret_cast<const __attribute__((address_space(3))) v4i*>((const lds_char*)lds_x + xo + 64 * h);
  st.sc = *reinterpret_cast<const __attribute__((address_space(3))) float*>(
      (const lds_char*)lds_x + cur.sv.s_lds + 4 * tt + opaque_zero());
}

template <int S, bool kLdsX>
__device__ __forceinline__ void issue_scale(Stage<S>& st, const Cursor& cur, int lane, int tokens) {
  const int t = lane & 15;
  const uint32_t z = opaque_zero();
  if constexpr (!kLdsX) st.sc = ld_global(&cur.sv.scale[(t < tokens ? t : 0) + z]);
  st.gm = ld_global(cur.sv.gamma + z);
}

// A operand of MFMA m = 2i + h: codes of fields 2m and 2m+1 of the chunk
template <int S>
__device__ __forceinline__ v4i a_operand(const uint32_t* w, int m, const uint32_t* lut_lane) {
  constexpr int kW = block_bytes(S) / 4;
  constexpr int kField = 8 + S;
  v4i a;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int off = (2 * m + q) * kField;
    const int offh = off + S;
    const uint32_t lo_hi = (off >> 5) + 1 < kW ? w[(off >> 5) + 1] : 0u;
    const uint32_t hi_hi = (offh >> 5) + 1 < kW ? w[(offh >> 5) + 1] : 0u;
    const uint32_t klo = funnel(lo_hi, w[off >> 5], off & 31) & 0xffu;
    const uint32_t khi = funnel(hi_hi, w[offh >> 5], offh & 31) & 0xffu;
    a[2 * q] = (int)lut_lane[(klo * 2 + 0) * kLutCopies];
    a[2 * q + 1] = (int)lut_lane[(khi * 2 + 1) * kLutCopies];
  }
  return a;
}

// one superblock: row tile i, k half h -> c[i]
template <int S>
__device__ __forceinline__ void decode_step(const Stage<S>& st, v4i* c, const uint32_t* lut_lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      c[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a_operand<S>(st.w, 2 * i + h, lut_lane),
                                                   st.b[h], c[i], 0, 0, 0);
}

// Outputs of lane (t, g) for one strip: rows row0 + 16i + 4g + j.
__device__ __forceinline__ void store_strip(const StripView& it, const v4i* c, int lane,
                                            int tokens, float gs) {
  const int64_t row0 = it.row0;
  const int t = lane & 15, g = lane >> 4;
  if (t >= tokens) return;
  const int64_t o = (int64_t)t * it.n_out + row0 + 4 * g;
  const bool vec = row0 + kStripRows <= it.n_out && (tokens == 1 || (it.n_out & 3) == 0);
  if (vec) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v4f v = v4f{out_value(c[i][0], gs), out_value(c[i][1], gs), out_value(c[i][2], gs),
                        out_value(c[i][3], gs)};
      if (it.Yb)
        st_global(reinterpret_cast<u32x2*>(it.Yb + o + 16 * i), bf16x4(v));
      else
        st_global(reinterpret_cast<v4f*>(it.Y + o + 16 * i), v);
      if (it.acc) st_global(reinterpret_cast<v4i*>(it.acc + o + 16 * i), c[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (row0 + 16 * i + 4 * g + j < it.n_out) {
          const float v = out_value(c[i][j], gs);
          if (it.Yb)
            st_global(it.Yb + o + 16 * i + j, f32_to_bf16_rne(v));
          else
            st_global(it.Y + o + 16 * i + j, v);
          if (it.acc) st_global(it.acc + o + 16 * i + j, (int32_t)c[i][j]);
        }
  }
}

__device__ __forceinline__ float strip_scale(const StripView& it, int lane, int tokens) {
  const int t = lane & 15;
  return out_scale(ld_global(it.gamma), ld_global(&it.scale[t < tokens ? t : 0]));
}

// A wavefront's first step and its number of steps.
struct WaveRange {
  Cursor first;
  int64_t count;
};

// Run one workgroup.  A source policy provides tokens, strip(sid) (the view
// of strip sid of the list), advance(cursor), range(w) -- the first step
// and step count of wavefront w of this workgroup -- and cross()/
// cross_sum() for strips that continue in another workgroup.
template <int S, class Src>
__device__ __forceinline__ void run_block(const Src& src, uint32_t* lut,
                                          int lane) {
  // the table reads go first (they depend on nothing); the first steps'
  // loads are in flight while the workgroup builds the code tables
  const LutVals lv = load_lut();
  // fused runs: the workgroup's activation segments, issued before the
  // first weight loads so that they return first (loads complete in order)
  const typename Src::Rows rows = src.load_rows(lane);
  const int tokens = src.tokens;
  const int w = wave_id();
  const uint32_t* lut_lane = lut + (lane & (kLutCopies - 1));
  const WaveRange wr = src.range(w);
  const int64_t count = wr.count;
  Cursor L = wr.first, C = wr.first;
  int64_t lleft = count, cleft = count;
  bool live = count > 0;
  const bool started_mid = count > 0 && C.kb > 0;
  bool first_open = started_mid;  // the first strip has not ended yet
  v4i c[4], cf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = v4i{0, 0, 0, 0};
    cf[i] = v4i{0, 0, 0, 0};
  }
  bool ended_mid = false;
  int32_t last_sid = -1;
  Stage<S> ring[kDepth];
  // once the load cursor has issued the last step it stops for good:
  // advance() may read the plan, and must never step past the range
  bool l_first = true, c_first = true;
  // output scale of the current strip, and of the wavefront's first strip.
  // Formed from the stage's registers when the strip's first step is
  // decoded: a plain copy of them let the compiler share the registers with
  // the ring, and every back edge then copied the next stage's scales out
  // of their load registers, waiting for all loads in flight.
  float cur_gs = 0.f;
  float first_gs = 0.f;
  auto load_step = [&](Stage<S>& st) {
    issue<S, Src::kLdsX>(st, L, live, lane, tokens);
    if (L.kb == 0 || l_first) issue_scale<S, Src::kLdsX>(st, L, lane, tokens);  // wave-uniform
    l_first = false;
    if (live) {
      if (--lleft == 0) live = false;
      else src.advance(L);
    }
  };
  // issued by idle wavefronts too (past-the-end offsets read zeros): the
  // same loads on every path keep the compiler's completion counts exact,
  // so the tables (loaded first) are written without waiting for the steps
#pragma unroll
  for (int s = 0; s < kDepth - 1; ++s) load_step(ring[s]);
  // lane v < 16 holds wavefront v's (first strip, first k block, step
  // count) for the end phase (no loads there); read after the first steps'
  // loads so that nothing waits for it before then
  const v4i winfo = src.wave_info(lane & 15);
  write_lut(lut, lv);
  if constexpr (Src::kLdsX) {
    // fused runs: segment maxima, then the codes from registers
    src.publish_max(rows, lane);
    __syncthreads();
    src.quantise(rows, lane);
  }
  __syncthreads();
  if (count > 0) {
    while (cleft > 0) {
#pragma unroll
      for (int s = 0; s < kDepth; ++s) {
        load_step(ring[(s + kDepth - 1) % kDepth]);
        if constexpr (Src::kLdsX) lds_operands<S>(ring[s], C, lane, tokens, src.lds_x);
        decode_step<S>(ring[s], c, lut_lane);
        if (C.kb == 0 || c_first) {  // the strip's scales came with this step
          cur_gs = out_scale(ring[s].gm, ring[s].sc);
          if (c_first) first_gs = cur_gs;
          c_first = false;
        }
        --cleft;
        if (C.kb == C.sv.nkb - 1) {  // strip end
          if (first_open) {
            // the tail of a strip begun by an earlier wavefront: keep it
#pragma unroll
            for (int i = 0; i < 4; ++i) cf[i] = c[i];
            first_open = false;
          } else {
            store_strip(C.sv, c, lane, tokens, cur_gs);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = v4i{0, 0, 0, 0};
        } else if (cleft == 0) {
          ended_mid = true;
          last_sid = C.sid;
        }
        if (cleft == 0) break;
        src.advance(C);
      }
    }
  }
  // ---- cut strips: the code tables are dead; their LDS holds one slot of
  // sums per wavefront: the part of its first strip when that strip began
  // in an earlier wavefront's range
  __syncthreads();
  int32_t* slots = reinterpret_cast<int32_t*>(lut);
  const int t = lane & 15, g = lane >> 4;
  if (started_mid && t < tokens) {
    int32_t* d = slots + w * kSlotDwords + t * kStripRows + 4 * g;
    const v4i* part = first_open ? c : cf;  // still open: the range lies inside that strip
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(d + 16 * i) = part[i];
  }
  __syncthreads();
  // The first wavefront touching a cut strip sums it: the wavefront whose
  // range ends inside a strip that began in its own range, and wavefront 0
  // for a strip that began in an earlier workgroup (both can hold).
  const bool head_last = ended_mid && !(started_mid && first_open);
  const bool head_first = w == 0 && started_mid;
  for (int role = 0; role < 2; ++role) {
    const bool last = role == 1;
    if (last ? !head_last : !head_first) continue;
    v4i tot[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] = last ? c[i] : v4i{0, 0, 0, 0};
    const int32_t sid = last ? last_sid : wr.first.sid;
    for (int v = last ? w + 1 : 0; v < kGemvWaves; ++v) {
      const int32_t v_sid = __builtin_amdgcn_readlane(winfo[0], v);
      const int32_t v_kb = __builtin_amdgcn_readlane(winfo[1], v);
      const int32_t v_count = __builtin_amdgcn_readlane(winfo[2], v);
      if (v_count == 0) continue;
      if (v_sid != sid || v_kb == 0) break;
      if (t < tokens) {
        const int32_t* q = slots + v * kSlotDwords + t * kStripRows + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] += *reinterpret_cast<const v4i*>(q + 16 * i);
      }
    }
    // the cursor still holds the view of the last strip; wavefront 0 the
    // view of its first
    const StripView sv = last ? C.sv : wr.first.sv;
    if (src.cross(sid))
      src.cross_sum(sv, sid, tot, lane);
    else
      // the scales came with the strip's first step (no load here: one at
      // the end of the kernel would expose a full memory latency)
      store_strip(sv, tot, lane, tokens, last ? cur_gs : first_gs);
  }
}

// ---------------------------------------------------------------- single call
// T = strips * nkb steps cut into NB equal workgroup ranges; a strip cut by
// a workgroup boundary meets in the workspace.  sid = strip index.
template <int S>
struct SingleSrc {
  static constexpr bool kLdsX = false;
  const char* lds_x;  // unused
  const char* packed;
  const int8_t* xq;
  float* Y;
  uint16_t* Yb;
  int32_t* acc;
  const float* scale;
  const double* gamma;
  int32_t* partial;   // [strips][tokens][64]
  uint32_t* tickets;  // [strips]
  int64_t n_out, T, NB;
  int32_t k, nkb;
  int tokens;
  __device__ StripView strip(int32_t sid) const {
    StripView v = make_strip<S>(packed + (int64_t)sid * nkb * kStripRows * block_bytes(S), xq,
                                tokens, k, n_out, sid * kStripRows);
    v.Y = Y;
    v.Yb = Yb;
    v.acc = acc;
    v.x_lds = 0;
    v.s_lds = 0;
    v.scale = scale;
    v.gamma = gamma;
    return v;
  }
  __device__ void advance(Cursor& c) const {
    if (++c.kb == nkb) {
      c.kb = 0;
      c.sv = strip(++c.sid);
    }
  }
  __device__ WaveRange range(int w) const {
    const int64_t b = blockIdx.x;
    const int64_t b0 = T * b / NB, n = T * (b + 1) / NB - b0;
    const int64_t s0 = b0 + wave_split(n, w), s1 = b0 + wave_split(n, w + 1);
    WaveRange r;
    r.count = s1 - s0;
    r.first.sid = (int32_t)(s0 / nkb);
    r.first.kb = (int32_t)(s0 - (int64_t)r.first.sid * nkb);
    r.first.sv = strip(r.first.sid);
    return r;
  }
  // (first strip, first k block, step count) of wavefront v
  __device__ v4i wave_info(int v) const {
    const int64_t b = blockIdx.x;
    const int64_t b0 = T * b / NB, n = T * (b + 1) / NB - b0;
    const int64_t s0 = b0 + wave_split(n, v), s1 = b0 + wave_split(n, v + 1);
    const int32_t sid = (int32_t)(s0 / nkb);
    return v4i{sid, (int32_t)(s0 - (int64_t)sid * nkb), (int32_t)(s1 - s0), 0};
  }
  struct Rows {};
  __device__ Rows load_rows(int) const { return Rows{}; }
  // does strip `sid` continue in another workgroup?
  __device__ bool cross(int32_t sid) const {
    const int64_t b = blockIdx.x;
    const int64_t a = (int64_t)sid * nkb, e = a + nkb;
    return a < T * b / NB || e > T * (b + 1) / NB;
  }
  // add this workgroup's part of the strip; the last workgroup writes it
  __device__ void cross_sum(const StripView& sv, int32_t sid, const v4i* tot, int lane) const {
    const int t = lane & 15, g = lane >> 4;
    int32_t* p = partial + ((int64_t)sid * tokens + (t < tokens ? t : 0)) * kStripRows + 4 * g;
    if (t < tokens) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tot[i][j] != 0) atomic_add_global(p + 16 * i + j, (int32_t)tot[i][j]);
    }
    const int64_t a = (int64_t)sid * nkb, e = a + nkb - 1;
    const int64_t blocks = block_of_step(e, T, NB) - block_of_step(a, T, NB) + 1;
    // every partial sum of this workgroup's part is performed before its ticket
    wait_memory_ops();
    uint32_t tk = 0;
    if (lane == 0) tk = atomic_fetch_add_global(&tickets[sid], 1u);
    tk = __shfl(tk, 0, 64);
    if ((int64_t)tk != blocks - 1) return;
    wait_memory_ops();
    v4i sum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sum[i][j] = t < tokens ? atomic_exchange_global(p + 16 * i + j, 0) : 0;
    store_strip(sv, sum, lane, tokens, strip_scale(sv, lane, tokens));
    if (lane == 0) atomic_exchange_global(&tickets[sid], 0u);
  }
};

// --------------------------------------------------------------- grouped
// sid = index of the strip descriptor in the plan.  kFused: the workgroup
// quantises the activation rows of its items into LDS first (segments of
// them, the wavefront's own read with its start record), and its steps
// read their B operands and scales there.
template <int S, bool kFused>
struct GroupSrc {
  static constexpr bool kLdsX = kFused;
  const StripDesc* strips;
  const WaveStart* starts;
  WaveStart mine;  // this wavefront's start record, read at entry
  int tokens;
  const char* lds_x;  // fused: LDS base of the activation codes
  FusedSeg seg[kFused ? kFusedSegsPerWave : 1];  // fused: this wavefront's segments
  __device__ StripView view(const StripDesc& d) const {
    StripView v = make_strip<S>(d.packed, d.xq, tokens, d.k, d.n_out, d.row0);
    v.Y = d.Y;
    v.Yb = nullptr;
    v.acc = nullptr;
    v.x_lds = (uint32_t)d.pad[0];
    v.s_lds = (uint32_t)d.pad[1];
    v.scale = d.scale;
    v.gamma = d.gamma;
    return v;
  }
  __device__ StripView strip(int32_t sid) const { return view(strips[sid]); }
  __device__ void advance(Cursor& c) const {
    if (++c.kb == c.sv.nkb) {
      c.kb = 0;
      c.sv = strip(++c.sid);
    }
  }
  __device__ WaveRange range(int) const {
    const WaveStart& ws = mine;
    WaveRange r;
    r.count = ws.count;
    r.first.sid = ws.rec;
    r.first.kb = ws.kb;
    r.first.sv = view(ws.first);
    return r;
  }
  // (first strip, first k block, step count) of wavefront v: the 12 bytes
  // after the wave start's descriptor.  Only those three are loaded: with a
  // fourth, unused word in the load, the compiler reused its register at
  // once and waited for the load (the newest of all) before the tables.
  __device__ v4i wave_info(int v) const {
    const u32x3 r = ld_global(reinterpret_cast<const u32x3*>(&starts[(int64_t)blockIdx.x * kGemvWaves + v].rec));
    return v4i{(int)r.x, (int)r.y, (int)r.z, 0};
  }
  // the plan never cuts a strip between workgroups
  __device__ bool cross(int32_t) const { return false; }
  __device__ void cross_sum(const StripView&, int32_t, const v4i*, int) const {}

  // Fused runs.  Lane l holds values [8l, 8l + 8) and [512 + 8l, ...) of
  // each of the wavefront's segments.  Every load and store below is issued
  // whatever the segment count: buffer accesses past a segment's end (or of
  // a missing segment, an empty buffer) read zeros and store nothing, so
  // the loads' completion counts stay exact and nothing waits early.
  struct Rows {
    u32x4 v[kFused ? kFusedSegsPerWave : 1][2];
  };
  __device__ Rows load_rows(int lane) const {
    Rows r;
    if constexpr (kFused) {
#pragma unroll
      for (int j = 0; j < kFusedSegsPerWave; ++j) {
        const __amdgpu_buffer_rsrc_t x = rsrc(seg[j].x, 2 * (uint32_t)seg[j].nvals);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          r.v[j][h] = __builtin_amdgcn_raw_buffer_load_b128(x, 16 * lane + 1024 * h, 0, 0);
      }
    }
    return r;
  }
  __device__ static float seg_absmax(const Rows& r, int j) {
    return fmaxf(absmax8(make_uint4(r.v[j][0].x, r.v[j][0].y, r.v[j][0].z, r.v[j][0].w)),
                 absmax8(make_uint4(r.v[j][1].x, r.v[j][1].y, r.v[j][1].z, r.v[j][1].w)));
  }
  typedef __attribute__((address_space(3))) float lds_float;
  __device__ lds_float* max_slots() const {
    typedef __attribute__((address_space(3))) char lds_char;
    return reinterpret_cast<lds_float*>((lds_char*)lds_x + kFusedCodeBytes);
  }
  // each segment's absmax into its LDS slot
  __device__ void publish_max(const Rows& r, int lane) const {
    if constexpr (kFused) {
      lds_float* slots = max_slots();
#pragma unroll
      for (int j = 0; j < kFusedSegsPerWave; ++j) {
        const float a = wave_max(seg_absmax(r, j));
        if (seg[j].nvals > 0 && lane == 0) slots[seg[j].slot] = a;
      }
    }
  }
  // the row's absmax (maximum over its segments' slots), then the codes
  // into LDS and, in the writer, into x_q and x_scale -- exactly as the
  // activation kernel forms them (quant8 / absmax8, s = a / 127)
  __device__ void quantise(const Rows& r, int lane) const {
    if constexpr (kFused) {
      typedef __attribute__((address_space(3))) char lds_char;
      const lds_float* slots = max_slots();
#pragma unroll
      for (int j = 0; j < kFusedSegsPerWave; ++j) {
        const FusedSeg& f = seg[j];
        const float a = wave_max(lane < f.row_slots ? slots[f.row_slot + lane] : 0.f);
        const __amdgpu_buffer_rsrc_t xq = rsrc(f.xq, f.xq ? (uint32_t)f.nvals : 0u);
        const __amdgpu_buffer_rsrc_t sc = rsrc(f.scale, f.scale ? 4u : 0u);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 x = r.v[j][h];
          const uint2 q = quant8(make_uint4(x.x, x.y, x.z, x.w), a);
          const int v = 512 * h + 8 * lane;
          if (f.nvals > 0 && v < f.nvals)
            *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
                (lds_char*)lds_x + f.lds_q + (uint32_t)v) = u32x2{q.x, q.y};
          __builtin_amdgcn_raw_buffer_store_b64(u32x2{q.x, q.y}, xq, (uint32_t)v, 0, 0);
        }
        const float s = a / 127.0f;
        if (f.first && lane == 0)
          *reinterpret_cast<__attribute__((address_space(3))) float*>((lds_char*)lds_x + f.lds_s) = s;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, s), sc, lane == 0 ? 0u : kOOB, 0, 0);
      }
    }
  }
};

template <int S>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(SingleSrc<S> src) {
  __shared__ __attribute__((aligned(16))) uint32_t lut[256 * 2 * kLutCopies];
  run_block<S>(src, lut, threadIdx.x & 63);
}

// every Y of every item of a plan set to a quiet NaN (grid-stride)
__device__ __noinline__ void poison_outputs(const char* plan, const GroupHeader* hdr) {
  const GroupItem* items =
      reinterpret_cast<const GroupItem*>(plan + group_items_offset(hdr->rows, hdr->strips));
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int32_t i = 0; i < hdr->count; ++i) {
    const int64_t n = (int64_t)hdr->tokens * items[i].n_out;
    float* y = items[i].Y;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride)
      st_global(y + e, __builtin_nanf(""));
  }
}

template <int S, bool kFused>
__global__ __launch_bounds__(kGemvThreads) void gemv_group_kernel(const char* __restrict__ plan) {
  // fused runs keep the workgroup's activation codes after the tables
  __shared__ __attribute__((aligned(16))) uint32_t lut[kFused ? 160 * 1024 / 4 : 256 * 2 * kLutCopies];
  GroupSrc<S, kFused> src;
  src.starts = reinterpret_cast<const WaveStart*>(plan + group_waves_offset());
  // The header fields and this wavefront's whole start record are read
  // before the first branch, in one round trip (read after the header
  // tests, each took a round trip of its own: ~0.5 us of a 20 us launch).
  // Each wavefront tests the flag in its own record; all records of a
  // workgroup carry the same flag, so the whole workgroup leaves or stays.
  const GroupHeader* hdr = reinterpret_cast<const GroupHeader*>(plan);
  const int64_t rows = hdr->rows;
  const int32_t h_s = hdr->S;
  src.tokens = hdr->tokens;
  // fused runs: the plan's flag and this wavefront's segments, in the same
  // round trip
  int32_t h_fused = 1;
  if constexpr (kFused) {
    h_fused = hdr->fused;
    const FusedSeg* fs = reinterpret_cast<const FusedSeg*>(plan + group_fused_offset()) +
                         ((int64_t)blockIdx.x * kGemvWaves + wave_id()) * kFusedSegsPerWave;
#pragma unroll
    for (int j = 0; j < kFusedSegsPerWave; ++j) src.seg[j] = fs[j];
  }
  src.mine = src.starts[(int64_t)blockIdx.x * kGemvWaves + wave_id()];
  if constexpr (kFused) {
    static_assert(kFusedSegsPerWave == 4, "one wait for all segment records");
#define BL_SEG_OPS(j) "+s"(src.seg[j].x), "+s"(src.seg[j].xq), "+s"(src.seg[j].scale), \
    "+s"(src.seg[j].lds_q), "+s"(src.seg[j].lds_s), "+s"(src.seg[j].nvals)
    asm volatile("" : BL_SEG_OPS(0), BL_SEG_OPS(1), BL_SEG_OPS(2), BL_SEG_OPS(3), "+s"(h_fused));
#undef BL_SEG_OPS
  }
  asm volatile("" : "+s"(src.mine.first.packed), "+s"(src.mine.first.xq), "+s"(src.mine.first.Y),
               "+s"(src.mine.first.scale), "+s"(src.mine.first.gamma), "+s"(src.mine.first.n_out),
               "+s"(src.mine.first.k), "+s"(src.mine.first.row0), "+s"(src.mine.rec), "+s"(src.mine.kb),
               "+s"(src.mine.count), "+s"(src.mine.active) : "s"(h_s), "s"(rows), "s"(src.tokens));
  if (h_s != S || !h_fused) {
    // a plan made for another sign-slot count (its strips are laid out for
    // that count), or a fused run of a plan whose workgroups' activations
    // do not fit LDS or the segment slots: no packed byte is read; every
    // output becomes a quiet NaN instead
    poison_outputs(plan, hdr);
    return;
  }
  if (!src.mine.active) return;
  src.strips = reinterpret_cast<const StripDesc*>(plan + group_strips_offset(rows));
  src.lds_x = reinterpret_cast<const char*>(lut + kDecodeLutBytes / 4);
  run_block<S>(src, lut, threadIdx.x & 63);
}

template <int S>
static hipError_t launch_gemv_s(const void* packed, const int8_t* xq, const float* scale,
                                const double* gamma, float* Y, uint16_t* Yb, int32_t* acc, void* ws,
                                int tokens, int64_t k, int64_t n_out, hipStream_t s) {
  SingleSrc<S> src;
  src.lds_x = nullptr;
  src.packed = reinterpret_cast<const char*>(packed);
  src.xq = xq;
  src.Y = Y;
  src.Yb = Yb;
  src.acc = acc;
  src.scale = scale;
  src.gamma = gamma;
  src.partial = reinterpret_cast<int32_t*>(ws);
  src.tickets = reinterpret_cast<uint32_t*>(
      reinterpret_cast<char*>(ws) + ((decode_partial_bytes(tokens, n_out) + 255) & ~(size_t)255));
  src.k = (int32_t)k;
  src.n_out = n_out;
  src.tokens = tokens;
  src.nkb = (int32_t)(k / kBlockK);
  src.T = ((n_out + kStripRows - 1) / kStripRows) * src.nkb;
  src.NB = decode_blocks(src.T);
  gemv_kernel<S><<<(unsigned)src.NB, kGemvThreads, 0, s>>>(src);
  return hipGetLastError();
}

hipError_t launch_gemv(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, uint16_t* Yb, int32_t* acc, void* ws,
                       int tokens, int64_t k, int64_t n_out, int S, hipStream_t s) {
  if (S == 8) return launch_gemv_s<8>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
  if (S == 6) return launch_gemv_s<6>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
  if (S == 2) return launch_gemv_s<2>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
  return launch_gemv_s<4>(packed, xq, scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, s);
}

template <bool kFused>
static void launch_group_s(const char* p, int S, hipStream_t s) {
  if (S == 8) gemv_group_kernel<8, kFused><<<kDecodeBlocks, kGemvThreads, 0, s>>>(p);
  else if (S == 6) gemv_group_kernel<6, kFused><<<kDecodeBlocks, kGemvThreads, 0, s>>>(p);
  else if (S == 2) gemv_group_kernel<2, kFused><<<kDecodeBlocks, kGemvThreads, 0, s>>>(p);
  else gemv_group_kernel<4, kFused><<<kDecodeBlocks, kGemvThreads, 0, s>>>(p);
}

hipError_t launch_gemv_group(const void* plan, int S, bool fused, hipStream_t s) {
  const char* p = reinterpret_cast<const char*>(plan);
  if (fused) launch_group_s<true>(p, S, s);
  else launch_group_s<false>(p, S, s);
  return hipGetLastError();
}

}  // namespace bl

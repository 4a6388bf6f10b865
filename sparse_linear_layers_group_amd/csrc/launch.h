// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/bitlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

// Mask + exact absmean scale: kernel 1 (mask_blocks workgroups, each a
// contiguous range of 8-groups) writes the mask and one exact partial sum
// per workgroup into the workspace; kernel 2 (one workgroup) adds the
// partials and writes gamma.  Workspace: a 32-byte record per workgroup,
// then 256 64-bit exponent bins per workgroup (written only by workgroups
// that met magnitudes outside the two fixed-point windows).
constexpr int kMaskBlocksMax = 1024;
constexpr int kMaskGroupsPerPass = 1024;  // 8-groups per workgroup pass
__host__ __device__ inline int64_t mask_blocks(int64_t n_out, int64_t k) {
  const int64_t passes = (n_out * k / 8 + kMaskGroupsPerPass - 1) / kMaskGroupsPerPass;
  return passes < 1 ? 1 : passes > kMaskBlocksMax ? kMaskBlocksMax : passes;
}
__host__ __device__ inline size_t gamma_ws_bytes(int64_t n_out, int64_t k) {
  return (size_t)mask_blocks(n_out, k) * (32 + 256 * 8);
}

hipError_t launch_mask_gamma(const uint16_t* W, int64_t n_out, int64_t k, int n, int m,
                             int gamma_over, uint8_t* mask, double* gamma, void* ws,
                             hipStream_t s);

// Grouped weight quantisation: one device plan describes many layers; the
// mask kernel, the gamma kernel and the pack kernel each run every layer
// in one launch.  Plan image: header (64 bytes) | item descriptors[count] |
// owner table (one int32 item index per mask workgroup, then one per pack
// workgroup).  Each layer keeps its own gamma workspace region.
struct QuantGroupHeader {
  int32_t count, pad;
  int64_t mask_blocks, pack_blocks;  // workgroups of the mask and pack launches
  int32_t n, m, gamma_over, pad1;    // what the plan was made for; a launch with
                                     // other values writes nothing
  int64_t pad2[3];
};
static_assert(sizeof(QuantGroupHeader) == 64, "quant plan header size");
struct QuantItemDesc {  // one layer (128 bytes)
  const uint16_t* W;
  uint8_t* mask;
  double* gamma;
  void* packed;
  char* ws;                   // the layer's gamma workspace (gamma_ws_bytes)
  int64_t n_out, k;
  int64_t ngroups, per;       // 8-groups, and 8-groups per mask workgroup
  int64_t mblock0, nmblocks;  // first mask workgroup of the layer, and how many
  int64_t pblock0;            // first pack workgroup of the layer
  int64_t pad[4];
};
static_assert(sizeof(QuantItemDesc) == 128, "quant item size");
__host__ __device__ inline size_t quant_owner_offset(int64_t count) {
  return sizeof(QuantGroupHeader) + (size_t)count * sizeof(QuantItemDesc);
}
inline size_t quant_plan_bytes(int64_t count, int64_t mask_blocks, int64_t pack_blocks) {
  return quant_owner_offset(count) + (size_t)(mask_blocks + pack_blocks) * 4;
}
// 8-groups per mask workgroup of a layer (a whole number of passes)
inline int64_t mask_groups_per_block(int64_t n_out, int64_t k) {
  const int64_t ngroups = n_out * k / 8, blocks = mask_blocks(n_out, k);
  const int64_t per = (ngroups + blocks - 1) / blocks;
  return (per + kMaskGroupsPerPass - 1) / kMaskGroupsPerPass * kMaskGroupsPerPass;
}
inline int64_t pack_blocks(int64_t n_out, int64_t k) {
  const int64_t chunks = ((n_out + 63) / 64) * 64 * (k / 128);
  return (chunks + 255) / 256;
}
// The three launches have fixed grids (the host does not read the plan);
// workgroup g of a launch takes the plan's workgroups g, g + grid, ...
constexpr int kQuantGrid = 2048;      // mask and pack launches: 8 workgroups per CU
constexpr int kQuantGammaGrid = 256;  // gamma launch: one workgroup per layer, strided
hipError_t launch_quant_group(const void* plan, int n, int m, int gamma_over, hipStream_t s);

// ternary codes -> packed blocks (packed may be null) and/or int8 codes (wq
// may be null); S = sign slots per 8-group
hipError_t launch_ternary_pack(const uint16_t* W, const uint8_t* mask, const double* gamma,
                               int64_t n_out, int64_t k, int S, void* packed, int8_t* wq,
                               hipStream_t s);

// 2:4 codes in the sparse-operand + index layout: 32 bytes per chunk, one
// chunk per (strip, 128-wide k block, lane)
inline size_t sp24_packed_bytes(int64_t n_out, int64_t k) {
  return (size_t)((n_out + 63) / 64) * 64 * (size_t)(k / 128) * 32;
}
hipError_t launch_pack_sp24(const uint16_t* W, const uint8_t* mask, const double* gamma,
                            int64_t n_out, int64_t k, void* packed, hipStream_t s);

// per-token int8 activations; also zero-fills zero_bytes of zero_ws
// latent-weight update: Wm = RN32(Wm - lr * dW) (one fused rounding), W =
// bf16 (nearest, ties to even) of the result; count a multiple of 8
hipError_t launch_latent_update(float* Wm, const float* dW, int64_t count, float lr, uint16_t* W,
                                hipStream_t s);

// squared-ReLU gating of a block's feed-forward: h = bf16((relu(g)^2) * u)
// (binary32 products), written to H (may be null), then per-token int8
// activations of h exactly as launch_act_quant forms them; and its
// backward, dU = bf16(dh * r^2), dG = bf16((dh * u) * 2r), r = relu(g)
hipError_t launch_relu2_gate(const float* G, const float* U, int64_t tokens, int64_t n, uint16_t* H,
                             int8_t* xq, float* scale, hipStream_t s);
hipError_t launch_relu2_gate_bwd(const float* dH, const float* G, const float* U, int64_t count,
                                 uint16_t* dG, uint16_t* dU, hipStream_t s);

hipError_t launch_act_quant(const uint16_t* X, int64_t tokens, int64_t k, int8_t* xq,
                            float* scale, void* zero_ws, int64_t zero_bytes, hipStream_t s);

// Decode-shaped contraction (tokens <= 16).  A step is one packed
// superblock (64 rows x 128 k); a strip is the nkb steps of one 64-row
// strip of one weight.  Each workgroup (16 wavefronts, one per CU) runs a
// list of steps; its wavefronts split that list into 16 equal contiguous
// ranges.  A strip cut between wavefronts of one workgroup is summed in
// LDS at the workgroup's end; a strip cut between workgroups (single calls
// with few strips only) meets in an int32 workspace, and the last
// workgroup to contribute writes it.
constexpr int kDecodeBlocks = 256;     // one workgroup per CU
constexpr int kDecodeLutCopies = 32;   // code table copies in the decode kernels' LDS
constexpr int kDecodeWavesPerBlock = 16;
constexpr int kMinStepsPerBlock = 16;  // at least ~1 step per wavefront
__host__ __device__ inline int64_t decode_blocks(int64_t steps) {
  int64_t nb = steps / kMinStepsPerBlock;
  return nb < 1 ? 1 : (nb > kDecodeBlocks ? kDecodeBlocks : nb);
}
// A workgroup's 16 wavefronts take contiguous ranges of its steps in
// proportion to kWaveWeight[w / 4].  Wavefront w runs on SIMD w % 4, and
// the SIMD favours its older wavefronts when several can issue, so with
// equal ranges the older ones finished early (measured on MI355X: ~14 us
// for wavefronts 0-3 against ~18 us for 12-15 in a 24-layer decode launch)
// and each SIMD ran its last microseconds with one wavefront.  The weights
// follow the measured rates (1 / duration).
constexpr int kWaveWeight[4] = {19, 17, 15, 13};  // sum 64: 256 over 16 wavefronts
__host__ __device__ inline int64_t wave_split(int64_t n, int w) {
  int64_t c = 0;
  for (int g = 0; g < 4; ++g) {
    const int in = w - 4 * g;
    c += (int64_t)kWaveWeight[g] * (in < 0 ? 0 : (in > 4 ? 4 : in));
  }
  return n * c / 256;  // first step of wavefront w, of n; wave_split(n, 16) == n
}
// workgroup owning global step s when T steps are cut into NB equal ranges
// [T*b/NB, T*(b+1)/NB)
__host__ __device__ inline int64_t block_of_step(int64_t s, int64_t T, int64_t NB) {
  return ((s + 1) * NB - 1) / T;
}
// single-call workspace: partial sums [strips][tokens][64] int32, tickets [strips]
inline size_t decode_partial_bytes(int64_t tokens, int64_t n_out) {
  const int64_t strips = (n_out + 63) / 64;
  return (size_t)strips * (size_t)tokens * 64 * 4;
}
inline size_t decode_ws_bytes(int64_t tokens, int64_t n_out) {
  const int64_t strips = (n_out + 63) / 64;
  return ((decode_partial_bytes(tokens, n_out) + 255) & ~(size_t)255) + (size_t)strips * 4;
}
// Y (binary32) or Yb (the same values rounded to bf16, ties to even): one of
// the two is given, the other is null (as in the prefill launchers).
hipError_t launch_gemv(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, uint16_t* Yb, int32_t* acc, void* ws,
                       int tokens, int64_t k, int64_t n_out, int S, hipStream_t s);

// Grouped decode: one plan in device memory describes many GEMVs that share
// the token count and N:M pattern; kernels read it, so a run needs only the
// plan pointer.  The plan hands every workgroup a list of whole strips
// (packed on the host for equal step counts), so no strip is cut between
// workgroups.  Each strip of the list is a self-contained descriptor, and
// each wavefront's start record carries its first one, so a wavefront
// starts streaming after a single scalar load.
struct GroupHeader {
  int32_t count, tokens, S, blocks;
  int64_t rows;    // activation rows = count * tokens
  int64_t steps;   // superblocks over all items
  int64_t strips;  // strip descriptors
  int32_t fused;   // 1: the contraction can quantise its own activations
  int32_t pad;
};
struct GroupItem {
  const uint16_t* X;
  const uint32_t* packed;
  const double* gamma;
  float* Y;
  int8_t* xq;
  float* scale;
  int64_t k, n_out;
};
struct StripDesc {            // one 64-row strip of one item (64 bytes)
  const char* packed;         // the strip's first superblock
  const int8_t* xq;           // the item's int8 activations [tokens][k]
  float* Y;                   // the item's outputs [tokens][n_out]
  const float* scale;         // the item's token scales
  const double* gamma;        // the item's weight scale
  int64_t n_out;
  int32_t k;
  int32_t row0;               // first row of the strip
  int32_t pad[2];
};
static_assert(sizeof(StripDesc) == 64, "strip descriptor size");
struct WaveStart {            // a wavefront's range (80 bytes)
  StripDesc first;            // its first strip
  int32_t rec, kb;            // that strip's list index and the first k block
  int32_t count;              // steps of the range (0: idle wavefront)
  int32_t active;             // the workgroup has work
};
static_assert(sizeof(WaveStart) == 80, "wave start size");
static_assert(offsetof(WaveStart, rec) == 64, "rec, kb, count, active: one 16-byte load");
// Fused runs (activation quantisation inside the contraction launch): each
// workgroup quantises the activation rows of the items its strips belong
// to into its LDS, after the code tables, and reads its B operands and
// token scales from there.  The rows are cut into segments of at most
// kFusedSegVals values, dealt round-robin to the workgroup's 16 wavefronts
// (at most kFusedSegsPerWave each, read with the wavefront's start record).
// A wavefront loads its segments once, before its first weight loads,
// publishes each segment's absmax in LDS, and after a barrier quantises
// from registers with the row's absmax (the maximum over the row's
// segments).  Each item's x_q and x_scale are written to memory by one
// workgroup (its writer).  A strip descriptor's pad[0] and pad[1] hold the
// LDS byte offsets of its item's codes and scales.
constexpr int kFusedSegVals = 1024;     // values per segment (two 16-byte loads per lane)
constexpr int kFusedSegsPerWave = 4;
constexpr int kFusedSegsPerBlock = kFusedSegsPerWave * kDecodeWavesPerBlock;
struct FusedSeg {          // one segment of one activation row (48 bytes)
  const uint16_t* x;       // bf16, the segment's first value
  int8_t* xq;              // x_q at the same place, or null (not the writer)
  float* scale;            // the row's x_scale, or null (not the row's first
                           // segment, or not the writer)
  uint32_t lds_q;          // LDS byte offset of the segment's codes
  uint32_t lds_s;          // LDS byte offset of the row's token scale
  int32_t nvals;           // values (a multiple of 8); 0: no segment
  int16_t slot;            // this segment's absmax slot in the workgroup
  int16_t row_slot;        // first slot of the row
  int16_t row_slots;       // slots of the row
  int16_t first;           // 1: the segment that stores the row's scale
  int32_t pad;
};
static_assert(sizeof(FusedSeg) == 48, "fused segment record");
constexpr int kDecodeLutBytes = 512 * 4 * kDecodeLutCopies;
constexpr int64_t kFusedLdsBytes = 160 * 1024 - kDecodeLutBytes;  // after the tables
constexpr int64_t kFusedMaxBytes = 4 * kFusedSegsPerBlock;           // segment maxima, at the end
constexpr int64_t kFusedCodeBytes = kFusedLdsBytes - kFusedMaxBytes;   // codes and scales
// one activation row of the plan (self-contained: one 32-byte load)
struct RowDesc {
  const uint16_t* X;  // bf16 [k]
  int8_t* xq;         // int8 [k]
  float* scale;       // one float
  int64_t k;
};
static_assert(sizeof(RowDesc) == 32, "row descriptor size");
// plan image: header (64 bytes) | wave starts[kDecodeBlocks * 16] |
//             fused segments[kDecodeBlocks * 16 * kFusedSegsPerWave] |
//             row descriptors[rows] | strip descriptors | items[count]
// (the row descriptors sit at a fixed offset, so the activation kernel
// reads its row without waiting for the header; the region holds at least
// one descriptor per activation workgroup, zero-padded)
constexpr size_t kGroupHeaderBytes = 64;
constexpr int kActGroupBlocks = 1024;  // activation workgroups of a grouped run
static_assert(sizeof(GroupHeader) <= kGroupHeaderBytes, "plan header size");
__host__ __device__ inline size_t group_waves_offset() { return kGroupHeaderBytes; }
__host__ __device__ inline size_t group_fused_offset() {
  return kGroupHeaderBytes + (size_t)kDecodeBlocks * kDecodeWavesPerBlock * sizeof(WaveStart);
}
__host__ __device__ inline size_t group_rows_offset() {
  return group_fused_offset() + (size_t)kDecodeBlocks * kFusedSegsPerBlock * sizeof(FusedSeg);
}
__host__ __device__ inline size_t group_strips_offset(int64_t rows) {
  return group_rows_offset() + (size_t)(rows > kActGroupBlocks ? rows : kActGroupBlocks) * sizeof(RowDesc);
}
__host__ __device__ inline size_t group_items_offset(int64_t rows, int64_t strips) {
  return group_strips_offset(rows) + (size_t)strips * sizeof(StripDesc);
}
inline size_t group_plan_bytes(int64_t strips, int64_t count, int64_t rows) {
  return group_items_offset(rows, strips) + (size_t)count * sizeof(GroupItem);
}
hipError_t launch_act_quant_group(const void* plan, hipStream_t s);
// fused: the contraction quantises its activations itself (one launch for
// both stages); a plan that does not fuse then gets NaN outputs
hipError_t launch_gemv_group(const void* plan, int S, bool fused, hipStream_t s);

// Prefill-shaped contraction (any token count).  Tiles are 256 rows x 64
// tokens; when there are too few tiles to give every CU three workgroups,
// the k blocks are split into gemm_splits() contiguous parts, one
// workgroup each.  Parts write exact int32 partial tiles to the workspace
// and take a ticket per (tile, wavefront); the last part adds the others
// and writes Y, then returns the ticket to zero.  Workspace: tickets
// (zero on entry, left zero), then the partial tiles.
constexpr int kGemmTileRows = 256, kGemmTileTokens = 64;
inline int64_t gemm_tiles(int64_t tokens, int64_t n_out) {
  return ((n_out + kGemmTileRows - 1) / kGemmTileRows) *
         ((tokens + kGemmTileTokens - 1) / kGemmTileTokens);
}
inline int gemm_splits(int64_t tokens, int64_t k, int64_t n_out) {
  const int64_t tiles = gemm_tiles(tokens, n_out), nkb = k / 128;
  // Every extra part adds a full int32 copy of the layer's output to write
  // and read back through memory; on MI355X that exchange cost more than
  // the parallelism it buys unless most CUs would otherwise idle (1536 x
  // 8960 at 2048 tokens, 192 tiles: 50.4 us unsplit, 50.7 us in 2 parts;
  // 2048 x 11008, 256 tiles: 62.9 vs 67.8 us).  So: two parts, and only
  // when the tiles would occupy at most half of the 256 CUs.
  if (tiles > 128 || nkb < 8) return 1;
  return 2;
}
inline size_t gemm_ticket_bytes(int64_t tokens, int64_t n_out) {
  return ((size_t)gemm_tiles(tokens, n_out) * 4 * 4 + 255) & ~(size_t)255;
}
inline size_t gemm_ws_bytes(int64_t tokens, int64_t k, int64_t n_out) {
  const int sp = gemm_splits(tokens, k, n_out);
  if (sp == 1) return 0;
  return gemm_ticket_bytes(tokens, n_out) +
         (size_t)gemm_tiles(tokens, n_out) * sp * kGemmTileRows * kGemmTileTokens * 4;
}
hipError_t launch_gemm(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, uint16_t* Yb, int32_t* acc, void* ws,
                       int64_t tokens, int64_t k, int64_t n_out, int S, hipStream_t s);

// Prefill-shaped contraction of 2:4 codes in the sparse-operand + index
// layout on the sparse int8 matrix instruction; same tiles, split-k and
// workspace as launch_gemm
hipError_t launch_gemm_sp24(const void* packed, const int8_t* xq, const float* scale,
                            const double* gamma, float* Y, int32_t* acc, void* ws, int64_t tokens,
                            int64_t k, int64_t n_out, hipStream_t s);

// Backward.  Workspace (bf16 operands of the two products, each region
// 256-byte aligned): (dY * s)^T [n_out x tp], x_q^T [k x tp] with tp the
// token count rounded up to 64, and codes^T [k x 64 * strips].
inline int64_t bwd_tokens_padded(int64_t tokens) { return (tokens + 63) / 64 * 64; }
inline size_t bwd_align(size_t b) { return (b + 255) & ~(size_t)255; }
inline size_t bwd_dys_offset(int64_t, int64_t, int64_t) { return 0; }
inline size_t bwd_xq_offset(int64_t tokens, int64_t, int64_t n_out) {
  return bwd_align((size_t)n_out * bwd_tokens_padded(tokens) * 2);
}
inline size_t bwd_codes_offset(int64_t tokens, int64_t k, int64_t n_out) {
  return bwd_xq_offset(tokens, k, n_out) + bwd_align((size_t)k * bwd_tokens_padded(tokens) * 2);
}
// A product C[M x N] (k depth K) with few 128 x 128 tiles (at most 128,
// half the CUs) and a deep k range is cut along k into `splits` ranges of
// bwd_split_len() (a multiple of 64): binary32 partial tiles in the
// workspace, summed in order by a second kernel.
inline int bwd_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (tiles > 128 || K < 2048) return 1;
  int64_t s = 512 / tiles;
  if (s > 8) s = 8;
  if (s > K / 512) s = K / 512;
  return s < 2 ? 1 : (int)s;
}
inline int64_t bwd_split_len(int64_t K, int splits) {
  return ((K + splits - 1) / splits + 63) / 64 * 64;
}
inline size_t bwd_partial_offset(int64_t tokens, int64_t k, int64_t n_out) {
  const int64_t np = (n_out + 63) / 64 * 64;
  return bwd_codes_offset(tokens, k, n_out) + bwd_align((size_t)k * np * 2);
}
inline size_t bwd_ws_bytes(int64_t tokens, int64_t k, int64_t n_out) {
  // dX: M = tokens, N = k, K = n_out; dW: M = n_out, N = k, K = tokens padded
  const int sx = bwd_splits(tokens, k, n_out), sw = bwd_splits(n_out, k, bwd_tokens_padded(tokens));
  const size_t px = sx > 1 ? (size_t)sx * tokens * k * 4 : 0;
  const size_t pw = sw > 1 ? (size_t)sw * n_out * k * 4 : 0;
  return bwd_partial_offset(tokens, k, n_out) + bwd_align(px > pw ? px : pw);
}
// dX (if non-null) and dW (if non-null) of one layer: operand preparation,
// then the products that are not split along k in one launch, then the
// split ones; tokens == 0 writes a zero dW
hipError_t launch_bwd(const uint16_t* dY, const int8_t* xq, const float* scale, const void* packed,
                      const double* gamma, float* dX, float* dW, void* ws, int64_t tokens, int64_t k,
                      int64_t n_out, int S, hipStream_t s);
// fixes the backward products' tiles (0: by tile count, 1: 128 x 128,
// 2: 256 x 128, 3: 256 x 256); -1 for another value
int bwd_set_tiles(int tiles);

}  // namespace bl

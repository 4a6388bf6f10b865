// launch.h -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/bitlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

constexpr size_t kGammaWsBytes = 4096;

// mask + exact absmean scale (two launches: workspace clear, mask/sum)
hipError_t launch_mask_gamma(const uint16_t* W, int64_t n_out, int64_t k, int n, int m,
                             int gamma_over, uint8_t* mask, double* gamma, void* ws,
                             hipStream_t s);

// ternary codes -> packed blocks (packed may be null) and/or int8 codes (wq
// may be null); S = sign slots per 8-group
hipError_t launch_ternary_pack(const uint16_t* W, const uint8_t* mask, const double* gamma,
                               int64_t n_out, int64_t k, int S, void* packed, int8_t* wq,
                               hipStream_t s);

// per-token int8 activations; also zero-fills zero_bytes of zero_ws
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
constexpr int kDecodeWavesPerBlock = 16;
constexpr int kMinStepsPerBlock = 16;  // at least ~1 step per wavefront
__host__ __device__ inline int64_t decode_blocks(int64_t steps) {
  int64_t nb = steps / kMinStepsPerBlock;
  return nb < 1 ? 1 : (nb > kDecodeBlocks ? kDecodeBlocks : nb);
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
hipError_t launch_gemv(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, int32_t* acc, void* ws, int tokens,
                       int64_t k, int64_t n_out, int S, hipStream_t s);

// Grouped decode: one plan in device memory describes many GEMVs that share
// the token count and N:M pattern; kernels read it, so a run needs only the
// plan pointer.  The plan hands every workgroup a list of whole strips
// (packed on the host for equal step counts), so no strip is cut between
// workgroups.
struct GroupHeader {
  int32_t count, tokens, S, blocks;
  int64_t rows;   // activation rows = count * tokens
  int64_t steps;  // superblocks over all items
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
struct StripRec {  // one strip of the list: (item, strip within the item)
  int32_t item, strip;
};
struct BlockRec {  // a workgroup's list: first strip record and step count
  int32_t first, steps;
};
struct WaveStart {  // a wavefront's first step: strip record and k block
  int32_t rec, kb;
};
// plan image: header | items[count] | row table[rows] | pad to 64 |
//             blocks[blocks] | wave starts[blocks * 16] | strip records
// row entry = item << 4 | token
__host__ __device__ inline size_t group_blocks_offset(int64_t count, int64_t rows) {
  size_t o = sizeof(GroupHeader) + (size_t)count * sizeof(GroupItem) + (size_t)rows * 4;
  return (o + 63) & ~(size_t)63;
}
__host__ __device__ inline size_t group_waves_offset(int64_t count, int64_t rows, int64_t blocks) {
  return group_blocks_offset(count, rows) + (size_t)blocks * sizeof(BlockRec);
}
__host__ __device__ inline size_t group_recs_offset(int64_t count, int64_t rows, int64_t blocks) {
  return group_waves_offset(count, rows, blocks) +
         (size_t)blocks * kDecodeWavesPerBlock * sizeof(WaveStart);
}
hipError_t launch_act_quant_group(const void* plan, hipStream_t s);
hipError_t launch_gemv_group(const void* plan, int S, hipStream_t s);

// prefill-shaped contraction (any token count)
hipError_t launch_gemm(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, int32_t* acc, int64_t tokens, int64_t k,
                       int64_t n_out, int S, hipStream_t s);

// backward
hipError_t launch_bwd_dx(const uint16_t* dY, const void* packed, const double* gamma, float* dX,
                         int64_t tokens, int64_t k, int64_t n_out, int S, hipStream_t s);
hipError_t launch_bwd_dw(const uint16_t* dY, const int8_t* xq, const float* scale, float* dW,
                         int64_t tokens, int64_t k, int64_t n_out, hipStream_t s);

}  // namespace bl

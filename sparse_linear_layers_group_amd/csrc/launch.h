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

// decode-shaped contraction (tokens <= 16), workspace layout and size
struct GemvPlan {
  int ksplit;        // k ranges per 16-row tile
  int st_per_unit;   // 512-wide k super-tiles per range
  int64_t units;     // tiles * ksplit
  size_t ws_bytes;   // partial sums + tickets (0 when ksplit == 1)
};
GemvPlan plan_gemv(int64_t tokens, int64_t k, int64_t n_out);
size_t gemv_ws_bytes_max(int64_t tokens, int64_t k, int64_t n_out);
hipError_t launch_gemv(const void* packed, const int8_t* xq, const float* scale,
                       const double* gamma, float* Y, int32_t* acc, void* ws, int tokens,
                       int64_t k, int64_t n_out, int S, hipStream_t s);

// grouped decode: one plan in device memory describes many GEMVs that share
// the token count and N:M pattern; kernels read it, so a run needs only the
// plan pointer.
constexpr int kGroupBlocks = 256;   // one 1024-thread block per CU
constexpr int kGroupWaves = 16;     // wavefronts per block
struct GroupHeader {
  int32_t count, tokens, S, waves;  // waves = per-wavefront ranges stored
  int64_t rows;                     // activation rows = count * tokens
  int64_t units;                    // 16-row tiles over all items
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
// where wavefront w starts: its first unit (16-row tile) index, that
// unit's item and tile; it walks units [start[w].unit, start[w+1].unit)
struct WaveStart {
  int32_t unit, item, tile, pad;
};
// plan image: header | items[count] | row table[rows] | pad to 64 |
//             wave starts[waves + 1]
// row entry = item << 4 | token
__host__ __device__ inline size_t group_starts_offset(int64_t count, int64_t rows) {
  size_t o = sizeof(GroupHeader) + (size_t)count * sizeof(GroupItem) + (size_t)rows * 4;
  return (o + 63) & ~(size_t)63;
}
inline size_t group_plan_bytes(int64_t count, int64_t rows, int64_t units) {
  (void)units;
  return group_starts_offset(count, rows) + (size_t)(kGroupBlocks * kGroupWaves + 1) * sizeof(WaveStart);
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

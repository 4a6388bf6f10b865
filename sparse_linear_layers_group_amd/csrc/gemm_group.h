// gemm_group.h -- grouped prefill contraction: several layers that read the
// same activations in shared launches of the prefill kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

// one layer of a grouped prefill contraction (Y or Yb non-null; acc optional)
struct GemmGroupLayer {
  const void* packed;
  const double* gamma;
  float* Y;
  uint16_t* Yb;
  int32_t* acc;
  int64_t n_out;
};

// tokens > 16; every layer's tiles in launches of up to 8 layers, never
// split along k (results equal per-layer launch_gemm calls: the int32 sums
// are exact in any order)
hipError_t launch_gemm_group(const GemmGroupLayer* layers, int count, const int8_t* xq, const float* scale,
                             int64_t tokens, int64_t k, int S, hipStream_t s);

}  // namespace bl

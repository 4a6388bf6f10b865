// bwd_group.h -- the grouped backward launcher (several layers' dX and dW
// products in shared launches).
#pragma once

#include "launch.h"

namespace bl {

// one layer of a grouped backward (pointers as for bitlinear_bwd; a null
// dX or dW skips that product)
struct BwdItem {
  const uint16_t* dY;
  const int8_t* xq;
  const float* scale;
  const void* packed;
  const double* gamma;
  float* dX;
  float* dW;
  int64_t k, n_out;
};

// workspace of one item of a grouped backward: its prepared operands (the
// grouped products are never split along k, so no partial tiles)
inline size_t bwd_group_item_bytes(int64_t tokens, int64_t k, int64_t n_out) {
  return bwd_align(bwd_partial_offset(tokens, k, n_out));
}

// every item's operands prepared into its own workspace region (x_q^T once
// per distinct x_q and k), then all products in launches of up to 16,
// deepest contraction first; tokens > 0.  phase 1 runs only the
// conversions of packed codes and x_q, phase 2 the rest (on what phase 1
// left in ws), phase 3 both
hipError_t launch_bwd_group(const BwdItem* items, int count, int64_t tokens, int S, void* ws, int phase,
                            hipStream_t s);

// the down projection's backward with the gating backward fused into its
// dX epilogue (dG, dU bf16 [tokens x k]; dW optional); tokens > 0
hipError_t launch_bwd_gate(const uint16_t* dY, const int8_t* xq, const float* scale, const void* packed,
                           const double* gamma, const float* G, const float* U, uint16_t* dG, uint16_t* dU,
                           float* dW, void* ws, int64_t tokens, int64_t k, int64_t n_out, int S,
                           hipStream_t s);

}  // namespace bl

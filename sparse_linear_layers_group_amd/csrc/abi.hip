// abi.hip -- the C ABI declared in include/bitlinear.h: host-side argument
// validation, then kernel launches on the caller's stream.  No exception
// leaves this file; no device memory is allocated.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <utility>
#include <vector>

#include "bitlinear.h"
#include "common.h"
#include "bwd_group.h"
#include "gemm_group.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return BL_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kLimit = (int64_t)1 << 31;

int check_nm(int n, int m) {
  if (bl::s_of(n, m) < 0)
    return fail(BL_EUNSUPPORTED, "N:M pattern %d:%d unsupported (use 8:8, 6:8, 4:8, 3:8, 2:8 or 2:4)", n, m);
  return BL_OK;
}

int check_layer(int64_t n_out, int64_t k) {
  if (n_out < 1) return fail(BL_ESHAPE, "n_out must be >= 1 (got %lld)", (long long)n_out);
  if (k < 128 || k % 128 != 0)
    return fail(BL_ESHAPE, "k must be a positive multiple of 128 (got %lld)", (long long)k);
  if (n_out >= kLimit || k >= kLimit || n_out * k >= kLimit)
    return fail(BL_ESHAPE, "n_out*k must stay below 2^31");
  return BL_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(BL_EINVAL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(BL_EINVAL, "%s is not %zu-byte aligned", name, align);
  return BL_OK;
}

int check_opt_ptr(const void* p, size_t align, const char* name) {
  if (p && !aligned(p, align)) return fail(BL_EINVAL, "%s is not %zu-byte aligned", name, align);
  return BL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BL_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define TRY(expr)            \
  do {                       \
    int _st = (expr);        \
    if (_st != BL_OK) return _st; \
  } while (0)

}  // namespace

namespace {
// Shape checks for a grouped decode plan; returns the total number of steps
// (64 x 128 superblocks) and of 64-row strips over all items.
int group_shape(const bitlinear_fwd_item* items, int count, int64_t tokens, int64_t* steps,
                int64_t* strips) {
  if (!items) return fail(BL_EINVAL, "items is NULL");
  if (count < 1 || count > 65535) return fail(BL_ESHAPE, "count must be in 1..65535 (got %d)", count);
  if (tokens < 1 || tokens > 16) return fail(BL_ESHAPE, "grouped decode takes 1..16 tokens (got %lld)", (long long)tokens);
  int64_t t = 0, ns = 0;
  for (int i = 0; i < count; ++i) {
    const bitlinear_fwd_item& it = items[i];
    int st = check_layer(it.n_out, it.k);
    if (st != BL_OK) return fail(st, "item %d: %s", i, g_last_error.c_str());
    if (tokens * it.k >= kLimit || tokens * it.n_out >= kLimit)
      return fail(BL_ESHAPE, "item %d: tokens*k and tokens*n_out must stay below 2^31", i);
    const int64_t strips = (it.n_out + bl::kStripRows - 1) / bl::kStripRows;
    ns += strips;
    t += strips * (it.k / 128);
    if (t >= ((int64_t)1 << 31)) return fail(BL_ESHAPE, "too many 64x128 weight blocks in one plan");
  }
  *steps = t;
  *strips = ns;
  return BL_OK;
}

int64_t group_blocks(int64_t steps, int64_t strips) {
  const int64_t nb = bl::decode_blocks(steps);
  return nb < strips ? nb : strips;
}

// Shape checks for a grouped quantisation plan; returns the mask and pack
// workgroups over all items and the workspace bytes (one 256-byte aligned
// gamma region per item).
int quant_shape(const bitlinear_quant_item* items, int count, int64_t* mask_blocks,
                int64_t* pack_blocks, size_t* ws) {
  if (!items) return fail(BL_EINVAL, "items is NULL");
  if (count < 1 || count > 65535) return fail(BL_ESHAPE, "count must be in 1..65535 (got %d)", count);
  int64_t mb = 0, pb = 0;
  size_t w = 0;
  for (int i = 0; i < count; ++i) {
    const bitlinear_quant_item& it = items[i];
    int st = check_layer(it.n_out, it.k);
    if (st != BL_OK) return fail(st, "item %d: %s", i, g_last_error.c_str());
    mb += bl::mask_blocks(it.n_out, it.k);
    pb += bl::pack_blocks(it.n_out, it.k);
    w += bl::bwd_align(bl::gamma_ws_bytes(it.n_out, it.k));
    if (mb + pb >= ((int64_t)1 << 30)) return fail(BL_ESHAPE, "too many workgroups in one plan");
  }
  *mask_blocks = mb;
  *pack_blocks = pb;
  *ws = w;
  return BL_OK;
}
}  // namespace

// ---------------------------------------------------------------------
// Static scratch of bitlinear_fwd_noalloc: the forward's workspace (decode
// split-k partial sums and counters, prefill split-k tickets and partial
// tiles) in a file-scope device array, so that call allocates nothing.
// Host code never passes the array's name to a kernel or a copy (on the
// host it is only a stand-in symbol): the first call on each device
// resolves the array's address on that device with hipGetSymbolAddress and
// keeps it; every later call on that device uses the kept address.
// ---------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// the scratch array's address on the current device (resolved once per
// device); BL_OK or BL_EHIP
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(BL_EHIP, "device index %d out of range", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(BL_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BL_OK;
}
}  // namespace

extern "C" {

size_t bitlinear_packed_bytes(int64_t n_out, int64_t k, int n, int m) {
  const int S = bl::s_of(n, m);
  if (S < 0 || n_out < 1 || k < 128 || k % 128 != 0 || n_out >= kLimit || k >= kLimit ||
      n_out * k >= kLimit)
    return 0;
  const int64_t strips = (n_out + bl::kStripRows - 1) / bl::kStripRows;
  return (size_t)(strips * bl::kStripRows * (k / 128) * bl::block_bytes(S));
}

size_t bitlinear_workspace_bytes(int64_t n_out, int64_t k) {
  if (n_out < 1 || k < 1 || n_out >= kLimit || k >= kLimit || n_out * k >= kLimit) return 0;
  return bl::gamma_ws_bytes(n_out, k);
}

size_t bitlinear_fwd_workspace_bytes(int64_t tokens, int64_t k, int64_t n_out) {
  if (tokens < 1 || n_out < 1 || k < 128 || tokens >= kLimit || n_out >= kLimit) return 0;
  // prefill: split-k tickets and partial tiles when the layer has few tiles
  if (tokens > 16) return bl::gemm_ws_bytes(tokens, k, n_out);
  // one k block per strip: no strip is ever cut between wavefronts
  if (k / 128 == 1) return 0;
  return bl::decode_ws_bytes(tokens, n_out);
}

size_t bitlinear_bwd_workspace_bytes(int64_t tokens, int64_t k, int64_t n_out) {
  if (tokens < 0 || n_out < 1 || k < 128 || k % 128 != 0 || n_out % 16 != 0 ||
      tokens >= kLimit || n_out >= kLimit || k >= kLimit)
    return 0;
  return bl::bwd_ws_bytes(tokens, k, n_out);
}

int bitlinear_quantize_mask(const uint16_t* W, int64_t n_out, int64_t k, int n, int m,
                            int gamma_over, uint8_t* mask, int8_t* wq, double* gamma, void* ws,
                            size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  TRY(check_ptr(W, 16, "W"));
  TRY(check_ptr(mask, 16, "mask"));
  TRY(check_opt_ptr(wq, 16, "wq"));
  TRY(check_ptr(gamma, 8, "gamma"));
  if (gamma_over != BL_GAMMA_DENSE && gamma_over != BL_GAMMA_MASKED)
    return fail(BL_EINVAL, "gamma_over must be BL_GAMMA_DENSE or BL_GAMMA_MASKED (got %d)", gamma_over);
  const size_t need = bl::gamma_ws_bytes(n_out, k);
  if (!ws || ws_bytes < need)
    return fail(BL_EWORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  TRY(check_ptr(ws, 16, "ws"));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = bl::launch_mask_gamma(W, n_out, k, n, m, gamma_over, mask, gamma, ws, s);
  if (e != hipSuccess) return hip_status(e, "mask/gamma launch");
  if (wq) {
    e = bl::launch_ternary_pack(W, mask, gamma, n_out, k, bl::s_of(n, m), nullptr, wq, s);
    if (e != hipSuccess) return hip_status(e, "ternary launch");
  }
  return ok();
}

int bitlinear_pack(const uint16_t* W, const uint8_t* mask, const double* gamma, int64_t n_out,
                   int64_t k, int n, int m, void* packed, size_t packed_bytes, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  TRY(check_ptr(W, 16, "W"));
  TRY(check_ptr(mask, 16, "mask"));
  TRY(check_ptr(gamma, 8, "gamma"));
  TRY(check_ptr(packed, 16, "packed"));
  const size_t need = bitlinear_packed_bytes(n_out, k, n, m);
  if (packed_bytes != need)
    return fail(BL_ESHAPE, "packed_bytes must be %zu for this layer (got %zu)", need, packed_bytes);
  hipError_t e = bl::launch_ternary_pack(W, mask, gamma, n_out, k, bl::s_of(n, m), packed, nullptr,
                                         reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "pack launch");
}

namespace {
// the forward with binary32 (Y) or bf16 (Yb) outputs: exactly one is given
int fwd_impl(const uint16_t* X, int64_t tokens, int64_t k, const void* packed, int64_t n_out,
             int n, int m, const double* gamma, float* Y, uint16_t* Yb, int8_t* xq, float* x_scale,
             int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  if (tokens < 0) return fail(BL_ESHAPE, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (tokens >= kLimit || tokens * k >= kLimit || tokens * n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens*k and tokens*n_out must stay below 2^31");
  if (tokens == 0) return ok();
  TRY(check_ptr(X, 16, "X"));
  TRY(check_ptr(packed, 16, "packed"));
  TRY(check_ptr(gamma, 8, "gamma"));
  if (Yb) TRY(check_ptr(Yb, 16, "Y"));
  else TRY(check_ptr(Y, 16, "Y"));
  TRY(check_ptr(xq, 16, "xq"));
  TRY(check_ptr(x_scale, 4, "x_scale"));
  TRY(check_opt_ptr(acc, 16, "acc"));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int S = bl::s_of(n, m);
  if (tokens <= 16) {
    const size_t need = bitlinear_fwd_workspace_bytes(tokens, k, n_out);
    if (need && (!ws || ws_bytes < need))
      return fail(BL_EWORKSPACE, "decode workspace needs %zu bytes (got %zu)", need,
                  ws ? ws_bytes : (size_t)0);
    if (need) TRY(check_ptr(ws, 16, "ws"));
    hipError_t e = bl::launch_act_quant(X, tokens, k, xq, x_scale, need ? ws : nullptr,
                                        (int64_t)need, s);
    if (e != hipSuccess) return hip_status(e, "activation quant launch");
    e = bl::launch_gemv(packed, xq, x_scale, gamma, Y, Yb, acc, ws, (int)tokens, k, n_out, S, s);
    return hip_status(e, "decode launch");
  }
  const size_t need = bitlinear_fwd_workspace_bytes(tokens, k, n_out);
  if (need && (!ws || ws_bytes < need))
    return fail(BL_EWORKSPACE, "prefill workspace needs %zu bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  if (need) TRY(check_ptr(ws, 16, "ws"));
  // the tickets start at zero (the partial tiles need no clearing)
  hipError_t e = bl::launch_act_quant(X, tokens, k, xq, x_scale, need ? ws : nullptr,
                                      need ? (int64_t)bl::gemm_ticket_bytes(tokens, n_out) : 0, s);
  if (e != hipSuccess) return hip_status(e, "activation quant launch");
  e = bl::launch_gemm(packed, xq, x_scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, S, s);
  return hip_status(e, "prefill launch");
}
}  // namespace

int bitlinear_fwd(const uint16_t* X, int64_t tokens, int64_t k, const void* packed, int64_t n_out,
                  int n, int m, const double* gamma, float* Y, int8_t* xq, float* x_scale,
                  int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  return fwd_impl(X, tokens, k, packed, n_out, n, m, gamma, Y, nullptr, xq, x_scale, acc, ws, ws_bytes,
                  stream);
}

int bitlinear_fwd_bf16(const uint16_t* X, int64_t tokens, int64_t k, const void* packed,
                       int64_t n_out, int n, int m, const double* gamma, uint16_t* Y, int8_t* xq,
                       float* x_scale, int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  if (!Y) return fail(BL_EINVAL, "Y is NULL");
  return fwd_impl(X, tokens, k, packed, n_out, n, m, gamma, nullptr, Y, xq, x_scale, acc, ws, ws_bytes,
                  stream);
}

int bitlinear_fwd_noalloc(const uint16_t* X, int64_t tokens, int64_t k, const void* packed,
                          int64_t n_out, int n, int m, const double* gamma, float* Y, int8_t* xq,
                          float* x_scale, int32_t* acc, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  if (tokens < 0) return fail(BL_ESHAPE, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (tokens >= kLimit || tokens * k >= kLimit || tokens * n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens*k and tokens*n_out must stay below 2^31");
  if (tokens == 0) return ok();
  const size_t need = bitlinear_fwd_workspace_bytes(tokens, k, n_out);
  if (need > kNoAllocScratchBytes)
    return fail(BL_EWORKSPACE,
                "this forward needs %zu bytes of workspace; the static scratch holds %zu "
                "(use bitlinear_fwd with a caller workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need) TRY(scratch_address(&ws));
  // the same kernels as bitlinear_fwd, which clears the counters it needs
  // inside its activation kernel (no memset node)
  return bitlinear_fwd(X, tokens, k, packed, n_out, n, m, gamma, Y, xq, x_scale, acc, ws,
                       need ? kNoAllocScratchBytes : 0, stream);
}

size_t bitlinear_sp24_packed_bytes(int64_t n_out, int64_t k) {
  if (n_out < 1 || k < 128 || k % 128 != 0 || n_out >= kLimit || k >= kLimit || n_out * k >= kLimit)
    return 0;
  return bl::sp24_packed_bytes(n_out, k);
}

size_t bitlinear_sp24_workspace_bytes(int64_t tokens, int64_t k, int64_t n_out) {
  if (tokens < 1 || n_out < 1 || k < 128 || tokens >= kLimit || n_out >= kLimit) return 0;
  return bl::gemm_ws_bytes(tokens, k, n_out);
}

int bitlinear_pack_sp24(const uint16_t* W, const uint8_t* mask, const double* gamma, int64_t n_out,
                        int64_t k, void* packed, size_t packed_bytes, void* stream) {
  TRY(check_layer(n_out, k));
  TRY(check_ptr(W, 16, "W"));
  TRY(check_ptr(mask, 16, "mask"));
  TRY(check_ptr(gamma, 8, "gamma"));
  TRY(check_ptr(packed, 16, "packed"));
  const size_t need = bl::sp24_packed_bytes(n_out, k);
  if (packed_bytes != need)
    return fail(BL_ESHAPE, "packed_bytes must be %zu for this layer (got %zu)", need, packed_bytes);
  hipError_t e = bl::launch_pack_sp24(W, mask, gamma, n_out, k, packed,
                                      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "sparse-operand pack launch");
}

int bitlinear_contract_sp24(const int8_t* xq, const float* x_scale, int64_t tokens, int64_t k,
                            const void* packed, int64_t n_out, const double* gamma, float* Y,
                            int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_layer(n_out, k));
  if (tokens < 0 || tokens >= kLimit || tokens * k >= kLimit || tokens * n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens must be >= 0 with tokens*k and tokens*n_out below 2^31");
  if (tokens == 0) return ok();
  TRY(check_ptr(xq, 16, "xq"));
  TRY(check_ptr(x_scale, 4, "x_scale"));
  TRY(check_ptr(packed, 16, "packed"));
  TRY(check_ptr(gamma, 8, "gamma"));
  TRY(check_ptr(Y, 16, "Y"));
  TRY(check_opt_ptr(acc, 16, "acc"));
  const size_t need = bl::gemm_ws_bytes(tokens, k, n_out);
  if (need && (!ws || ws_bytes < need))
    return fail(BL_EWORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : (size_t)0);
  if (need) TRY(check_ptr(ws, 16, "ws"));
  hipError_t e = bl::launch_gemm_sp24(packed, xq, x_scale, gamma, Y, acc, ws, tokens, k, n_out,
                                      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "sparse contraction launch");
}

int bitlinear_act_quant(const uint16_t* X, int64_t tokens, int64_t k, int8_t* xq, float* x_scale,
                        void* stream) {
  if (k < 128 || k % 128 != 0)
    return fail(BL_ESHAPE, "k must be a positive multiple of 128 (got %lld)", (long long)k);
  if (tokens < 0 || tokens >= kLimit || tokens * k >= kLimit)
    return fail(BL_ESHAPE, "tokens must be >= 0 with tokens*k below 2^31");
  if (tokens == 0) return ok();
  TRY(check_ptr(X, 16, "X"));
  TRY(check_ptr(xq, 16, "xq"));
  TRY(check_ptr(x_scale, 4, "x_scale"));
  hipError_t e = bl::launch_act_quant(X, tokens, k, xq, x_scale, nullptr, 0,
                                      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "activation quant launch");
}

int bitlinear_relu2_gate(const float* G, const float* U, int64_t tokens, int64_t n, uint16_t* H,
                         int8_t* xq, float* x_scale, void* stream) {
  if (n < 128 || n % 128 != 0)
    return fail(BL_ESHAPE, "n must be a positive multiple of 128 (got %lld)", (long long)n);
  if (tokens < 0 || tokens >= kLimit || tokens * n >= kLimit)
    return fail(BL_ESHAPE, "tokens must be >= 0 with tokens*n below 2^31");
  if (tokens == 0) return ok();
  TRY(check_ptr(G, 16, "G"));
  TRY(check_ptr(U, 16, "U"));
  if (H) TRY(check_ptr(H, 16, "H"));
  TRY(check_ptr(xq, 16, "xq"));
  TRY(check_ptr(x_scale, 4, "x_scale"));
  hipError_t e = bl::launch_relu2_gate(G, U, tokens, n, H, xq, x_scale, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "gating launch");
}

int bitlinear_relu2_gate_bwd(const float* dH, const float* G, const float* U, int64_t count,
                             uint16_t* dG, uint16_t* dU, void* stream) {
  if (count < 0 || count >= kLimit || count % 8 != 0)
    return fail(BL_ESHAPE, "count must be a multiple of 8 in [0, 2^31) (got %lld)", (long long)count);
  if (count == 0) return ok();
  TRY(check_ptr(dH, 16, "dH"));
  TRY(check_ptr(G, 16, "G"));
  TRY(check_ptr(U, 16, "U"));
  TRY(check_ptr(dG, 16, "dG"));
  TRY(check_ptr(dU, 16, "dU"));
  hipError_t e = bl::launch_relu2_gate_bwd(dH, G, U, count, dG, dU, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "gating backward launch");
}

int bitlinear_latent_update(float* W_master, const float* dW, int64_t count, float lr, uint16_t* W,
                            void* stream) {
  if (count < 0 || count >= kLimit || count % 8 != 0)
    return fail(BL_ESHAPE, "count must be a multiple of 8 in [0, 2^31) (got %lld)", (long long)count);
  if (count == 0) return ok();
  TRY(check_ptr(W_master, 16, "W_master"));
  TRY(check_ptr(dW, 16, "dW"));
  TRY(check_ptr(W, 16, "W"));
  hipError_t e = bl::launch_latent_update(W_master, dW, count, lr, W, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "latent update launch");
}

namespace {
int contract_impl(const int8_t* xq, const float* x_scale, int64_t tokens, int64_t k,
                  const void* packed, int64_t n_out, int n, int m, const double* gamma, float* Y,
                  uint16_t* Yb, int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  if (tokens < 0 || tokens >= kLimit || tokens * k >= kLimit || tokens * n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens must be >= 0 with tokens*k and tokens*n_out below 2^31");
  if (tokens == 0) return ok();
  TRY(check_ptr(xq, 16, "xq"));
  TRY(check_ptr(x_scale, 4, "x_scale"));
  TRY(check_ptr(packed, 16, "packed"));
  TRY(check_ptr(gamma, 8, "gamma"));
  if (Yb) TRY(check_ptr(Yb, 16, "Y"));
  else TRY(check_ptr(Y, 16, "Y"));
  TRY(check_opt_ptr(acc, 16, "acc"));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int S = bl::s_of(n, m);
  const size_t need = bitlinear_fwd_workspace_bytes(tokens, k, n_out);
  if (need && (!ws || ws_bytes < need))
    return fail(BL_EWORKSPACE, "%s workspace needs %zu bytes (got %zu)",
                tokens <= 16 ? "decode" : "prefill", need, ws ? ws_bytes : (size_t)0);
  if (need) TRY(check_ptr(ws, 16, "ws"));
  hipError_t e;
  if (tokens <= 16)
    e = bl::launch_gemv(packed, xq, x_scale, gamma, Y, Yb, acc, ws, (int)tokens, k, n_out, S, s);
  else
    e = bl::launch_gemm(packed, xq, x_scale, gamma, Y, Yb, acc, ws, tokens, k, n_out, S, s);
  return hip_status(e, "contraction launch");
}
}  // namespace

int bitlinear_contract(const int8_t* xq, const float* x_scale, int64_t tokens, int64_t k,
                       const void* packed, int64_t n_out, int n, int m, const double* gamma,
                       float* Y, int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  return contract_impl(xq, x_scale, tokens, k, packed, n_out, n, m, gamma, Y, nullptr, acc, ws, ws_bytes,
                       stream);
}

int bitlinear_contract_bf16(const int8_t* xq, const float* x_scale, int64_t tokens, int64_t k,
                            const void* packed, int64_t n_out, int n, int m, const double* gamma,
                            uint16_t* Y, int32_t* acc, void* ws, size_t ws_bytes, void* stream) {
  if (!Y) return fail(BL_EINVAL, "Y is NULL");
  return contract_impl(xq, x_scale, tokens, k, packed, n_out, n, m, gamma, nullptr, Y, acc, ws,
                       ws_bytes, stream);
}


size_t bitlinear_contract_group_workspace_bytes(const bitlinear_contract_item* items, int count,
                                                int64_t tokens, int64_t k) {
  if (!items || count < 1 || tokens < 0 || tokens >= kLimit || k < 128 || k % 128 != 0 || k >= kLimit) return 0;
  size_t need = 0;
  for (int i = 0; i < count; ++i) {
    if (items[i].n_out < 1 || items[i].n_out >= kLimit) return 0;
    if (tokens <= 16) need = std::max(need, bitlinear_fwd_workspace_bytes(tokens, k, items[i].n_out));
  }
  return need;
}

int bitlinear_contract_group(const bitlinear_contract_item* items, int count, const int8_t* xq,
                             const float* x_scale, int64_t tokens, int64_t k, int n, int m, void* ws,
                             size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  if (!items) return fail(BL_EINVAL, "items is NULL");
  if (count < 1) return fail(BL_ESHAPE, "count must be >= 1 (got %d)", count);
  for (int i = 0; i < count; ++i) {
    const bitlinear_contract_item& it = items[i];
    int st = check_layer(it.n_out, k);
    if (st == BL_OK && (tokens < 0 || tokens >= kLimit || tokens * k >= kLimit || tokens * it.n_out >= kLimit))
      st = fail(BL_ESHAPE, "tokens must be >= 0 with tokens*k and tokens*n_out below 2^31");
    if (st == BL_OK && (it.Y != nullptr) == (it.Y_bf16 != nullptr))
      st = fail(BL_EINVAL, "exactly one of Y and Y_bf16 must be given");
    if (st == BL_OK && tokens > 0) {
      st = check_ptr(it.packed, 16, "packed");
      if (st == BL_OK) st = check_ptr(it.gamma, 8, "gamma");
      if (st == BL_OK) st = it.Y ? check_ptr(it.Y, 16, "Y") : check_ptr(it.Y_bf16, 16, "Y_bf16");
    }
    if (st != BL_OK) {
      std::string detail = bitlinear_last_error();
      return fail(st, "item %d: %s", i, detail.c_str());
    }
  }
  if (tokens == 0) return ok();
  TRY(check_ptr(xq, 16, "xq"));
  TRY(check_ptr(x_scale, 4, "x_scale"));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int S = bl::s_of(n, m);
  if (tokens <= 16) {  // decode-shaped: each item in turn on the one workspace
    const size_t need = bitlinear_contract_group_workspace_bytes(items, count, tokens, k);
    if (need && (!ws || ws_bytes < need))
      return fail(BL_EWORKSPACE, "decode workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : (size_t)0);
    if (need) TRY(check_ptr(ws, 16, "ws"));
    for (int i = 0; i < count; ++i) {
      const bitlinear_contract_item& it = items[i];
      hipError_t e = bl::launch_gemv(it.packed, xq, x_scale, it.gamma, it.Y, it.Y_bf16, nullptr, ws, (int)tokens,
                                     k, it.n_out, S, s);
      if (e != hipSuccess) return hip_status(e, "contraction launch");
    }
    return ok();
  }
  std::vector<bl::GemmGroupLayer> layers;
  for (int i = 0; i < count; ++i)
    layers.push_back(bl::GemmGroupLayer{items[i].packed, items[i].gamma, items[i].Y, items[i].Y_bf16, nullptr,
                                        items[i].n_out});
  hipError_t e = bl::launch_gemm_group(layers.data(), count, xq, x_scale, tokens, k, S, s);
  return hip_status(e, "grouped contraction launch");
}

size_t bitlinear_fwd_group_plan_bytes(const bitlinear_fwd_item* items, int count, int64_t tokens) {
  int64_t steps = 0, strips = 0;
  if (group_shape(items, count, tokens, &steps, &strips) != BL_OK) return 0;
  return bl::group_plan_bytes(strips, count, count * tokens);
}

namespace {
// The plan image in host memory; uploading it is the only later step.
int fwd_group_image(const bitlinear_fwd_item* items, int count, int64_t tokens, int n, int m,
                    void* plan, size_t plan_bytes, std::vector<char>& img) {
  TRY(check_nm(n, m));
  int64_t steps = 0, nstrips = 0;
  TRY(group_shape(items, count, tokens, &steps, &nstrips));
  for (int i = 0; i < count; ++i) {
    const bitlinear_fwd_item& it = items[i];
    TRY(check_ptr(it.X, 16, "item X"));
    TRY(check_ptr(it.packed, 16, "item packed"));
    TRY(check_ptr(it.gamma, 8, "item gamma"));
    TRY(check_ptr(it.Y, 16, "item Y"));
    TRY(check_ptr(it.xq, 16, "item xq"));
    TRY(check_ptr(it.x_scale, 4, "item x_scale"));
  }
  const int64_t nb = group_blocks(steps, nstrips);
  const size_t need = bl::group_plan_bytes(nstrips, count, count * tokens);
  TRY(check_ptr(plan, 16, "plan"));
  if (plan_bytes < need) return fail(BL_EWORKSPACE, "plan needs %zu bytes (got %zu)", need, plan_bytes);
  const int S = bl::s_of(n, m);
  img.assign(need, 0);
  bl::GroupHeader* h = reinterpret_cast<bl::GroupHeader*>(img.data());
  h->count = count;
  h->tokens = (int32_t)tokens;
  h->S = S;
  h->blocks = (int32_t)nb;
  h->rows = count * tokens;
  h->steps = steps;
  h->strips = nstrips;
  bl::GroupItem* gi = reinterpret_cast<bl::GroupItem*>(img.data() + bl::group_items_offset(count * tokens, nstrips));
  bl::RowDesc* rows = reinterpret_cast<bl::RowDesc*>(img.data() + bl::group_rows_offset());
  int64_t r = 0;
  // every strip of every item: its descriptor and step count
  std::vector<bl::StripDesc> all;
  std::vector<int32_t> nkb, item_of;
  all.reserve((size_t)nstrips);
  for (int i = 0; i < count; ++i) {
    const bitlinear_fwd_item& it = items[i];
    gi[i] = bl::GroupItem{it.X, reinterpret_cast<const uint32_t*>(it.packed), it.gamma, it.Y,
                          it.xq, it.x_scale, it.k, it.n_out};
    for (int64_t t = 0; t < tokens; ++t)
      rows[r++] = bl::RowDesc{it.X + t * it.k, it.xq + t * it.k, it.x_scale + t, it.k};
    const int64_t strips = (it.n_out + bl::kStripRows - 1) / bl::kStripRows;
    const int64_t strip_bytes = (it.k / 128) * bl::kStripRows * bl::block_bytes(S);
    for (int64_t st = 0; st < strips; ++st) {
      all.push_back(bl::StripDesc{reinterpret_cast<const char*>(it.packed) + st * strip_bytes,
                                  it.xq, it.Y, it.x_scale, it.gamma, it.n_out, (int32_t)it.k,
                                  (int32_t)(st * bl::kStripRows)});
      nkb.push_back((int32_t)(it.k / 128));
      item_of.push_back(i);
    }
  }
  // whole strips to workgroups, longest first onto the least loaded (LPT);
  // each workgroup's list in (item, strip) order
  std::vector<int32_t> order(all.size());
  for (size_t j = 0; j < order.size(); ++j) order[j] = (int32_t)j;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return nkb[a] > nkb[b]; });
  typedef std::pair<int64_t, int32_t> Load;  // (steps so far, workgroup)
  std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
  for (int32_t b = 0; b < (int32_t)nb; ++b) heap.push(Load(0, b));
  std::vector<std::vector<int32_t>> lists((size_t)nb);
  for (int32_t j : order) {
    Load l = heap.top();
    heap.pop();
    lists[(size_t)l.second].push_back(j);
    l.first += nkb[j];
    heap.push(l);
  }
  bl::WaveStart* wst = reinterpret_cast<bl::WaveStart*>(img.data() + bl::group_waves_offset());
  bl::StripDesc* descs = reinterpret_cast<bl::StripDesc*>(img.data() + bl::group_strips_offset(count * tokens));
  // fused runs: each workgroup's items (in order of first use) get LDS room
  // for their codes, then their scales, after the code tables; an item's
  // first workgroup writes its x_q and x_scale.  Every (item, token) row is
  // cut into segments of at most kFusedSegVals values, numbered in that
  // order and dealt round-robin to the 16 wavefronts.  The plan fuses when
  // every workgroup's room and segment count fit.
  bl::FusedSeg* fseg = reinterpret_cast<bl::FusedSeg*>(img.data() + bl::group_fused_offset());
  bool fused = true;
  std::vector<char> written((size_t)count, 0);
  for (int64_t b = 0; b < nb; ++b) {
    std::vector<int32_t>& lst = lists[(size_t)b];
    std::sort(lst.begin(), lst.end());  // (item, strip) order: an item's strips are adjacent
    std::vector<int32_t> its;
    for (int32_t j : lst)
      if (its.empty() || its.back() != item_of[j]) its.push_back(item_of[j]);
    std::vector<uint32_t> xo(its.size()), so(its.size());
    uint64_t off = 0;
    for (size_t q = 0; q < its.size(); ++q) {
      xo[q] = (uint32_t)off;
      off += ((uint64_t)tokens * (uint64_t)items[its[q]].k + 15) / 16 * 16;
    }
    for (size_t q = 0; q < its.size(); ++q) {
      so[q] = (uint32_t)off;
      off += ((uint64_t)tokens * 4 + 15) / 16 * 16;
    }
    if (off > (uint64_t)bl::kFusedCodeBytes) fused = false;
    int64_t g = 0;  // segments of the workgroup so far
    for (size_t q = 0; q < its.size(); ++q) {
      const bitlinear_fwd_item& it = items[its[q]];
      const bool writer = !written[(size_t)its[q]];
      written[(size_t)its[q]] = 1;
      const int64_t per_row = (it.k + bl::kFusedSegVals - 1) / bl::kFusedSegVals;
      for (int64_t t = 0; t < tokens; ++t) {
        const int64_t g_row = g;
        for (int64_t v0 = 0; v0 < it.k; v0 += bl::kFusedSegVals, ++g) {
          if (g >= bl::kFusedSegsPerBlock) {
            fused = false;
            continue;
          }
          bl::FusedSeg& f = fseg[(b * bl::kDecodeWavesPerBlock + g % bl::kDecodeWavesPerBlock) *
                                     bl::kFusedSegsPerWave +
                                 g / bl::kDecodeWavesPerBlock];
          const int64_t o = t * it.k + v0;
          f.x = it.X + o;
          f.xq = writer ? it.xq + o : nullptr;
          f.scale = writer && v0 == 0 ? it.x_scale + t : nullptr;
          f.lds_q = xo[q] + (uint32_t)o;
          f.lds_s = so[q] + 4 * (uint32_t)t;
          f.nvals = (int32_t)std::min<int64_t>(bl::kFusedSegVals, it.k - v0);
          f.slot = (int16_t)g;
          f.row_slot = (int16_t)g_row;
          f.row_slots = (int16_t)per_row;
          f.first = v0 == 0 ? 1 : 0;
        }
      }
    }
    size_t q = 0;
    for (int32_t j : lst) {
      while (its[q] != item_of[j]) ++q;
      all[j].pad[0] = (int32_t)xo[q];
      all[j].pad[1] = (int32_t)so[q];
    }
  }
  // a plan that does not fuse carries no segments (its fused runs write
  // NaN outputs and read nothing else)
  if (!fused)
    std::memset(fseg, 0, (size_t)nb * bl::kFusedSegsPerBlock * sizeof(bl::FusedSeg));
  h->fused = fused ? 1 : 0;
  int32_t next = 0;
  for (int64_t b = 0; b < nb; ++b) {
    std::vector<int32_t>& lst = lists[(size_t)b];
    std::sort(lst.begin(), lst.end());  // strip index order = (item, strip) order
    int64_t n_b = 0;
    for (int32_t j : lst) n_b += nkb[j];
    // wavefront w runs local steps [wave_split(n_b, w), wave_split(n_b, w + 1))
    size_t pos = 0;
    int64_t cum = 0;
    for (int w = 0; w < bl::kDecodeWavesPerBlock; ++w) {
      const int64_t s0 = bl::wave_split(n_b, w);
      const int64_t s1 = bl::wave_split(n_b, w + 1);
      while (pos + 1 < lst.size() && cum + nkb[lst[pos]] <= s0) cum += nkb[lst[pos++]];
      bl::WaveStart& ws = wst[b * bl::kDecodeWavesPerBlock + w];
      ws.active = n_b > 0 ? 1 : 0;
      ws.count = (int32_t)(s1 - s0);
      if (!lst.empty()) {
        ws.first = all[lst[pos]];
        ws.rec = next + (int32_t)pos;
        ws.kb = (int32_t)(s0 - cum);
      }
    }
    for (int32_t j : lst) descs[next++] = all[j];
  }
  return BL_OK;
}
}  // namespace

int bitlinear_fwd_group_plan(const bitlinear_fwd_item* items, int count, int64_t tokens, int n,
                             int m, void* plan, size_t plan_bytes, void* stream) {
  std::vector<char> img;
  TRY(fwd_group_image(items, count, tokens, n, m, plan, plan_bytes, img));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(plan, img.data(), img.size(), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, "plan upload");
}

int bitlinear_fwd_group_plan_host(const bitlinear_fwd_item* items, int count, int64_t tokens, int n,
                                  int m, void* image, size_t image_bytes) {
  std::vector<char> img;
  TRY(fwd_group_image(items, count, tokens, n, m, image, image_bytes, img));
  std::memcpy(image, img.data(), img.size());
  return ok();
}

int bitlinear_fwd_group_plan_fuses(const bitlinear_fwd_item* items, int count, int64_t tokens, int n,
                                   int m) {
  // errors come back negated (1 and 0 are answers)
  int64_t steps = 0, strips = 0;
  int st = group_shape(items, count, tokens, &steps, &strips);
  if (st != BL_OK) return -st;
  std::vector<char> img;
  st = fwd_group_image(items, count, tokens, n, m, reinterpret_cast<void*>(16),
                       bl::group_plan_bytes(strips, count, count * tokens), img);
  if (st != BL_OK) return -st;
  return reinterpret_cast<const bl::GroupHeader*>(img.data())->fused ? 1 : 0;
}

int bitlinear_fwd_group(const void* plan, int n, int m, int stages, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_ptr(plan, 16, "plan"));
  if (stages < 1 || stages > 4) return fail(BL_EINVAL, "stages must be 1, 2, 3 or 4 (got %d)", stages);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (stages == 4) {
    hipError_t e = bl::launch_gemv_group(plan, bl::s_of(n, m), true, s);
    return e != hipSuccess ? hip_status(e, "fused grouped decode launch") : ok();
  }
  if (stages & 1) {
    hipError_t e = bl::launch_act_quant_group(plan, s);
    if (e != hipSuccess) return hip_status(e, "grouped activation launch");
  }
  if (stages & 2) {
    hipError_t e = bl::launch_gemv_group(plan, bl::s_of(n, m), false, s);
    if (e != hipSuccess) return hip_status(e, "grouped decode launch");
  }
  return ok();
}

size_t bitlinear_quant_group_workspace_bytes(const bitlinear_quant_item* items, int count) {
  int64_t mb = 0, pb = 0;
  size_t w = 0;
  if (quant_shape(items, count, &mb, &pb, &w) != BL_OK) return 0;
  return w;
}

size_t bitlinear_quant_group_plan_bytes(const bitlinear_quant_item* items, int count) {
  int64_t mb = 0, pb = 0;
  size_t w = 0;
  if (quant_shape(items, count, &mb, &pb, &w) != BL_OK) return 0;
  return bl::quant_plan_bytes(count, mb, pb);
}

int bitlinear_quant_group_plan(const bitlinear_quant_item* items, int count, int n, int m,
                               int gamma_over, void* ws, size_t ws_bytes, void* plan,
                               size_t plan_bytes, void* stream) {
  TRY(check_nm(n, m));
  if (gamma_over != BL_GAMMA_DENSE && gamma_over != BL_GAMMA_MASKED)
    return fail(BL_EINVAL, "gamma_over must be BL_GAMMA_DENSE or BL_GAMMA_MASKED (got %d)", gamma_over);
  int64_t mb = 0, pb = 0;
  size_t need_ws = 0;
  TRY(quant_shape(items, count, &mb, &pb, &need_ws));
  for (int i = 0; i < count; ++i) {
    const bitlinear_quant_item& it = items[i];
    TRY(check_ptr(it.W, 16, "item W"));
    TRY(check_ptr(it.mask, 16, "item mask"));
    TRY(check_ptr(it.gamma, 8, "item gamma"));
    TRY(check_ptr(it.packed, 16, "item packed"));
  }
  if (!ws || ws_bytes < need_ws)
    return fail(BL_EWORKSPACE, "workspace needs %zu bytes (got %zu)", need_ws, ws ? ws_bytes : (size_t)0);
  TRY(check_ptr(ws, 16, "ws"));
  const size_t need = bl::quant_plan_bytes(count, mb, pb);
  TRY(check_ptr(plan, 16, "plan"));
  if (plan_bytes < need) return fail(BL_EWORKSPACE, "plan needs %zu bytes (got %zu)", need, plan_bytes);
  std::vector<char> img(need, 0);
  bl::QuantGroupHeader* h = reinterpret_cast<bl::QuantGroupHeader*>(img.data());
  h->count = count;
  h->mask_blocks = mb;
  h->pack_blocks = pb;
  h->n = n;
  h->m = m;
  h->gamma_over = gamma_over;
  bl::QuantItemDesc* d = reinterpret_cast<bl::QuantItemDesc*>(img.data() + sizeof(bl::QuantGroupHeader));
  int32_t* owner = reinterpret_cast<int32_t*>(img.data() + bl::quant_owner_offset(count));
  int64_t m0 = 0, p0 = 0;
  size_t w0 = 0;
  for (int i = 0; i < count; ++i) {
    const bitlinear_quant_item& it = items[i];
    bl::QuantItemDesc& q = d[i];
    q.W = it.W;
    q.mask = it.mask;
    q.gamma = it.gamma;
    q.packed = it.packed;
    q.ws = reinterpret_cast<char*>(ws) + w0;
    q.n_out = it.n_out;
    q.k = it.k;
    q.ngroups = it.n_out * it.k / 8;
    q.per = bl::mask_groups_per_block(it.n_out, it.k);
    q.mblock0 = m0;
    q.nmblocks = bl::mask_blocks(it.n_out, it.k);
    q.pblock0 = p0;
    for (int64_t b = 0; b < q.nmblocks; ++b) owner[m0 + b] = i;
    const int64_t npb = bl::pack_blocks(it.n_out, it.k);
    for (int64_t b = 0; b < npb; ++b) owner[mb + p0 + b] = i;
    m0 += q.nmblocks;
    p0 += npb;
    w0 += bl::bwd_align(bl::gamma_ws_bytes(it.n_out, it.k));
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(plan, img.data(), need, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return hip_status(e, "plan upload");
}

int bitlinear_quant_group(const void* plan, int n, int m, int gamma_over, void* stream) {
  TRY(check_nm(n, m));
  if (gamma_over != BL_GAMMA_DENSE && gamma_over != BL_GAMMA_MASKED)
    return fail(BL_EINVAL, "gamma_over must be BL_GAMMA_DENSE or BL_GAMMA_MASKED (got %d)", gamma_over);
  TRY(check_ptr(plan, 16, "plan"));
  hipError_t e = bl::launch_quant_group(plan, n, m, gamma_over, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "grouped quantisation launch");
}

namespace {
// bitlinear_bwd's validation of one item of a grouped backward (everything
// but the workspace)
int check_bwd_item(const bitlinear_bwd_item& it, int64_t tokens) {
  TRY(check_layer(it.n_out, it.k));
  if (it.n_out % 16 != 0)
    return fail(BL_ESHAPE, "the backward needs n_out to be a multiple of 16 (got %lld)", (long long)it.n_out);
  if (tokens >= kLimit || tokens * it.k >= kLimit || tokens * it.n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens*k and tokens*n_out must stay below 2^31");
  TRY(check_opt_ptr(it.dX, 16, "dX"));
  TRY(check_opt_ptr(it.dW, 16, "dW"));
  if (tokens == 0 || (!it.dX && !it.dW)) return BL_OK;
  const int64_t tp = bl::bwd_tokens_padded(tokens), np = (it.n_out + 63) / 64 * 64;
  if (tp * it.n_out >= kLimit / 2 || tp * it.k >= kLimit / 2 || it.k * np >= kLimit / 2)
    return fail(BL_ESHAPE, "the backward needs tokens*n_out, tokens*k and n_out*k below 2^30");
  TRY(check_ptr(it.dY, 16, "dY"));
  if (it.dX) {
    TRY(check_ptr(it.packed, 16, "packed"));
    TRY(check_ptr(it.gamma, 8, "gamma"));
  }
  if (it.dW) {
    TRY(check_ptr(it.xq, 16, "xq"));
    TRY(check_ptr(it.x_scale, 4, "x_scale"));
  }
  return BL_OK;
}
}  // namespace

size_t bitlinear_bwd_group_workspace_bytes(const bitlinear_bwd_item* items, int count, int64_t tokens) {
  if (!items || count < 1 || tokens < 0 || tokens >= kLimit) return 0;
  size_t total = 0;
  for (int i = 0; i < count; ++i) {
    const bitlinear_bwd_item& it = items[i];
    if (it.n_out < 1 || it.k < 128 || it.k % 128 != 0 || it.n_out % 16 != 0 || it.n_out >= kLimit ||
        it.k >= kLimit)
      return 0;
    total += bl::bwd_group_item_bytes(tokens, it.k, it.n_out);
  }
  return total;
}

static int bwd_group_run(const bitlinear_bwd_item* items, int count, int64_t tokens, int n, int m, int phase,
                         void* ws, size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  if (!items) return fail(BL_EINVAL, "items is NULL");
  if (count < 1) return fail(BL_ESHAPE, "count must be >= 1 (got %d)", count);
  if (tokens < 0) return fail(BL_ESHAPE, "tokens must be >= 0 (got %lld)", (long long)tokens);
  for (int i = 0; i < count; ++i) {
    const int st = check_bwd_item(items[i], tokens);
    if (st != BL_OK) {
      std::string detail = bitlinear_last_error();
      return fail(st, "item %d: %s", i, detail.c_str());
    }
  }
  bool any = false;
  for (int i = 0; i < count; ++i) any = any || items[i].dX || items[i].dW;
  if (!any) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (tokens == 0) {
    // no tokens: every dX is empty and every dW all zeros (no workspace);
    // the zeros belong to the second phase
    if (!(phase & 2)) return ok();
    for (int i = 0; i < count; ++i)
      if (items[i].dW) {
        hipError_t e = bl::launch_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, items[i].dW,
                                      nullptr, 0, items[i].k, items[i].n_out, bl::s_of(n, m), s);
        if (e != hipSuccess) return hip_status(e, "dW clear");
      }
    return ok();
  }
  const size_t need = bitlinear_bwd_group_workspace_bytes(items, count, tokens);
  if (!ws || ws_bytes < need)
    return fail(BL_EWORKSPACE, "grouped backward workspace needs %zu bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  TRY(check_ptr(ws, 256, "ws"));
  std::vector<bl::BwdItem> its;
  for (int i = 0; i < count; ++i) {
    const bitlinear_bwd_item& it = items[i];
    if (!it.dX && !it.dW) continue;
    its.push_back(bl::BwdItem{it.dY, it.xq, it.x_scale, it.packed, it.gamma, it.dX, it.dW, it.k, it.n_out});
  }
  if (its.empty()) return ok();
  hipError_t e = bl::launch_bwd_group(its.data(), (int)its.size(), tokens, bl::s_of(n, m), ws, phase, s);
  return hip_status(e, "grouped backward launch");
}

int bitlinear_bwd_group(const bitlinear_bwd_item* items, int count, int64_t tokens, int n, int m,
                        void* ws, size_t ws_bytes, void* stream) {
  return bwd_group_run(items, count, tokens, n, m, BL_BWD_PREPARE | BL_BWD_FINISH, ws, ws_bytes, stream);
}

int bitlinear_bwd_group_phase(const bitlinear_bwd_item* items, int count, int64_t tokens, int n, int m,
                              int phase, void* ws, size_t ws_bytes, void* stream) {
  if (phase < 1 || phase > (BL_BWD_PREPARE | BL_BWD_FINISH))
    return fail(BL_EINVAL, "phase must be BL_BWD_PREPARE, BL_BWD_FINISH or both (got %d)", phase);
  return bwd_group_run(items, count, tokens, n, m, phase, ws, ws_bytes, stream);
}

int bitlinear_bwd_relu2_gate(const uint16_t* dY, const int8_t* xq, const float* x_scale, const void* packed,
                             const double* gamma, int64_t tokens, int64_t k, int64_t n_out, int n, int m,
                             const float* G, const float* U, uint16_t* dG, uint16_t* dU, float* dW, void* ws,
                             size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  if (n_out % 16 != 0)
    return fail(BL_ESHAPE, "the backward needs n_out to be a multiple of 16 (got %lld)", (long long)n_out);
  if (tokens < 0) return fail(BL_ESHAPE, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (tokens >= kLimit || tokens * k >= kLimit || tokens * n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens*k and tokens*n_out must stay below 2^31");
  TRY(check_opt_ptr(dW, 16, "dW"));
  if (tokens == 0) {
    // no tokens: dG and dU are empty and dW is all zeros
    if (dW) {
      hipError_t e = bl::launch_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dW, nullptr, 0, k, n_out,
                                    bl::s_of(n, m), reinterpret_cast<hipStream_t>(stream));
      return hip_status(e, "dW clear");
    }
    return ok();
  }
  {
    const int64_t tp = bl::bwd_tokens_padded(tokens), np = (n_out + 63) / 64 * 64;
    if (tp * n_out >= kLimit / 2 || tp * k >= kLimit / 2 || k * np >= kLimit / 2)
      return fail(BL_ESHAPE, "the backward needs tokens*n_out, tokens*k and n_out*k below 2^30");
  }
  const size_t need = bl::bwd_ws_bytes(tokens, k, n_out);
  if (!ws || ws_bytes < need)
    return fail(BL_EWORKSPACE, "backward workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : (size_t)0);
  TRY(check_ptr(ws, 256, "ws"));
  TRY(check_ptr(dY, 16, "dY"));
  TRY(check_ptr(packed, 16, "packed"));
  TRY(check_ptr(gamma, 8, "gamma"));
  TRY(check_ptr(G, 16, "G"));
  TRY(check_ptr(U, 16, "U"));
  TRY(check_ptr(dG, 16, "dG"));
  TRY(check_ptr(dU, 16, "dU"));
  if (dW) {
    TRY(check_ptr(xq, 16, "xq"));
    TRY(check_ptr(x_scale, 4, "x_scale"));
  }
  hipError_t e = bl::launch_bwd_gate(dY, xq, x_scale, packed, gamma, G, U, dG, dU, dW, ws, tokens, k, n_out,
                                     bl::s_of(n, m), reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "backward launch");
}

int bitlinear_bwd_tiles(int tiles) {
  if (bl::bwd_set_tiles(tiles) != 0)
    return fail(BL_EINVAL, "bitlinear_bwd_tiles takes 0, 1, 2 or 3 (got %d)", tiles);
  return ok();
}

int bitlinear_bwd(const uint16_t* dY, const int8_t* xq, const float* x_scale, const void* packed,
                  const double* gamma, int64_t tokens, int64_t k, int64_t n_out, int n, int m,
                  float* dX, float* dW, void* ws, size_t ws_bytes, void* stream) {
  TRY(check_nm(n, m));
  TRY(check_layer(n_out, k));
  if (n_out % 16 != 0)
    return fail(BL_ESHAPE, "the backward needs n_out to be a multiple of 16 (got %lld)", (long long)n_out);
  if (tokens < 0) return fail(BL_ESHAPE, "tokens must be >= 0 (got %lld)", (long long)tokens);
  if (tokens >= kLimit || tokens * k >= kLimit || tokens * n_out >= kLimit)
    return fail(BL_ESHAPE, "tokens*k and tokens*n_out must stay below 2^31");
  TRY(check_opt_ptr(dX, 16, "dX"));
  TRY(check_opt_ptr(dW, 16, "dW"));
  if (!dX && !dW) return ok();
  if (tokens == 0) {
    // no tokens: dX is empty and dW is all zeros (no workspace needed)
    if (dW) {
      hipError_t e = bl::launch_bwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, dW, nullptr,
                                    0, k, n_out, bl::s_of(n, m), reinterpret_cast<hipStream_t>(stream));
      return hip_status(e, "dW clear");
    }
    return ok();
  }
  {  // every bf16 operand of the two products stays below 2 GiB
    const int64_t tp = bl::bwd_tokens_padded(tokens), np = (n_out + 63) / 64 * 64;
    if (tp * n_out >= kLimit / 2 || tp * k >= kLimit / 2 || k * np >= kLimit / 2)
      return fail(BL_ESHAPE, "the backward needs tokens*n_out, tokens*k and n_out*k below 2^30");
  }
  const size_t need = bl::bwd_ws_bytes(tokens, k, n_out);
  if (!ws || ws_bytes < need)
    return fail(BL_EWORKSPACE, "backward workspace needs %zu bytes (got %zu)", need,
                ws ? ws_bytes : (size_t)0);
  TRY(check_ptr(ws, 256, "ws"));
  TRY(check_ptr(dY, 16, "dY"));
  // every input of every requested output is checked before the first launch
  if (dX) {
    TRY(check_ptr(packed, 16, "packed"));
    TRY(check_ptr(gamma, 8, "gamma"));
  }
  if (dW) {
    TRY(check_ptr(xq, 16, "xq"));
    TRY(check_ptr(x_scale, 4, "x_scale"));
  }
  hipError_t e = bl::launch_bwd(dY, xq, x_scale, packed, gamma, dX, dW, ws, tokens, k, n_out,
                                bl::s_of(n, m), reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "backward launch");
}

const char* bitlinear_status_string(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_EINVAL: return "invalid argument (null or misaligned pointer, bad enum)";
    case BL_ESHAPE: return "unsupported shape";
    case BL_EUNSUPPORTED: return "unsupported N:M pattern";
    case BL_EWORKSPACE: return "workspace missing or too small";
    case BL_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bitlinear_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

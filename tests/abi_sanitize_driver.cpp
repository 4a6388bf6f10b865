// Drives the library's host code -- argument validation of every entry
// point, the size helpers, and the grouped decode plan builder -- under
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no
// device is needed, and no call here reaches a launch).  Built and run by
// tests/test_abi_sanitizers.py.  Exits non-zero if a status is not the
// expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bitlinear.h"

#define CHECK(c)                                                       \
  do {                                                                 \
    if (!(c)) {                                                        \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

int main() {
  // 16-byte aligned stand-in addresses: only stored, never dereferenced
  alignas(256) static unsigned char stand_in[4096];
  void* A = stand_in;
  int64_t tokens = 4;
  // size helpers across patterns and shapes
  const int pats[6][2] = {{8, 8}, {6, 8}, {4, 8}, {2, 4}, {3, 8}, {2, 8}};
  for (auto& p : pats) {
    CHECK(bitlinear_packed_bytes(72, 256, p[0], p[1]) > 0);
    CHECK(bitlinear_packed_bytes(72, 100, p[0], p[1]) == 0);
  }
  CHECK(bitlinear_packed_bytes(72, 256, 5, 8) == 0);
  CHECK(bitlinear_workspace_bytes(72, 256) > 0);
  CHECK(bitlinear_bwd_workspace_bytes(300, 256, 48) > 0);
  CHECK(bitlinear_fwd_workspace_bytes(3, 11008, 2048) > 0);
  CHECK(bitlinear_sp24_packed_bytes(72, 256) > 0);
  for (int s = -2; s < 12; ++s) CHECK(bitlinear_status_string(s) != nullptr);
  // validation failures: nothing is launched
  CHECK(bitlinear_quantize_mask(nullptr, 72, 256, 6, 8, 0, (uint8_t*)A, nullptr, (double*)A, A, 4096, nullptr) ==
        BL_EINVAL);
  CHECK(bitlinear_quantize_mask((const uint16_t*)A, 72, 100, 6, 8, 0, (uint8_t*)A, nullptr, (double*)A, A, 4096,
                                nullptr) == BL_ESHAPE);
  CHECK(bitlinear_pack((const uint16_t*)A, (const uint8_t*)A, (const double*)A, 72, 256, 5, 8, A, 4096, nullptr) ==
        BL_EUNSUPPORTED);
  CHECK(bitlinear_fwd((const uint16_t*)A, -1, 256, A, 72, 6, 8, (const double*)A, (float*)A, nullptr, nullptr,
                      nullptr, A, 0, nullptr) == BL_ESHAPE);
  CHECK(bitlinear_contract(nullptr, (const float*)A, tokens, 256, A, 72, 6, 8, (const double*)A, (float*)A,
                           nullptr, A, 4096, nullptr) == BL_EINVAL);
  CHECK(bitlinear_bwd((const uint16_t*)A, (const int8_t*)A, (const float*)A, A, (const double*)A, tokens, 256, 40,
                      6, 8, (float*)A, (float*)A, A, 1 << 20, nullptr) == BL_ESHAPE);  // n_out % 16
  CHECK(bitlinear_latent_update((float*)A, (const float*)A, 7, 1e-3f, (uint16_t*)A, nullptr) == BL_ESHAPE);
  CHECK(bitlinear_bwd_tiles(7) == BL_EINVAL);
  CHECK(std::strlen(bitlinear_last_error()) > 0);
  // grouped backward and grouped contraction: validation of every item
  std::vector<bitlinear_bwd_item> bi(3);
  for (auto& it : bi) it = bitlinear_bwd_item{(const uint16_t*)A, (const int8_t*)A, (const float*)A, A,
                                              (const double*)A, (float*)A, (float*)A, 256, 128};
  bi[2].n_out = 120;
  CHECK(bitlinear_bwd_group_workspace_bytes(bi.data(), 3, 300) == 0);
  CHECK(bitlinear_bwd_group(bi.data(), 3, 300, 6, 8, A, 4096, nullptr) == BL_ESHAPE);
  std::vector<bitlinear_contract_item> ci(2);
  ci[0] = bitlinear_contract_item{A, (const double*)A, (float*)A, nullptr, 896};
  ci[1] = bitlinear_contract_item{A, (const double*)A, (float*)A, (uint16_t*)A, 128};
  CHECK(bitlinear_contract_group(ci.data(), 2, (const int8_t*)A, (const float*)A, 64, 896, 6, 8, nullptr, 0,
                                 nullptr) == BL_EINVAL);
  CHECK(bitlinear_contract_group_workspace_bytes(ci.data(), 2, 4, 896) > 0);
  // grouped decode plans built in host memory: ragged layers, several
  // token counts and patterns, one-launch fit checks
  const int64_t shapes[7][2] = {{896, 896}, {128, 896}, {128, 896}, {896, 896}, {4864, 896}, {4864, 896},
                                {896, 4864}};
  for (int layers : {1, 3, 24}) {
    std::vector<bitlinear_fwd_item> items;
    for (int l = 0; l < layers; ++l)
      for (auto& sh : shapes)
        items.push_back(bitlinear_fwd_item{(const uint16_t*)A, A, (const double*)A, (float*)A, (int8_t*)A,
                                           (float*)A, sh[1], sh[0]});
    for (int64_t t : {1, 5, 16}) {
      for (auto& p : pats) {
        const int count = (int)items.size();
        const size_t bytes = bitlinear_fwd_group_plan_bytes(items.data(), count, t);
        CHECK(bytes > 0);
        std::vector<unsigned char> image(bytes + 64);
        CHECK(bitlinear_fwd_group_plan_host(items.data(), count, t, p[0], p[1], image.data(), bytes) == BL_OK);
        CHECK(bitlinear_fwd_group_plan_host(items.data(), count, t, p[0], p[1], image.data(), bytes - 1) !=
              BL_OK);
        const int fuses = bitlinear_fwd_group_plan_fuses(items.data(), count, t, p[0], p[1]);
        CHECK(fuses == 0 || fuses == 1);
      }
    }
  }
  std::puts("library host code ran clean");
  return 0;
}

// Drives the C ABI's argument checks under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; the kernel side is stubbed out
// by kernel_stub.cpp, so no device is touched).  Every rejected call must
// return its documented status, leave a message in wkv6_last_error and
// enqueue nothing; every accepted one must reach the (stub) kernel side
// exactly once.  Sizes near the int64 limits exercise the overflow-free size
// arithmetic.  Exits 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <thread>

#include "wkv6.h"

extern int g_enqueued;

namespace {

int failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", line, what, wkv6_last_error());
    ++failures;
  }
}
#define EXPECT(x) expect((x), #x, __LINE__)

// fake, 16-byte aligned addresses, far apart: never dereferenced
void* P(int i) { return reinterpret_cast<void*>(uintptr_t(0x100000000ull) * (i + 1)); }
float* F(int i) { return static_cast<float*>(P(i)); }

int fwd(int64_t B, int64_t T, int64_t C, int64_t H, int mode = 0, int dtype = 1, int bad = -1, int miss = -1) {
  void* p[6] = {P(0), P(1), P(2), P(3), P(4), P(5)};
  if (bad >= 0) p[bad] = nullptr;
  if (miss >= 0) p[miss] = static_cast<char*>(p[miss]) + 4;
  return wkv6_fwd(B, T, C, H, p[0], p[1], p[2], p[3], static_cast<float*>(p[4]), static_cast<float*>(p[5]), mode,
                  dtype, nullptr);
}

// a rejected call: the status, a message, and nothing enqueued
void rejected(int status, int want, int line) {
  const int before = g_enqueued;
  expect(status == want, "status", line);
  expect(std::strlen(wkv6_last_error()) > 0, "message", line);
  expect(g_enqueued == before, "nothing enqueued", line);
}
#define REJECT(call, want) rejected((call), (want), __LINE__)

}  // namespace

int main() {
  const int64_t big = std::numeric_limits<int64_t>::max();
  // sizes and enums
  REJECT(fwd(-1, 8, 128, 2), WKV6_ERR_INVALID_ARG);
  REJECT(fwd(2, -8, 128, 2), WKV6_ERR_INVALID_ARG);
  REJECT(fwd(2, 8, 128, 0), WKV6_ERR_INVALID_ARG);
  REJECT(fwd(2, 8, 130, 4), WKV6_ERR_INVALID_ARG);
  REJECT(fwd(2, 8, 128, 2, 7), WKV6_ERR_INVALID_ARG);
  REJECT(fwd(2, 8, 128, 2, 0, 9), WKV6_ERR_INVALID_ARG);
  REJECT(fwd(2, 8, 96, 2), WKV6_ERR_UNSUPPORTED);
  REJECT(fwd(big, big, 64, 1), WKV6_ERR_UNSUPPORTED);
  REJECT(fwd(big / 64, 3, 64 * 64, 64), WKV6_ERR_UNSUPPORTED);
  REJECT(fwd(1 << 24, 1, 64, 1), WKV6_ERR_UNSUPPORTED);
  REJECT(fwd(4, big / 2, 64, 1), WKV6_ERR_UNSUPPORTED);
  REJECT(fwd(1, int64_t(1) << 31, 64, 1), WKV6_ERR_UNSUPPORTED);
  REJECT(fwd(big, 1, big - (big % 64), big / 64), WKV6_ERR_UNSUPPORTED);
  // pointers
  for (int i = 0; i < 6; ++i) REJECT(fwd(2, 8, 128, 2, 0, 1, i), WKV6_ERR_INVALID_ARG);
  for (int i = 0; i < 6; ++i) REJECT(fwd(2, 8, 128, 2, 0, 1, -1, i), WKV6_ERR_MISALIGNED);
  {  // y overlapping an input
    const int st = wkv6_fwd(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), static_cast<float*>(P(1)), 0, 1, nullptr);
    REJECT(st, WKV6_ERR_INVALID_ARG);
  }
  // accepted calls reach the kernel side once; empty ones do not
  int before = g_enqueued;
  EXPECT(fwd(2, 8, 128, 2) == WKV6_OK && g_enqueued == before + 1 && wkv6_last_error()[0] == 0);
  before = g_enqueued;
  EXPECT(fwd(0, 8, 128, 2) == WKV6_OK && fwd(2, 0, 128, 2) == WKV6_OK && g_enqueued == before);
  before = g_enqueued;
  EXPECT(wkv6_fwd_noalloc(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, nullptr) == WKV6_OK &&
         g_enqueued == before + 1);
  REJECT(wkv6_fwd_noalloc(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), nullptr, 1, 1, nullptr), WKV6_ERR_INVALID_ARG);
  // RWKV-5: w_raw holds C values
  before = g_enqueued;
  EXPECT(wkv5_fwd(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), 0, 0, nullptr) == WKV6_OK &&
         g_enqueued == before + 1);
  // state passing
  REJECT(wkv6_fwd_state(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(6), 1, nullptr),
         WKV6_ERR_INVALID_ARG);   // s_out overlaps s_in
  REJECT(wkv6_fwd_state(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(1), 1, nullptr),
         WKV6_ERR_INVALID_ARG);   // s_out overlaps k
  REJECT(wkv6_fwd_state(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), F(6) + 1, F(7), 1, nullptr),
         WKV6_ERR_MISALIGNED);
  before = g_enqueued;
  EXPECT(wkv6_fwd_state(2, 0, 128, 2, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, F(6), F(7), 1,
                        nullptr) == WKV6_OK && g_enqueued == before + 1);   // T = 0 copies the state
  // fused epilogue: eps must be finite and >= 0
  const float bad_eps[3] = {-1.f, std::nanf(""), INFINITY};
  for (float e : bad_eps)
    REJECT(wkv6_fwd_gn(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), P(5), F(6), F(7), e, P(8), 1, 1, nullptr),
           WKV6_ERR_INVALID_ARG);
  REJECT(wkv6_fwd_gn(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), P(5), F(6), F(7), 1e-5f, P(5), 1, 1, nullptr),
         WKV6_ERR_INVALID_ARG);   // out overlaps g
  // standalone normalisation and gate
  for (float e : bad_eps)
    REJECT(wkv6_group_norm_gate(2, 8, 128, 2, F(0), P(1), F(2), F(3), e, P(4), 1, nullptr), WKV6_ERR_INVALID_ARG);
  REJECT(wkv6_group_norm_gate(2, 8, 128, 2, F(0), P(1), F(2), F(3), 1e-5f, P(0), 1, nullptr), WKV6_ERR_INVALID_ARG);
  REJECT(wkv6_group_norm_gate(2, 8, 96, 2, F(0), P(1), F(2), F(3), 1e-5f, P(4), 1, nullptr), WKV6_ERR_UNSUPPORTED);
  before = g_enqueued;
  EXPECT(wkv6_group_norm_gate(2, 8, 128, 2, F(0), P(1), F(2), F(3), 1e-5f, P(4), 0, nullptr) == WKV6_OK &&
         g_enqueued == before + 1);
  // RWKV-4
  REJECT(wkv4_fwd(-2, 8, 128, P(0), P(1), F(2), F(3), F(4), 1, nullptr), WKV6_ERR_INVALID_ARG);
  REJECT(wkv4_fwd(2, 8, 128, P(0), P(1), F(2), F(3), F(4), 3, nullptr), WKV6_ERR_INVALID_ARG);
  REJECT(wkv4_fwd(big, big, 128, P(0), P(1), F(2), F(3), F(4), 1, nullptr), WKV6_ERR_UNSUPPORTED);
  REJECT(wkv4_fwd(2, 8, 128, P(0), P(1), F(2), F(3), F(0), 1, nullptr), WKV6_ERR_INVALID_ARG);
  // backward: outputs must not overlap inputs or each other
  REJECT(wkv6_bwd(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(6), F(8), F(9), F(10), 0, 1, nullptr),
         WKV6_ERR_INVALID_ARG);
  REJECT(wkv6_bwd(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9), nullptr, 0, 1, nullptr),
         WKV6_ERR_INVALID_ARG);
  before = g_enqueued;
  EXPECT(wkv6_bwd(2, 8, 128, 2, P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9), F(10), 1, 1, nullptr) ==
             WKV6_OK && g_enqueued == before + 1);
  // workspace query: host arithmetic, 0 for invalid sizes
  EXPECT(wkv6_fwd_workspace_bytes(-1, 8, 128, 2, 0, 1) == 0);
  EXPECT(wkv6_fwd_workspace_bytes(big, big, 64, 1, 0, 1) == 0);
  // status strings and the per-thread message
  for (int s = -1; s <= 6; ++s) EXPECT(wkv6_status_str(s) != nullptr);
  EXPECT(wkv6_abi_version() == WKV6_ABI_VERSION);
  fwd(-1, 8, 128, 2);
  std::thread th([] { EXPECT(wkv6_last_error()[0] == 0 && fwd(2, 8, 128, 2) == WKV6_OK); });
  th.join();
  EXPECT(wkv6_last_error()[0] != 0);
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("all argument checks hold under the sanitizers\n");
  return 0;
}

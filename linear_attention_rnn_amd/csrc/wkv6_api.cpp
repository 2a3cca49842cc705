// C ABI of the WKV-6 forward library: argument checks, workspace, launch.
// The declarations and their contract live in include/wkv6.h.
#include "wkv6.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "wkv6_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Size, mode and dtype checks shared by the entry points.
int check_sizes(int64_t B, int64_t T, int64_t C, int64_t H, int mode, int dtype) {
  if (B < 0 || T < 0 || C < 0 || H < 1)
    return fail(WKV6_ERR_INVALID_ARG, "sizes must be B, T, C >= 0 and H >= 1");
  if (C % H != 0) return fail(WKV6_ERR_INVALID_ARG, "C must be a multiple of H");
  if (mode != WKV6_MODE_CAUSAL && mode != WKV6_MODE_BIDIRECTIONAL)
    return fail(WKV6_ERR_INVALID_ARG, "unknown mode");
  if (dtype != WKV6_DTYPE_F32 && dtype != WKV6_DTYPE_BF16)
    return fail(WKV6_ERR_INVALID_ARG, "unknown dtype");
  if (C / H != wkv6::kHead) return fail(WKV6_ERR_UNSUPPORTED, "head size C/H must be 64");
  if (B == 0 || T == 0) return WKV6_OK;
  // One workgroup of 256 work-items per (batch, head) pair: the launch's
  // B * H * 256 work-items must stay below 2^32.  (Segmented launches only
  // happen when B * H is below a few hundred.)  Checked by division, so that
  // no product overflows.
  if (H > wkv6::kMaxItems || B > wkv6::kMaxItems / H)
    return fail(WKV6_ERR_UNSUPPORTED, "B * H exceeds the supported number of (batch, head) pairs (2^24 - 1)");
  // the kernels address one (batch, head) slice with 32-bit byte offsets
  if (T > INT_MAX - wkv6::kChunk || B > INT64_MAX / T || B * T > INT64_MAX / (4 * C) ||
      T > (INT_MAX - 4096) / (4 * C))
    return fail(WKV6_ERR_UNSUPPORTED, "sizes exceed the supported index range");
  return WKV6_OK;
}

// Pointer checks for a call with B, T > 0: present, aligned, and the [B,T,C]
// float32 tensor y (named yname) clear of the inputs.
// w_static: w_raw holds C values (one decay for every token) instead of B*T*C.
int check_tensors(int64_t B, int64_t T, int64_t C, int dtype, const void* r, const void* k, const void* v,
                  const void* w_raw, const float* u, const float* y, const char* yname = "y",
                  bool w_static = false) {
  const void* ptrs[6] = {r, k, v, w_raw, u, y};
  const char* names[6] = {"r", "k", "v", "w_raw", "u", yname};
  for (int i = 0; i < 6; ++i) {
    if (!ptrs[i]) return fail(WKV6_ERR_INVALID_ARG, std::string("null pointer: ") + names[i]);
  }
  for (int i = 0; i < 6; ++i) {
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16)
      return fail(WKV6_ERR_MISALIGNED, std::string("pointer not 16-byte aligned: ") + names[i]);
  }
  const size_t elems = (size_t)B * (size_t)T * (size_t)C;
  const size_t isz = dtype == WKV6_DTYPE_BF16 ? 2 : 4;
  const size_t ybytes = elems * 4;
  for (int i = 0; i < 4; ++i) {
    const size_t n = (i == 3 && w_static) ? (size_t)C : elems;
    if (overlaps(y, ybytes, ptrs[i], n * isz))
      return fail(WKV6_ERR_INVALID_ARG, std::string(yname) + " overlaps " + names[i]);
  }
  if (overlaps(y, ybytes, u, (size_t)C * 4)) return fail(WKV6_ERR_INVALID_ARG, std::string(yname) + " overlaps u");
  return WKV6_OK;
}

// Workspace memory comes from a stream-ordered pool the library owns, one
// per device (allocating from the default pool cost 9-36 us per call).  The
// pool keeps up to WKV6_WORKSPACE_KEEP_BYTES of freed blocks for later calls;
// the runtime hands anything above that back to the device at the next
// synchronisation, and wkv6_trim_workspace releases the rest.
std::mutex g_pool_mu;
std::vector<hipMemPool_t> g_pools;

// The current device's pool (created on first use when `create`), or null.
hipError_t device_pool(hipMemPool_t* out, bool create) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if ((int)g_pools.size() <= dev) g_pools.resize(dev + 1, nullptr);
  if (!g_pools[dev] && create) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t created = nullptr;
    if ((e = hipMemPoolCreate(&created, &props)) != hipSuccess) return e;
    uint64_t keep = WKV6_WORKSPACE_KEEP_BYTES;
    if ((e = hipMemPoolSetAttribute(created, hipMemPoolAttrReleaseThreshold, &keep)) != hipSuccess) {
      (void)hipMemPoolDestroy(created);   // only a pool with the documented bound is kept
      return e;
    }
    g_pools[dev] = created;
  }
  *out = g_pools[dev];
  return hipSuccess;
}

hipError_t ws_alloc(void** p, size_t bytes, hipStream_t s) {
  hipMemPool_t pool = nullptr;
  const hipError_t e = device_pool(&pool, true);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(p, bytes, pool, s);
}

// Workspace (stream-ordered) and kernels.
int run(const wkv6::FwdArgs& a, hipStream_t s) {
  const size_t ws_bytes = wkv6::workspace_bytes(a);
  void* ws = nullptr;
  if (ws_bytes) {
    const hipError_t e = ws_alloc(&ws, ws_bytes, s);
    if (e != hipSuccess)
      return fail(WKV6_ERR_HIP, std::string("workspace allocation: ") + hipGetErrorString(e));
  }
  const hipError_t e = wkv6::enqueue_fwd(a, ws, s);
  if (ws) {
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e == hipSuccess && ef != hipSuccess)
      return fail(WKV6_ERR_HIP, std::string("workspace release: ") + hipGetErrorString(ef));
  }
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return WKV6_OK;
}

wkv6::FwdArgs make_args(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k,
                        const void* v, const void* w_raw, const float* u, float* y, int mode, int dtype) {
  wkv6::FwdArgs a;
  a.B = B;
  a.T = T;
  a.C = C;
  a.H = H;
  a.r = r;
  a.k = k;
  a.v = v;
  a.w_raw = w_raw;
  a.u = u;
  a.y = y;
  a.s_in = nullptr;
  a.s_out = nullptr;
  a.bidirectional = mode == WKV6_MODE_BIDIRECTIONAL;
  a.bf16 = dtype == WKV6_DTYPE_BF16;
  return a;
}

}  // namespace

extern "C" {

int wkv6_abi_version(void) { return WKV6_ABI_VERSION; }

const char* wkv6_status_str(int status) {
  switch (status) {
    case WKV6_OK: return "ok";
    case WKV6_ERR_INVALID_ARG: return "invalid argument";
    case WKV6_ERR_UNSUPPORTED: return "unsupported size";
    case WKV6_ERR_MISALIGNED: return "misaligned pointer";
    case WKV6_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* wkv6_last_error(void) { return g_last_error.c_str(); }

size_t wkv6_fwd_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t H, int mode, int dtype) {
  g_last_error.clear();
  if (check_sizes(B, T, C, H, mode, dtype) != WKV6_OK) return 0;
  if (B == 0 || T == 0) return 0;
  return wkv6::workspace_bytes(make_args(B, T, C, H, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, mode,
                                         dtype));
}

size_t wkv6_workspace_reserved_bytes(void) {
  hipMemPool_t pool = nullptr;
  if (device_pool(&pool, false) != hipSuccess || !pool) return 0;
  uint64_t v = 0;
  if (hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &v) != hipSuccess) return 0;
  return (size_t)v;
}

int wkv6_trim_workspace(void) {
  g_last_error.clear();
  hipMemPool_t pool = nullptr;
  hipError_t e = device_pool(&pool, false);
  if (e == hipSuccess && pool) e = hipMemPoolTrimTo(pool, 0);
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("workspace trim: ") + hipGetErrorString(e));
  return WKV6_OK;
}

int wkv6_fwd(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k,
             const void* v, const void* w_raw, const float* u, float* y, int mode, int dtype,
             void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, mode, dtype);
  if (st != WKV6_OK || B == 0 || T == 0) return st;
  if ((st = check_tensors(B, T, C, dtype, r, k, v, w_raw, u, y)) != WKV6_OK) return st;
  return run(make_args(B, T, C, H, r, k, v, w_raw, u, y, mode, dtype), static_cast<hipStream_t>(stream));
}

int wkv6_fwd_noalloc(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k,
                     const void* v, const void* w_raw, const float* u, float* y, int mode, int dtype,
                     void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, mode, dtype);
  if (st != WKV6_OK || B == 0 || T == 0) return st;
  if ((st = check_tensors(B, T, C, dtype, r, k, v, w_raw, u, y)) != WKV6_OK) return st;
  const hipError_t e = wkv6::enqueue_fwd_noalloc(make_args(B, T, C, H, r, k, v, w_raw, u, y, mode, dtype),
                                                 static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue)
    return fail(WKV6_ERR_UNSUPPORTED, "the call's workspace exceeds the library's 32 MiB scratch array");
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return WKV6_OK;
}

int wkv5_fwd(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k,
             const void* v, const void* w_raw, const float* u, float* y, int mode, int dtype,
             void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, mode, dtype);
  if (st != WKV6_OK || B == 0 || T == 0) return st;
  if ((st = check_tensors(B, T, C, dtype, r, k, v, w_raw, u, y, "y", true)) != WKV6_OK) return st;
  wkv6::FwdArgs a = make_args(B, T, C, H, r, k, v, w_raw, u, y, mode, dtype);
  a.w_static = true;
  return run(a, static_cast<hipStream_t>(stream));
}

int wkv6_fwd_state(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k,
                   const void* v, const void* w_raw, const float* u, float* y, const float* s_in,
                   float* s_out, int dtype, void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, WKV6_MODE_CAUSAL, dtype);
  if (st != WKV6_OK || B == 0) return st;
  if (B * H > INT_MAX / wkv6::kHead / wkv6::kHead)
    return fail(WKV6_ERR_UNSUPPORTED, "sizes exceed the supported index range");
  const size_t sbytes = (size_t)B * (size_t)H * wkv6::kHead * wkv6::kHead * 4;
  if ((s_in && reinterpret_cast<uintptr_t>(s_in) % 16) || (s_out && reinterpret_cast<uintptr_t>(s_out) % 16))
    return fail(WKV6_ERR_MISALIGNED, "state pointer not 16-byte aligned");
  if (s_in && s_out && overlaps(s_in, sbytes, s_out, sbytes))
    return fail(WKV6_ERR_INVALID_ARG, "s_out overlaps s_in");
  if (T > 0) {
    if ((st = check_tensors(B, T, C, dtype, r, k, v, w_raw, u, y)) != WKV6_OK) return st;
    const size_t elems = (size_t)B * (size_t)T * (size_t)C;
    const size_t isz = dtype == WKV6_DTYPE_BF16 ? 2 : 4;
    if (s_in && overlaps(y, elems * 4, s_in, sbytes)) return fail(WKV6_ERR_INVALID_ARG, "y overlaps s_in");
    if (s_out) {
      const void* ins[5] = {r, k, v, w_raw, y};
      const size_t nb[5] = {elems * isz, elems * isz, elems * isz, elems * isz, elems * 4};
      const char* names[5] = {"r", "k", "v", "w_raw", "y"};
      for (int i = 0; i < 5; ++i) {
        if (overlaps(s_out, sbytes, ins[i], nb[i]))
          return fail(WKV6_ERR_INVALID_ARG, std::string("s_out overlaps ") + names[i]);
      }
      if (overlaps(s_out, sbytes, u, (size_t)C * 4)) return fail(WKV6_ERR_INVALID_ARG, "s_out overlaps u");
    }
  }
  wkv6::FwdArgs a = make_args(B, T, C, H, r, k, v, w_raw, u, y, WKV6_MODE_CAUSAL, dtype);
  a.s_in = s_in;
  a.s_out = s_out;
  return run(a, static_cast<hipStream_t>(stream));
}

int wkv6_fwd_gn(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k, const void* v,
                const void* w_raw, const float* u, const void* g, const float* gamma, const float* beta,
                float eps, void* out, int mode, int dtype, void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, mode, dtype);
  if (st != WKV6_OK || B == 0 || T == 0) return st;
  if (!(std::isfinite(eps) && eps >= 0.f)) return fail(WKV6_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const void* ptrs[9] = {r, k, v, w_raw, u, g, gamma, beta, out};
  const char* names[9] = {"r", "k", "v", "w_raw", "u", "g", "gamma", "beta", "out"};
  for (int i = 0; i < 9; ++i)
    if (!ptrs[i]) return fail(WKV6_ERR_INVALID_ARG, std::string("null pointer: ") + names[i]);
  for (int i = 0; i < 9; ++i)
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16)
      return fail(WKV6_ERR_MISALIGNED, std::string("pointer not 16-byte aligned: ") + names[i]);
  const size_t elems = (size_t)B * (size_t)T * (size_t)C, isz = dtype == WKV6_DTYPE_BF16 ? 2 : 4;
  const size_t nb[8] = {elems * isz, elems * isz, elems * isz, elems * isz, (size_t)C * 4,
                        elems * isz, (size_t)C * 4, (size_t)C * 4};
  for (int i = 0; i < 8; ++i)
    if (overlaps(out, elems * 2, ptrs[i], nb[i]))
      return fail(WKV6_ERR_INVALID_ARG, std::string("out overlaps ") + names[i]);
  wkv6::FwdArgs a = make_args(B, T, C, H, r, k, v, w_raw, u, nullptr, mode, dtype);
  a.epi = true;
  a.out = static_cast<uint16_t*>(out);
  a.gate = g;
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  return run(a, static_cast<hipStream_t>(stream));
}

int wkv6_group_norm_gate(int64_t B, int64_t T, int64_t C, int64_t H, const float* y, const void* g,
                         const float* gamma, const float* beta, float eps, void* out, int dtype, void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, WKV6_MODE_CAUSAL, dtype);
  if (st != WKV6_OK || B == 0 || T == 0) return st;
  if (!(std::isfinite(eps) && eps >= 0.f)) return fail(WKV6_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const void* ptrs[5] = {y, g, gamma, beta, out};
  const char* names[5] = {"y", "g", "gamma", "beta", "out"};
  for (int i = 0; i < 5; ++i)
    if (!ptrs[i]) return fail(WKV6_ERR_INVALID_ARG, std::string("null pointer: ") + names[i]);
  for (int i = 0; i < 5; ++i)
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16)
      return fail(WKV6_ERR_MISALIGNED, std::string("pointer not 16-byte aligned: ") + names[i]);
  const size_t elems = (size_t)B * (size_t)T * (size_t)C, isz = dtype == WKV6_DTYPE_BF16 ? 2 : 4;
  const size_t nb[4] = {elems * 4, elems * isz, (size_t)C * 4, (size_t)C * 4};
  for (int i = 0; i < 4; ++i)
    if (overlaps(out, elems * 2, ptrs[i], nb[i]))
      return fail(WKV6_ERR_INVALID_ARG, std::string("out overlaps ") + names[i]);
  wkv6::GnArgs a;
  a.B = B;
  a.T = T;
  a.C = C;
  a.y = y;
  a.g = g;
  a.gamma = gamma;
  a.beta = beta;
  a.eps = eps;
  a.out = static_cast<uint16_t*>(out);
  a.bf16 = dtype == WKV6_DTYPE_BF16;
  const hipError_t e = wkv6::enqueue_gn_gate(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return WKV6_OK;
}

int wkv4_fwd(int64_t B, int64_t T, int64_t C, const void* k, const void* v, const float* w, const float* u,
             float* y, int dtype, void* stream) {
  g_last_error.clear();
  if (B < 0 || T < 0 || C < 0) return fail(WKV6_ERR_INVALID_ARG, "sizes must be B, T, C >= 0");
  if (dtype != WKV6_DTYPE_F32 && dtype != WKV6_DTYPE_BF16) return fail(WKV6_ERR_INVALID_ARG, "unknown dtype");
  if (B == 0 || T == 0 || C == 0) return WKV6_OK;
  // grid: batch items x segments in x (at most B * T / 64 + B), 256-channel blocks in y
  if (B > INT_MAX / 2 || T > INT64_MAX / B / C || (C + 255) / 256 > 65535 || B * ((T + 63) / 64 + 1) > INT_MAX)
    return fail(WKV6_ERR_UNSUPPORTED, "sizes exceed the supported index range");
  const void* ptrs[5] = {k, v, w, u, y};
  const char* names[5] = {"k", "v", "w", "u", "y"};
  for (int i = 0; i < 5; ++i)
    if (!ptrs[i]) return fail(WKV6_ERR_INVALID_ARG, std::string("null pointer: ") + names[i]);
  for (int i = 0; i < 5; ++i)
    if (reinterpret_cast<uintptr_t>(ptrs[i]) % 16)
      return fail(WKV6_ERR_MISALIGNED, std::string("pointer not 16-byte aligned: ") + names[i]);
  const size_t elems = (size_t)B * (size_t)T * (size_t)C, isz = dtype == WKV6_DTYPE_BF16 ? 2 : 4;
  const size_t nb[4] = {elems * isz, elems * isz, (size_t)C * 4, (size_t)C * 4};
  for (int i = 0; i < 4; ++i)
    if (overlaps(y, elems * 4, ptrs[i], nb[i])) return fail(WKV6_ERR_INVALID_ARG, std::string("y overlaps ") + names[i]);
  wkv6::Wkv4Args a;
  a.B = B;
  a.T = T;
  a.C = C;
  a.k = k;
  a.v = v;
  a.w = w;
  a.u = u;
  a.y = y;
  a.bf16 = dtype == WKV6_DTYPE_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t ws_bytes = wkv6::wkv4_workspace_bytes(a);
  void* ws = nullptr;
  if (ws_bytes) {
    const hipError_t e = ws_alloc(&ws, ws_bytes, s);
    if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("workspace allocation: ") + hipGetErrorString(e));
  }
  const hipError_t e = wkv6::enqueue_wkv4(a, ws, s);
  if (ws) {
    const hipError_t ef = hipFreeAsync(ws, s);
    if (e == hipSuccess && ef != hipSuccess)
      return fail(WKV6_ERR_HIP, std::string("workspace release: ") + hipGetErrorString(ef));
  }
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  return WKV6_OK;
}

int wkv6_bwd(int64_t B, int64_t T, int64_t C, int64_t H, const void* r, const void* k, const void* v,
             const void* w_raw, const float* u, const float* dy, float* dr, float* dk, float* dv,
             float* dw_raw, float* du, int mode, int dtype, void* stream) {
  g_last_error.clear();
  int st = check_sizes(B, T, C, H, mode, dtype);
  if (st != WKV6_OK || B == 0) return st;
  if (!du) return fail(WKV6_ERR_INVALID_ARG, "null pointer: du");
  if (reinterpret_cast<uintptr_t>(du) % 16) return fail(WKV6_ERR_MISALIGNED, "pointer not 16-byte aligned: du");
  if (T > 0) {
    if ((st = check_tensors(B, T, C, dtype, r, k, v, w_raw, u, dy, "dy")) != WKV6_OK) return st;
    const size_t elems = (size_t)B * (size_t)T * (size_t)C;
    const size_t isz = dtype == WKV6_DTYPE_BF16 ? 2 : 4;
    const void* outs[4] = {dr, dk, dv, dw_raw};
    const char* onames[4] = {"dr", "dk", "dv", "dw_raw"};
    const void* ins[6] = {r, k, v, w_raw, dy, u};
    const size_t inb[6] = {elems * isz, elems * isz, elems * isz, elems * isz, elems * 4, (size_t)C * 4};
    const char* inames[6] = {"r", "k", "v", "w_raw", "dy", "u"};
    for (int i = 0; i < 4; ++i) {
      if (!outs[i]) return fail(WKV6_ERR_INVALID_ARG, std::string("null pointer: ") + onames[i]);
      if (reinterpret_cast<uintptr_t>(outs[i]) % 16)
        return fail(WKV6_ERR_MISALIGNED, std::string("pointer not 16-byte aligned: ") + onames[i]);
      for (int j = 0; j < 6; ++j) {
        if (overlaps(outs[i], elems * 4, ins[j], inb[j]))
          return fail(WKV6_ERR_INVALID_ARG, std::string(onames[i]) + " overlaps " + inames[j]);
      }
      for (int j = 0; j < i; ++j) {
        if (overlaps(outs[i], elems * 4, outs[j], elems * 4))
          return fail(WKV6_ERR_INVALID_ARG, std::string(onames[i]) + " overlaps " + onames[j]);
      }
      if (overlaps(outs[i], elems * 4, du, (size_t)C * 4))
        return fail(WKV6_ERR_INVALID_ARG, std::string(onames[i]) + " overlaps du");
    }
    for (int j = 0; j < 6; ++j) {
      if (overlaps(du, (size_t)C * 4, ins[j], inb[j]))
        return fail(WKV6_ERR_INVALID_ARG, std::string("du overlaps ") + inames[j]);
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  wkv6::BwdArgs a;
  a.B = B;
  a.T = T;
  a.C = C;
  a.H = H;
  a.r = r;
  a.k = k;
  a.v = v;
  a.w_raw = w_raw;
  a.u = u;
  a.dy = dy;
  a.dr = dr;
  a.dk = dk;
  a.dv = dv;
  a.dw_raw = dw_raw;
  a.du = du;
  a.bidirectional = mode == WKV6_MODE_BIDIRECTIONAL;
  a.bf16 = dtype == WKV6_DTYPE_BF16;
  void* ws = nullptr;
  const size_t ws_bytes = wkv6::bwd_workspace_bytes(a);
  hipError_t e = ws_bytes ? ws_alloc(&ws, ws_bytes, s) : hipSuccess;
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("workspace allocation: ") + hipGetErrorString(e));
  e = wkv6::enqueue_bwd(a, ws, s);
  const hipError_t ef = ws ? hipFreeAsync(ws, s) : hipSuccess;
  if (e != hipSuccess) return fail(WKV6_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
  if (ef != hipSuccess) return fail(WKV6_ERR_HIP, std::string("workspace release: ") + hipGetErrorString(ef));
  return WKV6_OK;
}

}  // extern "C"

// Per-head group normalisation, affine and gate of a WKV output, as a pass of
// its own: out = ((y - mean_h) / sqrt(var_h + eps) * gamma + beta) * g, with
// the mean and the biased variance over the 64 channels of each head, for
// every (batch item, token) ("RWKV Architecture" on llms.blog, section
// "RWKV-5 Eagle": group normalisation per head and SiLU gating;
// deepglint/rwkv-clip "What is the WKV mechanism" page, section "Invocation
// Inside a Transformer-Style Block": the WKV output is normalised, then
// multiplied by the gate).  The fused epilogue of the forward kernels
// computes the same thing inside the sweep; this kernel takes a y already in
// memory (the unfused order: any forward entry point, then this one).
//
// Streaming kernel: 16 threads per head row, 4 channels each (a 16-byte y
// load, the gate as 8 bytes of bf16 or 16 of float32, an 8-byte bf16
// store); the row sums stay inside the 16-lane DPP row.  Two passes over the
// registers (mean, then the variance of the deviations), as the fused path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv6_internal.h"

namespace wkv6 {
namespace {

constexpr int NTG = 256;   // threads per workgroup: 16 head rows

// Sum over the 16 lanes of a DPP row (every lane receives it).
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));   // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));   // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));   // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));   // row_ror:1
  return x;
}

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {   // nearest even
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, b2));
}

template <bool BF16>
__global__ __launch_bounds__(NTG) void gn_gate_kernel(const float* __restrict__ y, const void* __restrict__ g,
                                                      const float* __restrict__ gamma, const float* __restrict__ beta,
                                                      float eps, uint16_t* __restrict__ out, int64_t rows, int64_t C) {
  const int lane16 = threadIdx.x & 15;
  const int64_t H = C / 64;
  for (int64_t row = (int64_t)blockIdx.x * (NTG / 16) + (threadIdx.x >> 4); row < rows;
       row += (int64_t)gridDim.x * (NTG / 16)) {
    // row = (b * T + t) * H + h: the head row starts at element row * 64
    const int64_t e = row * 64 + 4 * lane16;
    const int c = (int)((row % H) * 64) + 4 * lane16;
    const float4 yv = *reinterpret_cast<const float4*>(y + e);
    float gv[4];
    if constexpr (BF16) {
      const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g) + e);
      gv[0] = __uint_as_float(q.x << 16);
      gv[1] = __uint_as_float(q.x & 0xFFFF0000u);
      gv[2] = __uint_as_float(q.y << 16);
      gv[3] = __uint_as_float(q.y & 0xFFFF0000u);
    } else {
      const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(g) + e);
      gv[0] = q.x;
      gv[1] = q.y;
      gv[2] = q.z;
      gv[3] = q.w;
    }
    const float4 ga = *reinterpret_cast<const float4*>(gamma + c);
    const float4 be = *reinterpret_cast<const float4*>(beta + c);
    const float mean = row16_sum((yv.x + yv.y) + (yv.z + yv.w)) * (1.f / 64.f);
    const float d0 = yv.x - mean, d1 = yv.y - mean, d2 = yv.z - mean, d3 = yv.w - mean;
    const float var = row16_sum(fmaf(d0, d0, fmaf(d1, d1, fmaf(d2, d2, d3 * d3)))) * (1.f / 64.f);
    const float rstd = __builtin_amdgcn_rsqf(var + eps);
    const float o0 = fmaf(d0 * rstd, ga.x, be.x) * gv[0];
    const float o1 = fmaf(d1 * rstd, ga.y, be.y) * gv[1];
    const float o2 = fmaf(d2 * rstd, ga.z, be.z) * gv[2];
    const float o3 = fmaf(d3 * rstd, ga.w, be.w) * gv[3];
    *reinterpret_cast<uint2*>(out + e) = make_uint2(bf16_pair(o0, o1), bf16_pair(o2, o3));
  }
}

}  // namespace

hipError_t enqueue_gn_gate(const GnArgs& a, hipStream_t s) {
  const int64_t rows = a.B * a.T * (a.C / 64);
  if (rows == 0) return hipSuccess;
  // enough workgroups for several per CU; each walks its rows in a grid stride
  const int64_t want = (rows + NTG / 16 - 1) / (NTG / 16);
  const unsigned grid = (unsigned)(want < 8192 ? want : 8192);
  if (a.bf16)
    hipLaunchKernelGGL(gn_gate_kernel<true>, dim3(grid), dim3(NTG), 0, s, a.y, a.g, a.gamma, a.beta, a.eps, a.out,
                       rows, a.C);
  else
    hipLaunchKernelGGL(gn_gate_kernel<false>, dim3(grid), dim3(NTG), 0, s, a.y, a.g, a.gamma, a.beta, a.eps, a.out,
                       rows, a.C);
  return hipGetLastError();
}

}  // namespace wkv6

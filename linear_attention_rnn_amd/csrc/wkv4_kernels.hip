// RWKV-4 WKV forward for gfx950: the normalised, vector-state operator.
//
// Per channel c ("RWKV Architecture" on llms.blog, sections "The Fundamental
// Mathematical Duality" and "The Recurrent Inference Formulation"):
//
//   WKV_t = (a_{t-1} + e^{u+k_t} v_t) / (b_{t-1} + e^{u+k_t})
//   a_t = e^{-w} a_{t-1} + e^{k_t} v_t,   b_t = e^{-w} b_{t-1} + e^{k_t}
//
// from a = b = 0.  The exponentials overflow float32 for keys above about 88
// and the sums grow with the sequence, so the state is kept as (a, b, p):
// numerator a e^p and denominator b e^p, with p the largest exponent seen so
// far.  A step rescales both sides to the larger of p (decayed) and the new
// token's exponent, so every factor it forms is at most 1:
//
//   output:  q = max(p, u + k),     y = (e^{p-q} a + e^{u+k-q} v) / (e^{p-q} b + e^{u+k-q})
//   update:  p' = max(p - w, k),    a <- e^{p-w-p'} a + e^{k-p'} v,  b likewise,  p <- p'
//
// In each pair of factors the larger exponent's is exactly 1, so a step
// takes two exponentials (and one reciprocal) instead of four.
//
// The recurrence is linear in (a, b): a segment of L tokens run from zero
// yields a summary (A, Bs, P), and a state entering the segment leaves it
// decayed by e^{-wL} and plus that summary.  Long sequences over few
// channels are therefore cut into G segments: one kernel computes every
// segment's summary, one combines them into the state entering each segment
// (in order, per channel), and the output kernel runs every segment from its
// entering state.  One thread per (batch item, channel, segment); a wave's
// loads cover 64 consecutive channels of one token.  Grid: x = batch item x
// segment, y = block of 256 channels.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "wkv6_internal.h"

namespace wkv6 {
namespace {

constexpr int NT4 = 256;    // threads (channels) per workgroup
constexpr int U4 = 8;       // tokens loaded ahead
constexpr float kL2e = 1.4426950408889634f;

struct P4 {
  const void* k;
  const void* v;
  const float* w;
  const float* u;
  float* y;
  float* summ;    // [B][G][3][C]: (a, b, p) of each segment run from zero
  float* carry;   // [B][G][3][C]: state entering each segment
  int64_t T, C;
  int B, G;
  int64_t SEGL;   // tokens per segment (the last may be shorter)
};

__device__ __forceinline__ float e2(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF16>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  else
    return static_cast<const float*>(p)[i];
}

struct St {
  float a, b, p;
};

// Scale factors of two exponents x and z against their maximum: the larger
// one's factor is exactly 1, so one exponential serves both.
__device__ __forceinline__ void pair_scale(float x, float z, float& fx, float& fz) {
  const float d = x - z;
  const float e = e2(-fabsf(d));
  const bool xbig = d >= 0.f;   // also when x = z; a NaN d falls to the other side
  fx = xbig ? 1.f : e;
  fz = xbig ? e : 1.f;
}

// One token: output (OUT) then update; exponents in log2 units (x log2 e).
template <bool OUT>
__device__ __forceinline__ float step(St& s, float k, float v, float wl, float ul) {
  float y = 0.f;
  const float kl = k * kL2e;
  if (OUT) {
    float e1, e2v;   // 2^(p - q), 2^(u + k - q) with q = max(p, u + k)
    pair_scale(s.p, ul + kl, e1, e2v);
    y = fmaf(e1, s.a, e2v * v) * __builtin_amdgcn_rcpf(fmaf(e1, s.b, e2v));
  }
  const float pw = s.p - wl;
  float f1, f2;      // 2^(p - w - p'), 2^(k - p') with p' = max(p - w, k)
  pair_scale(pw, kl, f1, f2);
  s.a = fmaf(f1, s.a, f2 * v);
  s.b = fmaf(f1, s.b, f2);
  s.p = fmaxf(pw, kl);
  return y;
}

// Run tokens [t_lo, t_hi) of batch item b, channel c from state s.
template <bool BF16, bool OUT>
__device__ __forceinline__ void run(const P4& p, St& s, int b, int64_t c, int64_t t_lo, int64_t t_hi, float wl,
                                    float ul) {
  const int64_t base = (int64_t)b * p.T * p.C + c;
  float kc[U4], vc[U4], kn[U4], vn[U4];
  auto load = [&](int64_t t0, float (&kk)[U4], float (&vv)[U4]) {
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      const int64_t t = t0 + j < t_hi ? t0 + j : t_hi - 1;   // past the end: repeat the last token (unused)
      kk[j] = ld<BF16>(p.k, base + t * p.C);
      vv[j] = ld<BF16>(p.v, base + t * p.C);
    }
  };
  load(t_lo, kc, vc);
  for (int64_t t0 = t_lo; t0 < t_hi; t0 += U4) {
    load(t0 + U4 < t_hi ? t0 + U4 : t0, kn, vn);   // the next group is in flight during this one
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      if (t0 + j < t_hi) {
        const float y = step<OUT>(s, kc[j], vc[j], wl, ul);
        if (OUT) p.y[base + (t0 + j) * p.C] = y;
      }
    }
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      kc[j] = kn[j];
      vc[j] = vn[j];
    }
  }
}

__device__ __forceinline__ bool item(const P4& p, int& b, int& g, int64_t& c) {
  c = (int64_t)blockIdx.y * NT4 + threadIdx.x;
  b = blockIdx.x / p.G;
  g = blockIdx.x % p.G;
  return c < p.C;
}

template <bool BF16>
__global__ __launch_bounds__(NT4) void wkv4_summary_kernel(P4 p) {
  int b, g;
  int64_t c;
  if (!item(p, b, g, c)) return;
  const int64_t t_lo = g * p.SEGL, t_hi = min(p.T, t_lo + p.SEGL);
  St s{0.f, 0.f, -INFINITY};
  run<BF16, false>(p, s, b, c, t_lo, t_hi, p.w[c] * kL2e, 0.f);
  float* o = p.summ + ((int64_t)b * p.G + g) * 3 * p.C + c;
  o[0] = s.a;
  o[p.C] = s.b;
  o[2 * p.C] = s.p;
}

// State entering each segment: s_0 = 0, s_{g+1} = s_g decayed by e^{-w L_g} plus summary g.
__global__ __launch_bounds__(NT4) void wkv4_carry_kernel(P4 p) {
  const int64_t c = (int64_t)blockIdx.y * NT4 + threadIdx.x;
  const int b = blockIdx.x;
  if (c >= p.C) return;
  const float wl = p.w[c] * kL2e;
  St s{0.f, 0.f, -INFINITY};
  for (int g = 0; g < p.G; ++g) {
    const int64_t off = ((int64_t)b * p.G + g) * 3 * p.C + c;
    p.carry[off] = s.a;
    p.carry[off + p.C] = s.b;
    p.carry[off + 2 * p.C] = s.p;
    const float A = p.summ[off], Bs = p.summ[off + p.C], P = p.summ[off + 2 * p.C];
    const int64_t L = min(p.SEGL, p.T - g * p.SEGL);
    const float pd = s.p - wl * (float)L;
    const float p2 = fmaxf(pd, P);
    const float f1 = e2(pd - p2), f2 = e2(P - p2);
    s.a = fmaf(f1, s.a, f2 * A);
    s.b = fmaf(f1, s.b, f2 * Bs);
    s.p = p2;
  }
}

template <bool BF16>
__global__ __launch_bounds__(NT4) void wkv4_out_kernel(P4 p) {
  int b, g;
  int64_t c;
  if (!item(p, b, g, c)) return;
  const int64_t t_lo = g * p.SEGL, t_hi = min(p.T, t_lo + p.SEGL);
  St s{0.f, 0.f, -INFINITY};
  if (p.G > 1) {
    const float* ci = p.carry + ((int64_t)b * p.G + g) * 3 * p.C + c;
    s = St{ci[0], ci[p.C], ci[2 * p.C]};
  }
  run<BF16, true>(p, s, b, c, t_lo, t_hi, p.w[c] * kL2e, p.u[c] * kL2e);
}

struct Plan4 {
  int G;
  int64_t SEGL;
};

Plan4 plan4(const Wkv4Args& a) {
  // Segments cost a second read of k and v and two more launches, so short
  // sequences over at least 256 waves of channels run unsegmented (measured:
  // B64 T196 C768 takes 37 us unsegmented, 46 us in 3 segments); otherwise
  // enough segments of at least 64 tokens for several waves per SIMD.
  const int64_t lanes = a.B * a.C;
  int64_t G = (a.T <= 512 && lanes >= 16384) ? 1 : (262144 + lanes - 1) / lanes;
  if (const char* e = getenv("WKV4_SEGMENTS")) G = atoi(e);
  const int64_t gmax = a.T / 64 > 1 ? a.T / 64 : 1;
  if (G > gmax) G = gmax;
  if (G < 1) G = 1;
  Plan4 pl;
  pl.SEGL = (a.T + G - 1) / G;
  pl.G = (int)((a.T + pl.SEGL - 1) / pl.SEGL);
  return pl;
}

}  // namespace

size_t wkv4_workspace_bytes(const Wkv4Args& a) {
  if (a.B == 0 || a.T == 0) return 0;
  const Plan4 pl = plan4(a);
  if (pl.G == 1) return 0;
  return (size_t)2 * a.B * pl.G * 3 * a.C * sizeof(float);
}

hipError_t enqueue_wkv4(const Wkv4Args& a, void* workspace, hipStream_t s) {
  const Plan4 pl = plan4(a);
  P4 p;
  p.k = a.k;
  p.v = a.v;
  p.w = a.w;
  p.u = a.u;
  p.y = a.y;
  p.T = a.T;
  p.C = a.C;
  p.B = (int)a.B;
  p.G = pl.G;
  p.SEGL = pl.SEGL;
  p.summ = static_cast<float*>(workspace);
  p.carry = pl.G > 1 ? p.summ + (size_t)a.B * pl.G * 3 * a.C : nullptr;
  const unsigned cb = (unsigned)((a.C + NT4 - 1) / NT4);
  const dim3 block(NT4);
  hipError_t e;
  if (pl.G > 1) {
    const dim3 grid((unsigned)(a.B * pl.G), cb);
    if (a.bf16)
      hipLaunchKernelGGL(wkv4_summary_kernel<true>, grid, block, 0, s, p);
    else
      hipLaunchKernelGGL(wkv4_summary_kernel<false>, grid, block, 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(wkv4_carry_kernel, dim3((unsigned)a.B, cb), block, 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(a.B * pl.G), cb);
  if (a.bf16)
    hipLaunchKernelGGL(wkv4_out_kernel<true>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(wkv4_out_kernel<false>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace wkv6

// RWKV-6 WKV backward for gfx950: gradients of sum(y * dy) with respect to
// r, k, v, w_raw and u.
//
// The pages' CUDA extension pairs its forward kernel with a backward kernel
// that produces the gradients of all five inputs (CUDA-kernels page of
// deepglint/rwkv-clip, section "Backward Pass Gradient Computation"); they do
// not give its steps, so the ones below are derived from the recurrence
// (include/wkv6.h).  With S_t the state after token t and G_t = dL/dS_t:
//
//   dr_t[c] = sum_n dy_t[n] (S_{t-1}[c][n] + u[c] k_t[c] v_t[n])
//   G_{t-1} = w_t[c] G_t[c][n] + r_t[c] dy_t[n]              (G_{T-1} = 0)
//   dk_t[c] = sum_n G_t[c][n] v_t[n] + r_t[c] u[c] (dy_t . v_t)
//   dv_t[n] = sum_c G_t[c][n] k_t[c] + (sum_c r_t[c] u[c] k_t[c]) dy_t[n]
//   du[c]   = sum_{b,t} r_t[c] k_t[c] (dy_t . v_t)
//
// The decay gradient needs no state: token j's decay lies between the pairs
// (i, t) with i < j < t, and summing r dr over t > j and k dk over i >= j
// counts exactly those pairs (plus the u terms, which differ only at j), so
// with lambda = ln w = -exp(w_raw):
//
//   dlambda_j = sum_{t>j} r_t dr_t - sum_{i>=j} k_i dk_i + r_j u k_j (dy_j . v_j)
//   dw_raw_j  = dlambda_j * (-exp(w_raw_j))
//
// Two token-by-token passes per (batch, head), state and adjoint in
// registers, fp32 throughout: pass 1 runs forward, recomputes the state and
// writes dr; pass 2 runs backward with the adjoint, reads dr back and writes
// dk, dv and dw_raw.  dlambda is kept as one running sum D_j = sum_{t>j} r dr
// - sum_{i>=j} k dk (D_j = D_{j+1} + r_{j+1} dr_{j+1} - k_j dk_j), whose value
// stays the size of one gradient entry, with a compensation term (Kahan), so
// its rounding does not grow with the sequence as two separate sums would.  The bidirectional mode adds
// the gradients of the later-token sum, the causal problem of the reversed
// sequence without u: the same kernel with reversed token order,
// accumulating into the outputs (its dr goes through a workspace between
// the passes).
//
// Thread t of the 256 holds state rows 4 (t / 16) .. + 3 at columns
// 4 (t % 16) .. + 3: sums over the value channel n stay within a 16-lane row
// of the wave (shuffles), sums over the key channel c cross the 16 row groups
// (shuffles, then LDS across the four waves).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv6_internal.h"

namespace wkv6 {
namespace {

constexpr int HS = kHead;
constexpr int NT = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct BwdParams {
  const void* r;
  const void* k;
  const void* v;
  const void* w;
  const float* u;
  const float* dy;
  float* dr;       // output
  float* dk;
  float* dv;
  float* dw;
  float* dr_tmp;   // REV: the reversed problem's dr between the passes
  float* du_part;  // [B][C] per batch item (u gradient, causal part only)
  int64_t T;
  int64_t C;
  int H;
};

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* p, int64_t i) {
  if constexpr (BF16) {
    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u),
                       __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
  }
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the 16 lanes of a DPP row (the thread's column groups).
__device__ __forceinline__ float row_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

struct Tok {
  float r[4], k[4], wr[4], v[4], dy[4];
};

template <bool BF16>
__device__ __forceinline__ Tok load_tok(const BwdParams& p, int64_t row, int c0, int n0) {
  Tok o;
  const float4 r = load4<BF16>(p.r, row + c0), k = load4<BF16>(p.k, row + c0);
  const float4 w = load4<BF16>(p.w, row + c0), v = load4<BF16>(p.v, row + n0);
  const float4 d = *reinterpret_cast<const float4*>(p.dy + row + n0);
  o.r[0] = r.x; o.r[1] = r.y; o.r[2] = r.z; o.r[3] = r.w;
  o.k[0] = k.x; o.k[1] = k.y; o.k[2] = k.z; o.k[3] = k.w;
  o.wr[0] = w.x; o.wr[1] = w.y; o.wr[2] = w.z; o.wr[3] = w.w;
  o.v[0] = v.x; o.v[1] = v.y; o.v[2] = v.z; o.v[3] = v.w;
  o.dy[0] = d.x; o.dy[1] = d.y; o.dy[2] = d.z; o.dy[3] = d.w;
  return o;
}

// REV: the later-token part of a bidirectional call (reversed token order,
// no u term, outputs accumulated).
template <bool BF16, bool REV>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  __shared__ float sCol[NT / 64][HS];   // per wave: partial column sums
  __shared__ float sRuk[NT / 64];
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int rg = t >> 4, cg = t & 15;
  const int c0 = 4 * rg, n0 = 4 * cg;
  const int64_t T = p.T;
  auto row_of = [&](int64_t q) {   // sweep position q -> element offset of the token's head row
    const int64_t tok = REV ? T - 1 - q : q;
    return (b * T + tok) * p.C + (int64_t)h * HS;
  };
  float u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = REV ? 0.f : p.u[h * HS + c0 + i];
  float* drw = REV ? p.dr_tmp : p.dr;   // where pass 1 leaves dr

  // ---- pass 1: forward, state S, dr
  float S[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) S[i][j] = 0.f;
  Tok cur = load_tok<BF16>(p, row_of(0), c0, n0);
  for (int64_t q = 0; q < T; ++q) {
    const int64_t row = row_of(q);
    const Tok x = cur;
    if (q + 1 < T) cur = load_tok<BF16>(p, row_of(q + 1), c0, n0);
    float dyv = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dyv = fmaf(x.dy[j], x.v[j], dyv);
    dyv = row_sum(dyv);
    float dr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) a = fmaf(S[i][j], x.dy[j], a);
      dr[i] = fmaf(u[i] * x.k[i], dyv, row_sum(a));
    }
    if (cg == 0) *reinterpret_cast<float4*>(drw + row + c0) = make_float4(dr[0], dr[1], dr[2], dr[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w = ex2(-kLog2e * ex2(x.wr[i] * kLog2e));
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = fmaf(w, S[i][j], x.k[i] * x.v[j]);
    }
  }
  __syncthreads();   // pass 1's dr rows are visible to the whole workgroup

  // ---- pass 2: backward, adjoint G, dk, dv, dw_raw
  float G[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) G[i][j] = 0.f;
  // D (running dlambda without the u term), its compensation, and r dr of the
  // token after the current one
  float D[4] = {0.f, 0.f, 0.f, 0.f}, Dc[4] = {0.f, 0.f, 0.f, 0.f}, rdr_next[4] = {0.f, 0.f, 0.f, 0.f};
  float du[4] = {0.f, 0.f, 0.f, 0.f};
  cur = load_tok<BF16>(p, row_of(T - 1), c0, n0);
  for (int64_t q = T - 1; q >= 0; --q) {
    const int64_t row = row_of(q);
    const Tok x = cur;
    if (q > 0) cur = load_tok<BF16>(p, row_of(q - 1), c0, n0);
    const float4 drq = *reinterpret_cast<const float4*>(drw + row + c0);
    const float dr[4] = {drq.x, drq.y, drq.z, drq.w};
    float dyv = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) dyv = fmaf(x.dy[j], x.v[j], dyv);
    dyv = row_sum(dyv);
    // dk (rows), the decay gradient and the u gradient
    float dk[4], dwr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) a = fmaf(G[i][j], x.v[j], a);
      const float bonus = x.r[i] * u[i] * x.k[i] * dyv;
      dk[i] = fmaf(x.r[i] * u[i], dyv, row_sum(a));
      // D += r_{q+1} dr_{q+1} - k_q dk_q, compensated
      const float term = fmaf(-x.k[i], dk[i], rdr_next[i]) - Dc[i];
      const float sum = D[i] + term;
      Dc[i] = (sum - D[i]) - term;
      D[i] = sum;
      rdr_next[i] = x.r[i] * dr[i];
      dwr[i] = (D[i] + bonus) * -ex2(x.wr[i] * kLog2e);
      du[i] = fmaf(x.r[i] * x.k[i], dyv, du[i]);
    }
    // dv (columns): over the thread's rows, the wave's row groups, then the waves
    float dvp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) a = fmaf(G[i][j], x.k[i], a);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      dvp[j] = a;
    }
    float ruk = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) ruk = fmaf(x.r[i] * u[i], x.k[i], ruk);
    ruk += __shfl_xor(ruk, 16);
    ruk += __shfl_xor(ruk, 32);
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sCol[wave][n0 + j] = dvp[j];
      if (lane == 0) sRuk[wave] = ruk;
    }
    __syncthreads();
    if (t < 16) {   // row group 0 writes the 64 columns
      const float rk = sRuk[0] + sRuk[1] + sRuk[2] + sRuk[3];
      float dv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dv[j] = fmaf(rk, x.dy[j], sCol[0][n0 + j] + sCol[1][n0 + j] + sCol[2][n0 + j] + sCol[3][n0 + j]);
      float4* o = reinterpret_cast<float4*>(p.dv + row + n0);
      if (REV) {
        const float4 a = *o;
        dv[0] += a.x; dv[1] += a.y; dv[2] += a.z; dv[3] += a.w;
      }
      *o = make_float4(dv[0], dv[1], dv[2], dv[3]);
    }
    if (cg == 0) {
      float4* ok = reinterpret_cast<float4*>(p.dk + row + c0);
      float4* ow = reinterpret_cast<float4*>(p.dw + row + c0);
      float4 kk = make_float4(dk[0], dk[1], dk[2], dk[3]);
      float4 ww = make_float4(dwr[0], dwr[1], dwr[2], dwr[3]);
      if (REV) {
        const float4 a = *ok, c = *ow;
        float4* orr = reinterpret_cast<float4*>(p.dr + row + c0);
        const float4 d = *orr;
        kk.x += a.x; kk.y += a.y; kk.z += a.z; kk.w += a.w;
        ww.x += c.x; ww.y += c.y; ww.z += c.z; ww.w += c.w;
        *orr = make_float4(d.x + dr[0], d.y + dr[1], d.z + dr[2], d.w + dr[3]);
      }
      *ok = kk;
      *ow = ww;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w = ex2(-kLog2e * ex2(x.wr[i] * kLog2e));
#pragma unroll
      for (int j = 0; j < 4; ++j) G[i][j] = fmaf(w, G[i][j], x.r[i] * x.dy[j]);
    }
    __syncthreads();   // sCol / sRuk are rewritten by the next token
  }
  if (!REV && cg == 0)
    *reinterpret_cast<float4*>(p.du_part + (int64_t)b * p.C + h * HS + c0) = make_float4(du[0], du[1], du[2], du[3]);
}

// du[c] = sum over batch items of the per-item parts.
__global__ __launch_bounds__(NT) void du_reduce_kernel(const float* __restrict__ part, float* __restrict__ du,
                                                       int64_t B, int64_t C) {
  const int64_t c = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
  for (int64_t b = 0; b < B; ++b) s += part[b * C + c];
  du[c] = s;
}

}  // namespace

size_t bwd_workspace_bytes(const BwdArgs& a) {
  if (a.T == 0) return 0;
  size_t n = (size_t)a.B * a.C * 4;                                 // du parts
  if (a.bidirectional) n += (size_t)a.B * a.T * a.C * 4 + 256;      // reversed problem's dr
  return n;
}

hipError_t enqueue_bwd(const BwdArgs& a, void* workspace, hipStream_t s) {
  const dim3 block(NT);
  if (a.T == 0) {   // no tokens: du = 0 (a sum over nothing)
    hipLaunchKernelGGL(du_reduce_kernel, dim3((unsigned)((a.C + NT - 1) / NT)), block, 0, s, nullptr, a.du,
                       (int64_t)0, (int64_t)a.C);
    return hipGetLastError();
  }
  BwdParams p;
  p.r = a.r;
  p.k = a.k;
  p.v = a.v;
  p.w = a.w_raw;
  p.u = a.u;
  p.dy = a.dy;
  p.dr = a.dr;
  p.dk = a.dk;
  p.dv = a.dv;
  p.dw = a.dw_raw;
  p.du_part = static_cast<float*>(workspace);
  p.dr_tmp = a.bidirectional
                 ? reinterpret_cast<float*>((reinterpret_cast<uintptr_t>(p.du_part + a.B * a.C) + 255) & ~uintptr_t(255))
                 : nullptr;
  p.T = a.T;
  p.C = a.C;
  p.H = (int)a.H;
  const dim3 grid((unsigned)(a.B * a.H));
  if (a.bf16)
    hipLaunchKernelGGL((bwd_kernel<true, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((bwd_kernel<false, false>), grid, block, 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.bidirectional) {
    if (a.bf16)
      hipLaunchKernelGGL((bwd_kernel<true, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((bwd_kernel<false, true>), grid, block, 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(du_reduce_kernel, dim3((unsigned)((a.C + NT - 1) / NT)), block, 0, s, p.du_part, a.du,
                     (int64_t)a.B, (int64_t)a.C);
  return hipGetLastError();
}

}  // namespace wkv6

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

// Four consecutive channels of one input row, widened to float32.
template <bool BF16>
struct Raw4 {
  using type = float4;
};
template <>
struct Raw4<true> {
  using type = uint2;
};

template <bool BF16>
__device__ __forceinline__ typename Raw4<BF16>::type ld4(const void* p, int64_t i) {
  if constexpr (BF16)
    return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
  else
    return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
}

__device__ __forceinline__ float4 widen(float4 x) { return x; }
__device__ __forceinline__ float4 widen(uint2 q) {
  return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xFFFF0000u), __uint_as_float(q.y << 16),
                     __uint_as_float(q.y & 0xFFFF0000u));
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a DPP row (xor 1 and xor 2 within quads, then the
// half-row and row mirrors).  Every lane of the row ends with the same bits.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Four sums over the 16 lanes of a DPP row at once, transposed: lanes l and
// 15 - l trade the halves of the four values they do not keep, lanes l and
// 7 - l of each half-row the quarters, and the quads finish with xor 2 and
// xor 1, so each lane ends with the full sum of one of the four values (which
// one depends only on the lane; the kernel finds it by reducing 0, 1, 2, 3).
// hi: lane % 16 >= 8, hq: lane % 8 >= 4.
__device__ __forceinline__ float row_sums4(const float (&x)[4], bool hi, bool hq) {
  const float y0 = (hi ? x[2] : x[0]) + dpp<0x140>(hi ? x[0] : x[2]);
  const float y1 = (hi ? x[3] : x[1]) + dpp<0x140>(hi ? x[1] : x[3]);
  float z = (hq ? y1 : y0) + dpp<0x141>(hq ? y0 : y1);
  z += dpp<0x4E>(z);
  z += dpp<0xB1>(z);
  return z;
}

// Four sums over the four 16-lane rows of the wave (lanes l, l^16, l^32,
// l^48) at once, transposed: a swap of two values between partner rows
// leaves, after one add, the pair sum of the first value in one row of the
// pair and of the second value in the other; the 16-row swaps pair the rows,
// the 32-lane swap the halves.  Each lane ends with the full sum of one of
// the four values (found, like row_sums4's, by reducing 0, 1, 2, 3).
__device__ __forceinline__ float rows_sums4(const float (&a)[4]) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[0]), __float_as_uint(a[1]), false, false);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[2]), __float_as_uint(a[3]), false, false);
  const float s01 = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const float s23 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One sum over the four rows of the wave (every lane ends with it).
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float4 f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ float4 add4(float4 a, float4 b) {
  return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 keep(bool ok, float4 x) {
  return ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
}
__device__ __forceinline__ float at(float4 x, int i) { return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w; }

// Tokens are staged through LDS in blocks of TB: the 256 threads load a
// block with one coalesced access each per array (thread t: token t / 16 of
// the block, channels 4 (t % 16) .. + 3), one block ahead of its use, and
// the outputs of a block leave the same way after it has been processed.
constexpr int TB = 16;

struct Smem {
  float r[TB][HS], k[TB][HS], w[TB][HS], x[TB][HS], lam[TB][HS], v[TB][HS], dy[TB][HS];
  float dyv[TB];
  float oa[TB][HS], ob[TB][HS];        // per token: dr (pass 1); dk and D (pass 2)
  float ov[TB][NT / 64][HS];          // per token and wave: partial column sums for dv
};

// One thread's share of a block as loaded from HBM (zeros past the end).
template <bool BF16>
struct Pre {
  typename Raw4<BF16>::type r, k, w, v;
  float4 dy, dr;
};

// REV: the later-token part of a bidirectional call (reversed token order,
// no u term, outputs accumulated).
template <bool BF16, bool REV>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  __shared__ Smem sm;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // token steps: rows c0 .. c0 + 3 and columns n0 .. n0 + 3 of the state
  const int c0 = 4 * (t >> 4), n0 = 4 * (t & 15);
  // staging and output: token ts of the block, channels cc .. cc + 3
  const int ts = t >> 4, cc = 4 * (t & 15);
  const int64_t T = p.T, C = p.C;
  const int nblk = (int)((T + TB - 1) / TB);
  const int64_t head = (int64_t)b * T * C + (int64_t)h * HS;
  auto row_of = [&](int64_t q) {   // sweep position -> element offset of the token's head row
    return head + (REV ? T - 1 - q : q) * C;
  };
  // after row_sums4 this lane holds row c0 + ri; after rows_sums4, column n0 + cj
  const bool hi = (lane & 8) != 0, hq = (lane & 4) != 0;
  const float idx[4] = {0.f, 1.f, 2.f, 3.f};
  const int ri = (int)(row_sums4(idx, hi, hq) * (1.f / 16.f) + 0.5f);
  const int cj = (int)(rows_sums4(idx) * 0.25f + 0.5f);
  const float u_ri = REV ? 0.f : p.u[h * HS + c0 + ri];
  float uc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) uc[i] = REV ? 0.f : p.u[h * HS + cc + i];
  float* drw = REV ? p.dr_tmp : p.dr;   // where pass 1 leaves dr

  // decay of a staged value: lambda = -exp(w_raw), w = exp(lambda)
  auto decay = [](float4 wr, float4& lam, float4& w) {
    lam = make_float4(-ex2(wr.x * kLog2e), -ex2(wr.y * kLog2e), -ex2(wr.z * kLog2e), -ex2(wr.w * kLog2e));
    w = make_float4(ex2(lam.x * kLog2e), ex2(lam.y * kLog2e), ex2(lam.z * kLog2e), ex2(lam.w * kLog2e));
  };
  // Every prefetch reads a valid row: positions past the end repeat the last
  // token and staging zeroes them, so the loads need no branch (a branch
  // would make the compiler wait for them at once).
  auto at_q = [&](int bi) {
    const int64_t q = (int64_t)bi * TB + ts;
    return row_of(q < T ? q : T - 1) + cc;
  };
  auto stage_dyv = [&](float4 dy, float4 v) {
    const float d = row_sum(fmaf(dy.x, v.x, fmaf(dy.y, v.y, fmaf(dy.z, v.z, dy.w * v.w))));
    if (cc == 0) sm.dyv[ts] = d;
  };

  // ---------------- pass 1: forward sweep, state S, dr
  {
    Pre<BF16> x;
    float4 old_dr;   // REV: the causal part already in p.dr, for the block whose dr leaves next
    auto load = [&](int bi) {
      const int64_t o = at_q(bi);
      x.k = ld4<BF16>(p.k, o);
      x.w = ld4<BF16>(p.w, o);
      x.v = ld4<BF16>(p.v, o);
      x.dy = f4(p.dy + o);
    };
    auto out = [&](int bi) {   // dr of block bi: staged partial sums plus u k (dy . v)
      const int64_t q = (int64_t)bi * TB + ts;
      if (q >= T) return;
      const float4 a = f4(&sm.oa[ts][cc]), k = f4(&sm.k[ts][cc]);
      const float d = sm.dyv[ts];
      const float4 dr = make_float4(fmaf(uc[0] * k.x, d, a.x), fmaf(uc[1] * k.y, d, a.y), fmaf(uc[2] * k.z, d, a.z),
                                    fmaf(uc[3] * k.w, d, a.w));
      const int64_t o = row_of(q) + cc;
      st4(drw + o, dr);
      if (REV) st4(p.dr + o, add4(old_dr, dr));
    };
    float S[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = 0.f;
    load(0);
    for (int bi = 0; bi < nblk; ++bi) {
      __syncthreads();   // the previous block's token steps are done with the staging arrays
      if (bi > 0) out(bi - 1);
      {
        const bool ok = (int64_t)bi * TB + ts < T;
        const float4 k = keep(ok, widen(x.k)), v = keep(ok, widen(x.v)), dy = keep(ok, x.dy);
        float4 lam, w;
        decay(widen(x.w), lam, w);
        st4(&sm.k[ts][cc], k);
        st4(&sm.w[ts][cc], w);
        st4(&sm.v[ts][cc], v);
        st4(&sm.dy[ts][cc], dy);
        stage_dyv(dy, v);
      }
      __syncthreads();
      if (REV) old_dr = f4(p.dr + at_q(bi));
      load(bi + 1 < nblk ? bi + 1 : bi);
      struct Tk {
        float4 k, w, v, dy;
      };
      auto rd = [&](int tt) {
        Tk e;
        e.k = f4(&sm.k[tt][c0]);
        e.w = f4(&sm.w[tt][c0]);
        e.v = f4(&sm.v[tt][n0]);
        e.dy = f4(&sm.dy[tt][n0]);
        return e;
      };
      Tk nx = rd(0);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const Tk e = nx;
        if (tt + 1 < TB) nx = rd(tt + 1);   // the next token's operands are in flight during this one
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = fmaf(S[i][0], e.dy.x, fmaf(S[i][1], e.dy.y, fmaf(S[i][2], e.dy.z, S[i][3] * e.dy.w)));
        sm.oa[tt][c0 + ri] = row_sums4(a, hi, hq);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ki = at(e.k, i), wi = at(e.w, i);
          S[i][0] = fmaf(wi, S[i][0], ki * e.v.x);
          S[i][1] = fmaf(wi, S[i][1], ki * e.v.y);
          S[i][2] = fmaf(wi, S[i][2], ki * e.v.z);
          S[i][3] = fmaf(wi, S[i][3], ki * e.v.w);
        }
      }
    }
    __syncthreads();
    out(nblk - 1);
  }
  __syncthreads();   // pass 1's dr rows are written before pass 2 reads them

  // ---------------- pass 2: backward sweep, adjoint G, dk, dv, dw_raw
  {
    Pre<BF16> x;
    float4 old_k, old_v, old_w;   // REV: the causal parts already in the outputs, for the block that leaves next
    auto load = [&](int bi) {
      const int64_t o = at_q(bi);
      x.r = ld4<BF16>(p.r, o);
      x.k = ld4<BF16>(p.k, o);
      x.w = ld4<BF16>(p.w, o);
      x.v = ld4<BF16>(p.v, o);
      x.dy = f4(p.dy + o);
      x.dr = f4(drw + o);
    };
    auto load_old = [&](int bi) {
      const int64_t o = at_q(bi);
      old_k = f4(p.dk + o);
      old_v = f4(p.dv + o);
      old_w = f4(p.dw + o);
    };
    float du[4] = {0.f, 0.f, 0.f, 0.f};
    auto out = [&](int bi) {   // dk, dv, dw_raw of block bi
      const int64_t q = (int64_t)bi * TB + ts;
      const float4 r = f4(&sm.r[ts][cc]), k = f4(&sm.k[ts][cc]), dy = f4(&sm.dy[ts][cc]);
      const float d = sm.dyv[ts];
      const float4 ru = make_float4(r.x * uc[0], r.y * uc[1], r.z * uc[2], r.w * uc[3]);
      const float ruk = row_sum(fmaf(ru.x, k.x, fmaf(ru.y, k.y, fmaf(ru.z, k.z, ru.w * k.w))));
      if (q >= T) return;
      const float4 lam = f4(&sm.lam[ts][cc]), D = f4(&sm.ob[ts][cc]);
      float4 dk = f4(&sm.oa[ts][cc]);
      float4 dv = add4(add4(f4(&sm.ov[ts][0][cc]), f4(&sm.ov[ts][1][cc])),
                       add4(f4(&sm.ov[ts][2][cc]), f4(&sm.ov[ts][3][cc])));
      dv = make_float4(fmaf(ruk, dy.x, dv.x), fmaf(ruk, dy.y, dv.y), fmaf(ruk, dy.z, dv.z), fmaf(ruk, dy.w, dv.w));
      float4 dw = make_float4(fmaf(ru.x * k.x, d, D.x) * lam.x, fmaf(ru.y * k.y, d, D.y) * lam.y,
                              fmaf(ru.z * k.z, d, D.z) * lam.z, fmaf(ru.w * k.w, d, D.w) * lam.w);
      if (!REV) {
        du[0] = fmaf(r.x * k.x, d, du[0]);
        du[1] = fmaf(r.y * k.y, d, du[1]);
        du[2] = fmaf(r.z * k.z, d, du[2]);
        du[3] = fmaf(r.w * k.w, d, du[3]);
      } else {
        dk = add4(dk, old_k);
        dv = add4(dv, old_v);
        dw = add4(dw, old_w);
      }
      const int64_t o = row_of(q) + cc;
      st4(p.dk + o, dk);
      st4(p.dv + o, dv);
      st4(p.dw + o, dw);
    };
    float G[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) G[i][j] = 0.f;
    // D (running dlambda without the u term), its compensation, and r dr of
    // the token after the current one
    float D = 0.f, Dc = 0.f, rdr_next = 0.f;   // for row c0 + ri
    load(nblk - 1);
    for (int bi = nblk - 1; bi >= 0; --bi) {
      __syncthreads();   // the previous block's token steps are done with the staging arrays
      if (bi < nblk - 1) out(bi + 1);
      {
        const bool ok = (int64_t)bi * TB + ts < T;
        const float4 r = keep(ok, widen(x.r)), k = keep(ok, widen(x.k)), v = keep(ok, widen(x.v));
        const float4 dy = keep(ok, x.dy), dr = keep(ok, x.dr);
        float4 lam, w;
        decay(widen(x.w), lam, w);
        st4(&sm.r[ts][cc], r);
        st4(&sm.k[ts][cc], k);
        st4(&sm.w[ts][cc], w);
        st4(&sm.lam[ts][cc], lam);
        st4(&sm.x[ts][cc], make_float4(r.x * dr.x, r.y * dr.y, r.z * dr.z, r.w * dr.w));
        st4(&sm.v[ts][cc], v);
        st4(&sm.dy[ts][cc], dy);
        stage_dyv(dy, v);
      }
      __syncthreads();
      if (REV) load_old(bi);
      load(bi > 0 ? bi - 1 : 0);
      struct Tk {
        float4 r, k, w, v, dy;
        float d, ki, rdri, rui;   // dy . v; k, r dr and r u of row c0 + ri
      };
      auto rd = [&](int tt) {
        Tk e;
        e.r = f4(&sm.r[tt][c0]);
        e.k = f4(&sm.k[tt][c0]);
        e.w = f4(&sm.w[tt][c0]);
        e.v = f4(&sm.v[tt][n0]);
        e.dy = f4(&sm.dy[tt][n0]);
        e.d = sm.dyv[tt];
        e.ki = sm.k[tt][c0 + ri];
        e.rdri = sm.x[tt][c0 + ri];
        e.rui = sm.r[tt][c0 + ri] * u_ri;
        return e;
      };
      Tk nx = rd(TB - 1);
#pragma unroll
      for (int tt = TB - 1; tt >= 0; --tt) {
        const Tk e = nx;
        if (tt > 0) nx = rd(tt - 1);   // the next token's operands are in flight during this one
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[i] = fmaf(G[i][0], e.v.x, fmaf(G[i][1], e.v.y, fmaf(G[i][2], e.v.z, G[i][3] * e.v.w)));
        const float dk = fmaf(e.rui, e.d, row_sums4(a, hi, hq));
        // D += r_{q+1} dr_{q+1} - k_q dk_q, compensated
        const float term = fmaf(-e.ki, dk, rdr_next) - Dc;
        const float sum = D + term;
        Dc = (sum - D) - term;
        D = sum;
        rdr_next = e.rdri;
        sm.oa[tt][c0 + ri] = dk;
        sm.ob[tt][c0 + ri] = D;
        float b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = fmaf(G[0][j], e.k.x, fmaf(G[1][j], e.k.y, fmaf(G[2][j], e.k.z, G[3][j] * e.k.w)));
        sm.ov[tt][wave][n0 + cj] = rows_sums4(b);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ri_ = at(e.r, i), wi = at(e.w, i);
          G[i][0] = fmaf(wi, G[i][0], ri_ * e.dy.x);
          G[i][1] = fmaf(wi, G[i][1], ri_ * e.dy.y);
          G[i][2] = fmaf(wi, G[i][2], ri_ * e.dy.z);
          G[i][3] = fmaf(wi, G[i][3], ri_ * e.dy.w);
        }
      }
    }
    __syncthreads();
    out(0);
    if (!REV) {   // du over the threads that share the channels: rows of the wave, then the waves
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = rows_sum(du[i]);
      __syncthreads();
      if (lane < 16) st4(&sm.ov[0][wave][cc], make_float4(du[0], du[1], du[2], du[3]));
      __syncthreads();
      if (t < 16) {
        const float4 s = add4(add4(f4(&sm.ov[0][0][cc]), f4(&sm.ov[0][1][cc])),
                              add4(f4(&sm.ov[0][2][cc]), f4(&sm.ov[0][3][cc])));
        st4(p.du_part + (int64_t)b * C + h * HS + cc, s);
      }
    }
  }
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

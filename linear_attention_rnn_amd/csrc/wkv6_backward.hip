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
#include <stdlib.h>

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
  float* du_part;  // [B][G][C] per batch item and segment (u gradient, causal part only)
  int64_t T;
  int64_t C;
  int H;
  // A sequence may be cut into G segments of SEGL sweep positions each (the
  // last may be shorter), handled by different workgroups.  Carries of the
  // launch's direction, [B*H][G][64][64] (entry [c][n]) and [B*H][G][64]:
  int G;
  int64_t SEGL;
  float* Sl;    // the segment's state after its last token, from zero
  float* Gl;    // the segment's adjoint before its first token, from zero after its last
  float* Wl;    // sum over the segment of lambda = ln w, per channel
  float* Sin;   // state entering the segment (from the earlier segments)
  float* Gin;   // adjoint after the segment's last token (from the later segments)
  float* sig;   // per channel: sum over the segment of r dr - k dk
  const int* only;   // if set, only items with a nonzero entry run (the others return at once)
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

template <bool BF16>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  else
    return static_cast<const float*>(p)[i];
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
  float r[TB][HS], k[TB][HS], dlt[TB][HS], x[TB][HS], lam[TB][HS], v[TB][HS], dy[TB][HS];   // dlt = 1 - w
  float dyv[TB];
  float oa[TB][HS], ob[TB][HS];        // per token: dr (pass 1); dk and D (pass 2)
  float ov[TB][NT / 64][HS];          // per token and wave: partial column sums for dv
};

// Decay of a staged value: lambda = -exp(w_raw) and dlt = 1 - w =
// -expm1(lambda).  The recurrences decay by x <- x - dlt x, never by a product
// with w itself: for slow decays w lies within 1e-4 of 1, where float32
// keeps only a few significant digits of 1 - w, and that relative error of
// the decay compounds over thousands of tokens (1e-4 of the state after 4096
// tokens at w_raw = -9), while dlt keeps full float32 precision.
__device__ __forceinline__ void decay4(float4 wr, float4& lam, float4& dlt) {
  lam = make_float4(-ex2(wr.x * kLog2e), -ex2(wr.y * kLog2e), -ex2(wr.z * kLog2e), -ex2(wr.w * kLog2e));
  dlt = make_float4(-expm1f(lam.x), -expm1f(lam.y), -expm1f(lam.z), -expm1f(lam.w));
}

// x <- w x + a with w = 1 - dlt.
__device__ __forceinline__ float decay_add(float dlt, float x, float a) { return fmaf(-dlt, x, x + a); }

// One thread's share of a block as loaded from HBM (zeros past the end).
template <bool BF16>
struct Pre {
  typename Raw4<BF16>::type r, k, w, v;
  float4 dy, dr;
};

// REV: the later-token part of a bidirectional call (reversed token order,
// no u term, outputs accumulated).  One workgroup per (batch item, head,
// segment); the segments of a segmented call start from the carries.
template <bool BF16, bool REV>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
  __shared__ Smem sm;
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  if (p.only != nullptr && p.only[bh] == 0) return;
  const int b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // token steps: rows c0 .. c0 + 3 and columns n0 .. n0 + 3 of the state
  const int c0 = 4 * (t >> 4), n0 = 4 * (t & 15);
  // staging and output: token ts of the block, channels cc .. cc + 3
  const int ts = t >> 4, cc = 4 * (t & 15);
  const int64_t T = p.T, C = p.C;
  // the segment's sweep positions [q0, q1); block bi covers q0 + bi TB ..
  const int64_t q0 = (int64_t)seg * p.SEGL, q1 = T < q0 + p.SEGL ? T : q0 + p.SEGL;
  const int nblk = (int)((q1 - q0 + TB - 1) / TB);
  const bool segmented = p.G > 1;
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

  // Every prefetch reads a valid row: positions past the end repeat the last
  // token and staging zeroes them, so the loads need no branch (a branch
  // would make the compiler wait for them at once).
  auto pos = [&](int bi) { return q0 + (int64_t)bi * TB + ts; };
  auto at_q = [&](int bi) {
    const int64_t q = pos(bi);
    return row_of(q < q1 ? q : q1 - 1) + cc;
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
      const int64_t q = pos(bi);
      if (q >= q1) return;
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
    if (segmented) {   // the state the earlier segments hand over
      const float* si = p.Sin + ((int64_t)bh * p.G + seg) * (HS * HS);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 q = f4(si + (c0 + i) * HS + n0);
        S[i][0] = q.x;
        S[i][1] = q.y;
        S[i][2] = q.z;
        S[i][3] = q.w;
      }
    }
    load(0);
    for (int bi = 0; bi < nblk; ++bi) {
      __syncthreads();   // the previous block's token steps are done with the staging arrays
      if (bi > 0) out(bi - 1);
      {
        const bool ok = pos(bi) < q1;
        const float4 k = keep(ok, widen(x.k)), v = keep(ok, widen(x.v));
        float4 lam, dlt;
        decay4(widen(x.w), lam, dlt);
        st4(&sm.k[ts][cc], k);
        st4(&sm.dlt[ts][cc], dlt);
        st4(&sm.v[ts][cc], v);
        const float4 dy = keep(ok, x.dy);
        st4(&sm.dy[ts][cc], dy);
        stage_dyv(dy, v);
      }
      __syncthreads();
      if (REV) old_dr = f4(p.dr + at_q(bi));
      load(bi + 1 < nblk ? bi + 1 : bi);
      struct Tk {
        float4 k, dl, v, dy;   // dl = 1 - w
      };
      auto rd = [&](int tt) {
        Tk e;
        e.k = f4(&sm.k[tt][c0]);
        e.dl = f4(&sm.dlt[tt][c0]);
        e.v = f4(&sm.v[tt][n0]);
        e.dy = f4(&sm.dy[tt][n0]);
        return e;
      };
      Tk nx = rd(0);
#pragma unroll
      for (int tt = 0; tt < TB; ++tt) {
        const Tk e = nx;
        if (tt + 1 < TB) nx = rd(tt + 1);   // the next token's operands are in flight during this one
        {
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            a[i] = fmaf(S[i][0], e.dy.x, fmaf(S[i][1], e.dy.y, fmaf(S[i][2], e.dy.z, S[i][3] * e.dy.w)));
          sm.oa[tt][c0 + ri] = row_sums4(a, hi, hq);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ki = at(e.k, i), di = at(e.dl, i);
          S[i][0] = decay_add(di, S[i][0], ki * e.v.x);
          S[i][1] = decay_add(di, S[i][1], ki * e.v.y);
          S[i][2] = decay_add(di, S[i][2], ki * e.v.z);
          S[i][3] = decay_add(di, S[i][3], ki * e.v.w);
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
      x.w = ld4<BF16>(p.w, o);
      x.dy = f4(p.dy + o);
      x.k = ld4<BF16>(p.k, o);
      x.v = ld4<BF16>(p.v, o);
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
      const int64_t q = pos(bi);
      const float4 r = f4(&sm.r[ts][cc]), k = f4(&sm.k[ts][cc]), dy = f4(&sm.dy[ts][cc]);
      const float d = sm.dyv[ts];
      const float4 ru = make_float4(r.x * uc[0], r.y * uc[1], r.z * uc[2], r.w * uc[3]);
      const float ruk = row_sum(fmaf(ru.x, k.x, fmaf(ru.y, k.y, fmaf(ru.z, k.z, ru.w * k.w))));
      if (q >= q1) return;
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
    if (segmented) {   // the adjoint the later segments hand back
      const float* gi = p.Gin + ((int64_t)bh * p.G + seg) * (HS * HS);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 q = f4(gi + (c0 + i) * HS + n0);
        G[i][0] = q.x;
        G[i][1] = q.y;
        G[i][2] = q.z;
        G[i][3] = q.w;
      }
    }
    // D (running dlambda without the u term), its compensation, and r dr of
    // the token after the current one
    float D = 0.f, Dc = 0.f, rdr_next = 0.f;   // for row c0 + ri
    load(nblk - 1);
    for (int bi = nblk - 1; bi >= 0; --bi) {
      __syncthreads();   // the previous block's token steps are done with the staging arrays
      if (bi < nblk - 1) out(bi + 1);
      {
        const bool ok = pos(bi) < q1;
        const float4 r = keep(ok, widen(x.r)), dy = keep(ok, x.dy);
        float4 lam, dlt;
        decay4(widen(x.w), lam, dlt);
        st4(&sm.r[ts][cc], r);
        st4(&sm.dlt[ts][cc], dlt);
        st4(&sm.dy[ts][cc], dy);
        const float4 k = keep(ok, widen(x.k)), v = keep(ok, widen(x.v)), dr = keep(ok, x.dr);
        st4(&sm.k[ts][cc], k);
        st4(&sm.lam[ts][cc], lam);
        st4(&sm.x[ts][cc], make_float4(r.x * dr.x, r.y * dr.y, r.z * dr.z, r.w * dr.w));
        st4(&sm.v[ts][cc], v);
        stage_dyv(dy, v);
      }
      __syncthreads();
      if (REV) load_old(bi);
      load(bi > 0 ? bi - 1 : 0);
      struct Tk {
        float4 r, k, dl, v, dy;   // dl = 1 - w
        float d, ki, rdri, rui;   // dy . v; k, r dr and r u of row c0 + ri
      };
      auto rd = [&](int tt) {
        Tk e;
        e.r = f4(&sm.r[tt][c0]);
        e.dl = f4(&sm.dlt[tt][c0]);
        e.dy = f4(&sm.dy[tt][n0]);
        e.k = f4(&sm.k[tt][c0]);
        e.v = f4(&sm.v[tt][n0]);
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
        {
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
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ri_ = at(e.r, i), di = at(e.dl, i);
          G[i][0] = decay_add(di, G[i][0], ri_ * e.dy.x);
          G[i][1] = decay_add(di, G[i][1], ri_ * e.dy.y);
          G[i][2] = decay_add(di, G[i][2], ri_ * e.dy.z);
          G[i][3] = decay_add(di, G[i][3], ri_ * e.dy.w);
        }
      }
    }
    __syncthreads();
    out(0);
    // the segment's sum of r dr - k dk: D at its first token plus that token's r dr
    if (segmented && (lane & 3) == 0) p.sig[((int64_t)bh * p.G + seg) * HS + c0 + ri] = (D - Dc) + rdr_next;
    if (!REV) {   // du over the threads that share the channels: rows of the wave, then the waves
#pragma unroll
      for (int i = 0; i < 4; ++i) du[i] = rows_sum(du[i]);
      __syncthreads();
      if (lane < 16) st4(&sm.ov[0][wave][cc], make_float4(du[0], du[1], du[2], du[3]));
      __syncthreads();
      if (t < 16) {
        const float4 s = add4(add4(f4(&sm.ov[0][0][cc]), f4(&sm.ov[0][1][cc])),
                              add4(f4(&sm.ov[0][2][cc]), f4(&sm.ov[0][3][cc])));
        st4(p.du_part + ((int64_t)b * p.G + seg) * C + h * HS + cc, s);
      }
    }
  }
}

// A segment's summaries for the carry kernel, in one pass over its sweep
// positions in order (one workgroup per batch item, head and segment):
//   Sl  its state after its last token, from zero: S <- w S + k^T v;
//       (every decay here is applied as x - (1 - w) x; see decay4)
//   Gl  its adjoint before its first token, from zero after its last:
//       sum_q (prod of w over the segment's positions before q) r_q^T dy_q.
//       No term of that sum depends on another, so it accumulates in the
//       same pass as the state, with the running decay product P
//       (P <- w P after each position, from 1);
//   Wl  its total log decay, sum_q lambda_q, per channel.
// The state of the last segment and the adjoint of the first are never read
// and not stored.
struct SummSmem {
  float r[TB][HS], k[TB][HS], dlt[TB][HS], v[TB][HS], dy[TB][HS];   // dlt = 1 - w
  float red[NT / 64][HS];
};

template <bool BF16, bool REV>
__global__ __launch_bounds__(NT) void bwd_summary_kernel(BwdParams p) {
  __shared__ SummSmem sm;
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  if (p.only != nullptr && p.only[bh] == 0) return;
  const int b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // token steps: rows c0 .. c0 + 3 and columns n0 .. n0 + 3 of both summaries
  const int c0 = 4 * (t >> 4), n0 = 4 * (t & 15);
  // staging: token ts of the block, channels cc .. cc + 3
  const int ts = t >> 4, cc = 4 * (t & 15);
  const int64_t T = p.T, C = p.C;
  const int64_t q0 = (int64_t)seg * p.SEGL, q1 = T < q0 + p.SEGL ? T : q0 + p.SEGL;
  const int nblk = (int)((q1 - q0 + TB - 1) / TB);
  const int64_t head = (int64_t)b * T * C + (int64_t)h * HS;
  auto row_of = [&](int64_t q) { return head + (REV ? T - 1 - q : q) * C; };
  auto pos = [&](int bi) { return q0 + (int64_t)bi * TB + ts; };
  // positions past the end repeat the last token (staging zeroes them), so
  // the prefetch needs no branch
  auto at_q = [&](int bi) {
    const int64_t q = pos(bi);
    return row_of(q < q1 ? q : q1 - 1) + cc;
  };

  Pre<BF16> x;
  auto load = [&](int bi) {
    const int64_t o = at_q(bi);
    x.r = ld4<BF16>(p.r, o);
    x.k = ld4<BF16>(p.k, o);
    x.w = ld4<BF16>(p.w, o);
    x.v = ld4<BF16>(p.v, o);
    x.dy = f4(p.dy + o);
  };
  float S[4][4], G[4][4], P[4] = {1.f, 1.f, 1.f, 1.f}, lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      S[i][j] = 0.f;
      G[i][j] = 0.f;
    }
  load(0);
  for (int bi = 0; bi < nblk; ++bi) {
    __syncthreads();   // the previous block's token steps are done with the staging arrays
    {
      // past the end: zero keys, values, queries and output gradients (their
      // decays only touch summaries after the last real position)
      const bool ok = pos(bi) < q1;
      float4 lam, dlt;
      decay4(widen(x.w), lam, dlt);
      st4(&sm.r[ts][cc], keep(ok, widen(x.r)));
      st4(&sm.k[ts][cc], keep(ok, widen(x.k)));
      st4(&sm.dlt[ts][cc], dlt);
      st4(&sm.v[ts][cc], keep(ok, widen(x.v)));
      st4(&sm.dy[ts][cc], keep(ok, x.dy));
      if (ok) {
        lsum[0] += lam.x;
        lsum[1] += lam.y;
        lsum[2] += lam.z;
        lsum[3] += lam.w;
      }
    }
    __syncthreads();
    load(bi + 1 < nblk ? bi + 1 : bi);
    struct Tk {
      float4 r, k, dl, v, dy;   // dl = 1 - w
    };
    auto rd = [&](int tt) {
      Tk e;
      e.r = f4(&sm.r[tt][c0]);
      e.k = f4(&sm.k[tt][c0]);
      e.dl = f4(&sm.dlt[tt][c0]);
      e.v = f4(&sm.v[tt][n0]);
      e.dy = f4(&sm.dy[tt][n0]);
      return e;
    };
    Tk nx = rd(0);
#pragma unroll
    for (int tt = 0; tt < TB; ++tt) {
      const Tk e = nx;
      if (tt + 1 < TB) nx = rd(tt + 1);   // the next token's operands are in flight during this one
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ki = at(e.k, i), di = at(e.dl, i), pr = P[i] * at(e.r, i);
        S[i][0] = decay_add(di, S[i][0], ki * e.v.x);
        S[i][1] = decay_add(di, S[i][1], ki * e.v.y);
        S[i][2] = decay_add(di, S[i][2], ki * e.v.z);
        S[i][3] = decay_add(di, S[i][3], ki * e.v.w);
        G[i][0] = fmaf(pr, e.dy.x, G[i][0]);
        G[i][1] = fmaf(pr, e.dy.y, G[i][1]);
        G[i][2] = fmaf(pr, e.dy.z, G[i][2]);
        G[i][3] = fmaf(pr, e.dy.w, G[i][3]);
        P[i] = fmaf(-di, P[i], P[i]);
      }
    }
  }
  const int64_t item = (int64_t)bh * p.G + seg;
  if (seg < p.G - 1) {
    float* so = p.Sl + item * (HS * HS);
#pragma unroll
    for (int i = 0; i < 4; ++i) st4(so + (c0 + i) * HS + n0, make_float4(S[i][0], S[i][1], S[i][2], S[i][3]));
  }
  if (seg > 0) {
    float* go = p.Gl + item * (HS * HS);
#pragma unroll
    for (int i = 0; i < 4; ++i) st4(go + (c0 + i) * HS + n0, make_float4(G[i][0], G[i][1], G[i][2], G[i][3]));
  }
  // the total log decay per channel: over the staging rows, then the waves
#pragma unroll
  for (int i = 0; i < 4; ++i) lsum[i] = rows_sum(lsum[i]);
  if (lane < 16) st4(&sm.red[wave][cc], make_float4(lsum[0], lsum[1], lsum[2], lsum[3]));
  __syncthreads();
  if (t < 16) {
    const float4 s4 = add4(add4(f4(&sm.red[0][cc]), f4(&sm.red[1][cc])), add4(f4(&sm.red[2][cc]), f4(&sm.red[3][cc])));
    st4(p.Wl + item * HS + cc, s4);
  }
}

// Segment carries of one direction, per (batch item, head): the state
// entering segment g, Sin[g] = e^{Wl[g-1]} Sin[g-1] + Sl[g-1] from zero, and
// the adjoint after segment g's last token, Gin[g] = e^{Wl[g+1]} Gin[g+1] +
// Gl[g+1] from zero after the last segment (the decays scale the rows: the
// key channel).  Thread t: row t / 4, columns 16 (t % 4) .. + 15.
__global__ __launch_bounds__(NT) void bwd_carry_kernel(BwdParams p) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const int c = t >> 2, n0 = 16 * (t & 3);
  const int64_t base = (int64_t)bh * p.G;
  const int64_t off = (int64_t)c * HS + n0;
  constexpr int64_t PLS = HS * HS;
  // One direction: for each segment in order, store the running value, then
  // fold the segment in (acc = e^{Wl} acc + summary).  The next segment's
  // summary and decay are loaded before the current store, so the loads of
  // consecutive segments overlap.
  auto run = [&](const float* summ, float* dst, int g0, int dg) {
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.f;
    float4 cur[4];
    float e = 0.f;
    auto fetch = [&](int g, float4 (&x)[4], float& ex) {
      const float4* q = reinterpret_cast<const float4*>(summ + (base + g) * PLS + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = q[j];
      ex = ex2(p.Wl[(base + g) * HS + c] * kLog2e);
    };
    fetch(g0, cur, e);
    for (int i = 0, g = g0; i < p.G; ++i, g += dg) {
      float4 nxt[4];
      float en = 0.f;
      const bool more = i + 2 < p.G;   // the last segment's summary is never folded in
      if (more) fetch(g + dg, nxt, en);
      float4* o = reinterpret_cast<float4*>(dst + (base + g) * PLS + off);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
      if (i + 1 < p.G) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[4 * j] = fmaf(e, acc[4 * j], cur[j].x);
          acc[4 * j + 1] = fmaf(e, acc[4 * j + 1], cur[j].y);
          acc[4 * j + 2] = fmaf(e, acc[4 * j + 2], cur[j].z);
          acc[4 * j + 3] = fmaf(e, acc[4 * j + 3], cur[j].w);
        }
      }
      if (more) {
#pragma unroll
        for (int j = 0; j < 4; ++j) cur[j] = nxt[j];
        e = en;
      }
    }
  };
  run(p.Sl, p.Sin, 0, 1);            // state entering each segment, first to last
  run(p.Gl, p.Gin, p.G - 1, -1);     // adjoint after each segment, last to first
}

// The decay gradient's running sum reaches past a segment: for token j of
// segment g, D_j also holds the sum over every later segment of r dr - k dk
// (per direction, in that direction's sweep order).  dw_raw_j += lambda_j
// times those sums.  One workgroup per (batch item, head, causal segment);
// thread t: channel t % 64, tokens t / 64, + 4, ...
template <bool BF16>
__global__ __launch_bounds__(NT) void bwd_dwfix_kernel(BwdParams p, const float* sigc, const float* sigr) {
  __shared__ float sT[64][HS];   // [0]: causal tail of this segment; [1 + g']: reverse tail of reverse segment g'
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  const int b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x;
  const int64_t base = (int64_t)bh * p.G;
  if (t < HS) {
    float acc = 0.f;
    for (int g2 = p.G - 1; g2 > seg; --g2) acc += sigc[(base + g2) * HS + t];
    sT[0][t] = acc;
    if (sigr) {
      acc = 0.f;
      for (int g2 = p.G - 1; g2 >= 0; --g2) {
        sT[1 + g2][t] = acc;
        acc += sigr[(base + g2) * HS + t];
      }
    }
  }
  __syncthreads();
  const int c = t & (HS - 1);
  const int64_t t_lo = (int64_t)seg * p.SEGL, t_hi = p.T < t_lo + p.SEGL ? p.T : t_lo + p.SEGL;
  constexpr int U = 8;   // tokens per thread in flight
  for (int64_t t0 = t_lo + (t >> 6); t0 < t_hi; t0 += U * (NT / HS)) {
    float wr[U], dw[U];
    int64_t o[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      int64_t tok = t0 + j * (NT / HS);
      tok = tok < t_hi ? tok : t_hi - 1;   // past the end: reread the last row (not stored)
      o[j] = ((int64_t)b * p.T + tok) * p.C + (int64_t)h * HS + c;
      wr[j] = ld1<BF16>(p.w, o[j]);
      dw[j] = p.dw[o[j]];
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t tok = t0 + j * (NT / HS);
      if (tok < t_hi) {
        float tail = sT[0][c];
        if (sigr) tail += sT[1 + (int)((p.T - 1 - tok) / p.SEGL)][c];
        p.dw[o[j]] = fmaf(-ex2(wr[j] * kLog2e), tail, dw[j]);
      }
    }
  }
}

// du[c] = sum over the rows (batch items x segments) of the parts: 64
// channels per workgroup, four threads per channel each taking every fourth
// row with eight loads in flight, then the four partial sums through LDS.
__global__ __launch_bounds__(NT) void du_reduce_kernel(const float* __restrict__ part, float* __restrict__ du,
                                                       int64_t R, int64_t C) {
  __shared__ float sp[NT / HS][HS];
  const int cl = threadIdx.x & (HS - 1), q = threadIdx.x / HS;
  const int64_t c = (int64_t)blockIdx.x * HS + cl;
  float acc = 0.f;
  if (c < C) {
    int64_t r = q;
    for (; r + 28 < R; r += 32) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = part[(r + 4 * j) * C + c];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += x[j];
    }
    for (; r < R; r += 4) acc += part[r * C + c];
  }
  sp[q][cl] = acc;
  __syncthreads();
  if (q == 0 && c < C) du[c] = (sp[0][cl] + sp[1][cl]) + (sp[2][cl] + sp[3][cl]);
}

}  // namespace

namespace {

constexpr int kMaxSeg = 63;   // the dw fix-up keeps one row per reverse segment in LDS

struct BwdPlan {
  int G;
  int64_t SEGL;
};

// Fewer items (batch x head) than CUs: cut the sequences into segments of
// whole 16-token blocks, at least 64 tokens each, for about three resident
// workgroups per CU.  With every CU already holding an item, segments only
// add the summary pass (about half a main pass), which costs more than the
// extra occupancy gains (measured: B8 T4096 H32 is fastest unsegmented,
// B4 T4096 H16 fastest with 12 segments).
BwdPlan bwd_plan(const BwdArgs& a) {
  const int64_t bh = a.B * a.H;
  int64_t G = 1;
  if (const char* e = getenv("WKV6_BWD_SEGMENTS")) {
    G = atoi(e);
  } else if (bh < 256) {
    G = (768 + bh - 1) / bh;
  }
  const int64_t gmax = a.T / 64 > 1 ? a.T / 64 : 1;
  if (G > gmax) G = gmax;
  if (G > kMaxSeg) G = kMaxSeg;
  if (G < 1) G = 1;
  BwdPlan pl;
  pl.SEGL = ((a.T + G - 1) / G + TB - 1) / TB * TB;
  pl.G = (int)((a.T + pl.SEGL - 1) / pl.SEGL);
  return pl;
}

struct BwdWs {
  size_t du, drtmp, dir[2], sst[2], slow, total;   // byte offsets; dir: carries, sst: chunk states of each direction
};

// The chunked kernels take bf16 calls whose items run unsegmented, over at
// least one whole chunk: they work in 64-token chunks, so on shorter
// sequences the token-serial kernels are faster (B64 T33 H12 bidirectional:
// 101 against 114 us); from one chunk on the chunked kernels are (same box:
// T64 134 against 139 us, T196 382 against 391 us, T320 507 against 622 us;
// B8 T1000 H32 causal 241 against 479 us).
// WKV6_BWD_CHUNKED=1 / 0 forces the choice for such calls.
constexpr int64_t kChunkedMinT = 64;

bool use_chunked(const BwdArgs& a, const BwdPlan& pl) {
  if (!a.bf16 || pl.G != 1) return false;
  if (const char* e = getenv("WKV6_BWD_CHUNKED")) return atoi(e) != 0;
  return a.T >= kChunkedMinT;
}

size_t up256(size_t n) { return (n + 255) & ~size_t(255); }

BwdWs bwd_ws(const BwdArgs& a, const BwdPlan& pl) {
  BwdWs w;
  size_t n = 0;
  w.du = n;
  n += up256((size_t)a.B * pl.G * a.C * 4);
  w.drtmp = n;
  if (a.bidirectional) n += up256((size_t)a.B * a.T * a.C * 4);
  const size_t per = pl.G > 1 ? (size_t)a.B * a.H * pl.G * (4 * HS * HS + 2 * HS) * 4 : 0;
  for (int d = 0; d < 2; ++d) {
    w.dir[d] = n;
    if (d == 0 || a.bidirectional) n += up256(per);
  }
  w.sst[0] = w.sst[1] = w.slow = n;
  if (use_chunked(a, pl)) {
    const size_t nch = (size_t)((a.T + 63) / 64);
    for (int d = 0; d < (a.bidirectional ? 2 : 1); ++d) {
      w.sst[d] = n;
      n += up256((size_t)a.B * a.H * nch * NT * 16 * 4);
    }
    w.slow = n;
    n += up256((size_t)a.B * a.H * 4);
  }
  w.total = n;
  return w;
}

void set_carries(BwdParams& p, char* ws, size_t off, int64_t bh, int G) {
  float* f = reinterpret_cast<float*>(ws + off);
  const size_t st = (size_t)bh * G * HS * HS, vec = (size_t)bh * G * HS;
  p.Sl = f;
  p.Gl = f + st;
  p.Sin = f + 2 * st;
  p.Gin = f + 3 * st;
  p.Wl = f + 4 * st;
  p.sig = f + 4 * st + vec;
}

// sum: the segment summaries (bwd_summary_kernel), else the gradient passes.
template <bool BF16, bool REV>
void launch_one(bool sum, dim3 grid, hipStream_t s, const BwdParams& p) {
  if (sum)
    hipLaunchKernelGGL((bwd_summary_kernel<BF16, REV>), grid, dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_kernel<BF16, REV>), grid, dim3(NT), 0, s, p);
}

void launch_bwd(bool bf16, bool rev, bool sum, dim3 grid, hipStream_t s, const BwdParams& p) {
  if (bf16)
    rev ? launch_one<true, true>(sum, grid, s, p) : launch_one<true, false>(sum, grid, s, p);
  else
    rev ? launch_one<false, true>(sum, grid, s, p) : launch_one<false, false>(sum, grid, s, p);
}

}  // namespace

size_t bwd_workspace_bytes(const BwdArgs& a) {
  if (a.T == 0) return 0;
  return bwd_ws(a, bwd_plan(a)).total;
}

hipError_t enqueue_bwd(const BwdArgs& a, void* workspace, hipStream_t s) {
  const dim3 block(NT);
  if (a.T == 0) {   // no tokens: du = 0 (a sum over nothing)
    hipLaunchKernelGGL(du_reduce_kernel, dim3((unsigned)((a.C + HS - 1) / HS)), block, 0, s, nullptr, a.du,
                       (int64_t)0, (int64_t)a.C);
    return hipGetLastError();
  }
  const BwdPlan pl = bwd_plan(a);
  const BwdWs lay = bwd_ws(a, pl);
  char* ws = static_cast<char*>(workspace);
  BwdParams p{};
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
  p.du_part = reinterpret_cast<float*>(ws + lay.du);
  p.dr_tmp = a.bidirectional ? reinterpret_cast<float*>(ws + lay.drtmp) : nullptr;
  p.T = a.T;
  p.C = a.C;
  p.H = (int)a.H;
  p.G = pl.G;
  p.SEGL = pl.SEGL;
  const int64_t bh = a.B * a.H;
  const dim3 grid((unsigned)(bh * pl.G));
  hipError_t e;
  if (use_chunked(a, pl)) {
    // chunked kernels, then the token-serial ones for the items they flagged
    // both directions' chunk states first (so that either direction's flag
    // skips an item in both gradient passes), then the two gradient passes
    // back to back: the reversed one adds to outputs the forward one has
    // just written
    int* slow = reinterpret_cast<int*>(ws + lay.slow);
    const int nd = a.bidirectional ? 2 : 1;
    for (int d = 0; d < nd; ++d)
      if ((e = enqueue_bwd_chunk_states(a, reinterpret_cast<float*>(ws + lay.sst[d]), slow, d == 1, s)) != hipSuccess)
        return e;
    for (int d = 0; d < nd; ++d)
      if ((e = enqueue_bwd_chunk_grads(a, p.du_part, reinterpret_cast<const float*>(ws + lay.sst[d]), slow, d == 1,
                                       s)) != hipSuccess)
        return e;
    p.only = slow;
    for (int d = 0; d < (a.bidirectional ? 2 : 1); ++d) {
      launch_bwd(a.bf16, d == 1, false, grid, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(du_reduce_kernel, dim3((unsigned)((a.C + HS - 1) / HS)), block, 0, s, p.du_part, a.du,
                       (int64_t)a.B, (int64_t)a.C);
    return hipGetLastError();
  }
  float* sig[2] = {nullptr, nullptr};
  for (int d = 0; d < (a.bidirectional ? 2 : 1); ++d) {
    const bool rev = d == 1;
    if (pl.G > 1) {
      set_carries(p, ws, lay.dir[d], bh, pl.G);
      sig[d] = p.sig;
      launch_bwd(a.bf16, rev, true, grid, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL(bwd_carry_kernel, dim3((unsigned)bh), block, 0, s, p);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    launch_bwd(a.bf16, rev, false, grid, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (pl.G > 1) {
    if (a.bf16)
      hipLaunchKernelGGL(bwd_dwfix_kernel<true>, grid, block, 0, s, p, sig[0], sig[1]);
    else
      hipLaunchKernelGGL(bwd_dwfix_kernel<false>, grid, block, 0, s, p, sig[0], sig[1]);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(du_reduce_kernel, dim3((unsigned)((a.C + HS - 1) / HS)), block, 0, s, p.du_part, a.du,
                     (int64_t)(a.B * pl.G), (int64_t)a.C);
  return hipGetLastError();
}

}  // namespace wkv6

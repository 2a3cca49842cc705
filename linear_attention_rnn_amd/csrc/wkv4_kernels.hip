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

template <bool BF16, bool NT = false>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  if constexpr (BF16) {
    const uint16_t* q = static_cast<const uint16_t*>(p) + i;
    return __uint_as_float((uint32_t)(NT ? __builtin_nontemporal_load(q) : *q) << 16);
  } else {
    const float* q = static_cast<const float*>(p) + i;
    return NT ? __builtin_nontemporal_load(q) : *q;
  }
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
      kk[j] = ld<BF16, OUT>(p.k, base + t * p.C);   // the output pass reads them last
      vv[j] = ld<BF16, OUT>(p.v, base + t * p.C);
    }
  };
  load(t_lo, kc, vc);
  for (int64_t t0 = t_lo; t0 < t_hi; t0 += U4) {
    load(t0 + U4 < t_hi ? t0 + U4 : t0, kn, vn);   // the next group is in flight during this one
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      if (t0 + j < t_hi) {
        const float y = step<OUT>(s, kc[j], vc[j], wl, ul);
        if (OUT) __builtin_nontemporal_store(y, &p.y[base + (t0 + j) * p.C]);   // not read again
      }
    }
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      kc[j] = kn[j];
      vc[j] = vn[j];
    }
  }
}

// The summary of tokens [t_lo, t_hi) taken from the last token to the first:
// token t weighs 2^(k_t log2 e - (t_hi - 1 - t) w log2 e), so with d the
// decay since the segment's end the same running-maximum form accumulates
// (a, b, p) with every factor at most 1.  The tokens it reads last, the
// segment's first, are then the likeliest still to be in the caches when
// the output kernel starts there.
template <bool BF16>
__device__ __forceinline__ void summary_backwards(const P4& p, St& s, int b, int64_t c, int64_t t_lo,
                                                  int64_t t_hi, float wl) {
  const int64_t base = (int64_t)b * p.T * p.C + c;
  float kc[U4], vc[U4], kn[U4], vn[U4];
  auto load = [&](int64_t t0, float (&kk)[U4], float (&vv)[U4]) {   // tokens t0, t0 - 1, ..
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      const int64_t t = t0 - j >= t_lo ? t0 - j : t_lo;   // past the start: repeat the first token (unused)
      kk[j] = ld<BF16>(p.k, base + t * p.C);
      vv[j] = ld<BF16>(p.v, base + t * p.C);
    }
  };
  float d = 0.f;
  load(t_hi - 1, kc, vc);
  for (int64_t t0 = t_hi - 1; t0 >= t_lo; t0 -= U4) {
    load(t0 - U4 >= t_lo ? t0 - U4 : t0, kn, vn);   // the next group is in flight during this one
#pragma unroll
    for (int j = 0; j < U4; ++j) {
      if (t0 - j >= t_lo) {
        const float e = kc[j] * kL2e - d;
        float f1, f2;   // 2^(p - p'), 2^(e - p') with p' = max(p, e)
        pair_scale(s.p, e, f1, f2);
        s.a = fmaf(f1, s.a, f2 * vc[j]);
        s.b = fmaf(f1, s.b, f2);
        s.p = fmaxf(s.p, e);
        d += wl;
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
  summary_backwards<BF16>(p, s, b, c, t_lo, t_hi, p.w[c] * kL2e);
  float* o = p.summ + ((int64_t)b * p.G + g) * 3 * p.C + c;
  o[0] = s.a;
  o[p.C] = s.b;
  o[2 * p.C] = s.p;
}

// The same summaries for bf16 inputs with C a multiple of 8, their k and v
// rows staged through LDS by direct-to-LDS loads (global_load_lds_dwordx4):
// the bytes in flight then need no registers, so a workgroup keeps three
// groups of kRowsL tokens of k and v in flight (24 KB) while it reads a
// fourth, where the register-staged kernel keeps 8 KB.  Each thread loads one 16-byte
// piece (8 channels of one token) of each array per group; a group's tile
// is kRowsL rows of the workgroup's 256 channels.  Pieces past the last
// channel (wholly, since C % 8 == 0) re-read the block's first piece, and
// rows before the segment re-read its first token; neither is used.
constexpr int kRowsL = 8;     // tokens per staged group
constexpr int kSlotsL = 4;    // groups resident in LDS
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ void lds_barrier4() {   // waits for LDS operations only
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(NT4) void wkv4_summary_lds_kernel(P4 p) {
  __shared__ __attribute__((aligned(16))) char tiles[kSlotsL][2][kRowsL * NT4 * 2];
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t c0 = (int64_t)blockIdx.y * NT4, c = c0 + tid;
  const int b = blockIdx.x / p.G, g = blockIdx.x % p.G;
  const int64_t t_lo = g * p.SEGL, t_hi = min(p.T, t_lo + p.SEGL);
  const int ngr = (int)((t_hi - t_lo + kRowsL - 1) / kRowsL);
  // this thread's piece of a group tile: row tid / 32, channels 8 (tid % 32)..
  const int prow = tid >> 5;
  const int64_t pch = c0 + 8 * (tid & 31);
  const int64_t rowb = p.C * 2;   // bytes per token row
  const int64_t off0 = ((int64_t)b * p.T * p.C + (pch < p.C ? pch : c0)) * 2;
  const char* kb = static_cast<const char*>(p.k) + off0;
  const char* vb = static_cast<const char*>(p.v) + off0;
  // group gi: tokens t_hi - 1 - (gi kRowsL + r), r = 0.., the segment's last first
  auto issue = [&](int gi) {
    int64_t t = t_hi - 1 - ((int64_t)gi * kRowsL + prow);
    if (t < t_lo) t = t_lo;
    char* tk = tiles[gi % kSlotsL][0] + wv * 1024;   // lane l's 16 bytes land at + 16 l
    char* tv = tiles[gi % kSlotsL][1] + wv * 1024;
    __builtin_amdgcn_global_load_lds(kb + t * rowb, (lds_void*)tk, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + t * rowb, (lds_void*)tv, 16, 0, 0);
  };
  // The channel's decay goes to LDS the same way, ahead of group 0 (so it has
  // landed when group 0 has); the first groups are issued unconditionally
  // (past a short segment's end they re-read its first token).
  __shared__ __attribute__((aligned(16))) float wsh[NT4];
  __builtin_amdgcn_global_load_lds(p.w + (c < p.C ? c : c0), (lds_void*)(wsh + 64 * wv), 4, 0, 0);
#pragma unroll
  for (int gi = 0; gi < kSlotsL - 1; ++gi) issue(gi);
  St s{0.f, 0.f, -INFINITY};
  float d = 0.f;
  for (int gi = 0; gi < ngr; ++gi) {
    // this wave's two loads of group gi are done once at most those of the
    // groups issued after it remain: on gfx9 the vector-memory counter of a
    // wave's loads drains in issue order (the compiler's own vmcnt(N) waits
    // between loads rely on the same), and the loop issues no stores.  Near
    // the end, where fewer were issued after it than the count allows for,
    // the wait is only longer than needed.
    const int later = min(ngr - 1 - gi, kSlotsL - 2);
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // every wave's loads of group gi have landed, and every wave has read
    // group gi - 1, whose slot the next issue reuses
    lds_barrier4();
    if (gi + kSlotsL - 1 < ngr) issue(gi + kSlotsL - 1);
    // The group's rows (and the decay) are read in one asm block that waits
    // for its own LDS reads: written as plain reads, they would get a wait
    // for every direct-to-LDS load in flight (the compiler cannot tell the
    // slots apart), the ones just issued included.
    const uint32_t la = (uint32_t)(uintptr_t)(lds_char*)(tiles[gi % kSlotsL][0]) + 2u * (uint32_t)tid;
    const uint32_t lw = (uint32_t)(uintptr_t)(lds_char*)(wsh) + 4u * (uint32_t)tid;
    uint32_t kr[kRowsL], vr[kRowsL], wbits;
    asm volatile(
        "ds_read_u16 %0, %17\n\tds_read_u16 %1, %17 offset:512\n\t"
        "ds_read_u16 %2, %17 offset:1024\n\tds_read_u16 %3, %17 offset:1536\n\t"
        "ds_read_u16 %4, %17 offset:2048\n\tds_read_u16 %5, %17 offset:2560\n\t"
        "ds_read_u16 %6, %17 offset:3072\n\tds_read_u16 %7, %17 offset:3584\n\t"
        "ds_read_u16 %8, %17 offset:4096\n\tds_read_u16 %9, %17 offset:4608\n\t"
        "ds_read_u16 %10, %17 offset:5120\n\tds_read_u16 %11, %17 offset:5632\n\t"
        "ds_read_u16 %12, %17 offset:6144\n\tds_read_u16 %13, %17 offset:6656\n\t"
        "ds_read_u16 %14, %17 offset:7168\n\tds_read_u16 %15, %17 offset:7680\n\t"
        "ds_read_b32 %16, %18\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7]), "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]),
          "=&v"(vr[6]), "=&v"(vr[7]), "=&v"(wbits)
        : "v"(la), "v"(lw));
    const float wl = __uint_as_float(wbits) * kL2e;
#pragma unroll
    for (int r = 0; r < kRowsL; ++r) {
      if (t_hi - 1 - ((int64_t)gi * kRowsL + r) < t_lo) break;   // uniform
      const float kv = __uint_as_float(kr[r] << 16);
      const float vv = __uint_as_float(vr[r] << 16);
      const float e = kv * kL2e - d;
      float f1, f2;   // 2^(p - p'), 2^(e - p') with p' = max(p, e)
      pair_scale(s.p, e, f1, f2);
      s.a = fmaf(f1, s.a, f2 * vv);
      s.b = fmaf(f1, s.b, f2);
      s.p = fmaxf(s.p, e);
      d += wl;
    }
  }
  if (c < p.C) {
    float* o = p.summ + ((int64_t)b * p.G + g) * 3 * p.C + c;
    o[0] = s.a;
    o[p.C] = s.b;
    o[2 * p.C] = s.p;
  }
}

// State entering each segment: s_0 = 0, s_{g+1} = s_g decayed by e^{-w L_g} plus summary g.
// The summaries are loaded kCarryGrp at a time, all before the group's
// stores (written in the loop, the next summary's loads waited behind the
// previous entering state's stores: the two regions could alias as far as
// the compiler knew); slots past the last segment re-read it and are skipped.
constexpr int kCarryGrp = 8;

__global__ __launch_bounds__(NT4) void wkv4_carry_kernel(P4 p) {
  const int64_t c = (int64_t)blockIdx.y * NT4 + threadIdx.x;
  const int b = blockIdx.x;
  if (c >= p.C) return;
  const float wl = p.w[c] * kL2e;
  St s{0.f, 0.f, -INFINITY};
  for (int g0 = 0; g0 < p.G; g0 += kCarryGrp) {
    float A[kCarryGrp], Bs[kCarryGrp], P[kCarryGrp];
#pragma unroll
    for (int u = 0; u < kCarryGrp; ++u) {
      const int g = min(g0 + u, p.G - 1);
      const int64_t off = ((int64_t)b * p.G + g) * 3 * p.C + c;
      A[u] = p.summ[off];
      Bs[u] = p.summ[off + p.C];
      P[u] = p.summ[off + 2 * p.C];
    }
#pragma unroll
    for (int u = 0; u < kCarryGrp; ++u) {
      const int g = g0 + u;
      if (g >= p.G) break;   // uniform
      const int64_t off = ((int64_t)b * p.G + g) * 3 * p.C + c;
      p.carry[off] = s.a;
      p.carry[off + p.C] = s.b;
      p.carry[off + 2 * p.C] = s.p;
      const int64_t L = min(p.SEGL, p.T - g * p.SEGL);
      const float pd = s.p - wl * (float)L;
      const float p2 = fmaxf(pd, P[u]);
      const float f1 = e2(pd - p2), f2 = e2(P[u] - p2);
      s.a = fmaf(f1, s.a, f2 * A[u]);
      s.b = fmaf(f1, s.b, f2 * Bs[u]);
      s.p = p2;
    }
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

// The output pass for bf16 inputs with C a multiple of 8, its k and v rows
// staged through LDS like the summaries' (same groups, slots and pieces),
// by workgroups of two roles: four loader waves issue the direct-to-LDS
// loads and wait for them, four compute waves read the staged rows, run the
// recurrence and store y.  The vector-memory counter is per wave, so the
// loader waves' waits count their loads alone, never the compute waves' y
// stores.  Both roles pass the same one barrier per group.
__global__ __launch_bounds__(2 * NT4) void wkv4_out_lds_kernel(P4 p) {
  __shared__ __attribute__((aligned(16))) char tiles[kSlotsL][2][kRowsL * NT4 * 2];
  const bool loader = threadIdx.x >= NT4;   // uniform per wave
  const int ct = loader ? threadIdx.x - NT4 : threadIdx.x;   // the thread's channel in the block
  const int wv = __builtin_amdgcn_readfirstlane(ct >> 6);
  const int64_t c0 = (int64_t)blockIdx.y * NT4, c = c0 + ct;
  const int b = blockIdx.x / p.G, g = blockIdx.x % p.G;
  const int64_t t_lo = g * p.SEGL, t_hi = min(p.T, t_lo + p.SEGL);
  const int ngr = (int)((t_hi - t_lo + kRowsL - 1) / kRowsL);
  // loader: this thread's piece of a group tile (row ct / 32, channels 8 (ct % 32)..)
  const int prow = ct >> 5;
  const int64_t pch = c0 + 8 * (ct & 31);
  const int64_t rowb = p.C * 2;
  const int64_t off0 = ((int64_t)b * p.T * p.C + (pch < p.C ? pch : c0)) * 2;
  const char* kb = static_cast<const char*>(p.k) + off0;
  const char* vb = static_cast<const char*>(p.v) + off0;
  // group gi: tokens t_lo + gi kRowsL + r, r = 0..; rows past the segment re-read its last token
  auto issue = [&](int gi) {
    int64_t t = t_lo + (int64_t)gi * kRowsL + prow;
    if (t >= t_hi) t = t_hi - 1;
    __builtin_amdgcn_global_load_lds(kb + t * rowb, (lds_void*)(tiles[gi % kSlotsL][0] + wv * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + t * rowb, (lds_void*)(tiles[gi % kSlotsL][1] + wv * 1024), 16, 0, 0);
  };
  // compute: the channel's state, decay and bonus (loaded, and waited for,
  // before the loop)
  const int64_t cc = c < p.C ? c : c0;
  St s{0.f, 0.f, -INFINITY};
  float wl = 0.f, ul = 0.f;
  if (loader) {
#pragma unroll
    for (int gi = 0; gi < kSlotsL - 1; ++gi) issue(gi);
  } else {
    if (p.G > 1) {
      const float* ci = p.carry + ((int64_t)b * p.G + g) * 3 * p.C + cc;
      s = St{ci[0], ci[p.C], ci[2 * p.C]};
    }
    wl = p.w[cc] * kL2e;
    ul = p.u[cc] * kL2e;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  float* yp = p.y + (int64_t)b * p.T * p.C + c;
  for (int gi = 0; gi < ngr; ++gi) {
    if (loader) {
      // this wave's loads of group gi are done once at most those of the
      // groups issued after it remain (in issue order: the wave issues no
      // other vector-memory operation in the loop)
      const int later = min(ngr - 1 - gi, kSlotsL - 2);
      if (later >= 2)
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else if (later == 1)
        asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    lds_barrier4();   // group gi has landed; group gi - 1's slot is free
    if (loader) {
      if (gi + kSlotsL - 1 < ngr) issue(gi + kSlotsL - 1);
      continue;
    }
    // the group's rows, read in one asm block that waits for its own reads
    const uint32_t la = (uint32_t)(uintptr_t)(lds_char*)(tiles[gi % kSlotsL][0]) + 2u * (uint32_t)ct;
    uint32_t kr[kRowsL], vr[kRowsL];
    asm volatile(
        "ds_read_u16 %0, %16\n\tds_read_u16 %1, %16 offset:512\n\t"
        "ds_read_u16 %2, %16 offset:1024\n\tds_read_u16 %3, %16 offset:1536\n\t"
        "ds_read_u16 %4, %16 offset:2048\n\tds_read_u16 %5, %16 offset:2560\n\t"
        "ds_read_u16 %6, %16 offset:3072\n\tds_read_u16 %7, %16 offset:3584\n\t"
        "ds_read_u16 %8, %16 offset:4096\n\tds_read_u16 %9, %16 offset:4608\n\t"
        "ds_read_u16 %10, %16 offset:5120\n\tds_read_u16 %11, %16 offset:5632\n\t"
        "ds_read_u16 %12, %16 offset:6144\n\tds_read_u16 %13, %16 offset:6656\n\t"
        "ds_read_u16 %14, %16 offset:7168\n\tds_read_u16 %15, %16 offset:7680\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3]), "=&v"(kr[4]), "=&v"(kr[5]), "=&v"(kr[6]),
          "=&v"(kr[7]), "=&v"(vr[0]), "=&v"(vr[1]), "=&v"(vr[2]), "=&v"(vr[3]), "=&v"(vr[4]), "=&v"(vr[5]),
          "=&v"(vr[6]), "=&v"(vr[7])
        : "v"(la));
#pragma unroll
    for (int r = 0; r < kRowsL; ++r) {
      const int64_t t = t_lo + (int64_t)gi * kRowsL + r;
      if (t >= t_hi) break;   // uniform
      const float y = step<true>(s, __uint_as_float(kr[r] << 16), __uint_as_float(vr[r] << 16), wl, ul);
      if (c < p.C) __builtin_nontemporal_store(y, yp + t * p.C);   // not read again
    }
  }
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
    if (a.bf16 && a.C % 8 == 0)
      hipLaunchKernelGGL(wkv4_summary_lds_kernel, grid, block, 0, s, p);
    else if (a.bf16)
      hipLaunchKernelGGL(wkv4_summary_kernel<true>, grid, block, 0, s, p);
    else
      hipLaunchKernelGGL(wkv4_summary_kernel<false>, grid, block, 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(wkv4_carry_kernel, dim3((unsigned)a.B, cb), block, 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(a.B * pl.G), cb);
  if (a.bf16 && a.C % 8 == 0)
    hipLaunchKernelGGL(wkv4_out_lds_kernel, grid, dim3(2 * NT4), 0, s, p);
  else if (a.bf16)
    hipLaunchKernelGGL(wkv4_out_kernel<true>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(wkv4_out_kernel<false>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace wkv6

// Device helpers shared by the WKV-6 kernels (gfx950): MFMA operands carried
// as split bf16 parts, swizzled 64x64 LDS planes and their direct and
// transposed reads, buffer-descriptor loads and stores, DPP and permlane
// reductions.
//
// MFMA layouts (v_mfma_f32_16x16x32_bf16, wave64; lane l, g = l / 16,
// i = l % 16): A operand: row i, k-slots 8g..8g+7; B operand: column i, the
// same k-slots; D: column i, rows 4g..4g+3.  The k-slot -> k mapping only has
// to agree between A and B.
#ifndef WKV6_DEVICE_H
#define WKV6_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv6_internal.h"

namespace wkv6 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int HS = kHead;      // head size
constexpr int LC = kChunk;     // chunk length
constexpr int NT = 256;        // threads per workgroup
constexpr int PL = HS * LC;    // elements of one 64x64 plane
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kBlockSpan = 24.f;  // fast path: every 16-token block decays by less than 2^-24


__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier for LDS hand-offs only.  Waves of a workgroup exchange
// data through LDS alone, so the barrier waits for this wave's LDS operations
// (lgkmcnt) but leaves global loads (the next chunk's prefetch) and global
// stores in flight; __syncthreads() would drain those as well.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Lane i of each 16-lane row receives lane i - N of the row (0 if none).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xF, 0xF, true));
}

// An MFMA operand (8 k-slots of one lane) carried as S bf16 parts.
template <int S>
struct Op {
  bf16x8 p[S];
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// A pair rounded to bf16 by one packed conversion.
__device__ __forceinline__ bf16x2 round_pair(float a, float b) {
  return __builtin_convertvector(f32x2{a, b}, bf16x2);
}

// r0 -= h[0], r1 -= h[1] for h = round_pair(r0, r1); the differences are
// exactly representable.  DOT: one bf16 dot product per element, with the
// operand (-1, 0) or (0, -1), accumulating in place (for operands that die
// here); else the rounded parts are unpacked and subtracted.  (-1, 0) is
// loaded into a scalar register by hand: written as a constant the compiler
// encodes it as the inline constant -1.0, which the dot product reads as the
// 32-bit pattern of -1.0f, i.e. the pair (0, -1).
template <bool DOT>
__device__ __forceinline__ void drop_rounded(bf16x2 h, float& r0, float& r1) {
  if constexpr (DOT) {
    uint32_t neg_lo;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(neg_lo));
    r0 = __builtin_amdgcn_fdot2_f32_bf16(h, __builtin_bit_cast(bf16x2, neg_lo), r0, false);
    r1 = __builtin_amdgcn_fdot2_f32_bf16(h, bf16x2{(__bf16)0.f, (__bf16)-1.f}, r1, false);
  } else {
    const uint32_t bits = __builtin_bit_cast(uint32_t, h);
    r0 -= __uint_as_float(bits << 16);
    r1 -= __uint_as_float(bits & 0xFFFF0000u);
  }
}

template <int S, bool DOT = true>
__device__ __forceinline__ Op<S> split8(const float* x) {
  Op<S> o;
#pragma unroll
  for (int jp = 0; jp < 4; ++jp) {
    float r0 = x[2 * jp], r1 = x[2 * jp + 1];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const bf16x2 h = round_pair(r0, r1);
      o.p[s][2 * jp] = h[0];
      o.p[s][2 * jp + 1] = h[1];
      if (s + 1 < S) drop_rounded<DOT>(h, r0, r1);
    }
  }
  return o;
}

// acc += A * B keeping the part products p_i q_j with i + j < max(SA, SB),
// smallest terms first.
template <int SA, int SB>
__device__ __forceinline__ f32x4 mma(const Op<SA>& a, const Op<SB>& b, f32x4 c) {
  constexpr int M = SA > SB ? SA : SB;
#pragma unroll
  for (int d = M - 1; d >= 0; --d)
#pragma unroll
    for (int i = 0; i <= d; ++i) {
      const int j = d - i;
      if (i < SA && j < SB) c = mfma(a.p[i], b.p[j], c);
    }
  return c;
}

// ---- 64x64 bf16 planes in LDS, 16-byte chunks XOR-swizzled by row
__device__ __forceinline__ int swz(int row, int col) {
  return row * 64 + ((((col >> 3) ^ (row & 7)) << 3) | (col & 7));
}

template <int S>
__device__ __forceinline__ Op<S> rd8(const __bf16* P, int off) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) o.p[s] = *reinterpret_cast<const bf16x8*>(P + s * PL + off);
  return o;
}

template <int S>
__device__ __forceinline__ Op<S> rd4x2(const __bf16* P, int o0, int o1) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(P + s * PL + o0);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(P + s * PL + o1);
    o.p[s] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return o;
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// 4m + n supplies the address of 4 consecutive bf16 values; lane i of the
// group receives element i % 4 of the values addressed by lanes 4m + i / 4,
// m = 0..3, in the order of m.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 ld_tr(const __bf16* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// A column of a plane as an MFMA A operand: lane (g, i) gets k-slots
// 8g..8g+7 = rows 8g..8g+7 of column 16 J + i (offsets kt, plus add).
template <int S>
__device__ __forceinline__ Op<S> rdcol8(const __bf16* P, const int (&kt)[2], int add) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bf16x4 a = ld_tr(P + s * PL + add + kt[0]);
    const bf16x4 b = ld_tr(P + s * PL + add + kt[1]);
    o.p[s] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return o;
}

template <int S>
__device__ __forceinline__ void wr8(__bf16* P, int off, const float* x) {
  const Op<S> o = split8<S>(x);
#pragma unroll
  for (int s = 0; s < S; ++s) *reinterpret_cast<bf16x8*>(P + s * PL + off) = o.p[s];
}

template <int S>
__device__ __forceinline__ void wr4(__bf16* P, int off, const float* x) {
  float r[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    bf16x4 q;
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const bf16x2 h = round_pair(r[2 * jp], r[2 * jp + 1]);
      q[2 * jp] = h[0];
      q[2 * jp + 1] = h[1];
      if (s + 1 < S) drop_rounded<false>(h, r[2 * jp], r[2 * jp + 1]);
    }
    *reinterpret_cast<bf16x4*>(P + s * PL + off) = q;
  }
}

template <int S>
__device__ __forceinline__ void wr1(__bf16* P, int off, float x) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const __bf16 h = (__bf16)x;
    P[s * PL + off] = h;
    x -= (float)h;
  }
}

// Global tensors are read and written through buffer descriptors whose base
// is the (batch, head) slice: the base lives in scalar registers, a lane needs
// one 32-bit byte offset, and an offset past the slice's last row reads zero
// and drops a store.  Lanes whose token lies past the segment use such an
// offset, so their keys, values and queries are zero without any masking.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcFlags = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)
// A byte offset past every slice (slices stay below 2^31 - 4096 bytes), small
// enough that adding a row's in-row offset does not overflow.
constexpr int kOffNone = 0x7FFFF000;

__device__ __forceinline__ Rsrc slice_rsrc(const void* p, int64_t elem_off, int isz, int64_t T, int64_t C) {
  char* base = const_cast<char*>(static_cast<const char*>(p)) + elem_off * isz;
  const int nbytes = (int)(((T - 1) * C + HS) * isz);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nbytes, kRsrcFlags);
}

template <int AUX = 0>
__device__ __forceinline__ uint4 bload16(Rsrc r, int off) {
  const auto q = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
  return make_uint4(q[0], q[1], q[2], q[3]);
}

__device__ __forceinline__ float4 bloadf4(Rsrc r, int off) {
  const auto q = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_float4(__uint_as_float(q[0]), __uint_as_float(q[1]), __uint_as_float(q[2]), __uint_as_float(q[3]));
}

// AUX: the cache policy bits of the access (kStream: the non-temporal hint,
// for data not read again soon)
constexpr int kStream = 2;
template <int AUX = 0>
__device__ __forceinline__ void bstoref4(Rsrc r, int off, float a, float b, float c, float d) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 q = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
  __builtin_amdgcn_raw_buffer_store_b128(q, r, off, 0, AUX);
}

// Sum over the four 16-lane rows of the wave (lanes l, l^16, l^32, l^48):
// each swap hands a value to the partner row, so the two halves of its
// result add to the pair's sum in every lane.
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ void load8f(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Offsets of the transposed column reads (rdcol8) of column block cb: lane
// (g, li) reads rows 8 g + li / 4 (+ 4) at columns 16 cb + 4 (li % 4).
__device__ __forceinline__ void col_offsets(int cb, int g, int li, int (&kt)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = (li >> 2) + 4 * h, q = li & 3;
    kt[h] = (8 * g + m) * 64 + (((2 * cb + (q >> 1)) ^ m) << 3) + 4 * (q & 1);
  }
}

// bf16x8 operand of 8 consecutive tokens (down a column) as floats.
__device__ __forceinline__ void widen8(const bf16x8& x, float (&o)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = (float)x[j];
}

}  // namespace
}  // namespace wkv6

#endif

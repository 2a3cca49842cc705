// RWKV-6 WKV forward for gfx950 (CDNA4): chunked evaluation on MFMA.
//
// The operator (include/wkv6.h) keeps, per (batch, head), a 64x64 fp32 state
// that decays by w_t = exp(-exp(w_raw_t)) along the key channel and gains
// k_t^T v_t every token; y_t reads r_t times the state plus the u-weighted
// current token.  Bidirectional mode adds the mirrored sum over strictly later
// tokens.  (CUDA-kernels page of deepglint/rwkv-clip, section "Forward Pass
// Implementation in kernel_forward"; "RWKV Architecture" page, sections
// "RWKV-5 Eagle" and "RWKV-6 Finch".)
//
// Sweeps.  The later-token sum of the bidirectional mode is the causal sum of
// the reversed sequence without the u term, so one sweep routine serves both
// directions: the reverse sweep runs over the tokens from the last one down
// and writes y, then the forward sweep adds its part (same workgroup, so the
// partial rows come back from the XCD's L2).  A causal call is the forward
// sweep alone.
//
// Chunked form.  A sweep takes its tokens in chunks of L = 64 (in sweep order;
// only the last chunk may be short).  With lambda = log2 of the decay
// (computed directly as -log2(e) exp(w_raw), never as the log of a rounded w)
// and Lin / Lex its inclusive / exclusive prefix sums over the chunk, every
// decay product the definition needs is a power of two of a difference of
// prefix sums (the log-space prefix-scan view of the "RWKV Architecture" page,
// section "The Parallel Training Formulation"):
//   earlier token i < t of the chunk:  2^(Lex_t - Lin_i)
//   state entering the chunk:          2^(Lex_t)            (scales r_t)
//   state leaving the chunk:           2^Ltot S + sum_i (k_i 2^(Ltot - Lin_i))^T v_i
//
// Fast path (every 16-token block of the chunk decays by less than 2^-24 in
// every channel, so the chunk by less than 2^-96): the in-chunk decay splits
// at the chunk start, keys k 2^(-Lin) and queries r 2^(Lex), so one query
// operand serves both the in-chunk scores and the state product, and the
// state update becomes 2^Ltot (S + (k 2^(-Lin))^T V) with the row scale
// applied to the fp32 accumulator.  Two exponentials per element.
// Slow path (some channel decays faster): the score tile of key block I
// splits at that block's end, 2^(Lex_t - E_I) 2^(E_I - Lin_i) with E_I the
// prefix at the end of block I; off the diagonal both factors are <= 1 and
// each is >= the true weight, so a factor only underflows where the weight is
// below 2^-126, and on the diagonal they stay within 2^(+-15 |lambda|).
// Valid for w_raw <= 1.5.  The fast kernels give up on an item at its first
// slow chunk and a fix-up kernel recomputes that item with the general
// sweeps (see the kernels at the end of this file).
//
// Segments.  When few (batch, head) pairs exist, each sequence is cut into G
// segments of whole chunks handled by different workgroups.  A summary pass
// sweeps each segment from a zero state and stores its end state and total
// log2 decay g per direction; each segment's sweep then starts from the
// combination of the earlier segments' summaries (in sweep order) under the
// associative rule (g1, S1) o (g2, S2) = (g1 + g2, 2^g2 S1 + S2).
//
// Precision.  Every contraction runs on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation.  An fp32 operand x is carried as SP bf16 parts (x = p0 + p1
// [+ p2], p_k the bf16 rounding of what the earlier parts leave), and a
// product keeps the part products p_i q_j with i + j < max(SP_a, SP_b).  bf16
// inputs use SP = 2 (v is an exact bf16 input and enters as one part); float32
// inputs use SP = 3 for every operand, v included.
//
// MFMA layouts (16x16x32, wave64; lane l, g = l / 16, i = l % 16):
//   A operand: row i, k-slots 8g..8g+7;  B operand: column i, same k-slots;
//   D: column i, rows 4g..4g+3.
// The k-slot -> k mapping only has to agree between A and B.  The scores
// feed the score x value product straight from their accumulators: slot
// 8g+j holds row 4g+j of the first D tile for j < 4 and row 4g+j-4 of the
// second for j >= 4, and the value operand is read from LDS in that order.
//
// Workgroup: 256 threads = 4 waves.  Wave J owns token block J (16 tokens) of
// the chunk: its lanes hold, for token 16J + i, channels {8g..8g+7,
// 32+8g..32+8g+7} -- exactly the query-operand slots of the MFMA B operand --
// so the prefix scan over tokens runs in registers (DPP row shifts inside each
// 16-lane row) and the query operands never touch LDS.  Wave J also owns
// state rows 16J..16J+15 (all 64 value columns); the state is exchanged
// through LDS once per chunk, pre-split.  LDS tiles are 64x64 bf16 planes
// whose 16-byte chunks are XOR-swizzled by row; a workgroup holds 41 KB of
// LDS (bf16 inputs), so three fit on a CU.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>
#include <mutex>
#include <vector>

#include "wkv6_device.h"
#include "wkv6_internal.h"

namespace wkv6 {
namespace {

struct Params {
  const void* r;
  const void* k;
  const void* v;
  const void* w;
  const float* u;
  float* y;
  float* summ;   // [B*H][G][direction]{S^T[64][64], g[64]} when G > 1
  const float* s_in;   // causal: state entering token 0, [B*H][64][64] (row c, column n), or null
  float* s_out;        // causal: state after the last token, same layout, or null
  int64_t T;
  int64_t C;
  int H;
  int G;      // segments per sequence
  int SEGC;   // chunks per segment (the last segment may be shorter)
  int w_static;   // w_raw is [C], the same decay for every token (RWKV-5; decode kernel)
  // fused epilogue (wkv6_fwd_gn): out = (GroupNorm(y) gamma + beta) gate, bf16
  uint16_t* out;
  const void* gate;     // [B, T, C], dtype of r
  const float* gamma;   // [C]
  const float* beta;    // [C]
  float eps;
  float* mark;          // one fix-up marker per (item, segment): y is not an output there
};

constexpr int kSummFloats = PL + HS;

enum SweepMode { kState = 0, kOut = 1, kOutAcc = 2 };

template <bool BF16>
struct SweepLds {
  static constexpr int SP = BF16 ? 2 : 3, SV = BF16 ? 1 : 3;
  static constexpr int kK = 0;                      // decayed keys [i][c]
  static constexpr int kV = kK + SP * PL * 2;       // V^T [n][t]
  static constexpr int kS = kV + SV * PL * 2;       // S^T [n][c]
  static constexpr int kBT = kS + SP * PL * 2;      // block totals [4][64]
  static constexpr int kU = kBT + 4 * 64 * 4;
  static constexpr int kFlag = kU + 64 * 4;
  static constexpr int kBytes = kFlag + 16;
  static constexpr int kGB = kBytes;                // fused epilogue: gamma[64], beta[64] of the head
  static constexpr int kBytesEpi = kGB + 128 * 4;
};



// Lane offsets into the swizzled planes, computed once per kernel so that
// every plane access is a per-lane base plus an immediate offset.
//   a[ks]     row li, 16-byte chunk 4 ks + g          (+1024 per 16 rows)
//   v[pr][h]  row li, 8 bytes at column 16 (2 pr + h) + 4 g
//   c[j]      row 8 g + j, column tau                  (+2048 per 32 rows)
//   kt[h]     row 8 g + li / 4 + 4 h, 8 bytes at column 16 J + 4 (li % 4)
//             (transposed reads, +2048 per 32 rows)
//   s         row li, 8 bytes at column 16 J + 4 g
struct LdsOff {
  int a[2];
  int v[2][2];
  int c[8];
  int kt[2];
  int s;
};

__device__ __forceinline__ LdsOff lds_offsets(int J, int g, int li) {
  LdsOff o;
  const int x = li & 7, tau = 16 * J + li;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) o.a[ks] = li * 64 + (((4 * ks + g) ^ x) << 3);
#pragma unroll
  for (int pr = 0; pr < 2; ++pr)
#pragma unroll
    for (int h = 0; h < 2; ++h) o.v[pr][h] = li * 64 + (((4 * pr + 2 * h + (g >> 1)) ^ x) << 3) + 4 * (g & 1);
#pragma unroll
  for (int j = 0; j < 8; ++j) o.c[j] = (8 * g + j) * 64 + ((((tau >> 3)) ^ j) << 3) + (tau & 7);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int m = (li >> 2) + 4 * h, q = li & 3;
    o.kt[h] = (8 * g + m) * 64 + (((2 * J + (q >> 1)) ^ m) << 3) + 4 * (q & 1);
  }
  o.s = li * 64 + (((2 * J + (g >> 1)) ^ x) << 3) + 4 * (g & 1);
  return o;
}

// ---- input rows: the 16 home elements of a lane (channels 8g.. and 32+8g..)
template <bool BF16>
struct Raw {
  uint4 q[BF16 ? 2 : 4];
};

// Gate values of the lane's output channels 16 nt + 4 g .. + 3, nt = 0..3,
// as loaded (bf16: 8 bytes per nt; fp32: 16 bytes).
template <bool BF16>
struct GateRaw {
  uint32_t q[4][BF16 ? 2 : 4];
};

template <bool BF16>
__device__ __forceinline__ GateRaw<BF16> load_gate(Rsrc rs, int off) {
  GateRaw<BF16> g;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if constexpr (BF16) {
      const auto q = __builtin_amdgcn_raw_buffer_load_b64(rs, off + 32 * nt, 0, 0);
      g.q[nt][0] = q[0];
      g.q[nt][1] = q[1];
    } else {
      const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 64 * nt, 0, 0);
      g.q[nt][0] = q[0];
      g.q[nt][1] = q[1];
      g.q[nt][2] = q[2];
      g.q[nt][3] = q[3];
    }
  }
  return g;
}

template <bool BF16>
__device__ __forceinline__ float gate_at(const GateRaw<BF16>& g, int nt, int j) {
  if constexpr (BF16)
    return __uint_as_float((j & 1) ? (g.q[nt][j >> 1] & 0xFFFF0000u) : (g.q[nt][j >> 1] << 16));
  else
    return __uint_as_float(g.q[nt][j]);
}

// Fused epilogue of one token row held by the four lanes of a 16-lane column
// (lane li + 16 g holds channels 16 nt + 4 g + j): per-head GroupNorm of y
// (mean and variance over the 64 channels, eps inside the square root), the
// per-channel affine gamma, beta, times the gate, rounded to bf16 (nearest
// even) and stored.  Lanes of a token past the segment store nothing
// (their byte offset lies outside the slice).
// Y is overwritten (its deviations from the row mean are formed in place, so
// that no second set of 16 registers is live at this peak of the sweep).
template <bool BF16>
__device__ __forceinline__ void gn_gate_store(f32x4 (&Y)[4], const GateRaw<BF16>& gt, const float* sGm,
                                              const float* sBt, int g, float eps, Rsrc ro, int ooff) {
  float s = 0.f;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) s += (Y[nt][0] + Y[nt][1]) + (Y[nt][2] + Y[nt][3]);
  const float mean = rows_sum(s) * (1.f / 64.f);
  float q = 0.f;
  f32x4 (&d)[4] = Y;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      d[nt][j] = Y[nt][j] - mean;
      q = fmaf(d[nt][j], d[nt][j], q);
    }
  const float rstd = __builtin_amdgcn_rsqf(fmaf(rows_sum(q), 1.f / 64.f, eps));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const float4 ga = *reinterpret_cast<const float4*>(sGm + 16 * nt + 4 * g);
    const float4 be = *reinterpret_cast<const float4*>(sBt + 16 * nt + 4 * g);
    const float o0 = fmaf(d[nt][0] * rstd, ga.x, be.x) * gate_at<BF16>(gt, nt, 0);
    const float o1 = fmaf(d[nt][1] * rstd, ga.y, be.y) * gate_at<BF16>(gt, nt, 1);
    const float o2 = fmaf(d[nt][2] * rstd, ga.z, be.z) * gate_at<BF16>(gt, nt, 2);
    const float o3 = fmaf(d[nt][3] * rstd, ga.w, be.w) * gate_at<BF16>(gt, nt, 3);
    const u32x2 w = {__builtin_bit_cast(uint32_t, round_pair(o0, o1)), __builtin_bit_cast(uint32_t, round_pair(o2, o3))};
    __builtin_amdgcn_raw_buffer_store_b64(w, ro, ooff + 32 * nt, 0, 0);
  }
}

// The lane's row: row_off is the row's byte offset in the slice.
template <bool BF16, int AUX = 0>
__device__ __forceinline__ Raw<BF16> gload(Rsrc rs, int row_off, int g) {
  Raw<BF16> r;
  if constexpr (BF16) {
    r.q[0] = bload16<AUX>(rs, row_off + 16 * g);
    r.q[1] = bload16<AUX>(rs, row_off + 64 + 16 * g);
  } else {
    r.q[0] = bload16<AUX>(rs, row_off + 32 * g);
    r.q[1] = bload16<AUX>(rs, row_off + 32 * g + 16);
    r.q[2] = bload16<AUX>(rs, row_off + 128 + 32 * g);
    r.q[3] = bload16<AUX>(rs, row_off + 128 + 32 * g + 16);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ void unpack(const Raw<BF16>& r, float (&o)[2][8]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if constexpr (BF16) {
      const uint4 q = r.q[ks];
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[ks][2 * j] = __uint_as_float(w4[j] << 16);
        o[ks][2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
      }
    } else {
      const uint4 a = r.q[2 * ks], b = r.q[2 * ks + 1];
      const uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) o[ks][j] = __uint_as_float(w8[j]);
    }
  }
}


// ---- prefix sums of the chunk for the lane's 16 home elements
//
// block_scan: lambda and its inclusive prefix inside the lane's 16-token block
// (DPP row shifts within each 16-lane row).  nl is -log2(e) for a token of the
// segment and 0 past it, so such tokens contribute lambda = 0 (their w_raw
// reads as 0).  Lane 15 of each row then holds the block totals,
// which go to sBT[J][c].  Block offsets and chunk totals are summed from sBT
// in block order everywhere, so an exclusive prefix and the preceding
// inclusive prefix are bit-identical.
template <bool BF16>
__device__ __forceinline__ void block_scan(const Raw<BF16>& rw, float nl, float (&lin)[2][8]) {
  float w[2][8];
  unpack<BF16>(rw, w);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = nl * ex2(w[ks][j] * kLog2e);
      x += row_shr<1>(x);
      x += row_shr<2>(x);
      x += row_shr<4>(x);
      x += row_shr<8>(x);
      lin[ks][j] = x;
    }
}

// Publish the block totals of wave J and whether any channel of the block
// decays by 2^-kBlockSpan or more (then the chunk takes the slow path).
__device__ __forceinline__ void publish_block(const float (&lin)[2][8], float* sBT, int* sFlag, int J, int g,
                                              int li, int lane) {
  float mn = lin[0][0];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) mn = fminf(mn, lin[ks][j]);
  const bool big = __any(li == 15 && mn < -kBlockSpan);
  if (li == 15) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; j += 4)
        *reinterpret_cast<float4*>(&sBT[J * 64 + 32 * ks + 8 * g + j]) =
            make_float4(lin[ks][j], lin[ks][j + 1], lin[ks][j + 2], lin[ks][j + 3]);
  }
  if (lane == 0) sFlag[J] = big ? 1 : 0;
}

// A wave whose 16 tokens all lie past the sequence end publishes zero totals.
__device__ __forceinline__ void publish_empty_block(float* sBT, int* sFlag, int J, int lane) {
  sBT[J * 64 + lane] = 0.f;
  if (lane == 0) sFlag[J] = 0;
}

__device__ __forceinline__ bool chunk_is_slow(const int* sFlag) {
  const int4 f = *reinterpret_cast<const int4*>(sFlag);
  return (f.x | f.y | f.z | f.w) != 0;
}

// Sum of the block totals before block J (the block's offset) for 8
// consecutive channels.
__device__ __forceinline__ void block_offset(const float* sBT, int J, int cb, float (&off)[8]) {
  if (J == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) off[j] = 0.f;
    return;
  }
  load8f(&sBT[cb], off);
#pragma unroll
  for (int I = 1; I < 3; ++I) {
    if (I < J) {
      float b[8];
      load8f(&sBT[I * 64 + cb], b);
#pragma unroll
      for (int j = 0; j < 8; ++j) off[j] += b[j];
    }
  }
}

// Prefix at the end of token block I (E_I) for 8 consecutive channels.
__device__ __forceinline__ void block_end8(const float* sBT, int I, int cb, float (&e)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) e[j] = 0.f;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    if (jj <= I) {
      float b[8];
      load8f(&sBT[jj * 64 + cb], b);
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] += b[j];
    }
  }
}

// Chunk totals (Ltot) of 4 consecutive channels.
__device__ __forceinline__ void chunk_total4(const float* sBT, int cb, float (&t)[4]) {
  float4 a = *reinterpret_cast<const float4*>(&sBT[cb]);
  t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w;
#pragma unroll
  for (int I = 1; I < 4; ++I) {
    a = *reinterpret_cast<const float4*>(&sBT[I * 64 + cb]);
    t[0] += a.x; t[1] += a.y; t[2] += a.z; t[3] += a.w;
  }
}

// Prefix at the end of token block I (E_I) for one channel.
__device__ __forceinline__ float block_end(const float* sBT, int I, int c) {
  float o = 0.f;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    if (jj <= I) o += sBT[jj * 64 + c];
  return o;
}

// ---- LDS clears for token blocks past the sequence end
// planes stored [row][t]: columns t0 .. t0 + 15 of all 64 rows
template <int S>
__device__ __forceinline__ void zero_cols16(__bf16* P, int t0, int lane) {
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int hq = 0; hq < 2; ++hq)
      *reinterpret_cast<uint4*>(P + s * PL + swz(lane, t0 + 8 * hq)) = make_uint4(0u, 0u, 0u, 0u);
}

// planes stored [t][col]: rows t0 .. t0 + 15, all 64 columns
template <int S>
__device__ __forceinline__ void zero_rows16(__bf16* P, int t0, int lane) {
  const int row = t0 + (lane >> 2), cb = 16 * (lane & 3);
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int hq = 0; hq < 2; ++hq)
      *reinterpret_cast<uint4*>(P + s * PL + swz(row, cb + 8 * hq)) = make_uint4(0u, 0u, 0u, 0u);
}

template <int S>
__device__ __forceinline__ void join8(const Op<S>& o, float (&x)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v = 0.f;
#pragma unroll
    for (int s = S - 1; s >= 0; --s) v += (float)o.p[s][j];
    x[j] = v;
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack_half(const Raw<BF16>& r, int ks, float (&o)[8]) {
  if constexpr (BF16) {
    const uint4 q = r.q[ks];
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[2 * j] = __uint_as_float(w4[j] << 16);
      o[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
    }
  } else {
    const uint4 a = r.q[2 * ks], b = r.q[2 * ks + 1];
    o[0] = __uint_as_float(a.x); o[1] = __uint_as_float(a.y);
    o[2] = __uint_as_float(a.z); o[3] = __uint_as_float(a.w);
    o[4] = __uint_as_float(b.x); o[5] = __uint_as_float(b.y);
    o[6] = __uint_as_float(b.z); o[7] = __uint_as_float(b.w);
  }
}

// V^T columns of the lane's token: element (32 ks + 8 g + j, tau) for its 16
// home channels.  bf16 values are stored as they were read.
template <bool BF16>
__device__ __forceinline__ void write_vT(__bf16* sV, const int (&c)[8], const Raw<BF16>& r) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if constexpr (BF16) {
      const uint4 q = r.q[ks];
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sV[2048 * ks + c[2 * j]] = __builtin_bit_cast(__bf16, (unsigned short)(w4[j] & 0xFFFFu));
        sV[2048 * ks + c[2 * j + 1]] = __builtin_bit_cast(__bf16, (unsigned short)(w4[j] >> 16));
      }
    } else {
      float v[8];
      unpack_half<BF16>(r, ks, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) wr1<3>(sV, 2048 * ks + c[j], v[j]);
    }
  }
}



// A chunk in which some 16-token block decays by 2^-kBlockSpan or more:
// phases B and C with references at the key blocks' own boundaries.  Past
// keys of block J carry k 2^(E_J - Lin) (E_I: prefix at the end of block I);
// the queries r 2^(Lex - E_I) of each key block and r 2^Lex of the state
// product are built in phase C from the raw r and w words.
// FIN: the final outputs go through the fused epilogue (gate rows at goff of
// rg, bf16 rows at ooff of ro) instead of y.
template <bool BF16, int MODE, bool DIAG, bool FIN = false>
__device__ __forceinline__ void slow_chunk(const Params& p, char* lds, Raw<BF16> rraw, Raw<BF16> kraw,
                                                     Raw<BF16> wraw, Rsrc ry, int yoff, int Lv, bool left,
                                                     Rsrc rg = Rsrc(), int goff = 0, Rsrc ro = Rsrc(), int ooff = 0) {
  constexpr int SP = BF16 ? 2 : 3;
  constexpr int SV = BF16 ? 1 : 3;
  constexpr bool OUT = MODE != kState;
  using L = SweepLds<BF16>;
  __bf16* sK = reinterpret_cast<__bf16*>(lds + L::kK);
  __bf16* sV = reinterpret_cast<__bf16*>(lds + L::kV);
  __bf16* sS = reinterpret_cast<__bf16*>(lds + L::kS);
  float* sBT = reinterpret_cast<float*>(lds + L::kBT);
  float* sU = reinterpret_cast<float*>(lds + L::kU);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tau = 16 * J + li;
  const LdsOff lo = lds_offsets(J, g, li);
  const float nl = tau < Lv ? -kLog2e : 0.f;
  const bool active = 16 * J < Lv;
  float lin[2][8];
  if (active) block_scan<BF16>(wraw, nl, lin);

  // ---- phase B (slow)
  float dg = 0.f;
  if (active) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cb = 32 * ks + 8 * g;
      float off[8], k[8], kf[8];
      block_offset(sBT, J, cb, off);
      unpack_half<BF16>(kraw, ks, k);
      float r[8], uu[8];
      if (DIAG) {
        unpack_half<BF16>(rraw, ks, r);
        load8f(&sU[cb], uu);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float eJ = off[j] + sBT[J * 64 + cb + j];
        kf[j] = k[j] * ex2(eJ - (lin[ks][j] + off[j]));
        if (DIAG) dg += r[j] * uu[j] * k[j];
      }
      wr8<SP>(sK, 1024 * J + lo.a[ks], kf);
    }
    if (DIAG) {
      dg += __shfl_xor(dg, 16);
      dg += __shfl_xor(dg, 32);
    }
  }
  lds_barrier();

  // ---- phase C (slow)
  if (OUT && active) {
    // Lin and Lex of the lane's elements, rebuilt from the raw w words
    float lns[2][8], lxs[2][8];
    block_scan<BF16>(wraw, nl, lns);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float off[8];
      block_offset(sBT, J, 32 * ks + 8 * g, off);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lxs[ks][j] = row_shr<1>(lns[ks][j]) + off[j];
        lns[ks][j] += off[j];
      }
    }
    f32x4 Y[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) Y[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (left) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float r[8], qv[8];
        unpack_half<BF16>(rraw, ks, r);
#pragma unroll
        for (int j = 0; j < 8; ++j) qv[j] = r[j] * ex2(lxs[ks][j]);
        const Op<SP> qo = split8<SP>(qv);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) Y[nt] = mma(rd8<SP>(sS, 1024 * nt + lo.a[ks]), qo, Y[nt]);
      }
    }
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
      const int I0 = 2 * pr;
      if (I0 > J) break;
      float mx[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int I = I0 + hh;
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (I <= J) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            float e[8], r[8], qv[8];
            block_end8(sBT, I, 32 * ks + 8 * g, e);
            unpack_half<BF16>(rraw, ks, r);
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[j] = r[j] * ex2(lxs[ks][j] - e[j]);
            a = mma(rd8<SP>(sK, 1024 * I + lo.a[ks]), split8<SP>(qv), a);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 16 * I + 4 * g + j;
          float val = (i < tau) ? a[j] : 0.f;
          if (DIAG) val += (i == tau) ? dg : 0.f;
          mx[4 * hh + j] = val;
        }
      }
      const Op<SP> mo = split8<SP>(mx);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        Y[nt] = mma(rd4x2<SV>(sV, 1024 * nt + lo.v[pr][0], 1024 * nt + lo.v[pr][1]), mo, Y[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      float4 o = make_float4(Y[nt][0], Y[nt][1], Y[nt][2], Y[nt][3]);
      if (MODE == kOutAcc) {
        const float4 yo = bloadf4(ry, yoff + 64 * nt);
        o.x += yo.x;
        o.y += yo.y;
        o.z += yo.z;
        o.w += yo.w;
      }
      if constexpr (FIN)
        Y[nt] = f32x4{o.x, o.y, o.z, o.w};
      else
        bstoref4(ry, yoff + 64 * nt, o.x, o.y, o.z, o.w);
    }
    if constexpr (FIN) {
      const float* sGm = reinterpret_cast<const float*>(lds + L::kGB);
      gn_gate_store<BF16>(Y, load_gate<BF16>(rg, goff), sGm, sGm + 64, g, p.eps, ro, ooff);
    }
  }
}

// ---------------------------------------------------------------------------
// One sweep of one segment in one direction.  Sweep position q runs over the
// segment's tokens in sweep order (REV: from its last token down), so the
// reverse sum of the bidirectional mode is the causal sum of the reversed
// sequence without the u term, and both directions share this code.
//   MODE kState:  no outputs; writes the segment's end state and total log2
//                 decay (started from zero) to the summaries.
//   MODE kOut:    y = the sweep's outputs.
//   MODE kOutAcc: y += the sweep's outputs (y holds the reverse sweep's part).
//   CARRY:        start from the state the earlier segments (in sweep order)
//                 hand over, combined from their summaries.
// Wave priority from the workgroup's progress through its item (done of
// total chunk steps).  Workgroups sharing a CU otherwise advance oldest
// first, and the last one finishes alone at low occupancy; lowering the
// priority of a workgroup as it gets ahead keeps them level.
__device__ __forceinline__ void progress_priority(int done, int total) {
  const int level = 3 - (4 * done) / total;
  if (level >= 3)
    __builtin_amdgcn_s_setprio(3);
  else if (level == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (level == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// npass / pass: the item's number of sweeps and this sweep's place among
// them (for progress_priority).
// WS: w_raw is one row of C values used for every token (RWKV-5).
// EPI: the sweep that produces the final outputs (the causal sweep, or the
// forward sweep of a bidirectional call) writes them through the fused
// GroupNorm / gate epilogue as bf16 instead of writing y.
// OCC only tells apart the instantiations of kernels allocated for
// different occupancies, so that each has its own copy of the sweep.
template <bool BF16, bool REV, int MODE, bool CARRY, bool SLOW, bool WS = false, bool EPI = false, int OCC = 0>
__device__ __forceinline__ bool sweep(const Params& p, char* lds, int bh, int seg, int npass = 1,
                                      int pass = 0) {
  constexpr int SP = BF16 ? 2 : 3;
  constexpr int SV = BF16 ? 1 : 3;
  constexpr bool OUT = MODE != kState;
  constexpr bool DIAG = OUT && !REV;   // the u term belongs to the forward sweep
  using L = SweepLds<BF16>;
  __bf16* sK = reinterpret_cast<__bf16*>(lds + L::kK);
  __bf16* sV = reinterpret_cast<__bf16*>(lds + L::kV);
  __bf16* sS = reinterpret_cast<__bf16*>(lds + L::kS);
  float* sBT = reinterpret_cast<float*>(lds + L::kBT);
  float* sU = reinterpret_cast<float*>(lds + L::kU);
  int* sFlag = reinterpret_cast<int*>(lds + L::kFlag);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tau = 16 * J + li;   // the lane's position in the chunk (also its output column)
  const LdsOff lo = lds_offsets(J, g, li);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const int64_t t_lo = (int64_t)seg * p.SEGC * LC;
  const int64_t t_hi = min(T, t_lo + (int64_t)p.SEGC * LC);
  const int64_t n = t_hi - t_lo;
  const int nch = (int)((n + LC - 1) / LC);
  // Sweep position q is token t_lo + q (REV: t_hi - 1 - q).  Byte offsets of
  // the lane's rows in chunk ch are row0 + ch * step (32-bit: slices stay
  // below 2^31 bytes).
  const int dir_rows = REV ? -1 : 1;
  const int tok0 = (int)(REV ? t_hi - 1 : t_lo) + dir_rows * tau;
  const int Ci = (int)C;

  if (DIAG && tid < 64) sU[tid] = p.u[h * HS + tid];   // read after the first barrier
  constexpr bool FIN = EPI && OUT && !REV;
  float* sGm = reinterpret_cast<float*>(lds + L::kGB);
  if (FIN && tid < 64) {
    sGm[tid] = p.gamma[h * HS + tid];
    sGm[64 + tid] = p.beta[h * HS + tid];
  }

  // ---- state, rows 16J + 4g + j, columns 16 nt + li
  f32x4 S[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool have_S = false;
  // causal calls may start from a given state (the forward sweep of a causal
  // call: MODE kOut and not REV; never a bidirectional call)
  constexpr bool CAUSAL_OUT = !REV && MODE == kOut;
  if (CAUSAL_OUT && p.s_in) {
    const float* si = p.s_in + (int64_t)bh * PL;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[nt][j] = si[(16 * J + 4 * g + j) * HS + 16 * nt + li];
    have_S = true;
  }
  if (CARRY) {
    // (g1, S1) o (g2, S2) = (g1 + g2, 2^g2 S1 + S2) over the earlier segments,
    // in sweep order.  The summaries are loaded kGrp at a time, every load of
    // a group issued before the first combine, so a group costs one memory
    // latency rather than kGrp.  Slots past the last summary re-read the last
    // one (addresses stay valid, loads stay unconditional) and are skipped.
    constexpr int kGrp = 4;
    const int nprev = REV ? p.G - 1 - seg : seg;
    for (int k0 = 0; k0 < nprev; k0 += kGrp) {
      const int cnt = min(kGrp, nprev - k0);
      float4 gl[kGrp], f[kGrp][4];
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        const int k2 = k0 + min(u, cnt - 1);
        const int s2 = REV ? p.G - 1 - k2 : k2;
        const float* Ss = p.summ + (((int64_t)bh * p.G + s2) * 2 + (REV ? 1 : 0)) * kSummFloats;
        gl[u] = *reinterpret_cast<const float4*>(Ss + PL + 16 * J + 4 * g);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          f[u][nt] = *reinterpret_cast<const float4*>(Ss + (16 * nt + li) * HS + 16 * J + 4 * g);
      }
#pragma unroll
      for (int u = 0; u < kGrp; ++u) {
        if (u >= cnt) break;   // uniform
        const float gj[4] = {ex2(gl[u].x), ex2(gl[u].y), ex2(gl[u].z), ex2(gl[u].w)};
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          S[nt][0] = S[nt][0] * gj[0] + f[u][nt].x;
          S[nt][1] = S[nt][1] * gj[1] + f[u][nt].y;
          S[nt][2] = S[nt][2] * gj[2] + f[u][nt].z;
          S[nt][3] = S[nt][3] * gj[3] + f[u][nt].w;
        }
      }
    }
    have_S = have_S || nprev > 0;
  }
  float gsum[4] = {0.f, 0.f, 0.f, 0.f};   // kState: total log2 decay of the state rows
  // the sweep that ends at the sequence's last token also updates the state
  // with the last chunk when the caller wants the final state
  const bool keep_state = CAUSAL_OUT && p.s_out && seg == p.G - 1;

  // The state entering a chunk goes to sS (pre-split) right after the chunk's
  // first barrier: every wave has then finished the previous chunk's phase C,
  // the last reader of sS, so phase D itself needs no barrier in front.
  auto publish_state = [&]() {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float x[4] = {S[nt][0], S[nt][1], S[nt][2], S[nt][3]};
      wr4<SP>(sS, 1024 * nt + lo.s, x);
    }
  };

  // Raw rows of the lane's token for the chunk: [0] r, [1] k, [2] v, [3] w.
  // The next chunk's loads are issued after the current chunk's outputs (the
  // other resident workgroups cover their latency); the loads are
  // unconditional, tokens past the segment reading zero.
  constexpr int ISZ = BF16 ? 2 : 4;
  const Rsrc rr = slice_rsrc(p.r, base, ISZ, T, C), rk = slice_rsrc(p.k, base, ISZ, T, C);
  const Rsrc rv = slice_rsrc(p.v, base, ISZ, T, C);
  // a static decay (RWKV-5) is one row per head: every token reads row 0
  const Rsrc rw = WS ? slice_rsrc(p.w, (int64_t)h * HS, ISZ, 1, C) : slice_rsrc(p.w, base, ISZ, T, C);
  const Rsrc ry = slice_rsrc(p.y, base, 4, T, C);
  // fused epilogue: gate rows (input dtype) and bf16 output rows, lane's channels 4g..
  const Rsrc rg = FIN ? slice_rsrc(p.gate, base, ISZ, T, C) : Rsrc();
  const Rsrc ro = FIN ? slice_rsrc(p.out, base, 2, T, C) : Rsrc();
  Raw<BF16> buf[4];
  // Byte offsets are formed in unsigned 32-bit arithmetic: a lane past the
  // segment's end may address up to 63 rows beyond the slice, past 2^31 at
  // the largest accepted T; such lanes use kOffNone instead, and every real
  // row's offset is below 2^31.
  const uint32_t utok = (uint32_t)tok0, uC = (uint32_t)Ci, udir = (uint32_t)dir_rows;
  const uint32_t in_row0 = utok * uC * ISZ, in_step = udir * LC * uC * ISZ;
  const uint32_t y_row0 = utok * uC * 4 + 16 * g, y_step = udir * LC * uC * 4;
  const uint32_t g_row0 = in_row0 + 4 * g * ISZ;                             // fused epilogue: gate rows
  const uint32_t o_row0 = utok * uC * 2 + 8 * g, o_step = udir * LC * uC * 2;   // and bf16 output rows
  // the offset of the lane's row in chunk ch, or kOffNone for a lane past the end
  auto at = [](bool ok, uint32_t row0, uint32_t step, int ch) {
    return ok ? (int)(row0 + (uint32_t)ch * step) : kOffNone;
  };
  auto fetch = [&](int ch) {
    // tokens past the segment read zero
    const bool in_seg = tau < (int)min<int64_t>(LC, n - (int64_t)ch * LC);
    const int off = at(in_seg, in_row0, in_step, ch);
    if (OUT) buf[0] = gload<BF16, CAUSAL_OUT ? kStream : 0>(rr, off, g);
    buf[1] = gload<BF16>(rk, off, g);
    buf[2] = gload<BF16>(rv, off, g);
    buf[3] = gload<BF16>(rw, WS ? (in_seg ? 0 : kOffNone) : off, g);
  };
  fetch(0);

  // Chunks run on the fast path until the first chunk that needs the slow
  // one; from there on every chunk takes the slow path (it is valid for any
  // chunk), so that neither loop carries the other's registers.
  int ch = 0;
  for (; ch < nch; ++ch) {
    const int Lv = (int)min<int64_t>(LC, n - (int64_t)ch * LC);
    const bool valid = tau < Lv;
    const bool active = 16 * J < Lv;   // uniform in the wave
    const bool left = ch > 0 || have_S;
    progress_priority(pass * nch + ch, npass * nch);
    lds_barrier();
    if (OUT && left) publish_state();

    // ---- phase A: in-block scan, block totals, values
    float lin[2][8];
    if (active) {
      block_scan<BF16>(buf[3], valid ? -kLog2e : 0.f, lin);
      publish_block(lin, sBT, sFlag, J, g, li, lane);
      write_vT<BF16>(sV, lo.c, buf[2]);
    } else {
      publish_empty_block(sBT, sFlag, J, lane);
      zero_cols16<SV>(sV, 16 * J, lane);
      zero_rows16<SP>(sK, 16 * J, lane);
    }
    lds_barrier();
    if (chunk_is_slow(sFlag)) break;   // uniform: every wave reads the same flags

    // ---- phase B (fast): keys k 2^(-Lin) to LDS; queries r 2^Lex split in
    // registers; bonus diagonal.
    Op<SP> q[2];
    float dg = 0.f;
    // byte offset of the lane's output row; lanes past the segment get an
    // offset outside every slice, so their loads read zero and their stores
    // are dropped without a branch
    const int yoff = at(valid, y_row0, y_step, ch);
    f32x4 Y[4];
    GateRaw<BF16> gt;
    if (OUT && active) {
      // the output accumulators start from the rows of y the reverse sweep
      // left (kOutAcc) or from zero; loaded here, a phase ahead of their use
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        Y[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (MODE == kOutAcc) {
          const float4 yo = bloadf4(ry, yoff + 64 * nt);
          Y[nt] = f32x4{yo.x, yo.y, yo.z, yo.w};
        }
      }
    }
    if (active) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int cb = 32 * ks + 8 * g;
        float off[8], k[8], kf[8];
        block_offset(sBT, J, cb, off);
        unpack_half<BF16>(buf[1], ks, k);
        float r[8], uu[8], qf[8];
        if (OUT) unpack_half<BF16>(buf[0], ks, r);
        if (DIAG) load8f(&sU[cb], uu);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kf[j] = k[j] * ex2(-(lin[ks][j] + off[j]));
          if (OUT) qf[j] = r[j] * ex2(row_shr<1>(lin[ks][j]) + off[j]);
          if (DIAG) dg += r[j] * uu[j] * k[j];
        }
        wr8<SP>(sK, 1024 * J + lo.a[ks], kf);
        if (OUT) q[ks] = split8<SP>(qf);
      }
      if (DIAG) {
        dg += __shfl_xor(dg, 16);
        dg += __shfl_xor(dg, 32);
      }
    }
    lds_barrier();

    // ---- phase C (fast): scores of the key blocks up to the lane's own,
    // outputs
    if (OUT && active) {
      // the gate rows for the fused epilogue, in flight during the products
      if (FIN) gt = load_gate<BF16>(rg, at(valid, g_row0, in_step, ch));
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        const int I0 = 2 * pr;
        if (I0 > J) break;
        float mx[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int I = I0 + hh;
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          if (I <= J) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) a = mma(rd8<SP>(sK, 1024 * I + lo.a[ks]), q[ks], a);
          }
          // every key of an earlier block keeps its score (a is zero for a
          // later block); in the query's own block only the keys before it
          // do, and its own key takes the bonus.  The lane masks depend on
          // j alone, so four of each serve every block.
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d = 4 * g + j - li;   // key minus query inside the block
            const float own = d < 0 ? a[j] : ((DIAG && d == 0) ? dg : 0.f);
            mx[4 * hh + j] = I == J ? own : a[j];
          }
        }
        const Op<SP> mo = split8<SP>(mx);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          Y[nt] = mma(rd4x2<SV>(sV, 1024 * nt + lo.v[pr][0], 1024 * nt + lo.v[pr][1]), mo, Y[nt]);
      }
      // Y^T += S^T (r 2^Lex)^T : state from the earlier chunks
      if (left) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) Y[nt] = mma(rd8<SP>(sS, 1024 * nt + lo.a[ks]), q[ks], Y[nt]);
      }
      if constexpr (FIN) {
        gn_gate_store<BF16>(Y, gt, sGm, sGm + 64, g, p.eps, ro, at(valid, o_row0, o_step, ch));
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          bstoref4<CAUSAL_OUT ? kStream : 0>(ry, yoff + 64 * nt, Y[nt][0], Y[nt][1], Y[nt][2], Y[nt][3]);
      }
    }
    // unconditional (past the end it reads zeros): with the fetch on one path
    // only, the compiler's waits where the paths meet covered these loads
    fetch(ch + 1);
    if (ch == nch - 1 && OUT && !keep_state) {
      ch = nch;
      break;
    }

    // ---- phase D: state rows 16J + 4g + j (registers only; sS is written
    // after the next barrier).  Keys are read down the columns of sK; fast:
    // S <- 2^Ltot (S + K^T V) with keys k 2^(-Lin); slow: the keys of token
    // block I are rescaled to k 2^(Ltot - Lin) and S <- 2^Ltot S + K^T V.
    float tot4[4], dec[4];
    chunk_total4(sBT, 16 * J + 4 * g, tot4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dec[j] = ex2(tot4[j]);
      if (!OUT) gsum[j] += tot4[j];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks >= Lv) break;
      const Op<SP> key = rdcol8<SP>(sK, lo.kt, 2048 * ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) S[nt] = mma(key, rd8<SV>(sV, 1024 * nt + lo.a[ks]), S[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[nt][j] *= dec[j];
  }


  // ch < nch here: a chunk needs the slow path
  if constexpr (!SLOW) {
    if (ch < nch) return false;
  } else {
    for (; ch < nch; ++ch) {
      const int Lv = (int)min<int64_t>(LC, n - (int64_t)ch * LC);
      const bool valid = tau < Lv;
      const bool active = 16 * J < Lv;   // uniform in the wave
      const bool left = ch > 0 || have_S;
      lds_barrier();
      if (OUT && left) publish_state();

      // ---- phase A: in-block scan, block totals, values
      float lin[2][8];
      if (active) {
        block_scan<BF16>(buf[3], valid ? -kLog2e : 0.f, lin);
        publish_block(lin, sBT, sFlag, J, g, li, lane);
        write_vT<BF16>(sV, lo.c, buf[2]);
      } else {
        publish_empty_block(sBT, sFlag, J, lane);
        zero_cols16<SV>(sV, 16 * J, lane);
        zero_rows16<SP>(sK, 16 * J, lane);
      }
      lds_barrier();

      slow_chunk<BF16, MODE, DIAG, FIN>(p, lds, buf[0], buf[1], buf[3], ry,
                                        at(valid, y_row0, y_step, ch), Lv, left, rg,
                                        at(valid, g_row0, in_step, ch), ro,
                                        at(valid, o_row0, o_step, ch));
      if (ch == nch - 1) {
        if (OUT && !keep_state) break;
      } else {
        fetch(ch + 1);
      }

      // ---- phase D (slow), registers only as above
      float tot4[4], dec[4];
      chunk_total4(sBT, 16 * J + 4 * g, tot4);
  #pragma unroll
      for (int j = 0; j < 4; ++j) {
        dec[j] = ex2(tot4[j]);
        if (!OUT) gsum[j] += tot4[j];
      }
  #pragma unroll
      for (int nt = 0; nt < 4; ++nt)
  #pragma unroll
        for (int j = 0; j < 4; ++j) S[nt][j] *= dec[j];
  #pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (32 * ks >= Lv) break;
        Op<SP> key = rdcol8<SP>(sK, lo.kt, 2048 * ks);
        // rows 32ks + 8g .. + 7 lie in token block I = 2ks + g / 2
        const int c = 16 * J + li;
        const int I = 2 * ks + (g >> 1);
        const float f = ex2(block_end(sBT, 3, c) - block_end(sBT, I, c));
        float x[8];
        join8<SP>(key, x);
  #pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= f;
        key = split8<SP>(x);
  #pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[nt] = mma(key, rd8<SV>(sV, 1024 * nt + lo.a[ks]), S[nt]);
      }
    }
  }

  if (!OUT) {
    float* dst = p.summ + (((int64_t)bh * p.G + seg) * 2 + (REV ? 1 : 0)) * kSummFloats;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<float4*>(dst + (16 * nt + li) * HS + 16 * J + 4 * g) =
          make_float4(S[nt][0], S[nt][1], S[nt][2], S[nt][3]);
    if (li == 0)
      *reinterpret_cast<float4*>(dst + PL + 16 * J + 4 * g) = make_float4(gsum[0], gsum[1], gsum[2], gsum[3]);
  }
  if (keep_state) {
    float* so = p.s_out + (int64_t)bh * PL;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) so[(16 * J + 4 * g + j) * HS + 16 * nt + li] = S[nt][j];
  }
  return true;
}

// ---------------------------------------------------------------------------
// Kernels.  One workgroup of 256 threads per (batch, head[, segment]).
// Bidirectional calls run the reverse sweep first (it writes y) and then the
// forward sweep (it adds its part to y) in the same workgroup, so the partial
// rows are read back from the L2 of the same XCD.
//
// bf16 items first run with the fast path alone (wkv_kernel),
// register-allocated for three resident workgroups per CU.  A workgroup that
// meets a chunk needing the slow path stops and leaves a marker in the first
// word of its output (y at the segment's first token and the head's first
// channel); the fix-up kernel launched next recomputes exactly the marked
// items with the general sweeps, which need more registers than the fast
// kernel has.  float32 sweeps carry the general sweeps themselves (see
// inline_slow).  (The summary kernels need no such split: see there.)
// A marker bit pattern produced by the arithmetic itself (a NaN input that
// propagates there) only costs a needless recomputation.
constexpr uint32_t kRedo = 0x7FC0D1A5u;   // quiet NaN with a payload

template <bool BF16>
constexpr int occupancy() {
  return BF16 ? 3 : 2;
}

template <bool EPI = false>
__device__ __forceinline__ float* item_marker(const Params& p, int bh, int seg) {
  if constexpr (EPI) return p.mark + (int64_t)bh * p.G + seg;   // the fused epilogue writes no y
  const int b = bh / p.H, h = bh % p.H;
  return p.y + ((int64_t)b * p.T + (int64_t)seg * p.SEGC * LC) * p.C + (int64_t)h * HS;
}

__device__ __forceinline__ void set_marker(float* m) {
  __syncthreads();   // the workgroup's earlier stores to this word are done
  if (threadIdx.x == 0) *reinterpret_cast<uint32_t*>(m) = kRedo;
}

__device__ __forceinline__ bool marker_set(const float* m) {
  return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(m)) == kRedo;
}

// Outputs of one item with the sweeps on the fast path (SLOW = false: false
// as soon as a chunk needs the slow path) or the general sweeps.
template <bool BF16, bool BIDIR, bool CARRY, bool SLOW, bool WS, bool EPI, int OCC = 0>
__device__ __forceinline__ bool run_item(const Params& p, char* lds, int bh, int seg) {
  if (BIDIR) {
    // the forward sweep runs even after the reverse one gave up (its result is
    // then recomputed anyway): one straight path keeps the registers of the
    // two sweeps apart
    const bool ok = sweep<BF16, true, kOut, CARRY, SLOW, WS, EPI, OCC>(p, lds, bh, seg, 2, 0);
    __syncthreads();   // partial rows of y written; LDS free for reuse
    return sweep<BF16, false, kOutAcc, CARRY, SLOW, WS, EPI, OCC>(p, lds, bh, seg, 2, 1) && ok;
  }
  return sweep<BF16, false, kOut, CARRY, SLOW, WS, EPI, OCC>(p, lds, bh, seg);
}

// float32 sweeps run at the fix-up kernel's occupancy (two workgroups per
// CU) already, and with the general sweeps inside they still fit its register
// budget without spills (resource report, gfx950): they carry them and need
// no fix-up launch.  bf16 sweeps keep the split (three workgroups per CU).
template <bool BF16>
constexpr bool inline_slow() {
  return !BF16;
}

// OCC: workgroups per CU the registers are allocated for.  A bf16
// bidirectional grid of at most two workgroups per CU runs a variant
// allocated for two: 192 VGPRs and no spills, where three per CU spill.
template <bool BF16, bool BIDIR, bool CARRY, bool WS, bool EPI, int OCC = occupancy<BF16>()>
__global__ __launch_bounds__(NT, OCC) void wkv_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char lds[EPI ? SweepLds<BF16>::kBytesEpi : SweepLds<BF16>::kBytes];
  const int bh = CARRY ? blockIdx.x / p.G : blockIdx.x, seg = CARRY ? blockIdx.x % p.G : 0;
  if (EPI && threadIdx.x == 0) *item_marker<EPI>(p, bh, seg) = 0.f;   // clear a marker left by an earlier call
  if (!run_item<BF16, BIDIR, CARRY, inline_slow<BF16>(), WS, EPI, OCC>(p, lds, bh, seg))
    set_marker(item_marker<EPI>(p, bh, seg));
}

template <bool BF16, bool BIDIR, bool CARRY, bool WS, bool EPI>
__global__ __launch_bounds__(NT, 2) void wkv_fixup_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char lds[EPI ? SweepLds<BF16>::kBytesEpi : SweepLds<BF16>::kBytes];
  const int bh = CARRY ? blockIdx.x / p.G : blockIdx.x, seg = CARRY ? blockIdx.x % p.G : 0;
  if (!marker_set(item_marker<EPI>(p, bh, seg))) return;
  run_item<BF16, BIDIR, CARRY, true, WS, EPI>(p, lds, bh, seg);
}

// Segment summaries of causal calls: the forward sweep's end state and total
// log2 decay of every segment but the last, from a zero state.  A segment
// with a chunk that needs the slow path is recomputed at once with the
// general sweep: without outputs it fits the same register budget, so no
// fix-up launch is needed.
template <bool BF16, bool WS>
__global__ __launch_bounds__(NT, occupancy<BF16>()) void summary_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char lds[SweepLds<BF16>::kBytes];
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  if (seg == p.G - 1) return;   // no later segment needs it
  if (!sweep<BF16, false, kState, false, false, WS>(p, lds, bh, seg)) {
    __syncthreads();   // every wave is done with the fast attempt's LDS
    sweep<BF16, false, kState, false, true, WS>(p, lds, bh, seg);
  }
}

// Both directions' summaries of one segment of a bidirectional call in one
// pass over its chunks in token order (fast path only: false at the first
// chunk that needs the slow path).
//   forward:  the state the causal sweep leaves, S <- 2^Ltot (S + (k 2^-Lin)^T V)
//             per chunk, exactly as sweep() computes it;
//   reverse:  the sweep from the segment's last token down leaves
//             sum_i 2^(E_i) k_i^T v_i, with E_i the log2 decay of the segment's
//             tokens before token i.  No term depends on another, so this sum
//             accumulates in the same pass, with keys k 2^(P + Lex) (P: the
//             decay of the segment's earlier chunks, Lex: the exclusive prefix
//             inside the chunk), every factor at most 1.
// Both share the loads, the scan and the value operands of each chunk.  The
// reverse keys take the place of the state planes and P that of the bonus
// row, neither of which a summary uses.
template <bool BF16, bool WS>
__device__ __forceinline__ bool summary_both(const Params& p, char* lds, int bh, int seg) {
  constexpr int SP = BF16 ? 2 : 3;
  constexpr int SV = BF16 ? 1 : 3;
  using L = SweepLds<BF16>;
  __bf16* sK = reinterpret_cast<__bf16*>(lds + L::kK);
  __bf16* sV = reinterpret_cast<__bf16*>(lds + L::kV);
  __bf16* sKr = reinterpret_cast<__bf16*>(lds + L::kS);
  float* sBT = reinterpret_cast<float*>(lds + L::kBT);
  float* sP = reinterpret_cast<float*>(lds + L::kU);
  int* sFlag = reinterpret_cast<int*>(lds + L::kFlag);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tau = 16 * J + li;
  const LdsOff lo = lds_offsets(J, g, li);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const int64_t t_lo = (int64_t)seg * p.SEGC * LC;
  const int64_t n = min(T, t_lo + (int64_t)p.SEGC * LC) - t_lo;
  const int nch = (int)((n + LC - 1) / LC);
  const int Ci = (int)C;
  if (tid < 64) sP[tid] = 0.f;   // read after the first barrier

  f32x4 S[4], R[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    R[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float gsum[4] = {0.f, 0.f, 0.f, 0.f};

  constexpr int ISZ = BF16 ? 2 : 4;
  const Rsrc rk = slice_rsrc(p.k, base, ISZ, T, C), rv = slice_rsrc(p.v, base, ISZ, T, C);
  const Rsrc rw = WS ? slice_rsrc(p.w, (int64_t)h * HS, ISZ, 1, C) : slice_rsrc(p.w, base, ISZ, T, C);
  // byte offsets in unsigned 32-bit arithmetic, as in sweep()
  const uint32_t in_row0 = (uint32_t)(t_lo + tau) * (uint32_t)Ci * ISZ, in_step = LC * (uint32_t)Ci * ISZ;
  Raw<BF16> buf[3];   // k, v, w rows of the lane's token
  auto fetch = [&](int ch) {
    const bool in_seg = tau < (int)min<int64_t>(LC, n - (int64_t)ch * LC);
    const int off = in_seg ? (int)(in_row0 + (uint32_t)ch * in_step) : kOffNone;
    buf[0] = gload<BF16>(rk, off, g);
    buf[1] = gload<BF16>(rv, off, g);
    buf[2] = gload<BF16>(rw, WS ? (in_seg ? 0 : kOffNone) : off, g);
  };
  fetch(0);

  for (int ch = 0; ch < nch; ++ch) {
    const int Lv = (int)min<int64_t>(LC, n - (int64_t)ch * LC);
    const bool valid = tau < Lv;
    const bool active = 16 * J < Lv;   // uniform in the wave
    progress_priority(ch, nch);
    lds_barrier();

    // ---- phase A: in-block scan, block totals, values
    float lin[2][8];
    if (active) {
      block_scan<BF16>(buf[2], valid ? -kLog2e : 0.f, lin);
      publish_block(lin, sBT, sFlag, J, g, li, lane);
      write_vT<BF16>(sV, lo.c, buf[1]);
    } else {
      publish_empty_block(sBT, sFlag, J, lane);
      zero_cols16<SV>(sV, 16 * J, lane);
      zero_rows16<SP>(sK, 16 * J, lane);
      zero_rows16<SP>(sKr, 16 * J, lane);
    }
    lds_barrier();
    if (chunk_is_slow(sFlag)) return false;   // uniform: every wave reads the same flags

    // ---- phase B: forward keys k 2^(-Lin), reverse keys k 2^(P + Lex)
    if (active) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int cb = 32 * ks + 8 * g;
        float off[8], k[8], pr[8], kf[8], kr[8];
        block_offset(sBT, J, cb, off);
        unpack_half<BF16>(buf[0], ks, k);
        load8f(&sP[cb], pr);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kf[j] = k[j] * ex2(-(lin[ks][j] + off[j]));
          kr[j] = k[j] * ex2(pr[j] + (row_shr<1>(lin[ks][j]) + off[j]));
        }
        wr8<SP>(sK, 1024 * J + lo.a[ks], kf);
        wr8<SP>(sKr, 1024 * J + lo.a[ks], kr);
      }
    }
    if (ch + 1 < nch) fetch(ch + 1);
    lds_barrier();   // keys written; every wave has read P for this chunk

    // ---- phase D: both states, rows 16J + 4g + j
    float tot4[4], dec[4];
    chunk_total4(sBT, 16 * J + 4 * g, tot4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dec[j] = ex2(tot4[j]);
      gsum[j] += tot4[j];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks >= Lv) break;
      const Op<SP> key = rdcol8<SP>(sK, lo.kt, 2048 * ks);
      const Op<SP> keyr = rdcol8<SP>(sKr, lo.kt, 2048 * ks);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const Op<SV> val = rd8<SV>(sV, 1024 * nt + lo.a[ks]);
        S[nt] = mma(key, val, S[nt]);
        R[nt] = mma(keyr, val, R[nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[nt][j] *= dec[j];
    // P of the next chunk (read there after two barriers)
    if (li == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sP[16 * J + 4 * g + j] += tot4[j];
    }
  }

#pragma unroll
  for (int d = 0; d < 2; ++d) {
    float* dst = p.summ + (((int64_t)bh * p.G + seg) * 2 + d) * kSummFloats;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const f32x4 x = d == 0 ? S[nt] : R[nt];
      *reinterpret_cast<float4*>(dst + (16 * nt + li) * HS + 16 * J + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
    }
    if (li == 0)
      *reinterpret_cast<float4*>(dst + PL + 16 * J + 4 * g) = make_float4(gsum[0], gsum[1], gsum[2], gsum[3]);
  }
  return true;
}

// Summaries of bidirectional calls, both directions per workgroup.  A
// segment with a chunk that needs the slow path is recomputed at once with
// the general sweeps, one direction after the other (the forward summary of
// the last segment and the reverse one of the first are never read).
template <bool BF16, bool WS>
__global__ __launch_bounds__(NT, occupancy<BF16>()) void summary_both_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char lds[SweepLds<BF16>::kBytes];
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  if (!summary_both<BF16, WS>(p, lds, bh, seg)) {
    __syncthreads();   // every wave is done with the fast attempt's LDS
    if (seg < p.G - 1) sweep<BF16, false, kState, false, true, WS>(p, lds, bh, seg);
    __syncthreads();
    if (seg > 0) sweep<BF16, true, kState, false, true, WS>(p, lds, bh, seg);
  }
}

// ---------------------------------------------------------------------------
// Segment summaries with the state split by rows (bf16 inputs, per-token
// decay).  The decay acts on the key channel c alone, so row c of a state
// never mixes with another row: wave J owns rows c = 16J .. 16J + 15 of both
// summaries for the whole segment, and the waves share nothing but the
// staged input tiles.  Per 64-token chunk (tokens in order, t local):
//   forward  S <- 2^Ltot S + sum_t (k_t 2^(Ltot - Lin_t))^T v_t
//   reverse  R <- R + sum_t (k_t 2^(P + Lex_t))^T v_t   (P: the segment's
//            decay before the chunk, so 2^(P + Lex_t) is the decay of the
//            segment's tokens before t)
// Every factor is at most 1, so no range guard or slow path is needed.  The
// products run as S^T[n][c] += sum_t V[t][n] eta[t][c] on MFMA: lane (g, i)
// of wave J holds channel c = 16J + i in all four accumulator tiles, so the
// per-channel row scaling 2^Ltot is a per-lane factor, and its operand slots
// (tokens 8g .. 8g + 7 of k-step ks) are where it scans lambda, in
// registers.  The k, v and w tiles are staged row-major in swizzled LDS
// planes (two buffers), read down their columns with transposed LDS reads;
// the next chunk's loads are issued as soon as the current chunk is staged,
// so they are in flight for a whole chunk step, and one barrier per chunk
// orders the staging.
//   BOTH: also the reverse summary (bidirectional calls); else the forward
//         one of every segment but the last (causal calls).
struct RowSummLds {
  static constexpr int kTile = PL * 2;            // one 64 x 64 bf16 plane
  static constexpr int kBuf = 3 * kTile;          // k, v, w
  static constexpr int kBytes = 2 * kBuf;         // two buffers
};


//   WS:   the decay is one bf16 value per channel for every token (RWKV-5):
//         each lane reads its channel's value once and uses it in place of
//         the staged w column, so the arithmetic, and the result, are those
//         of the per-token kernel given that value repeated.
template <bool BOTH, bool WS>
__global__ __launch_bounds__(NT, 3) void summary_rows_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char lds[RowSummLds::kBytes];
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  if (!BOTH && seg == p.G - 1) return;   // no later segment needs it
  const int tid = threadIdx.x, lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const int64_t t_lo = (int64_t)seg * p.SEGC * LC;
  const int64_t n = min(T, t_lo + (int64_t)p.SEGC * LC) - t_lo;
  const int nch = (int)((n + LC - 1) / LC);
  const Rsrc rk = slice_rsrc(p.k, base, 2, T, C), rv = slice_rsrc(p.v, base, 2, T, C);
  const Rsrc rw = slice_rsrc(p.w, WS ? (int64_t)h * HS : base, 2, WS ? 1 : T, C);
  const float w_ch = WS ? (float)reinterpret_cast<const __bf16*>(p.w)[h * HS + 16 * J + li] : 0.f;

  // staging: thread tid moves 16-byte pieces tid and tid + 256 of each tile
  // (row = piece / 8, 8-channel column group = piece % 8)
  int srow[2], scol[2], sdst[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int pc = tid + 256 * hh;
    srow[hh] = pc >> 3;
    scol[hh] = pc & 7;
    sdst[hh] = swz(srow[hh], 8 * scol[hh]);
  }
  const uint32_t row0 = (uint32_t)t_lo * (uint32_t)C * 2u, rstep = (uint32_t)C * 2u;
  uint4 stg[3][2];
  auto fetch = [&](int ch) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int t = ch * LC + srow[hh];   // rows outside the segment read zero
      const int off = t >= 0 && t < n ? (int)(row0 + (uint32_t)t * rstep) + 16 * scol[hh] : kOffNone;
      stg[0][hh] = bload16(rk, off);
      stg[1][hh] = bload16(rv, off);
      if (!WS) stg[2][hh] = bload16(rw, off);
    }
  };
  int ktJ[2], ktV[4][2];
  col_offsets(J, g, li, ktJ);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) col_offsets(nt, g, li, ktV[nt]);

  f32x4 S[4], R[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    R[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // BOTH: the segment's log2 decay before the chunk; else the decay after it
  // (the forward summary runs the chunks last to first), channel 16J + li
  float P = 0.f;
  const bool odd = (g & 1) != 0, upper = (g & 2) != 0;

  // chunk ch staged into buffer i (the two alternate); nx: the chunk to fetch
  // next (past either end it reads zeros)
  auto step = [&](int ch, int i, int nx) {
    char* buf = lds + i * RowSummLds::kBuf;
    // stage this chunk, then send the next chunk's loads out at once
#pragma unroll
    for (int ti = 0; ti < (WS ? 2 : 3); ++ti)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<uint4*>(buf + ti * RowSummLds::kTile + 2 * sdst[hh]) = stg[ti][hh];
    fetch(nx);
    lds_barrier();   // (the other buffer's readers finished before the previous barrier)
    const __bf16* sK = reinterpret_cast<const __bf16*>(buf);
    const __bf16* sV = reinterpret_cast<const __bf16*>(buf + RowSummLds::kTile);
    const __bf16* sW = reinterpret_cast<const __bf16*>(buf + 2 * RowSummLds::kTile);
    const int Lv = (int)min<int64_t>(LC, n - (int64_t)ch * LC);

    // lambda's inclusive (Lin) and exclusive (Lex) prefix over the chunk for
    // tokens 32 ks + 8 g + j of channel 16J + li (tokens past the segment
    // have lambda = 0)
    float lin[2][8], lex[2][8], tot = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float w8[8];
      if constexpr (WS) {
#pragma unroll
        for (int j = 0; j < 8; ++j) w8[j] = w_ch;
      } else {
        widen8(rdcol8<1>(sW, ktJ, 2048 * ks).p[0], w8);
      }
      float run = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 32 * ks + 8 * g + j;
        const float lam = t < Lv ? -kLog2e * ex2(w8[j] * kLog2e) : 0.f;
        lex[ks][j] = run;
        run += lam;
        lin[ks][j] = run;
      }
      // exclusive prefix of the four 8-token groups: rows g of the wave hold
      // the groups of one channel (permlane swaps with the row g ^ 1, g ^ 2)
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(run), __float_as_uint(run), false, false);
      const float partner = __uint_as_float(odd ? a[0] : a[1]);
      const float pair = run + partner;
      const auto c2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
      const float other = __uint_as_float(upper ? c2[0] : c2[1]);
      const float pre = tot + (odd ? partner : 0.f) + (upper ? other : 0.f);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lin[ks][j] += pre;
        lex[ks][j] += pre;
      }
      tot += pair + other;
    }

    // BOTH: S <- 2^tot S + (k 2^(tot - Lin))^T V;  R <- R + (k 2^(P + Lex))^T V.
    // Else, the chunks last to first: S <- S + (k 2^(P + tot - Lin))^T V,
    // every part decayed once to the segment's end.  The accumulator entries
    // of a lane all belong to its channel, so a decay is one factor per lane.
    if constexpr (BOTH) {
      const float dec = ex2(tot);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[nt][j] *= dec;
    }
    const float post = BOTH ? tot : P + tot;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks >= Lv) break;
      float k8[8], ef[8], er[8];
      widen8(rdcol8<1>(sK, ktJ, 2048 * ks).p[0], k8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ef[j] = k8[j] * ex2(post - lin[ks][j]);
        if (BOTH) er[j] = k8[j] * ex2(P + lex[ks][j]);
      }
      const Op<2> eo = split8<2>(ef);
      Op<2> ro;
      if (BOTH) ro = split8<2>(er);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const Op<1> vt = rdcol8<1>(sV, ktV[nt], 2048 * ks);
        S[nt] = mma(vt, eo, S[nt]);
        if (BOTH) R[nt] = mma(vt, ro, R[nt]);
      }
    }
    P += tot;
  };
  // The forward-only summary runs its chunks last to first: the ones it
  // reads last, a segment's first, are then the likeliest still to be in
  // the caches when the sweeps start there.
  if constexpr (BOTH) {
    fetch(0);
    for (int ch = 0; ch < nch; ++ch) step(ch, ch & 1, ch + 1);
  } else {
    fetch(nch - 1);
    for (int ch = nch - 1; ch >= 0; --ch) step(ch, ch & 1, ch - 1);
  }

  // S^T[n][c] (and R^T) with n = 16 nt + 4g + j, c = 16J + li; the segment's
  // total log2 decay of channel 16J + li from the lanes of row 0
#pragma unroll
  for (int d = 0; d < (BOTH ? 2 : 1); ++d) {
    float* dst = p.summ + (((int64_t)bh * p.G + seg) * 2 + d) * kSummFloats;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[(16 * nt + 4 * g + j) * HS + 16 * J + li] = d == 0 ? S[nt][j] : R[nt][j];
    if (g == 0) dst[PL + 16 * J + li] = P;
  }
}

// State passing through an empty sequence: s_out = s_in (zero without s_in).
__global__ __launch_bounds__(NT) void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                                       int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)gridDim.x * NT)
    dst[i] = src ? src[i] : 0.f;
}

// ---------------------------------------------------------------------------
// Causal calls of a few tokens (decoding): the recurrence itself, one token
// after the other, with the state in registers.  One workgroup per
// (batch, head); thread t holds state rows 4 (t / 16) .. + 3 at columns
// 4 (t % 16) .. + 3.  Per token: y_t[n] = sum_c r_t[c] S[c][n] + d_t v_t[n]
// with d_t = sum_c r_t[c] u[c] k_t[c] (partial sums over the thread's rows,
// combined across the 16 row groups through LDS), then
// S[c][n] <- w_t[c] S[c][n] + k_t[c] v_t[n] (as S + kv - (1 - w) S).  fp32
// throughout.
constexpr int kDecodeMaxT = 4;

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (BF16) {
    const uint16_t b = static_cast<const uint16_t*>(p)[i];
    return __uint_as_float((uint32_t)b << 16);
  } else {
    return static_cast<const float*>(p)[i];
  }
}

template <bool BF16>
__global__ __launch_bounds__(NT) void decode_kernel(Params p) {
  __shared__ float sPart[NT / 64][HS];   // per wave: partial y over its row groups
  __shared__ float sBonus;
  const int bh = blockIdx.x;
  const int b = bh / p.H, h = bh % p.H;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = 4 * (t & 15), c0 = 4 * (t >> 4);
  float S[4][4];   // S[i][j] = state row c0 + i, column n0 + j
  if (p.s_in) {
    const float* si = p.s_in + (int64_t)bh * PL;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 q = *reinterpret_cast<const float4*>(si + (c0 + i) * HS + n0);
      S[i][0] = q.x; S[i][1] = q.y; S[i][2] = q.z; S[i][3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = 0.f;
  }
  const float ul = p.u[h * HS + lane];
  for (int tok = 0; tok < p.T; ++tok) {
    const int64_t row = ((int64_t)b * p.T + tok) * p.C + (int64_t)h * HS;
    // dl = 1 - w = -expm1(-exp(w_raw)): the state decays as S - dl S, so a
    // decay within 1e-4 of 1 keeps its full precision over many calls (a
    // product with w rounded to float32 would bias a long-memory state)
    float r[4], k[4], dl[4], v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = load_elem<BF16>(p.r, row + c0 + i);
      k[i] = load_elem<BF16>(p.k, row + c0 + i);
      dl[i] = -expm1f(-ex2(load_elem<BF16>(p.w, (p.w_static ? (int64_t)h * HS : row) + c0 + i) * kLog2e));
      v[i] = load_elem<BF16>(p.v, row + n0 + i);
    }
    // partial y over the thread's four rows, summed over the row groups of
    // the wave (lanes 16 apart share the columns)
    float yp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) a = fmaf(r[i], S[i][j], a);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      yp[j] = a;
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sPart[wave][n0 + j] = yp[j];
    }
    if (wave == 0) {
      // d = sum_c r[c] u[c] k[c] over the head's 64 channels (lane = c)
      float d = load_elem<BF16>(p.r, row + lane) * ul * load_elem<BF16>(p.k, row + lane);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) d += __shfl_xor(d, m);
      if (lane == 0) sBonus = d;
    }
    __syncthreads();
    if (wave == 0) {
      float y = sBonus * load_elem<BF16>(p.v, row + lane);
#pragma unroll
      for (int wv = 0; wv < NT / 64; ++wv) y += sPart[wv][lane];
      p.y[row + lane] = y;
    }
    __syncthreads();   // sPart and sBonus are reused by the next token
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = fmaf(-dl[i], S[i][j], fmaf(k[i], v[j], S[i][j]));
  }
  if (p.s_out) {
    float* so = p.s_out + (int64_t)bh * PL;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(so + (c0 + i) * HS + n0) = make_float4(S[i][0], S[i][1], S[i][2], S[i][3]);
  }
}

struct Plan {
  int NC, G, SEGC;
};

Plan plan(const FwdArgs& a) {
  Plan pl;
  pl.NC = (int)((a.T + LC - 1) / LC);
  const int64_t bh = a.B * a.H;
  int G = 1;
  if (const char* e = getenv("WKV6_SEGMENTS")) {
    G = atoi(e);
  } else {
    // enough workgroups to fill every CU at the kernel's occupancy
    const int64_t target = 256 * (a.bf16 ? 3 : 2);
    if (bh < target) G = (int)((target + bh - 1) / bh);
    // bf16: a grid that gives every CU the same number of workgroups, three
    // or else two, wins over a fuller but uneven one (segments are whole
    // chunks, so the count above can round to, say, 704 workgroups: two on
    // some CUs, three on others).  Measured at T = 4096: 64 pairs in 8
    // segments against 11 (bidirectional 153.6 against 158.2 us, causal 88.8
    // against 90.5), 32 pairs in 16 against 22 (86.6 against 100.7, 58.8
    // against 67.2); 128 pairs stay at 6 segments (768 workgroups), which
    // beat 4 (281 against 296 us).
    if (a.bf16 && bh < target) {
      for (int per = 3; per >= 2; --per) {
        const int64_t want = 256 * per;
        if (want % bh != 0) continue;
        const int64_t g0 = want / bh;
        if (g0 > pl.NC) continue;
        const int64_t segc = (pl.NC + g0 - 1) / g0;
        if ((pl.NC + segc - 1) / segc == g0) {
          G = (int)g0;
          break;
        }
      }
    }
  }
  G = max(1, min(G, pl.NC));
  pl.SEGC = (pl.NC + G - 1) / G;
  pl.G = (pl.NC + pl.SEGC - 1) / pl.SEGC;
  return pl;
}

// Workspace: [segment summaries (G > 1)] [fused epilogue, bidirectional: the
// reverse sweep's fp32 rows, B*T*C] [fused epilogue: one marker per item and
// segment], each part 256-byte aligned.
struct WsLayout {
  size_t summ, ypart, mark, total;
};

WsLayout ws_layout(const FwdArgs& a, const Plan& pl) {
  auto up = [](size_t n) { return (n + 255) & ~size_t(255); };
  WsLayout l;
  l.summ = 0;
  size_t n = pl.G > 1 ? up((size_t)a.B * a.H * pl.G * 2 * kSummFloats * sizeof(float)) : 0;
  l.ypart = n;
  if (a.epi && a.bidirectional) n += up((size_t)a.B * a.T * a.C * sizeof(float));
  l.mark = n;
  if (a.epi) n += up((size_t)a.B * a.H * pl.G * sizeof(float));
  l.total = n;
  return l;
}

template <bool BF16, bool BIDIR, bool WS, bool EPI>
hipError_t launch_t(const FwdArgs& a, const Plan& pl, void* ws, hipStream_t s) {
  Params p;
  p.r = a.r;
  p.k = a.k;
  p.v = a.v;
  p.w = a.w_raw;
  p.u = a.u;
  p.y = a.y;
  p.summ = static_cast<float*>(ws);
  p.s_in = a.s_in;
  p.s_out = a.s_out;
  p.T = a.T;
  p.C = a.C;
  p.H = (int)a.H;
  p.G = pl.G;
  p.SEGC = pl.SEGC;
  p.w_static = a.w_static ? 1 : 0;
  p.out = a.out;
  p.gate = a.gate;
  p.gamma = a.gamma;
  p.beta = a.beta;
  p.eps = a.eps;
  p.mark = nullptr;
  if (EPI) {
    const WsLayout l = ws_layout(a, pl);
    char* wsb = static_cast<char*>(ws);
    p.y = BIDIR ? reinterpret_cast<float*>(wsb + l.ypart) : nullptr;   // the reverse sweep's rows
    p.mark = reinterpret_cast<float*>(wsb + l.mark);
  }
  const unsigned bh = (unsigned)(a.B * a.H);
  const dim3 block(NT);
  hipError_t e;
  if (pl.G > 1) {
    const dim3 sgrid(bh * pl.G);
    if constexpr (BF16)   // bf16 rows: the row-split summaries
      hipLaunchKernelGGL((summary_rows_kernel<BIDIR, WS>), sgrid, block, 0, s, p);
    else if constexpr (BIDIR)
      hipLaunchKernelGGL((summary_both_kernel<BF16, WS>), sgrid, block, 0, s, p);
    else
      hipLaunchKernelGGL((summary_kernel<BF16, WS>), sgrid, block, 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const dim3 grid(bh * pl.G);
  constexpr bool kSplit = !inline_slow<BF16>();   // a fix-up launch follows
  // a bf16 bidirectional grid of at most two workgroups per CU: the variant
  // with their registers (the causal sweeps fit three per CU unspilled)
  constexpr bool kTwo = BF16 && BIDIR && !EPI;
  const bool two = kTwo && grid.x <= 2u * 256u;
  if (pl.G > 1) {
    if constexpr (kTwo) {
      if (two)
        hipLaunchKernelGGL((wkv_kernel<BF16, BIDIR, true, WS, EPI, 2>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((wkv_kernel<BF16, BIDIR, true, WS, EPI>), grid, block, 0, s, p);
    } else {
      hipLaunchKernelGGL((wkv_kernel<BF16, BIDIR, true, WS, EPI>), grid, block, 0, s, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (kSplit) hipLaunchKernelGGL((wkv_fixup_kernel<BF16, BIDIR, true, WS, EPI>), grid, block, 0, s, p);
  } else {
    if constexpr (kTwo) {
      if (two)
        hipLaunchKernelGGL((wkv_kernel<BF16, BIDIR, false, WS, EPI, 2>), grid, block, 0, s, p);
      else
        hipLaunchKernelGGL((wkv_kernel<BF16, BIDIR, false, WS, EPI>), grid, block, 0, s, p);
    } else {
      hipLaunchKernelGGL((wkv_kernel<BF16, BIDIR, false, WS, EPI>), grid, block, 0, s, p);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (kSplit) hipLaunchKernelGGL((wkv_fixup_kernel<BF16, BIDIR, false, WS, EPI>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

template <bool BF16, bool WS, bool EPI>
hipError_t launch_ws(const FwdArgs& a, const Plan& pl, void* ws, hipStream_t s) {
  return a.bidirectional ? launch_t<BF16, true, WS, EPI>(a, pl, ws, s)
                         : launch_t<BF16, false, WS, EPI>(a, pl, ws, s);
}

// Workspace of wkv6_fwd_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
__device__ __align__(256) char scratch[kScratchBytes];

hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace

size_t workspace_bytes(const FwdArgs& a) {
  if (a.B == 0 || a.T == 0 || (!a.bidirectional && !a.epi && a.T <= kDecodeMaxT)) return 0;
  return ws_layout(a, plan(a)).total;
}

hipError_t enqueue_fwd_noalloc(const FwdArgs& a, hipStream_t stream) {
  if (a.epi || a.s_in || a.s_out || a.w_static) return hipErrorInvalidValue;   // plain forward only
  if (a.T == 0 || a.B == 0) return hipSuccess;
  if (!a.bidirectional && a.T <= kDecodeMaxT) return enqueue_fwd(a, nullptr, stream);   // no workspace
  // the planner's segment count, lowered until the summaries fit the scratch
  Plan pl = plan(a);
  while (ws_layout(a, pl).total > kScratchBytes && pl.G > 1) {
    const int G = pl.G - 1;
    pl.SEGC = (pl.NC + G - 1) / G;
    pl.G = (pl.NC + pl.SEGC - 1) / pl.SEGC;
  }
  if (ws_layout(a, pl).total > kScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  if (a.bf16) return launch_ws<true, false, false>(a, pl, ws, stream);
  return launch_ws<false, false, false>(a, pl, ws, stream);
}

hipError_t enqueue_fwd(const FwdArgs& a, void* workspace, hipStream_t stream) {
  if (a.T == 0) {
    if (!a.s_out) return hipSuccess;
    const int64_t n = a.B * a.H * PL;
    const int64_t nblk = (n + NT - 1) / NT;
    const unsigned grid = (unsigned)(nblk < 1024 ? nblk : 1024);
    hipLaunchKernelGGL(state_copy_kernel, dim3(grid), dim3(NT), 0, stream, a.s_in, a.s_out, n);
    return hipGetLastError();
  }
  if (!a.bidirectional && !a.epi && a.T <= kDecodeMaxT) {
    Params p{};
    p.r = a.r;
    p.k = a.k;
    p.v = a.v;
    p.w = a.w_raw;
    p.u = a.u;
    p.y = a.y;
    p.s_in = a.s_in;
    p.s_out = a.s_out;
    p.T = a.T;
    p.C = a.C;
    p.H = (int)a.H;
    p.w_static = a.w_static ? 1 : 0;
    const dim3 grid((unsigned)(a.B * a.H));
    if (a.bf16)
      hipLaunchKernelGGL(decode_kernel<true>, grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL(decode_kernel<false>, grid, dim3(NT), 0, stream, p);
    return hipGetLastError();
  }
  const Plan pl = plan(a);
  // variants: plain, static decay (RWKV-5), fused epilogue (never both)
  if (a.bf16) {
    if (a.epi) return launch_ws<true, false, true>(a, pl, workspace, stream);
    return a.w_static ? launch_ws<true, true, false>(a, pl, workspace, stream)
                      : launch_ws<true, false, false>(a, pl, workspace, stream);
  }
  if (a.epi) return launch_ws<false, false, true>(a, pl, workspace, stream);
  return a.w_static ? launch_ws<false, true, false>(a, pl, workspace, stream)
                    : launch_ws<false, false, false>(a, pl, workspace, stream);
}

}  // namespace wkv6

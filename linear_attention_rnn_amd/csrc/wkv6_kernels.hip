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
// Chunked form.  Tokens are processed in chunks of L = 64.  With lambda = log2
// of the decay (computed directly as -log2(e) exp(w_raw), never as the log of
// a rounded w) and Lin / Lex its inclusive / exclusive prefix sums over the
// chunk, every decay product the definition needs is a power of two of a
// difference of prefix sums (the log-space prefix-scan view of the "RWKV
// Architecture" page, section "The Parallel Training Formulation"):
//   past token i < t of the chunk:   2^(Lex_t - Lin_i)
//   later token i > t of the chunk:  2^(Lex_i - Lin_t)
//   state entering from the left:    2^(Lex_t)           (scales r_t)
//   state entering from the right:   2^(Ltot - Lin_t)
//   state leaving to the right:      2^Ltot S + sum_i (k_i 2^(Ltot - Lin_i))^T v_i
//   state leaving to the left:       2^Ltot S + sum_i (k_i 2^(Lex_i))^T v_i
//
// Fast path (chunk span |Ltot| < 96 for every channel): the in-chunk decay
// splits at the chunk start, keys k 2^(-Lin) and queries r 2^(Lex) (and
// k 2^(Lex - Ltot), r 2^(Ltot - Lin) for later tokens), so one query operand
// serves both the in-chunk scores and the state product, and the state update
// becomes 2^Ltot (S + (k 2^(-Lin))^T V) with the row scale applied to the fp32
// accumulator.  Two exponentials per element.
// Slow path (some channel decays by more than 2^-96 over the chunk): the
// score tile of key block I (16 tokens) splits at that block's boundary,
// 2^(Lex_t - E_I) 2^(E_I - Lin_i) for i < t with E_I the prefix at the end of
// block I, and 2^(B_I - Lin_t) 2^(Lex_i - B_I) for i > t with B_I the prefix
// before block I.  Off the diagonal both factors are <= 1 and each is >= the
// true weight, so a factor only underflows where the weight is below 2^-126;
// on the diagonal they stay within 2^(+-15 |lambda|).  Valid for w_raw <= 1.5.
// The choice is made per chunk, uniformly for the workgroup.
//
// Segments.  When few (batch, head) pairs exist, each sequence is cut into G
// segments of whole chunks handled by different workgroups.  seg_kernel
// sweeps each segment from its last chunk to its first and writes (a) the
// state each chunk receives from the later chunks of its own segment
// (bidirectional mode) and (b) per segment the forward end state F, the
// backward start state R and the total log2 decay g (G > 1).  fwd_kernel
// combines the other segments' summaries with the associative rule
// (g1, S1) o (g2, S2) = (g1 + g2, 2^g2 S1 + S2) and sweeps its segment.
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
// whose 16-byte chunks are XOR-swizzled by row.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdlib>

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

struct Params {
  const void* r;
  const void* k;
  const void* v;
  const void* w;
  const float* u;
  float* y;
  __bf16* rev;   // [B*H][NC][SP planes][64 n][64 c]: state from the later chunks of the segment
  float* summ;   // [B*H][G]{F^T[64][64], R^T[64][64], g[64]} when G > 1
  int64_t T;
  int64_t C;
  int H;
  int NC;   // chunks per sequence
  int CPS;  // chunks per segment
  int G;    // segments per sequence
};

constexpr int kSummFloats = 2 * PL + HS;

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 of the decay: log2(exp(-exp(w_raw))) = -log2(e) exp(w_raw).
__device__ __forceinline__ float log2_decay(float w_raw) { return -kLog2e * ex2(w_raw * kLog2e); }

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

template <int S>
__device__ __forceinline__ Op<S> split8(const float* x) {
  Op<S> o;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float r = x[j];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const __bf16 h = (__bf16)r;
      o.p[s][j] = h;
      r -= (float)h;
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
__device__ __forceinline__ Op<S> lds_read8(const __bf16* P, int row, int col0) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) o.p[s] = *reinterpret_cast<const bf16x8*>(P + s * PL + swz(row, col0));
  return o;
}

// slots 0..3 from columns c0..c0+3, slots 4..7 from columns c1..c1+3
template <int S>
__device__ __forceinline__ Op<S> lds_read4x2(const __bf16* P, int row, int c0, int c1) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(P + s * PL + swz(row, c0));
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(P + s * PL + swz(row, c1));
    o.p[s] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return o;
}

template <int S>
__device__ __forceinline__ void lds_write8(__bf16* P, int row, int col0, const float* x) {
  const Op<S> o = split8<S>(x);
#pragma unroll
  for (int s = 0; s < S; ++s) *reinterpret_cast<bf16x8*>(P + s * PL + swz(row, col0)) = o.p[s];
}

template <int S>
__device__ __forceinline__ void lds_write4(__bf16* P, int row, int col0, const float* x) {
  float r[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    bf16x4 q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 h = (__bf16)r[j];
      q[j] = h;
      r[j] -= (float)h;
    }
    *reinterpret_cast<bf16x4*>(P + s * PL + swz(row, col0)) = q;
  }
}

template <int S>
__device__ __forceinline__ void lds_write1(__bf16* P, int row, int col, float x) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const __bf16 h = (__bf16)x;
    P[s * PL + swz(row, col)] = h;
    x -= (float)h;
  }
}

// Lane offsets into the swizzled planes, computed once per kernel so that
// every plane access is a per-lane base plus an immediate offset.
//   a[ks]     row li, 16-byte chunk 4 ks + g          (+1024 per 16 rows)
//   v[pr][h]  row li, 8 bytes at column 16 (2 pr + h) + 4 g
//   c[j]      row 8 g + j, column tau                  (+2048 per 32 rows)
//   s         row li, 8 bytes at column 16 J + 4 g
struct LdsOff {
  int a[2];
  int v[2][2];
  int c[8];
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
  o.s = li * 64 + (((2 * J + (g >> 1)) ^ x) << 3) + 4 * (g & 1);
  return o;
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

// k-slot j from offset add + c[j] (a column read down 8 stored rows)
template <int S>
__device__ __forceinline__ Op<S> rdcol8(const __bf16* P, const int (&c)[8], int add) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) o.p[s][j] = P[s * PL + add + c[j]];
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
    for (int j = 0; j < 4; ++j) {
      const __bf16 h = (__bf16)r[j];
      q[j] = h;
      r[j] -= (float)h;
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

// ---- split planes in global memory (row-major, unswizzled)
template <int S>
__device__ __forceinline__ Op<S> gl_read8(const __bf16* P, int row, int col0) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) o.p[s] = *reinterpret_cast<const bf16x8*>(P + s * PL + row * 64 + col0);
  return o;
}

template <int S>
__device__ __forceinline__ void gl_write4(__bf16* P, int row, int col0, const float* x) {
  float r[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
  for (int s = 0; s < S; ++s) {
    bf16x4 q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const __bf16 h = (__bf16)r[j];
      q[j] = h;
      r[j] -= (float)h;
    }
    *reinterpret_cast<bf16x4*>(P + s * PL + row * 64 + col0) = q;
  }
}

// ---- input rows: the 16 home elements of a lane (channels 8g.. and 32+8g..)
template <bool BF16>
struct Raw {
  uint4 q[BF16 ? 2 : 4];
};

template <bool BF16>
__device__ __forceinline__ Raw<BF16> gload(const void* base, int64_t row_off, int g) {
  Raw<BF16> r;
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + row_off;
    r.q[0] = *reinterpret_cast<const uint4*>(p + 8 * g);
    r.q[1] = *reinterpret_cast<const uint4*>(p + 32 + 8 * g);
  } else {
    const float* p = static_cast<const float*>(base) + row_off;
    r.q[0] = *reinterpret_cast<const uint4*>(p + 8 * g);
    r.q[1] = *reinterpret_cast<const uint4*>(p + 8 * g + 4);
    r.q[2] = *reinterpret_cast<const uint4*>(p + 32 + 8 * g);
    r.q[3] = *reinterpret_cast<const uint4*>(p + 32 + 8 * g + 4);
  }
  return r;
}

template <bool BF16>
__device__ __forceinline__ Raw<BF16> rzero() {
  Raw<BF16> r;
#pragma unroll
  for (int i = 0; i < (BF16 ? 2 : 4); ++i) r.q[i] = make_uint4(0u, 0u, 0u, 0u);
  return r;
}

// Zero the raw words of a row that lies past the end of the sequence (the
// loads themselves are unconditional: they read a clamped, valid row).
template <bool BF16>
__device__ __forceinline__ void mask_row(Raw<BF16>& r, bool valid) {
#pragma unroll
  for (int i = 0; i < (BF16 ? 2 : 4); ++i) {
    r.q[i].x = valid ? r.q[i].x : 0u;
    r.q[i].y = valid ? r.q[i].y : 0u;
    r.q[i].z = valid ? r.q[i].z : 0u;
    r.q[i].w = valid ? r.q[i].w : 0u;
  }
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

__device__ __forceinline__ void load8f(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// ---- prefix sums of the chunk for the lane's 16 home elements
//
// block_scan: lambda and its inclusive prefix inside the lane's 16-token block
// (DPP row shifts within each 16-lane row; lanes past the sequence end
// contribute lambda = 0).  Lane 15 of each row then holds the block totals,
// which go to sBT[J][c].  Block offsets and chunk totals are summed from sBT
// in block order everywhere, so an exclusive prefix and the preceding
// inclusive prefix are bit-identical.
template <bool BF16>
__device__ __forceinline__ void block_scan(const Raw<BF16>& rw, bool valid, float (&lin)[2][8]) {
  float w[2][8];
  unpack<BF16>(rw, w);
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float x = valid ? log2_decay(w[ks][j]) : 0.f;
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
  bool big = false;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) big |= lin[ks][j] < -kBlockSpan;
  big = __any(li == 15 && big);
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
#pragma unroll
  for (int j = 0; j < 8; ++j) off[j] = 0.f;
#pragma unroll
  for (int I = 0; I < 3; ++I) {
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

// Column read of a split plane set: k-slots j = 0..7 are rows r0 + j of
// column col (an A operand whose K dimension runs down the stored rows).
template <int S>
__device__ __forceinline__ Op<S> lds_read_col8(const __bf16* P, int r0, int col) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int j = 0; j < 8; ++j) o.p[s][j] = P[s * PL + swz(r0 + j, col)];
  return o;
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

// ---------------------------------------------------------------------------
// Segment pre-pass: one workgroup per (batch, head, segment); sweeps the
// segment's chunks from last to first.  The state each chunk receives from
// the later chunks of its segment is stored split, multiplied by the chunk's
// own total decay 2^Ltot when the chunk takes the fast path (the forward
// kernel then pairs it with the query r 2^(-Lin)), unscaled otherwise.
template <bool BF16, bool BIDIR, bool CARRY>
__global__ __launch_bounds__(NT, BF16 ? 2 : 1) void seg_kernel(Params p) {
  constexpr int SP = BF16 ? 2 : 3;
  constexpr int SV = BF16 ? 1 : 3;
  __shared__ __attribute__((aligned(16))) __bf16 sEb[BIDIR ? SP * PL : 8];   // (k 2^Lex)^T   [c][t]
  __shared__ __attribute__((aligned(16))) __bf16 sEf[CARRY ? SP * PL : 8];   // (k 2^(Ltot-Lin+D))^T
  __shared__ __attribute__((aligned(16))) __bf16 sV[SV * PL];                 // V^T [n][t]
  __shared__ __attribute__((aligned(16))) float sBT[4 * 64];
  __shared__ __attribute__((aligned(16))) int sFlag[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tau = 16 * J + li;
  const LdsOff lo = lds_offsets(J, g, li);
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const int c0 = seg * p.CPS;
  const int c1 = min(p.NC, c0 + p.CPS);   // chunks [c0, c1)

  f32x4 Sb[4], F[4];   // rows 16J + 4g + j, columns 16 nt + li
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) Sb[nt] = F[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float D[2][8];       // log2 decay from the end of the current chunk to the segment end
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) D[ks][j] = 0.f;

  // buffers: [0] k, [1] v, [2] w.  Loads are unconditional (rows clamped to
  // the sequence) so the compiler can keep them in flight across the chunk.
  auto fetch = [&](int ch, Raw<BF16> (&buf)[3]) {
    const int64_t t = min((int64_t)ch * LC + tau, T - 1);
    const int64_t off = base + t * C;
    buf[0] = gload<BF16>(p.k, off, g);
    buf[1] = gload<BF16>(p.v, off, g);
    buf[2] = gload<BF16>(p.w, off, g);
  };

  auto body = [&](int ch, Raw<BF16> (&cur)[3], Raw<BF16> (&nxt)[3]) __attribute__((always_inline)) {
    const int Lv = (int)min<int64_t>(LC, T - (int64_t)ch * LC);
    const bool valid = tau < Lv;
    const bool active = 16 * J < Lv;   // uniform in the wave
    lds_barrier();
    fetch(max(ch - 1, c0), nxt);

    // ---- phase A: scan, block totals, values
    float lin[2][8];
    if (active) {
      if (Lv < LC) {
#pragma unroll
        for (int i = 0; i < 3; ++i) mask_row<BF16>(cur[i], valid);
      }
      block_scan<BF16>(cur[2], valid, lin);
      publish_block(lin, sBT, sFlag, J, g, li, lane);
      float v[8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        unpack_half<BF16>(cur[1], ks, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) wr1<SV>(sV, 2048 * ks + lo.c[j], v[j]);
      }
    } else {
      publish_empty_block(sBT, sFlag, J, lane);
      zero_cols16<SV>(sV, 16 * J, lane);
      if (BIDIR) zero_cols16<SP>(sEb, 16 * J, lane);
      if (CARRY) zero_cols16<SP>(sEf, 16 * J, lane);
    }
    lds_barrier();

    // ---- phase B: decayed keys, stored transposed
    const bool slow = chunk_is_slow(sFlag);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int cb = 32 * ks + 8 * g;
      float tot[8];
      if (CARRY) {
        float4 t0, t1;
        t0 = *reinterpret_cast<const float4*>(&sBT[cb]);
        t1 = *reinterpret_cast<const float4*>(&sBT[cb + 4]);
        tot[0] = t0.x; tot[1] = t0.y; tot[2] = t0.z; tot[3] = t0.w;
        tot[4] = t1.x; tot[5] = t1.y; tot[6] = t1.z; tot[7] = t1.w;
#pragma unroll
        for (int I = 1; I < 4; ++I) {
          float bb[8];
          load8f(&sBT[I * 64 + cb], bb);
#pragma unroll
          for (int j = 0; j < 8; ++j) tot[j] += bb[j];
        }
      }
      if (active) {
        float off[8], k[8];
        block_offset(sBT, J, cb, off);
        unpack_half<BF16>(cur[0], ks, k);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (BIDIR) wr1<SP>(sEb, 2048 * ks + lo.c[j], k[j] * ex2(row_shr<1>(lin[ks][j]) + off[j]));
          if (CARRY) wr1<SP>(sEf, 2048 * ks + lo.c[j], k[j] * ex2(tot[j] - (lin[ks][j] + off[j]) + D[ks][j]));
        }
      }
      if (CARRY) {
#pragma unroll
        for (int j = 0; j < 8; ++j) D[ks][j] += tot[j];
      }
    }
    lds_barrier();

    // ---- phase D: state rows 16J + 4g + j
    float tot4[4], dec[4];
    chunk_total4(sBT, 16 * J + 4 * g, tot4);
#pragma unroll
    for (int j = 0; j < 4; ++j) dec[j] = ex2(tot4[j]);
    // state each chunk receives from the later chunks of the segment
    if (BIDIR && ch < c1 - 1) {
      __bf16* dst = p.rev + ((int64_t)bh * p.NC + ch) * (SP * PL);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = slow ? Sb[nt][j] : Sb[nt][j] * dec[j];
        gl_write4<SP>(dst, 16 * nt + li, 16 * J + 4 * g, x);
      }
    }
    // Sb <- 2^Ltot Sb + (k 2^Lex)^T V ;  F += (k 2^(Ltot - Lin + D))^T V
    if (BIDIR) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) Sb[nt][j] *= dec[j];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      if (32 * ks >= Lv) break;
      Op<SP> eb, ef;
      if (BIDIR) eb = rd8<SP>(sEb, 1024 * J + lo.a[ks]);
      if (CARRY) ef = rd8<SP>(sEf, 1024 * J + lo.a[ks]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const Op<SV> vb = rd8<SV>(sV, 1024 * nt + lo.a[ks]);
        if (BIDIR) Sb[nt] = mma(eb, vb, Sb[nt]);
        if (CARRY) F[nt] = mma(ef, vb, F[nt]);
      }
    }
  };

  Raw<BF16> X[3], Y[3];
  fetch(c1 - 1, X);
  for (int ch = c1 - 1; ch >= c0; ch -= 2) {
    body(ch, X, Y);
    if (ch - 1 >= c0) body(ch - 1, Y, X);
  }

  if (CARRY) {
    float* dst = p.summ + ((int64_t)bh * p.G + seg) * kSummFloats;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int n = 16 * nt + li;
      *reinterpret_cast<float4*>(dst + n * HS + 16 * J + 4 * g) = make_float4(F[nt][0], F[nt][1], F[nt][2], F[nt][3]);
      *reinterpret_cast<float4*>(dst + PL + n * HS + 16 * J + 4 * g) =
          make_float4(Sb[nt][0], Sb[nt][1], Sb[nt][2], Sb[nt][3]);
    }
    if (J == 0 && li == 0) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[2 * PL + 32 * ks + 8 * g + j] = D[ks][j];
    }
  }
}

// ---------------------------------------------------------------------------
// Main sweep: outputs of one segment, left to right.
template <bool BF16, bool BIDIR, bool CARRY>
__global__ __launch_bounds__(NT, BF16 ? 2 : 1) void fwd_kernel(Params p) {
  constexpr int SP = BF16 ? 2 : 3;
  constexpr int SV = BF16 ? 1 : 3;
  constexpr bool RIN = BIDIR && CARRY;
  __shared__ __attribute__((aligned(16))) __bf16 sKf[SP * PL];              // keys, past tokens [i][c]
  __shared__ __attribute__((aligned(16))) __bf16 sKb[BIDIR ? SP * PL : 8];  // keys, later tokens [i][c]
  __shared__ __attribute__((aligned(16))) __bf16 sV[SV * PL];               // V^T [n][t]
  __shared__ __attribute__((aligned(16))) __bf16 sS[SP * PL];               // S^T [n][c]
  __shared__ __attribute__((aligned(16))) __bf16 sSr[BIDIR ? SP * PL : 8];  // S'^T [n][c] entering this chunk
  __shared__ __attribute__((aligned(16))) float sBT[4 * 64];
  __shared__ __attribute__((aligned(16))) float sU[64];
  __shared__ __attribute__((aligned(16))) int sFlag[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int tau = 16 * J + li;   // home token of the lane (also its output column)
  const LdsOff lo = lds_offsets(J, g, li);
  const int bh = blockIdx.x / p.G, seg = blockIdx.x % p.G;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const int c0 = seg * p.CPS;
  const int c1 = min(p.NC, c0 + p.CPS);

  if (tid < 64) sU[tid] = p.u[h * HS + tid];   // read after the first barrier

  // ---- carries from the other segments
  f32x4 S[4];   // S[16J + 4g + j][16 nt + li]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // State from the later segments, for the staging elements of this thread
  // (row tid / 4, columns 16 (tid % 4) .. + 15 of S'^T), and the log2 decay
  // from the current chunk's start to the end of this segment for those columns.
  float Rr[RIN ? 16 : 1], rf[RIN ? 16 : 1];
#pragma unroll
  for (int j = 0; j < (RIN ? 16 : 1); ++j) Rr[j] = rf[j] = 0.f;
  const int srow = tid >> 2, scol = 16 * (tid & 3);
  bool have_S = false, have_R = false;
  if (CARRY) {
    const float* sm = p.summ + (int64_t)bh * p.G * kSummFloats;
    for (int s2 = 0; s2 < seg; ++s2) {
      const float* Fs = sm + (int64_t)s2 * kSummFloats;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float4 f = *reinterpret_cast<const float4*>(Fs + (16 * nt + li) * HS + 16 * J + 4 * g);
        const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) S[nt][j] = S[nt][j] * ex2(Fs[2 * PL + 16 * J + 4 * g + j]) + fv[j];
      }
    }
    have_S = seg > 0;
    if (have_S) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const float x[4] = {S[nt][0], S[nt][1], S[nt][2], S[nt][3]};
        wr4<SP>(sS, 1024 * nt + lo.s, x);
      }
    }
    if (RIN) {
      have_R = seg < p.G - 1;
      if (have_R) {
        for (int s2 = p.G - 1; s2 > seg; --s2) {
          const float* Rs = sm + (int64_t)s2 * kSummFloats + PL;
          const float* gs = sm + (int64_t)s2 * kSummFloats + 2 * PL;
#pragma unroll
          for (int j = 0; j < (RIN ? 16 : 1); ++j) Rr[j] = Rr[j] * ex2(gs[scol + j]) + Rs[srow * HS + scol + j];
        }
        const float* gseg = sm + (int64_t)seg * kSummFloats + 2 * PL;
#pragma unroll
        for (int j = 0; j < (RIN ? 16 : 1); ++j) rf[j] = gseg[scol + j];
      }
    }
  }

  // Per-chunk global data: [0] r, [1] k, [2] v, [3] w rows of the lane's home
  // token, and 2 SP 16-byte pieces of the chunk's reverse-state tile (thread t
  // holds row t / 4, columns 16 (t % 4) .. + 15 of each plane).  The next
  // chunk's loads are issued once the current chunk's operands are built and
  // stay in flight through the contractions.  Rows and chunks are clamped to
  // valid memory so the loads are unconditional.
  struct Buf {
    Raw<BF16> in[4];
    uint4 sr[BIDIR ? 2 * SP : 1];
  };
  auto fetch = [&](int ch, Buf& buf) {
    const int64_t t = min((int64_t)ch * LC + tau, T - 1);
    const int64_t off = base + t * C;
    buf.in[0] = gload<BF16>(p.r, off, g);
    buf.in[1] = gload<BF16>(p.k, off, g);
    buf.in[2] = gload<BF16>(p.v, off, g);
    buf.in[3] = gload<BF16>(p.w, off, g);
    if constexpr (BIDIR) {
      const __bf16* src = p.rev + ((int64_t)bh * p.NC + ch) * (SP * PL) + srow * 64 + scol;
#pragma unroll
      for (int s = 0; s < SP; ++s) {
        buf.sr[2 * s] = *reinterpret_cast<const uint4*>(src + s * PL);
        buf.sr[2 * s + 1] = *reinterpret_cast<const uint4*>(src + s * PL + 8);
      }
    }
  };
  Buf buf;
  fetch(c0, buf);

  for (int ch = c0; ch < c1; ++ch) {
    const int64_t s0 = (int64_t)ch * LC;
    const int Lv = (int)min<int64_t>(LC, T - s0);
    const bool valid = tau < Lv;
    const bool active = 16 * J < Lv;   // uniform in the wave
    const bool left = ch > c0 || have_S;
    const bool right = BIDIR && (ch < c1 - 1 || have_R);
    lds_barrier();

    // ---- phase A: in-block scan, block totals, values
    float lin[2][8];
    if (active) {
      if (Lv < LC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) mask_row<BF16>(buf.in[i], valid);
      }
      block_scan<BF16>(buf.in[3], valid, lin);
      publish_block(lin, sBT, sFlag, J, g, li, lane);
      float v[8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        unpack_half<BF16>(buf.in[2], ks, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) wr1<SV>(sV, 2048 * ks + lo.c[j], v[j]);
      }
    } else {
      publish_empty_block(sBT, sFlag, J, lane);
      zero_cols16<SV>(sV, 16 * J, lane);
      zero_rows16<SP>(sKf, 16 * J, lane);
      if (BIDIR) zero_rows16<SP>(sKb, 16 * J, lane);
    }
    lds_barrier();

    const bool slow = chunk_is_slow(sFlag);
    // ---- phase B0: state entering this chunk from the right: the later
    // chunks of the segment (prefetched, pre-split) plus, with segments, R of
    // the later segments decayed to this chunk
    if (BIDIR) {
      if (!RIN || !have_R) {
        if (ch < c1 - 1) {
#pragma unroll
          for (int s = 0; s < SP; ++s) {
            *reinterpret_cast<uint4*>(sSr + s * PL + swz(srow, scol)) = buf.sr[2 * s];
            *reinterpret_cast<uint4*>(sSr + s * PL + swz(srow, scol + 8)) = buf.sr[2 * s + 1];
          }
        }
      } else {
        float x[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) x[j] = 0.f;
        if (ch < c1 - 1) {
#pragma unroll
          for (int s = 0; s < SP; ++s)
#pragma unroll
            for (int hq = 0; hq < 2; ++hq) {
              const uint4 q = buf.sr[2 * s + hq];
              const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                x[8 * hq + 2 * j] += __uint_as_float(w4[j] << 16);
                x[8 * hq + 2 * j + 1] += __uint_as_float(w4[j] & 0xFFFF0000u);
              }
            }
        }
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float t2[4];
          chunk_total4(sBT, scol + 4 * q4, t2);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int jj = 4 * q4 + j;
            // fast: the query carries 2^(-Lin), so R enters with the decay from
            // the chunk start; slow: the query carries 2^(Ltot - Lin)
            const float before = rf[jj];
            rf[jj] -= t2[j];
            x[jj] += ex2(slow ? rf[jj] : before) * Rr[jj];
          }
        }
        lds_write8<SP>(sSr, srow, scol, x);
        lds_write8<SP>(sSr, srow, scol + 8, x + 8);
      }
    }

    if (!slow) {
      // ---- phase B (fast): keys k 2^(-Lin) (past) and k 2^Lex (later) to LDS;
      // queries r 2^Lex and r 2^(-Lin) kept split in registers; bonus diagonal
      Op<SP> rq[2], rbq[2];
      float dg = 0.f;
      if (active) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int cb = 32 * ks + 8 * g;
          float off[8], r[8], k[8], uu[8];
          block_offset(sBT, J, cb, off);
          unpack_half<BF16>(buf.in[0], ks, r);
          unpack_half<BF16>(buf.in[1], ks, k);
          load8f(&sU[cb], uu);
          float kf[8], kb[8], qf[8], qb[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float Fc = ex2(-(lin[ks][j] + off[j]));
            const float Ec = ex2(row_shr<1>(lin[ks][j]) + off[j]);
            kf[j] = k[j] * Fc;
            kb[j] = k[j] * Ec;
            qf[j] = r[j] * Ec;
            qb[j] = r[j] * Fc;
            dg += r[j] * uu[j] * k[j];
          }
          wr8<SP>(sKf, 1024 * J + lo.a[ks], kf);
          if (BIDIR) wr8<SP>(sKb, 1024 * J + lo.a[ks], kb);
          rq[ks] = split8<SP>(qf);
          if (BIDIR) rbq[ks] = split8<SP>(qb);
        }
        dg += __shfl_xor(dg, 16);
        dg += __shfl_xor(dg, 32);
      }
      fetch(min(ch + 1, c1 - 1), buf);
      lds_barrier();

      // ---- phase C (fast): scores, outputs
      if (active) {
        f32x4 Y[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) Y[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int I0 = 2 * pr;
          if ((!BIDIR && I0 > J) || 16 * I0 >= Lv) break;
          float mx[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int I = I0 + hh;
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
            if (16 * I < Lv) {
              if (I <= J) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) a = mma(rd8<SP>(sKf, 1024 * I + lo.a[ks]), rq[ks], a);
              }
              if (BIDIR && I >= J) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) a2 = mma(rd8<SP>(sKb, 1024 * I + lo.a[ks]), rbq[ks], a2);
              }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 16 * I + 4 * g + j;
              float val;
              if (I < J) val = a[j];
              else if (I > J) val = a2[j];
              else val = i < tau ? a[j] : (i > tau ? a2[j] : dg);
              mx[4 * hh + j] = val;
            }
          }
          const Op<SP> mo = split8<SP>(mx);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            Y[nt] = mma(rd4x2<SV>(sV, 1024 * nt + lo.v[pr][0], 1024 * nt + lo.v[pr][1]), mo, Y[nt]);
        }
        // Y^T += S^T (r 2^Lex)^T : state from the left
        if (left) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              Y[nt] = mma(rd8<SP>(sS, 1024 * nt + lo.a[ks]), rq[ks], Y[nt]);
        }
        // Y^T += S'^T (r 2^(-Lin))^T : state from the right (carries 2^Ltot)
        if (right) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
              Y[nt] = mma(rd8<SP>(sSr, 1024 * nt + lo.a[ks]), rbq[ks], Y[nt]);
        }
        if (valid) {
          float* yrow = p.y + base + (s0 + tau) * C;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            *reinterpret_cast<float4*>(yrow + 16 * nt + 4 * g) = make_float4(Y[nt][0], Y[nt][1], Y[nt][2], Y[nt][3]);
        }
      }
    } else {
      // ---- phase B (slow): each key block I uses references at its own
      // boundaries: past keys k 2^(E_J - Lin) with queries r 2^(Lex - E_I),
      // later keys k 2^(Lex - B_J) with queries r 2^(B_I - Lin).  The state
      // products use r 2^Lex and r 2^(Ltot - Lin).  All queries are built in
      // phase C from the raw r and w words, so the next chunk's loads wait
      // until phase C is done.
      float dg = 0.f;
      if (active) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int cb = 32 * ks + 8 * g;
          float off[8], r[8], k[8], uu[8];
          block_offset(sBT, J, cb, off);
          unpack_half<BF16>(buf.in[0], ks, r);
          unpack_half<BF16>(buf.in[1], ks, k);
          load8f(&sU[cb], uu);
          float kf[8], kb[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = cb + j;
            const float lin_c = lin[ks][j] + off[j];
            const float lex_c = row_shr<1>(lin[ks][j]) + off[j];
            const float eJ = off[j] + sBT[J * 64 + c];
            kf[j] = k[j] * ex2(eJ - lin_c);
            kb[j] = k[j] * ex2(lex_c - off[j]);
            dg += r[j] * uu[j] * k[j];
          }
          wr8<SP>(sKf, 1024 * J + lo.a[ks], kf);
          if (BIDIR) wr8<SP>(sKb, 1024 * J + lo.a[ks], kb);
        }
        dg += __shfl_xor(dg, 16);
        dg += __shfl_xor(dg, 32);
      }
      lds_barrier();

      // ---- phase C (slow)
      if (active) {
        // Lin and Lex of the lane's elements, rebuilt from the raw w words
        float lns[2][8], lxs[2][8];
        block_scan<BF16>(buf.in[3], valid, lns);
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
        // state products: S^T (r 2^Lex)^T and S'^T (r 2^(Ltot - Lin))^T
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float r[8], q[8];
          unpack_half<BF16>(buf.in[0], ks, r);
          if (left) {
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = r[j] * ex2(lxs[ks][j]);
            const Op<SP> qo = split8<SP>(q);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) Y[nt] = mma(rd8<SP>(sS, 1024 * nt + lo.a[ks]), qo, Y[nt]);
          }
          if (right) {
            float tot[8];
            block_end8(sBT, 3, 32 * ks + 8 * g, tot);
#pragma unroll
            for (int j = 0; j < 8; ++j) q[j] = r[j] * ex2(tot[j] - lns[ks][j]);
            const Op<SP> qo = split8<SP>(q);
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) Y[nt] = mma(rd8<SP>(sSr, 1024 * nt + lo.a[ks]), qo, Y[nt]);
          }
        }
        // score tiles, key block by key block
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const int I0 = 2 * pr;
          if ((!BIDIR && I0 > J) || 16 * I0 >= Lv) break;
          float mx[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int I = I0 + hh;
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, a2 = {0.f, 0.f, 0.f, 0.f};
            if (16 * I < Lv) {
              if (I <= J) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                  float e[8], r[8], q[8];
                  block_end8(sBT, I, 32 * ks + 8 * g, e);
                  unpack_half<BF16>(buf.in[0], ks, r);
#pragma unroll
                  for (int j = 0; j < 8; ++j) q[j] = r[j] * ex2(lxs[ks][j] - e[j]);
                  a = mma(rd8<SP>(sKf, 1024 * I + lo.a[ks]), split8<SP>(q), a);
                }
              }
              if (BIDIR && I >= J) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                  float e[8], r[8], q[8];
                  if (I) {
                    block_end8(sBT, I - 1, 32 * ks + 8 * g, e);
                  } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = 0.f;
                  }
                  unpack_half<BF16>(buf.in[0], ks, r);
#pragma unroll
                  for (int j = 0; j < 8; ++j) q[j] = r[j] * ex2(e[j] - lns[ks][j]);
                  a2 = mma(rd8<SP>(sKb, 1024 * I + lo.a[ks]), split8<SP>(q), a2);
                }
              }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 16 * I + 4 * g + j;
              float val = (i < tau) ? a[j] : 0.f;
              if (BIDIR) val += (i > tau) ? a2[j] : 0.f;
              val += (i == tau) ? dg : 0.f;
              mx[4 * hh + j] = val;
            }
          }
          const Op<SP> mo = split8<SP>(mx);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            Y[nt] = mma(rd4x2<SV>(sV, 1024 * nt + lo.v[pr][0], 1024 * nt + lo.v[pr][1]), mo, Y[nt]);
        }
        if (valid) {
          float* yrow = p.y + base + (s0 + tau) * C;
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            *reinterpret_cast<float4*>(yrow + 16 * nt + 4 * g) = make_float4(Y[nt][0], Y[nt][1], Y[nt][2], Y[nt][3]);
        }
      }
      fetch(min(ch + 1, c1 - 1), buf);
    }

    if (ch == c1 - 1) break;
    lds_barrier();   // every wave has finished reading sS

    // ---- phase D: state rows 16J + 4g + j.  Keys k 2^(-Lin) are read down the
    // columns of sKf; fast: S <- 2^Ltot (S + K^T V); slow: the keys of token
    // block I are rescaled to k 2^(Ltot - Lin) and S <- 2^Ltot S + K^T V.
    float tot4[4], dec[4];
    chunk_total4(sBT, 16 * J + 4 * g, tot4);
#pragma unroll
    for (int j = 0; j < 4; ++j) dec[j] = ex2(tot4[j]);
    if (!slow) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const Op<SP> key = rdcol8<SP>(sKf, lo.c, 2048 * ks);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          S[nt] = mma(key, rd8<SV>(sV, 1024 * nt + lo.a[ks]), S[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[nt][j] *= dec[j];
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[nt][j] *= dec[j];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Op<SP> key = rdcol8<SP>(sKf, lo.c, 2048 * ks);
        // rows 32ks + 8g .. + 7 lie in token block I = 2ks + g / 2
        const int c = 16 * J + li;
        const int I = 2 * ks + (g >> 1);
        const float eI = block_end(sBT, I, c);
        const float tc = block_end(sBT, 3, c);
        float x[8];
        join8<SP>(key, x);
        const float f = ex2(tc - eI);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= f;
        key = split8<SP>(x);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          S[nt] = mma(key, rd8<SV>(sV, 1024 * nt + lo.a[ks]), S[nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const float x[4] = {S[nt][0], S[nt][1], S[nt][2], S[nt][3]};
      wr4<SP>(sS, 1024 * nt + lo.s, x);
    }
  }
}

struct Plan {
  int NC, CPS, G;
};

Plan plan(const FwdArgs& a) {
  Plan pl;
  pl.NC = (int)((a.T + LC - 1) / LC);
  const int64_t bh = a.B * a.H;
  int G = 1;
  if (const char* e = getenv("WKV6_SEGMENTS")) {
    G = atoi(e);
  } else {
    // enough workgroups for every CU: two resident per CU for bf16 inputs
    const int64_t target = a.bf16 ? 512 : 256;
    if (bh < target) G = (int)((target + bh - 1) / bh);
  }
  G = max(1, min(G, pl.NC));
  pl.CPS = (pl.NC + G - 1) / G;
  pl.G = (pl.NC + pl.CPS - 1) / pl.CPS;
  return pl;
}

template <bool BF16>
constexpr int planes() {
  return BF16 ? 2 : 3;
}

template <bool BF16, bool BIDIR, bool CARRY>
hipError_t launch_t(const FwdArgs& a, const Plan& pl, void* ws, hipStream_t s) {
  Params p;
  p.r = a.r;
  p.k = a.k;
  p.v = a.v;
  p.w = a.w_raw;
  p.u = a.u;
  p.y = a.y;
  const size_t rev_bytes = BIDIR ? (size_t)a.B * a.H * pl.NC * planes<BF16>() * PL * sizeof(__bf16) : 0;
  p.rev = static_cast<__bf16*>(ws);
  p.summ = CARRY ? reinterpret_cast<float*>(static_cast<char*>(ws) + rev_bytes) : nullptr;
  p.T = a.T;
  p.C = a.C;
  p.H = (int)a.H;
  p.NC = pl.NC;
  p.CPS = pl.CPS;
  p.G = pl.G;
  const dim3 grid((unsigned)(a.B * a.H * pl.G)), block(NT);
  if (BIDIR || CARRY) {
    hipLaunchKernelGGL((seg_kernel<BF16, BIDIR, CARRY>), grid, block, 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((fwd_kernel<BF16, BIDIR, CARRY>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <bool BF16, bool BIDIR>
hipError_t launch_c(const FwdArgs& a, const Plan& pl, void* ws, hipStream_t s) {
  return pl.G > 1 ? launch_t<BF16, BIDIR, true>(a, pl, ws, s) : launch_t<BF16, BIDIR, false>(a, pl, ws, s);
}

}  // namespace

size_t workspace_bytes(const FwdArgs& a) {
  const Plan pl = plan(a);
  size_t n = 0;
  if (a.bidirectional) n += (size_t)a.B * a.H * pl.NC * (a.bf16 ? 2 : 3) * PL * sizeof(__bf16);
  if (pl.G > 1) n += (size_t)a.B * a.H * pl.G * kSummFloats * sizeof(float);
  return n;
}

hipError_t enqueue_fwd(const FwdArgs& a, void* workspace, hipStream_t stream) {
  const Plan pl = plan(a);
  if (a.bf16)
    return a.bidirectional ? launch_c<true, true>(a, pl, workspace, stream)
                           : launch_c<true, false>(a, pl, workspace, stream);
  return a.bidirectional ? launch_c<false, true>(a, pl, workspace, stream)
                         : launch_c<false, false>(a, pl, workspace, stream);
}

}  // namespace wkv6

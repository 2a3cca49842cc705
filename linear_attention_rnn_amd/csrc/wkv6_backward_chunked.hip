// Chunked backward of the RWKV-6 WKV operator on MFMA (gfx950), bf16 inputs.
//
// The gradients of L = sum(y * dy) (CUDA-kernels page of deepglint/rwkv-clip,
// section "Backward Pass Gradient Computation", whose steps the pages leave
// open; the adjoint of the recurrence in include/wkv6.h) evaluated in chunks
// of 64 tokens, like the forward.  One direction (a causal sweep, or the
// reversed sweep of a bidirectional call, which has no u term) at a time.
//
// Notation per chunk, in sweep order (positions 0..63): lambda = log2 of the
// decay per token and key channel c, Lin / Lex its inclusive / exclusive
// prefix over the chunk, Ltot the chunk total; q_t = r_t 2^Lex_t,
// kap_i = k_i 2^-Lin_i (both per channel c); S_in the state entering the
// chunk, G the adjoint dL/dS of the state leaving it, G' = 2^Ltot G (rows c);
// Bm[t][i] = dy_t . v_i.  Then
//
//   dr_t  = 2^Lex_t  (sum_{i<t} Bm[t][i] kap_i + S_in dy_t)      + u k_t Bm[t][t]
//   dk_i  = 2^-Lin_i (sum_{t>i} Bm[t][i] q_t  + G' v_i)          + u r_i Bm[i][i]
//   dv_i  = sum_{t>=i} A[t][i] dy_t + sum_c kap_i[c] G'[c][.],
//           A[t][i] = q_t . kap_i (t > i), A[i][i] = sum_c r_i u k_i
//   G_in  = G' + sum_t q_t^T dy_t   (the adjoint of the state entering the chunk)
//
// and the decay gradient needs no per-token state: with P_j = <G_j, S_j>_c
// (the row-wise inner product of the adjoint and the state after token j),
// P_j = P_end + sum_{t>j in chunk} (r_t dr_t - k_t dk_t), where P_end =
// <G_in, S_in> of the next chunk in sweep order (0 after the last), and
//   dlambda_j = P_j - k_j dk_j + r_j u k_j Bm[j][j],  dw_raw_j = dlambda_j (-exp(w_raw_j)).
// (dlambda_j = <G_j, w_j S_{j-1}>, and S_j - w_j S_{j-1} = k_j^T v_j.)
//
// Two kernels per direction:
//   bwd_states_kernel  sweeps the chunks in order and stores every chunk's
//                      S_in (fp32, in the lane order of the reader); it also
//                      flags items with a 16-token block that decays by
//                      2^-24 or more in some channel (kap would overflow
//                      there): those items are left to the token-serial
//                      kernels.
//   bwd_chunk_kernel   sweeps the chunks from the last to the first with G in
//                      registers and writes (reversed direction: adds) dr,
//                      dk, dv, dw_raw and the u gradient's partial sums.
//
// Precision: every MFMA operand is carried as three bf16 parts except v (an
// exact bf16 input, one part); every product keeps the part products of
// order < 3.  That keeps dr, dk and dw_raw at the float32 level (two parts
// leave dw_raw near 2e-4 of its scale, through the running sums P).
//
// Layout of kernel B: wave J owns positions 16J..16J+15 of the chunk, lane
// (g, li) position 16J + li.  Its per-channel data sit at channels
// 16 ct + 4 g + j (ct, j = 0..3), exactly the rows of the D tiles it holds
// for outputs indexed (channel, own token), so the decay factors of dr and dk
// are per-lane values.  As MFMA k-slots (contraction over c) they are taken
// in the order slot 8 g + j' of step ks -> 32 ks + 16 (j' / 4) + 4 g + j' % 4
// ("pi order"), which is also the order in which two D tiles of consecutive
// row blocks feed a contraction over their rows.  Planes in LDS hold kap, q,
// dy (token-major) and S_in, G' (row c); reads along a plane's first index in
// pi order use the transposed LDS read with the matching addresses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv6_device.h"
#include "wkv6_internal.h"

namespace wkv6 {
namespace {

struct CbParams {
  const void* r;
  const void* k;
  const void* v;
  const void* w;
  const float* u;
  const float* dy;
  float* dr;
  float* dk;
  float* dv;
  float* dw;
  float* du_part;   // [B][C]: the u gradient summed over one item's tokens
  float* sst;       // [B*H][nch][256][16]: S_in of every chunk, lane order
  int* slow;        // [B*H]: nonzero = left to the token-serial kernels
  int64_t T;
  int64_t C;
  int H;
  int nch;
};

// ---------------------------------------------------------------- kernel A

struct StLds {
  static constexpr int kTile = PL * 2;     // one 64 x 64 bf16 plane
  static constexpr int kBuf = 3 * kTile;   // k, v, w
  static constexpr int kBytes = 2 * kBuf;  // two buffers
};

// Chunk-entry states of one direction, by state rows: wave J owns rows
// (key channels) 16J..16J+15 for the whole sequence; the k, v, w tiles of a
// chunk are staged through swizzled LDS and read down their columns.
template <bool REV>
__global__ __launch_bounds__(NT, 2) void bwd_states_kernel(CbParams p) {
  __shared__ __attribute__((aligned(16))) char lds[StLds::kBytes];
  __shared__ int sSlow[4];
  const int bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int J = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const int nch = p.nch;
  const Rsrc rk = slice_rsrc(p.k, base, 2, T, C), rv = slice_rsrc(p.v, base, 2, T, C);
  const Rsrc rw = slice_rsrc(p.w, base, 2, T, C);

  int srow[2], scol[2], sdst[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int pc = tid + 256 * hh;
    srow[hh] = pc >> 3;
    scol[hh] = pc & 7;
    sdst[hh] = swz(srow[hh], 8 * scol[hh]);
  }
  const uint32_t rstep = (uint32_t)C * 2u;
  uint4 stg[3][2];
  auto fetch = [&](int ch) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int64_t s = (int64_t)ch * LC + srow[hh];   // sweep position
      const int64_t t = REV ? T - 1 - s : s;
      const int off = s < T ? (int)((uint32_t)t * rstep) + 16 * scol[hh] : kOffNone;
      stg[0][hh] = bload16(rk, off);
      stg[1][hh] = bload16(rv, off);
      stg[2][hh] = bload16(rw, off);
    }
  };
  int ktJ[2], ktV[4][2];
  col_offsets(J, g, li, ktJ);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) col_offsets(nt, g, li, ktV[nt]);

  f32x4 S[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) S[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool slow = false;
  const bool odd = (g & 1) != 0, upper = (g & 2) != 0;

  fetch(0);
  for (int ch = 0; ch < nch; ++ch) {
    // S_in of this chunk: lane tid holds S[c = 16J + li][n = 16 nt + 4 g + j]
    float* dst = p.sst + (((int64_t)bh * nch + ch) * NT + tid) * 16;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      *reinterpret_cast<float4*>(dst + 4 * nt) = make_float4(S[nt][0], S[nt][1], S[nt][2], S[nt][3]);

    char* buf = lds + (ch & 1) * StLds::kBuf;
#pragma unroll
    for (int ti = 0; ti < 3; ++ti)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<uint4*>(buf + ti * StLds::kTile + 2 * sdst[hh]) = stg[ti][hh];
    if (ch + 1 < nch) fetch(ch + 1);
    lds_barrier();
    const __bf16* sK = reinterpret_cast<const __bf16*>(buf);
    const __bf16* sV = reinterpret_cast<const __bf16*>(buf + StLds::kTile);
    const __bf16* sW = reinterpret_cast<const __bf16*>(buf + 2 * StLds::kTile);
    const int Lv = (int)min<int64_t>(LC, T - (int64_t)ch * LC);

    // lambda's inclusive prefix for positions 32 ks + 8 g + j of channel
    // 16J + li; the 16-position block sums decide the slow flag
    float lin[2][8], tot = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float w8[8];
      widen8(rdcol8<1>(sW, ktJ, 2048 * ks).p[0], w8);
      float run = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 32 * ks + 8 * g + j;
        run += t < Lv ? -kLog2e * ex2(w8[j] * kLog2e) : 0.f;
        lin[ks][j] = run;
      }
      const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(run), __float_as_uint(run), false, false);
      const float partner = __uint_as_float(odd ? a[0] : a[1]);
      const float pair = run + partner;   // the 16-position block (2 ks + g / 2)
      slow = slow || pair < -kBlockSpan;
      const auto c2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
      const float other = __uint_as_float(upper ? c2[0] : c2[1]);
      const float pre = tot + (odd ? partner : 0.f) + (upper ? other : 0.f);
#pragma unroll
      for (int j = 0; j < 8; ++j) lin[ks][j] += pre;
      tot += pair + other;
    }
    if (ch + 1 < nch) {
      // S <- 2^tot S + (k 2^(tot - Lin))^T V; every factor is at most 1
      const float dec = ex2(tot);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[nt][j] *= dec;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float k8[8], ef[8];
        widen8(rdcol8<1>(sK, ktJ, 2048 * ks).p[0], k8);
#pragma unroll
        for (int j = 0; j < 8; ++j) ef[j] = k8[j] * ex2(tot - lin[ks][j]);
        const Op<3> eo = split8<3>(ef);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) S[nt] = mma(rdcol8<1>(sV, ktV[nt], 2048 * ks), eo, S[nt]);
      }
    }
  }
  const bool any = __any(slow);
  if (lane == 0) sSlow[J] = any ? 1 : 0;
  __syncthreads();
  if (tid == 0) {
    const int f = sSlow[0] | sSlow[1] | sSlow[2] | sSlow[3];
    if (!REV)
      p.slow[bh] = f;
    else if (f)
      p.slow[bh] = 1;
  }
}

// ---------------------------------------------------------------- kernel B

struct CbLds {
  static constexpr int kPlane = PL * 2;            // one bf16 plane
  static constexpr int kK = 0;                     // kap [i][c], 3 parts
  static constexpr int kQ = kK + 3 * kPlane;       // q [t][c], 3 parts
  static constexpr int kS = kQ + 3 * kPlane;       // S_in [c][n], 3 parts
  static constexpr int kG = kS + 3 * kPlane;       // G' [c][n], 3 parts
  static constexpr int kV = kG + 3 * kPlane;       // v [i][n], 1 part
  static constexpr int kD = kV + kPlane;           // dy [t][n], 3 parts
  static constexpr int kBT = kD + 3 * kPlane;      // lambda block totals [4][64]
  static constexpr int kXT = kBT + 4 * 64 * 4;     // block totals of r dr - k dk [4][64]
  static constexpr int kQS = kXT + 4 * 64 * 4;     // per wave: sum_t q_t (S_in dy_t) [4][64]
  static constexpr int kPend = kQS + 4 * 64 * 4;   // P at a chunk's end [2][64]
  static constexpr int kU = kPend + 2 * 64 * 4;    // u of the head [64]
  static constexpr int kDU = kU + 64 * 4;          // u gradient per token block [4][64]
  static constexpr int kPG = kDU + 4 * 64 * 4;     // <G', S_in> per column half [2][64]; sum r u k [2][64]
  static constexpr int kBytes = kPG + 4 * 64 * 4;
};

// DPP: lane i of each 16-lane row receives lane i + N of the row (0 if none).
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 | N, 0xF, 0xF, true));
}

// Inclusive sums within each 16-lane row: towards higher lanes (prefix) or
// towards lower lanes (suffix).
__device__ __forceinline__ float row_prefix(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  return x + row_shr<8>(x);
}
__device__ __forceinline__ float row_suffix(float x) {
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  return x + row_shl<8>(x);
}

// Offsets of transposed reads in pi order: lane (g, li) addresses rows
// 4 g + li / 4 (+ 16) at columns x0 + 4 (li % 4), so that lane (g, i)
// receives, for column x0 + i, the rows 4 g .. 4 g + 3 and 16 + 4 g .. + 3
// (k-slots 8 g .. 8 g + 7 of a 32-row step; add 2048 per step).
__device__ __forceinline__ void colpi_offsets(int x0, int g, int li, int (&kt)[2]) {
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) kt[hh] = swz(4 * g + (li >> 2) + 16 * hh, x0 + 4 * (li & 3));
}

template <int S>
__device__ __forceinline__ Op<S> rdcolpi(const __bf16* P, const int (&kt)[2], int add) {
  Op<S> o;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bf16x4 a = ld_tr(P + s * PL + add + kt[0]);
    const bf16x4 b = ld_tr(P + s * PL + add + kt[1]);
    o.p[s] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  }
  return o;
}

// Two D tiles of consecutive row blocks as one 32-row contraction operand.
__device__ __forceinline__ Op<3> tiles_op(const f32x4& lo, const f32x4& hi) {
  const float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return split8<3>(x);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// 4 bf16 values (8 bytes) as floats.
__device__ __forceinline__ void bf4(const u32x2& q, float (&o)[4]) {
  o[0] = __uint_as_float(q[0] << 16);
  o[1] = __uint_as_float(q[0] & 0xFFFF0000u);
  o[2] = __uint_as_float(q[1] << 16);
  o[3] = __uint_as_float(q[1] & 0xFFFF0000u);
}

__device__ __forceinline__ u32x2 bload8(Rsrc r, int off) { return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0); }

// Stores (ACC: adds to what is there) 4 floats at byte offset off.
template <bool ACC>
__device__ __forceinline__ void out4(Rsrc r, int off, float a, float b, float c, float d) {
  if constexpr (ACC) {
    const float4 o = bloadf4(r, off);
    a += o.x;
    b += o.y;
    c += o.z;
    d += o.w;
  }
  bstoref4(r, off, a, b, c, d);
}

// Workgroup of kernel B: 8 waves, two per token block.  Wave (J, H), J = 0..3,
// H = 0..1, owns positions 16J..16J+15 and, of every output indexed by a
// channel, the tiles 2H and 2H + 1 (channels 32H .. 32H + 31); the score-like
// tiles both need are computed by both.
constexpr int NTB = 512;

// REV: the reversed sweep of a bidirectional call (no u term; outputs added).
template <bool REV>
__global__ __launch_bounds__(NTB, 1) void bwd_chunk_kernel(CbParams p) {
  __shared__ __attribute__((aligned(16))) char lds[CbLds::kBytes];
  // the reversed sweep visits the items in reverse order: it runs right
  // after the forward direction's pass, whose last outputs, which it adds
  // to first, are then the likeliest still to be in the caches
  const int bh = REV ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  if (p.slow[bh]) return;   // the token-serial kernels take this item
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int J = wv & 3, H = wv >> 2;
  const int g = lane >> 4, li = lane & 15;
  const int b = bh / p.H, h = bh % p.H;
  const int64_t T = p.T, C = p.C;
  const int nch = p.nch;
  const int64_t base = (int64_t)b * T * C + (int64_t)h * HS;
  const Rsrc rr = slice_rsrc(p.r, base, 2, T, C), rk = slice_rsrc(p.k, base, 2, T, C);
  const Rsrc rv = slice_rsrc(p.v, base, 2, T, C), rw = slice_rsrc(p.w, base, 2, T, C);
  const Rsrc rdy = slice_rsrc(p.dy, base, 4, T, C);
  const Rsrc odr = slice_rsrc(p.dr, base, 4, T, C), odk = slice_rsrc(p.dk, base, 4, T, C);
  const Rsrc odv = slice_rsrc(p.dv, base, 4, T, C), odw = slice_rsrc(p.dw, base, 4, T, C);

  __bf16* sK = reinterpret_cast<__bf16*>(lds + CbLds::kK);
  __bf16* sQ = reinterpret_cast<__bf16*>(lds + CbLds::kQ);
  __bf16* sS = reinterpret_cast<__bf16*>(lds + CbLds::kS);
  __bf16* sG = reinterpret_cast<__bf16*>(lds + CbLds::kG);
  __bf16* sV = reinterpret_cast<__bf16*>(lds + CbLds::kV);
  __bf16* sD = reinterpret_cast<__bf16*>(lds + CbLds::kD);
  float* sBT = reinterpret_cast<float*>(lds + CbLds::kBT);
  float* sXT = reinterpret_cast<float*>(lds + CbLds::kXT);
  float* sQS = reinterpret_cast<float*>(lds + CbLds::kQS);
  float* sPend = reinterpret_cast<float*>(lds + CbLds::kPend);
  float* sU = reinterpret_cast<float*>(lds + CbLds::kU);
  float* sDU = reinterpret_cast<float*>(lds + CbLds::kDU);
  float* sPG = reinterpret_cast<float*>(lds + CbLds::kPG);
  if (tid < 256) sDU[tid] = 0.f;
  if (tid < 64) {
    sU[tid] = REV ? 0.f : p.u[h * HS + tid];
    sPend[64 * ((nch - 1) & 1) + tid] = 0.f;   // after the last chunk the adjoint is zero
  }

  const int pos = 16 * J + li;   // the lane's position in every chunk
  const uint32_t rstep2 = (uint32_t)C * 2u, rstep4 = (uint32_t)C * 4u;
  // byte offsets (bf16 rows; fp32 rows) of the lane's token in chunk m, or none
  auto row2 = [&](int m) -> int {
    const int64_t s = (int64_t)m * LC + pos;
    return s < T ? (int)((uint32_t)(REV ? T - 1 - s : s) * rstep2) : kOffNone;
  };
  auto row4 = [&](int m) -> int {
    const int64_t s = (int64_t)m * LC + pos;
    return s < T ? (int)((uint32_t)(REV ? T - 1 - s : s) * rstep4) : kOffNone;
  };
  // the lane's inputs of one token: r, k, w at its channels 16 (2H + cl) + 4 g
  // + j, v and dy at channels 32 ks + 8 g + j; its half of the chunk's S_in
  u32x2 nr[2], nk[2], nw[2];
  uint4 nv[2];
  float4 ndy[4], ns[2];
  auto fetch_in = [&](int m) {
    const int o2 = row2(m), o4 = row4(m);
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
      const int o = o2 + 32 * (2 * H + cl) + 8 * g;
      nr[cl] = bload8(rr, o);
      nk[cl] = bload8(rk, o);
      nw[cl] = bload8(rw, o);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      nv[ks] = bload16(rv, o2 + 64 * ks + 16 * g);
      ndy[2 * ks] = bloadf4(rdy, o4 + 128 * ks + 32 * g);
      ndy[2 * ks + 1] = bloadf4(rdy, o4 + 128 * ks + 32 * g + 16);
    }
  };
  auto fetch_s = [&](int m) {
    const float4* src =
        reinterpret_cast<const float4*>(p.sst + (((int64_t)bh * nch + m) * NT + 64 * J + lane) * 16 + 8 * H);
    ns[0] = src[0];
    ns[1] = src[1];
  };

  // transposed-read offsets: pi order at the column blocks 2H, 2H + 1 (kap^T,
  // q^T, dy^T, G'^T operands), sigma order at blocks 2H, 2H + 1 and J (the
  // adjoint update)
  int kpi[2][2], ksg[2][2], ksj[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    colpi_offsets(16 * (2 * H + x), g, li, kpi[x]);
    col_offsets(2 * H + x, g, li, ksg[x]);
  }
  col_offsets(J, g, li, ksj);

  f32x4 Gc[2];   // adjoint, lane: G[c = 16J + li][n = 16 (2H + nl) + 4 g + j]
  Gc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
  Gc[1] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch_in(nch - 1);
  fetch_s(nch - 1);
  for (int m = nch - 1; m >= 0; --m) {
    const int Lv = (int)min<int64_t>(LC, T - (int64_t)m * LC);
    const bool valid = pos < Lv;
    const int o4 = row4(m);
    // ---- this chunk's raw values, then the next chunk's loads
    u32x2 cr[2], ck[2];
    float lam[2][4], dyf[2][8];
    uint4 vq[2];
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
      cr[cl] = nr[cl];
      ck[cl] = nk[cl];
      float w4[4];
      bf4(nw[cl], w4);
#pragma unroll
      for (int j = 0; j < 4; ++j) lam[cl][j] = valid ? -kLog2e * ex2(w4[j] * kLog2e) : 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      vq[ks] = nv[ks];
      const float4 a = ndy[2 * ks], c = ndy[2 * ks + 1];
      dyf[ks][0] = a.x; dyf[ks][1] = a.y; dyf[ks][2] = a.z; dyf[ks][3] = a.w;
      dyf[ks][4] = c.x; dyf[ks][5] = c.y; dyf[ks][6] = c.z; dyf[ks][7] = c.w;
    }
    if (m > 0) fetch_in(m - 1);

    // ---- lambda prefix within the 16-position block (DPP), block totals
    float lin[2][4];
#pragma unroll
    for (int cl = 0; cl < 2; ++cl)
#pragma unroll
      for (int j = 0; j < 4; ++j) lin[cl][j] = row_prefix(lam[cl][j]);
    if (li == 15) {
#pragma unroll
      for (int cl = 0; cl < 2; ++cl)
        *reinterpret_cast<float4*>(&sBT[J * 64 + 16 * (2 * H + cl) + 4 * g]) =
            make_float4(lin[cl][0], lin[cl][1], lin[cl][2], lin[cl][3]);
    }
    // dy_t . v_t of the lane's token (over its four lane groups)
    float bmd = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t vw[4] = {vq[ks].x, vq[ks].y, vq[ks].z, vq[ks].w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        bmd = fmaf(dyf[ks][2 * jj], __uint_as_float(vw[jj] << 16), bmd);
        bmd = fmaf(dyf[ks][2 * jj + 1], __uint_as_float(vw[jj] & 0xFFFF0000u), bmd);
      }
    }
    bmd = rows_sum(bmd);
    lds_barrier();   // B1: block totals visible; the previous chunk's readers are done

    // ---- prefixes; planes kap, q, S_in, G', v, dy; <G', S_in> by rows
    float tot_row = 0.f;   // Ltot of channel 16J + li (the adjoint's rows)
#pragma unroll
    for (int I = 0; I < 4; ++I) tot_row += sBT[I * 64 + 16 * J + li];
    float q16[2][4];
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
      const int ct = 2 * H + cl;
      float off[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int I = 0; I < 3; ++I)
        if (I < J) {
          const float4 a = *reinterpret_cast<const float4*>(&sBT[I * 64 + 16 * ct + 4 * g]);
          off[0] += a.x; off[1] += a.y; off[2] += a.z; off[3] += a.w;
        }
      float r4[4], k4[4], kap[4];
      bf4(cr[cl], r4);
      bf4(ck[cl], k4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lin[cl][j] += off[j];
        kap[j] = k4[j] * ex2(-lin[cl][j]);
        q16[cl][j] = r4[j] * ex2(lin[cl][j] - lam[cl][j]);
      }
      wr4<3>(sK, swz(pos, 16 * ct + 4 * g), kap);
      wr4<3>(sQ, swz(pos, 16 * ct + 4 * g), q16[cl]);
    }
    float dsum = 0.f;   // sum_c r u k of the lane's token (the wave's channels)
    if (!REV) {
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        float r4[4], k4[4];
        bf4(cr[cl], r4);
        bf4(ck[cl], k4);
        const float4 uu = *reinterpret_cast<const float4*>(&sU[16 * (2 * H + cl) + 4 * g]);
        dsum = fmaf(r4[0] * uu.x, k4[0], dsum);
        dsum = fmaf(r4[1] * uu.y, k4[1], dsum);
        dsum = fmaf(r4[2] * uu.z, k4[2], dsum);
        dsum = fmaf(r4[3] * uu.w, k4[3], dsum);
      }
      dsum = rows_sum(dsum);
      if (g == 0) sPG[128 + 64 * H + pos] = dsum;
    }
    {
      const float dec = ex2(tot_row);
      float pgs = 0.f;
#pragma unroll
      for (int nl = 0; nl < 2; ++nl) {
        const int nt = 2 * H + nl;
        const float s4[4] = {ns[nl].x, ns[nl].y, ns[nl].z, ns[nl].w};
        wr4<3>(sS, swz(16 * J + li, 16 * nt + 4 * g), s4);
        float g4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Gc[nl][j] *= dec;
          g4[j] = Gc[nl][j];
          pgs = fmaf(g4[j], s4[j], pgs);
        }
        wr4<3>(sG, swz(16 * J + li, 16 * nt + 4 * g), g4);
      }
      pgs = rows_sum(pgs);
      if (g == 0) sPG[64 * H + 16 * J + li] = pgs;
    }
    if (m > 0) fetch_s(m - 1);
    if (H == 0) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        *reinterpret_cast<uint4*>(sV + swz(pos, 32 * ks + 8 * g)) = vq[ks];
        wr8<3>(sD, swz(pos, 32 * ks + 8 * g), dyf[ks]);
      }
    }
    lds_barrier();   // B2: the planes are ready
    if (!REV) dsum = sPG[128 + pos] + sPG[192 + pos];

    // ---- dr: D rows c (tiles 2H, 2H + 1), column = own position
    float x16[2][4];
    {
      f32x4 acc[2], bmt[4];   // bmt: Bm^T[i][t], rows i (block I <= J), column t
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int I = 0; I < 4; ++I) bmt[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const Op<3> dyo = split8<3>(dyf[ks]);
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
          acc[cl] = mma(rd8<3>(sS, swz(16 * (2 * H + cl) + li, 32 * ks + 8 * g)), dyo, acc[cl]);
#pragma unroll
        for (int I = 0; I < 4; ++I)
          if (I <= J) {
            Op<1> va;
            va.p[0] = *reinterpret_cast<const bf16x8*>(sV + swz(16 * I + li, 32 * ks + 8 * g));
            bmt[I] = mma(va, dyo, bmt[I]);
          }
      }
      // q_t (S_in dy_t), summed over the wave's positions, for <q^T dY, S_in>
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        float zs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) zs[j] = row_prefix(q16[cl][j] * acc[cl][j]);
        if (li == 15)
          *reinterpret_cast<float4*>(&sQS[J * 64 + 16 * (2 * H + cl) + 4 * g]) = make_float4(zs[0], zs[1], zs[2], zs[3]);
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if (I == J) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * g + j >= li) bmt[I][j] = 0.f;   // keep i < t
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb > J) break;
        const Op<3> bo = tiles_op(bmt[2 * kb], bmt[2 * kb + 1]);
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) acc[cl] = mma(rdcolpi<3>(sK, kpi[cl], 2048 * kb), bo, acc[cl]);
      }
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * H + cl;
        float r4[4], k4[4];
        bf4(cr[cl], r4);
        bf4(ck[cl], k4);
        const float4 uu = *reinterpret_cast<const float4*>(&sU[16 * ct + 4 * g]);
        const float u4[4] = {uu.x, uu.y, uu.z, uu.w};
        float d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          d[j] = ex2(lin[cl][j] - lam[cl][j]) * acc[cl][j];
          if (!REV) d[j] = fmaf(u4[j] * k4[j], bmd, d[j]);
          x16[cl][j] = r4[j] * d[j];
        }
        out4<REV>(odr, o4 + 64 * ct + 16 * g, d[0], d[1], d[2], d[3]);
      }
    }

    // ---- dk: D rows c, column = own position (key i); then the local part
    // of the decay gradient
    Op<1> vo[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vo[ks].p[0] = __builtin_bit_cast(bf16x8, vq[ks]);
    {
      f32x4 bm[4], acc[2];   // bm: Bm[t][i], rows t (block >= J), column i
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        bm[I] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (I >= J) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) bm[I] = mma(rd8<3>(sD, swz(16 * I + li, 32 * ks + 8 * g)), vo[ks], bm[I]);
        }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if (I == J) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * g + j <= li) bm[I][j] = 0.f;   // keep t > i
        }
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        acc[cl] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc[cl] = mma(rd8<3>(sG, swz(16 * (2 * H + cl) + li, 32 * ks + 8 * g)), vo[ks], acc[cl]);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb + 1 < J) continue;
        const Op<3> bo = tiles_op(bm[2 * kb], bm[2 * kb + 1]);
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) acc[cl] = mma(rdcolpi<3>(sQ, kpi[cl], 2048 * kb), bo, acc[cl]);
      }
      float xb[2][4], Lj[2][4];
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * H + cl;
        float r4[4], k4[4];
        bf4(cr[cl], r4);
        bf4(ck[cl], k4);
        const float4 uu = *reinterpret_cast<const float4*>(&sU[16 * ct + 4 * g]);
        const float u4[4] = {uu.x, uu.y, uu.z, uu.w};
        float d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          d[j] = ex2(-lin[cl][j]) * acc[cl][j];
          if (!REV) d[j] = fmaf(u4[j] * r4[j], bmd, d[j]);
          const float kdk = k4[j] * d[j];
          const float x = x16[cl][j] - kdk;
          const float xi = row_suffix(x);   // this position and the later ones of the block
          xb[cl][j] = xi;
          // P_j's part from this block, minus k dk, plus r u k (dy . v)
          float L = xi - x - kdk;
          if (!REV) L = fmaf(r4[j] * u4[j] * k4[j], bmd, L);
          Lj[cl][j] = L;
        }
        out4<REV>(odk, o4 + 64 * ct + 16 * g, d[0], d[1], d[2], d[3]);
      }
      if (li == 0) {
#pragma unroll
        for (int cl = 0; cl < 2; ++cl)
          *reinterpret_cast<float4*>(&sXT[J * 64 + 16 * (2 * H + cl) + 4 * g]) =
              make_float4(xb[cl][0], xb[cl][1], xb[cl][2], xb[cl][3]);
      }
      lds_barrier();   // B5: block sums of x and the q (S dy) sums visible
      if (H == 0 && g == 0) {   // P at the end of the previous chunk in sweep order
        const int c = 16 * J + li;
        sPend[64 * ((m - 1) & 1) + c] =
            sPG[c] + sPG[64 + c] + sQS[c] + sQS[64 + c] + sQS[128 + c] + sQS[192 + c];
      }
      // dw: P_end + block sums of later waves + the local part, times ln w
#pragma unroll
      for (int cl = 0; cl < 2; ++cl) {
        const int ct = 2 * H + cl;
        float4 pe = *reinterpret_cast<const float4*>(&sPend[64 * (m & 1) + 16 * ct + 4 * g]);
#pragma unroll
        for (int I = 1; I < 4; ++I)
          if (I > J) {
            const float4 a = *reinterpret_cast<const float4*>(&sXT[I * 64 + 16 * ct + 4 * g]);
            pe.x += a.x; pe.y += a.y; pe.z += a.z; pe.w += a.w;
          }
        constexpr float kLn2 = 1.f / kLog2e;
        out4<REV>(odw, o4 + 64 * ct + 16 * g, (pe.x + Lj[cl][0]) * lam[cl][0] * kLn2,
                  (pe.y + Lj[cl][1]) * lam[cl][1] * kLn2, (pe.z + Lj[cl][2]) * lam[cl][2] * kLn2,
                  (pe.w + Lj[cl][3]) * lam[cl][3] * kLn2);
      }
      if (!REV) {
        // u gradient: r k (dy . v) summed over the wave's positions
#pragma unroll
        for (int cl = 0; cl < 2; ++cl) {
          const int ct = 2 * H + cl;
          float r4[4], k4[4];
          bf4(cr[cl], r4);
          bf4(ck[cl], k4);
          float z[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) z[j] = row_prefix(r4[j] * k4[j] * bmd);
          if (li == 15) {
            float4* d = reinterpret_cast<float4*>(&sDU[J * 64 + 16 * ct + 4 * g]);
            const float4 o = *d;
            *d = make_float4(o.x + z[0], o.y + z[1], o.z + z[2], o.w + z[3]);
          }
        }
      }
    }

    // ---- dv: D rows n (tiles 2H, 2H + 1), column = own position (key i)
    {
      f32x4 acc[2], at[4];   // at: A[t][i], rows t (block >= J), column i
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int I = 0; I < 4; ++I) at[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // the own token's kap over all 64 channels, in pi order, from its plane row
        const Op<3> ko = rd4x2<3>(sK, swz(pos, 32 * ks + 4 * g), swz(pos, 32 * ks + 16 + 4 * g));
#pragma unroll
        for (int nl = 0; nl < 2; ++nl) acc[nl] = mma(rdcolpi<3>(sG, kpi[nl], 2048 * ks), ko, acc[nl]);
#pragma unroll
        for (int I = 0; I < 4; ++I)
          if (I >= J) {
            const int row = 16 * I + li;
            at[I] = mma(rd4x2<3>(sQ, swz(row, 32 * ks + 4 * g), swz(row, 32 * ks + 16 + 4 * g)), ko, at[I]);
          }
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if (I == J) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (4 * g + j < li) at[I][j] = 0.f;   // keep t > i
            if (4 * g + j == li) at[I][j] = REV ? 0.f : dsum;
          }
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (2 * kb + 1 < J) continue;
        const Op<3> bo = tiles_op(at[2 * kb], at[2 * kb + 1]);
#pragma unroll
        for (int nl = 0; nl < 2; ++nl) acc[nl] = mma(rdcolpi<3>(sD, kpi[nl], 2048 * kb), bo, acc[nl]);
      }
#pragma unroll
      for (int nl = 0; nl < 2; ++nl)
        out4<REV>(odv, o4 + 64 * (2 * H + nl) + 16 * g, acc[nl][0], acc[nl][1], acc[nl][2], acc[nl][3]);
    }

    // ---- adjoint entering the chunk: G <- G' + q^T dY (rows c of block J)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const Op<3> qb = rdcol8<3>(sQ, ksj, 2048 * ks);
#pragma unroll
      for (int nl = 0; nl < 2; ++nl) Gc[nl] = mma(rdcol8<3>(sD, ksg[nl], 2048 * ks), qb, Gc[nl]);
    }
  }

  if (!REV) {
    lds_barrier();   // every wave's u gradient sums are in
    if (tid < 64) p.du_part[(int64_t)b * C + h * HS + tid] = sDU[tid] + sDU[64 + tid] + sDU[128 + tid] + sDU[192 + tid];
  }
}

CbParams chunk_params(const BwdArgs& a, float* du_part, const float* sst, const int* slow) {
  CbParams p{};
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
  p.du_part = du_part;
  p.sst = const_cast<float*>(sst);
  p.slow = const_cast<int*>(slow);
  p.T = a.T;
  p.C = a.C;
  p.H = (int)a.H;
  p.nch = (int)((a.T + LC - 1) / LC);
  return p;
}

}  // namespace

hipError_t enqueue_bwd_chunk_states(const BwdArgs& a, float* sst, int* slow, bool rev, hipStream_t s) {
  const CbParams p = chunk_params(a, nullptr, sst, slow);
  const dim3 grid((unsigned)(a.B * a.H));
  if (rev)
    hipLaunchKernelGGL(bwd_states_kernel<true>, grid, dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_states_kernel<false>, grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

hipError_t enqueue_bwd_chunk_grads(const BwdArgs& a, float* du_part, const float* sst, const int* slow, bool rev,
                                   hipStream_t s) {
  const CbParams p = chunk_params(a, du_part, sst, slow);
  const dim3 grid((unsigned)(a.B * a.H));
  if (rev)
    hipLaunchKernelGGL(bwd_chunk_kernel<true>, grid, dim3(NTB), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_chunk_kernel<false>, grid, dim3(NTB), 0, s, p);
  return hipGetLastError();
}

}  // namespace wkv6

// Internal interface between the C ABI layer (wkv6_api.cpp) and the HIP
// kernels (wkv6_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv6 {

// Head size and chunk length the kernels are built for.
constexpr int kHead = 64;
constexpr int kChunk = 64;
// Most (batch, head) pairs one call accepts: one 256-work-item workgroup
// each, and a launch holds fewer than 2^32 work-items.
constexpr int64_t kMaxItems = (int64_t(1) << 24) - 1;

struct FwdArgs {
  int64_t B, T, C, H;
  const void* r;
  const void* k;
  const void* v;
  const void* w_raw;
  const float* u;
  float* y;
  const float* s_in;   // causal only: initial state [B*H][64][64] or null (zero)
  float* s_out;        // causal only: final state, same layout, or null
  bool bidirectional;
  bool bf16;
  bool w_static = false;   // w_raw is [C]: one decay for every token (RWKV-5)
  // fused epilogue: out = (GroupNorm_head(y) * gamma + beta) * gate as bf16
  // [B, T, C]; y is then not written (it may be null)
  bool epi = false;
  uint16_t* out = nullptr;
  const void* gate = nullptr;   // [B, T, C], dtype of r
  const float* gamma = nullptr;
  const float* beta = nullptr;
  float eps = 0.f;
};

// Bytes of device workspace a call needs (0 when none).
size_t workspace_bytes(const FwdArgs& a);

// Enqueue the kernels on `stream` (T == 0: only the state copy, if any).
// `workspace` must hold workspace_bytes(a) bytes (or be null when that is 0).
// Returns the first HIP error, if any.
hipError_t enqueue_fwd(const FwdArgs& a, void* workspace, hipStream_t stream);

// Size of the library's static per-device scratch array (wkv6_fwd_noalloc).
constexpr size_t kScratchBytes = size_t(32) << 20;

// The plain forward (no state, no epilogue) with its workspace in the
// static scratch array instead of an allocation: the segment count is
// lowered until the segment summaries fit in kScratchBytes.  Fails with
// hipErrorInvalidValue if even an unsegmented call would need more.
hipError_t enqueue_fwd_noalloc(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
  int64_t B, T, C, H;
  const void* r;
  const void* k;
  const void* v;
  const void* w_raw;
  const float* u;
  const float* dy;   // [B, T, C] float32
  float* dr;         // [B, T, C] float32 outputs
  float* dk;
  float* dv;
  float* dw_raw;
  float* du;         // [C]
  bool bidirectional;
  bool bf16;
};

// Workspace of a backward call (always > 0) and its kernels (wkv6_backward.hip).
size_t bwd_workspace_bytes(const BwdArgs& a);
hipError_t enqueue_bwd(const BwdArgs& a, void* workspace, hipStream_t stream);

// The chunked backward on MFMA (bf16 inputs, one workgroup per (batch,
// head); wkv6_backward_chunked.hip), one direction per call.  States: the
// chunk-entry states into sst ([B*H][ceil(T/64)][256][16] floats); items
// that need the general decay path are flagged in slow ([B*H]; the forward
// direction sets every flag, the reversed one only adds flags).  Gradients:
// from those states, skipping flagged items.  rev: the reversed sweep of a
// bidirectional call (adds to the outputs).
hipError_t enqueue_bwd_chunk_states(const BwdArgs& a, float* sst, int* slow, bool rev, hipStream_t stream);
hipError_t enqueue_bwd_chunk_grads(const BwdArgs& a, float* du_part, const float* sst, const int* slow, bool rev,
                                   hipStream_t stream);

// Per-head group normalisation, affine and gate of a y in memory
// (wkv6_groupnorm.hip): out = ((y - mean) * rstd * gamma + beta) * g, bf16.
struct GnArgs {
  int64_t B, T, C;
  const float* y;       // [B, T, C] float32
  const void* g;        // [B, T, C], float32 or bfloat16
  const float* gamma;   // [C]
  const float* beta;    // [C]
  float eps;
  uint16_t* out;        // [B, T, C] bfloat16
  bool bf16;
};
hipError_t enqueue_gn_gate(const GnArgs& a, hipStream_t stream);

// RWKV-4 (wkv4_kernels.hip): per-channel normalised WKV, causal.
struct Wkv4Args {
  int64_t B, T, C;
  const void* k;     // [B, T, C] float32 or bfloat16
  const void* v;
  const float* w;    // [C] decay rate (each step multiplies by exp(-w))
  const float* u;    // [C] bonus of the current token
  float* y;          // [B, T, C] float32
  bool bf16;
};

// Workspace of an RWKV-4 call (segment summaries and carries; 0 if none).
size_t wkv4_workspace_bytes(const Wkv4Args& a);
hipError_t enqueue_wkv4(const Wkv4Args& a, void* workspace, hipStream_t stream);

}  // namespace wkv6

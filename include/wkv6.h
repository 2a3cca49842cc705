/*
 * wkv6.h -- C ABI of the MI355X (gfx950) RWKV-6 WKV forward operator.
 *
 * What the operator computes (the WKV-6 forward of the deepglint/rwkv-clip
 * pages: "How Custom CUDA Kernels (wkv6_cuda.cu) Implement the WKV Operation",
 * section "Forward Pass Implementation in kernel_forward", and "RWKV
 * Architecture" on llms.blog, sections "RWKV-5 Eagle" and "RWKV-6 Finch"):
 *
 *   For every batch item b and head h (head h owns channels [64h, 64h+64) of
 *   the [B, T, C] tensors, C = 64*H), with the per-token, per-channel decay
 *   w_t[c] = exp(-exp(w_raw_t[c])) and a 64x64 fp32 state S (rows: key /
 *   receptance channel c, columns: value channel n) starting at zero:
 *
 *     y_t[n] = sum_c r_t[c] * ( S[c][n] + u[c] * k_t[c] * v_t[n] )
 *     S[c][n] <- w_t[c] * S[c][n] + k_t[c] * v_t[n]
 *
 *   i.e. token i < t reaches t with weight prod_{i<j<t} w_j and token t
 *   itself with weight u.  Bidirectional mode adds, from a second zero state
 *   swept from the last token to the first, the strictly later tokens:
 *
 *     y_t[n] += sum_c r_t[c] * sum_{i>t} (prod_{t<j<i} w_j[c]) k_i[c] v_i[n]
 *
 *   (u is applied once; the wrapper on the "What is the WKV mechanism" page,
 *   section "CUDA Wrapper (Image Side)", supplies the decay as minus the
 *   exponential of w, which the kernel exponentiates again; here the library
 *   takes w_raw itself and applies both exponentials on the GPU.)
 *
 * All arithmetic runs in the library's HIP kernels.  The kernels evaluate the
 * definition in chunks of 64 tokens with matrix-core (MFMA) contractions on
 * split bf16 operands (each fp32 operand carried as a high and a low bf16
 * part) and fp32 accumulation; results agree with an exact evaluation to
 * about 1e-4 of the output's rms (see the tests for the bounds checked).
 */
#ifndef WKV6_H
#define WKV6_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WKV6_ABI_VERSION 7

/* mode */
#define WKV6_MODE_CAUSAL        0
#define WKV6_MODE_BIDIRECTIONAL 1

/* dtype of r, k, v, w_raw (u and y are always float32) */
#define WKV6_DTYPE_F32  0
#define WKV6_DTYPE_BF16 1

/* status codes */
#define WKV6_OK               0  /* success; also B == 0 or T == 0 (nothing done) */
#define WKV6_ERR_INVALID_ARG  1  /* negative size, H < 1, C % H != 0, null pointer,
                                    unknown mode/dtype, y overlapping an input */
#define WKV6_ERR_UNSUPPORTED  2  /* head size C / H other than 64, or sizes whose
                                    index arithmetic would overflow (the kernels
                                    need T * C * 4 < 2^31 - 4096) */
#define WKV6_ERR_MISALIGNED   3  /* a pointer not aligned to 16 bytes */
#define WKV6_ERR_HIP          4  /* a HIP runtime error (launch, allocation) */

/*
 * wkv6_fwd -- enqueue one WKV-6 forward on `stream`.
 *
 *   B, T, C, H    batch, tokens, channels, heads; C must equal 64 * H.
 *   r, k, v,      device pointers to contiguous row-major [B, T, C] tensors of
 *   w_raw         `dtype` (float32, or bfloat16 stored as 16-bit words).
 *                 w_raw is the pre-transform decay: w = exp(-exp(w_raw)).
 *                 Supported w_raw: finite values up to 1.5 (w >= 0.011), or
 *                 -inf (w = 1).  Larger values can overflow the in-chunk
 *                 decay factors; +inf and NaN are not supported.
 *   u             device pointer to C float32 values, laid out [H, 64].
 *   y             device pointer to a [B, T, C] float32 output.  Fully
 *                 overwritten (never accumulated into); must not overlap any
 *                 input.
 *   mode          WKV6_MODE_CAUSAL or WKV6_MODE_BIDIRECTIONAL.
 *   dtype         WKV6_DTYPE_F32 or WKV6_DTYPE_BF16.
 *   stream        a hipStream_t passed as void* (NULL = the null stream).
 *
 * Ownership: every pointer is caller-owned device memory; the library keeps
 * none of them after returning.  When B*H is small the library cuts each
 * sequence into segments handled by different workgroups (more when the
 * sequences are long enough); such calls take a temporary device workspace
 * of B*H*segments*2*(64*64+64)*4 bytes for the segment summaries
 * (wkv6_fwd_workspace_bytes gives the exact figure), allocated and released
 * in stream order on `stream` from the library's workspace pool (see
 * WKV6_WORKSPACE_KEEP_BYTES below).  Other calls allocate nothing.  y is written in place while the call runs:
 * a bidirectional call first stores the later-token part of every row and
 * then adds the rest, so y must not be read before the stream has run the
 * call.
 *
 * Execution: asynchronous on `stream`; the call does not synchronise the
 * host.  The caller keeps the buffers alive until the stream has run the
 * work.  Calls are thread-safe; the only library state is a per-thread last
 * error message (wkv6_last_error).
 *
 * Errors: returns a WKV6_* status.  On INVALID_ARG, UNSUPPORTED and
 * MISALIGNED nothing is enqueued.  Input values are not checked: NaN and Inf
 * propagate to y.
 */
int wkv6_fwd(int64_t B, int64_t T, int64_t C, int64_t H,
             const void* r, const void* k, const void* v, const void* w_raw,
             const float* u, float* y, int mode, int dtype, void* stream);

/*
 * Workspace pool.  Calls that need device workspace (segmented calls, the
 * backward, the bidirectional fused epilogue, segmented RWKV-4 calls) take it
 * in stream order from a memory pool the library creates on each device on
 * first use (hipMemPoolCreate).  Freed blocks stay in the pool for later
 * calls up to WKV6_WORKSPACE_KEEP_BYTES per device; the runtime returns
 * memory above that to the device when a stream or the device synchronises.
 * This departs from a library that allocates nothing: the long sequences
 * over few (batch, head) pairs need per-segment summaries, and allocating
 * them from the default pool on every call cost 9-36 us.  Callers that
 * cannot allocate use wkv6_fwd_noalloc.
 */
#define WKV6_WORKSPACE_KEEP_BYTES ((size_t)256 << 20)

/* Bytes of workspace a wkv6_fwd call with these arguments takes from the pool
 * (0: none, or the arguments are invalid).  Host arithmetic only: no device
 * is touched. */
size_t wkv6_fwd_workspace_bytes(int64_t B, int64_t T, int64_t C, int64_t H, int mode, int dtype);

/* Bytes the current device's workspace pool holds now (in use and kept), or
 * 0 if the library has not created it. */
size_t wkv6_workspace_reserved_bytes(void);

/* Hands every unused block of the current device's workspace pool back to
 * the device (hipMemPoolTrimTo); blocks of calls still in flight are kept.
 * Returns WKV6_OK or WKV6_ERR_HIP. */
int wkv6_trim_workspace(void);

/*
 * wkv6_fwd_noalloc -- wkv6_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  It calls no hipMalloc, hipFree or allocating library
 * routine.
 *
 * Arguments, layout, results, execution and errors as wkv6_fwd.  The segment
 * summaries of a segmented call live in a static device array of the
 * library, 32 MiB per GPU, held from the first use until the process ends
 * (its address is taken once per device, on the first call on that device).
 * A call whose planned segment count would need more than that runs with
 * fewer segments (the result differs from wkv6_fwd's by rounding only);
 * since an unsegmented call needs no scratch, every size wkv6_fwd accepts is
 * accepted here.  UNSUPPORTED reports a workspace beyond the array should a
 * future variant need one.
 *
 * Every call on one GPU shares that GPU's array and leaves its contents
 * there: calls that can overlap on one GPU (on different streams, or from
 * different host threads without ordering) race on it and must not be made.
 * Calls ordered on one stream are safe; nothing in the array needs to start
 * at zero.
 */
int wkv6_fwd_noalloc(int64_t B, int64_t T, int64_t C, int64_t H,
                     const void* r, const void* k, const void* v, const void* w_raw,
                     const float* u, float* y, int mode, int dtype, void* stream);

/*
 * wkv6_fwd_gn -- wkv6_fwd followed by the block's output normalisation and
 * gate, fused into the kernel that produces the final outputs, with a bf16
 * result: y is never written to memory.
 *
 *   out[b,t,c] = ( (y[b,t,c] - mean_h) / sqrt(var_h + eps) * gamma[c] + beta[c] ) * g[b,t,c]
 *
 * with mean_h and var_h (biased, divided by 64) over the 64 channels of the
 * head h that holds c, for each (b, t): a per-head group normalisation
 * ("RWKV Architecture" on llms.blog, section "RWKV-5 Eagle": group
 * normalisation across the individual heads, and output gating by SiLU)
 * and the gate g the spatial-mix block forms as SiLU of a linear map of its
 * input (deepglint/rwkv-clip "What is the WKV mechanism" page, sections
 * "Spatial-Mix Block Generating the WKV Inputs" and "Invocation Inside a
 * Transformer-Style Block": the WKV output is normalised, then multiplied by
 * g).  g is taken as that page computes it, i.e. after the SiLU.
 *
 *   r, k, v, w_raw, u, B, T, C, H, mode, dtype   as wkv6_fwd
 *   g       device pointer to [B, T, C] values of `dtype`
 *   gamma, beta   device pointers to C float32 values each ([H, 64])
 *   eps     added to the variance; finite and >= 0 (else INVALID_ARG)
 *   out     device pointer to a [B, T, C] bfloat16 output (16-bit words,
 *           rounded to nearest even); must not overlap any input
 *
 * Workspace: a bidirectional call keeps the reverse sweep's float32 rows,
 * B*T*C*4 bytes, plus 4 bytes per (batch item, head, segment) for its
 * fix-up markers, and the segment summaries as in wkv6_fwd; allocated and
 * released in stream order.  Execution and errors as wkv6_fwd.
 */
int wkv6_fwd_gn(int64_t B, int64_t T, int64_t C, int64_t H,
                const void* r, const void* k, const void* v, const void* w_raw,
                const float* u, const void* g, const float* gamma, const float* beta,
                float eps, void* out, int mode, int dtype, void* stream);

/*
 * wkv6_group_norm_gate -- the output normalisation and gate of wkv6_fwd_gn as
 * a pass of its own over a y already in memory (the unfused order: any
 * forward entry point, then this one):
 *
 *   out[b,t,c] = ( (y[b,t,c] - mean_h) / sqrt(var_h + eps) * gamma[c] + beta[c] ) * g[b,t,c]
 *
 * with the same readings as wkv6_fwd_gn (one group per head of 64 channels,
 * biased variance, eps inside the root, g after its SiLU).
 *
 *   B, T, C, H    as wkv6_fwd (C = 64 * H)
 *   y       device pointer to [B, T, C] float32
 *   g       device pointer to [B, T, C] values of `dtype`
 *   gamma, beta   device pointers to C float32 values each
 *   eps     finite and >= 0 (else INVALID_ARG)
 *   out     device pointer to a [B, T, C] bfloat16 output (nearest even);
 *           must not overlap any input
 *
 * Allocates nothing; execution and errors as wkv6_fwd.
 */
int wkv6_group_norm_gate(int64_t B, int64_t T, int64_t C, int64_t H, const float* y, const void* g,
                         const float* gamma, const float* beta, float eps, void* out, int dtype,
                         void* stream);

/*
 * wkv5_fwd -- the RWKV-5 ("Eagle") operator: the same matrix-state recurrence
 * and output as wkv6_fwd, with a decay that is a fixed per-channel parameter
 * instead of a per-token input ("RWKV Architecture" on llms.blog, section
 * "RWKV-5 Eagle": each head's 64x64 state decays by exp(-w) per step, with w
 * a learned vector; RWKV-6 made w depend on the token).
 *
 *   w_raw   device pointer to C values of `dtype`, laid out [H, 64]: every
 *           token uses w[c] = exp(-exp(w_raw[c])), i.e. the pages' w is
 *           exp(w_raw).  Same supported range as wkv6_fwd.
 *   Every other argument, the workspace, execution and errors: as wkv6_fwd
 *   (y must not overlap the C values of w_raw either).
 */
int wkv5_fwd(int64_t B, int64_t T, int64_t C, int64_t H,
             const void* r, const void* k, const void* v, const void* w_raw,
             const float* u, float* y, int mode, int dtype, void* stream);

/*
 * wkv4_fwd -- the RWKV-4 operator: a normalised weighted average of the
 * values with one independent recurrence per channel ("RWKV Architecture"
 * on llms.blog, section "The Fundamental Mathematical Duality", the baseline
 * WKV formula, and "The Recurrent Inference Formulation"):
 *
 *   WKV_t[c] = ( sum_{i<t} e^{-(t-1-i) w[c] + k_i[c]} v_i[c] + e^{u[c] + k_t[c]} v_t[c] )
 *            / ( sum_{i<t} e^{-(t-1-i) w[c] + k_i[c]}        + e^{u[c] + k_t[c]} )
 *
 * Causal only (the pages give no bidirectional form); no heads.
 *
 *   B, T, C   batch, tokens, channels (any C >= 0).
 *   k, v      device pointers to contiguous row-major [B, T, C] tensors of
 *             `dtype` (WKV6_DTYPE_F32 or WKV6_DTYPE_BF16).
 *   w         device pointer to C float32 decay rates: every step multiplies
 *             the history by exp(-w) (the pages take w >= 0; +inf keeps
 *             only the previous token; -inf and NaN are not supported).
 *   u         device pointer to C float32 bonuses of the current token.
 *   y         device pointer to a [B, T, C] float32 output, fully
 *             overwritten; must not overlap k, v, w or u.
 *   stream    a hipStream_t passed as void* (NULL = the null stream).
 *
 * The kernels keep each channel's numerator and denominator scaled by the
 * largest exponent seen so far, so any finite keys work in float32.  Long
 * sequences over few channels are cut into segments; such calls take a
 * temporary device workspace of 2 * B * segments * 3 * C * 4 bytes,
 * allocated and released in stream order from the library's pool (as wkv6_fwd).
 * Ownership, execution and errors as wkv6_fwd (status codes, nothing
 * enqueued on a failed check, values not checked); B, T or C = 0 is a no-op.
 */
int wkv4_fwd(int64_t B, int64_t T, int64_t C, const void* k, const void* v,
             const float* w, const float* u, float* y, int dtype, void* stream);

/*
 * wkv6_fwd_state -- a causal forward that starts from a given state and hands
 * back the state after the last token, for processing a sequence in pieces
 * (streaming, or decoding one token at a time).  The pages describe the
 * state as the operator's whole memory, updated token by token and kept
 * between calls at inference ("RWKV Architecture" on llms.blog, sections
 * "The Recurrent Inference Formulation" and "RWKV-5 Eagle"; the yarian.com
 * RWKV page, section "7. Hidden State = Persistent Memory").
 *
 * Same operator and arguments as wkv6_fwd in causal mode, except that the
 * state starts at s_in instead of zero:
 *
 *     y_t[n] = sum_c r_t[c] * ( S[c][n] + u[c] * k_t[c] * v_t[n] )
 *     S[c][n] <- w_t[c] * S[c][n] + k_t[c] * v_t[n],   S = s_in before token 0
 *
 * and s_out receives S after token T-1.  Splitting a sequence at any token
 * and passing s_out of the first piece as s_in of the second gives the same
 * y and final state as one call (up to rounding).
 *
 *   s_in    device pointer to B*H float32 64x64 states, [B, H, 64, 64]
 *           row-major: element [b][h][c][n] is the state entry of key
 *           channel c and value channel n of head h.  NULL: zero state.
 *   s_out   device pointer to a [B, H, 64, 64] float32 output in the same
 *           layout, or NULL (final state not wanted).  Must not overlap
 *           s_in, y or any input: successive calls alternate two buffers.
 *   T       may be 0: then y, r, k, v, w_raw and u are not used and s_out
 *           (if given) receives s_in (zeros when s_in is NULL).
 *
 * Other arguments, ownership, execution and errors as for wkv6_fwd; the
 * state pointers must be 16-byte aligned (MISALIGNED otherwise) and their
 * overlaps give INVALID_ARG.  Bidirectional mode has no state passing (its
 * later-token part needs the whole sequence).
 */
int wkv6_fwd_state(int64_t B, int64_t T, int64_t C, int64_t H,
                   const void* r, const void* k, const void* v, const void* w_raw,
                   const float* u, float* y, const float* s_in, float* s_out,
                   int dtype, void* stream);

/*
 * wkv6_bwd -- gradients of L = sum(y * dy) for y = the wkv6_fwd result, for
 * training.  The pages' CUDA extension has a backward kernel next to the
 * forward one that returns the gradients of all five inputs (CUDA-kernels
 * page of deepglint/rwkv-clip, section "Backward Pass Gradient
 * Computation"); the steps here are derived from the recurrence above.
 *
 *   r, k, v, w_raw, u, B, T, C, H, mode, dtype
 *           as for wkv6_fwd (same layouts and types).
 *   dy      device pointer to the float32 [B, T, C] gradient of y.
 *   dr, dk, dv, dw_raw
 *           device pointers to float32 [B, T, C] outputs (always float32,
 *           whatever dtype): dL/dr, dL/dk, dL/dv and dL/dw_raw (the
 *           derivative through w = exp(-exp(w_raw))).  Fully overwritten.
 *   du      device pointer to a float32 [C] output: dL/du summed over the
 *           batch and the tokens.  T == 0 sets it to zero.
 *
 * B == 0 is a no-op.  The outputs must not overlap one another or any input
 * (INVALID_ARG).  Two kernel families compute the same result:
 *   - bf16 calls with T >= 64 that run unsegmented (at least 256 (batch,
 *     head) pairs, or T < 128) run in chunks of 64 tokens on matrix cores: a pass stores every chunk's
 *     entering state, then a reverse pass with the adjoint in registers
 *     writes the gradients (operands carried as three bf16 parts, float32
 *     accumulation; within about 1e-5 of the output's rms).  A (batch, head)
 *     pair with a 16-token block that decays by 2^-24 or more in some
 *     channel is recomputed by the other family.
 *   - every other call runs two token-by-token passes per (batch, head) in
 *     float32.  With fewer than 256 (batch, head) pairs it cuts each
 *     sequence into up to 63 segments (whole 16-token blocks, at least 64
 *     tokens each): a summary pass then gives each segment its entering
 *     state and leaving adjoint, and a last pass completes the decay
 *     gradient across segments.
 * Workspace (stream-ordered, from the library's pool as for wkv6_fwd):
 * B*segments*C*4 bytes, plus B*T*C*4 in bidirectional mode, plus
 * B*H*segments*(4*64*64 + 2*64)*4 per direction when segmented, plus, on
 * the chunked kernels, B*H*ceil(T/64)*64*64*4 bytes of chunk states per
 * direction and B*H*4 bytes of flags.  Errors otherwise as for wkv6_fwd.
 */
int wkv6_bwd(int64_t B, int64_t T, int64_t C, int64_t H,
             const void* r, const void* k, const void* v, const void* w_raw,
             const float* u, const float* dy, float* dr, float* dk, float* dv,
             float* dw_raw, float* du, int mode, int dtype, void* stream);

/* Static text for a status code (never NULL). */
const char* wkv6_status_str(int status);

/* Detail of the last error on the calling thread ("" if none). */
const char* wkv6_last_error(void);

/* WKV6_ABI_VERSION of the loaded library. */
int wkv6_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WKV6_H */

/*
 * mamba_scan.h -- C ABI of the MI355X (gfx950) Mamba-1 selective scan (S6)
 * forward pass and the single-token selective state update, the backward pass
 * of the scan, and the causal depthwise conv1d + SiLU that produces the scan
 * input with its one-token update (the last two groups declared last).
 *
 * What the calls compute (pages cited by title and section):
 *   "Mamba 模型" (gaos6e.github.io), full-step flowchart nodes H to M and
 *     their step notes: delta = softplus(delta_raw + bias); Abar = exp(delta A);
 *     Bbar from (delta, A, B); h_t = Abar h_{t-1} + Bbar u_t;
 *     y_t = C_t h_t + D u_t; output gated by z * sigmoid(z).
 *   "Mamba模型：高效序列建模的新突破" (mhpn.cn) section 3.1 and
 *   "Mamba 状态空间模型架构深度解析" (pnsm.cn) "状态空间模型（SSM）基础":
 *     zero-order hold, Abar = exp(delta A), Bbar = (Abar - 1) A^-1 B, with A
 *     diagonal ("Mamba-1：选择性状态空间"), so per state n:
 *     Bbar_n = (exp(delta A_n) - 1) / A_n * B_n  (limit delta * B_n at A_n = 0).
 *   "Mamba 与状态空间模型" (world.lapla.si, plate F56), "模型省略了什么": the
 *     simplified rule Bbar = delta * B, selectable with MAMBA_FLAG_DELTA_B.
 *   Same page, section 07: the scan is fused -- inputs are read once from
 *     HBM, discretisation and the recurrence stay on chip, only y (and the
 *     final state, when asked for) is written back.  The (B, D, L, N) state
 *     is never materialised.
 *   "Mamba 模型", "为什么 Mamba 推理更省": decoding updates a fixed-size state
 *     one token at a time (mamba_state_update).
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller, to dense
 *     row-major data on the device that `stream` belongs to.  The library keeps
 *     no reference to any pointer after the call returns.
 *   - The library allocates nothing.  The scan's scratch memory is the
 *     caller's `workspace` (size from mamba_scan_workspace_size).
 *   - All argument checks run on the host before any HIP call; a failed check
 *     returns a negative mamba_status_t and launches nothing.
 *   - Work is enqueued on `stream` and runs asynchronously; MAMBA_OK means the
 *     launches were accepted.  A fault inside a kernel surfaces at the
 *     caller's next synchronisation with the stream.
 *   - Outputs must not alias inputs (except `state`, which is updated in
 *     place by design).  Calls that share an output or a workspace must not
 *     run concurrently.
 *   - No C++ exception crosses this interface.  The only process-wide state
 *     is a per-device cache of the compute-unit count (read once), an atomic
 *     launch counter that tags the scan's hand-over slots in the workspace,
 *     so a workspace is reused without being cleared, and the test knobs of
 *     mamba_set_test_knobs.  Concurrent calls on different streams with
 *     disjoint buffers (workspaces included) are safe.
 *   - Graph capture: every call may be recorded into a HIP graph.  A scan
 *     recorded while its stream is capturing clears its hand-over flags with
 *     a small kernel of its own before the scan kernel, so every replay starts
 *     from cleared flags (a replay cannot take a new launch tag from the
 *     host).
 *   - Supported sizes: 1 <= N <= 16; B, D, L >= 1; B*D*L < 2^46.
 *   - Arithmetic is fp32 throughout (state, discretisation, accumulation);
 *     bf16 inputs are widened exactly, outputs are rounded to nearest-even.
 */
#ifndef MAMBA_SCAN_H_
#define MAMBA_SCAN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MAMBA_F32 = 0,   /* IEEE binary32 */
  MAMBA_BF16 = 1   /* bfloat16, stored as 16-bit patterns */
} mamba_dtype_t;

typedef enum {
  MAMBA_OK = 0,
  MAMBA_ERR_NULL = -1,          /* a required pointer is NULL */
  MAMBA_ERR_SHAPE = -2,         /* a size is <= 0 or the problem is too large */
  MAMBA_ERR_DTYPE = -3,         /* unknown dtype */
  MAMBA_ERR_ALIGN = -4,         /* a pointer is not 16-byte aligned */
  MAMBA_ERR_UNSUPPORTED = -5,   /* N > 16, or an unknown flag bit */
  MAMBA_ERR_WORKSPACE = -6,     /* workspace NULL or smaller than required */
  MAMBA_ERR_HIP = -7            /* a HIP launch or runtime call failed */
} mamba_status_t;

/* Flag bits (the `flags` argument of both calls). */
#define MAMBA_FLAG_DELTA_B 0x1u          /* Bbar = delta * B instead of zero-order hold */
#define MAMBA_FLAG_ACCURATE_EXPM1 0x2u   /* force the cancellation-free (Abar - 1) path;
                                            always on in mamba_state_update and, in
                                            mamba_scan_fwd and mamba_scan_bwd, when
                                            in_dtype is MAMBA_F32 or for the channels
                                            of a 16-channel tile (64 for L % 8 != 0
                                            or L < 32)
                                            with some |A| < 1/16 */

/*
 * Bytes of device workspace mamba_scan_fwd needs for a problem of this shape.
 * Depends only on the shape (no device query, callable without a GPU).
 * Returns 0 when the shape is scanned in one pass per channel (no scratch),
 * and (size_t)-1 for an invalid shape.
 */
size_t mamba_scan_workspace_size(int64_t B, int64_t D, int64_t N, int64_t L);

/*
 * The kernel mamba_scan_fwd runs for a problem of this shape (shape only, no
 * device query; callable without a GPU), or a negative status for an invalid
 * shape:
 *   MAMBA_KERNEL_GENERAL    64 channels per 4-wave workgroup, L staged in
 *                           32-step chunks through LDS (L < 32);
 *   MAMBA_KERNEL_WAVE_TILE  16 channels per wave, 16 states per lane-quad,
 *                           optionally chunked along L or balanced over the
 *                           SIMDs with state hand-over (L % 8 == 0, L >= 32);
 *                           chosen for very few 16-channel tiles over a long L;
 *   MAMBA_KERNEL_ROW        16 channels per 4-wave workgroup, one state per
 *                           lane, one pass or two over chunks of L with a
 *                           carry between them; chosen when the wave tiles
 *                           would leave SIMDs idle or need chunking, and,
 *                           by a cost model, for L % 32 != 0 (element loads
 *                           and a shifted last chunk);
 *   MAMBA_KERNEL_ROW_LEAN   the same layout with fewer registers and less LDS
 *                           per workgroup (five workgroups per CU instead of
 *                           three), chosen from four 16-channel workgroups
 *                           per CU on (L % 32 == 0).
 * The row kernels step each workgroup's issue priority down as it advances
 * through L, so that the workgroups sharing a CU finish together.
 * The choice depends on the shape only; every kernel computes the same
 * result to fp32 rounding.
 */
#define MAMBA_KERNEL_GENERAL 1
#define MAMBA_KERNEL_WAVE_TILE 2
#define MAMBA_KERNEL_ROW 3
#define MAMBA_KERNEL_ROW_LEAN 4
int mamba_scan_kernel(int64_t B, int64_t D, int64_t N, int64_t L);

/*
 * Selective scan forward over a whole sequence.
 *
 *   u, delta, z : (B, D, L) in_dtype.  `delta` is the raw step before the bias
 *                 and softplus.  z may be NULL: then no gate is applied.
 *   Bt, Ct      : (B, N, L) in_dtype, one B_t / C_t per batch row and token,
 *                 shared by all D channels.
 *   A           : (D, N) fp32, the diagonal state matrix of each channel.
 *   Dskip       : (D) fp32 or NULL (treated as zeros).
 *   delta_bias  : (D) fp32 or NULL (treated as zeros); added before softplus.
 *   y           : (B, D, L) out_dtype, written.
 *   final_state : (B, D, N) fp32, written iff return_final_state != 0
 *                 (must then be non-NULL; ignored otherwise).
 *   workspace   : scratch of at least mamba_scan_workspace_size(B, D, N, L)
 *                 bytes (may be NULL when that size is 0); contents on entry
 *                 are ignored (hand-over slots are tagged with a per-launch
 *                 64-bit value, so stale contents are never mistaken for
 *                 this launch's), contents on exit are unspecified.
 *   flags       : MAMBA_FLAG_* bits.
 *
 * The initial state is zero.  Alignment: u, delta, z, Bt, Ct, y must be
 * 16-byte aligned; A, Dskip, delta_bias and final_state 4-byte aligned.
 */
int mamba_scan_fwd(const void* u, const void* delta, const void* z,
                   const void* Bt, const void* Ct, const float* A,
                   const float* Dskip, const float* delta_bias,
                   void* y, float* final_state,
                   int64_t B, int64_t D, int64_t N, int64_t L,
                   mamba_dtype_t in_dtype, mamba_dtype_t out_dtype,
                   int return_final_state, unsigned flags,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mamba_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of mamba_scan_fwd.  The scratch memory the scan needs (hand-over slots of
 * the balanced split, chunk carries of long sequences) comes from a buffer
 * the library holds in device memory, one per GPU, 8 MiB, kept until the
 * process ends; this call allocates nothing.  A shape whose plan needs more
 * (mamba_scan_workspace_size above 8 MiB, e.g. very long sequences over many
 * channels) returns MAMBA_ERR_WORKSPACE and launches nothing.  The buffer is
 * shared by every call on that GPU: calls of this function that overlap in
 * time on one GPU (different streams, or host threads) race and give wrong
 * results; serialise them.  The stream must belong to the current device.
 */
int mamba_scan_fwd_noalloc(const void* u, const void* delta, const void* z,
                           const void* Bt, const void* Ct, const float* A,
                           const float* Dskip, const float* delta_bias,
                           void* y, float* final_state,
                           int64_t B, int64_t D, int64_t N, int64_t L,
                           mamba_dtype_t in_dtype, mamba_dtype_t out_dtype,
                           int return_final_state, unsigned flags, hipStream_t stream);

/*
 * One decoding step for every (b, d): the scan above with L = 1, starting
 * from `state` instead of zero.
 *
 *   state       : (B, D, N) fp32, read and overwritten in place with h_t.
 *   u, delta, z : (B, D) in_dtype (z may be NULL: no gate).
 *   Bt, Ct      : (B, N) in_dtype.
 *   A           : (D, N) fp32.  Dskip, delta_bias : (D) fp32 or NULL.
 *   y           : (B, D) out_dtype, written.
 *
 * Alignment: state, A 16-byte aligned; the rest 4-byte (fp32) or 2-byte
 * (bf16) aligned.  No workspace is used.
 */
int mamba_state_update(float* state, const void* u, const void* delta, const void* z,
                       const void* Bt, const void* Ct, const float* A,
                       const float* Dskip, const float* delta_bias, void* y,
                       int64_t B, int64_t D, int64_t N,
                       mamba_dtype_t in_dtype, mamba_dtype_t out_dtype,
                       unsigned flags, hipStream_t stream);

/*
 * Bytes of device workspace mamba_scan_bwd needs (shape only; callable
 * without a GPU), (size_t)-1 for an invalid shape.  It holds fp32 chunk-start
 * states (one per 8 steps), the segment summaries and carries, and per-tile
 * partial sums of dB_t / dC_t: about 18 bytes per (B, D, L) element for
 * D = 5120, N = 16.
 */
size_t mamba_scan_bwd_workspace_size(int64_t B, int64_t D, int64_t N, int64_t L);

/*
 * Backward pass of mamba_scan_fwd (initial state zero): the gradients of all
 * inputs for an output gradient dy.  The states are recomputed from the inputs
 * rather than read back ("Mamba论文研读笔记" 3.2.3 C, recomputation;
 * "Mamba 与状态空间模型" section 07).
 *
 *   u, delta, z, Bt, Ct, A, Dskip, delta_bias : as for mamba_scan_fwd
 *                 (in_dtype; z, Dskip, delta_bias may be NULL).
 *   dy          : (B, D, L) grad_dtype, gradient of y.
 *   du, ddelta  : (B, D, L) grad_dtype, written; ddelta is the gradient of
 *                 the raw delta (before bias and softplus).
 *   dz          : (B, D, L) grad_dtype, written; required iff z is given.
 *   dBt, dCt    : (B, N, L) fp32, written (summed over the D channels).
 *   dA          : (D, N) fp32; dDskip, ddelta_bias : (D) fp32, written
 *                 (summed over batch rows and time), also when Dskip or
 *                 delta_bias is NULL.
 *   flags       : MAMBA_FLAG_DELTA_B selects the simplified rule, and
 *                 MAMBA_FLAG_ACCURATE_EXPM1 the cancellation-free (Abar - 1)/A
 *                 for bf16 inputs, as in the forward pass (fp32 inputs, and a
 *                 16-channel tile holding a |A| < 1/16, always take it).
 *   workspace   : at least mamba_scan_bwd_workspace_size bytes, 256-byte
 *                 aligned; contents on entry ignored.
 *
 * Alignment: the dtype inputs and gradients to their element size; fp32
 * arrays 4-byte.  All outputs are overwritten (not accumulated into); the
 * result is deterministic (fixed-order reductions).  1 <= N <= 16.
 */
int mamba_scan_bwd(const void* u, const void* delta, const void* z, const void* Bt, const void* Ct,
                   const float* A, const float* Dskip, const float* delta_bias, const void* dy,
                   void* du, void* ddelta, void* dz, float* dBt, float* dCt, float* dA, float* dDskip,
                   float* ddelta_bias, int64_t B, int64_t D, int64_t N, int64_t L,
                   mamba_dtype_t in_dtype, mamba_dtype_t grad_dtype, unsigned flags,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Causal depthwise convolution along the sequence, then SiLU: the step that
 * produces the scan input u.
 *   "Mamba 模型", full-step flowchart node E: Uc_t = sum_i W_i U_(t-i), one
 *     filter per channel over the current and earlier positions only; node F:
 *     u_t = Uc_t * sigmoid(Uc_t).
 *   "Mamba 与状态空间模型", section 03: each channel also keeps its short
 *     convolution's most recent inputs (4 for Mamba) between tokens.
 *
 *   x           : (B, D, L) in_dtype.
 *   weight      : (D, K) fp32; weight[d*K + i] multiplies x[b, d, t - i]
 *                 (i = 0 is the current position).
 *   bias        : (D) fp32 or NULL (no bias); added before SiLU.
 *   y           : (B, D, L) out_dtype, written: silu of the convolution.
 *   final_state : (B, D, K) fp32, written iff return_final_state != 0: the K
 *                 most recent inputs x[b, d, L-K .. L-1], oldest first (zero
 *                 where L - K + k < 0) -- the state mamba_conv1d_update
 *                 continues from.  Ignored (may be NULL) otherwise.
 *
 * Positions before t = 0 read zero.  1 <= K <= 4 (MAMBA_ERR_UNSUPPORTED
 * above).  Alignment: x, y to their element size (16 bytes, with L % 8 == 0,
 * selects the vectorised kernel); weight, bias, final_state 4-byte.
 */
int mamba_conv1d_fwd(const void* x, const float* weight, const float* bias, void* y, float* final_state,
                     int64_t B, int64_t D, int64_t L, int64_t K,
                     mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state,
                     hipStream_t stream);

/*
 * One decoding step of the convolution for every (b, d).
 *
 *   state  : (B, D, K) fp32, read and overwritten in place: on entry the K
 *            most recent inputs (oldest first), on return the K most recent
 *            including x.
 *   x      : (B, D) in_dtype, the new input.
 *   weight : (D, K) fp32, as in mamba_conv1d_fwd.  bias : (D) fp32 or NULL.
 *   y      : (B, D) out_dtype, written: silu(sum_i weight[d*K+i] * x_(t-i) + bias).
 *
 * 1 <= K <= 4.  Alignment: state, weight, bias 4-byte (state 16-byte with
 * K = 4 selects vector accesses); x, y to their element size.  No workspace.
 */
int mamba_conv1d_update(float* state, const void* x, const float* weight, const float* bias, void* y,
                        int64_t B, int64_t D, int64_t K, mamba_dtype_t in_dtype, mamba_dtype_t out_dtype,
                        hipStream_t stream);

/*
 * Mamba-2 layer forward (state space duality), one scalar A per head.
 *   "Mamba 与状态空间模型" section 09 and "Mamba 状态空间模型架构深度解析"
 *   (Mamba-2): with A a scalar times the identity, a layer multiplies the
 *   sequence by a lower-triangular matrix, entry (t, s) = C_t . B_s times the
 *   decay between steps s and t times B-bar's coefficient; it is computed in
 *   chunks, with matrix products inside a chunk and the state passed between
 *   chunks.  Per head h of P channels (channel d = h P + p):
 *     delta_t = softplus(delta_raw[b,h,t] + delta_bias[h]),
 *     h_t = exp(delta_t A[h]) h_(t-1) + coef_t B_t x_t  (state N per channel,
 *     coef = (exp(delta A) - 1)/A, or delta with MAMBA_FLAG_DELTA_B),
 *     y_t = (C_t . h_t + Dskip[d] x_t) * silu(z_t)  (no gate when z is NULL).
 *
 *   x, z        : (B, H*P, L) bf16; z may be NULL.
 *   delta       : (B, H, L) bf16, raw step sizes, one per head.
 *   Bt, Ct      : (B, N, L) bf16, shared by all heads.
 *   A           : (H) fp32.  Dskip : (H*P) fp32 or NULL.  delta_bias : (H) fp32 or NULL.
 *   y           : (B, H*P, L) out_dtype (bf16 or fp32), written.
 *   final_state : (B, H*P, N) fp32, written iff return_final_state.
 *
 *   workspace   : at least mamba_ssd_workspace_size bytes (may be NULL when
 *                 that is 0), 256-byte aligned; contents on entry ignored.
 *
 * in_dtype must be MAMBA_BF16 (MAMBA_ERR_UNSUPPORTED otherwise); N must be 64
 * or 128 and P a multiple of 64 (MAMBA_ERR_UNSUPPORTED).  Alignment: bf16
 * arrays 2-byte, fp32 arrays 4-byte (16-byte pointers and L % 8 == 0 select
 * vector accesses).  The initial state is zero.
 */
int mamba_ssd_fwd(const void* x, const void* delta, const void* z, const void* Bt, const void* Ct,
                  const float* A, const float* Dskip, const float* delta_bias, void* y, float* final_state,
                  int64_t B, int64_t H, int64_t P, int64_t N, int64_t L,
                  mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state,
                  unsigned flags, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace mamba_ssd_fwd needs (shape only; callable without
 * a GPU): L is cut into segments that run in parallel, and the workspace
 * holds each segment's fp32 end state (N per channel) and decay.  0 when one
 * segment suffices; (size_t)-1 for an invalid or unsupported shape.
 */
size_t mamba_ssd_workspace_size(int64_t B, int64_t H, int64_t P, int64_t N, int64_t L);

/*
 * Test and diagnostic knobs.  They change how a call is carried out, never
 * what it computes (every setting gives the same result to fp32 rounding --
 * summation order, and on the fast ZOH quotient the row kernels' state scaled
 * by A -- and the hand-over settings bit for bit).  Process-wide:
 * every later call uses them, so a workspace size queried before a change
 * does not fit a launch after it.  Not for production use.
 *
 *   scan_chunks           > 0: mamba_scan_fwd cuts L into this many chunks
 *                         (summary pass, carry, full pass) whatever the shape;
 *                         0: the planner decides.
 *   scan_kernel           which kernel mamba_scan_fwd runs: 0 the planner's
 *                         choice; 1 the general 64-channel kernel (normally
 *                         only for L < 32); 2 the wave-tile kernel with 16
 *                         states per lane (L % 8 == 0, L >= 32); 3 the row
 *                         kernel with one state per lane (L >= 32); 4 its
 *                         lean variant (L % 32 == 0; the row kernel at other
 *                         L).  A kernel that cannot take the shape gives way
 *                         to the planner's choice.
 *   scan_no_balance       != 0: no balanced split with state hand-over.
 *   handover_spin         >= 0: bound of a workgroup's wait for the state handed
 *                         over by the previous one, in polls (0: every split
 *                         tile recomputes its state instead of waiting);
 *                         < 0: the default, max(8192, 256 polls per 32-step
 *                         block of a workgroup's share).
 *   ssd_segments          > 0: mamba_ssd_fwd cuts L into this many segments
 *                         (at most one per 32 steps); 0: the planner decides.
 *
 * mamba_set_test_knobs(NULL) restores the defaults {0, 0, 0, -1, 0}.
 * Returns MAMBA_ERR_SHAPE for a negative chunk or segment count.
 */
typedef struct {
  int64_t scan_chunks;
  int32_t scan_kernel;
  int32_t scan_no_balance;
  int64_t handover_spin;
  int64_t ssd_segments;
} mamba_test_knobs_t;

int mamba_set_test_knobs(const mamba_test_knobs_t* knobs);

/* Static, human-readable text for a status code (never NULL). */
const char* mamba_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MAMBA_SCAN_H_ */

// kernels.hpp -- launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mamba {

enum class Dt : int { F32 = 0, BF16 = 1 };

// Discretisation variants of the inner loop (chosen per wave at run time).
enum LoopMode : int {
  kZohFast = 0,      // (Abar - 1) / A as fma(Abar, 1/A, -1/A)
  kZohAccurate = 1,  // (Abar - 1) from a series for small |delta A|
  kDeltaB = 2        // simplified rule Bbar = delta * B
};

// kZohFast rounds Abar before subtracting 1, so B-bar carries a relative
// error of about 1.2e-7 / (delta |A|): 1.2e-5 at |A| = 1, delta = 0.01, but
// all of it once delta |A| nears 2^-24.  A wave takes kZohAccurate instead
// when one of its |A| is below this bound.  At the bound the per-step error
// is up to 1.9e-3 for delta = 1e-3; a state averages these independent
// errors over about 1 / (delta |A|) steps, so the state and y carry about
// 1.2e-7 / sqrt(delta |A|) = 1.5e-5 there.
constexpr float kFastZohMinAbsA = 0x1p-4f;

struct ScanParams {
  const void* u;
  const void* delta;
  const void* z;        // may be null
  const void* Bt;
  const void* Ct;
  const float* A;
  const float* Dskip;   // may be null
  const float* bias;    // may be null
  void* y;
  float* final_state;   // may be null
  int64_t B, D, N, L;
  int64_t tiles_d;      // ceil(D / 64)
  int64_t n_chunks;     // L-chunks per channel tile (1 = whole sequence in one pass)
  int64_t chunk_len;    // time steps per chunk, a multiple of the staging chunk
  float* h_local;       // (n_chunks, B, D, N): chunk end states from a zero start
  float* s_sum;         // (n_chunks, B, D): sum of delta over each chunk
  float* h_start;       // (n_chunks, B, D, N): true start state of each chunk
  int accurate;         // force the accurate (Abar - 1) loop
  int delta_b;          // simplified discretisation
  int vec;              // rows are 16-byte aligned multiples of 8 elements
};

// Extra parameters of the wave-tile scan kernel (scan_v4.hpp, L % 8 == 0, L >= 32).
struct V2Params {
  int balanced;          // 1: equal (tile x time) ranges per workgroup with state hand-over
  int64_t groups;        // workgroups in balanced mode
  uint64_t epoch;        // value that marks a hand-over slot as published by this launch
  uint32_t spin_limit;   // bounded wait for a hand-over before recomputing it
  float* pub_state;      // (groups, 64, 16) fp32 hand-over states
  uint64_t* pub_flag;    // (groups) epoch flags
};

struct UpdateParams {
  float* state;
  const void* u;
  const void* delta;
  const void* z;
  const void* Bt;
  const void* Ct;
  const float* A;
  const float* Dskip;
  const float* bias;
  void* y;
  int64_t B, D, N;
  double inv_d;    // 1.0 / D
  int accurate;
  int delta_b;
};

// Causal depthwise conv1d (+ SiLU) and its one-token update.
struct ConvParams {
  const void* x;          // (rows, L) or (rows) for the update
  const float* w;         // (D, K)
  const float* bias;      // (D) or null
  void* y;                // like x
  float* final_state;     // (rows, K) or null (forward)
  float* state;           // (rows, K) in/out (update)
  int64_t rows, D, L, K;  // rows = B * D
};

// Issue priority from progress (s_setprio).  A SIMD issues to the oldest
// ready wave first, so co-resident workgroups that run the same long loop
// finish one after another, and the last one runs its end alone, with its
// latencies uncovered.  A wave that steps its priority down as it advances
// through its range (3 before 1/2, 2 before 3/4, 1 before 7/8, then 0)
// lets the workgroups behind it catch up at each step, so that they stay
// within an eighth of the range of each other and finish nearly together.
// It changes only the order of issue, never what is computed.
struct ProgressPrio {
  int lvl = 0;
  __device__ __forceinline__ void begin() { __builtin_amdgcn_s_setprio(3); }
  // done of total units of the wave's range are behind it (uniform over the
  // wave).  With 32-bit unsigned counts (total < 2^29) the compares run on the
  // scalar unit; 64-bit signed ones need the vector unit.
  template <typename T>
  __device__ __forceinline__ void at(T done, T total) {
    const T a = 8 * done;
    const int l = a >= 7 * total ? 3 : a >= 6 * total ? 2 : a >= 4 * total ? 1 : 0;   // scalar selects
    if (l != lvl) {
      lvl = l;
      if (l == 1) __builtin_amdgcn_s_setprio(2);
      else if (l == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
  }
};

// Backward pass of the scan.
// Backward pass: L is cut into segments of seg_len steps (a multiple of
// kBwdChunk); each segment is cut into chunks of kBwdChunk steps, the unit
// that is recomputed on chip.
constexpr int kBwdChunk = 8;
// Steps staged at a time (four chunks); the summary pass stores one state per
// channel at the start of each such block.
constexpr int kBwdBlock = 4 * kBwdChunk;
// 16-channel tiles per workgroup of the backward segment pass; the workgroup
// sums its tiles' dB_t / dC_t contributions before storing one partial.
constexpr int kBwdGroup = 4;

struct BwdParams {
  const void *u, *delta, *z, *Bt, *Ct, *dy;
  const float *A, *Dskip, *bias;
  void *du, *ddelta, *dz;                       // grad dtype, (B, D, L)
  float *dBt, *dCt, *dA, *dDskip, *dbias;       // fp32 results
  float *ckpt_h;                                // (B, nck, D, 16) block-start states from a zero segment start
  float *ckpt_cd;                               // (B, nck, D) sum of delta from the segment start to the block
  float *seg_P, *seg_h, *seg_H;                 // (B, S, D, 16) segment summaries
  float *h_in, *g_in;                           // (B, S, D, 16) state entering / adjoint leaving each segment
  float *part_dB, *part_dC;                     // (B, groups, 16, L) sums over a workgroup's channels
  float *part_dA, *part_dD, *part_dbias;        // (B, S, D, 16), (B, S, D), (B, S, D) per-segment sums
  int64_t B, D, N, L, tiles_d, nck, S, seg_len;   // nck: kBwdBlock-step blocks over L
  int64_t groups;                               // ceil(tiles_d / kBwdGroup)
  int delta_b;
  int accurate; // cancellation-free (Abar - 1)/A for bf16 inputs too
  int vec;      // L % 8 == 0 and every (B, D, L) / (B, N, L) array 16-byte aligned
};

// Mamba-2 (SSD) layer forward: H heads of P channels, one scalar A per head.
struct SsdParams {
  const void *x, *delta, *z, *Bt, *Ct;          // bf16: x, z (B, H P, L); delta (B, H, L); Bt, Ct (B, N, L)
  const float *A, *Dskip, *bias;                // (H), (H P), (H)
  void* y;                                      // (B, H P, L) out dtype
  float* final_state;                           // (B, H P, N) or null
  float* ws_h;                                  // per (b, segment, h, 64-channel block): [64][N] states (S > 1)
  float* ws_P;                                  // per segment slot: decay over the segment (S > 1)
  int64_t B, H, P, N, L;
  int64_t S, seg_len;                           // segments of L (multiple of 32 steps)
  int delta_b;
  int vec;      // L % 8 == 0 and every pointer 16-byte aligned
};

// Each returns hipSuccess or the launch error.
hipError_t launch_scan_full(const ScanParams& p, Dt in, Dt out, hipStream_t s);
hipError_t launch_scan_summary(const ScanParams& p, Dt in, hipStream_t s);
hipError_t launch_scan_carry(const ScanParams& p, hipStream_t s);
hipError_t launch_clear_u64(uint64_t* p, int64_t n, hipStream_t s);
hipError_t launch_scan_v4(const ScanParams& p, const V2Params& q, Dt in, Dt out, bool summary, hipStream_t s);
// phase 0: whole sequences; 1 and 2: the two passes over L in p.n_chunks
// chunks (before and after the carry kernel), not for the lean variant.
hipError_t launch_scan_row(const ScanParams& p, Dt in, Dt out, bool lean, int phase, hipStream_t s);
hipError_t launch_state_update(const UpdateParams& p, Dt in, Dt out, hipStream_t s);
hipError_t launch_scan_bwd(const BwdParams& p, Dt in, Dt grad, hipStream_t s);
hipError_t launch_conv1d_fwd(const ConvParams& p, Dt in, Dt out, bool vec, hipStream_t s);
hipError_t launch_conv1d_update(const ConvParams& p, Dt in, Dt out, hipStream_t s);
hipError_t launch_ssd(const SsdParams& p, Dt out, hipStream_t s);

}  // namespace mamba

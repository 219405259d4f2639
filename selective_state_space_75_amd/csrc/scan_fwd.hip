// scan_fwd.hip -- selective scan (S6) forward kernels for gfx950.
//
// What is computed ("Mamba 模型", full-step flowchart nodes H to M; ZOH from
// "Mamba模型：高效序列建模的新突破" 3.1 and "Mamba 状态空间模型架构深度解析"):
//   delta = softplus(delta_raw + bias_d)
//   Abar_n = exp(delta A_dn),  Bbar_n = (Abar_n - 1) / A_dn * B_n   (ZOH)
//   h_n  <- Abar_n h_n + Bbar_n u
//   y     = (sum_n C_n h_n + D_d u) * silu(z)
//
// How it is laid out on the GPU (the fused-kernel idea of "Mamba 与状态空间模型"
// section 07 -- inputs read once, state kept on chip, only y written -- mapped
// to CDNA4 rather than copied from the A100 design):
//   * one workgroup = one batch row b x a tile of 64 channels, one channel per
//     lane; the N <= 16 states of a channel are split over 4 waves (4 states
//     per wave), held in VGPRs for the whole sequence;
//   * the sequence is walked in chunks of 32 steps.  Per chunk the workgroup
//     stages u and delta (softplus applied once per element) channel-major in
//     LDS, and B_t / C_t (shared by all channels of the row) state-major;
//   * each wave runs the recurrence for its states and writes a partial
//     readout per (channel, step) to LDS; the workgroup then sums the four
//     partials, adds D u, applies the gate, and stores y with coalesced
//     16-byte stores.
// The (B, D, L, N) state is never written to memory.
//
// Long sequences with few channels (batch-1) are split along L into chunks
// handled by different workgroups ("Mamba论文研读笔记" 3.2.3 B: the recurrence
// is associative, so chunk results can be combined):
//   pass 1 (summary): each chunk scans from a zero state and records its end
//            state and sum of delta;
//   pass 2 (carry):   per (b, d, n) the chunk transitions
//            h_end = exp(A sum_delta) h_start + h_local are chained in order;
//   pass 3 (full):    every chunk rescans from its true start state and
//            writes y.
#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

constexpr int kTile = 64;             // channels per workgroup, one per lane
constexpr int kWaves = 4;             // waves per workgroup
constexpr int kNSW = 16 / kWaves;     // states per wave
constexpr int kCT = 32;               // time steps staged per chunk
constexpr int kRow = kCT + 1;         // padded channel-major LDS row
constexpr int kThreads = 64 * kWaves;
static_assert(kTile * kCT / 8 == kThreads, "staging maps one 8-step piece per thread");
static_assert(16 * kCT / 2 == kThreads, "B/C staging maps two steps per thread");

// ------------------------------------------------------------------ loads / stores of 8 consecutive steps
template <bool kBF16, bool kVec>
__device__ __forceinline__ void load8(const void* base, int64_t off, int64_t t, int64_t t_end, bool ok,
                                      float out[8]) {
  if constexpr (kVec) {
    // off + t is a multiple of 8 and t_end - t is either <= 0 or >= 8.
    if (ok && t < t_end) {
      if constexpr (kBF16) {
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off + t);
        out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x); out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
        out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z); out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
      } else {
        const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off + t);
        const float4 a = q[0], b = q[1];
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool in = ok && (t + j < t_end);
      if constexpr (kBF16)
        out[j] = in ? bf16_to_f32(static_cast<const uint16_t*>(base)[off + t + j]) : 0.0f;
      else
        out[j] = in ? static_cast<const float*>(base)[off + t + j] : 0.0f;
    }
  }
}

template <bool kBF16, bool kVec>
__device__ __forceinline__ void store8(void* base, int64_t off, int64_t t, int64_t t_end, bool ok,
                                       const float v[8]) {
  if constexpr (kVec) {
    if (ok && t < t_end) {
      if constexpr (kBF16) {
        uint4 w;
        w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
        w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off + t) = w;
      } else {
        float4* q = reinterpret_cast<float4*>(static_cast<float*>(base) + off + t);
        q[0] = make_float4(v[0], v[1], v[2], v[3]);
        q[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (ok && (t + j < t_end)) {
        if constexpr (kBF16)
          static_cast<uint16_t*>(base)[off + t + j] = f32_to_bf16(v[j]);
        else
          static_cast<float*>(base)[off + t + j] = v[j];
      }
    }
  }
}

template <bool kBF16>
__device__ __forceinline__ float load1(const void* base, int64_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

// ------------------------------------------------------------------ the recurrence over one staged chunk
// dl_row / u_row: this lane's channel row in LDS; sB / sC: state-major B_t, C_t
// of the chunk; y_row: this wave's partial-readout row for the lane's channel.
// Steps past the end of the data were staged with delta = u = B = C = 0, which
// leaves h unchanged (Abar = 1, input term 0) and adds 0 to the readout.
template <int kMode, bool kSummary>
__device__ __forceinline__ void run_chunk(const float* __restrict__ dl_row, const float* __restrict__ u_row,
                                          const float* __restrict__ sB, const float* __restrict__ sC,
                                          float* __restrict__ y_row, float (&h)[kNSW],
                                          const float (&a2)[kNSW], const float (&ia)[kNSW], int n0) {
#pragma unroll 2
  for (int t = 0; t < kCT; t += 4) {
    float dl[4], uu[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) { dl[j] = dl_row[t + j]; uu[j] = u_row[t + j]; }
    float4 Bv[kNSW], Cv[kNSW];
#pragma unroll
    for (int i = 0; i < kNSW; ++i) {
      Bv[i] = *reinterpret_cast<const float4*>(sB + (n0 + i) * kCT + t);
      if constexpr (!kSummary) Cv[i] = *reinterpret_cast<const float4*>(sC + (n0 + i) * kCT + t);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = 0.0f;
      const float du = dl[j] * uu[j];
#pragma unroll
      for (int i = 0; i < kNSW; ++i) {
        const float bn = (j == 0) ? Bv[i].x : (j == 1) ? Bv[i].y : (j == 2) ? Bv[i].z : Bv[i].w;
        const float x = dl[j] * a2[i];          // delta * A in base-2 units
        const float e = hw_exp2(x);             // Abar
        float inp;
        if constexpr (kMode == kDeltaB) {
          inp = du * bn;                        // delta * B * u
        } else {
          // (Abar - 1) / A: exact product of the rounded Abar (fast), or from a
          // series where Abar - 1 would cancel (accurate).
          const float k = (kMode == kZohFast) ? __builtin_fmaf(e, ia[i], -ia[i])
                                              : expm1_from_exp2(x, e) * ia[i];
          inp = k * (bn * uu[j]);
        }
        h[i] = __builtin_fmaf(e, h[i], inp);
        if constexpr (!kSummary) {
          const float cn = (j == 0) ? Cv[i].x : (j == 1) ? Cv[i].y : (j == 2) ? Cv[i].z : Cv[i].w;
          acc = __builtin_fmaf(cn, h[i], acc);
        }
      }
      if constexpr (!kSummary) y_row[t + j] = acc;
    }
  }
}

template <bool kInBF16, bool kOutBF16, bool kVec, bool kSummary>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanParams p) {
  __shared__ float s_dl[kTile * kRow];
  __shared__ float s_u[kTile * kRow];
  __shared__ __attribute__((aligned(16))) float s_B[16 * kCT];
  __shared__ __attribute__((aligned(16))) float s_C[16 * kCT];
  __shared__ float s_y[kSummary ? 1 : kWaves * kTile * kRow];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int64_t D = p.D, N = p.N, L = p.L;
  const int64_t per_chunk = p.B * p.tiles_d;
  const int64_t wg = blockIdx.x;
  const int64_t chunk = wg / per_chunk;
  const int64_t rem = wg - chunk * per_chunk;
  const int64_t b = rem / p.tiles_d;
  const int64_t d0 = (rem - b * p.tiles_d) * kTile;
  const int64_t t_begin = chunk * p.chunk_len;
  const int64_t t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;

  // ---- recurrence role: lane = channel d, wave = states n0 .. n0+3
  const int64_t d = d0 + lane;
  const bool d_ok = d < D;
  const int n0 = wave * kNSW;
  float h[kNSW], a2[kNSW], ia[kNSW];
  bool small_a = false;
#pragma unroll
  for (int i = 0; i < kNSW; ++i) {
    const int n = n0 + i;
    const bool ok = d_ok && n < N;
    float a = ok ? p.A[d * N + n] : -1.0f;
    if (__builtin_fabsf(a) < kFastZohMinAbsA) small_a = true;
    // |A| below 2^-40 (including 0) is replaced by -2^-40 (sign kept): the
    // coefficient (e^{delta A} - 1)/A then equals delta to within delta*2^-41,
    // which the accurate loop resolves; 1/A stays finite.
    if (__builtin_fabsf(a) < 0x1p-40f) a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f;
    a2[i] = a * kLog2e;
    ia[i] = 1.0f / a;
    h[i] = 0.0f;
    if constexpr (!kSummary) {
      if (p.h_start != nullptr && chunk > 0 && ok) h[i] = p.h_start[((chunk * p.B + b) * D + d) * N + n];
    }
  }
  const int mode = p.delta_b ? kDeltaB : ((p.accurate || __any(small_a)) ? kZohAccurate : kZohFast);

  // ---- staging role: thread = (channel c, 8-step piece pc); B/C: (state sn, 2 steps)
  const int c = tid >> 2, pc = tid & 3;
  const int64_t dc = d0 + c;
  const bool c_ok = dc < D;
  const int64_t row_off = (b * D + (c_ok ? dc : 0)) * L;
  const float bias_c = (c_ok && p.bias) ? p.bias[dc] : 0.0f;
  const float dskip_c = (c_ok && p.Dskip) ? p.Dskip[dc] : 0.0f;
  const int sn = tid >> 4, stp = (tid & 15) * 2;
  const bool sn_ok = sn < N;
  const int64_t bc_off = (b * N + (sn_ok ? sn : 0)) * L;

  float ur[8], zr[8];
  float dsum = 0.0f;  // summary: sum of delta over this workgroup's steps (lane role)

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kCT) {
    // -------- stage the chunk
    {
      float dr[8];
      const int64_t tp = t0 + 8 * pc;
      load8<kInBF16, kVec>(p.delta, row_off, tp, t_end, c_ok, dr);
      load8<kInBF16, kVec>(p.u, row_off, tp, t_end, c_ok, ur);
      if constexpr (!kSummary) {
        if (p.z) load8<kInBF16, kVec>(p.z, row_off, tp, t_end, c_ok, zr);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool in = c_ok && (tp + j < t_end);
        s_dl[c * kRow + 8 * pc + j] = in ? softplus(dr[j] + bias_c) : 0.0f;
        s_u[c * kRow + 8 * pc + j] = ur[j];
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t tt = t0 + stp + e;
        const bool in = sn_ok && tt < t_end;
        s_B[sn * kCT + stp + e] = in ? load1<kInBF16>(p.Bt, bc_off + tt) : 0.0f;
        if constexpr (!kSummary) s_C[sn * kCT + stp + e] = in ? load1<kInBF16>(p.Ct, bc_off + tt) : 0.0f;
      }
    }
    __syncthreads();
    // -------- recurrence
    {
      const float* dl_row = s_dl + lane * kRow;
      const float* u_row = s_u + lane * kRow;
      float* y_row = s_y + (kSummary ? 0 : (wave * kTile + lane) * kRow);
      if (mode == kZohFast) run_chunk<kZohFast, kSummary>(dl_row, u_row, s_B, s_C, y_row, h, a2, ia, n0);
      else if (mode == kZohAccurate) run_chunk<kZohAccurate, kSummary>(dl_row, u_row, s_B, s_C, y_row, h, a2, ia, n0);
      else run_chunk<kDeltaB, kSummary>(dl_row, u_row, s_B, s_C, y_row, h, a2, ia, n0);
      if constexpr (kSummary) {
        float part = 0.0f;
#pragma unroll 8
        for (int t = 0; t < kCT; ++t) part += dl_row[t];
        dsum += part;
      }
    }
    __syncthreads();
    // -------- combine partial readouts, skip term and gate; store y
    if constexpr (!kSummary) {
      float out[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tl = 8 * pc + j;
        float v = s_y[(0 * kTile + c) * kRow + tl];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += s_y[(w * kTile + c) * kRow + tl];
        v = __builtin_fmaf(dskip_c, ur[j], v);
        if (p.z) v *= silu(zr[j]);
        out[j] = v;
      }
      store8<kOutBF16, kVec>(p.y, row_off, t0 + 8 * pc, t_end, c_ok, out);
    }
  }

  // ---- results of this workgroup's state
#pragma unroll
  for (int i = 0; i < kNSW; ++i) {
    const int n = n0 + i;
    if (!(d_ok && n < N)) continue;
    if constexpr (kSummary) {
      p.h_local[((chunk * p.B + b) * D + d) * N + n] = h[i];
    } else {
      if (p.final_state != nullptr && chunk == p.n_chunks - 1) p.final_state[(b * D + d) * N + n] = h[i];
    }
  }
  if constexpr (kSummary) {
    if (wave == 0 && d_ok) p.s_sum[(chunk * p.B + b) * D + d] = dsum;
  }
}

// Chains the chunk transitions h_end = exp(A * sum_delta) h_start + h_local
// for one (b, d, n) and records the true start state of every chunk.
__global__ __launch_bounds__(256) void carry_kernel(ScanParams p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = p.B * p.D * p.N;
  if (g >= total) return;
  const int64_t n = g % p.N;
  const int64_t bd = g / p.N;
  const int64_t d = bd % p.D;
  float a = p.A[d * p.N + n];
  if (__builtin_fabsf(a) < 0x1p-40f) a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f;
  const float a2 = a * kLog2e;
  const int64_t stride_bdn = p.B * p.D * p.N;
  const int64_t stride_bd = p.B * p.D;
  float hcur = 0.0f;
  for (int64_t k = 0; k + 1 < p.n_chunks; ++k) {
    const float decay = hw_exp2(p.s_sum[k * stride_bd + bd] * a2);
    hcur = __builtin_fmaf(decay, hcur, p.h_local[k * stride_bdn + g]);
    p.h_start[(k + 1) * stride_bdn + g] = hcur;
  }
}

template <bool kInBF16, bool kOutBF16, bool kSummary>
hipError_t launch_scan_t(const ScanParams& p, hipStream_t s) {
  // The summary pass is not needed for the last chunk.
  const int64_t grid = (kSummary ? p.n_chunks - 1 : p.n_chunks) * p.B * p.tiles_d;
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid), blk(kThreads);
  if (p.vec)
    hipLaunchKernelGGL((scan_kernel<kInBF16, kOutBF16, true, kSummary>), g, blk, 0, s, p);
  else
    hipLaunchKernelGGL((scan_kernel<kInBF16, kOutBF16, false, kSummary>), g, blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_full(const ScanParams& p, Dt in, Dt out, hipStream_t s) {
  if (in == Dt::BF16) {
    return out == Dt::BF16 ? launch_scan_t<true, true, false>(p, s) : launch_scan_t<true, false, false>(p, s);
  }
  return out == Dt::BF16 ? launch_scan_t<false, true, false>(p, s) : launch_scan_t<false, false, false>(p, s);
}

hipError_t launch_scan_summary(const ScanParams& p, Dt in, hipStream_t s) {
  return in == Dt::BF16 ? launch_scan_t<true, false, true>(p, s) : launch_scan_t<false, false, true>(p, s);
}

// Sets n 64-bit words to zero with ordinary stores: the hand-over flags of a
// scan recorded into a graph are cleared this way on every replay.
__global__ __launch_bounds__(256) void clear_u64_kernel(uint64_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_clear_u64(uint64_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_u64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_scan_carry(const ScanParams& p, hipStream_t s) {
  const int64_t total = p.B * p.D * p.N;
  const dim3 g((unsigned)((total + 255) / 256)), blk(256);
  hipLaunchKernelGGL(carry_kernel, g, blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace mamba

// conv1d.hip -- causal depthwise convolution along the sequence, then SiLU,
// for gfx950: the step that produces the scan input u ("Mamba 模型",
// flowchart nodes E and F: Uc_t = sum_i W_i U_(t-i), u_t = Uc_t sigmoid(Uc_t)),
// and its one-token decoding update ("Mamba 与状态空间模型" section 03: each
// channel keeps its most recent inputs between tokens).
//
// Both kernels stream: every input is read once and every output written once,
// with 4 fused multiply-adds and one SiLU per element, so HBM bandwidth bounds
// them.  Taps past K are treated as zero, so every K in 1..4 runs the same code.
#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

typedef float f4c __attribute__((ext_vector_type(4)));

template <bool kBF16>
__device__ __forceinline__ float ldx(const void* base, int64_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <bool kBF16>
__device__ __forceinline__ void stx(void* base, int64_t i, float v) {
  if constexpr (kBF16) static_cast<uint16_t*>(base)[i] = f32_to_bf16(v);
  else static_cast<float*>(base)[i] = v;
}

// Taps of channel d padded to 4 (zero past K) and its bias.
__device__ __forceinline__ void load_taps(const ConvParams& p, int64_t d, float (&w)[4], float& bias) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (i < p.K) ? p.w[d * p.K + i] : 0.0f;
  bias = p.bias ? p.bias[d] : 0.0f;
}

// Vector path: L % G == 0, x and y 16-byte aligned.  One thread computes G
// (16, or 8 when L % 16 != 0) consecutive outputs of one (b, d) row from G/8
// 16-byte loads; the 3 inputs before them come from one more 16-byte load of
// the preceding 8 (a cache hit: the neighbouring lane fetched them), or are
// zero at the start of the row.  y is written once and never re-read, so its
// stores carry non-temporal hints; x stays cacheable because the neighbouring
// lane reads each 16-byte block a second time (non-temporal x loads measured
// 1.15x the algorithmic bytes read).  16 outputs per thread with the hints
// measured 44.2 us per launch at B=4 D=5120 L=2048, 8 without them 47.0 us.
constexpr bool kConvNT = true;

template <bool kBF16, bool kNT>
__device__ __forceinline__ void load8s(const void* base, int64_t off, float (&v)[8]) {
  if constexpr (kBF16) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const u4v* p = reinterpret_cast<const u4v*>(static_cast<const uint16_t*>(base) + off);
    const u4v w = kNT ? __builtin_nontemporal_load(p) : *p;
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
    const f4c* p = reinterpret_cast<const f4c*>(static_cast<const float*>(base) + off);
    const f4c a = kNT ? __builtin_nontemporal_load(p) : p[0];
    const f4c b = kNT ? __builtin_nontemporal_load(p + 1) : p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool kBF16, bool kNT>
__device__ __forceinline__ void store8s(void* base, int64_t off, const float (&o)[8]) {
  if constexpr (kBF16) {
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    const u4v w = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                   pack_bf16x2(o[6], o[7])};
    u4v* p = reinterpret_cast<u4v*>(static_cast<uint16_t*>(base) + off);
    if constexpr (kNT) __builtin_nontemporal_store(w, p);
    else *p = w;
  } else {
    f4c* p = reinterpret_cast<f4c*>(static_cast<float*>(base) + off);
    const f4c a = {o[0], o[1], o[2], o[3]}, b = {o[4], o[5], o[6], o[7]};
    if constexpr (kNT) { __builtin_nontemporal_store(a, p); __builtin_nontemporal_store(b, p + 1); }
    else { p[0] = a; p[1] = b; }
  }
}

template <bool kInBF16, bool kOutBF16, int G>
__global__ __launch_bounds__(256) void conv1d_vec_kernel(ConvParams p) {
  constexpr int H = G / 8;
  const int64_t groups_per_row = p.L / G;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= p.rows * groups_per_row) return;
  const int64_t row = g / groups_per_row;
  const int64_t t0 = (g - row * groups_per_row) * G;
  const int64_t d = row % p.D;
  const int64_t base = row * p.L + t0;

  float in[8 + G];                 // in[8 + j] = x[t0 + j]; in[0..7] = the 8 before
#pragma unroll
  for (int h = 0; h < H; ++h) {
    float v[8];
    load8s<kInBF16, false>(p.x, base + 8 * h, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) in[8 + 8 * h + j] = v[j];
  }
  if (t0 > 0) {
    float v[8];
    load8s<kInBF16, false>(p.x, base - 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) in[j] = v[j];
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) in[j] = 0.0f;
  }
  float w[4], bias;
  load_taps(p, d, w, bias);

#pragma unroll
  for (int h = 0; h < H; ++h) {
    float out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float acc = bias;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(w[i], in[8 + 8 * h + j - i], acc);
      out[j] = silu(acc);
    }
    store8s<kOutBF16, kConvNT>(p.y, base + 8 * h, out);
  }
  if (p.final_state && t0 + G == p.L) {
    // the K most recent inputs, oldest first: x[L - K + k] = in[8 + G - K + k],
    // picked with selects so that the array stays in registers
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < p.K) {
        const int64_t idx = 8 + G - p.K + k;   // 4 + G .. 7 + G
        const float v = idx == 4 + G ? in[4 + G] : idx == 5 + G ? in[5 + G] : idx == 6 + G ? in[6 + G] : in[7 + G];
        p.final_state[row * p.K + k] = v;
      }
    }
  }
}

// General path: one thread per output element.
template <bool kInBF16, bool kOutBF16>
__global__ __launch_bounds__(256) void conv1d_elem_kernel(ConvParams p) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= p.rows * p.L) return;
  const int64_t row = e / p.L;
  const int64_t t = e - row * p.L;
  const int64_t d = row % p.D;
  float w[4], bias;
  load_taps(p, d, w, bias);
  float acc = bias;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float in = (i < p.K && t - i >= 0) ? ldx<kInBF16>(p.x, e - i) : 0.0f;
    acc = __builtin_fmaf(w[i], in, acc);
  }
  stx<kOutBF16>(p.y, e, silu(acc));
  if (p.final_state && t == p.L - 1) {
    for (int k = 0; k < p.K; ++k) {
      const int64_t s = p.L - p.K + k;
      p.final_state[row * p.K + k] = (s >= 0) ? ldx<kInBF16>(p.x, row * p.L + s) : 0.0f;
    }
  }
}

// One decoding step: state (rows, K) holds the K most recent inputs, oldest
// first; it becomes [state[1..K-1], x] and y = silu(sum_i w_i * input(t - i) + bias).
template <bool kInBF16, bool kOutBF16, int K, bool kVec>
__global__ __launch_bounds__(256) void conv1d_update_kernel(ConvParams p) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= p.rows) return;
  const int64_t d = r % p.D;
  float s[K];
  if constexpr (kVec) {           // K == 4, 16-byte aligned rows
    const f4c v = *reinterpret_cast<const f4c*>(p.state + r * 4);
    s[0] = v.x; s[1] = v.y; s[2] = v.z; s[3] = v.w;
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) s[k] = p.state[r * K + k];
  }
  // shifted state: n[k] = s[k+1] for k < K-1, n[K-1] = x
  float n[K];
#pragma unroll
  for (int k = 0; k + 1 < K; ++k) n[k] = s[k + 1];
  n[K - 1] = ldx<kInBF16>(p.x, r);
  float w[4], bias;
  load_taps(p, d, w, bias);
  float acc = bias;
#pragma unroll
  for (int i = 0; i < K; ++i) acc = __builtin_fmaf(w[i], n[K - 1 - i], acc);
  if constexpr (kVec) {
    *reinterpret_cast<f4c*>(p.state + r * 4) = f4c{n[0], n[1], n[2], n[3]};
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) p.state[r * K + k] = n[k];
  }
  stx<kOutBF16>(p.y, r, silu(acc));
}

template <bool kInBF16, bool kOutBF16>
hipError_t fwd_t(const ConvParams& p, bool vec, hipStream_t s) {
  if (vec && p.L % 16 == 0) {
    const int64_t threads = p.rows * (p.L / 16);
    hipLaunchKernelGGL((conv1d_vec_kernel<kInBF16, kOutBF16, 16>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, p);
  } else if (vec) {
    const int64_t threads = p.rows * (p.L / 8);
    hipLaunchKernelGGL((conv1d_vec_kernel<kInBF16, kOutBF16, 8>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, p);
  } else {
    const int64_t threads = p.rows * p.L;
    hipLaunchKernelGGL((conv1d_elem_kernel<kInBF16, kOutBF16>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                       0, s, p);
  }
  return hipGetLastError();
}

template <bool kInBF16, bool kOutBF16>
hipError_t upd_t(const ConvParams& p, hipStream_t s) {
  const dim3 g((unsigned)((p.rows + 255) / 256)), b(256);
  switch (p.K) {
    case 1: hipLaunchKernelGGL((conv1d_update_kernel<kInBF16, kOutBF16, 1, false>), g, b, 0, s, p); break;
    case 2: hipLaunchKernelGGL((conv1d_update_kernel<kInBF16, kOutBF16, 2, false>), g, b, 0, s, p); break;
    case 3: hipLaunchKernelGGL((conv1d_update_kernel<kInBF16, kOutBF16, 3, false>), g, b, 0, s, p); break;
    default:
      if ((reinterpret_cast<uintptr_t>(p.state) % 16) == 0)
        hipLaunchKernelGGL((conv1d_update_kernel<kInBF16, kOutBF16, 4, true>), g, b, 0, s, p);
      else
        hipLaunchKernelGGL((conv1d_update_kernel<kInBF16, kOutBF16, 4, false>), g, b, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_conv1d_fwd(const ConvParams& p, Dt in, Dt out, bool vec, hipStream_t s) {
  if (in == Dt::BF16) return out == Dt::BF16 ? fwd_t<true, true>(p, vec, s) : fwd_t<true, false>(p, vec, s);
  return out == Dt::BF16 ? fwd_t<false, true>(p, vec, s) : fwd_t<false, false>(p, vec, s);
}

hipError_t launch_conv1d_update(const ConvParams& p, Dt in, Dt out, hipStream_t s) {
  if (in == Dt::BF16) return out == Dt::BF16 ? upd_t<true, true>(p, s) : upd_t<true, false>(p, s);
  return out == Dt::BF16 ? upd_t<false, true>(p, s) : upd_t<false, false>(p, s);
}

}  // namespace mamba

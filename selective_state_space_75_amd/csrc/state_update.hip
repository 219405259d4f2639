// state_update.hip -- single-token selective state update for gfx950.
//
// One decoding step ("Mamba 模型", 为什么 Mamba 推理更省: the state is updated
// in place one token at a time; "Mamba 与状态空间模型" section 03: the state
// of a layer is channels x 16 numbers, independent of the sequence length):
//   delta = softplus(delta_raw + bias_d)
//   h_n  <- exp(delta A_dn) h_n + (exp(delta A_dn) - 1)/A_dn B_n u     (ZOH)
//   y     = (sum_n C_n h_n + D_d u) * silu(z)
//
// The step is a stream over the fp32 state (B, D, N): every state number is
// read once and written once, so the kernel is bound by HBM bandwidth and the
// arithmetic per element is free.  Mapping: four lanes per channel, each lane
// owning four consecutive states (one 16-byte load and store of state and of
// A); the quad reduces the readout with two lane exchanges, and its first lane
// applies the skip term and the gate and stores y.
#include <type_traits>

#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

template <bool kBF16>
__device__ __forceinline__ float ld(const void* base, int64_t i) {
  if constexpr (kBF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return static_cast<const float*>(base)[i];
}

template <bool kInBF16, bool kOutBF16, bool kVec>
__global__ __launch_bounds__(256) void state_update_kernel(UpdateParams p) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ch = g >> 2;                 // flattened (b, d)
  const int q = (int)(g & 3);                // quad lane: states 4q .. 4q+3
  const int64_t N = p.N, D = p.D;
  const bool ok = ch < p.B * D;
  const int64_t b = ok ? ch / D : 0;
  const int64_t d = ok ? ch - b * D : 0;

  float acc = 0.0f, uu = 0.0f;
  if (ok) {
    uu = ld<kInBF16>(p.u, ch);
    const float bias = p.bias ? p.bias[d] : 0.0f;
    const float delta = softplus(ld<kInBF16>(p.delta, ch) + bias);
    float hs[4], av[4];
    float* srow = p.state + ch * N;
    const float* arow = p.A + d * N;
    if constexpr (kVec) {
      const float4 s4 = *reinterpret_cast<const float4*>(srow + 4 * q);
      const float4 a4 = *reinterpret_cast<const float4*>(arow + 4 * q);
      hs[0] = s4.x; hs[1] = s4.y; hs[2] = s4.z; hs[3] = s4.w;
      av[0] = a4.x; av[1] = a4.y; av[2] = a4.z; av[3] = a4.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = 4 * q + i;
        hs[i] = n < N ? srow[n] : 0.0f;
        av[i] = n < N ? arow[n] : -1.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = 4 * q + i;
      if (!kVec && n >= N) continue;
      const float bn = ld<kInBF16>(p.Bt, b * N + n);
      const float cn = ld<kInBF16>(p.Ct, b * N + n);
      float a = av[i];
      if (__builtin_fabsf(a) < 0x1p-40f) a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f;
      const float x = delta * (a * kLog2e);
      const float e = hw_exp2(x);
      // Bandwidth-bound: always the cancellation-free (Abar - 1) / A.
      const float k = p.delta_b ? delta : expm1_from_exp2(x, e) / a;
      hs[i] = __builtin_fmaf(e, hs[i], k * (bn * uu));
      acc = __builtin_fmaf(cn, hs[i], acc);
    }
    if constexpr (kVec) {
      *reinterpret_cast<float4*>(srow + 4 * q) = make_float4(hs[0], hs[1], hs[2], hs[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = 4 * q + i;
        if (n < N) srow[n] = hs[i];
      }
    }
  }
  // Sum the four partial readouts of the quad (all lanes take part).
  acc += __shfl_xor(acc, 1, 4);
  acc += __shfl_xor(acc, 2, 4);
  if (ok && q == 0) {
    float v = acc + (p.Dskip ? p.Dskip[d] : 0.0f) * uu;
    if (p.z) v *= silu(ld<kInBF16>(p.z, ch));
    if constexpr (kOutBF16) static_cast<uint16_t*>(p.y)[ch] = f32_to_bf16(v);
    else static_cast<float*>(p.y)[ch] = v;
  }
}


// Streaming variant for N == 16 (the usual state size), used when B_t and C_t
// allow vector loads.  Each thread owns one quarter (4 states) of kStreamR
// channels spaced one workgroup-width apart; all of its loads (state, A, B_n,
// C_n, u, delta, bias) are issued before any arithmetic, B_n and C_n as one
// 8- or 16-byte load each.  The state is read and written with non-temporal
// hints: it is touched once per step, and keeping it out of the caches leaves
// them to A, B_t and C_t, which every batch row re-reads.  Measured on
// B=128 D=4096: one channel per thread (32768 waves) beats 2, 4 or 8 per thread;
// wave count matters more here than loads in flight per wave.
typedef float f4 __attribute__((ext_vector_type(4)));

template <int M> struct ModeTag { static constexpr int kValue = M; };
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamR = 1;
constexpr int kStreamBlock = 256;
constexpr uint32_t kStreamStride = kStreamBlock / 4;             // channels per pass of a workgroup
constexpr int kStreamChannels = kStreamStride * kStreamR;         // channels per workgroup

// Four consecutive B_n or C_n, kept in their storage type until used.
template <bool kBF16> struct Vec4In { using T = f4; };
template <> struct Vec4In<true> { using T = u16x4; };

template <bool kBF16>
__device__ __forceinline__ typename Vec4In<kBF16>::T ld4(const void* base, uint32_t i) {
  using T = typename Vec4In<kBF16>::T;
  using E = typename std::conditional<kBF16, uint16_t, float>::type;
  return *reinterpret_cast<const T*>(static_cast<const E*>(base) + i);
}

template <bool kBF16>
__device__ __forceinline__ float elem(const typename Vec4In<kBF16>::T& v, int i) {
  if constexpr (kBF16) return bf16_to_f32(v[i]);
  else return v[i];
}

template <bool kInBF16, bool kOutBF16>
__global__ __launch_bounds__(kStreamBlock) void state_update_stream_kernel(UpdateParams p) {
  const int q = threadIdx.x & 3;
  const uint32_t BD = (uint32_t)(p.B * p.D), D = (uint32_t)p.D;
  const uint32_t first = blockIdx.x * (uint32_t)kStreamChannels + (threadIdx.x >> 2);

  f4 h[kStreamR], a[kStreamR];
  typename Vec4In<kInBF16>::T bn[kStreamR], cn[kStreamR];
  float uu[kStreamR], dr[kStreamR], bias[kStreamR], zz[kStreamR], dsk[kStreamR];
  // Issue every load first.  Out-of-range channels read the last channel
  // (always valid) and store nothing.
#pragma unroll
  for (int r = 0; r < kStreamR; ++r) {
    const uint32_t ch0 = first + kStreamStride * r;
    const uint32_t ch = ch0 < BD ? ch0 : BD - 1;
    // b = ch / D: the fp64 estimate is q or q - 1 (ch < 2^31), one step fixes it
    uint32_t b = (uint32_t)((double)ch * p.inv_d);
    b += (ch - b * D >= D) ? 1u : 0u;
    const uint32_t d = ch - b * D;
    h[r] = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p.state + (size_t)ch * 16 + 4 * q));
    a[r] = *reinterpret_cast<const f4*>(p.A + (size_t)d * 16 + 4 * q);
    bn[r] = ld4<kInBF16>(p.Bt, b * 16 + 4 * q);
    cn[r] = ld4<kInBF16>(p.Ct, b * 16 + 4 * q);
    uu[r] = ld<kInBF16>(p.u, ch);
    dr[r] = ld<kInBF16>(p.delta, ch);
    bias[r] = p.bias ? p.bias[d] : 0.0f;
    // the gate's input and the skip weight with the others, so that no load is
    // left after the arithmetic
    zz[r] = p.z ? ld<kInBF16>(p.z, ch) : 0.0f;
    dsk[r] = p.Dskip ? p.Dskip[d] : 0.0f;
  }
  // The arithmetic is cheap next to the state traffic, so ZOH always takes
  // the cancellation-free (Abar - 1) / A (measured: no cost on B=128 D=4096).
  const int mode = p.delta_b ? kDeltaB : kZohAccurate;
  float acc[kStreamR];
  auto steps = [&](auto mc) {
    constexpr int M = decltype(mc)::kValue;
#pragma unroll
    for (int r = 0; r < kStreamR; ++r) {
      const float delta = softplus(dr[r] + bias[r]);
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // |A| < 2^-40 (including 0) is used as +-2^-40, where the coefficient
        // equals delta to within delta * 2^-41.
        float an = a[r][i];
        if (__builtin_fabsf(an) < 0x1p-40f) an = (an > 0.0f) ? 0x1p-40f : -0x1p-40f;
        const float x = delta * (an * kLog2e);
        const float e = hw_exp2(x);
        float k;
        if constexpr (M == kDeltaB) k = delta;
        else k = expm1_from_exp2(x, e) * hw_rcp(an);
        h[r][i] = __builtin_fmaf(e, h[r][i], k * (elem<kInBF16>(bn[r], i) * uu[r]));
        sum = __builtin_fmaf(elem<kInBF16>(cn[r], i), h[r][i], sum);
      }
      acc[r] = sum;
    }
  };
  if (mode == kDeltaB) steps(ModeTag<kDeltaB>{});
  else steps(ModeTag<kZohAccurate>{});

#pragma unroll
  for (int r = 0; r < kStreamR; ++r) {
    const uint32_t ch0 = first + kStreamStride * r;
    const uint32_t ch = ch0 < BD ? ch0 : BD - 1;
    float sum = acc[r];
    sum += __shfl_xor(sum, 1, 4);
    sum += __shfl_xor(sum, 2, 4);
    if (ch0 < BD) {
      __builtin_nontemporal_store(h[r], reinterpret_cast<f4*>(p.state + (size_t)ch * 16 + 4 * q));
      if (q == 0) {
        float v = sum + dsk[r] * uu[r];
        if (p.z) v *= silu(zz[r]);
        if constexpr (kOutBF16) static_cast<uint16_t*>(p.y)[ch] = f32_to_bf16(v);
        else static_cast<float*>(p.y)[ch] = v;
      }
    }
  }
}

template <bool kInBF16, bool kOutBF16>
hipError_t launch_t(const UpdateParams& p, hipStream_t s) {
  const size_t vec = kInBF16 ? 8 : 16;
  const bool stream = p.N == 16 && (reinterpret_cast<uintptr_t>(p.Bt) % vec) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.Ct) % vec) == 0 && p.B * p.D < (int64_t(1) << 31);
  if (stream) {
    const int64_t blocks = (p.B * p.D + kStreamChannels - 1) / kStreamChannels;
    hipLaunchKernelGGL((state_update_stream_kernel<kInBF16, kOutBF16>), dim3((unsigned)blocks),
                       dim3(kStreamBlock), 0, s, p);
    return hipGetLastError();
  }
  const int64_t threads = p.B * p.D * 4;
  const dim3 g((unsigned)((threads + 255) / 256)), blk(256);
  if (p.N == 16)
    hipLaunchKernelGGL((state_update_kernel<kInBF16, kOutBF16, true>), g, blk, 0, s, p);
  else
    hipLaunchKernelGGL((state_update_kernel<kInBF16, kOutBF16, false>), g, blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_state_update(const UpdateParams& p, Dt in, Dt out, hipStream_t s) {
  if (in == Dt::BF16) return out == Dt::BF16 ? launch_t<true, true>(p, s) : launch_t<true, false>(p, s);
  return out == Dt::BF16 ? launch_t<false, true>(p, s) : launch_t<false, false>(p, s);
}

}  // namespace mamba

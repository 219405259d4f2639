// scan_bwd.hip -- backward pass of the selective scan for gfx950.
//
// What it computes: the gradients of the forward pass ("Mamba 模型" flowchart
// nodes H to M; ZOH per "Mamba模型：高效序列建模的新突破" 3.1) with respect to
// u, delta_raw, z, B_t, C_t, A, D and the delta bias, for a given dy.  The
// states are recomputed on chip instead of being stored by the forward pass
// ("Mamba论文研读笔记" 3.2.3 C, recomputation; "Mamba 与状态空间模型" section 07).
//
// Per channel and state (lane layout of the forward kernel: one wave owns 16
// channels of one batch row, four lanes per channel, four states per lane).
// L is cut into segments (2.8B layer: 8 of 256 steps), each segment into
// 8-step chunks, and five launches run:
//   summary:  each segment's recurrence from a zero start; stores the state
//             and the running sum of delta at the start of every 32-step
//             block, and per segment the end state, the product of Abar and
//             the adjoint term it passes to the previous segment;
//   carry:    one thread per (batch row, channel, state) chains the segments:
//             the state entering each segment and the adjoint leaving it;
//   segment:  walks the segment's blocks from the last: rebuilds the
//             block's start state (stored state + decayed entering state),
//             runs the recurrence over its first three chunks for the chunk
//             starts, then per chunk from the last reruns its 8 steps keeping
//             h_t in registers and walks them in reverse with the state
//             adjoint g_t = dyc_t C_t + Abar_(t+1) g_(t+1):
//             dyc  = dy * silu(z)            dz = dy * yc * s (1 + z (1 - s))
//             dAbar = g h_(t-1)              dcoef = g B u
//             du   = dyc D + sum_n g coef B
//             ddelta = sum_n (dAbar a Abar + dcoef dcoef/ddelta)
//             dA  += dAbar delta Abar + dcoef delta^2 phi(delta a)   (ZOH)
//             ddelta_raw = ddelta * sigmoid(delta_raw + bias)
//             with phi(x) = (x e^x - e^x + 1) / x^2 (a series near 0);
//   two reductions: the per-tile dB_t / dC_t partials and the per-segment
//             dA, dD, bias-gradient partials, each in a fixed order.
// The ZOH coefficient follows the forward pass: (Abar - 1)/A from a
// cancellation-free series for fp32 inputs (or when asked), else as
// fma(Abar, 1/A, -1/A) from Abar itself.  With the latter, dA also takes the
// short route: Abar and coef depend on delta and A only through delta A (coef
// with one more factor delta), so A dA = sum_t (delta ddelta - dcoef coef)
// summed per state, which needs no phi.
// Each chunk's inputs are loaded with vector loads one chunk ahead and
// staged in LDS; the per-element terms (softplus, its derivative, the gate)
// are evaluated once there, not once per lane of a channel.
// dB_t and dC_t are shared by the D channels of a batch row: each step, the
// wave sums its 16 channels' contributions with cross-lane swaps (permlane32,
// permlane16, two DPP row rotations) into one value per state; the segment
// pass runs four such waves per workgroup (four adjacent tiles), which add
// their values in tile order after each block and store one partial; a
// second kernel adds the workgroups' partials in a fixed order, and the
// per-batch-row partials of dA, dD and the bias gradient likewise, so results
// are deterministic.
#include <type_traits>

#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

constexpr int kT = kBwdChunk;      // steps recomputed at a time
constexpr int kBlk = kBwdBlock;     // steps staged at a time (four chunks)

// Sum over the four lanes of a quad (DPP quad permutations).
__device__ __forceinline__ float quad_sum4(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

__device__ __forceinline__ float sigmoidf(float x) { return hw_rcp(1.0f + hw_exp2(-x * kLog2e)); }

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// x + y summed across the two wave halves: lanes 0-31 get the sum of x over
// lanes l and l + 32, lanes 32-63 the sum of y over lanes l - 32 and l.
__device__ __forceinline__ float swap32_sum(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned r0 = r[0], r1 = r[1];   // elements as scalars: bit-casting a subscript reads element 0
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}
// The same across the two rows of each 32-lane half: even rows get the sum of
// x over the row pair, odd rows the sum of y.
__device__ __forceinline__ float swap16_sum(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// Eight consecutive elements of one row as loaded from global memory (16
// bytes of bf16, 32 of fp32); they are widened only where they are consumed,
// so the loads stay in flight across the block being computed.
template <bool kBF16> struct Raw8;
template <> struct Raw8<true> {
  uint4 w;
  __device__ __forceinline__ float get(int j) const {
    const uint32_t x = j < 2 ? w.x : j < 4 ? w.y : j < 6 ? w.z : w.w;
    return (j & 1) ? bf16_hi(x) : bf16_lo(x);
  }
};
template <> struct Raw8<false> {
  float4 f0, f1;
  __device__ __forceinline__ float get(int j) const {
    const float4& f = j < 4 ? f0 : f1;
    const int k = j & 3;
    return k == 0 ? f.x : k == 1 ? f.y : k == 2 ? f.z : f.w;
  }
};

// Elements off .. off + 7 of `base`: vector loads when `vec` (the caller
// guarantees alignment and bounds), else element loads with zeros from index
// `valid` on (and everywhere when !ok).
template <bool kBF16>
__device__ __forceinline__ void ld_raw8(Raw8<kBF16>& r, const void* base, int64_t off, bool vec, bool ok, int valid) {
  if constexpr (kBF16) {
    const uint16_t* q = static_cast<const uint16_t*>(base) + off;
    if (vec) {
      r.w = ok ? *reinterpret_cast<const uint4*>(q) : make_uint4(0u, 0u, 0u, 0u);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (ok && j < valid) ? (uint32_t)q[j] : 0u;
      r.w = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
    }
  } else {
    const float* q = static_cast<const float*>(base) + off;
    if (vec) {
      r.f0 = ok ? *reinterpret_cast<const float4*>(q) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      r.f1 = ok ? *reinterpret_cast<const float4*>(q + 4) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    } else {
      float h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = (ok && j < valid) ? q[j] : 0.0f;
      r.f0 = make_float4(h[0], h[1], h[2], h[3]);
      r.f1 = make_float4(h[4], h[5], h[6], h[7]);
    }
  }
}

// Stores v[0..7] at off .. off + 7 (vector stores when `vec`, else the first `valid`).
template <bool kBF16>
__device__ __forceinline__ void st8(void* base, int64_t off, bool vec, int valid, const float (&v)[8]) {
  if constexpr (kBF16) {
    uint16_t* q = static_cast<uint16_t*>(base) + off;
    if (vec) {
      *reinterpret_cast<uint4*>(q) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < valid) q[j] = f32_to_bf16(v[j]);
    }
  } else {
    float* q = static_cast<float*>(base) + off;
    if (vec) {
      *reinterpret_cast<float4*>(q) = make_float4(v[0], v[1], v[2], v[3]);
      *reinterpret_cast<float4*>(q + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < valid) q[j] = v[j];
    }
  }
}

// Inputs of one block of kBlk steps for the wave's 16 channels, staged in
// LDS.  The reverse walk over a step overwrites that step's entries with its
// results, which are then stored for the whole block at once.
struct Stage {
  float4 V[kBlk][16];   // [step][channel] {u, delta, dyc, kz}; after the walk {du, ddelta/sigmoid', dz, -}
  float B[kBlk][16];    // [step][state] B_t; after the walk the tile's dB_t partial
  float C[kBlk][16];    // [step][state] C_t; after the walk the tile's dC_t partial
};

// One wave's task: 16 channels of one batch row over one segment of L.
// Lane roles: (c, g) = (lane / 4, lane % 4) is channel c, states 4 g .. 4 g + 3
// in the recurrence; and steps 8 g .. 8 g + 7 of a block when loading and
// storing the rows of channel c and of state c (B_t, C_t and their gradients).
// Each row of a block is thus read and written as 4 lanes x 8 contiguous
// elements, whole cache lines at a time.
template <bool kInBF16, bool kGradBF16>
struct Wave {
  const BwdParams& p;
  int lane, c, g;
  int64_t b, s, td, d, dd, row, brow, t_begin, t_end;
  bool c_ok, sn_ok, has_z, vecp, small_a;
  float bias, Dd;
  float a[4], a2[4], ia[4];

  struct Raw {
    Raw8<kInBF16> u, r, z, bt, ct;
    Raw8<kGradBF16> dy;
  };

  // lane of the wave; tile td (tiles past the last have no channel), segment
  // ss, batch row bb
  __device__ Wave(const BwdParams& pp, int lane_, int64_t td_, int64_t ss, int64_t bb) : p(pp) {
    lane = lane_;
    c = lane >> 2;
    g = lane & 3;
    td = td_;
    s = ss;
    b = bb;
    d = td * 16 + c;
    c_ok = d < p.D;
    dd = c_ok ? d : 0;          // channels past D read channel 0 and contribute nothing
    row = (b * p.D + dd) * p.L;
    sn_ok = c < p.N;            // state role: state c
    brow = (b * p.N + (sn_ok ? c : 0)) * p.L;
    t_begin = s * p.seg_len;
    t_end = t_begin + p.seg_len < p.L ? t_begin + p.seg_len : p.L;
    has_z = p.z != nullptr;
    vecp = p.vec != 0;
    bias = p.bias ? p.bias[dd] : 0.0f;
    Dd = p.Dskip ? p.Dskip[dd] : 0.0f;
    small_a = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = 4 * g + i;
      float an = n < p.N ? p.A[dd * p.N + n] : -1.0f;
      // |A| < 2^-40 (including 0) as +-2^-40: the coefficient is then delta to
      // within delta * 2^-41, and its derivative in A is delta^2 / 2
      if (__builtin_fabsf(an) < kFastZohMinAbsA) small_a = true;
      if (__builtin_fabsf(an) < 0x1p-40f) an = (an > 0.0f) ? 0x1p-40f : -0x1p-40f;
      a[i] = an;
      a2[i] = an * kLog2e;
      ia[i] = 1.0f / an;
    }
  }

  __device__ int64_t nblocks() const { return (t_end - t_begin + kBlk - 1) / kBlk; }
  // block-major: a wave's 16 channels of one block are 1 KB of contiguous states
  __device__ int64_t ckpt_index(int64_t t) const { return (b * p.nck + t / kBlk) * p.D + d; }

  // global loads of the block at t0 (z / dy / C_t only when `adjoint`)
  __device__ void fetch(int64_t t0, Raw& x, bool adjoint) const {
    const bool vec = vecp && t0 + kBlk <= t_end;
    const int vc = (int)(t_end - t0 - 8 * g);
    ld_raw8<kInBF16>(x.u, p.u, row + t0 + 8 * g, vec, true, vc);
    ld_raw8<kInBF16>(x.r, p.delta, row + t0 + 8 * g, vec, true, vc);
    ld_raw8<kInBF16>(x.bt, p.Bt, brow + t0 + 8 * g, vec, sn_ok, vc);
    if (adjoint) {
      ld_raw8<kInBF16>(x.ct, p.Ct, brow + t0 + 8 * g, vec, sn_ok, vc);
      ld_raw8<kInBF16>(x.z, has_z ? p.z : p.u, row + t0 + 8 * g, vec, true, vc);
      ld_raw8<kGradBF16>(x.dy, p.dy, row + t0 + 8 * g, vec, true, vc);
    }
  }

  // per element, once: delta, the gated output gradient dyc = dy silu(z),
  // the factor kz of dz = kz yc (kz = dy s (1 + z (1 - s)), s = sigmoid(z)),
  // and (for the write-out) the softplus derivative sigmoid(delta_raw + bias)
  __device__ void stage(const Raw& x, Stage& st, bool adjoint, float (&sg)[8], float& accD) const {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float xr = x.r.get(j) + bias;
      const float uu = x.u.get(j);
      float dyc = 0.0f, kz = 0.0f;
      if (adjoint) {
        const float dy = x.dy.get(j);
        dyc = dy;
        if (has_z) {
          const float zv = x.z.get(j);
          const float sz = sigmoidf(zv);
          dyc = dy * (zv * sz);
          kz = dy * sz * __builtin_fmaf(zv, 1.0f - sz, 1.0f);
        }
        if (!c_ok) { dyc = 0.0f; kz = 0.0f; }
        sg[j] = sigmoidf(xr);
        accD = __builtin_fmaf(dyc, uu, accD);
        st.C[8 * g + j][c] = x.ct.get(j);
      }
      st.V[8 * g + j][c] = make_float4(uu, softplus(xr), dyc, kz);
      st.B[8 * g + j][c] = x.bt.get(j);
    }
  }
};

// Segment pass 1: per segment, the recurrence from a zero start.  Stores
// the state and the running sum of delta at every block start,
// and per segment the end state h, the product P of Abar over the segment,
// and H = sum_t (prod_(r <= t) Abar_r) dyc_t C_t, which carry the state into
// the next segment and the adjoint into the previous one.
template <bool kInBF16, bool kGradBF16, int M>
__device__ __forceinline__ void summary_body(const BwdParams& p, const Wave<kInBF16, kGradBF16>& w, Stage& st) {
  using W = Wave<kInBF16, kGradBF16>;
  float h[4] = {0.0f, 0.0f, 0.0f, 0.0f}, R[4] = {1.0f, 1.0f, 1.0f, 1.0f}, H[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float cum = 0.0f, sg[8], accD = 0.0f;
  const int64_t nb = w.nblocks();
  typename W::Raw x;
  w.fetch(w.t_begin, x, true);
  w.stage(x, st, true, sg, accD);
  __syncthreads();
  for (int64_t ib = 0; ib < nb; ++ib) {
    const int64_t t0 = w.t_begin + ib * kBlk;
    const bool more = ib + 1 < nb;
    if (more) w.fetch(t0 + kBlk, x, true);
    // the block's start state: 64 contiguous bytes per channel
    if (w.c_ok) {
      *reinterpret_cast<float4*>(p.ckpt_h + w.ckpt_index(t0) * 16 + 4 * w.g) = make_float4(h[0], h[1], h[2], h[3]);
      if (w.g == 0) p.ckpt_cd[w.ckpt_index(t0)] = cum;
    }
    // whole blocks take a copy of the steps with every count known at compile time
    auto steps = [&](auto whole) {
      constexpr bool kWhole = decltype(whole)::value;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t tk = t0 + k * kT;
        if (kWhole || tk < w.t_end) {
          const int len = kWhole ? kT : ((w.t_end - tk) < kT ? (int)(w.t_end - tk) : kT);
#pragma unroll
          for (int tl = 0; tl < kT; ++tl) {
            if (tl < len) {
              const int ts = k * kT + tl;
              const float4 v = st.V[ts][w.c];
              const float4 Bq = *reinterpret_cast<const float4*>(&st.B[ts][4 * w.g]);
              const float4 Cq = *reinterpret_cast<const float4*>(&st.C[ts][4 * w.g]);
              const float bv[4] = {Bq.x, Bq.y, Bq.z, Bq.w}, cv[4] = {Cq.x, Cq.y, Cq.z, Cq.w};
              cum += v.y;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float xx = v.y * w.a2[i];
                const float e = hw_exp2(xx);
                const float coef = M == kDeltaB ? v.y
                                   : M == kZohFast ? __builtin_fmaf(e, w.ia[i], -w.ia[i])
                                                   : expm1_from_exp2(xx, e) * w.ia[i];
                h[i] = __builtin_fmaf(e, h[i], coef * (bv[i] * v.x));
                R[i] *= e;
                H[i] = __builtin_fmaf(R[i], v.z * cv[i], H[i]);
              }
            }
          }
        }
      }
    };
    if (t0 + kBlk <= w.t_end) steps(std::true_type{});
    else steps(std::false_type{});
    if (more) {
      __syncthreads();
      w.stage(x, st, true, sg, accD);
      __syncthreads();
    }
  }
  if (w.c_ok) {
    const int64_t o = ((w.b * p.S + w.s) * p.D + w.d) * 16 + 4 * w.g;
    *reinterpret_cast<float4*>(p.seg_h + o) = make_float4(h[0], h[1], h[2], h[3]);
    *reinterpret_cast<float4*>(p.seg_P + o) = make_float4(R[0], R[1], R[2], R[3]);
    *reinterpret_cast<float4*>(p.seg_H + o) = make_float4(H[0], H[1], H[2], H[3]);
  }
}

// M = kZohFast falls back to the cancellation-free quotient for a wave with
// an |A| below kFastZohMinAbsA, as the forward pass does.
template <bool kInBF16, bool kGradBF16, int M>
__global__ __launch_bounds__(64) void bwd_summary_kernel(BwdParams p) {
  __shared__ Stage st;
  const int64_t task = blockIdx.x, rest = task / p.tiles_d;
  const Wave<kInBF16, kGradBF16> w(p, (int)threadIdx.x, task % p.tiles_d, rest % p.S, rest / p.S);
  if (M == kZohFast && __any(w.small_a)) summary_body<kInBF16, kGradBF16, kZohAccurate>(p, w, st);
  else summary_body<kInBF16, kGradBF16, M>(p, w, st);
}

// Segment carries, one thread per (batch row, channel, state): the state
// entering segment s, h_in(s + 1) = P(s) h_in(s) + h(s), and the adjoint term
// entering from segment s + 1, g_in(s - 1) = H(s) + P(s) g_in(s).
__global__ __launch_bounds__(256) void bwd_carry_kernel(BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.B * p.D * 16) return;
  const int64_t b = i / (p.D * 16), dn = i - b * p.D * 16;
  float h = 0.0f;
  for (int64_t s = 0; s < p.S; ++s) {
    const int64_t o = (b * p.S + s) * p.D * 16 + dn;
    p.h_in[o] = h;
    h = __builtin_fmaf(p.seg_P[o], h, p.seg_h[o]);
  }
  float gc = 0.0f;
  for (int64_t s = p.S - 1; s >= 0; --s) {
    const int64_t o = (b * p.S + s) * p.D * 16 + dn;
    p.g_in[o] = gc;
    gc = __builtin_fmaf(p.seg_P[o], gc, p.seg_H[o]);
  }
}

// Segment pass 2: blocks of the segment from the last, and the chunks of a
// block from the last: rebuild the block's start state from the stored one
// and the segment's entering state, run the recurrence forward for the
// starts of its chunks, then per chunk rerun its steps keeping h_t and
// (Abar_t - 1) in registers and walk them in reverse with the adjoint.
template <bool kInBF16, bool kGradBF16, int M>
__device__ __forceinline__ void segment_body(const BwdParams& p, const Wave<kInBF16, kGradBF16>& w,
                                             Stage (&sts)[kBwdGroup], int wv, int64_t tg) {
  using W = Wave<kInBF16, kGradBF16>;
  Stage& st = sts[wv];
  const int lane = w.lane, c = w.c, g = w.g;
  const bool red_c = lane >= 32;
  const bool bit3 = (lane >> 3) & 1, bit2 = (lane >> 2) & 1;
  // lane's slot for the reduced dB/dC value of a step: type (lane bit 5),
  // state 4 g + 2 (lane bit 4) + (lane bit 3)
  const int red_state = 4 * g + 2 * ((lane >> 4) & 1) + ((lane >> 3) & 1);
  float ia2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ia2[i] = w.ia[i] * w.ia[i];

  float hin[4] = {0.0f, 0.0f, 0.0f, 0.0f}, gs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (w.c_ok) {
    const int64_t o = ((w.b * p.S + w.s) * p.D + w.d) * 16 + 4 * g;
    const float4 hv = *reinterpret_cast<const float4*>(p.h_in + o);
    const float4 gv = *reinterpret_cast<const float4*>(p.g_in + o);
    hin[0] = hv.x; hin[1] = hv.y; hin[2] = hv.z; hin[3] = hv.w;
    gs[0] = gv.x; gs[1] = gv.y; gs[2] = gv.z; gs[3] = gv.w;
  }
  float anext[4] = {1.0f, 1.0f, 1.0f, 1.0f};
  float dAacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float accD = 0.0f, accBias = 0.0f;
  float sg_cur[8], sg_next[8];
  float4 ckh_cur, ckh_next;
  float ckc_cur, ckc_next;
  const int64_t nb = w.nblocks();
  // the start state of the block at t0 (64 contiguous bytes per channel)
  auto fetch_ckpt = [&](int64_t t0, float4& ckh, float& ckc) {
    ckh = w.c_ok ? *reinterpret_cast<const float4*>(p.ckpt_h + w.ckpt_index(t0) * 16 + 4 * g)
                 : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    ckc = w.c_ok ? p.ckpt_cd[w.ckpt_index(t0)] : 0.0f;
  };
  typename W::Raw x;
  {
    const int64_t tl0 = w.t_begin + (nb - 1) * kBlk;
    w.fetch(tl0, x, true);
    fetch_ckpt(tl0, ckh_next, ckc_next);
    w.stage(x, st, true, sg_next, accD);
  }
  __syncthreads();

  for (int64_t ib = nb - 1; ib >= 0; --ib) {
    const int64_t t0 = w.t_begin + ib * kBlk;
    const bool more = ib > 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) sg_cur[j] = sg_next[j];
    ckh_cur = ckh_next;
    ckc_cur = ckc_next;
    if (more) {
      w.fetch(t0 - kBlk, x, true);
      fetch_ckpt(t0 - kBlk, ckh_next, ckc_next);
    }
    const int blen = (w.t_end - t0) < kBlk ? (int)(w.t_end - t0) : kBlk;
    // chunk-start states: the block's start is the stored state (from a zero
    // segment start) + P(segment start .. block) h_in; every chunk but the
    // last is then run forward for the next chunk's start (a chunk that is
    // followed by another is whole)
    float hs[4][4];
    {
      const float hl[4] = {ckh_cur.x, ckh_cur.y, ckh_cur.z, ckh_cur.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[0][i] = __builtin_fmaf(hw_exp2(w.a2[i] * ckc_cur), hin[i], hl[i]);
    }
#pragma unroll
    for (int k = 1; k < 4; ++k) {
#pragma unroll
      for (int i = 0; i < 4; ++i) hs[k][i] = hs[k - 1][i];
      if (k * kT < blen) {
#pragma unroll
        for (int tl = 0; tl < kT; ++tl) {
          const int ts = (k - 1) * kT + tl;
          const float2 v = *reinterpret_cast<const float2*>(&st.V[ts][c]);
          const float4 Bq = *reinterpret_cast<const float4*>(&st.B[ts][4 * g]);
          const float bv[4] = {Bq.x, Bq.y, Bq.z, Bq.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float xx = v.y * w.a2[i];
            const float e = hw_exp2(xx);
            const float coef = M == kDeltaB ? v.y
                               : M == kZohFast ? __builtin_fmaf(e, w.ia[i], -w.ia[i])
                                               : expm1_from_exp2(xx, e) * w.ia[i];
            hs[k][i] = __builtin_fmaf(e, hs[k][i], coef * (bv[i] * v.x));
          }
        }
      }
    }
#pragma unroll
    for (int k = 3; k >= 0; --k) {
      if (k * kT < blen) {
        const int len = (blen - k * kT) < kT ? blen - k * kT : kT;
        // er: Abar - 1 (cancellation-free quotient) or Abar (the other rules)
        float hist[kT + 1][4], er[kT][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[0][i] = hs[k][i];
#pragma unroll
        for (int tl = 0; tl < kT; ++tl) {
          if (tl < len) {
            const int ts = k * kT + tl;
            const float2 v = *reinterpret_cast<const float2*>(&st.V[ts][c]);
            const float4 Bq = *reinterpret_cast<const float4*>(&st.B[ts][4 * g]);
            const float bv[4] = {Bq.x, Bq.y, Bq.z, Bq.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float xx = v.y * w.a2[i];
              const float e = hw_exp2(xx);
              float coef;
              if constexpr (M == kDeltaB) {
                er[tl][i] = e;
                coef = v.y;
              } else if constexpr (M == kZohFast) {
                er[tl][i] = e;
                coef = __builtin_fmaf(e, w.ia[i], -w.ia[i]);
              } else {
                const float E = expm1_from_exp2(xx, e);
                er[tl][i] = E;
                coef = E * w.ia[i];
              }
              hist[tl + 1][i] = __builtin_fmaf(e, hist[tl][i], coef * (bv[i] * v.x));
            }
          }
        }
#pragma unroll
        for (int tl = kT - 1; tl >= 0; --tl) {
          if (tl < len) {
            const int ts = k * kT + tl;
            const float4 v = st.V[ts][c];
            const float4 Bq = *reinterpret_cast<const float4*>(&st.B[ts][4 * g]);
            const float4 Cq = *reinterpret_cast<const float4*>(&st.C[ts][4 * g]);
            const float u = v.x, delta = v.y, dyc = v.z, kz = v.w;
            const float Bv[4] = {Bq.x, Bq.y, Bq.z, Bq.w}, Cv[4] = {Cq.x, Cq.y, Cq.z, Cq.w};
            float sy = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) sy = __builtin_fmaf(Cv[i], hist[tl + 1][i], sy);
            const float dz = kz * __builtin_fmaf(w.Dd, u, quad_sum4(sy));
            const float d2 = delta * delta;
            float sdu = 0.0f, sdd = 0.0f, dBv[4], dCv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e = M == kZohAccurate ? er[tl][i] + 1.0f : er[tl][i];
              const float coef = M == kDeltaB ? delta
                                 : M == kZohFast ? __builtin_fmaf(e, w.ia[i], -w.ia[i]) : er[tl][i] * w.ia[i];
              const float gn = __builtin_fmaf(dyc, Cv[i], anext[i] * gs[i]);
              const float dabar = gn * hist[tl][i];
              const float gc = gn * coef;
              dBv[i] = gc * u;
              dCv[i] = dyc * hist[tl + 1][i];
              sdu = __builtin_fmaf(gc, Bv[i], sdu);
              const float dcoef = gn * (Bv[i] * u);
              const float de = dabar * e;
              if constexpr (M == kDeltaB) {
                sdd = __builtin_fmaf(de, w.a[i], sdd + dcoef);
                dAacc[i] = __builtin_fmaf(de, delta, dAacc[i]);
              } else if constexpr (M == kZohFast) {
                // Abar and coef depend on delta and A only through delta A,
                // coef with one more factor delta, so the step's A-gradient is
                // (delta ddelta - dcoef coef) / A: accumulated here, divided by A
                // at the end.  It cancels like the fast quotient does (relative
                // error about 2.4e-7 / (delta |A|)).
                const float sc = __builtin_fmaf(dabar, w.a[i], dcoef) * e;
                sdd += sc;
                dAacc[i] = __builtin_fmaf(delta, sc, __builtin_fmaf(-dcoef, coef, dAacc[i]));
              } else {
                sdd = __builtin_fmaf(__builtin_fmaf(dabar, w.a[i], dcoef), e, sdd);
                // d coef / dA = delta^2 phi(delta A), phi(y) = (y e^y - e^y + 1) / y^2:
                // its series to y^5 for |y| < 1/4 (next term y^6 / 5760, below 2^-24
                // of phi there), else (y e^y - e^y + 1) / A^2
                const float y = delta * w.a[i];
                float ps = __builtin_fmaf(y, 1.0f / 840.0f, 1.0f / 144.0f);
                ps = __builtin_fmaf(y, ps, 1.0f / 30.0f);
                ps = __builtin_fmaf(y, ps, 1.0f / 8.0f);
                ps = __builtin_fmaf(y, ps, 1.0f / 3.0f);
                ps = __builtin_fmaf(y, ps, 0.5f);
                const float em1 = M == kZohFast ? 1.0f - e : -er[tl][i];   // -(Abar - 1)
                const float closed = __builtin_fmaf(y, e, em1) * ia2[i];
                const float q = (__builtin_fabsf(y) < 0.25f) ? d2 * ps : closed;
                dAacc[i] = __builtin_fmaf(dcoef, q, __builtin_fmaf(de, delta, dAacc[i]));
              }
              gs[i] = gn;
              anext[i] = e;
            }
            const float du = __builtin_fmaf(dyc, w.Dd, quad_sum4(sdu));
            const float dpre = quad_sum4(sdd);
            // results of this step over its inputs: lane g writes component g
            reinterpret_cast<float*>(&st.V[ts][c])[g] = g == 0 ? du : (g == 1 ? dpre : dz);
            // dB_t, dC_t over the wave's 16 channels (lane bits 2..5)
            const float w0 = swap32_sum(dBv[0], dCv[0]);
            const float w1 = swap32_sum(dBv[1], dCv[1]);
            const float w2 = swap32_sum(dBv[2], dCv[2]);
            const float w3 = swap32_sum(dBv[3], dCv[3]);
            const float q0 = swap16_sum(w0, w2);
            const float q1 = swap16_sum(w1, w3);
            const float keep = bit3 ? q1 : q0, send = bit3 ? q0 : q1;
            const float rr = keep + dpp_mov<0x128>(send);           // row_ror:8 pairs lane bit 3
            // partner lane ^ 4: row_ror:4 reads lane i - 4, row_ror:12 lane i + 4
            // (both evaluated with the whole wave active, then selected)
            const float from_m4 = dpp_mov<0x124>(rr), from_p4 = dpp_mov<0x12C>(rr);
            const float fin = rr + (bit2 ? from_m4 : from_p4);
            (red_c ? st.C[ts] : st.B[ts])[red_state] = fin;
          }
        }
      }
    }
    __syncthreads();
    // write out the block: lane (c, g) owns steps 8 g .. 8 g + 7 of channel c
    // and of state c
    {
      const bool vec = w.vecp && blen == kBlk;
      const int valid = blen - 8 * g;
      float du[8], dr[8], dz[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 o = st.V[8 * g + j][c];
        du[j] = o.x;
        dr[j] = o.y * sg_cur[j];
        dz[j] = o.z;
        if (j < valid) accBias += dr[j];
      }
      if (w.c_ok) {
        st8<kGradBF16>(p.du, w.row + t0 + 8 * g, vec, valid, du);
        st8<kGradBF16>(p.ddelta, w.row + t0 + 8 * g, vec, valid, dr);
        if (w.has_z) st8<kGradBF16>(p.dz, w.row + t0 + 8 * g, vec, valid, dz);
      }
      // the workgroup's dB_t (wave 0) and dC_t (wave 1) for state c: the
      // tiles' partials summed in tile order
      if (wv < 2 && w.sn_ok) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float acc = wv == 0 ? sts[0].B[8 * g + j][c] : sts[0].C[8 * g + j][c];
#pragma unroll
          for (int q = 1; q < kBwdGroup; ++q) acc += wv == 0 ? sts[q].B[8 * g + j][c] : sts[q].C[8 * g + j][c];
          v[j] = acc;
        }
        const int64_t o = ((w.b * p.groups + tg) * 16 + c) * p.L + t0 + 8 * g;
        st8<false>(wv == 0 ? p.part_dB : p.part_dC, o, vec, valid, v);
      }
    }
    if (more) {
      __syncthreads();
      w.stage(x, st, true, sg_next, accD);
      __syncthreads();
    }
  }
  accD = quad_sum4(accD);
  accBias = quad_sum4(accBias);
  if (w.c_ok) {
    const int64_t o = (w.b * p.S + w.s) * p.D + w.d;
    if constexpr (M == kZohFast) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dAacc[i] *= w.ia[i];
    }
    *reinterpret_cast<float4*>(p.part_dA + o * 16 + 4 * g) = make_float4(dAacc[0], dAacc[1], dAacc[2], dAacc[3]);
    if (g == 0) {
      p.part_dD[o] = accD;
      p.part_dbias[o] = accBias;
    }
  }
}

// A workgroup is kBwdGroup waves, one per 16-channel tile of a group of
// adjacent tiles, all on the same segment and batch row (so they pass the
// same barriers).  The cancellation-free quotient is chosen per wave.
template <bool kInBF16, bool kGradBF16, int M>
__global__ __launch_bounds__(64 * kBwdGroup) void bwd_segment_kernel(BwdParams p) {
  __shared__ Stage st[kBwdGroup];
  const int wv = (int)(threadIdx.x >> 6);
  const int64_t task = blockIdx.x, rest = task / p.groups;
  const int64_t tg = task % p.groups;
  const Wave<kInBF16, kGradBF16> w(p, (int)(threadIdx.x & 63), tg * kBwdGroup + wv, rest % p.S, rest / p.S);
  if (M == kZohFast && __any(w.small_a)) segment_body<kInBF16, kGradBF16, kZohAccurate>(p, w, st, wv, tg);
  else segment_body<kInBF16, kGradBF16, M>(p, w, st, wv, tg);
}

// dB_t, dC_t: sum of the per-workgroup partials, in tile order.
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = p.B * p.N * p.L;
  if (i >= total) return;
  const int64_t b = i / (p.N * p.L);
  const int64_t rem = i - b * p.N * p.L;
  const int64_t n = rem / p.L, t = rem - n * p.L;
  const float* pb = p.part_dB + (b * p.groups * 16 + n) * p.L + t;
  const float* pc = p.part_dC + (b * p.groups * 16 + n) * p.L + t;
  const int64_t stride = 16 * p.L;
  float sb = 0.0f, sc = 0.0f;
#pragma unroll 8
  for (int64_t q = 0; q < p.groups; ++q) {
    sb += pb[q * stride];
    sc += pc[q * stride];
  }
  p.dBt[i] = sb;
  p.dCt[i] = sc;
}

// dA, dD, bias gradient: sum of the per-segment partials, batch rows outer,
// segments inner.
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(BwdParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.D * 16) return;
  const int64_t d = i >> 4, n = i & 15;
  const int64_t rows = p.B * p.S;
  if (n < p.N) {
    float s = 0.0f;
#pragma unroll 8
    for (int64_t r = 0; r < rows; ++r) s += p.part_dA[(r * p.D + d) * 16 + n];
    p.dA[d * p.N + n] = s;
  }
  if (n == 0) {
    float sd = 0.0f, sb = 0.0f;
#pragma unroll 8
    for (int64_t r = 0; r < rows; ++r) {
      sd += p.part_dD[r * p.D + d];
      sb += p.part_dbias[r * p.D + d];
    }
    p.dDskip[d] = sd;
    p.dbias[d] = sb;
  }
}

template <bool kInBF16, bool kGradBF16, int M>
hipError_t bwd_t(const BwdParams& p, hipStream_t s) {
  const dim3 tasks((unsigned)(p.B * p.tiles_d * p.S));
  hipLaunchKernelGGL((bwd_summary_kernel<kInBF16, kGradBF16, M>), tasks, dim3(64), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_carry_kernel, dim3((unsigned)((p.B * p.D * 16 + 255) / 256)), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_segment_kernel<kInBF16, kGradBF16, M>), dim3((unsigned)(p.B * p.groups * p.S)),
                     dim3(64 * kBwdGroup), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nbc = p.B * p.N * p.L;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3((unsigned)((nbc + 255) / 256)), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_params_kernel, dim3((unsigned)((p.D * 16 + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

// The forward's rules: bf16 inputs take (Abar - 1)/A from Abar unless the
// accurate quotient is asked for; fp32 inputs always take it.
template <bool kInBF16, bool kGradBF16>
hipError_t bwd_d(const BwdParams& p, hipStream_t s) {
  if (p.delta_b) return bwd_t<kInBF16, kGradBF16, kDeltaB>(p, s);
  if constexpr (kInBF16) {
    if (!p.accurate) return bwd_t<kInBF16, kGradBF16, kZohFast>(p, s);
  }
  return bwd_t<kInBF16, kGradBF16, kZohAccurate>(p, s);
}

}  // namespace

hipError_t launch_scan_bwd(const BwdParams& p, Dt in, Dt grad, hipStream_t s) {
  if (in == Dt::BF16) return grad == Dt::BF16 ? bwd_d<true, true>(p, s) : bwd_d<true, false>(p, s);
  return grad == Dt::BF16 ? bwd_d<false, true>(p, s) : bwd_d<false, false>(p, s);
}

}  // namespace mamba

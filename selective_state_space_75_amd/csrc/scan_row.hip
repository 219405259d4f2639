// scan_row.hip -- selective-scan kernels with one state per lane (gfx950).
// Same computation as scan_v4.hpp ("Mamba 模型", full-step flowchart nodes H
// to M; ZOH per "Mamba模型：高效序列建模的新突破" 3.1): softplus step, ZOH
// discretisation, recurrence, readout, skip, gate.  Two variants:
// scan_row_kernel for shapes whose 16-channel tiles do not fill the chip (the
// batch-1 long sequence, the 130M layer), and scan_row_lean_kernel, which
// trades in-wave lookahead for five workgroups per CU, for shapes with many
// tiles per CU.
//
// Layout -- a workgroup of 4 waves owns 16 channels of one batch row:
//  * wave w holds channels 4w .. 4w+3, one per 16-lane DPP row; lane n of a
//    row holds state n in a VGPR (N <= 16; lanes past N hold a zero state).
//    A tile therefore occupies 4 SIMDs instead of one, so a sequence that
//    would need chunking along L with 16 states per lane (summary pass, carry
//    and a rescan) is scanned in a single pass;
//  * the sequence is walked in 32-step chunks.  Lane j of a row loads
//    elements 2j, 2j+1 of its channel's u, delta_raw and z (one 4-byte load
//    each for bf16), evaluates softplus and the gate for them once, and later
//    owns their two outputs.  Step t reads delta and u from lane t/2 of the
//    row through a DPP row broadcast (row_newbcast) folded into the consuming
//    multiply;
//  * B_t and C_t of a chunk are staged once per workgroup in LDS as fp32,
//    state-major with padded rows, double-buffered; a lane reads 4 steps of
//    its state with one 16-byte read (the 4 rows of a wave read the same
//    addresses).  One workgroup barrier per chunk guards the buffers;
//  * the readout's per-state products C_t,n h_t,n go through LDS once per
//    chunk: each lane writes its 32 products, then reads the 16 products of
//    each of its 2 output steps and sums them (15 adds per output);
//  * outputs leave in whole 128-byte lines, gathered across the lanes of a
//    row with ds_bpermute.
// Per state update: 6 fp32 VALU + 1 v_exp_f32, as in the 4-states-per-lane
// kernel, plus a quarter of a 16-byte LDS read each for B_t and C_t.
#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

constexpr int kRCT = 32;          // steps per chunk
constexpr int kBCRow = 36;        // floats per staged B/C row (32 + padding)
constexpr int kPRowR = 36;        // floats per partial-readout row (32 + padding)
constexpr int kPWave = 4 * 16 * kPRowR + 32;   // floats per wave of partial readouts (+32: row-block skew)

struct alignas(16) RowLds {
  float bc[2][2][16 * kBCRow];    // [buffer][B, C][state * kBCRow + step]
  float part[4 * kPWave];         // [wave][row][state][step] partial readouts
  float ia[16 * 16];              // [channel][state] 1/A (the fast quotient's scaled state)
};

// Value of lane k of this lane's 16-lane row (DPP row_newbcast); folded by
// the compiler into the VOP2 instruction that consumes it.
template <int k>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + k, 0xF, 0xF, true));
}

// Value of lane n + k of this lane's 16-lane row, 0 past the row's end (DPP
// row_shl with bound control).
template <int k>
__device__ __forceinline__ float row_shl(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x100 + k, 0xF, 0xF, true));
}

// a + b rounded on its own: not contracted with the product that forms b, so
// that b's DPP broadcast operand keeps a single use and stays folded.
__device__ __forceinline__ float add_nc(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Value v of lane `src` of the wave (ds_bpermute: the LDS crossbar, no LDS memory).
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

template <bool kBF16> struct Raw2;                       // 2 consecutive elements
template <> struct Raw2<true> { uint32_t w; };
template <> struct Raw2<false> { float2 v; };

template <bool kBF16>
__device__ __forceinline__ Raw2<kBF16> load2(const void* base, int64_t off) {
  Raw2<kBF16> r;
  if constexpr (kBF16) r.w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + off);
  else r.v = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + off);
  return r;
}
template <bool kBF16>
__device__ __forceinline__ float at2(const Raw2<kBF16>& r, int j) {
  if constexpr (kBF16) return j ? bf16_hi(r.w) : bf16_lo(r.w);
  else return j ? r.v.y : r.v.x;
}

template <bool kBF16> struct Raw4;                       // 4 consecutive elements (B/C staging)
template <> struct Raw4<true> { uint2 w; };
template <> struct Raw4<false> { float4 v; };

template <bool kBF16>
__device__ __forceinline__ Raw4<kBF16> load4(const void* base, int64_t off, bool ok) {
  Raw4<kBF16> r;
  if constexpr (kBF16) {
    r.w = ok ? *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off) : make_uint2(0, 0);
  } else {
    r.v = ok ? *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off) : make_float4(0, 0, 0, 0);
  }
  return r;
}
template <bool kBF16>
__device__ __forceinline__ float4 widen4(const Raw4<kBF16>& r) {
  if constexpr (kBF16) return make_float4(bf16_lo(r.w.x), bf16_hi(r.w.x), bf16_lo(r.w.y), bf16_hi(r.w.y));
  else return r.v;
}

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maximum): this wave's
// LDS writes are complete, its global loads may still be in flight.
__device__ __forceinline__ void lds_wait_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that waits only for LDS: the prefetched global loads stay
// in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_wait_all();
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int M> struct Tag { static constexpr int kValue = M; };

template <int I, int E, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (I < E) {
    f(Tag<I>{});
    unroll<I + 1, E>(f);
  }
}

// The same values from element loads (rows that are not 4- or 8-byte aligned:
// L not a multiple of 32).
template <bool kBF16>
__device__ __forceinline__ Raw2<kBF16> load2e(const void* base, int64_t off) {
  Raw2<kBF16> r;
  if constexpr (kBF16) {
    const uint16_t* q = static_cast<const uint16_t*>(base) + off;
    r.w = (uint32_t)q[0] | ((uint32_t)q[1] << 16);
  } else {
    const float* q = static_cast<const float*>(base) + off;
    r.v = make_float2(q[0], q[1]);
  }
  return r;
}
template <bool kBF16>
__device__ __forceinline__ Raw4<kBF16> load4e(const void* base, int64_t off, bool ok) {
  Raw4<kBF16> r;
  if constexpr (kBF16) {
    const uint16_t* q = static_cast<const uint16_t*>(base) + off;
    r.w = ok ? make_uint2((uint32_t)q[0] | ((uint32_t)q[1] << 16), (uint32_t)q[2] | ((uint32_t)q[3] << 16))
             : make_uint2(0, 0);
  } else {
    const float* q = static_cast<const float*>(base) + off;
    r.v = ok ? make_float4(q[0], q[1], q[2], q[3]) : make_float4(0, 0, 0, 0);
  }
  return r;
}

template <bool kInBF16>
struct RowRaw {
  Raw2<kInBF16> u, d, z;     // this lane's 2 elements of its channel
  Raw4<kInBF16> bc;          // 4 steps of one B or C row (staging role)
};

// What one workgroup scans: steps t_begin .. t_end - 1 of its 16 channels,
// from the states h0 (null: a zero start).  h_end / s_sum (when not
// null) receive the end state and the sum of delta over the range (a chunk's
// summary for the carry); final_state says whether the end state is also the
// scan's final state.
struct RowTask {
  int64_t t_begin, t_end;
  const float* h0;      // (B, D, N)
  float* h_end;         // (B, D, N)
  float* s_sum;         // (B, D)
  bool final_state;
};

// kSum: the summary role -- the end state of a range that starts from zero,
// without readout, outputs or gate.  With the fast ZOH quotient it is not run
// as a recurrence: over a 32-step chunk with F_t = exp(A * (delta_t + ... +
// delta_31)) (F_32 = 1), unrolling h_t = Abar_t h_{t-1} + (Abar_t - 1)/A B_t u_t
// gives h_31 = F_0 h_{-1} + (1/A) sum_t (F_t - F_{t+1}) B_t u_t, since
// Abar_t F_{t+1} = F_t.  A step then costs 4 VALU + exp instead of 5 + exp;
// the suffix sums of delta come from a 16-lane scan once per chunk, and
// F_t - F_{t+1} cancels to the same degree as the quotient fma(Abar, 1/A, -1/A).
// The full role on the fast quotient keeps g = A h instead of h: the step
// g_t = Abar_t (g_{t-1} + B_t u_t) - B_t u_t is 5 VALU + exp instead of 6 + exp,
// the readout's sum over the row's 16 states weights each product C_t,n g_t,n
// by 1/A_n (an fma in place of an add, about a quarter of a VALU per update),
// and the state is scaled back at the end.  Its rounding error per step,
// 2^-24 max(|g|, |B u|), is that of the fast quotient's coefficient.
// kRag: L not a multiple of 32.  Loads and stores go element by element, and
// the range's last 32-step chunk is shifted back to end at t_end: its steps
// before the previous chunk's end are scanned again with delta = 0 (Abar = 1
// and Bbar u = 0 exactly, so the state is unchanged) and their outputs are
// not stored.
template <bool kInBF16, bool kOutBF16, int kMode, bool kSum, bool kRag>
__device__ __forceinline__ void row_scan(const ScanParams& p, RowLds& s, int64_t b, int64_t d0, const RowTask& task) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r = lane >> 4, n = lane & 15;
  const int64_t D = p.D, N = p.N, L = p.L;
  const int64_t d = d0 + 4 * w + r;
  const bool c_ok = d < D;
  const bool n_ok = n < N;
  const int64_t row = (b * D + (c_ok ? d : 0)) * L;

  // per-lane constants
  float a = (c_ok && n_ok) ? p.A[(c_ok ? d : 0) * N + n] : -1.0f;
  if (__builtin_fabsf(a) < 0x1p-40f) a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f;
  const float a2 = a * kLog2e, ia = 1.0f / a;
  const float bias = !c_ok ? -__builtin_inff() : (p.bias ? p.bias[d] : 0.0f);
  const float dskip = (c_ok && p.Dskip) ? p.Dskip[d] : 0.0f;
  const bool want_z = p.z != nullptr;
  const void* z_src = p.z ? p.z : p.u;

  // B/C staging role: threads 0..127 stage B, 128..255 C; state sn, steps 4*sg .. 4*sg+3
  const int s_arr = tid >> 7, sn = (tid >> 3) & 15, sg = tid & 7;
  const bool s_ok = sn < N;
  const void* s_base = s_arr ? p.Ct : p.Bt;
  const int64_t s_row = (b * N + (s_ok ? sn : 0)) * L;

  const int64_t tb = task.t_begin, te = task.t_end;
  const int64_t nck = (te - tb + kRCT - 1) / kRCT;
  const int64_t rep_end = tb + (nck - 1) * kRCT;   // kRag: the last chunk's steps before this repeat
  auto cstart = [&](int64_t c) -> int64_t {        // first step of chunk c
    const int64_t t = tb + c * kRCT;
    if constexpr (kRag) return c + 1 < nck ? t : te - kRCT;
    else return t;
  };
  auto fetch = [&](int64_t ck, RowRaw<kInBF16>& raw) {
    const int64_t t0 = cstart(ck < nck ? ck : nck - 1);   // clamp: prefetch past the end re-reads the last chunk
    // the summary role reads no C_t (its staging threads stage zeros)
    const bool bc_ok = s_ok && !(kSum && s_arr == 1);
    if constexpr (kRag) {
      raw.u = load2e<kInBF16>(p.u, row + t0 + 2 * n);
      raw.d = load2e<kInBF16>(p.delta, row + t0 + 2 * n);
      if constexpr (!kSum) raw.z = load2e<kInBF16>(z_src, row + t0 + 2 * n);
      raw.bc = load4e<kInBF16>(s_base, s_row + t0 + 4 * sg, bc_ok);
    } else {
      raw.u = load2<kInBF16>(p.u, row + t0 + 2 * n);
      raw.d = load2<kInBF16>(p.delta, row + t0 + 2 * n);
      if constexpr (!kSum) raw.z = load2<kInBF16>(z_src, row + t0 + 2 * n);
      raw.bc = load4<kInBF16>(s_base, s_row + t0 + 4 * sg, bc_ok);
    }
  };
  auto stage = [&](const RowRaw<kInBF16>& raw, int buf) {
    *reinterpret_cast<float4*>(&s.bc[buf][s_arr][sn * kBCRow + 4 * sg]) = widen4<kInBF16>(raw.bc);
  };

  constexpr bool kG = !kSum && kMode == kZohFast;  // the scaled state g = A h (above)
  float h = (task.h0 != nullptr && c_ok && n_ok) ? task.h0[(b * D + d) * N + n] : 0.0f;
  if constexpr (kG) h *= a;
  // kG: 1/A of the row's 16 states, staged once in LDS (the barrier before the
  // first chunk orders it) and read 8 at a time where the readout sums need them
  const float* ia_row = &s.ia[(4 * w + r) * 16];
  if constexpr (kG) s.ia[(4 * w + r) * 16 + n] = ia;
  auto ia8 = [&](int m0, float (&wv)[8]) {
    const float4 lo = *reinterpret_cast<const float4*>(ia_row + m0);
    const float4 hi = *reinterpret_cast<const float4*>(ia_row + m0 + 4);
    wv[0] = lo.x; wv[1] = lo.y; wv[2] = lo.z; wv[3] = lo.w;
    wv[4] = hi.x; wv[5] = hi.y; wv[6] = hi.z; wv[7] = hi.w;
  };
  float dsum = 0.0f;                     // this lane's 2 elements of delta per chunk, summed
  RowRaw<kInBF16> raw[2];
  float dv[2][2], uv[2][2], gv[2][2];   // [chunk parity][element]: delta, u, gate of this lane's 2 elements
  float duv[2][2];                       // delta * u (the simplified rule's per-step factor)
  float q[32];                           // partial readouts of the previous chunk: q[2 * n' + j]
  constexpr bool kW = kSum && kMode == kZohFast;   // the weighted summary (above)
  auto prep = [&](const RowRaw<kInBF16>& rr, int par, int j, int64_t ckx) {   // ckx: rr's chunk
    dv[par][j] = softplus(at2<kInBF16>(rr.d, j) + bias);
    if constexpr (kRag) {
      if (ckx >= nck - 1 && cstart(nck - 1) + 2 * n + j < rep_end) dv[par][j] = 0.0f;
    }
    uv[par][j] = at2<kInBF16>(rr.u, j);
    if constexpr (!kSum) {
      const float gz = silu(at2<kInBF16>(rr.z, j));
      gv[par][j] = want_z ? gz : 1.0f;
    }
    if constexpr (kMode == kDeltaB) duv[par][j] = dv[par][j] * uv[par][j];
  };
  // bf16 outputs leave in whole 128-byte lines: a lane packs its 2 outputs of
  // an even chunk (`held`) and of the following odd chunk, then lane j of a
  // row stores steps 4j .. 4j+3 of that 64-step window, gathered from lanes
  // 2j mod 16 and 2j+1 mod 16 of its row (the even chunk for j < 8, the odd
  // one for j >= 8).  Half lines written a chunk apart were evicted between
  // the halves at the batch-1 long sequence (1.33x the output bytes).
  uint32_t held = 0;
  auto put_pair = [&](int64_t t_even, uint32_t cur) {
    const int s1 = 16 * r + ((2 * n) & 15);
    const uint32_t h1 = lane_read(held, s1), c1 = lane_read(cur, s1);
    const uint32_t h2 = lane_read(held, s1 + 1), c2 = lane_read(cur, s1 + 1);
    const bool first = n < 8;
    if (c_ok)
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + row + t_even + 4 * n) =
          make_uint2(first ? h1 : c1, first ? h2 : c2);
  };
  float* prow = &s.part[w * kPWave + r * (16 * kPRowR + 8) + n * kPRowR];   // this lane's product row
  const float* pread = &s.part[w * kPWave + r * (16 * kPRowR + 8) + 2 * n]; // its outputs' column pair

  fetch(0, raw[0]);
  fetch(1, raw[1]);
  stage(raw[0], 0);
  prep(raw[0], 0, 0, 0);
  prep(raw[0], 0, 1, 0);
#pragma unroll
  for (int i = 0; i < 32; ++i) q[i] = 0.0f;
  uv[1][0] = uv[1][1] = gv[1][0] = gv[1][1] = 0.0f;
  lds_barrier();

  auto chunk = [&](auto ptag, int64_t ck) {
    constexpr int P = decltype(ptag)::kValue;
    constexpr int Q = P ^ 1;
    const int64_t t0 = tb + ck * kRCT;
    fetch(ck + 2, raw[P]);          // chunk ck+2 has the parity of ck; raw[P] was consumed by chunk ck-1
    const float dpair = dv[P][0] + dv[P][1];
    dsum += dpair;
    // kW: sf[j] = sum of delta from this lane's step 2n + j to the chunk's end
    float sf[2] = {0.0f, 0.0f};
    if constexpr (kW) {
      float x = row_shl<1>(dpair);   // exclusive suffix over the row: lanes n+1 .. 15
      x += row_shl<1>(x);
      x += row_shl<2>(x);
      x += row_shl<4>(x);
      x += row_shl<8>(x);
      sf[1] = x + dv[P][1];
      sf[0] = sf[1] + dv[P][0];
    }
    const float* Bs = &s.bc[P][0][n * kBCRow];
    const float* Cs = &s.bc[P][1][n * kBCRow];
    float4 Bq[3], Cq[3];            // B, C of 4-step groups g, g+1, g+2 (rotating)
    Bq[0] = *reinterpret_cast<const float4*>(Bs + 0);
    Cq[0] = *reinterpret_cast<const float4*>(Cs + 0);
    Bq[1] = *reinterpret_cast<const float4*>(Bs + 4);
    Cq[1] = *reinterpret_cast<const float4*>(Cs + 4);
    float e[2][4], in[2][4], o[2];  // [group parity][step of the group]: Abar and Bbar u, prepared a group ahead
    // state-independent part of step t: Abar and Bbar u
    auto pre = [&](auto tt, float& ee, float& ii) {
      constexpr int t = decltype(tt)::kValue;
      const float4& B4 = Bq[(t / 4) % 3];
      const float bn = (t % 4 == 0) ? B4.x : (t % 4 == 1) ? B4.y : (t % 4 == 2) ? B4.z : B4.w;
      if constexpr (kW) {             // ee = F_t, ii = B_t u_t
        ee = hw_exp2(row_bcast<t / 2>(sf[t % 2]) * a2);
        ii = row_bcast<t / 2>(uv[P][t % 2]) * bn;
        return;
      }
      if constexpr (kG) {             // ee = Abar_t, ii = B_t u_t
        ee = hw_exp2(row_bcast<t / 2>(dv[P][t % 2]) * a2);
        ii = row_bcast<t / 2>(uv[P][t % 2]) * bn;
        return;
      }
      const float x = row_bcast<t / 2>(dv[P][t % 2]) * a2;
      ee = hw_exp2(x);
      if constexpr (kMode == kDeltaB) {
        ii = row_bcast<t / 2>(duv[P][t % 2]) * bn;
      } else {
        const float kc = (kMode == kZohFast) ? __builtin_fmaf(ee, ia, -ia) : expm1_from_exp2(x, ee) * ia;
        ii = kc * (row_bcast<t / 2>(uv[P][t % 2]) * bn);
      }
    };
    // the four steps of a group: four independent chains, so that their
    // latencies overlap even with a single wave on the SIMD
    auto pre_group = [&](auto gt) {
      constexpr int G = decltype(gt)::kValue;
      unroll<0, 4>([&](auto it) {
        constexpr int i = decltype(it)::kValue;
        pre(Tag<4 * G + i>{}, e[G & 1][i], in[G & 1][i]);
      });
    };
    pre_group(Tag<0>{});
    const float f0 = e[0][0];       // kW: F_0, the chunk's decay
    float wacc[2] = {0.0f, 0.0f};   // kW: sum of (F_t - F_{t+1}) B_t u_t, even and odd steps
    unroll<0, kRCT / 4>([&](auto gc) {
      constexpr int G = decltype(gc)::kValue;
      // (no scheduling fence here: the compiler's own interleaving of the
      // groups measured 2% faster at the batch-1 long sequence)
      // B/C of group G + 2, two groups ahead
      if constexpr (G + 2 < kRCT / 4) {
        Bq[(G + 2) % 3] = *reinterpret_cast<const float4*>(Bs + 4 * G + 8);
        Cq[(G + 2) % 3] = *reinterpret_cast<const float4*>(Cs + 4 * G + 8);
      }
      // outputs of the previous chunk (parity Q) in the first half: output j
      // over groups 2j, 2j+1, 8 of its 16 products per group
      if constexpr (!kSum && G < 4) {
        constexpr int j = G / 2;            // output j: step 2n + j of chunk ck-1
        constexpr int m0 = 8 * (G % 2);     // products of states m0 .. m0+7
        if constexpr (kG) {   // products of g, each weighted by 1/A of its state
          float wv[8];
          ia8(m0, wv);
          float acc = (G % 2 == 0) ? wv[0] * q[2 * m0 + j] : __builtin_fmaf(wv[0], q[2 * m0 + j], o[j]);
#pragma unroll
          for (int i = 1; i < 8; ++i) acc = __builtin_fmaf(wv[i], q[2 * (m0 + i) + j], acc);
          if constexpr (G % 2 == 0) o[j] = acc;
          else o[j] = __builtin_fmaf(dskip, uv[Q][j], acc) * gv[Q][j];
        } else {
          const float s0 = (q[2 * m0 + j] + q[2 * (m0 + 1) + j]) + (q[2 * (m0 + 2) + j] + q[2 * (m0 + 3) + j]);
          const float s1 = (q[2 * (m0 + 4) + j] + q[2 * (m0 + 5) + j]) + (q[2 * (m0 + 6) + j] + q[2 * (m0 + 7) + j]);
          if constexpr (G % 2 == 0) o[j] = s0 + s1;
          else o[j] = __builtin_fmaf(dskip, uv[Q][j], o[j] + (s0 + s1)) * gv[Q][j];
        }
      }
      if constexpr (!kSum && kRag && G == 4) {
        // chunk ck-1 is not the last: element stores at its unshifted place
        if (c_ok && ck > 0) {
          const int64_t at = row + t0 - kRCT + 2 * n;
          if constexpr (kOutBF16) {
            static_cast<uint16_t*>(p.y)[at] = f32_to_bf16(o[0]);
            static_cast<uint16_t*>(p.y)[at + 1] = f32_to_bf16(o[1]);
          } else {
            static_cast<float*>(p.y)[at] = o[0];
            static_cast<float*>(p.y)[at + 1] = o[1];
          }
        }
      }
      if constexpr (!kSum && !kRag && G == 4) {
        if constexpr (kOutBF16) {
          // chunk ck-1 is even for P = 1 (keep its outputs), odd for P = 0 (store the pair)
          if constexpr (P == 1) held = pack_bf16x2(o[0], o[1]);
          else if (ck > 0) put_pair(t0 - 2 * kRCT, pack_bf16x2(o[0], o[1]));
        } else {
          // fp32: one chunk of a row is already a whole 128-byte line
          if (c_ok && ck > 0)
            *reinterpret_cast<float2*>(static_cast<float*>(p.y) + row + t0 - kRCT + 2 * n) = make_float2(o[0], o[1]);
        }
      }
      // unpack the next chunk (parity Q) in the second half, after its u and gate were used above
      if constexpr (G == 4) prep(raw[Q], Q, 0, ck + 1);
      if constexpr (G == 5) prep(raw[Q], Q, 1, ck + 1);
      if constexpr (G == 6) stage(raw[Q], Q);
      // the next group's state-independent part, then this group's recurrence and products
      if constexpr (G + 1 < kRCT / 4) pre_group(Tag<G + 1>{});
      if constexpr (kW) {
        const float f4 = (G + 1 < kRCT / 4) ? e[(G + 1) & 1][0] : 1.0f;   // F of the next group's first step
        wacc[0] = __builtin_fmaf(e[G & 1][0] - e[G & 1][1], in[G & 1][0], wacc[0]);
        wacc[1] = __builtin_fmaf(e[G & 1][1] - e[G & 1][2], in[G & 1][1], wacc[1]);
        wacc[0] = __builtin_fmaf(e[G & 1][2] - e[G & 1][3], in[G & 1][2], wacc[0]);
        wacc[1] = __builtin_fmaf(e[G & 1][3] - f4, in[G & 1][3], wacc[1]);
      } else if constexpr (kSum) {
        h = __builtin_fmaf(e[G & 1][0], h, in[G & 1][0]);
        h = __builtin_fmaf(e[G & 1][1], h, in[G & 1][1]);
        h = __builtin_fmaf(e[G & 1][2], h, in[G & 1][2]);
        h = __builtin_fmaf(e[G & 1][3], h, in[G & 1][3]);
      } else if constexpr (kG) {
        const float4& C4 = Cq[G % 3];
        float pt[4];
        h = __builtin_fmaf(e[G & 1][0], add_nc(h, in[G & 1][0]), -in[G & 1][0]);
        pt[0] = C4.x * h;
        h = __builtin_fmaf(e[G & 1][1], add_nc(h, in[G & 1][1]), -in[G & 1][1]);
        pt[1] = C4.y * h;
        h = __builtin_fmaf(e[G & 1][2], add_nc(h, in[G & 1][2]), -in[G & 1][2]);
        pt[2] = C4.z * h;
        h = __builtin_fmaf(e[G & 1][3], add_nc(h, in[G & 1][3]), -in[G & 1][3]);
        pt[3] = C4.w * h;
        *reinterpret_cast<float4*>(prow + 4 * G) = make_float4(pt[0], pt[1], pt[2], pt[3]);
      } else {
        const float4& C4 = Cq[G % 3];
        float pt[4];
        h = __builtin_fmaf(e[G & 1][0], h, in[G & 1][0]);
        pt[0] = C4.x * h;
        h = __builtin_fmaf(e[G & 1][1], h, in[G & 1][1]);
        pt[1] = C4.y * h;
        h = __builtin_fmaf(e[G & 1][2], h, in[G & 1][2]);
        pt[2] = C4.z * h;
        h = __builtin_fmaf(e[G & 1][3], h, in[G & 1][3]);
        pt[3] = C4.w * h;
        *reinterpret_cast<float4*>(prow + 4 * G) = make_float4(pt[0], pt[1], pt[2], pt[3]);
      }
    });
    if constexpr (kW) h = __builtin_fmaf(f0, h, (wacc[0] + wacc[1]) * ia);
    // all of this chunk's B/C reads and the next chunk's staging are done by
    // every wave; this wave's products are in LDS (in order before the reads below)
    lds_barrier();
    if constexpr (!kSum) {
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float2 v = *reinterpret_cast<const float2*>(pread + m * kPRowR);
        q[2 * m] = v.x;
        q[2 * m + 1] = v.y;
      }
    }
  };
  // kRag: the last chunk's outputs, element by element, its repeated steps left out
  auto put_last = [&](float o0, float o1) {
    const int64_t t = cstart(nck - 1) + 2 * n;
    if (!c_ok) return;
    if constexpr (kOutBF16) {
      if (t >= rep_end) static_cast<uint16_t*>(p.y)[row + t] = f32_to_bf16(o0);
      if (t + 1 >= rep_end) static_cast<uint16_t*>(p.y)[row + t + 1] = f32_to_bf16(o1);
    } else {
      if (t >= rep_end) static_cast<float*>(p.y)[row + t] = o0;
      if (t + 1 >= rep_end) static_cast<float*>(p.y)[row + t + 1] = o1;
    }
  };
  ProgressPrio prio;    // co-resident workgroups finish together (kernels.hpp)
  prio.begin();
  for (int64_t ck = 0;; ck += 2) {
    prio.at(ck, nck);
    chunk(Tag<0>{}, ck);
    if (ck + 1 >= nck) {
      if constexpr (kSum) break;
      // outputs of the last chunk (parity 0)
      float o0 = 0.0f, o1 = 0.0f;
      float wv[16];
      if constexpr (kG) { ia8(0, *reinterpret_cast<float(*)[8]>(&wv[0])); ia8(8, *reinterpret_cast<float(*)[8]>(&wv[8])); }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if constexpr (kG) { o0 = __builtin_fmaf(wv[m], q[2 * m], o0); o1 = __builtin_fmaf(wv[m], q[2 * m + 1], o1); }
        else { o0 += q[2 * m]; o1 += q[2 * m + 1]; }
      }
      o0 = __builtin_fmaf(dskip, uv[0][0], o0) * gv[0][0];
      o1 = __builtin_fmaf(dskip, uv[0][1], o1) * gv[0][1];
      if constexpr (kRag) {
        put_last(o0, o1);
      } else if (c_ok) {   // an even last chunk: no partner, a half line
        const int64_t at = row + tb + ck * kRCT + 2 * n;
        if constexpr (kOutBF16) *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(p.y) + at) = pack_bf16x2(o0, o1);
        else *reinterpret_cast<float2*>(static_cast<float*>(p.y) + at) = make_float2(o0, o1);
      }
      break;
    }
    chunk(Tag<1>{}, ck + 1);
    if (ck + 2 >= nck) {
      if constexpr (kSum) break;
      float o0 = 0.0f, o1 = 0.0f;
      float wv[16];
      if constexpr (kG) { ia8(0, *reinterpret_cast<float(*)[8]>(&wv[0])); ia8(8, *reinterpret_cast<float(*)[8]>(&wv[8])); }
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        if constexpr (kG) { o0 = __builtin_fmaf(wv[m], q[2 * m], o0); o1 = __builtin_fmaf(wv[m], q[2 * m + 1], o1); }
        else { o0 += q[2 * m]; o1 += q[2 * m + 1]; }
      }
      o0 = __builtin_fmaf(dskip, uv[1][0], o0) * gv[1][0];
      o1 = __builtin_fmaf(dskip, uv[1][1], o1) * gv[1][1];
      if constexpr (kRag) {
        put_last(o0, o1);
      } else if constexpr (kOutBF16) {
        put_pair(tb + ck * kRCT, pack_bf16x2(o0, o1));   // an odd last chunk pairs with the held even one
      } else if (c_ok) {
        *reinterpret_cast<float2*>(static_cast<float*>(p.y) + row + tb + (ck + 1) * kRCT + 2 * n) = make_float2(o0, o1);
      }
      break;
    }
  }
  if constexpr (kG) h *= ia;     // back from g = A h
  if (task.h_end != nullptr && c_ok && n_ok) task.h_end[(b * D + d) * N + n] = h;
  if (task.s_sum != nullptr) {
    // the channel's sum over the 16 lanes of its row (each lane summed 2 elements per chunk)
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1)
      dsum += __builtin_bit_cast(float, lane_read(__builtin_bit_cast(uint32_t, dsum), lane ^ off));
    if (c_ok && n == 0) task.s_sum[b * D + d] = dsum;
  }
  if (task.final_state && p.final_state != nullptr && c_ok && n_ok) p.final_state[(b * D + d) * N + n] = h;
}

// ---------------------------------------------------------------------------
// Lean variant: the same lane layout and arithmetic with registers and LDS cut
// so that five workgroups (five waves per SIMD) fit on a CU, for shapes with
// four or more workgroups per CU, where other waves rather than lookahead
// inside a wave hide latencies.  Differences from row_scan:
//  * lane n of a row holds steps n and n + 16 of a chunk (two 2-byte loads
//    per input for bf16), so that in each 16-step half lane n also owns the
//    output of step n;
//  * the readout goes through LDS every 16 steps (16 products per lane, read
//    back as one 16-state column: 15 adds per output), in a per-wave buffer
//    half the size;
//  * B_t/C_t are read one 4-step group ahead and the step-dependent terms are
//    formed in the step that uses them (inputs are still fetched two chunks
//    ahead, as in row_scan).
// bf16 outputs of two chunks (one 128-byte line per channel) are gathered
// with ds_bpermute so that lane n writes steps 4n .. 4n+3 of the line.

constexpr int kLPitch = 20;                            // floats per product row (16 + padding)
constexpr int kLRowBlk = 16 * kLPitch + 16;            // floats per DPP row (+16: bank skew between rows)
constexpr int kLWave = 3 * kLRowBlk + 16 * kLPitch;    // floats per wave

struct alignas(16) RowLeanLds {
  float bc[2][2][16 * kBCRow];    // [buffer][B, C][state * kBCRow + step], as in RowLds
  float part[4 * kLWave];         // [wave][row][state][step of the half] products
};
static_assert(sizeof(RowLeanLds) <= 32768, "five workgroups per CU need at most 32 KiB of LDS each");

template <bool kBF16> struct Raw1;
template <> struct Raw1<true> { uint32_t h; };   // bf16 pattern in the low half
template <> struct Raw1<false> { float v; };

template <bool kBF16>
__device__ __forceinline__ Raw1<kBF16> load1(const void* base, int64_t off) {
  Raw1<kBF16> r;
  if constexpr (kBF16) r.h = *(static_cast<const uint16_t*>(base) + off);
  else r.v = *(static_cast<const float*>(base) + off);
  return r;
}
template <bool kBF16>
__device__ __forceinline__ float at1(const Raw1<kBF16>& r) {
  if constexpr (kBF16) return __builtin_bit_cast(float, r.h << 16);
  else return r.v;
}

template <bool kInBF16>
struct LeanRaw {
  Raw1<kInBF16> u[2], d[2], z[2];   // steps n and n + 16 of this lane's channel
  Raw4<kInBF16> bc;                 // 4 steps of one B or C row (staging role)
};

__device__ __forceinline__ float comp4(const float4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <bool kInBF16, bool kOutBF16, int kMode>
__device__ __forceinline__ void row_scan_lean(const ScanParams& p, RowLeanLds& s, int64_t b, int64_t d0) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int r = lane >> 4, n = lane & 15;
  const int64_t D = p.D, N = p.N, L = p.L;
  const int64_t d = d0 + 4 * w + r;
  const bool c_ok = d < D;
  const bool n_ok = n < N;
  const int64_t row = (b * D + (c_ok ? d : 0)) * L;

  float a = (c_ok && n_ok) ? p.A[(c_ok ? d : 0) * N + n] : -1.0f;
  if (__builtin_fabsf(a) < 0x1p-40f) a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f;
  const float a2 = a * kLog2e, ia = 1.0f / a;
  const float bias = !c_ok ? -__builtin_inff() : (p.bias ? p.bias[d] : 0.0f);
  const float dskip = (c_ok && p.Dskip) ? p.Dskip[d] : 0.0f;
  const bool want_z = p.z != nullptr;
  const void* z_src = p.z ? p.z : p.u;

  const int s_arr = tid >> 7, sn = (tid >> 3) & 15, sg = tid & 7;
  const bool s_ok = sn < N;
  const void* s_base = s_arr ? p.Ct : p.Bt;
  const int64_t s_row = (b * N + (s_ok ? sn : 0)) * L;

  // chunk counts in 32 bits (the planner gives this kernel L < 2^33), so that
  // the loop's uniform compares stay on the scalar unit
  const int nck = (int)(L / kRCT);
  LeanRaw<kInBF16> raw[2];           // inputs of chunks of each parity, fetched two chunks ahead
  auto fetch = [&](int ck, LeanRaw<kInBF16>& rr) {
    const int c = ck < nck ? ck : nck - 1;     // clamp: the prefetch past the end re-reads the last chunk
    const int64_t at = row + (int64_t)c * kRCT + n;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      rr.u[e] = load1<kInBF16>(p.u, at + 16 * e);
      rr.d[e] = load1<kInBF16>(p.delta, at + 16 * e);
      rr.z[e] = load1<kInBF16>(z_src, at + 16 * e);
    }
    rr.bc = load4<kInBF16>(s_base, s_row + c * kRCT + 4 * sg, s_ok);
  };
  float dv[2], uv[2], gv[2], duv[2];    // [element]: delta, u, gate (and delta * u) of steps n, n + 16
  auto prep = [&](const LeanRaw<kInBF16>& rr) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      dv[e] = softplus(at1<kInBF16>(rr.d[e]) + bias);
      uv[e] = at1<kInBF16>(rr.u[e]);
      const float gz = silu(at1<kInBF16>(rr.z[e]));
      gv[e] = want_z ? gz : 1.0f;
      if constexpr (kMode == kDeltaB) duv[e] = dv[e] * uv[e];
    }
  };
  auto stage = [&](const LeanRaw<kInBF16>& rr, int buf) {
    *reinterpret_cast<float4*>(&s.bc[buf][s_arr][sn * kBCRow + 4 * sg]) = widen4<kInBF16>(rr.bc);
  };

  float* prow = &s.part[w * kLWave + r * kLRowBlk + n * kLPitch];   // this lane's product row
  const float* pcol = &s.part[w * kLWave + r * kLRowBlk + n];       // column of its output step

  // Outputs.  bf16: packed per chunk (held[chunk parity]: steps n, n+16), a
  // 64-step line stored after every odd chunk.  fp32: a 32-step line per chunk.
  uint32_t held[2] = {0u, 0u};
  auto put_bf16 = [&](int64_t t_line, bool whole) {
    const int qh = n >> 2;                        // half of the line's 4 halves that steps 4n.. lie in
    const int src = 16 * r + 4 * (n & 3);         // lanes holding steps 4n .. 4n+3
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x0 = lane_read(held[0], src + j), x1 = lane_read(held[1], src + j);
      v[j] = qh < 2 ? x0 : x1;
    }
    const bool hi = qh & 1;
    const uint32_t w01 = hi ? ((v[0] >> 16) | (v[1] & 0xffff0000u)) : ((v[0] & 0xffffu) | (v[1] << 16));
    const uint32_t w23 = hi ? ((v[2] >> 16) | (v[3] & 0xffff0000u)) : ((v[2] & 0xffffu) | (v[3] << 16));
    if (c_ok && (whole || qh < 2))
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + row + t_line + 4 * n) = make_uint2(w01, w23);
  };
  auto put_f32 = [&](int64_t t0, float o0, float o1) {
    const int src = 16 * r + ((2 * n) & 15);      // lanes holding steps 2n, 2n+1 (half n >> 3)
    const bool second = n >= 8;
    const float a0 = __builtin_bit_cast(float, lane_read(__builtin_bit_cast(uint32_t, o0), src));
    const float b0 = __builtin_bit_cast(float, lane_read(__builtin_bit_cast(uint32_t, o1), src));
    const float a1 = __builtin_bit_cast(float, lane_read(__builtin_bit_cast(uint32_t, o0), src + 1));
    const float b1 = __builtin_bit_cast(float, lane_read(__builtin_bit_cast(uint32_t, o1), src + 1));
    if (c_ok)
      *reinterpret_cast<float2*>(static_cast<float*>(p.y) + row + t0 + 2 * n) =
          make_float2(second ? b0 : a0, second ? b1 : a1);
  };

  // On the fast quotient the state is kept scaled by A, as in row_scan: g = A h,
  // g_t = Abar_t (g_{t-1} + B_t u_t) - B_t u_t, and the readout weights each
  // state's product by 1/A (the row's 16 values, held in registers).
  constexpr bool kG = kMode == kZohFast;
  float iam[16];
  if constexpr (kG) unroll<0, 16>([&](auto mt) { iam[decltype(mt)::kValue] = row_bcast<decltype(mt)::kValue>(ia); });
  float h = 0.0f;
  fetch(0, raw[0]);
  fetch(1, raw[1]);
  stage(raw[0], 0);
  prep(raw[0]);
  lds_barrier();

  auto chunk = [&](auto ptag, int ck) {
    constexpr int P = decltype(ptag)::kValue;
    const int64_t t0 = (int64_t)ck * kRCT;
    fetch(ck + 2, raw[P]);          // raw[P] held chunk ck, already unpacked and staged
    const float* Bs = &s.bc[P][0][n * kBCRow];
    const float* Cs = &s.bc[P][1][n * kBCRow];
    float oh[2];
    unroll<0, 2>([&](auto ht) {
      constexpr int hf = decltype(ht)::kValue;
      float4 Bq = *reinterpret_cast<const float4*>(Bs + 16 * hf);
      float4 Cq = *reinterpret_cast<const float4*>(Cs + 16 * hf);
      unroll<0, 4>([&](auto gt) {
        constexpr int g = decltype(gt)::kValue;
        float4 Bn = Bq, Cn = Cq;
        if constexpr (g < 3) {
          Bn = *reinterpret_cast<const float4*>(Bs + 16 * hf + 4 * g + 4);
          Cn = *reinterpret_cast<const float4*>(Cs + 16 * hf + 4 * g + 4);
        }
        float pt[4];
        unroll<0, 4>([&](auto it) {
          constexpr int i = decltype(it)::kValue;
          constexpr int k = 4 * g + i;     // step 16 hf + k: element hf of lane k of the row
          const float bn = comp4(Bq, i);
          const float x = row_bcast<k>(dv[hf]) * a2;
          const float ee = hw_exp2(x);
          float ii;
          if constexpr (kG) {
            ii = row_bcast<k>(uv[hf]) * bn;
            h = __builtin_fmaf(ee, add_nc(h, ii), -ii);
          } else {
            if constexpr (kMode == kDeltaB) {
              ii = row_bcast<k>(duv[hf]) * bn;
            } else {
              ii = (expm1_from_exp2(x, ee) * ia) * (row_bcast<k>(uv[hf]) * bn);
            }
            h = __builtin_fmaf(ee, h, ii);
          }
          pt[i] = comp4(Cq, i) * h;
        });
        *reinterpret_cast<float4*>(prow + 4 * g) = make_float4(pt[0], pt[1], pt[2], pt[3]);
        Bq = Bn;
        Cq = Cn;
      });
      // readout of step 16 hf + n: the 16 states' products of this row (this
      // wave's own LDS writes, which the LDS performs in order)
      float v[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) v[m] = pcol[m * kLPitch];
      float y;
      if constexpr (kG) {
        float y0 = iam[0] * v[0], y1 = iam[8] * v[8];
#pragma unroll
        for (int m = 1; m < 8; ++m) {
          y0 = __builtin_fmaf(iam[m], v[m], y0);
          y1 = __builtin_fmaf(iam[8 + m], v[8 + m], y1);
        }
        y = y0 + y1;
      } else {
        y = (((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]))) +
            (((v[8] + v[9]) + (v[10] + v[11])) + ((v[12] + v[13]) + (v[14] + v[15])));
      }
      oh[hf] = __builtin_fmaf(dskip, uv[hf], y) * gv[hf];
    });
    if constexpr (kOutBF16) {
      held[P] = pack_bf16x2(oh[0], oh[1]);
      if constexpr (P == 1) put_bf16(t0 - kRCT, true);
      else if (ck + 1 == nck) put_bf16(t0, false);   // an even last chunk: the first half of a line
    } else {
      put_f32(t0, oh[0], oh[1]);
    }
    if (ck + 1 < nck) {
      prep(raw[P ^ 1]);
      stage(raw[P ^ 1], P ^ 1);
    }
    lds_barrier();
  };
  ProgressPrio prio;    // co-resident workgroups finish together (kernels.hpp)
  prio.begin();
  for (int ck = 0;; ck += 2) {
    prio.at((uint32_t)ck, (uint32_t)nck);
    chunk(Tag<0>{}, ck);
    if (ck + 1 >= nck) break;
    chunk(Tag<1>{}, ck + 1);
    if (ck + 2 >= nck) break;
  }
  if constexpr (kG) h *= ia;     // back from g = A h
  if (p.final_state != nullptr && c_ok && n_ok) p.final_state[(b * D + d) * N + n] = h;
}

template <bool kInBF16, bool kOutBF16>
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(5)))
scan_row_lean_kernel(ScanParams p) {
  __shared__ RowLeanLds s;
  const int64_t tiles_d = (p.D + 15) / 16;
  const int64_t b = (int64_t)blockIdx.x / tiles_d;
  const int64_t d0 = ((int64_t)blockIdx.x - b * tiles_d) * 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t d = d0 + 4 * w + (lane >> 4);
  const int n = lane & 15;
  const bool small_a = d < p.D && n < p.N && __builtin_fabsf(p.A[d * p.N + n]) < kFastZohMinAbsA;
  const int any_small = __syncthreads_or(small_a ? 1 : 0);
  if (p.delta_b) row_scan_lean<kInBF16, kOutBF16, kDeltaB>(p, s, b, d0);
  else if (!kInBF16 || p.accurate || any_small) row_scan_lean<kInBF16, kOutBF16, kZohAccurate>(p, s, b, d0);
  else row_scan_lean<kInBF16, kOutBF16, kZohFast>(p, s, b, d0);
}

// phase 0: the whole sequence, one workgroup per 16-channel tile.  With L in
// K chunks of p.chunk_len steps (p.n_chunks = K): phase 1 runs chunk 0 in
// full and chunks 1 .. K-2 as summaries (workgroup index = chunk x tiles +
// tile), each storing its end state and sum of delta from a zero start; the
// carry kernel then chains them into start states; phase 2 runs chunks
// 1 .. K-1 in full from those.  Both phases put (K - 1) workgroups on every
// tile, so a sequence with one tile per CU runs three or more per CU.
template <bool kInBF16, bool kOutBF16>
// Three workgroups per CU (the LDS allows three): the register budget is held
// to the 168 VGPRs that three waves per SIMD leave.
__global__ void __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(3)))
scan_row_kernel(ScanParams p, int phase) {
  __shared__ RowLds s;
  const int64_t tiles_d = (p.D + 15) / 16;
  const int64_t bt = p.B * tiles_d;
  const int64_t tile = (int64_t)blockIdx.x % bt, c = (int64_t)blockIdx.x / bt;
  const int64_t b = tile / tiles_d;
  const int64_t d0 = (tile - b * tiles_d) * 16;
  const int64_t bdn = p.B * p.D * p.N, bd = p.B * p.D;
  RowTask task{0, p.L, nullptr, nullptr, nullptr, true};
  bool sum_role = false;
  if (phase == 1) {
    task.t_begin = c * p.chunk_len;
    task.t_end = task.t_begin + p.chunk_len;
    task.h_end = p.h_local + c * bdn;
    task.s_sum = p.s_sum + c * bd;
    task.final_state = false;
    sum_role = c > 0;
  } else if (phase == 2) {
    const int64_t ch = c + 1;
    task.t_begin = ch * p.chunk_len;
    task.t_end = p.L - task.t_begin < p.chunk_len ? p.L : task.t_begin + p.chunk_len;
    task.h0 = p.h_start + ch * bdn;
    task.final_state = ch == p.n_chunks - 1;
  }
  // the discretisation loop, uniform over the workgroup: the cancellation-free
  // quotient when asked for or when any |A| of the tile is small; fp32 inputs
  // always ask for it, so their instance has no fast-quotient loop at all
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t d = d0 + 4 * w + (lane >> 4);
  const int n = lane & 15;
  const bool small_a = d < p.D && n < p.N && __builtin_fabsf(p.A[d * p.N + n]) < kFastZohMinAbsA;
  const int any_small = __syncthreads_or(small_a ? 1 : 0);
  // L not a multiple of 32: rows start at any element (element loads), and a
  // range that ends at L has a shifted last chunk
  const bool rag = p.L % kRCT != 0;
  if (sum_role && rag) {
    if (p.delta_b) row_scan<kInBF16, kOutBF16, kDeltaB, true, true>(p, s, b, d0, task);
    else if (!kInBF16 || p.accurate || any_small) row_scan<kInBF16, kOutBF16, kZohAccurate, true, true>(p, s, b, d0, task);
    else row_scan<kInBF16, kOutBF16, kZohFast, true, true>(p, s, b, d0, task);
  } else if (sum_role) {
    if (p.delta_b) row_scan<kInBF16, kOutBF16, kDeltaB, true, false>(p, s, b, d0, task);
    else if (!kInBF16 || p.accurate || any_small) row_scan<kInBF16, kOutBF16, kZohAccurate, true, false>(p, s, b, d0, task);
    else row_scan<kInBF16, kOutBF16, kZohFast, true, false>(p, s, b, d0, task);
  } else if (rag) {
    if (p.delta_b) row_scan<kInBF16, kOutBF16, kDeltaB, false, true>(p, s, b, d0, task);
    else if (!kInBF16 || p.accurate || any_small) row_scan<kInBF16, kOutBF16, kZohAccurate, false, true>(p, s, b, d0, task);
    else row_scan<kInBF16, kOutBF16, kZohFast, false, true>(p, s, b, d0, task);
  } else {
    if (p.delta_b) row_scan<kInBF16, kOutBF16, kDeltaB, false, false>(p, s, b, d0, task);
    else if (!kInBF16 || p.accurate || any_small) row_scan<kInBF16, kOutBF16, kZohAccurate, false, false>(p, s, b, d0, task);
    else row_scan<kInBF16, kOutBF16, kZohFast, false, false>(p, s, b, d0, task);
  }
}

template <bool kInBF16, bool kOutBF16>
hipError_t launch_row_t(const ScanParams& p, bool lean, int phase, hipStream_t st) {
  const int64_t tiles = p.B * ((p.D + 15) / 16);
  const int64_t grid = phase == 0 ? tiles : (p.n_chunks - 1) * tiles;
  if (grid <= 0) return hipSuccess;
  if (lean) hipLaunchKernelGGL((scan_row_lean_kernel<kInBF16, kOutBF16>), dim3((unsigned)grid), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((scan_row_kernel<kInBF16, kOutBF16>), dim3((unsigned)grid), dim3(256), 0, st, p, phase);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_row(const ScanParams& p, Dt in, Dt out, bool lean, int phase, hipStream_t s) {
  if (lean && phase != 0) return hipErrorInvalidValue;   // the lean variant runs whole sequences only
  if (in == Dt::BF16) return out == Dt::BF16 ? launch_row_t<true, true>(p, lean, phase, s) : launch_row_t<true, false>(p, lean, phase, s);
  return out == Dt::BF16 ? launch_row_t<false, true>(p, lean, phase, s) : launch_row_t<false, false>(p, lean, phase, s);
}

}  // namespace mamba

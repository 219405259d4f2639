// scan_v4.hpp -- main selective-scan kernel for gfx950 (L a multiple of 8, at
// least 32; 16-byte aligned rows).  Included by scan_v4_bf16.hip and scan_v4_f32.hip,
// which instantiate it for one input dtype each (they compile in parallel).  Computes what scan_fwd.hip computes ("Mamba 模型",
// full-step flowchart nodes H to M; ZOH per "Mamba模型：高效序列建模的新突破"
// 3.1): softplus step, ZOH discretisation, recurrence, readout, skip, gate.
//
// Layout on the GPU -- one wave is a whole, independent unit of work:
//  * a wave owns a tile of 16 channels of one batch row; four lanes (a quad)
//    per channel, each lane holding 4 of the 16 states in VGPRs;
//  * the readout sum over the 16 states is 4 in-lane FMAs per step; the
//    quad's partial sums go through LDS once per chunk to the lane that owns
//    the step (3 adds per output);
//  * the sequence is walked in 32-step chunks.  A lane loads u, delta_raw, z
//    of its channel for 8 consecutive steps (8g .. 8g+7) with one 16-byte
//    load each, two chunks ahead; delta = softplus(delta_raw + bias) is
//    evaluated once per element, and u and delta stay in VGPRs: step t reads
//    them from lane t/8 of the quad through a DPP broadcast folded into the
//    consuming instruction.  B_t and C_t of a chunk are staged step-major in
//    the wave's own double-buffered LDS region, so a lane reads its 4 states
//    of B or C with one 16-byte LDS read;
//  * lane g of a quad keeps the outputs of steps 8g..8g+7, adds D u, applies
//    the gate and writes them with one 16-byte store;
//  * workgroups are single waves, so no workgroup barrier is ever needed.
// Balanced split: with at least as many tiles as waves, the (tile x 32-step
// block) work is cut into equal contiguous ranges, one per wave.  A tile cut
// between waves g and g+1 is scanned by g from t = 0 to the cut (done first,
// its end state published to a slot marked with this launch's epoch) and by
// g+1 from the cut to the end (done last, after reading the slot).  The wait
// is bounded; if it runs out, g+1 recomputes the state at the cut itself, so
// the kernel always finishes.
// Per ZOH state update: 6 fp32 VALU + 1 v_exp_f32; per 32-step chunk and lane
// 64 LDS reads of B/C, 16 staging writes, 8 + 8 readout-transpose accesses.
#pragma once

#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

constexpr int kTile = 16;     // channels per wave
constexpr int kNS = 4;        // states per lane
constexpr int kCT = 32;       // steps per chunk
constexpr int kSlot = kTile * 16;   // floats per hand-over slot

constexpr int kPRow = 36;     // floats per lane row of the readout transpose (32 + padding)

struct WaveLds {
  float4 B4[2][kCT * 4];      // B_t, [buffer][step][state quad] (16-byte reads of 4 states)
  float4 C4[2][kCT * 4];      // C_t, same layout
  float P[64 * kPRow];        // per-lane partial readouts of one chunk, [lane][step]
};

template <bool kBF16> struct Raw8;   // 8 consecutive elements
template <> struct Raw8<true> { uint4 w; };
template <> struct Raw8<false> { float4 a, b; };

template <bool kBF16>
__device__ __forceinline__ Raw8<kBF16> load8(const void* base, int64_t off, bool ok) {
  Raw8<kBF16> r;
  if constexpr (kBF16) {
    r.w = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off) : make_uint4(0, 0, 0, 0);
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    r.a = ok ? p[0] : make_float4(0, 0, 0, 0);
    r.b = ok ? p[1] : make_float4(0, 0, 0, 0);
  }
  return r;
}

template <bool kBF16>
__device__ __forceinline__ float at8(const Raw8<kBF16>& r, int j) {
  if constexpr (kBF16) {
    const uint32_t w = (j < 2) ? r.w.x : (j < 4) ? r.w.y : (j < 6) ? r.w.z : r.w.w;
    return (j & 1) ? bf16_hi(w) : bf16_lo(w);
  } else {
    const float4 v = (j < 4) ? r.a : r.b;
    const int k = j & 3;
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
  }
}

// Value of lane q of this lane's quad (DPP quad_perm [q,q,q,q]); folded by
// the compiler into the instruction that consumes it.
template <int q>
__device__ __forceinline__ float quad_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), q * 0x55, 0xF, 0xF, true));
}

// Sum over the four lanes of a quad (result in every lane): two adds whose
// second operand comes from another lane of the quad through DPP.
__device__ __forceinline__ float quad_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  return v;
}

struct Consts {
  float a2[kNS];   // A * log2(e)
  float ia[kNS];   // 1 / A
  float bias, dskip;
  int accurate;    // wave-uniform
};

__device__ __forceinline__ Consts load_consts(const ScanParams& p, int64_t d, bool d_ok, int g) {
  Consts k;
  bool small_a = false;
#pragma unroll
  for (int i = 0; i < kNS; ++i) {
    const int n = 4 * g + i;
    float a = (d_ok && n < p.N) ? p.A[d * p.N + n] : -1.0f;
    if (__builtin_fabsf(a) < kFastZohMinAbsA) small_a = true;
    // |A| < 2^-40 (including 0) becomes -2^-40 (sign kept): the ZOH coefficient
    // is then delta to within delta * 2^-41 (resolved by the accurate loop).
    if (__builtin_fabsf(a) < 0x1p-40f) a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f;
    k.a2[i] = a * kLog2e;
    k.ia[i] = 1.0f / a;
  }
  // -inf for channels past D: their delta is then exactly 0 (softplus(-inf)),
  // so their state stays 0 whatever they read.
  k.bias = !d_ok ? -__builtin_inff() : (p.bias ? p.bias[d] : 0.0f);
  k.dskip = (d_ok && p.Dskip) ? p.Dskip[d] : 0.0f;
  k.accurate = (p.accurate || __any(small_a)) ? 1 : 0;
  return k;
}

template <int M> struct ModeTag { static constexpr int kValue = M; };

// Calls f(ModeTag<i>{}) for i = I .. E-1 (compile-time step indices).
template <int I, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < E) {
    f(ModeTag<I>{});
    static_for<I + 1, E>(f);
  }
}

template <bool kBF16>
struct ChunkRaw {
  Raw8<kBF16> u, d, z;        // channel c, steps 8g .. 8g+7
  Raw8<kBF16> bc0, bc1;       // B or C row n, steps 16h .. 16h+15
};

// One tile-segment scan.  Every lane of the wave must call it.
//
// Software pipeline over 32-step chunks, all within one wave (so no
// barriers; the wave's LDS accesses are processed in order).  While the 32
// steps of chunk k run, the wave also
//   * has the global loads of chunk k+2 in flight,
//   * unpacks chunk k+1 (softplus of delta, u, the gate of z) in its second
//     half and stages its B_t/C_t in the other LDS buffer,
//   * finishes chunk k-1's outputs (sum of the quad's partial readouts, skip
//     term, gate) in its first half and stores them at step 16,
// so that independent work fills the latency of the recurrence.  Inside the
// chunk, B/C of step t+3 are read, the state-independent part of step t+1 is
// computed and step t updates h and forms this lane's partial readout
// (4 states).  After the steps the 32 partials go through LDS to the lane
// that owns each step's output (lane g owns steps 8g .. 8g+7), and the first
// step of chunk k+1 is prepared.
//
// Every per-chunk buffer alternates between two copies, selected by the
// chunk's parity, and the chunk loop is unrolled twice, so nothing is copied
// between chunks.  Prefetch addresses past the segment are clamped to its
// last chunk, so the step loop has no branches.
//
// kN16: N == 16.  Then every B/C lane holds a real state and all loads are
// unconditional; otherwise lanes of absent states load zeros.
// kRagged: the segment's length may not be a multiple of kCT (see below);
// a separate instance, so that aligned lengths run the plain loop.
template <bool kInBF16, bool kOutBF16, bool kReadout, bool kN16, bool kRagged = false>
struct Segment {
  static __device__ __forceinline__ float run(const ScanParams& p, WaveLds& s, int64_t b, int64_t d0,
                                              int64_t t_begin, int64_t t_end, float (&h)[kNS], const Consts& k,
                                              int mode) {
    const int lane = threadIdx.x & 63;
    const int c = lane >> 2, g = lane & 3;
    const int64_t D = p.D, N = p.N, L = p.L;
    const int64_t d = d0 + c;
    const bool c_ok = d < D;
    // Channels past D read channel 0 (always in bounds); their delta is 0 (bias
    // -inf), so their state stays 0, and their outputs are not stored.
    const int64_t row = (b * D + (c_ok ? d : 0)) * L;
    // B/C staging role: lanes 0..31 -> B, 32..63 -> C; state bc_n, steps 16*bc_h .. +15
    const int bc_arr = lane >> 5, bc_n = (lane >> 1) & 15, bc_h = lane & 1;
    const bool bc_ok = kN16 || (bc_n < N && (kReadout || bc_arr == 0));
    const void* bc_base = bc_arr ? p.Ct : p.Bt;
    const int64_t bc_row = (b * N + (bc_n < N ? bc_n : 0)) * L;
    const bool want_z = kReadout && p.z != nullptr;
    // z is always loaded (from u when there is no gate, then discarded): a
    // conditional load would leave the compiler unsure how many loads are in
    // flight, and its waits would then cover the newest prefetch as well.
    const void* z_src = p.z ? p.z : p.u;

    // A segment whose length is not a multiple of kCT (the sequence's end,
    // L % kCT != 0, L % 8 == 0) ends with a chunk shifted back to [t_end - kCT,
    // t_end): its first `skip` steps were already scanned, so they run with
    // delta = 0 (bias -inf: Abar = 1 and Bbar = 0 exactly, h unchanged) and
    // their outputs are not stored.  skip is a multiple of 8, so each lane's
    // 8 steps are either all repeated or all new.
    const int64_t nck = kRagged ? (t_end - t_begin + kCT - 1) / kCT : (t_end - t_begin) / kCT;
    if (nck <= 0) return 0.0f;
    const int64_t t_last = t_end - kCT;
    const int skip = kRagged ? (int)(nck * kCT - (t_end - t_begin)) : 0;
    const bool new_steps = 8 * g >= skip;     // this lane's steps of the last chunk are not repeats
    const bool out_last = kRagged ? (c_ok && new_steps) : c_ok;
    const float bias_last = (kRagged && !new_steps) ? -__builtin_inff() : k.bias;

    auto fetch = [&](int64_t t0, ChunkRaw<kInBF16>& r) {
      t0 = t0 < t_last ? t0 : t_last;     // clamp: stays inside the segment
      r.u = load8<kInBF16>(p.u, row + t0 + 8 * g, true);
      r.d = load8<kInBF16>(p.delta, row + t0 + 8 * g, true);
      if constexpr (kReadout) r.z = load8<kInBF16>(z_src, row + t0 + 8 * g, true);
      r.bc0 = load8<kInBF16>(bc_base, bc_row + t0 + 16 * bc_h, bc_ok);
      r.bc1 = load8<kInBF16>(bc_base, bc_row + t0 + 16 * bc_h + 8, bc_ok);
    };
    auto stage_bc = [&](const ChunkRaw<kInBF16>& r, int buf, int j) {   // values j and 8+j of this lane's 16
      float* dst = reinterpret_cast<float*>(bc_arr ? s.C4[buf] : s.B4[buf]);
      dst[(16 * bc_h + j) * 16 + bc_n] = at8<kInBF16>(r.bc0, j);
      dst[(16 * bc_h + 8 + j) * 16 + bc_n] = at8<kInBF16>(r.bc1, j);
    };
    // Channels past D carry bias = -inf, so delta = softplus(-inf) = 0 there
    // without a per-element select; so do the repeated steps of a shifted
    // last chunk (bias_last).
    auto delta_of = [&](const ChunkRaw<kInBF16>& r, int j, float bias) {
      return softplus(at8<kInBF16>(r.d, j) + bias);
    };
    auto gate_of = [&](const Raw8<kInBF16>& z, int j) {
      const float gz = silu(at8<kInBF16>(z, j));
      return want_z ? gz : 1.0f;
    };
    auto pack8 = [&](const float (&o)[8]) {
      return make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                        pack_bf16x2(o[6], o[7]));
    };
    auto store_w = [&](int64_t t0, const uint4& wv) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.y) + row + t0 + 8 * g) = wv;
    };
    uint4 held = make_uint4(0, 0, 0, 0);   // bf16 outputs of the last even chunk, not yet stored
    int64_t held_at = 0;
    auto store_out = [&](int64_t t0, const float (&o)[8]) {
      const int64_t at = row + t0 + 8 * g;
      if constexpr (kOutBF16) {
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.y) + at) =
            make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7]));
      } else {
        float4* q4 = reinterpret_cast<float4*>(static_cast<float*>(p.y) + at);
        q4[0] = make_float4(o[0], o[1], o[2], o[3]);
        q4[1] = make_float4(o[4], o[5], o[6], o[7]);
      }
    };

    float dsum = 0.0f;
    ChunkRaw<kInBF16> raw[2];          // raw inputs, chunk parity
    float dv[2][8], uv[2][8], gv[2][8];  // delta, u, gate of this lane's steps 8g..8g+7, chunk parity
    float q[32];                       // partial readouts of the previous chunk, q[8*g' + j]:
                                       // lane g' of the quad, step 8g + j

    fetch(t_begin, raw[0]);
    const float bias0 = (kRagged && nck == 1) ? bias_last : k.bias;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dv[0][j] = delta_of(raw[0], j, bias0);
      uv[0][j] = at8<kInBF16>(raw[0].u, j);
      if constexpr (kReadout) gv[0][j] = gate_of(raw[0].z, j);
      stage_bc(raw[0], 0, j);
    }
    fetch(t_begin + kCT, raw[1]);
#pragma unroll
    for (int j = 0; j < 32; ++j) q[j] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) { uv[1][j] = 0.0f; gv[1][j] = 0.0f; }   // read (unused) by chunk 0

    auto pipeline = [&](auto mode_tag) {
      constexpr int M = decltype(mode_tag)::kValue;
      // state-independent part of a step: Abar and Bbar u for this lane's 4 states
      auto pre = [&](float dt, float ut, const float4& B, float (&e)[kNS], float (&in)[kNS]) {
        const float bn[4] = {B.x, B.y, B.z, B.w};
#pragma unroll
        for (int i = 0; i < kNS; ++i) {
          const float x = dt * k.a2[i];
          e[i] = hw_exp2(x);
          if constexpr (M == kDeltaB) {
            in[i] = (dt * ut) * bn[i];
          } else {
            const float kc = (M == kZohFast) ? __builtin_fmaf(e[i], k.ia[i], -k.ia[i])
                                             : expm1_from_exp2(x, e[i]) * k.ia[i];
            in[i] = kc * (ut * bn[i]);
          }
        }
      };
      float4 Bn0, Bn1, Bn2, Cn0, Cn1, Cn2;   // B/C of steps 0..2 of the coming chunk
      float evn[kNS], invn[kNS];      // its step 0, prepared
      auto read_next = [&](int buf) {
        Bn0 = s.B4[buf][0 * 4 + g];
        Bn1 = s.B4[buf][1 * 4 + g];
        Bn2 = s.B4[buf][2 * 4 + g];
        if constexpr (kReadout) {
          Cn0 = s.C4[buf][0 * 4 + g];
          Cn1 = s.C4[buf][1 * 4 + g];
          Cn2 = s.C4[buf][2 * 4 + g];
        }
      };
      auto pre_next = [&](auto pc) {
        constexpr int Pn = decltype(pc)::kValue;
        pre(quad_bcast<0>(dv[Pn][0]), quad_bcast<0>(uv[Pn][0]), Bn0, evn, invn);
      };
      read_next(0);
      pre_next(ModeTag<0>{});

      auto chunk = [&](auto ptag, int64_t ck) {
        constexpr int P = decltype(ptag)::kValue;
        constexpr int Q = P ^ 1;
        const int64_t t0 = t_begin + ck * kCT;
        fetch(t0 + 2 * kCT, raw[P]);            // chunk ck+2 has the parity of ck
        const float bias_n = (kRagged && ck + 2 == nck) ? bias_last : k.bias;   // for chunk ck+1
        if constexpr (!kReadout) {
#pragma unroll
          for (int j = 0; j < 8; ++j) dsum += dv[P][j];
        }
        float4 Bv[kCT], Cv[kCT];
        float ev[2][kNS], inv[2][kNS];
        float pt[4], o[8];
        float4* row_w = reinterpret_cast<float4*>(&s.P[lane * kPRow]);
        const float4* B4 = s.B4[P];
        const float4* C4 = s.C4[P];
        Bv[0] = Bn0; Bv[1] = Bn1; Bv[2] = Bn2;
        if constexpr (kReadout) { Cv[0] = Cn0; Cv[1] = Cn1; Cv[2] = Cn2; }
#pragma unroll
        for (int i = 0; i < kNS; ++i) { ev[0][i] = evn[i]; inv[0][i] = invn[i]; }
        static_for<0, kCT>([&](auto tc) {
          constexpr int t = decltype(tc)::kValue;
          // Keep the software pipeline as written: without this fence the
          // scheduler sinks the B/C reads of step t+3 next to their use and
          // every step then waits for LDS.
          __builtin_amdgcn_sched_barrier(0);
          // independent work of the neighbouring chunks, two items every 4 steps
          if constexpr (kReadout && t % 2 == 1 && t < 16) {   // output t/2 of chunk ck-1 (parity Q)
            constexpr int jo = t / 2;
            const float y = (q[jo] + q[8 + jo]) + (q[16 + jo] + q[24 + jo]);
            o[jo] = __builtin_fmaf(k.dskip, uv[Q][jo], y) * gv[Q][jo];
          }
          // Outputs of chunk ck-1 leave at mid-chunk, long before the next
          // chunk waits on its loads (stores count in the same counter).  Chunk
          // 0 has none yet: it writes its own first chunk (where the last
          // chunk's outputs go when it is the only one), which the real
          // outputs overwrite later (same lane, same address, program order).
          if constexpr (kReadout && t == 16) {
            if constexpr (kOutBF16) {
              // bf16: a quad writes 64 bytes of a channel per chunk, half a
              // 128-byte line.  An even chunk's outputs are held and stored
              // right before the next chunk's, so each line's halves reach the
              // L2 back to back; a chunk apart they were evicted in between
              // (1.2x the output bytes).
              const uint4 wv = pack8(o);
              if constexpr (P == 1) {
                held = wv;
                held_at = t0 - kCT;
              } else if (ck > 0 && c_ok) {
                store_w(held_at, held);
                store_w(t0 - kCT, wv);
              }
            } else if constexpr (kRagged) {
              if (ck > 0 || nck > 1 ? c_ok : out_last) store_out(ck > 0 ? t0 - kCT : (nck > 1 ? t0 : t_last), o);
            } else {
              if (c_ok) store_out(ck > 0 ? t0 - kCT : t0, o);
            }
          }
          // Unpack chunk ck+1 (parity Q) in the second half: its loads were
          // issued at the start of chunk ck-1, so they have 1.5 chunks to land,
          // and output t/2 of chunk ck-1 has already used uv[Q], gv[Q].
          if constexpr (t >= 17 && t % 2 == 1) {
            constexpr int ju = (t - 17) / 2;
            dv[Q][ju] = delta_of(raw[Q], ju, bias_n);
            uv[Q][ju] = at8<kInBF16>(raw[Q].u, ju);
            if constexpr (kReadout) gv[Q][ju] = gate_of(raw[Q].z, ju);
            stage_bc(raw[Q], Q, ju);
          }
          // the recurrence
          if constexpr (t + 3 < kCT) {
            Bv[t + 3] = B4[(t + 3) * 4 + g];
            if constexpr (kReadout) Cv[t + 3] = C4[(t + 3) * 4 + g];
          }
          if constexpr (t + 1 < kCT)
            pre(quad_bcast<(t + 1) / 8>(dv[P][(t + 1) % 8]), quad_bcast<(t + 1) / 8>(uv[P][(t + 1) % 8]),
                Bv[t + 1], ev[(t + 1) & 1], inv[(t + 1) & 1]);
          float acc = 0.0f;
#pragma unroll
          for (int i = 0; i < kNS; ++i) {
            h[i] = __builtin_fmaf(ev[t & 1][i], h[i], inv[t & 1][i]);
            if constexpr (kReadout) {
              const float cn = (i == 0) ? Cv[t].x : (i == 1) ? Cv[t].y : (i == 2) ? Cv[t].z : Cv[t].w;
              acc = (i == 0) ? cn * h[i] : __builtin_fmaf(cn, h[i], acc);
            }
          }
          if constexpr (kReadout) {
            pt[t % 4] = acc;
            if constexpr (t % 4 == 3) row_w[t / 4] = make_float4(pt[0], pt[1], pt[2], pt[3]);
          }
          // step 0 of chunk ck+1 (B/C of its steps 0..2 were staged at steps 17..21)
          if constexpr (t == kCT - 5) read_next(Q);
          if constexpr (t == kCT - 2) pre_next(ModeTag<Q>{});
        });
        if constexpr (kReadout) {
          // partial readouts (written every 4 steps) to the lanes that own the steps
#pragma unroll
          for (int gs = 0; gs < 4; ++gs) {
            const float4* row_r = reinterpret_cast<const float4*>(&s.P[(4 * c + gs) * kPRow + 8 * g]);
            const float4 lo = row_r[0], hi = row_r[1];
            q[8 * gs + 0] = lo.x; q[8 * gs + 1] = lo.y; q[8 * gs + 2] = lo.z; q[8 * gs + 3] = lo.w;
            q[8 * gs + 4] = hi.x; q[8 * gs + 5] = hi.y; q[8 * gs + 6] = hi.z; q[8 * gs + 7] = hi.w;
          }
        }
      };
      auto finish_last = [&](auto ptag) {   // outputs of the segment's last chunk
        constexpr int P = decltype(ptag)::kValue;
        if constexpr (kReadout) {
          float o[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float y = (q[j] + q[8 + j]) + (q[16 + j] + q[24 + j]);
            o[j] = __builtin_fmaf(k.dskip, uv[P][j], y) * gv[P][j];
          }
          if constexpr (kOutBF16) {
            if constexpr (P == 1) {   // an odd last chunk: the held even one goes first
              if (c_ok) store_w(held_at, held);
            }
            if (out_last) store_w(t_last, pack8(o));
          } else {
            if (out_last) store_out(t_last, o);
          }
        }
      };
      for (int64_t ck = 0;; ck += 2) {
        chunk(ModeTag<0>{}, ck);
        if (ck + 1 >= nck) { finish_last(ModeTag<0>{}); break; }
        chunk(ModeTag<1>{}, ck + 1);
        if (ck + 2 >= nck) { finish_last(ModeTag<1>{}); break; }
      }
    };
    if (mode == kZohFast) pipeline(ModeTag<kZohFast>{});
    else if (mode == kZohAccurate) pipeline(ModeTag<kZohAccurate>{});
    else pipeline(ModeTag<kDeltaB>{});

    if constexpr (!kReadout) dsum = quad_sum(dsum);
    __syncthreads();   // the next segment restages the LDS buffers
    return dsum;
  }
};

// ------------------------------------------------------------------ state hand-over between waves
// The slot (16 channels x 16 states) and its flag are written and read only
// with system-scope atomic accesses, which gfx950 performs with cache-bypass
// bits (write-through on store, miss on load), so they are coherent across
// the XCDs' separate L2 caches without any cache-wide writeback/invalidate.
// The producer waits for its slot stores to complete (vmcnt(0)) before it
// stores the flag; the consumer reads the slot only after it has seen the
// flag.  The slot holds this launch's epoch only once its data is in memory.
__device__ __forceinline__ void vmem_wait_all() {
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ void publish(const V2Params& q, int64_t slot, const float (&h)[kNS]) {
  const int lane = threadIdx.x & 63;
  const int c = lane >> 2, g = lane & 3;
  float* dst = q.pub_state + slot * kSlot;
#pragma unroll
  for (int i = 0; i < kNS; ++i)
    __hip_atomic_store(dst + c * 16 + 4 * g + i, h[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  vmem_wait_all();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(q.pub_flag + slot, q.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ bool receive(const V2Params& q, int64_t slot, float (&h)[kNS]) {
  const int lane = threadIdx.x & 63;
  const int c = lane >> 2, g = lane & 3;
  int ok = 0;
  if (lane == 0) {
    for (uint32_t it = 0; it < q.spin_limit; ++it) {
      if (__hip_atomic_load(q.pub_flag + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == q.epoch) { ok = 1; break; }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  ok = __builtin_amdgcn_readfirstlane(ok);   // the workgroup is this one wave
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (ok) {
    const float* src = q.pub_state + slot * kSlot;
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      h[i] = __hip_atomic_load(src + c * 16 + 4 * g + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  return ok != 0;
}

// The full pass of a scan is a set of "virtual tiles": one per (chunk of L,
// channel tile), chunk-major.  Every chunk but the last has nbf staging
// blocks of kCT steps, the last has nbl (a single chunk: nbf = nbl = L/kCT).
// The balanced split flattens (virtual tile, block) and gives every workgroup
// an equal range of it.
struct VtGeom {
  int64_t tiles, nbf, nbl, split;   // split: virtual tiles before the last chunk
};

__device__ __forceinline__ VtGeom vt_geom(const ScanParams& p, int64_t tiles) {
  VtGeom v;
  v.tiles = tiles;
  v.nbf = p.chunk_len / kCT;
  v.nbl = (p.L - (p.n_chunks - 1) * p.chunk_len + kCT - 1) / kCT;   // the last block may be short
  v.split = (p.n_chunks - 1) * tiles;
  return v;
}
__device__ __forceinline__ int64_t vt_pos(const VtGeom& v, int64_t vt) {
  return vt < v.split ? vt * v.nbf : v.split * v.nbf + (vt - v.split) * v.nbl;
}
__device__ __forceinline__ int64_t vt_len(const VtGeom& v, int64_t vt) { return vt < v.split ? v.nbf : v.nbl; }
__device__ __forceinline__ int64_t vt_at(const VtGeom& v, int64_t x) {   // virtual tile holding block x
  const int64_t xs = v.split * v.nbf;
  return x < xs ? x / v.nbf : v.split + (x - xs) / v.nbl;
}

struct Range {
  int64_t first, last, lo_off, hi_off, ft_begin;   // virtual tiles; offsets in blocks
  int has_head, has_tail, count;
};

__device__ __forceinline__ Range balanced_range(const VtGeom& v, const V2Params& q) {
  Range w;
  const int64_t gi = blockIdx.x;
  const int64_t U = v.split * v.nbf + v.tiles * v.nbl;
  const int64_t lo = gi * U / q.groups, hi = (gi + 1) * U / q.groups;
  w.first = vt_at(v, lo);
  w.last = vt_at(v, hi - 1);
  w.lo_off = lo - vt_pos(v, w.first);
  const int64_t hi_rel = hi - vt_pos(v, w.last);          // in [1, length of last]
  w.hi_off = hi_rel == vt_len(v, w.last) ? 0 : hi_rel;
  w.has_head = (w.hi_off != 0 && !(w.first == w.last && w.lo_off != 0)) ? 1 : 0;
  w.has_tail = (w.lo_off != 0) ? 1 : 0;
  w.ft_begin = (w.lo_off == 0) ? w.first : w.first + 1;
  const int64_t ft_end = (w.hi_off == 0) ? w.last + 1 : w.last;
  w.count = w.has_head + (int)(ft_end > w.ft_begin ? ft_end - w.ft_begin : 0) + w.has_tail;
  return w;
}

enum SegKind : int { kPlain = 0, kHead = 1, kWhole = 2, kTail = 3 };

// kRagged: L % kCT != 0 (full pass only; every summary chunk is whole).
template <bool kInBF16, bool kOutBF16, bool kSummary, bool kN16, bool kRagged>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void scan_v4_kernel(ScanParams p, V2Params q) {
  __shared__ WaveLds s;
  const int lane = threadIdx.x & 63;
  const int c = lane >> 2, g = lane & 3;
  const int64_t D = p.D, N = p.N, L = p.L;
  const int64_t tiles_d = (D + kTile - 1) / kTile;
  const int64_t tiles = p.B * tiles_d;
  using Full = Segment<kInBF16, kOutBF16, true, kN16, kRagged>;
  using StateOnly = Segment<kInBF16, kOutBF16, false, kN16>;

  Range w{};
  VtGeom v{};
  int nseg = 1;
  if (q.balanced) {
    v = vt_geom(p, tiles);
    w = balanced_range(v, q);
    nseg = w.count;
  }
  for (int si = 0; si < nseg; ++si) {
    // The segment [t_begin, t_end) lies in chunk `chunk`, which spans
    // [c_begin, c_end); a segment that starts at c_begin takes the chunk's
    // start state (zero for chunk 0), any other one the state handed over.
    int kind;
    int64_t tile, chunk, t_begin, t_end, c_begin, c_end;
    if (!q.balanced) {
      kind = kPlain;
      chunk = (int64_t)blockIdx.x / tiles;
      tile = (int64_t)blockIdx.x - chunk * tiles;
      c_begin = chunk * p.chunk_len;
      c_end = (c_begin + p.chunk_len < L) ? c_begin + p.chunk_len : L;
      t_begin = c_begin;
      t_end = c_end;
    } else {
      int64_t vt, b_lo, b_hi;
      if (w.has_head && si == 0) {
        kind = kHead; vt = w.last; b_lo = 0; b_hi = w.hi_off;
      } else if (w.has_tail && si == nseg - 1) {
        kind = kTail; vt = w.first; b_lo = w.lo_off;
        b_hi = (w.first == w.last && w.hi_off != 0) ? w.hi_off : vt_len(v, vt);
      } else {
        kind = kWhole; vt = w.ft_begin + (si - w.has_head); b_lo = 0; b_hi = vt_len(v, vt);
      }
      chunk = vt / tiles;
      tile = vt - chunk * tiles;
      c_begin = chunk * p.chunk_len;
      c_end = c_begin + vt_len(v, vt) * kCT;
      c_end = c_end < L ? c_end : L;
      t_begin = c_begin + b_lo * kCT;
      t_end = c_begin + b_hi * kCT;
      t_end = t_end < L ? t_end : L;
    }
    const int64_t b = tile / tiles_d;
    const int64_t d0 = (tile - b * tiles_d) * kTile;
    const int64_t d = d0 + c;
    const bool d_ok = d < D;
    const Consts k = load_consts(p, d, d_ok, g);
    const int mode = p.delta_b ? kDeltaB : (k.accurate ? kZohAccurate : kZohFast);

    float h[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
      h[i] = 0.0f;
      if (!kSummary && p.h_start != nullptr && chunk > 0 && d_ok && 4 * g + i < N)
        h[i] = p.h_start[((chunk * p.B + b) * D + d) * N + 4 * g + i];
    }
    if (!kSummary && kind == kTail) {
      if (!receive(q, (int64_t)blockIdx.x - 1, h)) {
        // recompute the state at t_begin from the chunk's start state
#pragma unroll
        for (int i = 0; i < kNS; ++i)
          if (p.h_start == nullptr || chunk == 0) h[i] = 0.0f;
        StateOnly::run(p, s, b, d0, c_begin, t_begin, h, k, mode);
      }
    }
    if constexpr (kSummary) {
      const float ds = StateOnly::run(p, s, b, d0, t_begin, t_end, h, k, mode);
#pragma unroll
      for (int i = 0; i < kNS; ++i)
        if (d_ok && 4 * g + i < N) p.h_local[((chunk * p.B + b) * D + d) * N + 4 * g + i] = h[i];
      if (g == 0 && d_ok) p.s_sum[(chunk * p.B + b) * D + d] = ds;
    } else {
      Full::run(p, s, b, d0, t_begin, t_end, h, k, mode);
      if (kind == kHead || (kind == kTail && t_end != c_end)) {
        publish(q, (int64_t)blockIdx.x, h);
      } else if (t_end == L && p.final_state != nullptr && d_ok) {
#pragma unroll
        for (int i = 0; i < kNS; ++i)
          if (4 * g + i < N) p.final_state[(b * D + d) * N + 4 * g + i] = h[i];
      }
    }
  }
}

template <bool kInBF16, bool kOutBF16, bool kSummary>
hipError_t launch_t(const ScanParams& p, const V2Params& q, hipStream_t st) {
  constexpr bool kR = !kSummary;   // a ragged instance for the full pass only
  const bool ragged = kR && p.L % kCT != 0;
  auto kern = p.N == 16 ? (ragged ? scan_v4_kernel<kInBF16, kOutBF16, kSummary, true, kR>
                                  : scan_v4_kernel<kInBF16, kOutBF16, kSummary, true, false>)
                        : (ragged ? scan_v4_kernel<kInBF16, kOutBF16, kSummary, false, kR>
                                  : scan_v4_kernel<kInBF16, kOutBF16, kSummary, false, false>);
  const int64_t tiles = p.B * ((p.D + kTile - 1) / kTile);
  int64_t grid;
  if (q.balanced) grid = q.groups;
  else grid = (kSummary ? p.n_chunks - 1 : p.n_chunks) * tiles;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64), 0, st, p, q);
  return hipGetLastError();
}

}  // namespace

// Launches of one input dtype (defined in scan_v4_bf16.hip / scan_v4_f32.hip).
hipError_t launch_scan_v4_bf16in(const ScanParams& p, const V2Params& q, Dt out, bool summary, hipStream_t s);
hipError_t launch_scan_v4_f32in(const ScanParams& p, const V2Params& q, Dt out, bool summary, hipStream_t s);

}  // namespace mamba

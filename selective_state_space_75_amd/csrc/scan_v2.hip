// scan_v2.hip -- the main selective-scan kernel for gfx950 (sequence lengths
// that are multiples of 32, 16-byte aligned rows).
//
// Same computation as scan_fwd.hip ("Mamba 模型" flowchart nodes H to M; ZOH
// per "Mamba模型：高效序列建模的新突破" 3.1), organised for throughput:
//
//  * Workgroup = 8 waves = one tile of 64 channels of one batch row; lane =
//    channel, wave w owns states 2w and 2w+1 in VGPRs.  One workgroup per
//    compute unit (LDS ~92 KB), two waves per SIMD.
//  * B_t and C_t are the same for every channel of a batch row, so within a
//    wave they are uniform: they are read with scalar loads into SGPRs (16
//    steps at a time, the next block requested while the current one is
//    used) and widened on the scalar unit, costing no VALU or LDS bandwidth.
//  * u, delta and z are read with coalesced loads, one 32-step chunk ahead of
//    use; delta = softplus(delta_raw + bias) is evaluated once per element
//    and both delta and u are staged channel-major in LDS, where every wave
//    reads its channel's 16 steps with 16-byte reads.
//  * Each wave writes its partial readout sum_n C_n h_n per (channel, step)
//    to LDS; after a barrier the workgroup adds the 8 partials, the skip term
//    and the gate, and stores y.
//  * Balanced split: when there are at least as many tiles as workgroups, the
//    (tile x 32-step block) work is cut into equal contiguous ranges, one per
//    workgroup.  A tile cut between workgroups g and g+1 is scanned by g from
//    t = 0 to the cut (done first, its end state published with an epoch
//    flag) and by g+1 from the cut to the end (done last, after reading the
//    published state).  The wait is bounded; if it runs out, g+1 recomputes
//    the state itself, so the kernel always finishes.
// Per ZOH state update the inner loop issues 6 fp32 VALU operations and one
// v_exp_f32 (delta*A, exp, (e-1)/A, B*u, *coefficient, fma into h, fma into y).
#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

constexpr int kW = 8;                 // waves per workgroup
constexpr int kNS = 2;                // states per wave (kW * kNS = 16)
constexpr int kThreads = 64 * kW;
constexpr int kTile = 64;             // channels per tile
constexpr int kCT = 32;               // steps per staged chunk
constexpr int kRS = 36;               // LDS row stride in floats (16-byte aligned rows)
constexpr int kStagePer = kCT * kTile / kThreads;   // steps per staging thread (4)
static_assert(kW * kNS == 16, "16 states per tile");
static_assert(kStagePer == 4, "staging thread handles 4 steps");

typedef __attribute__((address_space(4))) const uint32_t* sptr_u32;

template <bool kBF16> struct Raw;
template <> struct Raw<true> { uint2 u, d, z; };
template <> struct Raw<false> { float4 u, d, z; };

template <bool kBF16>
__device__ __forceinline__ void unpack4(const Raw<kBF16>& r, int which, float v[4]) {
  if constexpr (kBF16) {
    const uint2 w = which == 0 ? r.u : which == 1 ? r.d : r.z;
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  } else {
    const float4 w = which == 0 ? r.u : which == 1 ? r.d : r.z;
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
}

template <bool kBF16>
__device__ __forceinline__ void load_raw(const ScanParams& p, int64_t row_off, int64_t t, bool ok, bool want_z,
                                         Raw<kBF16>& r) {
  if constexpr (kBF16) {
    if (ok) {
      const uint16_t* u = static_cast<const uint16_t*>(p.u) + row_off + t;
      const uint16_t* d = static_cast<const uint16_t*>(p.delta) + row_off + t;
      r.u = *reinterpret_cast<const uint2*>(u);
      r.d = *reinterpret_cast<const uint2*>(d);
      if (want_z) r.z = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.z) + row_off + t);
      else r.z = make_uint2(0, 0);
    } else {
      r.u = r.d = r.z = make_uint2(0, 0);
    }
  } else {
    if (ok) {
      r.u = *reinterpret_cast<const float4*>(static_cast<const float*>(p.u) + row_off + t);
      r.d = *reinterpret_cast<const float4*>(static_cast<const float*>(p.delta) + row_off + t);
      if (want_z) r.z = *reinterpret_cast<const float4*>(static_cast<const float*>(p.z) + row_off + t);
      else r.z = make_float4(0, 0, 0, 0);
    } else {
      r.u = r.d = r.z = make_float4(0, 0, 0, 0);
    }
  }
}

// B_t / C_t words of one wave for a block of steps: 4 words per state and
// array, i.e. 8 steps of bf16 (two per word) or 4 steps of fp32.
constexpr int kWords = 4;
struct BCWords { uint32_t b[kNS][kWords]; uint32_t c[kNS][kWords]; };

template <bool kBF16, bool kReadout>
__device__ __forceinline__ void load_bc(const ScanParams& p, int64_t b, int n0, int64_t t, BCWords& w) {
  const int64_t N = p.N, L = p.L;
#pragma unroll
  for (int i = 0; i < kNS; ++i) {
    // Branch-free: a state beyond N reads row 0 and is masked to zero.
    const int n = n0 + i;
    const uint32_t keep = (n < N) ? 0xffffffffu : 0u;
    const int64_t off = (b * N + ((n < N) ? n : 0)) * L + t;
    sptr_u32 pb = kBF16 ? (sptr_u32)(static_cast<const uint16_t*>(p.Bt) + off)
                        : (sptr_u32)(static_cast<const float*>(p.Bt) + off);
#pragma unroll
    for (int k = 0; k < kWords; ++k) w.b[i][k] = pb[k] & keep;
    if constexpr (kReadout) {
      sptr_u32 pc = kBF16 ? (sptr_u32)(static_cast<const uint16_t*>(p.Ct) + off)
                          : (sptr_u32)(static_cast<const float*>(p.Ct) + off);
#pragma unroll
      for (int k = 0; k < kWords; ++k) w.c[i][k] = pc[k] & keep;
    }
  }
}

template <bool kBF16>
__device__ __forceinline__ float bc_at(const uint32_t (&w)[kWords], int j) {
  if constexpr (kBF16) return (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
  else return __builtin_bit_cast(float, w[j]);
}

struct Shared {
  float dl[kTile * kRS];
  float u[kTile * kRS];
  float y[kW * kTile * kRS];
  float sum[kW];
  int flag;
};

// Per-state constants of the lane's channel for this wave's two states.
struct StateConst {
  float a2[kNS];   // A * log2(e)
  float ia[kNS];   // 1 / A
  int accurate;    // wave-uniform: use the cancellation-free (e - 1)
};

__device__ __forceinline__ void load_consts(const ScanParams& p, int64_t d, bool d_ok, int n0, StateConst& sc) {
  bool tiny = false;
#pragma unroll
  for (int i = 0; i < kNS; ++i) {
    const int n = n0 + i;
    float a = (d_ok && n < p.N) ? p.A[d * p.N + n] : -1.0f;
    // |A| < 2^-40 (including 0) is replaced by -2^-40 (sign kept): the ZOH
    // coefficient then equals delta to within delta * 2^-41 (resolved by the
    // accurate loop) and 1/A stays finite.
    if (__builtin_fabsf(a) < 0x1p-40f) { tiny = true; a = (a > 0.0f) ? 0x1p-40f : -0x1p-40f; }
    sc.a2[i] = a * kLog2e;
    sc.ia[i] = 1.0f / a;
  }
  sc.accurate = (p.accurate || __any(tiny)) ? 1 : 0;
}

// One 8-step (bf16) or 4-step (fp32) block of the recurrence for the lane's
// channel and the wave's two states.  dl/uu: delta and u of the block.
template <int kMode, bool kReadout, int kSteps, bool kBF16>
__device__ __forceinline__ void run_block(const float* dl, const float* uu, const BCWords& w, float (&h)[kNS],
                                          const StateConst& sc, float* acc) {
#pragma unroll
  for (int j = 0; j < kSteps; ++j) {
    float y = 0.0f;
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
      const float bn = bc_at<kBF16>(w.b[i], j);
      const float x = dl[j] * sc.a2[i];
      const float e = hw_exp2(x);
      float inp;
      if constexpr (kMode == kDeltaB) {
        inp = (dl[j] * uu[j]) * bn;
      } else {
        const float k = (kMode == kZohFast) ? __builtin_fmaf(e, sc.ia[i], -sc.ia[i])
                                            : expm1_from_exp2(x, e) * sc.ia[i];
        inp = k * (bn * uu[j]);
      }
      h[i] = __builtin_fmaf(e, h[i], inp);
      if constexpr (kReadout) y = (i == 0) ? bc_at<kBF16>(w.c[i], j) * h[i] : __builtin_fmaf(bc_at<kBF16>(w.c[i], j), h[i], y);
    }
    if constexpr (kReadout) acc[j] = y;
  }
}

__device__ __forceinline__ void lgkm_wait_all() {
  // s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maximum)
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

template <bool kBF16In, bool kBF16Out, bool kReadout>
struct Seg {
  // Scan steps [t_begin, t_end) of tile (b, d0) from state h (updated in place).
  // kReadout: compute and store y.  Otherwise only the state (and the sum of
  // delta, returned) is computed.  Must be called by the whole workgroup.
  static __device__ __forceinline__ float run(const ScanParams& p, Shared& sh, int64_t b, int64_t d0, int64_t t_begin,
                              int64_t t_end, float (&h)[kNS], const StateConst& sc, int mode) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
    const int n0 = wave * kNS;
    const int64_t D = p.D, L = p.L;
    // staging role
    const int c = tid >> 3, pc = tid & 7;
    const int64_t dc = d0 + c;
    const bool c_ok = dc < D;
    const int64_t row_off = (b * D + (c_ok ? dc : 0)) * L;
    const float bias_c = (c_ok && p.bias) ? p.bias[dc] : 0.0f;
    const float dskip_c = (c_ok && p.Dskip) ? p.Dskip[dc] : 0.0f;
    const bool want_z = kReadout && (p.z != nullptr);
    float dsum = 0.0f;

    const int64_t nck = (t_end - t_begin) / kCT;
    Raw<kBF16In> cur, nxt;
    load_raw<kBF16In>(p, row_off, t_begin + kStagePer * pc, c_ok, want_z, cur);

    auto stage = [&](const Raw<kBF16In>& r) {
      float dr[4], uv[4];
      unpack4<kBF16In>(r, 1, dr);
      unpack4<kBF16In>(r, 0, uv);
      float4 dv;
      dv.x = c_ok ? softplus(dr[0] + bias_c) : 0.0f;
      dv.y = c_ok ? softplus(dr[1] + bias_c) : 0.0f;
      dv.z = c_ok ? softplus(dr[2] + bias_c) : 0.0f;
      dv.w = c_ok ? softplus(dr[3] + bias_c) : 0.0f;
      if constexpr (!kReadout) dsum += (dv.x + dv.y) + (dv.z + dv.w);
      *reinterpret_cast<float4*>(&sh.dl[c * kRS + kStagePer * pc]) = dv;
      *reinterpret_cast<float4*>(&sh.u[c * kRS + kStagePer * pc]) = make_float4(uv[0], uv[1], uv[2], uv[3]);
    };
    stage(cur);
    __syncthreads();

    constexpr int kBlk = kBF16In ? 2 * kWords : kWords;   // steps per B/C register block
    constexpr int kNB = kCT / kBlk;
    for (int64_t k = 0; k < nck; ++k) {
      const int64_t t0 = t_begin + k * kCT;
      if (k + 1 < nck) load_raw<kBF16In>(p, row_off, t0 + kCT + kStagePer * pc, c_ok, want_z, nxt);
      // ---- recurrence over the chunk, kBlk steps at a time.  The scalar
      // loads of B/C and the LDS reads of delta/u for block s+1 are issued
      // before block s is computed, and waited for at the start of block
      // s+1 (scalar and LDS accesses share one counter, so they are issued
      // together and waited for together).
      {
        const float* dl_row = &sh.dl[lane * kRS];
        const float* u_row = &sh.u[lane * kRS];
        float* y_row = &sh.y[(wave * kTile + lane) * kRS];
        BCWords wc, wn;
        float dlc[kBlk], uuc[kBlk], dln[kBlk], uun[kBlk];
        auto read_lds = [&](int s, float (&dl)[kBlk], float (&uu)[kBlk]) {
#pragma unroll
          for (int q4 = 0; q4 < kBlk / 4; ++q4) {
            const float4 a = *reinterpret_cast<const float4*>(dl_row + s * kBlk + 4 * q4);
            const float4 v = *reinterpret_cast<const float4*>(u_row + s * kBlk + 4 * q4);
            dl[4 * q4] = a.x; dl[4 * q4 + 1] = a.y; dl[4 * q4 + 2] = a.z; dl[4 * q4 + 3] = a.w;
            uu[4 * q4] = v.x; uu[4 * q4 + 1] = v.y; uu[4 * q4 + 2] = v.z; uu[4 * q4 + 3] = v.w;
          }
        };
        load_bc<kBF16In, kReadout>(p, b, n0, t0, wc);
        read_lds(0, dlc, uuc);
#pragma unroll
        for (int s = 0; s < kNB; ++s) {
          lgkm_wait_all();
          __builtin_amdgcn_sched_barrier(0);
          if (s + 1 < kNB) {
            load_bc<kBF16In, kReadout>(p, b, n0, t0 + (s + 1) * kBlk, wn);
            read_lds(s + 1, dln, uun);
          }
          __builtin_amdgcn_sched_barrier(0);
          float acc[kBlk];
          if (mode == kZohFast) run_block<kZohFast, kReadout, kBlk, kBF16In>(dlc, uuc, wc, h, sc, acc);
          else if (mode == kZohAccurate) run_block<kZohAccurate, kReadout, kBlk, kBF16In>(dlc, uuc, wc, h, sc, acc);
          else run_block<kDeltaB, kReadout, kBlk, kBF16In>(dlc, uuc, wc, h, sc, acc);
          if constexpr (kReadout) {
#pragma unroll
            for (int q4 = 0; q4 < kBlk / 4; ++q4)
              *reinterpret_cast<float4*>(y_row + s * kBlk + 4 * q4) =
                  make_float4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
          }
          if (s + 1 < kNB) {
            wc = wn;
#pragma unroll
            for (int j = 0; j < kBlk; ++j) { dlc[j] = dln[j]; uuc[j] = uun[j]; }
          }
        }
      }
      __syncthreads();
      // ---- readout of the chunk: 8 partials + D u, gate, store
      if constexpr (kReadout) {
        float4 acc = *reinterpret_cast<const float4*>(&sh.y[(0 * kTile + c) * kRS + kStagePer * pc]);
#pragma unroll
        for (int w = 1; w < kW; ++w) {
          const float4 v = *reinterpret_cast<const float4*>(&sh.y[(w * kTile + c) * kRS + kStagePer * pc]);
          acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        float uv[4], zv[4], o[4];
        unpack4<kBF16In>(cur, 0, uv);
        unpack4<kBF16In>(cur, 2, zv);
        o[0] = __builtin_fmaf(dskip_c, uv[0], acc.x);
        o[1] = __builtin_fmaf(dskip_c, uv[1], acc.y);
        o[2] = __builtin_fmaf(dskip_c, uv[2], acc.z);
        o[3] = __builtin_fmaf(dskip_c, uv[3], acc.w);
        if (want_z) {
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] *= silu(zv[j]);
        }
        if (c_ok) {
          const int64_t at = row_off + t0 + kStagePer * pc;
          if constexpr (kBF16Out) {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + at) =
                make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(p.y) + at) = make_float4(o[0], o[1], o[2], o[3]);
          }
        }
      }
      if (k + 1 < nck) {
        stage(nxt);
        cur = nxt;
      }
      __syncthreads();
    }
    // sum of delta over the segment for the staging channel (summary use)
    if constexpr (!kReadout) {
      dsum += __shfl_xor(dsum, 1, 8);
      dsum += __shfl_xor(dsum, 2, 8);
      dsum += __shfl_xor(dsum, 4, 8);
    }
    return dsum;
  }
};

// ------------------------------------------------------------------ state hand-over between workgroups
__device__ __forceinline__ void publish(const ScanParams& p, const V2Params& q, Shared& sh, int64_t slot,
                                        const float (&h)[kNS]) {
  const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  float* dst = q.pub_state + slot * (kTile * 16);
#pragma unroll
  for (int i = 0; i < kNS; ++i)
    __hip_atomic_store(dst + lane * 16 + wave * kNS + i, h[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __threadfence();
  __syncthreads();
  if (tid == 0) __hip_atomic_store(q.pub_flag + slot, q.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Returns true and fills h when the state of `slot` was published in time.
__device__ __forceinline__ bool receive(const V2Params& q, Shared& sh, int64_t slot, float (&h)[kNS]) {
  const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  if (tid == 0) {
    int ok = 0;
    for (uint32_t it = 0; it < q.spin_limit; ++it) {
      if (__hip_atomic_load(q.pub_flag + slot, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == q.epoch) { ok = 1; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    sh.flag = ok;
  }
  __syncthreads();
  const bool ok = sh.flag != 0;
  __syncthreads();
  if (ok) {
    __threadfence();
    const float* src = q.pub_state + slot * (kTile * 16);
#pragma unroll
    for (int i = 0; i < kNS; ++i)
      h[i] = __hip_atomic_load(src + lane * 16 + wave * kNS + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return ok;
}

// Work of one workgroup as a short list of segments, each a step range of
// one tile.  Plain mode: one (chunk, tile) item.  Balanced mode: a contiguous
// range [lo, hi) of (tile, 32-step block) units, done in the order
//   head of the last tile (ends mid-tile; published for the next group),
//   whole tiles,
//   tail of the first tile (starts mid-tile; state from the previous group).
struct Plan2 {
  int64_t lo, hi, nb, first, last, lo_off, hi_off, ft_begin, ft_end;
  int has_head, has_tail, count;
};

__device__ __forceinline__ Plan2 plan_balanced(const ScanParams& p, const V2Params& q) {
  Plan2 w;
  const int64_t g = blockIdx.x;
  w.nb = p.L / kCT;
  const int64_t U = p.B * p.tiles_d * w.nb;
  w.lo = g * U / q.groups;
  w.hi = (g + 1) * U / q.groups;
  w.first = w.lo / w.nb;
  w.last = (w.hi - 1) / w.nb;
  w.lo_off = w.lo % w.nb;
  w.hi_off = w.hi % w.nb;
  w.has_head = (w.hi_off != 0 && !(w.first == w.last && w.lo_off != 0)) ? 1 : 0;
  w.has_tail = (w.lo_off != 0) ? 1 : 0;
  w.ft_begin = (w.lo_off == 0) ? w.first : w.first + 1;
  w.ft_end = (w.hi_off == 0) ? w.last + 1 : w.last;
  const int64_t nfull = w.ft_end > w.ft_begin ? w.ft_end - w.ft_begin : 0;
  w.count = w.has_head + (int)nfull + w.has_tail;
  return w;
}

enum SegKind : int { kPlain = 0, kHead = 1, kWhole = 2, kTail = 3 };

template <bool kBF16In, bool kBF16Out, bool kSummary>
__global__ __launch_bounds__(kThreads) void scan_v2_kernel(ScanParams p, V2Params q) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int n0 = wave * kNS;
  const int64_t D = p.D, N = p.N, L = p.L;
  using Full = Seg<kBF16In, kBF16Out, true>;
  using StateOnly = Seg<kBF16In, kBF16Out, false>;

  Plan2 w{};
  int nseg = 1;
  if (q.balanced) {
    w = plan_balanced(p, q);
    nseg = w.count;
  }
  const int64_t per_chunk = p.B * p.tiles_d;
  for (int si = 0; si < nseg; ++si) {
    // ---- decode the segment (workgroup-uniform)
    int kind;
    int64_t tile, chunk = 0, t_begin, t_end;
    if (!q.balanced) {
      kind = kPlain;
      chunk = (int64_t)blockIdx.x / per_chunk;
      tile = (int64_t)blockIdx.x - chunk * per_chunk;
      t_begin = chunk * p.chunk_len;
      t_end = (t_begin + p.chunk_len < L) ? t_begin + p.chunk_len : L;
    } else if (w.has_head && si == 0) {
      kind = kHead; tile = w.last; t_begin = 0; t_end = w.hi_off * kCT;
    } else if (w.has_tail && si == nseg - 1) {
      kind = kTail; tile = w.first; t_begin = w.lo_off * kCT;
      t_end = (w.first == w.last && w.hi_off != 0) ? w.hi_off * kCT : L;
    } else {
      kind = kWhole; tile = w.ft_begin + (si - w.has_head); t_begin = 0; t_end = L;
    }
    const int64_t b = tile / p.tiles_d;
    const int64_t d0 = (tile - b * p.tiles_d) * kTile;
    const int64_t d = d0 + lane;
    const bool d_ok = d < D;
    StateConst sc;
    load_consts(p, d, d_ok, n0, sc);
    const int mode = p.delta_b ? kDeltaB : (sc.accurate ? kZohAccurate : kZohFast);

    // ---- starting state
    float h[kNS];
#pragma unroll
    for (int i = 0; i < kNS; ++i) {
      h[i] = 0.0f;
      if (!kSummary && kind == kPlain && p.h_start != nullptr && chunk > 0 && d_ok && n0 + i < N)
        h[i] = p.h_start[((chunk * p.B + b) * D + d) * N + n0 + i];
    }
    if (!kSummary && kind == kTail) {
      if (!receive(q, sh, (int64_t)blockIdx.x - 1, h)) {
        // not published in time: recompute the state at the cut
#pragma unroll
        for (int i = 0; i < kNS; ++i) h[i] = 0.0f;
        StateOnly::run(p, sh, b, d0, 0, t_begin, h, sc, mode);
      }
    }

    // ---- the scan of the segment
    if constexpr (kSummary) {
      const float ds = StateOnly::run(p, sh, b, d0, t_begin, t_end, h, sc, mode);
#pragma unroll
      for (int i = 0; i < kNS; ++i)
        if (d_ok && n0 + i < N) p.h_local[((chunk * p.B + b) * D + d) * N + n0 + i] = h[i];
      const int c = tid >> 3;
      if ((tid & 7) == 0 && d0 + c < D) p.s_sum[(chunk * p.B + b) * D + d0 + c] = ds;
    } else {
      Full::run(p, sh, b, d0, t_begin, t_end, h, sc, mode);
      // ---- what follows the segment
      if (kind == kHead || (kind == kTail && t_end != L)) {
        publish(p, q, sh, (int64_t)blockIdx.x, h);
      } else if (t_end == L && p.final_state != nullptr && d_ok) {
#pragma unroll
        for (int i = 0; i < kNS; ++i)
          if (n0 + i < N) p.final_state[(b * D + d) * N + n0 + i] = h[i];
      }
    }
  }
}

template <bool kBF16In, bool kBF16Out, bool kSummary>
hipError_t launch_t(const ScanParams& p, const V2Params& q, hipStream_t s) {
  int64_t grid;
  if (q.balanced) grid = q.groups;
  else grid = (kSummary ? p.n_chunks - 1 : p.n_chunks) * p.B * p.tiles_d;
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((scan_v2_kernel<kBF16In, kBF16Out, kSummary>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                     p, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_v2(const ScanParams& p, const V2Params& q, Dt in, Dt out, bool summary, hipStream_t s) {
  if (summary) return in == Dt::BF16 ? launch_t<true, false, true>(p, q, s) : launch_t<false, false, true>(p, q, s);
  if (in == Dt::BF16)
    return out == Dt::BF16 ? launch_t<true, true, false>(p, q, s) : launch_t<true, false, false>(p, q, s);
  return out == Dt::BF16 ? launch_t<false, true, false>(p, q, s) : launch_t<false, false, false>(p, q, s);
}

}  // namespace mamba

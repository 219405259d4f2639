// ssd.hip -- Mamba-2 layer (state space duality) forward for gfx950, with the
// products inside each chunk on the matrix cores.
//
// What it computes ("Mamba 与状态空间模型" section 09; "Mamba 状态空间模型架构深度解析",
// Mamba-2): A is a scalar times the identity, one A_h and one step size per
// head of P channels.  With delta_t = softplus(delta_raw_t + bias_h),
// coef_t = (exp(delta_t A_h) - 1) / A_h (or delta_t under the simplified rule)
// and cum_t = A_h sum_(r <= t) delta_r, each channel's output is
//   y_t = sum_(s <= t) (C_t . B_s) exp(cum_t - cum_s) coef_s x_s + D x_t,
// times silu(z_t) when z is given: the lower-triangular matrix of section 09,
// C like a query, B like a key, x like the values, no softmax.
//
// Chunked as section 09 describes (matrix products inside a chunk, only the
// state passed between chunks).  For a chunk of Q = 32 steps from t0, with the
// entering state H (N x P) and cum counted from t0:
//   S = C B^T (Q x Q);  G = S o exp(cum_t - cum_s) coef_s [s <= t]
//   y = G x + exp(cum_t) (C H) + D x
//   H <- exp(cum_last) H + B^T (w o x),  w_s = exp(cum_last - cum_s) coef_s
// Every product is v_mfma_f32_16x16x32_bf16.  x, B and C are bf16 inputs and
// exact operands; the fp32 intermediates G, w o x and H are each split into a
// bf16 high part and a bf16 remainder that are multiplied separately, which
// keeps about 16 significant bits per operand; all sums are fp32.
//
// One workgroup (4 waves) per (batch row, segment of L, head, 64-channel
// block).  Wave w owns channels 16 w .. 16 w + 15 of the block and their whole
// N x 16 state, held in MFMA accumulators across chunks; the accumulator
// layout is exactly the B operand layout of the C H product, so the state
// never goes through LDS.
//
// L is cut into segments so that there are enough workgroups to hide latency
// (a head alone is a chain of dependent chunks).  A first launch computes the
// end state of every segment but the last from a zero state at its start (one
// weighted product over the segment's steps) and the segment's total decay;
// the full launch then runs every segment from its entering state, which it
// chains from those of the segments before it (the associative combination
// of "Mamba论文研读笔记" 3.2.3 B over segment aggregates).
#include "device_math.hpp"
#include "kernels.hpp"

namespace mamba {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQ = 32;     // steps per chunk
constexpr int kP = 64;     // channels per workgroup
constexpr int kPad = 8;    // bf16 of padding per LDS row (16 bytes): conflict-free operand reads

template <int kN>
struct SsdLds {
  uint16_t Cc[kQ][kN + kPad];     // C_t   [step][state]
  uint16_t Bc[kQ][kN + kPad];     // B_t   [step][state]
  uint16_t BcT[kN][kQ + kPad];    // B_t   [state][step]
  uint16_t X[kP][kQ + kPad];      // x     [channel][step]
  uint16_t Xh[kP][kQ + kPad];     // w o x [channel][step], high part
  uint16_t Xl[kP][kQ + kPad];     //                        remainder
  uint16_t Gh[kQ][kQ + kPad];     // G     [t][s], high part
  uint16_t Gl[kQ][kQ + kPad];     //               remainder
  // per step of a chunk, double-buffered by chunk parity (the next chunk's
  // values are computed while the current one runs)
  float cum[2][kQ];               // A sum_(t0 <= r <= t) delta_r
  float coef[2][kQ];
  float ecum[2][kQ];              // exp(cum_t)
  float wl[2][kQ];                // exp(cum_last - cum_s) coef_s
  float elast[2];                 // exp(cum_last)
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 consecutive bf16 from LDS (16-byte aligned)
__device__ __forceinline__ bf16x8 lds8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
// 4 + 4 bf16 from two 8-byte aligned LDS addresses
__device__ __forceinline__ bf16x8 lds4x2(const uint16_t* p, const uint16_t* q) {
  const uint2 a = *reinterpret_cast<const uint2*>(p), b = *reinterpret_cast<const uint2*>(q);
  return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}

// fp32 -> bf16 high part and bf16 remainder (both round-to-nearest-even)
__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(v);
  lo = f32_to_bf16(v - bf16_to_f32(hi));
}

// Four consecutive bf16 of a row: one 8-byte load when `vec`, else element
// loads with zeros from index `valid` on.
__device__ __forceinline__ uint2 ld_row4(const uint16_t* row, int64_t t, bool vec, int64_t valid) {
  if (vec) return *reinterpret_cast<const uint2*>(row + t);
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = (j < valid) ? (uint32_t)row[t + j] : 0u;
  return make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
}

// Work item of workgroup `id` out of `n`, so that each of the 8 XCDs (which
// take workgroups round-robin: id % 8) gets a contiguous range of work items:
// the heads of one (batch row, segment) then share that XCD's L2, and its
// copy of B_t/C_t (1 MB per batch row at N = 128) is read from HBM once
// rather than by every XCD.  The tail past the last multiple of 8 keeps its
// index.
__device__ __forceinline__ int64_t xcd_item(int64_t id, int64_t n) {
  const int64_t per = n / 8;
  if (id >= 8 * per) return id;
  return (id % 8) * per + id / 8;
}

template <int kN, bool kOutBF16, bool kDeltaB>
__global__ __launch_bounds__(256, 3) void ssd_chunk_kernel(SsdParams p) {
  __shared__ SsdLds<kN> S;
  constexpr int kNT = kN / 16;     // 16-row tiles of the state
  constexpr int kNK = kN / 32;     // 32-wide K blocks over the states
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int g = l >> 4, r = l & 15;
  const int64_t pblocks = p.P / kP;
  const int64_t wg = xcd_item(blockIdx.x, gridDim.x);      // ((b S + seg) H + h) pblocks + pb
  const int64_t pb = wg % pblocks;
  const int64_t h = (wg / pblocks) % p.H;
  const int64_t bs = wg / (pblocks * p.H);
  const int64_t seg = bs % p.S, b = bs / p.S;
  const int64_t d0 = h * p.P + pb * kP;                      // first channel of the block
  const int64_t t_begin = seg * p.seg_len;
  const int64_t t_end = t_begin + p.seg_len < p.L ? t_begin + p.seg_len : p.L;
  const int64_t L = p.L, D = p.H * p.P, N = p.N;
  const float a = p.A[h];
  const float a2 = a * kLog2e;
  const float ia = 1.0f / a;
  const float bias = p.bias ? p.bias[h] : 0.0f;
  const bool vecp = p.vec != 0;

  // staging roles: (nq, tb4) = 4 states x 4 steps of B_t / C_t; (px, tb8) = 8 steps of one channel of x
  const int nq = tid >> 3, tb4 = tid & 7;
  const int px = tid >> 2, tb8 = tid & 3;
  // output role: channel 16 w + r, steps 16 tm + 4 g .. + 3 (tm = 0, 1)
  const int pc = 16 * w + r;
  const float Dp = p.Dskip ? p.Dskip[d0 + pc] : 0.0f;
  const uint16_t* xrow = static_cast<const uint16_t*>(p.x) + (b * D + d0 + px) * L;
  const uint16_t* zrow = p.z ? static_cast<const uint16_t*>(p.z) + (b * D + d0 + pc) * L : nullptr;
  const uint16_t* dtrow = static_cast<const uint16_t*>(p.delta) + (b * p.H + h) * L;
  const uint16_t* Brow = static_cast<const uint16_t*>(p.Bt) + b * N * L;
  const uint16_t* Crow = static_cast<const uint16_t*>(p.Ct) + b * N * L;

  // the upper off-diagonal 16 x 16 block of G is zero in every chunk
  for (int i = tid; i < 16 * 16; i += 256) {
    S.Gh[i >> 4][16 + (i & 15)] = 0;
    S.Gl[i >> 4][16 + (i & 15)] = 0;
  }

  struct Raw {
    uint2 c[4], bb[4];   // states 4 nq + j, steps 4 tb4 .. + 3
    uint4 x;             // channel px, steps 8 tb8 .. + 7
    uint2 z[2];          // channel pc, steps 16 tm + 4 g .. + 3
    uint32_t dt;         // step l of the chunk after this one (wave 3, lanes < 32)
  };
  // A chunk that lies wholly inside the rows (and rows that allow 8- and
  // 16-byte loads) is fetched without per-load conditions, as buffer loads:
  // a descriptor per array (the batch row's B_t / C_t, the block's x / z
  // rows), this lane's fixed 32-bit byte offset, and a uniform offset per
  // row and chunk.  Byte ranges must fit 32 bits: L < 2^24.
  const bool off32 = L < (int64_t(1) << 24);
  constexpr int kRawWord3 = 0x00020000;   // 32-bit data format, as raw buffer loads need
  const uint32_t voff_bc = (uint32_t)((4 * nq) * L + 4 * tb4) * 2u;
  const uint32_t voff_x = (uint32_t)(px * L + 8 * tb8) * 2u;
  const uint32_t voff_z = (uint32_t)(pc * L + 4 * g) * 2u;
  const int bc_bytes = (int)(uint32_t)(off32 ? N * L * 2 : 0);
  const int blk_bytes = (int)(uint32_t)(off32 ? kP * L * 2 : 0);
  const __amdgpu_buffer_rsrc_t rsC = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Crow), 0, bc_bytes, kRawWord3);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Brow), 0, bc_bytes, kRawWord3);
  const __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(static_cast<const uint16_t*>(p.x) + (b * D + d0) * L), 0, blk_bytes, kRawWord3);
  const __amdgpu_buffer_rsrc_t rsZ = __builtin_amdgcn_make_buffer_rsrc(
      p.z ? const_cast<uint16_t*>(static_cast<const uint16_t*>(p.z) + (b * D + d0) * L) : nullptr, 0, blk_bytes, kRawWord3);
  auto fetch = [&](int64_t t0, Raw& R) {
    const int64_t valid = L - t0;
    if (vecp && off32 && valid >= kQ) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (kN == 128 || 4 * nq < kN) {   // rows past kN are not staged
          const int so = (int)((j * L + t0) * 2);
          R.c[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsC, voff_bc, so, 0));
          R.bb[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsB, voff_bc, so, 0));
        }
      }
      R.x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsX, voff_x, (int)(t0 * 2), 0));
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
        R.z[tm] = p.z ? __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rsZ, voff_z, (int)((t0 + 16 * tm) * 2), 0))
                      : make_uint2(0u, 0u);
      R.dt = (w == 3 && l < valid - kQ && l < kQ) ? (uint32_t)dtrow[t0 + kQ + l] : 0u;
      return;
    }
    const bool vec = vecp && valid >= kQ;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = 4 * nq + j;
      const bool ok = n < N;
      const int64_t off = (ok ? n : 0) * L + t0;
      R.c[j] = ok ? ld_row4(Crow + off, 4 * tb4, vec, valid - 4 * tb4) : make_uint2(0u, 0u);
      R.bb[j] = ok ? ld_row4(Brow + off, 4 * tb4, vec, valid - 4 * tb4) : make_uint2(0u, 0u);
    }
    if (vec) {
      R.x = *reinterpret_cast<const uint4*>(xrow + t0 + 8 * tb8);
    } else {
      const uint2 lo = ld_row4(xrow + t0, 8 * tb8, false, valid - 8 * tb8);
      const uint2 hi = ld_row4(xrow + t0, 8 * tb8 + 4, false, valid - 8 * tb8 - 4);
      R.x = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
      R.z[tm] = zrow ? ld_row4(zrow + t0, 16 * tm + 4 * g, vec, valid - 16 * tm - 4 * g)
                                    : make_uint2(0u, 0u);
    const int64_t vnext = valid - kQ;
    R.dt = (w == 3 && l < vnext && l < kQ) ? (uint32_t)dtrow[t0 + kQ + l] : 0u;
  };
  // step sizes, decays and coefficients of the chunk at t0 from its raw delta
  // (wave 3 only; lane l = step l)
  auto chunk_params = [&](int64_t t0, uint32_t dtw, int buf) {
    const int64_t valid = L - t0;
    float dl = 0.0f, cf = 0.0f;
    if (l < valid && l < kQ) {
      dl = softplus(bf16_to_f32((uint16_t)dtw) + bias);
      cf = kDeltaB ? dl : expm1_from_exp2(dl * a2, hw_exp2(dl * a2)) * ia;
    }
    float v = dl * a;
#pragma unroll
    for (int off = 1; off < kQ; off <<= 1) {
      const float o = __shfl_up(v, off, 64);
      if (l >= off) v += o;
    }
    const float last = __shfl(v, kQ - 1, 64);
    if (l < kQ) {
      S.cum[buf][l] = v;
      S.coef[buf][l] = cf;
      S.ecum[buf][l] = hw_exp2(v * kLog2e);
      S.wl[buf][l] = hw_exp2((last - v) * kLog2e) * cf;
    }
    if (l == 0) S.elast[buf] = hw_exp2(last * kLog2e);
  };
  auto stage = [&](const Raw& R) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = 4 * nq + j;
      if (n < kN) {
        *reinterpret_cast<uint2*>(&S.BcT[n][4 * tb4]) = R.bb[j];
      }
    }
    // transpose 4 states x 4 steps into [step][state]
    const uint32_t c16[4][2] = {{R.c[0].x, R.c[0].y}, {R.c[1].x, R.c[1].y}, {R.c[2].x, R.c[2].y}, {R.c[3].x, R.c[3].y}};
    const uint32_t b16[4][2] = {{R.bb[0].x, R.bb[0].y}, {R.bb[1].x, R.bb[1].y}, {R.bb[2].x, R.bb[2].y},
                                {R.bb[3].x, R.bb[3].y}};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      auto el = [&](const uint32_t (&m)[4][2], int j) -> uint32_t {
        const uint32_t word = m[j][s >> 1];
        return (s & 1) ? (word >> 16) : (word & 0xffffu);
      };
      const uint2 cv = make_uint2(el(c16, 0) | (el(c16, 1) << 16), el(c16, 2) | (el(c16, 3) << 16));
      const uint2 bv = make_uint2(el(b16, 0) | (el(b16, 1) << 16), el(b16, 2) | (el(b16, 3) << 16));
      if (4 * nq < kN) {
        *reinterpret_cast<uint2*>(&S.Cc[4 * tb4 + s][4 * nq]) = cv;
        *reinterpret_cast<uint2*>(&S.Bc[4 * tb4 + s][4 * nq]) = bv;
      }
    }
    *reinterpret_cast<uint4*>(&S.X[px][8 * tb8]) = R.x;
  };

  // the entering state: the earlier segments' end states (from zero) and
  // decays chained in order, h_in(j + 1) = P(j) h_in(j) + h_end(j) -- the
  // associative combination over segment aggregates.  Slots are
  // ((b S + j) H + h) pblocks + pb, [channel][state] fp32.
  f32x4 Hs[kNT];
#pragma unroll
  for (int i = 0; i < kNT; ++i) Hs[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t j = 0; j < seg; ++j) {
    const int64_t sj = ((b * p.S + j) * p.H + h) * pblocks + pb;
    const float Pj = p.ws_P[sj];
    const float* hl = p.ws_h + (sj * kP + pc) * N;
#pragma unroll
    for (int tn = 0; tn < kNT; ++tn) {
      const float4 v = *reinterpret_cast<const float4*>(hl + 16 * tn + 4 * g);
      Hs[tn] = f32x4{__builtin_fmaf(Pj, Hs[tn][0], v.x), __builtin_fmaf(Pj, Hs[tn][1], v.y),
                     __builtin_fmaf(Pj, Hs[tn][2], v.z), __builtin_fmaf(Pj, Hs[tn][3], v.w)};
    }
  }

  const int64_t ck0 = t_begin / kQ, nchunks = (t_end + kQ - 1) / kQ;
  // One register set: once staged (and past the barrier that follows), it
  // receives the next chunk's loads, so nothing is copied between chunks.
  Raw cur;
  fetch(t_begin, cur);
  if (w == 3) chunk_params(t_begin, (l < L - t_begin && l < kQ) ? (uint32_t)dtrow[t_begin + l] : 0u, (int)(ck0 & 1));
  for (int64_t c = ck0; c < nchunks; ++c) {
    const int64_t t0 = c * kQ;
    const int64_t valid = L - t0;
    const int cb = (int)(c & 1);
    __syncthreads();                       // the previous chunk's LDS reads are done
    stage(cur);
    const uint2 zc[2] = {cur.z[0], cur.z[1]};   // cur receives the next chunk below
    const uint4 xc = cur.x;
    const uint32_t dtn = cur.dt;
    __syncthreads();
    if (c + 1 < nchunks) fetch(t0 + kQ, cur);

    // ---- S = C B^T on the three lower 16 x 16 tiles and G from it (waves
    // 0..2); the next chunk's step sizes, decays and coefficients (wave 3)
    const int tm1 = (w == 0) ? 0 : 1, tn1 = (w == 2) ? 1 : 0;
    if (w < 3) {
      f32x4 St = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < kNK; ++kb)
        St = mfma(lds8(&S.Cc[16 * tm1 + r][32 * kb + 8 * g]), lds8(&S.Bc[16 * tn1 + r][32 * kb + 8 * g]), St);
      const int s = 16 * tn1 + r;
      const float cs = S.cum[cb][s], fs = S.coef[cb][s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tm1 + 4 * g + e;
        const float gv = (s <= t) ? St[e] * hw_exp2((S.cum[cb][t] - cs) * kLog2e) * fs : 0.0f;
        split_bf16(gv, S.Gh[t][s], S.Gl[t][s]);
      }
    } else if (w == 3 && c + 1 < nchunks) {
      chunk_params(t0 + kQ, dtn, cb ^ 1);
    }
    {
      const uint32_t xw[4] = {xc.x, xc.y, xc.z, xc.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint16_t h0, l0, h1, l1;
        split_bf16(bf16_lo(xw[j]) * S.wl[cb][8 * tb8 + 2 * j], h0, l0);
        split_bf16(bf16_hi(xw[j]) * S.wl[cb][8 * tb8 + 2 * j + 1], h1, l1);
        hw[j] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[j] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      *reinterpret_cast<uint4*>(&S.Xh[px][8 * tb8]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&S.Xl[px][8 * tb8]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    }
    __syncthreads();

    // ---- y = G x + exp(cum_t) C H + D x for the wave's 16 channels
    f32x4 Yd[2], Yo[2];
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const bf16x8 xb = lds8(&S.X[pc][8 * g]);
      Yd[tm] = mfma(lds8(&S.Gh[16 * tm + r][8 * g]), xb, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
      Yd[tm] = mfma(lds8(&S.Gl[16 * tm + r][8 * g]), xb, Yd[tm]);
      Yo[tm] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // the entering state as B operands of C H, one K block at a time (its
    // split overlaps the products of the block before): K block kb holds
    // states 32 kb + 4 g + e (tile 2 kb) and 32 kb + 16 + 4 g + e (tile 2 kb + 1)
#pragma unroll
    for (int kb = 0; kb < kNK; ++kb) {
      bf16x8 hh, hl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (e < 4) ? Hs[2 * kb][e] : Hs[2 * kb + 1][e - 4];
        uint16_t hi, lo;
        split_bf16(v, hi, lo);
        hh[e] = __builtin_bit_cast(__bf16, hi);
        hl[e] = __builtin_bit_cast(__bf16, lo);
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        const bf16x8 ca = lds4x2(&S.Cc[16 * tm + r][32 * kb + 4 * g], &S.Cc[16 * tm + r][32 * kb + 16 + 4 * g]);
        Yo[tm] = mfma(ca, hh, Yo[tm]);
        Yo[tm] = mfma(ca, hl, Yo[tm]);
      }
    }
    // ---- H <- exp(cum_last) H + B^T (w o x)
    {
      const float el = S.elast[cb];
      const bf16x8 xh = lds8(&S.Xh[pc][8 * g]), xl = lds8(&S.Xl[pc][8 * g]);
#pragma unroll
      for (int tn = 0; tn < kNT; ++tn) {
        Hs[tn] *= el;
        const bf16x8 bt = lds8(&S.BcT[16 * tn + r][8 * g]);
        Hs[tn] = mfma(bt, xh, Hs[tn]);
        Hs[tn] = mfma(bt, xl, Hs[tn]);
      }
    }
    // ---- gate and store: lane holds steps 16 tm + 4 g + e of channel pc
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const int tb = 16 * tm + 4 * g;
      const uint2 xv = *reinterpret_cast<const uint2*>(&S.X[pc][tb]);
      const float xs[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
      const float zs[4] = {bf16_lo(zc[tm].x), bf16_hi(zc[tm].x), bf16_lo(zc[tm].y), bf16_hi(zc[tm].y)};
      float yv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = __builtin_fmaf(S.ecum[cb][tb + e], Yo[tm][e], Yd[tm][e]);
        v = __builtin_fmaf(Dp, xs[e], v);
        if (zrow) v *= silu(zs[e]);
        yv[e] = v;
      }
      const int64_t o = (b * D + d0 + pc) * L + t0 + tb;
      const int64_t nv = valid - tb;
      if (kOutBF16) {
        uint16_t* yp = static_cast<uint16_t*>(p.y) + o;
        if (vecp && nv >= 4) {
          *reinterpret_cast<uint2*>(yp) = make_uint2(pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < nv) yp[e] = f32_to_bf16(yv[e]);
        }
      } else {
        float* yp = static_cast<float*>(p.y) + o;
        if (vecp && nv >= 4) {
          *reinterpret_cast<float4*>(yp) = make_float4(yv[0], yv[1], yv[2], yv[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (e < nv) yp[e] = yv[e];
        }
      }
    }
  }
  if (p.final_state && seg == p.S - 1) {
    float* fs = p.final_state + (b * D + d0 + pc) * N;
#pragma unroll
    for (int tn = 0; tn < kNT; ++tn)
      *reinterpret_cast<float4*>(fs + 16 * tn + 4 * g) = make_float4(Hs[tn][0], Hs[tn][1], Hs[tn][2], Hs[tn][3]);
  }
}

// End state of every segment but the last, from a zero state at its start,
// and the segment's decay exp(A sum delta), for the carry:
//   H = sum_s exp(A sum_(s < r <= end) delta_r) coef_s x_s B_s^T.
// Each step's weight folds in its decay to the segment end, so the segment
// is one weighted product over its steps: no chunk products, no rescaling of
// the state.  Per 32-step block the workgroup stages B_t ([state][step], as
// read) and the weighted x split into two bf16 parts in LDS, double-buffered
// with one barrier per block, with the global loads two blocks ahead; wave w
// then accumulates channels 16 w .. 16 w + 15 exactly as the chunk kernel
// holds its state.  The weights of up to kPiece steps at a time are computed
// from the segment end backwards: suffix sums of delta stay small, and
// exact, where the decay is near 1.
constexpr int kPiece = 512;

template <int V> struct IntTag { static constexpr int kValue = V; };
// f(IntTag<i>{}) for i = I .. E-1, unrolled
template <int I, int E, typename F>
__device__ __forceinline__ void unroll_for(F&& f) {
  if constexpr (I < E) {
    f(IntTag<I>{});
    unroll_for<I + 1, E>(f);
  }
}

// Rows of 32 bf16 with no padding; the 16-byte block q of row n is stored at
// block q ^ swz(n), so that 16 lanes reading block q of rows n .. n + 15 (an
// MFMA operand) or writing 4 blocks of 4 rows touch every LDS bank once.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int kN>
struct StateLds {
  uint16_t BT[2][kN][kQ];          // B_t [state][step], swizzled blocks
  uint16_t Xh[2][kP][kQ];          // w o x [channel][step], high part, swizzled blocks
  uint16_t Xl[2][kP][kQ];          //                        remainder
  float Wt[kPiece];                // w of the piece's steps
  float wave_sum[2][4];
};

template <int kN, bool kDeltaB, bool kVec>
__global__ __launch_bounds__(256, 4) void ssd_state_kernel(SsdParams p) {
  __shared__ StateLds<kN> S;
  constexpr int kNT = kN / 16;
  constexpr int kBR = kN / 64;                               // B rows per staging thread
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int g = l >> 4, r = l & 15;
  const int lr = tid >> 2, lq = tid & 3;                     // staging: row lr (+ 64 i), steps 8 lq .. + 7
  const int64_t pblocks = p.P / kP;
  const int64_t segs = p.S - 1;                              // the last segment needs no end state
  const int64_t wg = xcd_item(blockIdx.x, gridDim.x);      // ((b segs + seg) H + h) pblocks + pb
  const int64_t pb = wg % pblocks;
  const int64_t h = (wg / pblocks) % p.H;
  const int64_t bs = wg / (pblocks * p.H);
  const int64_t seg = bs % segs, b = bs / segs;
  const int64_t slot = ((b * p.S + seg) * p.H + h) * pblocks + pb;
  const int64_t t_begin = seg * p.seg_len;                   // whole segment: t_begin + seg_len < L
  const int64_t L = p.L, D = p.H * p.P, N = p.N;
  const float a = p.A[h];
  const float a2 = a * kLog2e;
  const float ia = 1.0f / a;
  const float bias = p.bias ? p.bias[h] : 0.0f;
  const int pc = 16 * w + r;
  const uint16_t* xrow = static_cast<const uint16_t*>(p.x) + (b * D + h * p.P + pb * kP + lr) * L;
  const uint16_t* dtrow = static_cast<const uint16_t*>(p.delta) + (b * p.H + h) * L;
  const uint16_t* Bbase = static_cast<const uint16_t*>(p.Bt) + b * N * L;

  f32x4 Hs[kNT];
#pragma unroll
  for (int i = 0; i < kNT; ++i) Hs[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // 8 consecutive bf16 of a row at t (one 16-byte load when the rows allow it)
  auto ld8 = [&](const uint16_t* row, int64_t t) -> uint4 {
    if constexpr (kVec) return *reinterpret_cast<const uint4*>(row + t);
    uint32_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = row[t + j];
    return make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
  };
  struct Raw {
    uint4 x;
    uint4 bt[kBR];
  };
  auto fetch = [&](int64_t t, Raw& o) {
    o.x = ld8(xrow, t + 8 * lq);
#pragma unroll
    for (int i = 0; i < kBR; ++i) o.bt[i] = ld8(Bbase + (lr + 64 * i) * L, t + 8 * lq);
  };

  float after = 0.0f;   // sum of delta over the segment's steps after the current piece
  const int64_t npieces = (p.seg_len + kPiece - 1) / kPiece;
  ProgressPrio prio;    // one round of workgroups: they finish together (kernels.hpp)
  prio.begin();
  for (int64_t pi = npieces - 1; pi >= 0; --pi) {
    const int64_t p0 = t_begin + pi * kPiece;
    const int plen = (int)((p.seg_len - pi * kPiece) < kPiece ? (p.seg_len - pi * kPiece) : kPiece);
    // weights of steps 2 tid and 2 tid + 1 of the piece
    const int s0 = 2 * tid;
    float dl[2] = {0.0f, 0.0f}, cf[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (s0 + j < plen) {
        dl[j] = softplus(bf16_to_f32(dtrow[p0 + s0 + j]) + bias);
        cf[j] = kDeltaB ? dl[j] : expm1_from_exp2(dl[j] * a2, hw_exp2(dl[j] * a2)) * ia;
      }
    }
    const float own = dl[0] + dl[1];
    float v = own;                                      // sum over this lane and the lanes above it
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_down(v, off, 64);
      if (l + off < 64) v += o;
    }
    const int par = (int)(pi & 1);
    if (l == 0) S.wave_sum[par][w] = v;
    __syncthreads();                                    // also: the previous piece's blocks are consumed
    float later_waves = 0.0f;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (w + j < 4) later_waves += S.wave_sum[par][w + j];
    const float beyond = (v - own) + later_waves + after;   // delta after step s0 + 1
    if (s0 < plen) S.Wt[s0] = hw_exp2(a2 * (beyond + dl[1])) * cf[0];
    if (s0 + 1 < plen) S.Wt[s0 + 1] = hw_exp2(a2 * beyond) * cf[1];
    after += (S.wave_sum[par][0] + S.wave_sum[par][1]) + (S.wave_sum[par][2] + S.wave_sum[par][3]);
    __syncthreads();

    // the piece's 32-step blocks: global loads two blocks ahead in three
    // rotating register sets (none is copied: a copy would wait for the loads
    // in flight), issued unconditionally with addresses past the piece
    // clamped to its last block (a conditional load would leave the compiler
    // unsure how many loads are in flight, and its waits would then cover the
    // newest ones as well)
    const int nblk = plen / 32;
    auto block = [&](const Raw& o, int k) {
      const int buf = k & 1;
      const float4 w0 = *reinterpret_cast<const float4*>(&S.Wt[32 * k + 8 * lq]);
      const float4 w1 = *reinterpret_cast<const float4*>(&S.Wt[32 * k + 8 * lq + 4]);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      const uint32_t xw[4] = {o.x.x, o.x.y, o.x.z, o.x.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint16_t h0, l0, h1, l1;
        split_bf16(bf16_lo(xw[i]) * wv[2 * i], h0, l0);
        split_bf16(bf16_hi(xw[i]) * wv[2 * i + 1], h1, l1);
        hw[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      }
      const int wq = 8 * (lq ^ swz(lr));                 // rows lr + 64 i share the swizzle
      *reinterpret_cast<uint4*>(&S.Xh[buf][lr][wq]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      *reinterpret_cast<uint4*>(&S.Xl[buf][lr][wq]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
#pragma unroll
      for (int i = 0; i < kBR; ++i) *reinterpret_cast<uint4*>(&S.BT[buf][lr + 64 * i][wq]) = o.bt[i];
      // the other buffer's readers finished before they reached this barrier
      __syncthreads();
      const int rq = 8 * (g ^ swz(r));                   // rows pc and 16 tn + r have r's swizzle
      const bf16x8 xh = lds8(&S.Xh[buf][pc][rq]), xl = lds8(&S.Xl[buf][pc][rq]);
#pragma unroll
      for (int tn = 0; tn < kNT; ++tn) {
        const bf16x8 bt = lds8(&S.BT[buf][16 * tn + r][rq]);
        Hs[tn] = mfma(bt, xh, Hs[tn]);
        Hs[tn] = mfma(bt, xl, Hs[tn]);
      }
    };
    auto blk_t = [&](int k) { return p0 + 32 * (k < nblk ? k : nblk - 1); };
    constexpr int kAhead = 2, kSets = 3;
    Raw o[kSets];
    unroll_for<0, kAhead>([&](auto jc) { fetch(blk_t(decltype(jc)::kValue), o[decltype(jc)::kValue]); });
    const int ngroups = nblk / kSets;
    for (int gi = 0; gi < ngroups; ++gi) {
      prio.at((npieces - 1 - pi) * kPiece + gi * kSets * 32, p.seg_len);
      unroll_for<0, kSets>([&](auto jc) {
        constexpr int j = decltype(jc)::kValue;
        const int k = gi * kSets + j;
        fetch(blk_t(k + kAhead), o[(j + kAhead) % kSets]);
        block(o[j], k);
      });
    }
    // the last nblk % kSets blocks are already loaded, in o[0] ..
    const int rem = nblk - ngroups * kSets;
    unroll_for<0, kSets - 1>([&](auto jc) {
      constexpr int j = decltype(jc)::kValue;
      if (j < rem) block(o[j], ngroups * kSets + j);
    });
  }
  float* ho = p.ws_h + (slot * kP + pc) * N;
#pragma unroll
  for (int tn = 0; tn < kNT; ++tn)
    *reinterpret_cast<float4*>(ho + 16 * tn + 4 * g) = make_float4(Hs[tn][0], Hs[tn][1], Hs[tn][2], Hs[tn][3]);
  if (tid == 0) p.ws_P[slot] = hw_exp2(a2 * after);
}

template <int kN, bool kOutBF16, bool kDeltaB>
hipError_t ssd_d(const SsdParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.S * p.H * (p.P / kP)));
  if (p.S > 1) {
    const dim3 sgrid((unsigned)(p.B * (p.S - 1) * p.H * (p.P / kP)));
    if (p.vec)
      hipLaunchKernelGGL((ssd_state_kernel<kN, kDeltaB, true>), sgrid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((ssd_state_kernel<kN, kDeltaB, false>), sgrid, dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ssd_chunk_kernel<kN, kOutBF16, kDeltaB>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int kN, bool kOutBF16>
hipError_t ssd_t(const SsdParams& p, hipStream_t s) {
  return p.delta_b ? ssd_d<kN, kOutBF16, true>(p, s) : ssd_d<kN, kOutBF16, false>(p, s);
}

}  // namespace

hipError_t launch_ssd(const SsdParams& p, Dt out, hipStream_t s) {
  if (p.N == 128) return out == Dt::BF16 ? ssd_t<128, true>(p, s) : ssd_t<128, false>(p, s);
  return out == Dt::BF16 ? ssd_t<64, true>(p, s) : ssd_t<64, false>(p, s);
}

}  // namespace mamba

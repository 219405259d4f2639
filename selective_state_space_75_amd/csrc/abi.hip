// abi.hip -- the C ABI declared in include/mamba_scan.h: argument checks,
// the execution plan of a scan (single pass or chunked along L), and the
// kernel launches.  Every check runs before any HIP call.
#include <atomic>
#include <chrono>
#include <mutex>

#include "kernels.hpp"
#include "mamba_scan.h"

namespace {

using mamba::Dt;

constexpr int64_t kTile = 64;         // channels per scan workgroup
constexpr int64_t kStage = 32;        // staging chunk of the scan kernel (steps)
constexpr int64_t kMaxElems = int64_t(1) << 46;
constexpr int64_t kV4Step = 32;       // the wave-tile kernel's chunk: L at least this, and a multiple of 8
constexpr int64_t kV4Tile = 16;       // channels per wave in the wave-tile kernel
constexpr int64_t kGroupsPlan = 1024; // waves of the balanced split (one per SIMD on MI355X)
constexpr int64_t kRowStep = 32;      // the row kernel's chunk (its fast form: L a multiple of this)
constexpr int64_t kCUsPlan = 256;     // compute units the plan assumes (MI355X)
constexpr size_t kHandOverBytes = kV4Tile * 16 * sizeof(float);

struct Plan {
  int64_t tiles_d = 0;
  int64_t n_chunks = 1;
  int64_t chunk_len = 0;
  bool v4 = false;          // the wave-tile kernel (L a multiple of 8, L >= 32)
  bool row = false;         // the row kernel (one state per lane, L a multiple of 32)
  bool row_lean = false;    // its lean variant (five workgroups per CU)
  bool balanced = false;    // equal (tile x time) ranges with state hand-over
  size_t ws_bytes = 0;
  size_t off_local = 0, off_start = 0, off_sum = 0;
  size_t off_flag = 0, off_pub = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool shape_ok(int64_t B, int64_t D, int64_t N, int64_t L) {
  if (B < 1 || D < 1 || N < 1 || L < 1) return false;
  if (B > kMaxElems / D) return false;
  if (B * D > kMaxElems / L) return false;
  return true;
}

// Test knobs (mamba_set_test_knobs): process-wide, copied once per call so
// that a call sees one consistent set.  Zero-initialised fields and a negative
// hand-over bound are the defaults.
std::mutex g_knob_mu;
mamba_test_knobs_t g_knobs = {0, 0, 0, -1, 0};

mamba_test_knobs_t knobs() {
  std::lock_guard<std::mutex> lock(g_knob_mu);
  return g_knobs;
}

// Relative time of the wave-tile kernel over k chunks of L, in units of one
// wave's full pass over L, for G = kGroupsPlan waves (one per SIMD): the
// state-only summary pass over the first k - 1 chunks (no readout, gate or
// output: about 3/4 of the full pass per step) and the full pass, which is
// balanced over the G waves once there are at least G (chunk, tile) pairs.
double v4_chunk_cost(int64_t tiles, int64_t k) {
  const int64_t G = kGroupsPlan;
  auto rounds = [&](int64_t waves) { return double((waves + G - 1) / G); };
  const double full = k * tiles >= G ? double(tiles) / double(G) : rounds(k * tiles) / double(k);
  const double summary = k > 1 ? 0.75 * rounds((k - 1) * tiles) / double(k) : 0.0;
  return full + summary;
}

// Relative time of the row kernel (one state per lane, a 16-channel tile per
// 4-wave workgroup, up to three workgroups per CU) in the units of
// v4_chunk_cost.  Measured per 2048 steps on MI355X, against 190 us for a
// wave-tile pass of one tile per SIMD: 68, 103 and 133 us with one, two and
// three workgroups per CU (the last two with the issue priority stepped down
// by progress); from four on about 26.6 + 41.9 us per workgroup per CU (a
// fit over 5, 7, 8, 10 and 12 per CU at steady clocks, with the state scaled
// by A, within 1.5% of each; 198, 228 and 262 us at 4, 5 and 6 per CU with
// the priority).
double row_cost(int64_t wgs) {
  const int64_t per_cu = (wgs + kCUsPlan - 1) / kCUsPlan;
  static const double kFew[3] = {68.0, 103.0, 133.0};
  const double us = per_cu <= 3 ? kFew[per_cu - 1] : 26.6 + 41.9 * double(per_cu);
  return us / 190.0;
}

// Shape-only plan (no device query).  When L is a multiple of 32: the lean
// row kernel from four 16-channel workgroups per CU on.  Otherwise, and for
// any other L >= 32: the row kernel (element loads when L is not a multiple
// of 32), in chunks when there are few tiles, or when its cost model beats
// the wave-tile kernel's (few 16-channel tiles, as in the 130M layer and the
// batch-1 long sequence); else the wave-tile kernel, one pass per channel
// tile while there are enough tiles to occupy the GPU, otherwise (few
// channels, long L) split L into chunks of at least 2048 steps, their number
// minimising v4_chunk_cost.  The general kernel takes L < 32 (and plans about
// 1024 workgroups when forced on a long L).
Plan make_plan(int64_t B, int64_t D, int64_t N, int64_t L, const mamba_test_knobs_t& kn) {
  Plan p;
  p.tiles_d = (D + kTile - 1) / kTile;
  p.v4 = (L % 8 == 0) && L >= kV4Step && kn.scan_kernel != 1;
  // The row kernel takes any L >= 32 (element loads and a shifted last chunk
  // when L is not a multiple of 32).  With the state scaled by A its ragged
  // form beats the wave-tile kernel's shifted chunk as well (timed at steady
  // clocks: the 130M layer at L = 2040 153 against 191 us, the batch-1 long
  // sequence at L = 131064 4.1 against 4.68 ms, the 2.8B layer at L = 2040
  // within 2%), so the same rules apply to every L >= 32.
  const bool aligned = L % kRowStep == 0;
  const bool row_ok = L >= kRowStep && kn.scan_kernel != 1 && kn.scan_kernel != 2 &&
                      (kn.scan_chunks == 0 || kn.scan_kernel == 3);
  if (row_ok) {
    const int64_t tiles16 = B * ((D + kV4Tile - 1) / kV4Tile);
    const int64_t per_cu = (tiles16 + kCUsPlan - 1) / kCUsPlan;
    // The lean row kernel from four 16-channel workgroups per CU on (the
    // count rounded up).  Both kernels step their issue priority down by
    // progress (ProgressPrio); timed on MI355X at steady clocks (B = 4,
    // L = 2048, lean against row): 3 per CU 136 against 133 us, 3.5 per CU
    // 162 against 196 us, 4 per CU 164 against 198 us, 5 per CU (the 2.8B
    // layer) 200 against 228 us, 6 per CU 269 against 262 us.
    // (the lean variant has no ragged form: a forced lean at such an L runs the row
    // kernel; it counts chunks in 32 bits, so it takes L < 2^33 only)
    const bool lean = aligned && L < (int64_t(1) << 33) &&
                      (kn.scan_kernel == 4 || (kn.scan_kernel == 0 && per_cu >= 4));
    // With 64 to 384 tiles (1.5 per CU at most) the row kernel cuts L into K
    // chunks so that each of its two passes puts K - 1 workgroups on every
    // tile, about three per CU: the first pass runs chunk 0 in full and
    // chunks 1 .. K-2 as summaries, the second chunks 1 .. K-1 from the
    // carried states.  Chunks of at least 2048 steps, a multiple of 64.
    // Timed on MI355X this beat the wave-tile kernel's chunked path at every
    // shape tried (B = 1 with D = 1024, 2048, 4096 and 5120, L = 8192 to
    // 131072: by 1 to 14%), so it is taken whenever it applies.
    int64_t k = 1;
    if (!lean) {
      if (kn.scan_chunks > 0) {
        k = kn.scan_chunks;
      } else if ((tiles16 >= 64 || !p.v4) && tiles16 <= 384) {   // below 64 tiles only where the wave-tile kernel cannot go
        k = 768 / tiles16 + 1;
        if (k > L / 2048) k = L / 2048;
        if (k > 16) k = 16;
        if (k < 3) k = 1;
      }
    }
    bool row = kn.scan_kernel >= 3 || lean || (kn.scan_kernel == 0 && (k >= 3 || !p.v4));
    if (!row) {
      double best = v4_chunk_cost(tiles16, 1);
      const int64_t kmax = L >= 4096 && tiles16 < kGroupsPlan ? (L / 2048 < 64 ? L / 2048 : 64) : 1;
      for (int64_t c = 2; c <= kmax; ++c) best = v4_chunk_cost(tiles16, c) < best ? v4_chunk_cost(tiles16, c) : best;
      row = row_cost(tiles16) < best;
    }
    if (row) {
      p.row = true;
      p.row_lean = lean;
      p.v4 = false;
      p.tiles_d = (D + kV4Tile - 1) / kV4Tile;
      if (k > 1) {
        int64_t len = (L + k - 1) / k;
        len = (len + 2 * kRowStep - 1) / (2 * kRowStep) * (2 * kRowStep);
        p.chunk_len = len;
        p.n_chunks = (L + len - 1) / len;
      }
      if (p.n_chunks > 1) {
        const size_t state = size_t(p.n_chunks) * size_t(B) * size_t(D) * size_t(N) * sizeof(float);
        const size_t sums = size_t(p.n_chunks) * size_t(B) * size_t(D) * sizeof(float);
        p.off_local = 0;
        p.off_start = align256(state);
        p.off_sum = p.off_start + align256(state);
        p.ws_bytes = p.off_sum + align256(sums);
      }
      return p;   // one pass, or two over chunks with the carry between them
    }
  }
  // Units of independent sequential work: 16-channel tiles (wave-tile
  // kernel) or 64-channel tiles (general kernel).
  const int64_t tiles = p.v4 ? B * ((D + kV4Tile - 1) / kV4Tile) : B * p.tiles_d;
  int64_t k = 1;
  if (kn.scan_chunks > 0) {
    k = kn.scan_chunks;
  } else if (p.v4 && L >= 4096 && tiles < kGroupsPlan) {
    const int64_t kmax = L / 2048 < 64 ? L / 2048 : 64;
    double best = v4_chunk_cost(tiles, 1);
    for (int64_t c = 2; c <= kmax; ++c) {
      const double cost = v4_chunk_cost(tiles, c);
      if (cost < best) { best = cost; k = c; }
    }
  } else if (!p.v4 && L >= 4096 && tiles < 512) {
    k = (1024 + tiles - 1) / tiles;
    if (k > L / 2048) k = L / 2048;
    if (k > 64) k = 64;
    if (k < 1) k = 1;
  }
  int64_t len = (L + k - 1) / k;
  len = (len + kStage - 1) / kStage * kStage;
  p.chunk_len = len;
  p.n_chunks = (L + len - 1) / len;
  p.balanced = p.v4 && p.n_chunks * tiles >= kGroupsPlan && !kn.scan_no_balance;
  size_t o = 0;
  if (p.n_chunks > 1) {
    const size_t state = size_t(p.n_chunks) * size_t(B) * size_t(D) * size_t(N) * sizeof(float);
    const size_t sums = size_t(p.n_chunks) * size_t(B) * size_t(D) * sizeof(float);
    p.off_local = 0;
    p.off_start = align256(state);
    p.off_sum = p.off_start + align256(state);
    o = p.off_sum + align256(sums);
  }
  if (p.balanced) {
    p.off_flag = o;
    p.off_pub = o + align256(kGroupsPlan * sizeof(uint64_t));
    o = p.off_pub + kGroupsPlan * kHandOverBytes;
  }
  p.ws_bytes = o;
  return p;
}

// Compute units of the current device, cached per device id.
int64_t device_cus() {
  static std::mutex mu;
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

// Bound of the wait for a state hand-over between workgroups, in polls of a
// short sleep (each at least ~60 ns): 256 polls per 32-step block of a
// workgroup's share, at least 8192.  A share's blocks take well under 256
// polls each to scan, so the bound is several times the launch's own
// duration; when it runs out (the publishing workgroup is not resident), the
// waiting one recomputes the state instead.  The test knob sets it directly
// (0 forces every recompute).
uint32_t handover_spin_limit(int64_t blocks_per_group, const mamba_test_knobs_t& kn) {
  if (kn.handover_spin >= 0) return kn.handover_spin < (1ll << 30) ? (uint32_t)kn.handover_spin : (1u << 30);
  const int64_t v = 256 * blocks_per_group;
  return v < 8192 ? 8192u : (v > (1ll << 24) ? (1u << 24) : (uint32_t)v);
}

// Numbers launches of the balanced kernel: a hand-over slot counts as
// published only when its flag holds this launch's value, so stale flags
// left in a reused workspace are never mistaken for fresh ones.  These values
// always have the top bit set; a launch recorded into a graph uses the fixed
// value kCaptureEpoch instead (a replay cannot take a new value from the
// host), after a small kernel clears the flags on every replay.
constexpr uint64_t kCaptureEpoch = 1;

uint64_t next_epoch() {
  static std::atomic<uint64_t> counter{0};
  static std::once_flag once;
  std::call_once(once, [] {
    const uint64_t t = (uint64_t)std::chrono::high_resolution_clock::now().time_since_epoch().count();
    counter.store((t * 0x9E3779B97F4A7C15ull) | 1ull);
  });
  return counter.fetch_add(1) | (1ull << 63);
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }
bool dtype_ok(int t) { return t == MAMBA_F32 || t == MAMBA_BF16; }
constexpr unsigned kKnownFlags = MAMBA_FLAG_DELTA_B | MAMBA_FLAG_ACCURATE_EXPM1;

}  // namespace

struct BwdPlan {
  int64_t tiles_d = 0, groups = 0, nck = 0, S = 0, seg_len = 0;
  size_t off_ckh = 0, off_ckd = 0, off_sp = 0, off_sh = 0, off_sH = 0, off_hin = 0, off_gin = 0;
  size_t off_pb = 0, off_pc = 0, off_pa = 0, off_pd = 0, off_pbias = 0, bytes = 0;
};

// Segments: enough (batch row, channel tile, segment) tasks to give every
// SIMD of the chip several (at least 8192 in all), segments of at least 64
// steps, lengths a multiple of 32.  Where a count up to twice that minimum
// cuts L into equal whole 32-step blocks it is taken instead, so that no
// short last segment leaves the final round of waves half empty (2.8B
// layer: 8 segments of 256 steps rather than 6 of 320 and one of 128).
BwdPlan make_bwd_plan(int64_t B, int64_t D, int64_t L) {
  BwdPlan q;
  constexpr int64_t kC = mamba::kBwdBlock;
  q.tiles_d = (D + 15) / 16;
  q.groups = (q.tiles_d + mamba::kBwdGroup - 1) / mamba::kBwdGroup;
  q.nck = (L + kC - 1) / kC;
  const int64_t rows = B * q.tiles_d;
  int64_t S = (8192 + rows - 1) / rows;
  const int64_t smax = (L + 63) / 64;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  if (L % 32 == 0) {
    for (int64_t c = S; c <= 2 * S && c <= smax; ++c)
      if ((L / 32) % c == 0) { S = c; break; }
  }
  int64_t len = (L + S - 1) / S;
  len = (len + 31) / 32 * 32;     // whole 32-step staging blocks
  q.seg_len = len;
  q.S = (L + len - 1) / len;
  const size_t bd = size_t(B) * size_t(D), bsd = bd * size_t(q.S);
  size_t o = 0;
  q.off_ckh = o; o += align256(bd * size_t(q.nck) * 16 * sizeof(float));
  q.off_ckd = o; o += align256(bd * size_t(q.nck) * sizeof(float));
  q.off_sp = o; o += align256(bsd * 16 * sizeof(float));
  q.off_sh = o; o += align256(bsd * 16 * sizeof(float));
  q.off_sH = o; o += align256(bsd * 16 * sizeof(float));
  q.off_hin = o; o += align256(bsd * 16 * sizeof(float));
  q.off_gin = o; o += align256(bsd * 16 * sizeof(float));
  q.off_pb = o; o += align256(size_t(B) * size_t(q.groups) * 16 * size_t(L) * sizeof(float));
  q.off_pc = o; o += align256(size_t(B) * size_t(q.groups) * 16 * size_t(L) * sizeof(float));
  q.off_pa = o; o += align256(bsd * 16 * sizeof(float));
  q.off_pd = o; o += align256(bsd * sizeof(float));
  q.off_pbias = o; o += align256(bsd * sizeof(float));
  q.bytes = o;
  return q;
}

namespace {

// Argument checks shared by mamba_scan_fwd and mamba_scan_fwd_noalloc; no HIP call.
int check_scan_args(const void* u, const void* delta, const void* z, const void* Bt, const void* Ct,
                    const float* A, const float* Dskip, const float* delta_bias, const void* y,
                    const float* final_state, int64_t B, int64_t D, int64_t N, int64_t L,
                    mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state, unsigned flags) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return MAMBA_ERR_DTYPE;
  if (flags & ~kKnownFlags) return MAMBA_ERR_UNSUPPORTED;
  if (!shape_ok(B, D, N, L)) return MAMBA_ERR_SHAPE;
  if (N > 16) return MAMBA_ERR_UNSUPPORTED;
  if (!u || !delta || !Bt || !Ct || !A || !y) return MAMBA_ERR_NULL;
  if (return_final_state && !final_state) return MAMBA_ERR_NULL;
  for (const void* ptr : {u, delta, z, Bt, Ct, (const void*)y})
    if (ptr && !aligned(ptr, 16)) return MAMBA_ERR_ALIGN;
  for (const void* ptr : {(const void*)A, (const void*)Dskip, (const void*)delta_bias, (const void*)final_state})
    if (ptr && !aligned(ptr, 4)) return MAMBA_ERR_ALIGN;

  return MAMBA_OK;
}

// The launches of a checked scan whose workspace holds at least plan.ws_bytes.
int scan_fwd_run(const void* u, const void* delta, const void* z, const void* Bt, const void* Ct,
                 const float* A, const float* Dskip, const float* delta_bias, void* y,
                 float* final_state, int64_t B, int64_t D, int64_t N, int64_t L,
                 mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state,
                 unsigned flags, const Plan& plan, const mamba_test_knobs_t& kn, void* workspace,
                 hipStream_t stream) {
  mamba::ScanParams p{};
  p.u = u; p.delta = delta; p.z = z; p.Bt = Bt; p.Ct = Ct;
  p.A = A; p.Dskip = Dskip; p.bias = delta_bias;
  p.y = y; p.final_state = return_final_state ? final_state : nullptr;
  p.B = B; p.D = D; p.N = N; p.L = L;
  p.tiles_d = plan.tiles_d;
  p.n_chunks = plan.n_chunks;
  p.chunk_len = plan.chunk_len;
  p.accurate = (in_dtype == MAMBA_F32) || (flags & MAMBA_FLAG_ACCURATE_EXPM1);
  p.delta_b = (flags & MAMBA_FLAG_DELTA_B) ? 1 : 0;
  p.vec = (L % 8 == 0) ? 1 : 0;
  const Dt in = in_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  const Dt out = out_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;

  mamba::V2Params q{};
  if (plan.balanced) {
    const int64_t cus = device_cus();
    if (cus <= 0) return MAMBA_ERR_HIP;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MAMBA_ERR_HIP;
    q.balanced = 1;
    q.groups = 4 * cus < kGroupsPlan ? 4 * cus : kGroupsPlan;   // one wave per SIMD
    const int64_t tiles = B * ((D + kV4Tile - 1) / kV4Tile);
    const int64_t blocks = (plan.n_chunks - 1) * tiles * (plan.chunk_len / kV4Step) +
                           tiles * ((L - (plan.n_chunks - 1) * plan.chunk_len + kV4Step - 1) / kV4Step);
    q.spin_limit = handover_spin_limit((blocks + q.groups - 1) / q.groups, kn);
    char* ws = static_cast<char*>(workspace);
    q.pub_flag = reinterpret_cast<uint64_t*>(ws + plan.off_flag);
    q.pub_state = reinterpret_cast<float*>(ws + plan.off_pub);
    if (cs == hipStreamCaptureStatusNone) {
      q.epoch = next_epoch();
    } else {
      q.epoch = kCaptureEpoch;
      if (mamba::launch_clear_u64(q.pub_flag, q.groups, stream) != hipSuccess) return MAMBA_ERR_HIP;
    }
  }
  if (plan.n_chunks > 1) {
    char* ws = static_cast<char*>(workspace);
    p.h_local = reinterpret_cast<float*>(ws + plan.off_local);
    p.h_start = reinterpret_cast<float*>(ws + plan.off_start);
    p.s_sum = reinterpret_cast<float*>(ws + plan.off_sum);
    mamba::V2Params qs = q;   // the summary pass runs one workgroup per (chunk, tile)
    qs.balanced = 0;
    const hipError_t e = plan.row ? mamba::launch_scan_row(p, in, out, false, 1, stream)
                         : plan.v4 ? mamba::launch_scan_v4(p, qs, in, out, true, stream)
                                   : mamba::launch_scan_summary(p, in, stream);
    if (e != hipSuccess) return MAMBA_ERR_HIP;
    if (mamba::launch_scan_carry(p, stream) != hipSuccess) return MAMBA_ERR_HIP;
  }
  const hipError_t e = plan.row ? mamba::launch_scan_row(p, in, out, plan.row_lean, plan.n_chunks > 1 ? 2 : 0, stream)
                       : plan.v4 ? mamba::launch_scan_v4(p, q, in, out, false, stream)
                                 : mamba::launch_scan_full(p, in, out, stream);
  if (e != hipSuccess) return MAMBA_ERR_HIP;
  return MAMBA_OK;
}


// Scratch memory of mamba_scan_fwd_noalloc: the scan's hand-over slots and
// chunk carries for callers that cannot allocate.  One copy per GPU, held
// until the process ends; every call on a GPU shares it.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy at its own address).  In host code the
// array's name is only a handle for this lookup, never an address to pass on.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

size_t mamba_scan_workspace_size(int64_t B, int64_t D, int64_t N, int64_t L) {
  if (!shape_ok(B, D, N, L) || N > 16) return (size_t)-1;
  return make_plan(B, D, N, L, knobs()).ws_bytes;
}

int mamba_scan_kernel(int64_t B, int64_t D, int64_t N, int64_t L) {
  if (!shape_ok(B, D, N, L)) return MAMBA_ERR_SHAPE;
  if (N > 16) return MAMBA_ERR_UNSUPPORTED;
  const Plan p = make_plan(B, D, N, L, knobs());
  return p.row ? (p.row_lean ? MAMBA_KERNEL_ROW_LEAN : MAMBA_KERNEL_ROW) : p.v4 ? MAMBA_KERNEL_WAVE_TILE : MAMBA_KERNEL_GENERAL;
}

int mamba_set_test_knobs(const mamba_test_knobs_t* k) {
  mamba_test_knobs_t v = {0, 0, 0, -1, 0};
  if (k) {
    if (k->scan_chunks < 0 || k->ssd_segments < 0) return MAMBA_ERR_SHAPE;
    v = *k;
  }
  std::lock_guard<std::mutex> lock(g_knob_mu);
  g_knobs = v;
  return MAMBA_OK;
}

int mamba_scan_fwd(const void* u, const void* delta, const void* z, const void* Bt, const void* Ct,
                   const float* A, const float* Dskip, const float* delta_bias, void* y,
                   float* final_state, int64_t B, int64_t D, int64_t N, int64_t L,
                   mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state,
                   unsigned flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int st = check_scan_args(u, delta, z, Bt, Ct, A, Dskip, delta_bias, y, final_state, B, D, N, L, in_dtype,
                                 out_dtype, return_final_state, flags);
  if (st != MAMBA_OK) return st;
  const mamba_test_knobs_t kn = knobs();
  const Plan plan = make_plan(B, D, N, L, kn);
  if (plan.n_chunks * B * plan.tiles_d >= (int64_t(1) << 31)) return MAMBA_ERR_SHAPE;
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return MAMBA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return MAMBA_ERR_ALIGN;
  }
  return scan_fwd_run(u, delta, z, Bt, Ct, A, Dskip, delta_bias, y, final_state, B, D, N, L, in_dtype, out_dtype,
                      return_final_state, flags, plan, kn, workspace, stream);
}

int mamba_scan_fwd_noalloc(const void* u, const void* delta, const void* z, const void* Bt, const void* Ct,
                           const float* A, const float* Dskip, const float* delta_bias, void* y,
                           float* final_state, int64_t B, int64_t D, int64_t N, int64_t L,
                           mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state,
                           unsigned flags, hipStream_t stream) {
  const int st = check_scan_args(u, delta, z, Bt, Ct, A, Dskip, delta_bias, y, final_state, B, D, N, L, in_dtype,
                                 out_dtype, return_final_state, flags);
  if (st != MAMBA_OK) return st;
  const mamba_test_knobs_t kn = knobs();
  const Plan plan = make_plan(B, D, N, L, kn);
  if (plan.n_chunks * B * plan.tiles_d >= (int64_t(1) << 31)) return MAMBA_ERR_SHAPE;
  if (plan.ws_bytes > kNoAllocScratchBytes) return MAMBA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0) {
    ws = scratch_ptr();
    if (!ws) return MAMBA_ERR_HIP;
  }
  return scan_fwd_run(u, delta, z, Bt, Ct, A, Dskip, delta_bias, y, final_state, B, D, N, L, in_dtype, out_dtype,
                      return_final_state, flags, plan, kn, ws, stream);
}

int mamba_state_update(float* state, const void* u, const void* delta, const void* z,
                       const void* Bt, const void* Ct, const float* A, const float* Dskip,
                       const float* delta_bias, void* y, int64_t B, int64_t D, int64_t N,
                       mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, unsigned flags,
                       hipStream_t stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return MAMBA_ERR_DTYPE;
  if (flags & ~kKnownFlags) return MAMBA_ERR_UNSUPPORTED;
  if (!shape_ok(B, D, N, 1)) return MAMBA_ERR_SHAPE;
  if (N > 16) return MAMBA_ERR_UNSUPPORTED;
  if (!state || !u || !delta || !Bt || !Ct || !A || !y) return MAMBA_ERR_NULL;
  if (!aligned(state, 16) || !aligned(A, 16)) return MAMBA_ERR_ALIGN;
  const size_t ea = in_dtype == MAMBA_BF16 ? 2 : 4;
  for (const void* ptr : {u, delta, z, Bt, Ct})
    if (ptr && !aligned(ptr, ea)) return MAMBA_ERR_ALIGN;
  if (!aligned(y, out_dtype == MAMBA_BF16 ? 2 : 4)) return MAMBA_ERR_ALIGN;
  for (const void* ptr : {(const void*)Dskip, (const void*)delta_bias})
    if (ptr && !aligned(ptr, 4)) return MAMBA_ERR_ALIGN;
  if ((B * D * 4 + 255) / 256 >= (int64_t(1) << 31)) return MAMBA_ERR_SHAPE;

  mamba::UpdateParams p{};
  p.state = state; p.u = u; p.delta = delta; p.z = z; p.Bt = Bt; p.Ct = Ct;
  p.A = A; p.Dskip = Dskip; p.bias = delta_bias; p.y = y;
  p.B = B; p.D = D; p.N = N;
  p.inv_d = 1.0 / (double)D;
  p.accurate = 1;   // the step is bound by state traffic: always the cancellation-free form
  p.delta_b = (flags & MAMBA_FLAG_DELTA_B) ? 1 : 0;
  const Dt in = in_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  const Dt out = out_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  return mamba::launch_state_update(p, in, out, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

size_t mamba_scan_bwd_workspace_size(int64_t B, int64_t D, int64_t N, int64_t L) {
  if (!shape_ok(B, D, N, L) || N > 16) return (size_t)-1;
  return make_bwd_plan(B, D, L).bytes;
}

int mamba_scan_bwd(const void* u, const void* delta, const void* z, const void* Bt, const void* Ct,
                   const float* A, const float* Dskip, const float* delta_bias, const void* dy,
                   void* du, void* ddelta, void* dz, float* dBt, float* dCt, float* dA, float* dDskip,
                   float* ddelta_bias, int64_t B, int64_t D, int64_t N, int64_t L,
                   mamba_dtype_t in_dtype, mamba_dtype_t grad_dtype, unsigned flags,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(grad_dtype)) return MAMBA_ERR_DTYPE;
  if (flags & ~kKnownFlags) return MAMBA_ERR_UNSUPPORTED;
  if (!shape_ok(B, D, N, L)) return MAMBA_ERR_SHAPE;
  if (N > 16) return MAMBA_ERR_UNSUPPORTED;
  if (!u || !delta || !Bt || !Ct || !A || !dy || !du || !ddelta || !dBt || !dCt || !dA || !dDskip ||
      !ddelta_bias || (z && !dz))
    return MAMBA_ERR_NULL;
  const size_t ei = in_dtype == MAMBA_BF16 ? 2 : 4, eg = grad_dtype == MAMBA_BF16 ? 2 : 4;
  for (const void* ptr : {u, delta, z, Bt, Ct})
    if (ptr && !aligned(ptr, ei)) return MAMBA_ERR_ALIGN;
  for (const void* ptr : {dy, (const void*)du, (const void*)ddelta, (const void*)dz})
    if (ptr && !aligned(ptr, eg)) return MAMBA_ERR_ALIGN;
  for (const void* ptr : {(const void*)A, (const void*)Dskip, (const void*)delta_bias, (const void*)dBt,
                          (const void*)dCt, (const void*)dA, (const void*)dDskip, (const void*)ddelta_bias})
    if (ptr && !aligned(ptr, 4)) return MAMBA_ERR_ALIGN;
  const BwdPlan plan = make_bwd_plan(B, D, L);
  if (B * plan.tiles_d * plan.S >= (int64_t(1) << 31) || (B * N * L + 255) / 256 >= (int64_t(1) << 31) ||
      (B * D * 16 + 255) / 256 >= (int64_t(1) << 31))
    return MAMBA_ERR_SHAPE;
  if (!workspace || workspace_bytes < plan.bytes) return MAMBA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MAMBA_ERR_ALIGN;

  mamba::BwdParams p{};
  p.u = u; p.delta = delta; p.z = z; p.Bt = Bt; p.Ct = Ct; p.dy = dy;
  p.A = A; p.Dskip = Dskip; p.bias = delta_bias;
  p.du = du; p.ddelta = ddelta; p.dz = z ? dz : nullptr;
  p.dBt = dBt; p.dCt = dCt; p.dA = dA; p.dDskip = dDskip; p.dbias = ddelta_bias;
  char* ws = static_cast<char*>(workspace);
  auto at = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  p.ckpt_h = at(plan.off_ckh);
  p.ckpt_cd = at(plan.off_ckd);
  p.seg_P = at(plan.off_sp);
  p.seg_h = at(plan.off_sh);
  p.seg_H = at(plan.off_sH);
  p.h_in = at(plan.off_hin);
  p.g_in = at(plan.off_gin);
  p.part_dB = at(plan.off_pb);
  p.part_dC = at(plan.off_pc);
  p.part_dA = at(plan.off_pa);
  p.part_dD = at(plan.off_pd);
  p.part_dbias = at(plan.off_pbias);
  p.B = B; p.D = D; p.N = N; p.L = L; p.tiles_d = plan.tiles_d; p.groups = plan.groups; p.nck = plan.nck;
  p.S = plan.S; p.seg_len = plan.seg_len;
  p.delta_b = (flags & MAMBA_FLAG_DELTA_B) ? 1 : 0;
  p.accurate = (flags & MAMBA_FLAG_ACCURATE_EXPM1) ? 1 : 0;
  p.vec = L % 8 == 0;
  for (const void* ptr : {u, delta, z, Bt, Ct, dy, (const void*)du, (const void*)ddelta, (const void*)dz})
    if (ptr && !aligned(ptr, 16)) p.vec = 0;
  const Dt in = in_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  const Dt gd = grad_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  return mamba::launch_scan_bwd(p, in, gd, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

}  // extern "C"

namespace {

struct SsdPlan {
  int64_t S = 1, seg_len = 0;
  size_t off_h = 0, off_P = 0, bytes = 0;
};

// Segments of L when the (batch row, head, 64-channel block) workgroups are
// fewer than 512: about 1024 workgroups in all, segments of at least 256
// steps, lengths a multiple of 32 (the chunk).  Measured at B=4, 80 heads, L =
// 2048 (chunk launch + segment-state launch): 1 segment 281 us; 2: 248 + 43;
// 3: 210 + 45; 4: 209 + 46; 6: 221 + 56; 8: 221 + 56.  With 512 or more
// workgroups the state launch costs about what the added parallelism saves.
// Test knob ssd_segments = S asks for S segments (still at most one per
// 32-step chunk), for the size query and the launch alike.
SsdPlan make_ssd_plan(int64_t B, int64_t H, int64_t P, int64_t N, int64_t L, const mamba_test_knobs_t& kn) {
  SsdPlan q;
  const int64_t wgs = B * H * (P / 64);
  int64_t S = wgs < 512 ? (1024 + wgs - 1) / wgs : 1;
  const int64_t smax = (L + 255) / 256;
  if (S > smax) S = smax;
  if (kn.ssd_segments > 0) S = (kn.ssd_segments < (L + 31) / 32) ? kn.ssd_segments : (L + 31) / 32;
  if (S < 1) S = 1;
  int64_t len = (L + S - 1) / S;
  len = (len + 31) / 32 * 32;
  q.seg_len = len;
  q.S = (L + len - 1) / len;
  if (q.S > 1) {
    const size_t slots = size_t(q.S) * size_t(wgs);   // wgs counts the batch rows
    size_t o = 0;
    q.off_h = o; o += align256(slots * 64 * size_t(N) * sizeof(float));
    q.off_P = o; o += align256(slots * sizeof(float));
    q.bytes = o;
  }
  return q;
}

}  // namespace

extern "C" {

size_t mamba_ssd_workspace_size(int64_t B, int64_t H, int64_t P, int64_t N, int64_t L) {
  if (H < 1 || P < 1 || H > kMaxElems / P || !shape_ok(B, H * P, N, L)) return (size_t)-1;
  if ((N != 64 && N != 128) || P % 64 != 0) return (size_t)-1;
  return make_ssd_plan(B, H, P, N, L, knobs()).bytes;
}

int mamba_ssd_fwd(const void* x, const void* delta, const void* z, const void* Bt, const void* Ct,
                  const float* A, const float* Dskip, const float* delta_bias, void* y, float* final_state,
                  int64_t B, int64_t H, int64_t P, int64_t N, int64_t L,
                  mamba_dtype_t in_dtype, mamba_dtype_t out_dtype, int return_final_state,
                  unsigned flags, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return MAMBA_ERR_DTYPE;
  if (flags & ~MAMBA_FLAG_DELTA_B) return MAMBA_ERR_UNSUPPORTED;
  if (H < 1 || P < 1 || H > kMaxElems / P || !shape_ok(B, H * P, N, L)) return MAMBA_ERR_SHAPE;
  if (in_dtype != MAMBA_BF16 || (N != 64 && N != 128) || P % 64 != 0) return MAMBA_ERR_UNSUPPORTED;
  if (!x || !delta || !Bt || !Ct || !A || !y || (return_final_state && !final_state)) return MAMBA_ERR_NULL;
  for (const void* ptr : {x, delta, z, Bt, Ct})
    if (ptr && !aligned(ptr, 2)) return MAMBA_ERR_ALIGN;
  if (!aligned(y, out_dtype == MAMBA_BF16 ? 2 : 4)) return MAMBA_ERR_ALIGN;
  for (const void* ptr : {(const void*)A, (const void*)Dskip, (const void*)delta_bias,
                          (const void*)(return_final_state ? final_state : nullptr)})
    if (ptr && !aligned(ptr, 4)) return MAMBA_ERR_ALIGN;
  const SsdPlan plan = make_ssd_plan(B, H, P, N, L, knobs());
  if (B * plan.S * H * (P / 64) >= (int64_t(1) << 31)) return MAMBA_ERR_SHAPE;
  if (plan.bytes && (!workspace || workspace_bytes < plan.bytes)) return MAMBA_ERR_WORKSPACE;
  if (plan.bytes && !aligned(workspace, 256)) return MAMBA_ERR_ALIGN;
  mamba::SsdParams p{};
  p.S = plan.S; p.seg_len = plan.seg_len;
  if (plan.bytes) {
    p.ws_h = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.off_h);
    p.ws_P = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.off_P);
  }
  p.x = x; p.delta = delta; p.z = z; p.Bt = Bt; p.Ct = Ct;
  p.A = A; p.Dskip = Dskip; p.bias = delta_bias;
  p.y = y; p.final_state = return_final_state ? final_state : nullptr;
  p.B = B; p.H = H; p.P = P; p.N = N; p.L = L;
  p.delta_b = (flags & MAMBA_FLAG_DELTA_B) ? 1 : 0;
  p.vec = L % 8 == 0;
  for (const void* ptr : {x, delta, z, Bt, Ct, (const void*)y})
    if (ptr && !aligned(ptr, 16)) p.vec = 0;
  const Dt out = out_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  return mamba::launch_ssd(p, out, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_conv1d_fwd(const void* x, const float* weight, const float* bias, void* y, float* final_state,
                     int64_t B, int64_t D, int64_t L, int64_t K, mamba_dtype_t in_dtype,
                     mamba_dtype_t out_dtype, int return_final_state, hipStream_t stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return MAMBA_ERR_DTYPE;
  if (!shape_ok(B, D, 1, L) || K < 1) return MAMBA_ERR_SHAPE;
  if (K > 4) return MAMBA_ERR_UNSUPPORTED;
  if (!x || !weight || !y || (return_final_state && !final_state)) return MAMBA_ERR_NULL;
  const size_t ei = in_dtype == MAMBA_BF16 ? 2 : 4, eo = out_dtype == MAMBA_BF16 ? 2 : 4;
  if (!aligned(x, ei) || !aligned(y, eo)) return MAMBA_ERR_ALIGN;
  if (!aligned(weight, 4) || (bias && !aligned(bias, 4)) || (return_final_state && !aligned(final_state, 4)))
    return MAMBA_ERR_ALIGN;
  const bool vec = (L % 8 == 0) && aligned(x, 16) && aligned(y, 16);
  if ((B * D * L + 255) / 256 >= (int64_t(1) << 31)) return MAMBA_ERR_SHAPE;   // grid of the element kernel

  mamba::ConvParams p{};
  p.x = x; p.w = weight; p.bias = bias; p.y = y;
  p.final_state = return_final_state ? final_state : nullptr;
  p.rows = B * D; p.D = D; p.L = L; p.K = K;
  const Dt in = in_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  const Dt out = out_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  return mamba::launch_conv1d_fwd(p, in, out, vec, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

int mamba_conv1d_update(float* state, const void* x, const float* weight, const float* bias, void* y,
                        int64_t B, int64_t D, int64_t K, mamba_dtype_t in_dtype, mamba_dtype_t out_dtype,
                        hipStream_t stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return MAMBA_ERR_DTYPE;
  if (!shape_ok(B, D, 1, 1) || K < 1) return MAMBA_ERR_SHAPE;
  if (K > 4) return MAMBA_ERR_UNSUPPORTED;
  if (!state || !x || !weight || !y) return MAMBA_ERR_NULL;
  const size_t ei = in_dtype == MAMBA_BF16 ? 2 : 4, eo = out_dtype == MAMBA_BF16 ? 2 : 4;
  if (!aligned(state, 4) || !aligned(x, ei) || !aligned(y, eo) || !aligned(weight, 4) || (bias && !aligned(bias, 4)))
    return MAMBA_ERR_ALIGN;
  if ((B * D + 255) / 256 >= (int64_t(1) << 31)) return MAMBA_ERR_SHAPE;

  mamba::ConvParams p{};
  p.state = state; p.x = x; p.w = weight; p.bias = bias; p.y = y;
  p.rows = B * D; p.D = D; p.L = 1; p.K = K;
  const Dt in = in_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  const Dt out = out_dtype == MAMBA_BF16 ? Dt::BF16 : Dt::F32;
  return mamba::launch_conv1d_update(p, in, out, stream) == hipSuccess ? MAMBA_OK : MAMBA_ERR_HIP;
}

const char* mamba_status_string(int status) {
  switch (status) {
    case MAMBA_OK: return "ok";
    case MAMBA_ERR_NULL: return "a required pointer is NULL";
    case MAMBA_ERR_SHAPE: return "invalid or too large shape";
    case MAMBA_ERR_DTYPE: return "unknown dtype";
    case MAMBA_ERR_ALIGN: return "pointer is not sufficiently aligned";
    case MAMBA_ERR_UNSUPPORTED: return "unsupported argument (N > 16 or unknown flag)";
    case MAMBA_ERR_WORKSPACE: return "workspace missing or too small";
    case MAMBA_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"

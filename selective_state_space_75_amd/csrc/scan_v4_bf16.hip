// scan_v4_bf16.hip -- the main scan kernel instantiated for bf16 inputs, and
// the dispatcher over input dtypes.
#include "scan_v4.hpp"

namespace mamba {

hipError_t launch_scan_v4_bf16in(const ScanParams& p, const V2Params& q, Dt out, bool summary, hipStream_t s) {
  if (summary) return launch_t<true, false, true>(p, q, s);
  return out == Dt::BF16 ? launch_t<true, true, false>(p, q, s) : launch_t<true, false, false>(p, q, s);
}

hipError_t launch_scan_v4(const ScanParams& p, const V2Params& q, Dt in, Dt out, bool summary, hipStream_t s) {
  return in == Dt::BF16 ? launch_scan_v4_bf16in(p, q, out, summary, s) : launch_scan_v4_f32in(p, q, out, summary, s);
}

}  // namespace mamba

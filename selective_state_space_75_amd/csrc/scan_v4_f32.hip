// scan_v4_f32.hip -- the main scan kernel instantiated for fp32 inputs.
#include "scan_v4.hpp"

namespace mamba {

hipError_t launch_scan_v4_f32in(const ScanParams& p, const V2Params& q, Dt out, bool summary, hipStream_t s) {
  if (summary) return launch_t<false, false, true>(p, q, s);
  return out == Dt::BF16 ? launch_t<false, true, false>(p, q, s) : launch_t<false, false, false>(p, q, s);
}

}  // namespace mamba

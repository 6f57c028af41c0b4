// Prefill GEMMs (bf16 MFMA).  Not built yet: the regime reports itself unavailable.
#include "lb_prefill.h"

namespace lb {

size_t prefill_layer_bytes(int64_t, int64_t, const lb_path*, int) { return 0; }
hipError_t prefill_layer_build(PrefillLayer& out, void*, size_t, int64_t m, int64_t n, const PathDev*, int np,
                               hipStream_t) {
  out.m = (int)m; out.n = (int)n; out.np = np; out.ready = 0;
  return hipSuccess;
}
bool prefill_available() { return false; }
hipError_t prefill_prepare(PrefillPlan&, const PrefillLayer* const*, int, int) { return hipErrorNotSupported; }
hipError_t prefill_run(PrefillPlan&, const PrefillLayer* const*, int, const void* const*, void* const*, int,
                       hipStream_t, bool) {
  return hipErrorNotSupported;
}
void prefill_plan_release(PrefillPlan& P) { P.T = -1; P.count = 0; }

}  // namespace lb

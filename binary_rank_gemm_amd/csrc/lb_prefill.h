// Prefill (many tokens, bf16 I/O) layouts and launch plans.
#pragma once

#include "lb_internal.h"

namespace lb {

// Per-linear device data of the prefill GEMMs (carved from the linear's arena).
struct PrefillLayer {
  int m = 0, n = 0, np = 0;
  int ready = 0;           // nonzero once built
};

// Launch plan of the prefill kernels for a list of linears at T tokens.
struct PrefillPlan {
  int T = -1;
  int count = 0;
};

size_t prefill_layer_bytes(int64_t m, int64_t n, const lb_path* paths, int np);
hipError_t prefill_layer_build(PrefillLayer& out, void* mem, size_t bytes, int64_t m, int64_t n,
                               const PathDev* paths, int np, hipStream_t st);
bool prefill_available();
hipError_t prefill_prepare(PrefillPlan& P, const PrefillLayer* const* layers, int count, int T);
hipError_t prefill_run(PrefillPlan& P, const PrefillLayer* const* layers, int count, const void* const* xs,
                       void* const* ys, int T, hipStream_t st, bool sync_on_rebuild);
void prefill_plan_release(PrefillPlan& P);

}  // namespace lb

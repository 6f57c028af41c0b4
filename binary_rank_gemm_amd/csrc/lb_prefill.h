// Prefill (many tokens, bf16 I/O): two bf16 MFMA GEMMs per linear.
//   GEMM1: Z'[T][Rp] = (x . B1) o l',  B1[k][j] = s_kj |g_p(j)[k]|  (paths concatenated along j)
//   GEMM2: y[T][m]   = Z' . B2,        B2[j][i] = u_ij |h_p(j)[i]|
// Signs of g and h are folded into the stored sign bits at build time.
#pragma once

#include <vector>

#include "lb_internal.h"

namespace lb {

constexpr int kPreBM = 256, kPreBN = 256, kPreBK = 64;   // workgroup tile
constexpr int kPreWN = 128;                              // wave tile (N) = B tile width in the layouts

// Per-linear device data of the prefill GEMMs (carved from the linear's arena).
struct PrefillLayer {
  int m = 0, n = 0, np = 0;
  int rp[2] = {0, 0};        // per-path rank padded to 32
  int roff[2] = {0, 0};      // first concatenated latent of each path
  int Rp = 0;                // concatenated, padded to kPreBK
  int nt1 = 0, kb1 = 0;      // GEMM1 B: 128-column tiles x 64-row K blocks
  int nt2 = 0, kb2 = 0;      // GEMM2 B
  const uint32_t* b1 = nullptr;    // [nt1][kb1][64 lanes][4] sign words
  const uint32_t* b2 = nullptr;    // [nt2][kb2][64 lanes][4]
  const uint16_t* gabs = nullptr;  // [2][kb1 * 64] bf16 |g_p|
  const uint16_t* habs = nullptr;  // [2][nt2 * 128] bf16 |h_p|
  const float* lpad = nullptr;     // [Rp] l for real latents, 0 for padding
};

// Device descriptor of one prefill entry.
struct PreEntry {
  PrefillLayer L;
  const void* x;
  void* y;
  uint16_t* z;               // Z' scratch [T][Rp] bf16
};

struct PreItem {
  int entry;                 // < 0: idle slot
  int mt, nt;
  int str;                   // GEMM1: a wave's columns reach into both paths
};

// Launch plan of the prefill kernels for a list of linears at T tokens.
struct PrefillPlan {
  int T = -1;
  int count = 0;
  PreEntry* entries_d = nullptr;
  PreItem* items_d = nullptr;       // GEMM1 items (full row stripes, then the partial one), then GEMM2's
  int n1 = 0, n1p = 0, n2 = 0, n2p = 0;
  void* zbuf = nullptr;
  size_t zbytes = 0;
  std::vector<PreEntry> entries_h;
};

size_t prefill_layer_bytes(int64_t m, int64_t n, const lb_path* paths, int np);
hipError_t prefill_layer_build(PrefillLayer& out, void* mem, size_t bytes, int64_t m, int64_t n,
                               const PathDev* paths, int np, hipStream_t st);
bool prefill_available();
// Builds the plan for `count` linears at T tokens; xs / ys (host arrays of
// device pointers, or null) are stored in the device entries.  Synchronous.
hipError_t prefill_prepare(PrefillPlan& P, const PrefillLayer* const* layers, int count, int T,
                           const void* const* xs, void* const* ys);
// Launches GEMM1 and GEMM2.  single: one linear whose x / y go as kernel
// arguments (the plan is rebuilt here when T changes); otherwise the plan
// must have been prepared for these pointers and T.
hipError_t prefill_run(PrefillPlan& P, const PrefillLayer* const* layers, int count, const void* const* xs,
                       void* const* ys, int T, int yf32, hipStream_t st, bool single);
void prefill_plan_release(PrefillPlan& P);

}  // namespace lb

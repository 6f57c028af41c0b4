// Prefill (many tokens, bf16 I/O): two bf16 MFMA GEMMs per linear.
//   GEMM1: Z'[T][Rp] = (x . B1) o l',  B1[k][j] = s_kj |g_p(j)[k]|  (paths concatenated along j)
//   GEMM2: y[T][m]   = Z' . B2,        B2[j][i] = u_ij |h_p(j)[i]|
// Signs of g and h are folded into the stored sign bits at build time.
#pragma once

#include <vector>

#include "lb_internal.h"

namespace lb {

constexpr int kPreBM = 256, kPreBN = 256, kPreBK = 64;   // workgroup tile (rows: kPreBM, 128 or 64)
// Rows per tile of a forward at T tokens: 64-row tiles up to 64 tokens,
// 128-row tiles up to kPreSmallMaxTokens and from 256 tokens on, 256-row tiles
// in between (a 128-row stripe that runs past the last token costs about as
// much as a whole one, so 129 to 255 tokens take one 256-row stripe; measured
// on the Llama-2-13B and Llama-3-8B shapes).
constexpr int kPreSmallMaxTokens = 128;
// GEMM1 K parts.  With one row stripe (T tokens fit one tile's rows) a
// long-K linear has few GEMM1 tiles, each running all of K; when they are
// much longer than the launch's work per workgroup slot they alone set its
// length (the Llama-3-8B down projection at 16 tokens: 224 K blocks against
// 79 per slot).  Such a linear's GEMM1 is cut into K parts, summed by a
// second launch.  The cut depends on the launch, so a linear cut in a stack
// may be whole when run alone: the two then add in different orders.
constexpr int kPreSplitBlocks = 128;
inline int prefill_rows_per_tile(int T) {
  return T <= 64 ? 64 : (T <= kPreSmallMaxTokens || T >= 2 * kPreSmallMaxTokens) ? 128 : kPreBM;
}
// Workgroups of the prefill GEMMs resident at once (64-row tiles: three per
// CU, 128-row tiles two, 256-row one) on 256 CUs.
inline int prefill_slots(int T) {
  const int bm = prefill_rows_per_tile(T);
  return 256 * (bm == 64 ? 3 : bm < kPreBM ? 2 : 1);
}
// K parts of GEMM1 for a linear with kb1 K blocks at T tokens (1: not cut),
// in a GEMM1 launch whose whole-width tiles add up to `blocks` K blocks: cut
// when kb1 exceeds both kPreSplitBlocks and twice the blocks per slot, into
// parts of about the larger of kPreSplitBlocks and the blocks per slot.
inline int prefill_k_parts(int kb1, int T, double blocks) {
  const double per_slot = blocks / prefill_slots(T);
  if (T > prefill_rows_per_tile(T) || kb1 <= kPreSplitBlocks || kb1 <= 2.0 * per_slot) return 1;
  const double part = per_slot > kPreSplitBlocks ? per_slot : (double)kPreSplitBlocks;
  return (int)((kb1 + part - 1) / part);
}
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
  float* zpart;              // GEMM1 cut into K parts: fp32 partial sums [nks][T][Rp] (else null)
  int nks;                   // GEMM1 K parts (prefill_k_parts; 1: whole K per tile)
};

struct PreItem {
  int entry;                 // < 0: idle slot
  int mt, nt;
  int str;                   // GEMM1: a wave's columns reach into both paths
  int tn;                    // tile width: 256, or 128 / 64 for a narrow last column tile
  int ks;                    // GEMM1: the K part this item multiplies (0 when K is not cut)
};

// Work of the launch that adds the K parts of cut GEMM1s: 1024 Z' outputs
// (row-major [T][Rp]) of one entry from e0 on per workgroup.
struct PreComb {
  int entry, e0;
};

// Launch plan of the prefill kernels for a list of linears at T tokens.
struct PrefillPlan {
  int T = -1;
  int count = 0;
  PreEntry* entries_d = nullptr;
  PreItem* items_d = nullptr;       // GEMM1 items (full row stripes, then the partial one), then GEMM2's
  int n1 = 0, n1p = 0, n2 = 0, n2p = 0;
  int bm = kPreBM;                  // rows per tile (prefill_rows_per_tile(T))
  void* zbuf = nullptr;
  size_t zbytes = 0;
  PreComb* comb_d = nullptr;        // K-part sums (ncomb workgroups), between GEMM1 and GEMM2
  int ncomb = 0;
  void* pbuf = nullptr;             // fp32 partial sums of cut GEMM1s
  size_t pbytes = 0;
  std::vector<PreEntry> entries_h;
};

size_t prefill_layer_bytes(int64_t m, int64_t n, const lb_path* paths, int np);
hipError_t prefill_layer_build(PrefillLayer& out, void* mem, size_t bytes, int64_t m, int64_t n,
                               const PathDev* paths, int np, hipStream_t st);
bool prefill_available();
// K blocks of the whole-width GEMM1 tiles of these linears at T tokens (the
// launch's work for prefill_k_parts).
double prefill_gemm1_blocks(const PrefillLayer* const* layers, int count, int T);
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

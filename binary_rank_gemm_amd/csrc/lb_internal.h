// Internal declarations shared by the host API and the HIP kernels.
// Nothing here is part of the public ABI (include/littlebit.h).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "littlebit.h"

namespace lb {

// ---------------------------------------------------------------------------
// Geometry of the decode layouts (fp8 x fp4 MFMA, 16x16x128).
//   V (per path): [kc = n/128 chunks][ct = r/16 column tiles][64 lanes] uint32.
//     Lane l of tile (kc, ct) holds column j = 16 ct + l%16 and the 32 rows
//     k = 128 kc + 32 (l/16) + e, e = 8 v + q (v = 0..3, q = 0..7), with the
//     sign of row k at bit 4 q + 3 - v (bit set <=> -1).
//   U: [rt = m/16 row tiles][path][w = 0..W_p-1][16 rows] uint32, where word w
//     of output row i is canonical word w of that row with its bits permuted
//     the same way (latent j = 32 w + e at bit 4 q + 3 - v).
// ---------------------------------------------------------------------------
constexpr int kChunk = 128;   // K extent of one MFMA
constexpr int kTile = 16;     // M/N extent of one MFMA

__host__ __device__ inline int fp4_bit_of_elem(int e) { return 4 * (e & 7) + 3 - (e >> 3); }

// Per-path device pointers of a linear (library-owned).
struct PathDev {
  const uint32_t* u_can;   // [m][W] canonical
  const uint32_t* v_can;   // [n][W] canonical
  const uint16_t* h;       // [m] fp16
  const uint16_t* g;       // [n] fp16
  const uint16_t* l;       // [r] fp16
  const uint32_t* vdec;    // decode V layout
  int r, W, nct;
};

// One entry of a decode / exact launch: a linear plus its activations.
struct DecEntry {
  PathDev p[2];
  const uint32_t* udec;    // decode U layout, both paths
  float* zbuf;             // scratch [np][T][rpad] of z' = (x o g) V o l
  int m, n, np, nkc, nrt, rpad, uw;   // uw = sum_p W_p (words per row, U layout)
  int nv;                  // number of V work items of this entry
  int vct[2];              // column tiles per V work item, per path
  int woff[2];             // word offset of each path inside a U-layout row
};

// Work item of the decode kernel: kind 0 = V stage (entry, path, column group),
// kind 1 = U stage (entry, row group).
struct WorkItem {
  uint32_t entry;
  uint16_t kind_path;      // bit 15: kind, bits 0..14: path
  uint16_t group;
};

// Control words of one persistent launch (zero-initialised once, self-resetting).
struct Control {
  unsigned int ticket;     // next work item
  unsigned int done;       // workgroups finished
  unsigned int gen;        // launches completed
  unsigned int err;        // nonzero if a bounded wait gave up (never expected)
};

// Launch-wide arguments of the decode kernel.
struct DecArgs {
  const DecEntry* entries;
  const void* const* xs;   // per entry input (device array), or null: use x0 / y0
  void* const* ys;         // per entry output
  const void* x0;          // single-entry input when xs is null
  void* y0;
  const WorkItem* items;
  unsigned int* counters;  // per entry V-completion counter
  unsigned int* ready;     // per entry generation flag
  Control* ctl;
  int nitems, T, t0;       // tokens in this launch and the offset of its first token
  int spin_limit;          // polls before a wait gives up (sets ctl->err)
};

// Tokens one decode launch handles (token blocks of 8, at most 2 blocks).
constexpr int kDecodeMaxTokens = 16;
constexpr int kDecodeRowTilesPerItem = 16;   // U work item = 256 output rows
__host__ __device__ inline int decode_ct_max(int tb) { return tb == 1 ? 16 : 8; }

// ---------------------------------------------------------------------------
// kernel launchers (defined in the .hip files)
// ---------------------------------------------------------------------------
hipError_t launch_validate_signs(const int8_t* s, int64_t count, int* bad_flag, hipStream_t st);
hipError_t launch_pack_signs(const int8_t* s, int64_t rows, int64_t rank, uint32_t* out, hipStream_t st);
hipError_t launch_unpack_signs(const uint32_t* w, int64_t rows, int64_t rank, int8_t* out, hipStream_t st);
hipError_t launch_retile_v_decode(const uint32_t* vcan, int n, int r, uint32_t* vdec, hipStream_t st);
hipError_t launch_retile_u_decode(const uint32_t* ucan, int m, int r, int W, int uw, int woff,
                                  uint32_t* udec, hipStream_t st);

// fp32 exact path: z' then y, one linear
hipError_t launch_exact(const PathDev* p, int np, int m, int n, const void* x, void* y, int T,
                        int io_fp32, float* zbuf, int rpad, hipStream_t st);

// decode path: persistent fused kernel over a work list
hipError_t launch_decode(const DecArgs& a, int tb, hipStream_t st);
int decode_grid_size(int tb);

}  // namespace lb

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

// One entry of a decode launch: a linear plus its activations.
struct DecEntry {
  PathDev p[2];
  const uint32_t* udec;    // decode U layout, both paths
  uint8_t* aimg;           // U-stage fp8 A operand images [npc][tb][kABytes], written by the V stage
  float* cpart;            // U-stage C partial sums [np][kMaxGroups][16], written by the V stage
  int m, n, np, nkc, nrt, uw;   // uw = sum_p W_p (words per row, U layout)
  int vct[2];              // column tiles per V work item, per path
  int nvg[2];              // V work items (column groups) per path
  int woff[2];             // word offset of each path inside a U-layout row
  int pcoff[2];            // first 128-latent chunk of each path in aimg
  int npc;                 // chunks over both paths
};

constexpr int kMaxGroups = 32;          // column groups per path (rank <= 4096, >= 8 tiles per group)
constexpr int kABytes = 2048 + 64;      // one fp8 A operand image: 16 rows x 4 groups x 32 B + scales

// Work item: V stage (entry, path, column group) or U stage (entry, 16 row tiles).
struct WorkItem {
  uint32_t entry;
  uint16_t path;
  uint16_t group;
};

constexpr int kWavesPerGroup = 4;   // waves of a decode workgroup

// U-stage work item: a contiguous run of `count` quads (4 row tiles each) of the
// concatenated entries, starting at quad `quad0` of entry `entry`.
struct UItem {
  uint32_t entry, quad0, count, pad;
};

// Launch-wide arguments of the two decode kernels.
struct DecArgs {
  const DecEntry* entries;
  const void* const* xs;   // per entry input (device array), or null: use x0 / y0
  void* const* ys;         // per entry output
  const void* x0;          // single-entry input when xs is null
  void* y0;
  const WorkItem* items;   // V items, one workgroup each
  const UItem* uitems;     // U items, one workgroup each
  uint16_t* sink;          // write target of output lanes that hold no output (256 B per U wave)
  int nentries;
  int T, t0;               // tokens in this launch and the offset of its first token
};

// Tokens one decode launch handles (token blocks of 8, at most 2 blocks).
constexpr int kDecodeMaxTokens = 16;
constexpr int kDecodeRowTilesPerItem = 64;   // U work item = 1024 output rows
// U work items: batches of quads (4 row tiles); a batch is 4 quads per wave (2
// at 16 tokens) and an item holds kDecodeUBatches batches of all 4 waves
constexpr int kDecodeUBatches = 1;
__host__ __device__ constexpr int decode_u_quads_per_item(int bucket) { return bucket >= 16 ? 8 : 16; }
__host__ __device__ constexpr int decode_u_item_quads(int bucket) { return decode_u_quads_per_item(bucket) * kDecodeUBatches; }
constexpr int kDmaPad = 1024;                // slack after buffers read by 1 KB direct-to-LDS loads
// bytes of the decode U layout: quads of 4 row tiles x uw words x 16 rows x 4 B, plus slack
__host__ __device__ inline size_t decode_u_bytes(int nrt, int uw) {
  return (size_t)((nrt + 3) / 4) * uw * 256 + kDmaPad;
}
// Token-count bucket of a decode launch (per-token state is sized by it) and the
// most column tiles one V work item holds at that bucket.
__host__ __device__ inline int decode_bucket(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : T <= 8 ? 8 : 16; }
__host__ __device__ inline int decode_ct_max(int T) { return decode_bucket(T) >= 8 ? 8 : 16; }

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

// decode path: V-stage kernel then U-stage kernel, one workgroup per work item
hipError_t launch_decode_v(const DecArgs& a, int nitems, hipStream_t st);
hipError_t launch_decode_u(const DecArgs& a, int nitems, size_t lds_bytes, hipStream_t st);
// Workgroups of the U-stage kernel that run at once on the current device, and
// U items per such slot (several, so that slots that stream faster take more).
int decode_u_slots();
constexpr int kDecodeUItemsPerSlot = 1;
// LDS bytes of a U-stage launch over entries with npc[e] 128-latent units each
size_t decode_u_lds_bytes(const int* npc, int count, int T);

}  // namespace lb

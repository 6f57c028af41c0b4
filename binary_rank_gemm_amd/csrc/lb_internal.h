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
//   U: see UGeom; word w of output row i is canonical word w of that row
//     with its bits permuted the same way (latent j = 32 w + e at bit 4 q + 3 - v).
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

constexpr int kABytes = 2048 + 64;      // one fp8 A operand image: 16 rows x 4 groups x 32 B + scales
constexpr int kDmaPad = 1024;           // slack after buffers read by 1 KB direct-to-LDS loads

// Decode U layout of one linear: quads of 64 output rows; inside a quad, each
// path's 128-latent units in order, 1 KB each ([4 words][16 rows][4 row tiles]
// uint32, so that lane 16 w + row of a 64-lane load gets the four row tiles'
// word w), except that the last unit of a path is 512 B (words 0 and 1 only)
// when the path's rank leaves at most 64 latents in it.
struct UGeom {
  int nq;            // quads
  int nu0, nu;       // units of path 0; units of both paths
  int half0, half1;  // the last unit of path 0 / path 1 is a half unit
  int uoff1;         // byte offset of path 1's first unit inside a quad
  int qbytes;        // bytes of one quad
};
inline UGeom u_geom(int64_t m, const int64_t* r, int np) {
  UGeom g{};
  g.nq = (int)((m + 63) / 64);
  int bytes[2] = {0, 0}, nu[2] = {0, 0}, half[2] = {0, 0};
  for (int p = 0; p < np; ++p) {
    nu[p] = (int)((r[p] + kChunk - 1) / kChunk);
    const int rem = (int)(r[p] % kChunk);
    half[p] = rem != 0 && rem <= kChunk / 2;
    bytes[p] = nu[p] * 1024 - half[p] * 512;
  }
  g.nu0 = nu[0];
  g.nu = nu[0] + nu[1];
  g.half0 = half[0];
  g.half1 = half[1];
  g.uoff1 = bytes[0];
  g.qbytes = bytes[0] + bytes[1];
  return g;
}
inline size_t decode_u_bytes(const UGeom& g) { return (size_t)g.nq * g.qbytes + kDmaPad; }
// row scales of both paths per quad: [quad][path][64 rows] fp16
inline size_t decode_h_bytes(const UGeom& g) { return (size_t)g.nq * 256 + kDmaPad; }

// One entry of a decode launch: a linear plus its activations.
struct DecEntry {
  PathDev p[2];
  const uint16_t* gdec[2];   // g of each path, zero-padded to whole 128-row chunks
  const uint8_t* udec;       // decode U layout (UGeom)
  const uint16_t* hq;        // row scales per quad
  uint8_t* aimg;             // U-stage fp8 A operands [unit][tb][kABytes] (written by the mid kernel)
  float* cval;               // U-stage correction sums [path][16 tokens] (written by the mid kernel)
  int m, n, np, nkc;
  int xdirect;               // n % 8 == 0: rows of x are read with 16-byte loads
  UGeom ug;
};

// V-stage work item (one workgroup): column tiles [tile0, tile0 + ntiles) of
// one path over chunks [c0, c1) of 128 input rows; its partial sums go to
// partial slot `slot`; `mid` is the index of its (entry, path)'s mid item.
struct VItem {
  int entry, path, tile0, ntiles, c0, c1, slot, mid;
};
// Mid-stage work item (one workgroup): one path of one entry; its V items are
// `ngroups` column groups of `gtiles` tiles, each split into `nsplit` chunk
// ranges, with partial slots slot0 + group * nsplit + split.
struct MItem {
  int entry, path, slot0, ngroups, nsplit, gtiles, pad0, pad1;
};
// U-stage work item (one workgroup): quads [q0, q0 + nq) of one entry, qw
// consecutive quads per wave.
struct UItem {
  int entry, q0, nq, qw;
};

constexpr int kWavesPerGroup = 4;   // waves of a decode workgroup

// Launch-wide arguments of the decode kernels.
struct DecArgs {
  const DecEntry* entries;
  const void* const* xs;   // per entry input (device array), or null: use x0 / y0
  void* const* ys;         // per entry output
  const void* x0;          // single-entry input when xs is null
  void* y0;
  const VItem* vitems;
  const MItem* mitems;
  const UItem* uitems;
  float* part;             // V-stage partial sums, decode_slot_floats(bucket) per slot
  int T, t0;               // tokens in this launch and the offset of its first token
  int bucket;              // token bucket the plan was built for (T <= bucket): selects the kernels
  int yf32;                // y is fp32 (else bf16)
};

// Tokens one decode launch handles (token blocks of 8, at most 2 blocks).
constexpr int kDecodeMaxTokens = 16;
// Token-count bucket of a decode launch (per-token state is sized by it).
__host__ __device__ inline constexpr int decode_bucket(int T) {
  return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : T <= 8 ? 8 : 16;
}
// Column tiles of one V item (20 at every bucket: at 16 tokens the V
// workgroups then hold more registers and two fit a CU, but a 205-rank path
// stays one column group, so x is read once per path), and the floats of one
// partial slot: [tile][token][16 columns] sums, then 16 correction sums.
__host__ __device__ inline constexpr int decode_v_tiles(int bucket) { return 20; }
__host__ __device__ inline constexpr int decode_slot_floats(int bucket) {
  return decode_v_tiles(bucket) * 16 * bucket + 16;
}
// Most quads per wave of a U item at a token bucket.  The wave stages all of
// its outputs in LDS: 3 KB from 2 to 8 tokens, so that three workgroups of
// ring and staging (52 KB each) still fit a CU's 160 KB (fewer quads per item
// would make the A-operand prologue as large as the stream: at 8 tokens and 2
// quads a wave of a gate projection loaded 12 KB of operands for 11 KB of
// signs; 3 quads took the Llama-2-70B stack from 280 to 273 us, 4 tokens 225
// to 221); 2 KB at one token, where the items are not limited by it and the
// larger allocation measured 1 % slower; 8 KB at 16 tokens, where two fit a CU.
__host__ __device__ inline constexpr int decode_u_qw_max(int bucket) {
  return bucket >= 16 ? 4 : bucket == 1 ? 16 : 24 / bucket;
}
// Sizes the planner aims at per V and U work item (bytes of sign words).
// From 4 tokens on a V item's partial slot is large (20 KB at 16 tokens), so
// fewer, larger items pay: measured on the Llama-2-70B stack, 384 KB items
// take 2-4 % off the launches of 4, 8 and 16 tokens and add 2 % at one token.
// At one token, where four V workgroups fit a CU, 144 KB measured 0.5 % faster
// than 192 (96, 128 and 256 KB slower).
__host__ __device__ inline constexpr int decode_v_item_bytes(int bucket) {
  return bucket >= 4 ? 384 * 1024 : bucket == 1 ? 144 * 1024 : 192 * 1024;
}
// U items of 288 KB (capped from 4 tokens by the quads a wave can stage):
// with four V workgroups per CU at one token, 288 KB measured 1-2 % faster than
// 192 at one and two tokens (144 and 384 KB slower).
constexpr int kDecodeUItemBytes = 288 * 1024;
// U units (128 latents of both paths together) a U wave holds in registers in
// the fast form: 8 up to 8 tokens, 6 at 16 tokens (two workgroups per CU).
// At 16 tokens, entries of 7 or 8 units run in a second U launch whose
// workgroups hold 8 (one workgroup per CU: the registers of 8 units' operands
// for two token blocks); more units take the plain form.
__host__ __device__ inline constexpr int decode_u_fast_units(int bucket) { return bucket > 8 ? 6 : 8; }
constexpr int kDecodeWideUnits = 8;
__host__ __device__ inline constexpr bool decode_u_wide(int bucket, int nu) {
  return bucket > 8 && nu > decode_u_fast_units(bucket) && nu <= kDecodeWideUnits;
}

// ---------------------------------------------------------------------------
// kernel launchers (defined in the .hip files)
// ---------------------------------------------------------------------------
hipError_t launch_validate_signs(const int8_t* s, int64_t count, int* bad_flag, hipStream_t st);
hipError_t launch_pack_signs(const int8_t* s, int64_t rows, int64_t rank, uint32_t* out, hipStream_t st);
hipError_t launch_unpack_signs(const uint32_t* w, int64_t rows, int64_t rank, int8_t* out, hipStream_t st);
hipError_t launch_retile_v_decode(const uint32_t* vcan, int n, int r, uint32_t* vdec, hipStream_t st);

// fp32 exact path: z' then y, one linear
// K splits of the exact path's z stage: when tokens are few, the rows of V
// are cut into up to 64 ranges (at least 256 rows each) so the launch has
// about 512 workgroups.
inline int exact_splits(int rmax, int np, int64_t T, int n) {
  const int64_t blocks = (int64_t)((rmax + 63) / 64) * np * T;
  if (blocks >= 512) return 1;
  const int64_t want = (512 + blocks - 1) / blocks;
  const int64_t most = n / 256 < 1 ? 1 : (n / 256 > 64 ? 64 : n / 256);
  return (int)(want < most ? want : most);
}
// fp32 I/O with at least this many tokens runs the exact path's tiled form:
// two fp32 matrix-core contractions (lb_f32gemm.hip) instead of the per-token
// vector kernels.
constexpr int kF32GemmMinTokens = 16;
inline bool exact_uses_gemm(int64_t T, int x_fp32, int y_fp32) {
  return x_fp32 && y_fp32 && T >= kF32GemmMinTokens;
}
// Floats of Z' scratch of the tiled form: T x (r_p rounded up to 32), per path.
size_t f32_gemm_scratch_floats(const PathDev* p, int np, int64_t T);
hipError_t launch_f32_gemm(const PathDev* p, int np, int m, int n, const float* x, float* y, int T, float* zbuf,
                           hipStream_t st);
// Floats of scratch the exact path needs for one linear: the tiled form's Z',
// or splits x np x T x rpad latent sums of the vector kernels (rpad = the
// largest rank rounded up to 16).
inline size_t exact_scratch_floats(const PathDev* p, int np, int64_t T, int n, int x_fp32, int y_fp32) {
  if (exact_uses_gemm(T, x_fp32, y_fp32)) return f32_gemm_scratch_floats(p, np, T);
  int rmax = 0;
  for (int i = 0; i < np; ++i) rmax = rmax > p[i].r ? rmax : p[i].r;
  return (size_t)exact_splits(rmax, np, T, n) * np * T * ((rmax + 15) / 16 * 16);
}
// the exact path (either form, chosen by exact_uses_gemm)
hipError_t launch_exact(const PathDev* p, int np, int m, int n, const void* x, void* y, int T,
                        int x_fp32, int y_fp32, float* zbuf, hipStream_t st);

// decode path: V stage, mid stage, U stage, one workgroup per work item
hipError_t launch_decode_v(const DecArgs& a, int nitems, hipStream_t st);
hipError_t launch_decode_mid(const DecArgs& a, int nitems, hipStream_t st);
hipError_t launch_decode_u(const DecArgs& a, int nitems, hipStream_t st);
// the second U launch of a 16-token decode: entries with decode_u_wide
hipError_t launch_decode_u_wide(const DecArgs& a, int nitems, hipStream_t st);

// Persistent chained decode: one launch runs the levels of a chained stack in
// order, on the compute units of one XCD (hand-overs through its L2), each
// level a V phase (whose last V item of every (entry, path) runs that pair's
// mid step) and a U phase, with a barrier of the participating workgroups
// after each phase.  Every level has its own plan (tables and buffers),
// planned for the participants.
struct ChainLevel {
  DecArgs a;
  int nv, nm, nu, moff;    // items of the three stages; first counter of this level's mid items
};
// Synchronisation words (uint64, one per 128 bytes): launch epoch, abort flag,
// barrier counter, rank tickets; the mid items' arrival counters follow, one
// per 64 bytes.
constexpr int kChainEpoch = 0, kChainAbort = 16, kChainBar = 32, kChainTicket = 48;
constexpr int kChainCnt = 64;                                        // first mid counter (uint64 index)
constexpr int kChainCntStride = 8;                                   // uint64 per mid counter
inline size_t chain_sync_bytes(int mid_items) { return ((size_t)kChainCnt + (size_t)kChainCntStride * mid_items) * 8; }
struct ChainArgs {
  const ChainLevel* levels;
  uint64_t* sync;          // chain_sync_bytes, zero before the first launch of a plan
  int nlev;
  int stall;               // 1: the first barrier waits for one arrival more (abort-path tests)
};
// Entries the persistent kernel takes (x rows read with 16-byte loads, U units
// within the fast form) at a token bucket.
bool decode_chain_takes(const DecEntry& e, int bucket);
// Workgroups of the persistent kernel's launch at this token bucket (all
// resident at once: occupancy x compute units), or 0 when the device cannot
// run it; of these, decode_chain_participants(grid) do the work (those on
// XCD 0: the grid is a multiple of the 8 XCDs, which take workgroups in
// turn), and the plans are made for that many work-item slots.
int decode_chain_grid(int bucket, int device);
int decode_chain_participants(int grid);
hipError_t launch_decode_chain(const ChainArgs& c, int bucket, int grid, hipStream_t st);
// layouts of the decode U stage (built once per linear)
hipError_t launch_decode_u_layout(const uint32_t* ucan0, const uint32_t* ucan1, int m, const int* W, const UGeom& g,
                                  uint8_t* udec, hipStream_t st);
// Dual-SVID initialisation: per path, caller-owned device outputs in the
// interchange form of lb_linear_create's inputs
struct InitPathOut {
  uint32_t* u_packed;
  uint32_t* v_packed;
  uint16_t* h;
  uint16_t* g;
  uint16_t* l;
};
// W row-major [m][n] fp32 on the device; synchronous on st.  rocstatus: the
// rocBLAS / rocSOLVER status when one of their calls failed, else 0.
hipError_t dual_svid_init(const float* W, int64_t m, int64_t n, const int64_t* ranks, int np, const InitPathOut* out,
                          hipStream_t st, int* rocstatus);
// Bytes of the fixed per-device scratch of the no-allocation forward, and its
// device address on `device` (looked up on the first call for that device,
// which must then be current; later calls return the kept address).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
hipError_t noalloc_scratch(int device, void** ptr);
// calibration: one read-only streaming pass over a device buffer
hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, hipStream_t st);
hipError_t launch_decode_h_layout(const uint16_t* h0, const uint16_t* h1, int m, int nq, uint16_t* hq,
                                  hipStream_t st);

}  // namespace lb

// Prefill forward (many tokens, bf16 I/O): the factorised order of the paper
// notes ("LittleBit: Ultra Low-Bit Quantization via Latent Factorization",
// section "Key design": element-wise scales around binary matrix products)
// computed as two dense contractions on bf16 MFMA with fp32 accumulation:
//
//   GEMM1  Z'[T][Rp] = (x . B1) o l'     B1[k][j] = s_kj |g_p(j)[k]|, j over both paths
//   GEMM2  y [T][m]  = Z' . B2           B2[j][i] = u_ij |h_p(j)[i]|
//
// (section "Residual compensation": the two paths are simply concatenated
// along the latent axis, each padded to 32 with zero l so padding contributes
// nothing).  The signs of g and h are folded into the stored sign bits, so a
// B operand pair is one shift and one bit-field insert of the sign bits into
// a bf16 pair of magnitudes.
//
// Workgroup tile 256 x 256 (8 waves of 128 x 64, two per SIMD, 32x32x16
// MFMA, fp32 accumulators in AGPRs), K blocks of 64.  A, the packed B words and |g| go
// from global memory straight into LDS (four buffers, loads issued three
// blocks ahead; A rows unpadded with an XOR swizzle of their 16-byte chunks
// against bank conflicts); B operands are expanded from the sign bits in
// registers one K step ahead of the MFMAs that use them.  Each GEMM is one
// launch over every tile of every entry, tiles of one (entry, row stripe)
// placed on one XCD so the stripe is read into one L2.
#include <algorithm>
#include <type_traits>

#include "lb_prefill.h"
#include <hip/hip_fp16.h>

namespace lb {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

#define LB_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ inline LB_GLOBAL T* gp(T* p) { return (LB_GLOBAL T*)p; }
template <class T>
__device__ inline const LB_GLOBAL T* gp(const T* p) { return (const LB_GLOBAL T*)p; }


inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline int rup(int v, int m) { return (v + m - 1) / m * m; }

// bit position of (block b, element i) in a lane's per-K-step word
__host__ __device__ inline int pre_bit(int b, int i) { return (i & 1) ? 16 + 4 * b + (i >> 1) : 4 * b + (i >> 1); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct BuildArgs {
  PrefillLayer L;
  PathDev P[2];
};

__device__ inline int path_of_latent(const PrefillLayer& L, const PathDev* P, int j, int& jl) {
  for (int p = 0; p < L.np; ++p)
    if (j >= L.roff[p] && j < L.roff[p] + P[p].r) {
      jl = j - L.roff[p];
      return p;
    }
  return -1;
}

// GEMM1 B: thread per word (nt, kb, lane, ks)
__global__ void k_build_b1(BuildArgs a, uint32_t* out) {
  const PrefillLayer& L = a.L;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)L.nt1 * L.kb1 * 256;
  if (idx >= total) return;
  const int ks = idx & 3, lane = (idx >> 2) & 63;
  const int kb = (int)((idx >> 8) % L.kb1), nt = (int)((idx >> 8) / L.kb1);
  const int nin = lane & 31, kg = lane >> 5;
  uint32_t word = 0;
  for (int b = 0; b < 4; ++b) {
    int jl;
    const int p = path_of_latent(L, a.P, nt * kPreWN + 32 * b + nin, jl);
    if (p < 0) continue;
    const PathDev& P = a.P[p];
    for (int i = 0; i < 8; ++i) {
      const int k = kb * kPreBK + ks * 16 + 8 * kg + i;
      if (k >= L.n) continue;
      uint32_t bit = (P.v_can[(int64_t)k * P.W + (jl >> 5)] >> (jl & 31)) & 1u;
      bit ^= (uint32_t)(P.g[k] >> 15);   // sign of g folded in
      word |= bit << pre_bit(b, i);
    }
  }
  out[idx] = word;
}

// GEMM2 B: N = output row, K = concatenated latent
__global__ void k_build_b2(BuildArgs a, uint32_t* out) {
  const PrefillLayer& L = a.L;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)L.nt2 * L.kb2 * 256;
  if (idx >= total) return;
  const int ks = idx & 3, lane = (idx >> 2) & 63;
  const int kb = (int)((idx >> 8) % L.kb2), nt = (int)((idx >> 8) / L.kb2);
  const int nin = lane & 31, kg = lane >> 5;
  uint32_t word = 0;
  for (int b = 0; b < 4; ++b) {
    const int i_row = nt * kPreWN + 32 * b + nin;
    if (i_row >= L.m) continue;
    for (int i = 0; i < 8; ++i) {
      int jl;
      const int p = path_of_latent(L, a.P, kb * kPreBK + ks * 16 + 8 * kg + i, jl);
      if (p < 0) continue;
      const PathDev& P = a.P[p];
      uint32_t bit = (P.u_can[(int64_t)i_row * P.W + (jl >> 5)] >> (jl & 31)) & 1u;
      bit ^= (uint32_t)(P.h[i_row] >> 15);   // sign of h folded in
      word |= bit << pre_bit(b, i);
    }
  }
  out[idx] = word;
}

__device__ inline uint16_t abs_bf16_of_f16(uint16_t h) {
  return f32_to_bf16_rne(fabsf(__half2float(__ushort_as_half(h))));
}

__global__ void k_build_scales(BuildArgs a, uint16_t* gabs, uint16_t* habs, float* lpad) {
  const PrefillLayer& L = a.L;
  const int ng = L.kb1 * kPreBK, nh = L.nt2 * kPreWN;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < 2 * ng) {
    const int p = (int)(idx / ng), k = (int)(idx % ng);
    gabs[idx] = (p < L.np && k < L.n) ? abs_bf16_of_f16(a.P[p].g[k]) : (uint16_t)0;
  } else if (idx < 2 * ng + 2 * nh) {
    const int64_t r = idx - 2 * ng;
    const int p = (int)(r / nh), i = (int)(r % nh);
    habs[r] = (p < L.np && i < L.m) ? abs_bf16_of_f16(a.P[p].h[i]) : (uint16_t)0;
  } else if (idx < 2 * ng + 2 * nh + L.Rp) {
    const int j = (int)(idx - 2 * ng - 2 * nh);
    int jl;
    const int p = path_of_latent(L, a.P, j, jl);
    lpad[j] = p < 0 ? 0.f : __half2float(__ushort_as_half(a.P[p].l[jl]));
  }
}

// ---------------------------------------------------------------------------
// the GEMM kernel
// ---------------------------------------------------------------------------
struct PreArgs {
  const PreEntry* entries;
  const PreItem* items;
  const void* x0;   // when non-null: entry 0's input / output (single-linear forwards)
  void* y0;
  int T;
  int yf32;         // GEMM2 writes fp32 y (else bf16)
};

__device__ inline v16f mfma32(const u32x4& a, const u32x4& b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// B operand (4 dwords = 8 bf16) of block b from the lane's word for this K step
__device__ inline u32x4 expand_b(uint32_t d, int b, const u32x4& s2) {
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int sh = 15 - 4 * b - v;
    r[v] = ((sh ? d << sh : d) & 0x80008000u) | s2[v];   // magnitudes carry no sign bit
  }
  return r;
}

template <int N>
using Int = std::integral_constant<int, N>;

constexpr int kPreBufs = 4;                              // LDS buffers of the K-block pipeline

typedef __attribute__((address_space(3))) void lds_void;

// Buffer resource over plain byte offsets (no range check in practice: the
// record count is the largest allowed).  The loads into LDS go through buffer
// instructions rather than global ones: the compiler treats a pending global
// load into LDS as touching both memory and LDS and then waits for every
// outstanding LDS read wherever it needs one, which exposes the latency of
// the reads just issued for the next step.
// The base address is taken from the first lane: every base here is the same
// across the workgroup, but where the compiler cannot prove it, it keeps the
// resource in vector registers and wraps each load in a loop over the distinct
// values of the lanes (about a dozen instructions per load).
__device__ inline __amdgpu_buffer_rsrc_t byte_rsrc(const void* base) {
  // (readfirstlane returns a signed int: each half goes back through uint32_t,
  // or a low word with bit 31 set would fill the high word with ones)
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint64_t u = ((uint64_t)hi << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, 0x7fffffff, 0x00020000);
}

// Waits until at most VM vector-memory operations of this wave are
// outstanding and all of its LDS reads have returned, then the workgroup
// barrier.  The memory clobbers keep the compiler from moving LDS accesses
// across it.
template <int VM>
__device__ inline void vm_wait_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  constexpr int imm = (VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A tile in LDS: BM rows x 64 bf16 (128 bytes a row, unpadded), 16-byte
// chunk c of row r at slot 8 r + (c ^ f(r)), f(r) = (r & 7) ^ ((r >> 3) & 1).
// A fragment read has lane l32 on row base + l32 (base a multiple of 32), all
// lanes at the same logical chunk.  f puts any 8 consecutive rows of an
// aligned group on 8 distinct 16-byte positions of a 128-byte line, and the
// even rows (likewise the odd rows) of any aligned 16 on 8 distinct
// positions, so the rows a read serves together fall on distinct banks
// whether the LDS serves 8 lanes over 128 bytes or 16 lanes over 256 bytes
// per clock.  Slots are filled in order by the direct-to-LDS loads: wave w,
// instruction i, lane l writes slot 64 (W i + w) + l, W = waves.
__device__ inline int a_row_xor(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ inline int a_slot_row(int s) { return s >> 3; }
__device__ inline int a_slot_chunk(int s) { return (s & 7) ^ a_row_xor(s >> 3); }
// C staging: the 8-byte slots of tile row rt are XOR-ed with c_slot_xor(rt),
// so that the 16 rows a write phase covers hit distinct banks, while the two
// slots of each 16-byte chunk stay adjacent and in order (chunk ch of row rt
// sits at chunk ch ^ c_slot_xor(rt) / 2)
__device__ inline int c_slot_xor(int rt) { return (rt & 14) | ((rt & 1) << 4); }

// Wave layout of a BM x TN workgroup tile: WM x WN waves, each owning
// (BM / WM) x (TN / WN) outputs as MB x NB blocks of 32 x 32, every wave 64
// columns wide.  BM = 256 rows (tokens) between 129 and 255 tokens, eight
// waves; BM = 64 up to 64 tokens and BM = 128 otherwise, four waves (see
// prefill_rows_per_tile), so a row stripe holds no more empty rows than
// needed.  TN = 256 for whole tiles; the last column tile of a GEMM whose N
// leaves only 128 or 64 columns in it takes TN = 128 or 64 with the rows
// split over more waves (BM = 256: 4 x 2 waves of 64 x 64, 8 x 1 of 32 x 64;
// BM = 128: 2 x 2 of 64 x 64, 4 x 1 of 32 x 64; BM = 64: 2 x 2 of 32 x 64,
// and a 64-wide remainder takes the 128-wide tile), so every SIMD gets an
// equal share and a narrow tile takes a fraction of a whole one's time.
// STR (GEMM1 only): some wave's columns cross from the primary path into the
// residual one, so |g| is chosen per column block.  PART: the tile's rows run
// past the last token and a 32-row block is empty; each wave then reads and
// multiplies only its 32-row blocks that hold tokens.
// Threads of a workgroup: 256-row tiles take eight waves (two per SIMD, one
// workgroup per CU); 64- and 128-row tiles four waves of 64 x 64 and 128 x 64
// (one per SIMD, three and two workgroups per CU).  Measured against eight
// waves of 32 x 64 and 64 x 64, the four-wave forms take 18-29 % off 16 to 64
// tokens and 19-22 % off 128; 128-row tiles of four waves are also faster
// than 256-row tiles of eight from 256 tokens on (2048 tokens: 6-11 %).
constexpr int pre_threads(int bm) { return bm < kPreBM ? 256 : 512; }

template <int MODE, int BM, int WM, int WN, int TN, bool STR, bool PART>
__device__ __forceinline__ void prefill_tile(const PreArgs& a, const PreItem& it) {
  constexpr int kWaves = WM * WN, kNT = 64 * kWaves;
  constexpr int MB = BM / WM / 32, NB = TN / WN / 32;
  constexpr int kAI = BM * 8 / kNT;                     // A loads (16 B per lane) per wave per block
  static_assert(MB >= 1 && kAI >= 1, "a wave owns whole 32-row blocks; every wave loads A rows");
  static_assert(kWaves == 8 || kWaves == 4, "eight waves (two per SIMD) or four (one per SIMD)");
  static_assert(TN / WN == 64, "a wave covers 64 columns (half a 128-column B tile)");
  static_assert(NB == 2, "a wave covers two 32-column blocks (half a 128-column B tile)");
  static_assert(kWaves >= 3, "waves 0, 1, 2 carry the B words and |g|");
  static_assert(MODE == 1 || !STR, "only GEMM1 columns span paths");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const PreEntry& Eg = a.entries[it.entry];
  const PrefillLayer L = Eg.L;
  const int T = a.T;
  const bool first = it.entry == 0 && a.x0 != nullptr;
  const uint16_t* A;
  int lda, K, N, kbn, ntiles;
  const uint32_t* Bw;
  uint16_t* C;
  int ldc;
  if (MODE == 1) {
    A = reinterpret_cast<const uint16_t*>(first ? a.x0 : Eg.x);
    lda = L.n; K = L.n; N = L.Rp; kbn = L.kb1; Bw = L.b1; ntiles = L.nt1;
    C = Eg.z; ldc = L.Rp;
  } else {
    A = Eg.z;
    lda = L.Rp; K = L.Rp; N = L.m; kbn = L.kb2; Bw = L.b2; ntiles = L.nt2;
    C = reinterpret_cast<uint16_t*>(first ? a.y0 : Eg.y); ldc = L.m;
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
  const int wm = wave / WN, wn = wave % WN;
  const int m0 = it.mt * BM, n0 = it.nt * kPreBN;
  const int l32 = lane & 31, kg = lane >> 5;
  const int wcol = wn * (NB * 32);                       // first column of this wave in the tile
  // row blocks of this wave that hold tokens (all of them unless PART)
  int mba = MB;
  if constexpr (PART) {
    const int live = T - (m0 + wm * MB * 32);
    mba = __builtin_amdgcn_readfirstlane(live <= 0 ? 0 : min(MB, (live + 31) / 32));
  }
  const int bb0 = (wcol & (kPreWN - 1)) / 32;            // first 32-column block inside its B tile
  const bool vec_ok = (lda & 7) == 0;
  const int nkb = (K + kPreBK - 1) / kPreBK;
  // K blocks [kb_lo, kb_hi) of this item: all of K, or GEMM1 part it.ks of Eg.nks
  int kb_lo = 0, kb_hi = nkb;
  if (MODE == 1 && Eg.nks > 1) {
    const int kbs = (nkb + Eg.nks - 1) / Eg.nks;
    kb_lo = min(nkb, it.ks * kbs);
    kb_hi = min(nkb, kb_lo + kbs);
  }
  const int nloc = kb_hi - kb_lo;

  // LDS, kPreBufs buffers of: A [BM x 64] bf16 (swizzled) | B words [2 tiles][64 lanes] u32x4 | |g| [2][64] bf16
  constexpr int kBufA = BM * kPreBK * 2, kBufB = 2 * 64 * 16, kBufG = 2 * kPreBK * 2;
  constexpr int kBuf = kBufA + kBufB + kBufG;

  // ---- block loads: rows past T are clamped onto row T - 1 (a row of A only
  // reaches the same output row, which is not stored)
  // A: byte offsets inside the tile's row stripe; B: the wave's B tile; |g|
  const LB_GLOBAL uint16_t* asrc[kAI];
  int aoffb[kAI];
#pragma unroll
  for (int i = 0; i < kAI; ++i) {
    const int s = 64 * (kWaves * i + wave) + lane;
    const int r = min(m0 + a_slot_row(s), T - 1) - m0;
    asrc[i] = gp(A) + (int64_t)(m0 + r) * lda + a_slot_chunk(s) * 8;
    aoffb[i] = (r * lda + a_slot_chunk(s) * 8) * 2;
  }
  const __amdgpu_buffer_rsrc_t rsA = byte_rsrc(A + (int64_t)m0 * lda);
  const int btile = min(2 * it.nt + (wave & 1), ntiles - 1);
  const __amdgpu_buffer_rsrc_t rsB = byte_rsrc(Bw + (int64_t)btile * kbn * 64 * 4);
  const __amdgpu_buffer_rsrc_t rsG = byte_rsrc(L.gabs);
  const int goffb = ((lane >> 5) * L.kb1 * kPreBK + l32 * 2) * 2;
  // Issues block kb into LDS buffer buf.  Full blocks of 16-byte aligned rows
  // go straight to LDS (the B / |g| load first, so that a wait for "all but
  // the last kAI" covers it); a ragged or unaligned block goes through
  // registers with zero fill past K, synchronously.
  auto issue = [&](int kb, int buf) {
    uint8_t* base = lds + buf * kBuf;
    const int k0 = kb * kPreBK;
    if (wave < 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void*)(base + kBufA + wave * 1024), 16, (kb * 64 + lane) * 16, 0, 0, 0);
    else if (MODE == 1 && wave == 2)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsG, (lds_void*)(base + kBufA + kBufB), 4, goffb + k0 * 2, 0, 0, 0);
    if (vec_ok && k0 + kPreBK <= K) {
#pragma unroll
      for (int i = 0; i < kAI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void*)(base + (kWaves * i + wave) * 1024), 16, aoffb[i] + k0 * 2, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < kAI; ++i) {
        const int s = 64 * (kWaves * i + wave) + lane;
        const int k = k0 + a_slot_chunk(s) * 8;
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) e[q] = k + q < K ? asrc[i][k0 + q] : 0u;
        *reinterpret_cast<u32x4*>(base + s * 16) =
            u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
      }
    }
  };
  // A fragment of row block mb, K step ks: row R = wm 128 + 32 mb + l32,
  // chunk 2 ks + kg; R & 15 == l32 & 15
  int aoff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) aoff[ks] = (wm * MB * 32 + l32) * 128 + (((2 * ks + kg) ^ a_row_xor(l32)) * 16);
  auto read_a = [&](int buf, int ks, u32x4* af) {
    const uint8_t* Ab = lds + buf * kBuf + aoff[ks];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      if (!PART || mb < mba) af[mb] = *reinterpret_cast<const u32x4*>(Ab + mb * 32 * 128);
  };
  const int bsel = wcol / kPreWN;                        // which of the two B tiles
  auto read_b = [&](int buf) { return reinterpret_cast<const u32x4*>(lds + buf * kBuf + kBufA)[bsel * 64 + lane]; };

  // ---- B magnitudes.  GEMM1: |g| of the path of the wave's columns (per
  // column block when STR), per K step from LDS.  GEMM2: |h| of each column,
  // fixed along K, one set per path, chosen per K step.
  bool bpath[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) bpath[b] = MODE == 1 && L.np > 1 && n0 + wcol + (STR ? 32 * b : 0) >= L.roff[1];
  // LDS offsets of the |g| runs of the paths of the wave's first (gofs) and
  // last (gofs_x, STR only) column block, fixed for the tile: with the path
  // chosen per read, the STR body read both runs at every K step and selected
  const int gofs = kBufA + kBufB + __builtin_amdgcn_readfirstlane(bpath[0] ? kPreBK * 2 : 0) + 16 * kg;
  const int gofs_x = kBufA + kBufB + __builtin_amdgcn_readfirstlane(bpath[NB - 1] ? kPreBK * 2 : 0) + 16 * kg;
  auto read_g = [&](int buf, int ks, int ofs) {
    return *reinterpret_cast<const u32x4*>(lds + buf * kBuf + ofs + 32 * ks);
  };
  uint32_t h0[NB], h1[NB];
  if (MODE == 2) {
    const int tile = min((n0 + wcol) / kPreWN, ntiles - 1);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t i = (int64_t)tile * kPreWN + 32 * (bb0 + b) + l32;
      const uint32_t x0 = gp(L.habs)[i], x1 = gp(L.habs)[(int64_t)L.nt2 * kPreWN + i];
      h0[b] = x0 | (x0 << 16);
      h1[b] = x1 | (x1 << 16);
    }
  }
  // B operands of one K step: sign bits d (one word per step), magnitudes
  // gc (GEMM1, path of block 0) / gs (GEMM1, path of the last block; STR
  // only: a wave's 64 columns are two blocks) / the GEMM2 path of the step
  auto make_b = [&](uint32_t d, const u32x4& gc, const u32x4& gs, bool kp, u32x4* bf) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      u32x4 sc;
      if (MODE == 1) {
        sc = (STR && b == NB - 1) ? gs : gc;
      } else {
        const uint32_t h = kp ? h1[b] : h0[b];
        sc = u32x4{h, h, h, h};
      }
      bf[b] = expand_b(d, bb0 + b, sc);
    }
  };
  auto kpath = [&](int kb, int ks) { return MODE == 2 && L.np > 1 && kb * kPreBK + ks * 16 >= L.roff[1]; };

  // the first K step's MFMAs start from zero (see kblock); blocks a PART
  // wave skips keep these zeros
  v16f acc[MB][NB];
  if constexpr (PART) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  }

  // Pipeline over four LDS buffers: block kb + 3 is issued at the start of
  // block kb (into the buffer block kb - 1 used), and the barrier that ends
  // block kb waits for this wave's loads of block kb + 2 first, so both the
  // current and the next block are complete in LDS during a block.  Inside a
  // block, K step ks multiplies while the A fragments and B operands of step
  // ks + 1 are read and expanded (for ks = 3: step 0 of the next block, whose
  // buffer is complete since the previous barrier; past the last block the
  // buffer is stale and the result unused).
  issue(kb_lo, 0);
  if (nloc > 1) issue(kb_lo + 1, 1);
  if (nloc > 2) {
    issue(kb_lo + 2, 2);
    vm_wait_barrier<kAI>();
  } else {
    vm_wait_barrier<0>();
  }
  u32x4 af[2][MB], bf[2][NB];
  // GEMM1 magnitudes are read two K steps ahead (slot s & 1 holds step s's),
  // so that expanding the next step's B operand waits for no LDS read of
  // this step
  u32x4 gq[2][2] = {};
  read_a(0, 0, af[0]);
  u32x4 bw = read_b(0);
  {
    const u32x4 g0 = MODE == 1 ? read_g(0, 0, gofs) : u32x4{};
    const u32x4 g1 = (MODE == 1 && STR) ? read_g(0, 0, gofs_x) : u32x4{};
    if (MODE == 1) gq[1][0] = read_g(0, 1, gofs);
    if (MODE == 1 && STR) gq[1][1] = read_g(0, 1, gofs_x);
    make_b(bw[0], g0, g1, kpath(0, 0), bf[0]);
  }

  // one K block; FIRST (the item's first block) starts the sums from zero
  auto kblock = [&](int kb, auto first) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first)::value;
    const int cur = (kb - kb_lo) & 3, nxt = (kb - kb_lo + 1) & 3;
    const bool more = kb + 3 < kb_hi;
    if (more) issue(kb + 3, (kb - kb_lo + 3) & 3);
    const u32x4 bwn = read_b(nxt);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int rb = ks < 3 ? cur : nxt, rks = (ks + 1) & 3;
      const int gb = ks < 2 ? cur : nxt, gks = (ks + 2) & 3;
      read_a(rb, rks, af[(ks + 1) & 1]);
      const uint32_t dn = ks < 3 ? bw[ks + 1] : bwn[0];
      const u32x4 g0 = gq[(ks + 1) & 1][0], g1 = gq[(ks + 1) & 1][1];
      if (MODE == 1) gq[ks & 1][0] = read_g(gb, gks, gofs);
      if (MODE == 1 && STR) gq[ks & 1][1] = read_g(gb, gks, gofs_x);
      // the LDS reads of step ks + 1 go out before this step's MFMAs (the
      // scheduler would otherwise sink them next to their use and expose
      // their latency at every step)
      __builtin_amdgcn_sched_barrier(0);
      make_b(dn, g0, g1, kpath(ks < 3 ? kb : kb + 1, rks), bf[(ks + 1) & 1]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          if (!PART || mb < mba)
            acc[mb][b] = mfma32(bf[ks & 1][b], af[ks & 1][mb], (FIRST && ks == 0) ? v16f{} : acc[mb][b]);
    }
    bw = bwn;
    if (more) vm_wait_barrier<kAI>();
    else vm_wait_barrier<0>();
  };
  kblock(kb_lo, std::true_type{});
  for (int kb = kb_lo + 1; kb < kb_hi; ++kb) kblock(kb, std::false_type{});

  // ---- epilogue.  The MFMAs take the B operand as their first factor, so
  // block (mb, b) holds the transposed product: lane (l32, kg) has output row
  // l32 of the block and columns 8 j + 4 kg + i (j, i = 0..3) in q = 4 j + i,
  // i.e. four runs of four adjacent columns (8 bytes of bf16 each).  When rows
  // of C are 16-byte aligned, the workgroup stages its bf16 tile in LDS (free:
  // every wave is past the loop's last barrier, which waited for all LDS
  // reads) and writes whole 512-byte row segments; otherwise each run goes
  // straight out.
  if (MODE == 1 && Eg.nks > 1) {
    // one K part of a cut GEMM1: fp32 partial sums (l is applied where the
    // parts are added); N = Rp is a multiple of 64, so a run is wholly in or out
    LB_GLOBAL float* Cp = gp(Eg.zpart) + (int64_t)it.ks * T * ldc;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int cb = n0 + wcol + 32 * b + 4 * kg;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = m0 + wm * MB * 32 + mb * 32 + l32;
        if (row >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = cb + 8 * j;
          if (col < N)
            *reinterpret_cast<LB_GLOBAL f4*>(Cp + (int64_t)row * ldc + col) =
                f4{acc[mb][b][4 * j], acc[mb][b][4 * j + 1], acc[mb][b][4 * j + 2], acc[mb][b][4 * j + 3]};
        }
      }
    }
    return;
  }
  if (MODE == 2 && a.yf32) {
    // fp32 y: each run of four adjacent columns is one 16-byte store
    float* Cf = reinterpret_cast<float*>(first ? a.y0 : Eg.y);
    const bool vec4 = (ldc & 3) == 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int cb = n0 + wcol + 32 * b + 4 * kg;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = m0 + wm * MB * 32 + mb * 32 + l32;
        if (row >= T) continue;
        LB_GLOBAL float* cp = gp(Cf) + (int64_t)row * ldc;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = cb + 8 * j;
          const f4 v = {acc[mb][b][4 * j], acc[mb][b][4 * j + 1], acc[mb][b][4 * j + 2], acc[mb][b][4 * j + 3]};
          if (vec4 && col + 3 < N) {
            *reinterpret_cast<LB_GLOBAL f4*>(cp + col) = v;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (col + i < N) cp[col + i] = v[i];
          }
        }
      }
    }
    return;
  }
  const bool c_stage = (ldc & 7) == 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int cb = n0 + wcol + 32 * b + 4 * kg;
    float ls[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) ls[q] = 1.f;
    if (MODE == 1) {
      // GEMM1: N = Rp is a multiple of 64, so a run is wholly inside or outside
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (cb + 8 * j < N) {
          const f4 v = *reinterpret_cast<const LB_GLOBAL f4*>(gp(L.lpad) + cb + 8 * j);
#pragma unroll
          for (int i = 0; i < 4; ++i) ls[4 * j + i] = v[i];
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int rt = wm * MB * 32 + mb * 32 + l32;   // row inside the tile
      const int row = m0 + rt;
      LB_GLOBAL uint16_t* cp = gp(C) + (int64_t)row * ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = cb + 8 * j;
        const f2 lo = {acc[mb][b][4 * j] * ls[4 * j], acc[mb][b][4 * j + 1] * ls[4 * j + 1]};
        const f2 hi = {acc[mb][b][4 * j + 2] * ls[4 * j + 2], acc[mb][b][4 * j + 3] * ls[4 * j + 3]};
        const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf2));
        const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf2));
        if (c_stage) {
          // 8-byte slot (col - n0) / 4 of tile row rt, swizzled (c_slot_xor)
          const int slot = ((col - n0) >> 2) ^ c_slot_xor(rt);
          *reinterpret_cast<u32x2*>(lds + rt * (kPreBN * 2) + slot * 8) = u32x2{w0, w1};
        } else if (row < T) {
          if ((ldc & 3) == 0 && col + 3 < N) {
            *reinterpret_cast<LB_GLOBAL u32x2*>(cp + col) = u32x2{w0, w1};   // 8-byte aligned run
          } else {
            const uint32_t w[2] = {w0, w1};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (col + i < N) cp[col + i] = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
          }
        }
      }
    }
  }
  if (c_stage) {
    __syncthreads();
    // thread t copies 16-byte chunk ch = t % (TN / 8) of tile rows r0 + k RS
    // (r0 = t / (TN / 8)); C rows are whole multiples of 8 elements here
    // (ldc = N, a multiple of 8), so a chunk is wholly inside or outside.  Rows
    // r0 + k RS have the same swizzle when RS is a multiple of 16 and two that
    // alternate when it is 8.
    constexpr int kCPR = TN / 8, RS = kNT / kCPR, NIT = BM / RS;
    static_assert(RS % 8 == 0 && BM % RS == 0, "whole rows per pass, a multiple of 8");
    const int tid_all = threadIdx.x, ch = tid_all % kCPR, r0 = tid_all / kCPR;
    const int col = n0 + ch * 8;
    if (col < N) {
      const uint8_t* lb0 = lds + r0 * (kPreBN * 2) + ((ch ^ (c_slot_xor(r0) >> 1)) * 16);
      const uint8_t* lb1 = lds + (r0 + 8) * (kPreBN * 2) + ((ch ^ (c_slot_xor(r0 + 8) >> 1)) * 16);
      LB_GLOBAL uint16_t* cp = gp(C) + (int64_t)(m0 + r0) * ldc + col;
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        if (m0 + r0 + k * RS >= T) break;
        const uint8_t* lp = RS % 16 == 0 ? lb0 + k * RS * (kPreBN * 2) : (k & 1 ? lb1 : lb0) + (k >> 1) * 16 * (kPreBN * 2);
        *reinterpret_cast<LB_GLOBAL u32x4*>(cp + (int64_t)k * RS * ldc) = *reinterpret_cast<const u32x4*>(lp);
      }
    }
  }
}

// Adds the K parts of cut GEMM1s in part order and applies l:
// Z' = bf16((P_0 + P_1 + ...) l), four adjacent outputs per thread.
__global__ void __launch_bounds__(256) k_prefill_combine(const PreEntry* entries, const PreComb* items, int T) {
  const PreComb c = items[blockIdx.x];
  const PreEntry& E = entries[c.entry];
  const int Rp = E.L.Rp;
  const int64_t plane = (int64_t)T * Rp, e = (int64_t)c.e0 + threadIdx.x * 4;
  if (e >= plane) return;
  const LB_GLOBAL float* P = gp(E.zpart);
  f4 s = *reinterpret_cast<const LB_GLOBAL f4*>(P + e);
  for (int k = 1; k < E.nks; ++k) {
    const f4 v = *reinterpret_cast<const LB_GLOBAL f4*>(P + k * plane + e);
    s = f4{s[0] + v[0], s[1] + v[1], s[2] + v[2], s[3] + v[3]};
  }
  const f4 l = *reinterpret_cast<const LB_GLOBAL f4*>(gp(E.L.lpad) + (int)(e % Rp));
  const f2 lo = {s[0] * l[0], s[1] * l[1]}, hi = {s[2] * l[2], s[3] * l[3]};
  *reinterpret_cast<LB_GLOBAL u32x2*>(gp(E.z) + e) =
      u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf2)),
            __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf2))};
}

// One workgroup per tile; GEMM1 tiles where a wave's columns reach into both
// paths take the body that picks |g| per column block.
// PART: a launch over the tiles of row stripes that run past the last token
// (a separate launch, so the full tiles' kernel carries none of it).
// The tile width (it.tn: 256, 128 or 64) picks the wave layout, uniformly
// over the workgroup (64-row tiles are 256 or 128 wide).
template <int MODE, int BM, bool STR, bool PART>
__device__ __forceinline__ void prefill_tile_any(const PreArgs& a, const PreItem& it) {
  if constexpr (BM == 64) {
    if (it.tn == 256) prefill_tile<MODE, 64, 1, 4, 256, STR, PART>(a, it);
    else prefill_tile<MODE, 64, 2, 2, 128, STR, PART>(a, it);
  } else if constexpr (BM == 128) {
    if (it.tn == 256) prefill_tile<MODE, 128, 1, 4, 256, STR, PART>(a, it);
    else if (it.tn == 128) prefill_tile<MODE, 128, 2, 2, 128, STR, PART>(a, it);
    else prefill_tile<MODE, 128, 4, 1, 64, STR, PART>(a, it);
  } else {
    if (it.tn == 256) prefill_tile<MODE, BM, 2, 4, 256, STR, PART>(a, it);
    else if (it.tn == 128) prefill_tile<MODE, BM, 4, 2, 128, STR, PART>(a, it);
    else prefill_tile<MODE, BM, 8, 1, 64, STR, PART>(a, it);
  }
}

template <int MODE, int BM, bool PART>
__global__ void __launch_bounds__(pre_threads(BM), BM == 64 ? 3 : BM < kPreBM ? 2 : 1) k_prefill(PreArgs a) {
  const PreItem it = a.items[blockIdx.x];
  if (it.entry < 0) return;
  if constexpr (MODE == 1) {
    if (it.str) prefill_tile_any<1, BM, true, PART>(a, it);
    else prefill_tile_any<1, BM, false, PART>(a, it);
  } else {
    prefill_tile_any<2, BM, false, PART>(a, it);
  }
}

constexpr int kWaveCols = 64;   // columns of one wave in every layout

// width of column tile nt of a GEMM with N columns: 256, or 128 / 64 for a
// last tile that leaves at most that many columns
int tile_width(int N, int nt) {
  const int left = N - nt * kPreBN;
  return left >= kPreBN ? kPreBN : (left > 128 ? 256 : (left > 64 ? 128 : 64));
}

// true when a wave of GEMM1 tile nt has columns of both paths
bool tile_straddles(const PrefillLayer& L, int nt, int tn) {
  if (L.np < 2) return false;
  for (int w = 0; w < tn / kWaveCols; ++w) {
    const int c0 = nt * kPreBN + w * kWaveCols;
    if (c0 < L.roff[1] && c0 + kWaveCols - 32 >= L.roff[1]) return true;
  }
  return false;
}
constexpr size_t pre_lds(int bm) { return kPreBufs * (size_t)(bm * kPreBK * 2 + 2 * 64 * 16 + 2 * kPreBK * 2); }
static_assert(pre_lds(256) >= (size_t)256 * kPreBN * 2, "the epilogue stages the bf16 tile in the LDS buffers");
static_assert(pre_lds(64) >= (size_t)64 * kPreBN * 2, "the epilogue stages the bf16 tile in the LDS buffers");
static_assert(pre_lds(128) >= (size_t)128 * kPreBN * 2, "the epilogue stages the bf16 tile in the LDS buffers");
static_assert(2 * pre_lds(128) <= 160 * 1024, "two 128-row workgroups fit a CU's LDS");

}  // namespace

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

PrefillLayer layer_geometry(int64_t m, int64_t n, const int64_t* ranks, int np) {
  PrefillLayer L;
  L.m = (int)m;
  L.n = (int)n;
  L.np = np;
  int off = 0;
  for (int p = 0; p < np; ++p) {
    L.rp[p] = rup((int)ranks[p], 32);
    L.roff[p] = off;
    off += L.rp[p];
  }
  L.Rp = rup(off, kPreBK);
  L.nt1 = (L.Rp + kPreWN - 1) / kPreWN;
  L.kb1 = ((int)n + kPreBK - 1) / kPreBK;
  L.nt2 = ((int)m + kPreWN - 1) / kPreWN;
  L.kb2 = L.Rp / kPreBK;
  return L;
}

size_t layer_bytes(const PrefillLayer& L) {
  return align256((size_t)L.nt1 * L.kb1 * 256 * 4) + align256((size_t)L.nt2 * L.kb2 * 256 * 4) +
         align256((size_t)2 * L.kb1 * kPreBK * 2) + align256((size_t)2 * L.nt2 * kPreWN * 2) +
         align256((size_t)L.Rp * 4);
}

}  // namespace

size_t prefill_layer_bytes(int64_t m, int64_t n, const lb_path* paths, int np) {
  int64_t ranks[2] = {0, 0};
  for (int p = 0; p < np; ++p) ranks[p] = paths[p].rank;
  return layer_bytes(layer_geometry(m, n, ranks, np));
}

hipError_t prefill_layer_build(PrefillLayer& out, void* mem, size_t bytes, int64_t m, int64_t n,
                               const PathDev* paths, int np, hipStream_t st) {
  int64_t ranks[2] = {0, 0};
  for (int p = 0; p < np; ++p) ranks[p] = paths[p].r;
  PrefillLayer L = layer_geometry(m, n, ranks, np);
  if (layer_bytes(L) > bytes) return hipErrorInvalidValue;
  char* c = reinterpret_cast<char*>(mem);
  auto take = [&](size_t b) {
    void* p = c;
    c += align256(b);
    return p;
  };
  uint32_t* b1 = reinterpret_cast<uint32_t*>(take((size_t)L.nt1 * L.kb1 * 256 * 4));
  uint32_t* b2 = reinterpret_cast<uint32_t*>(take((size_t)L.nt2 * L.kb2 * 256 * 4));
  uint16_t* gabs = reinterpret_cast<uint16_t*>(take((size_t)2 * L.kb1 * kPreBK * 2));
  uint16_t* habs = reinterpret_cast<uint16_t*>(take((size_t)2 * L.nt2 * kPreWN * 2));
  float* lpad = reinterpret_cast<float*>(take((size_t)L.Rp * 4));
  BuildArgs a;
  a.L = L;
  a.P[0] = paths[0];
  a.P[1] = np > 1 ? paths[1] : paths[0];
  const int64_t t1 = (int64_t)L.nt1 * L.kb1 * 256, t2 = (int64_t)L.nt2 * L.kb2 * 256;
  const int64_t t3 = 2 * (int64_t)L.kb1 * kPreBK + 2 * (int64_t)L.nt2 * kPreWN + L.Rp;
  hipLaunchKernelGGL(k_build_b1, dim3((unsigned)((t1 + 255) / 256)), dim3(256), 0, st, a, b1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_build_b2, dim3((unsigned)((t2 + 255) / 256)), dim3(256), 0, st, a, b2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_build_scales, dim3((unsigned)((t3 + 255) / 256)), dim3(256), 0, st, a, gabs, habs, lpad);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  L.b1 = b1;
  L.b2 = b2;
  L.gabs = gabs;
  L.habs = habs;
  L.lpad = lpad;
  out = L;
  return hipSuccess;
}

bool prefill_available() { return true; }

namespace {

// Tiles of one (entry, row stripe) go to one XCD (workgroup b runs on XCD b % 8).
// Stripes are balanced over the XCDs by work (tiles x K blocks per tile),
// heaviest first, so each XCD's list starts with its longest tiles and the
// launch ends on short ones.
std::vector<PreItem> xcd_order(const std::vector<std::vector<PreItem>>& stripes, const std::vector<double>& kblocks) {
  constexpr int kXcd = 8;
  std::vector<int> order(stripes.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  auto work = [&](int s) { return (double)stripes[s].size() * kblocks[s]; };
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return work(a) > work(b); });
  std::vector<std::vector<PreItem>> per(kXcd);
  std::vector<double> load(kXcd, 0.0);
  for (int s : order) {
    int best = 0;
    for (int x = 1; x < kXcd; ++x)
      if (load[x] < load[best]) best = x;
    per[best].insert(per[best].end(), stripes[s].begin(), stripes[s].end());
    load[best] += work(s);
  }
  size_t len = 0;
  for (auto& v : per) len = std::max(len, v.size());
  std::vector<PreItem> out(len * kXcd, PreItem{-1, 0, 0, 0, 0, 0});
  for (int x = 0; x < kXcd; ++x)
    for (size_t i = 0; i < per[x].size(); ++i) out[i * kXcd + x] = per[x][i];
  return out;
}

}  // namespace

double prefill_gemm1_blocks(const PrefillLayer* const* layers, int count, int T) {
  const int bm = prefill_rows_per_tile(T), mts = (T + bm - 1) / bm;
  double blocks = 0;
  for (int e = 0; e < count; ++e)
    blocks += (double)mts * ((layers[e]->Rp + kPreBN - 1) / kPreBN) * layers[e]->kb1;
  return blocks;
}

hipError_t prefill_prepare(PrefillPlan& P, const PrefillLayer* const* layers, int count, int T,
                           const void* const* xs, void* const* ys) {
  // buffers and tables are rebuilt below: the plan is valid again only once
  // all of it has succeeded
  P.T = -1;
  P.count = 0;
  const int bm = prefill_rows_per_tile(T);
  const int mts = (T + bm - 1) / bm;
  std::vector<std::vector<PreItem>> s1, s2, s1p, s2p;   // full row stripes, stripes past the last token
  std::vector<double> k1, k2, k1p, k2p;                  // K blocks per tile of each stripe
  size_t zoff = 0, poff = 0;
  std::vector<size_t> zoffs(count), poffs(count);
  std::vector<PreComb> comb;
  P.entries_h.assign(count, PreEntry{});
  const double blocks1 = prefill_gemm1_blocks(layers, count, T);
  for (int e = 0; e < count; ++e) {
    const PrefillLayer& L = *layers[e];
    P.entries_h[e].L = L;
    zoffs[e] = zoff;
    zoff += align256((size_t)T * L.Rp * 2);
    const int nks = prefill_k_parts(L.kb1, T, blocks1);
    P.entries_h[e].nks = nks;
    poffs[e] = poff;
    if (nks > 1) {
      poff += align256((size_t)nks * T * L.Rp * 4);
      for (int64_t e0 = 0; e0 < (int64_t)T * L.Rp; e0 += 1024) comb.push_back(PreComb{e, (int)e0});
    }
    const int nt1 = (L.Rp + kPreBN - 1) / kPreBN, nt2 = (L.m + kPreBN - 1) / kPreBN;
    // work of one row stripe in whole-tile K blocks (a narrow tile counts its share)
    // (64-row tiles are at least 128 wide)
    auto width = [&](int N, int nt) { return bm == 64 ? std::max(tile_width(N, nt), 128) : tile_width(N, nt); };
    double w1 = 0, w2 = 0;
    for (int nt = 0; nt < nt1; ++nt) w1 += width(L.Rp, nt) / (double)kPreBN;
    for (int nt = 0; nt < nt2; ++nt) w2 += width(L.m, nt) / (double)kPreBN;
    for (int mt = 0; mt < mts; ++mt) {
      std::vector<PreItem> a, b;
      for (int ks = 0; ks < nks; ++ks)
        for (int nt = 0; nt < nt1; ++nt) {
          const int tn = width(L.Rp, nt);
          a.push_back(PreItem{e, mt, nt, tile_straddles(L, nt, tn) ? 1 : 0, tn, ks});
        }
      for (int nt = 0; nt < nt2; ++nt) b.push_back(PreItem{e, mt, nt, 0, width(L.m, nt), 0});
      // a stripe past the last token runs the kernel that skips empty 32-row
      // blocks, when it has one (with none the skipping costs more than it
      // saves: 112 tokens in one 128-row stripe, 9 % slower)
      const bool part = (mt + 1) * bm > T && T - mt * bm <= bm - 32;
      (part ? s1p : s1).push_back(a);
      (part ? s2p : s2).push_back(b);
      (part ? k1p : k1).push_back(L.kb1 * w1 / nt1 / nks);
      (part ? k2p : k2).push_back(L.kb2 * w2 / nt2);
    }
  }
  std::vector<PreItem> i1 = xcd_order(s1, k1), i2 = xcd_order(s2, k2);
  std::vector<PreItem> i1p = xcd_order(s1p, k1p), i2p = xcd_order(s2p, k2p);
  if (zoff > P.zbytes) {
    if (P.zbuf) {
      hipError_t e = hipFree(P.zbuf);
      if (e != hipSuccess) return e;
      P.zbuf = nullptr;
      P.zbytes = 0;
    }
    hipError_t e = hipMalloc(&P.zbuf, zoff);
    if (e != hipSuccess) return e;
    P.zbytes = zoff;
  }
  if (poff > P.pbytes) {
    if (P.pbuf) {
      hipError_t e = hipFree(P.pbuf);
      if (e != hipSuccess) return e;
      P.pbuf = nullptr;
      P.pbytes = 0;
    }
    hipError_t e = hipMalloc(&P.pbuf, poff);
    if (e != hipSuccess) return e;
    P.pbytes = poff;
  }
  for (int e = 0; e < count; ++e) {
    P.entries_h[e].z = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(P.zbuf) + zoffs[e]);
    P.entries_h[e].zpart = P.entries_h[e].nks > 1 ? reinterpret_cast<float*>(reinterpret_cast<char*>(P.pbuf) + poffs[e])
                                                  : nullptr;
    P.entries_h[e].x = xs ? xs[e] : nullptr;
    P.entries_h[e].y = ys ? ys[e] : nullptr;
  }
  if (P.entries_d) (void)hipFree(P.entries_d);
  if (P.items_d) (void)hipFree(P.items_d);
  if (P.comb_d) (void)hipFree(P.comb_d);
  P.entries_d = nullptr;
  P.items_d = nullptr;
  P.comb_d = nullptr;
  hipError_t e = hipMalloc(&P.entries_d, count * sizeof(PreEntry));
  if (e == hipSuccess && !comb.empty()) e = hipMalloc(&P.comb_d, comb.size() * sizeof(PreComb));
  if (e == hipSuccess && !comb.empty())
    e = hipMemcpy(P.comb_d, comb.data(), comb.size() * sizeof(PreComb), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMalloc(&P.items_d, std::max<size_t>(1, i1.size() + i1p.size() + i2.size() + i2p.size()) * sizeof(PreItem));
  if (e == hipSuccess) e = hipMemcpy(P.entries_d, P.entries_h.data(), count * sizeof(PreEntry), hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  std::vector<PreItem> all(i1);
  all.insert(all.end(), i1p.begin(), i1p.end());
  all.insert(all.end(), i2.begin(), i2.end());
  all.insert(all.end(), i2p.begin(), i2p.end());
  if (!all.empty() &&
      (e = hipMemcpy(P.items_d, all.data(), all.size() * sizeof(PreItem), hipMemcpyHostToDevice)) != hipSuccess)
    return e;
  P.n1 = (int)i1.size();
  P.n1p = (int)i1p.size();
  P.n2 = (int)i2.size();
  P.n2p = (int)i2p.size();
  P.ncomb = (int)comb.size();
  P.bm = bm;
  P.T = T;
  P.count = count;
  return hipSuccess;
}

namespace {

template <int BM>
hipError_t launch_gemms(const PrefillPlan& P, PreArgs a, hipStream_t st) {
  const size_t lds = pre_lds(BM);
  a.items = P.items_d;
  if (P.n1 > 0) hipLaunchKernelGGL((k_prefill<1, BM, false>), dim3(P.n1), dim3(pre_threads(BM)), lds, st, a);
  a.items = P.items_d + P.n1;
  if (P.n1p > 0) hipLaunchKernelGGL((k_prefill<1, BM, true>), dim3(P.n1p), dim3(pre_threads(BM)), lds, st, a);
  if (P.ncomb > 0) hipLaunchKernelGGL(k_prefill_combine, dim3(P.ncomb), dim3(256), 0, st, a.entries, P.comb_d, a.T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.items = P.items_d + P.n1 + P.n1p;
  if (P.n2 > 0) hipLaunchKernelGGL((k_prefill<2, BM, false>), dim3(P.n2), dim3(pre_threads(BM)), lds, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.items = P.items_d + P.n1 + P.n1p + P.n2;
  if (P.n2p > 0) hipLaunchKernelGGL((k_prefill<2, BM, true>), dim3(P.n2p), dim3(pre_threads(BM)), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t prefill_run(PrefillPlan& P, const PrefillLayer* const* layers, int count, const void* const* xs,
                       void* const* ys, int T, int yf32, hipStream_t st, bool single) {
  PreArgs a{};
  a.yf32 = yf32;
  if (single) {
    // single-linear forwards: the plan holds no pointers, they travel as kernel arguments
    if (P.T != T || P.count != 1) {
      if (P.T != -1) {
        hipError_t e = hipStreamSynchronize(st);   // the plan is rewritten below
        if (e != hipSuccess) return e;
      }
      hipError_t e = prefill_prepare(P, layers, 1, T, nullptr, nullptr);
      if (e != hipSuccess) return e;
    }
    a.x0 = xs[0];
    a.y0 = ys[0];
  } else if (P.T != T || P.count != count) {
    return hipErrorNotReady;   // stacks prepare their plan (with pointers) before launching
  }
  a.entries = P.entries_d;
  a.T = T;
  // GEMM1 over the full row stripes, then over the stripe past the last token;
  // the same for GEMM2
  return P.bm == 64 ? launch_gemms<64>(P, a, st) : P.bm == 128 ? launch_gemms<128>(P, a, st) : launch_gemms<256>(P, a, st);
}

void prefill_plan_release(PrefillPlan& P) {
  if (P.entries_d) (void)hipFree(P.entries_d);
  if (P.items_d) (void)hipFree(P.items_d);
  if (P.zbuf) (void)hipFree(P.zbuf);
  if (P.comb_d) (void)hipFree(P.comb_d);
  if (P.pbuf) (void)hipFree(P.pbuf);
  P.entries_d = nullptr;
  P.items_d = nullptr;
  P.zbuf = nullptr;
  P.zbytes = 0;
  P.comb_d = nullptr;
  P.ncomb = 0;
  P.pbuf = nullptr;
  P.pbytes = 0;
  P.T = -1;
  P.count = 0;
  P.entries_h.clear();
}

}  // namespace lb

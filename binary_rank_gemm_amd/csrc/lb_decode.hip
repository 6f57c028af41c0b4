// Fused decode forward (few tokens, bf16 I/O) over a list of linears.
//
// Computes, for every entry and path p, the factorised order of the paper
// notes ("LittleBit: Ultra Low-Bit Quantization via Latent Factorization",
// section "Key design"): t = x o g_p, z_p = t V_p, z'_p = z_p o l_p, and then
// y = sum_p (z'_p U_p^T) o h_p (section "Residual compensation" for the sum).
//
// Two launches per step, each over static per-workgroup lists of work items
// (balanced on the host, longest first), so workgroups never wait on each
// other and the kernel boundary is the only synchronisation:
//   V kernel, item (entry, path, column group): z'_p for up to 16 column tiles
//     of 16 latents, reducing over all d_in rows; the four waves split the
//     rows and combine partial sums in LDS in a fixed order (deterministic).
//     Its epilogue converts z'_p straight into the U stage's fp8 A operand
//     images and the U stage's correction sums.
//   U kernel, item (entry, 256 output rows): streams U's sign words against
//     those images and writes y for its rows, both paths.
//
// Arithmetic (gfx950 v_mfma_scale_f32_16x16x128_f8f6f4, fp32 accumulate):
//   * B operand = packed sign bits expanded to fp4 (e2m1) with one mask per
//     VGPR: nibble bit 3 over a 0x2 base gives +-1 (the sign class); nibble
//     bits 2, 1, 0 alone give {0, 2}, {0, 1}, {0, 0.5}.  For the latter three
//     classes b = (1 - s) / 2, and the A operand carries -2 t / beta so that
//     A*B = -2 t b = t s - t; the missing sum of t over those rows (C) is added
//     in the epilogue.  Four VALU ops expand 32 signs.
//   * A operand = activations as two e4m3 terms (hi = RNE(u), lo = RNE(16 (u -
//     hi))) in MFMA rows 2 t and 2 t + 1, with per-32-element power-of-two
//     block scales (the instruction's e8m0 scale operand), so the hi/lo pair
//     carries about 8 significant bits (as bf16 does) and the two terms cost no
//     extra MFMA for up to 8 tokens.
#include "lb_internal.h"
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

namespace lb {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kWavesPerGroup;

// Pointers read from the entry table are generic; naming them global lets the
// compiler use global (not flat) memory instructions.
#define LB_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ inline LB_GLOBAL T* gp(T* p) { return (LB_GLOBAL T*)p; }
template <class T>
__device__ inline const LB_GLOBAL T* gp(const T* p) { return (const LB_GLOBAL T*)p; }

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline float f16f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// float -> bf16 bits, round to nearest even (the hardware conversion)
__device__ inline uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <int N>
__device__ inline float ror16(float v) {  // rotate within a row of 16 lanes (DPP row_ror)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
__device__ inline float row16_max(float v) {
  v = fmaxf(v, ror16<8>(v));
  v = fmaxf(v, ror16<4>(v));
  v = fmaxf(v, ror16<2>(v));
  v = fmaxf(v, ror16<1>(v));
  return v;
}
__device__ inline float row16_sum(float v) {
  v += ror16<8>(v);
  v += ror16<4>(v);
  v += ror16<2>(v);
  v += ror16<1>(v);
  return v;
}
// Sum over the wave, identical in every lane, fixed association order.
__device__ inline float wave_sum(float v) {
  v = row16_sum(v);
  float r0 = __shfl(v, 0), r1 = __shfl(v, 16), r2 = __shfl(v, 32), r3 = __shfl(v, 48);
  return (r0 + r1) + (r2 + r3);
}

// Orders one wave's own LDS accesses: the LDS executes a wave's DS operations
// in issue order, so only the compiler must be kept from reordering them (a
// memory fence here would also wait for the prefetched global loads).
__device__ inline void wave_lds_fence() { __asm__ volatile("" ::: "memory"); }

// fp4 B operand from one packed word (bit layout of fp4_bit_of_elem).
__device__ inline v8i expand_signs(uint32_t w) {
  v8i b;
  b[0] = (int)((w & 0x88888888u) | 0x22222222u);  // +-1
  b[1] = (int)(w & 0x44444444u);                  // {0, 2}
  b[2] = (int)(w & 0x22222222u);                  // {0, 1}
  b[3] = (int)(w & 0x11111111u);                  // {0, 0.5}
  b[4] = b[5] = b[6] = b[7] = 0;
  return b;
}

// Byte offset of byte e (< 32) of MFMA row `row`, K group g in an fp8 A image:
// two 1 KB halves holding bytes 0-15 and 16-31 of every (row, group), so the
// two 16-byte reads of a wave each cover one contiguous 1 KB (no bank
// conflicts); the e8m0 scales follow at byte 2048.
__host__ __device__ inline int img_off(int row, int g, int e) { return (e >> 4) * 1024 + (row * 4 + g) * 16 + (e & 15); }

__device__ inline v4f mfma(const v8i& a, const v8i& b, v4f c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, scale_a, 0, 127);
}

// Lane roles while converting one 128-element K chunk: lane = 16 kb + sub holds
// elements 32 kb + 2 sub and +1 (class v = sub / 4 in the fp4 B layout).
struct ConvLane {
  int kloc, kb, sub, cls, gdst, edst;
  float fcls, finv;
  __device__ ConvLane(int lane) {
    kb = lane >> 4;
    sub = lane & 15;
    kloc = 32 * kb + 2 * sub;
    cls = sub >> 2;
    fcls = cls == 0 ? 1.f : (cls == 1 ? -1.f : (cls == 2 ? -2.f : -4.f));
    finv = cls == 0 ? 0.f : 1.f / fcls;
    // fp8 A layout: group g holds K = 16 g + e (e < 16) and 64 + 16 g + (e - 16)
    gdst = kloc < 64 ? kloc / 16 : (kloc - 64) / 16;
    edst = kloc < 64 ? kloc % 16 : 16 + (kloc - 64) % 16;
  }
};

// Converts this lane's two values (already multiplied by the class factor) of
// token slot tt into the A image `ab` at the lane's K position; the 16 lanes of
// a DPP row hold one 32-element block.  Returns the lane's contribution to C.
template <class Ptr>
__device__ inline float convert_pair(const ConvLane& L, float t0, float t1, int tt, Ptr ab) {
  float mx = row16_max(fmaxf(fabsf(t0), fabsf(t1)));
  int ex;
  frexpf(mx, &ex);
  int E = ex - 8;                       // max / 2^E in [128, 256)
  E = E < -123 ? -123 : (E > 127 ? 127 : E);
  float u0 = ldexpf(t0, -E), u1 = ldexpf(t1, -E);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(u0, u1, 0, false);
  float h0 = __builtin_amdgcn_cvt_f32_fp8(hi, 0), h1 = __builtin_amdgcn_cvt_f32_fp8(hi, 1);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32((u0 - h0) * 16.f, (u1 - h1) * 16.f, 0, false);
  float l0 = __builtin_amdgcn_cvt_f32_fp8(lo, 0), l1 = __builtin_amdgcn_cvt_f32_fp8(lo, 1);
  const int mhi = 2 * tt, mlo = 2 * tt + 1;
  using U16 = typename std::conditional<std::is_same<Ptr, uint8_t*>::value, uint16_t, LB_GLOBAL uint16_t>::type;
  *reinterpret_cast<U16*>(ab + img_off(mhi, L.gdst, L.edst)) = (uint16_t)hi;
  *reinterpret_cast<U16*>(ab + img_off(mlo, L.gdst, L.edst)) = (uint16_t)lo;
  if (L.sub == 0) {
    ab[2048 + mhi * 4 + L.kb] = (uint8_t)(E + 127);
    ab[2048 + mlo * 4 + L.kb] = (uint8_t)(E + 127 - 4);
  }
  // quantised value of t (A / class factor), summed over the three {0, beta} classes
  return ldexpf((h0 + h1) + (l0 + l1) * 0.0625f, E) * L.finv;
}

// Reads lane (mr, gr)'s A operand and scale from an A image (LDS or global).
// Rows past the real tokens hold stale values: MFMA rows are independent and
// those rows of the result are never read.
template <class Ptr>
__device__ inline void load_a(Ptr ab, int mr, int gr, v8i& a, int& sc) {
  using V4 = typename std::conditional<std::is_same<Ptr, const uint8_t*>::value || std::is_same<Ptr, uint8_t*>::value,
                                      const v4i, const LB_GLOBAL v4i>::type;
  const v4i lo = *reinterpret_cast<V4*>(ab + img_off(mr, gr, 0));
  const v4i hi = *reinterpret_cast<V4*>(ab + img_off(mr, gr, 16));
  a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  sc = ab[2048 + mr * 4 + gr];
}


// ---------------------------------------------------------------------------
// V stage
// ---------------------------------------------------------------------------
// TM: token-count bucket of the launch (1, 2, 4, 8 or 16): per-token state is
// sized by TM, MFMA token blocks of 8 by TB.
template <int TM>
__device__ void v_item(const DecArgs& a, const DecEntry& Eg, const void* xv, int p, int grp, uint8_t* lds) {
  constexpr int TB = (TM + 7) / 8;
  constexpr int CTM = TM >= 8 ? 8 : 16;
  // snapshot of the entry: the table lives in global memory this kernel also
  // writes, so fields read in the loops would be re-loaded (and waited for)
  struct {
    int nkc, n, vct, nvg, pcoff;
    uint8_t* aimg;
    float* cpart;
  } E = {Eg.nkc, Eg.n, Eg.vct[p], Eg.nvg[p], Eg.pcoff[p], Eg.aimg, Eg.cpart};
  const PathDev P = Eg.p[p];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mr = lane & 15, gr = lane >> 4;
  const int cti = E.vct;
  const int ct0 = grp * cti;
  const int nct = min(cti, P.nct - ct0);
  const int T = a.T, n = E.n;
  const LB_GLOBAL uint16_t* x = gp(reinterpret_cast<const uint16_t*>(xv)) + (int64_t)a.t0 * n;
  const LB_GLOBAL uint32_t* vdec = gp(P.vdec);
  const LB_GLOBAL uint16_t* gsc = gp(P.g);
  const LB_GLOBAL uint16_t* lsc = gp(P.l);

  uint8_t* abuf = lds + wave * TB * kABytes;
  float* red = reinterpret_cast<float*>(lds + kWaves * TB * kABytes);   // [CTM*TB][16][16]
  float* cred = red + CTM * TB * 256;                                   // [16]
  float* cblk = cred + 16;                                              // [16 tokens * 32 blocks]

  ConvLane L(lane);
  v4f acc[CTM][TB];
#pragma unroll
  for (int c = 0; c < CTM; ++c)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[c][tb] = v4f{0.f, 0.f, 0.f, 0.f};
  float cpart[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) cpart[t] = 0.f;

  // software pipeline: the next chunk's sign words, activations and column
  // scales are in flight while this chunk converts and multiplies.  Loads are
  // unconditional (clamped index) and their raw values are not touched until
  // the next iteration: any use (even a select) makes the compiler wait, and
  // the in-order load counter would then drain everything in flight.
  uint32_t wcur[CTM], wnxt[CTM];
  uint32_t xcur[TM], xnxt[TM], gcur = 0, gnxt = 0;
  const bool even_n = (n & 1) == 0;
  auto fetch = [&](int kc, uint32_t* w, uint32_t* xp, uint32_t& gpair) {
    const LB_GLOBAL uint32_t* vp = vdec + ((int64_t)kc * P.nct + ct0) * 64 + lane;
#pragma unroll
    for (int c = 0; c < CTM; ++c) w[c] = vp[min(c, nct - 1) * 64];
    // lane l holds chunk elements 2l and 2l + 1 (L.kloc == 2 * lane)
    const int k0 = min(kc * kChunk + L.kloc, (n - 1) & ~1);   // even, and k0 + 1 stays inside the arena
    gpair = *reinterpret_cast<const LB_GLOBAL uint32_t*>(gsc + k0);
    if (even_n) {
#pragma unroll
      for (int t = 0; t < TM; ++t)
        xp[t] = *reinterpret_cast<const LB_GLOBAL uint32_t*>(x + (int64_t)min(t, T - 1) * n + k0);
    } else {
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const LB_GLOBAL uint16_t* xr = x + (int64_t)min(t, T - 1) * n;
        xp[t] = (uint32_t)xr[k0] | ((uint32_t)xr[min(k0 + 1, n - 1)] << 16);
      }
    }
  };
  auto compute = [&](int kc, const uint32_t* wc, const uint32_t* xc, uint32_t gc) {
    const int k0 = kc * kChunk + L.kloc;
    const bool v0 = k0 < n, v1 = k0 + 1 < n;
    const float g0 = v0 ? f16f((uint16_t)(gc & 0xffff)) * L.fcls : 0.f;
    const float g1 = v1 ? f16f((uint16_t)(gc >> 16)) * L.fcls : 0.f;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      uint8_t* ab = abuf + tb * kABytes;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = tb * 8 + tt;
        if (t < TM && t < T) {
          const float x0 = bf16f((uint16_t)(xc[t] & 0xffff)), x1 = bf16f((uint16_t)(xc[t] >> 16));
          cpart[t] += convert_pair(L, x0 * g0, x1 * g1, tt, ab);
        }
      }
    }
    wave_lds_fence();
    v8i A[TB];
    int sc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) load_a(abuf + tb * kABytes, mr, gr, A[tb], sc[tb]);
#pragma unroll
    for (int c = 0; c < CTM; ++c) {
      if (c < nct) {
        const v8i B = expand_signs(wc[c]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[c][tb] = mfma(A[tb], B, acc[c][tb], sc[tb]);
      }
    }
    wave_lds_fence();
  };
  // chunks go in pairs (kc, kc + 4) with the next pair's loads in flight: up to
  // three chunks ahead of the one being multiplied
  uint32_t w2cur[CTM], w2nxt[CTM], x2cur[TM], x2nxt[TM], g2cur = 0, g2nxt = 0;
  const int nkc = E.nkc;
  if (wave < nkc) fetch(wave, wcur, xcur, gcur);
  if (wave + kWaves < nkc) fetch(wave + kWaves, w2cur, x2cur, g2cur);
  for (int kc = wave; kc < nkc; kc += 2 * kWaves) {
    if (kc + 2 * kWaves < nkc) fetch(kc + 2 * kWaves, wnxt, xnxt, gnxt);
    if (kc + 3 * kWaves < nkc) fetch(kc + 3 * kWaves, w2nxt, x2nxt, g2nxt);
    compute(kc, wcur, xcur, gcur);
    if (kc + kWaves < nkc) compute(kc + kWaves, w2cur, x2cur, g2cur);
#pragma unroll
    for (int c = 0; c < CTM; ++c) {
      wcur[c] = wnxt[c];
      w2cur[c] = w2nxt[c];
    }
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      xcur[t] = xnxt[t];
      x2cur[t] = x2nxt[t];
    }
    gcur = gnxt;
    g2cur = g2nxt;
  }

  // fixed-order combine across waves: wave 0 stores, waves 1..3 add in turn
  float cw[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) cw[t] = wave_sum(cpart[t]);
  __syncthreads();
  for (int wv = 0; wv < kWaves; ++wv) {
    if (wave == wv) {
#pragma unroll
      for (int c = 0; c < CTM; ++c) {
        if (c < nct) {
#pragma unroll
          for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float* dst = red + ((c * TB + tb) * 16 + 4 * gr + i) * 16 + mr;
              *dst = (wv == 0 ? 0.f : *dst) + acc[c][tb][i];
            }
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int t = 0; t < TM; ++t) cred[t] = (wv == 0 ? 0.f : cred[t]) + cw[t];
      }
    }
    __syncthreads();
  }

  // z' = (D_hi + D_lo + C) o l, converted into the U stage's A images: each
  // 16-lane row takes one (token, 32-latent block).  The group owning the last
  // column tile also writes the zero blocks that pad the path's last chunk.
  const int j0 = 16 * ct0;                         // a multiple of 32 (groups hold an even tile count)
  const int last = grp == E.nvg - 1;
  const int nchunk = (P.r + kChunk - 1) / kChunk;
  const int nblk = last ? 4 * nchunk - j0 / 32 : (nct + 1) / 2;
  const int row = tid >> 4;                        // 16 rows of 16 lanes
  ConvLane LR(lane);                               // lane role inside its 16-lane row: sub = lane & 15
  for (int u = row; u < T * nblk; u += 16) {
    const int t = u / nblk, blk = u % nblk;
    const int jj = j0 + 32 * blk + 2 * LR.sub;     // this lane's two latents jj, jj + 1
    const int tb = t / 8, tt = t % 8;
    float v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = jj + q;
      v[q] = 0.f;
      if (j < P.r) {
        const int c = (j - j0) / 16, col = j % 16;
        const float* base = red + (c * TB + tb) * 256;
        const float z = (base[(2 * tt) * 16 + col] + base[(2 * tt + 1) * 16 + col]) + cred[t];
        v[q] = z * f16f(lsc[j]) * LR.fcls;
      }
    }
    ConvLane LK(((jj % kChunk) / 32) * 16 + LR.sub);   // K position inside the 128-latent chunk
    uint8_t* ab = E.aimg + ((int64_t)(E.pcoff + jj / kChunk) * TB + tb) * kABytes;   // global
    const float cc = row16_sum(convert_pair(LK, v[0], v[1], tt, gp(ab)));
    if (LR.sub == 0) cblk[u] = cc;
  }
  __syncthreads();
  if (tid < T) {
    float s = 0.f;
    for (int blk = 0; blk < nblk; ++blk) s += cblk[tid * nblk + blk];
    gp(E.cpart)[(p * kMaxGroups + grp) * 16 + tid] = s;
  }
}

// One workgroup per V item; items are ordered longest first so the hardware
// dispatcher balances the load.
template <int TM>
__global__ void __launch_bounds__(kThreads, 2) k_decode_v(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const WorkItem wi = a.items[blockIdx.x];
  const void* x = a.xs ? a.xs[wi.entry] : a.x0;
  v_item<TM>(a, a.entries[wi.entry], x, wi.path, wi.group, lds);
}

// ---------------------------------------------------------------------------
// U stage
// ---------------------------------------------------------------------------
// Item = (entry, up to 16 quads of 4 row tiles); each wave takes every 4th
// quad (kQW of them) and runs unit-major: for each 128-latent unit (path 0's,
// then path 1's) it multiplies the unit's fp8 A operand (written by the V stage,
// read from global memory one unit ahead) against the sign words of its quads.
// The sign words stream through a private ring of kUDepth 1 KB LDS slots, one
// direct-to-LDS load per (unit, quad) step issued kUDepth - 1 steps ahead; each
// step's words are read from the ring one step ahead of the MFMAs.  Every step
// issues exactly one load (past the end of the work it re-reads its last block
// into a dead slot), so counting outstanding vector-memory operations tells
// when a slot has landed.  Row scales are loaded and outputs stored outside
// the stream.
constexpr int kUDepth = 12;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_block + 16 l.
__device__ inline void dma16(const LB_GLOBAL void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)lds_block, 16, 0, 0);
}
// Waits until at most VM vector-memory operations of this wave are outstanding
// (LDS and export counters untouched).  The memory clobbers keep the compiler
// from moving memory accesses across the wait.
template <int VM>
__device__ inline void vm_wait() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  constexpr int imm = (VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  asm volatile("" ::: "memory");
}
// Waits for this wave's outstanding LDS reads.
__device__ inline void lds_reads_wait() {
  constexpr int imm = 15 | (7 << 4) | (0 << 8) | (3 << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  asm volatile("" ::: "memory");
}

constexpr int kUSlotsPerCU = 2;   // U workgroups per CU (two waves per SIMD)

// Quads per wave and batch of a U segment: as many as fit next to the operands
// of the NPC units (NPC == 0: one unit's) in about 150 registers.
constexpr int u_quads_per_batch(int npc, int tb) {
  const int opr = (npc > 0 ? npc : 1) * tb * 9 + 4;
  const int per = 24 * tb + 4;
  return opr + 4 * per <= 150 ? 4 : opr + 2 * per <= 150 ? 2 : 1;
}

// One U-stage segment: quads [qa, qb) of one entry, on this workgroup.
//
// Each wave takes every 4th quad and runs batches of kQW of them.  The data of
// a batch streams through the wave's ring of kUDepth 1 KB LDS slots as steps,
// one direct-to-LDS load each, issued kUDepth - 1 steps ahead: first the
// batch's row scales, then for each 128-latent unit (path 0's, then path 1's)
// the sign words of each quad.  The operands of the NPC units (NPC == 0: any
// unit count, read from global memory unit by unit) are loaded before the
// stream starts and stay in registers.
//
// The in-order vector-memory counter tells when a slot has landed: each step
// issues exactly one load (past the end of the work it re-reads its last
// block into a dead slot), and each batch ends with exactly kStores output
// stores (lanes without an output write to a private sink), which the waits of
// the next kUDepth - 2 steps allow for.
template <int TM, int NPC>
__device__ __attribute__((always_inline)) inline void u_segment(const DecArgs& a, const DecEntry& Eg, int e, int qa,
                                                               int qb, uint8_t* ring) {
  constexpr int TB = (TM + 7) / 8;
  constexpr int kQW = u_quads_per_batch(NPC, TB);              // quads per wave per batch
  constexpr int kQQ = TM == 1 ? 1 : 2;                         // token slots per lane and block
  constexpr int kStores = kQW * 4 * TB * kQQ;                  // output stores of one batch
  static_assert(kUDepth - 2 + kStores < 64, "vmcnt range");
  // snapshot of the entry (the table is re-read otherwise)
  const int np = Eg.np, m = Eg.m, uw = Eg.uw, npc = NPC > 0 ? NPC : Eg.npc;
  const int npc0 = np > 1 ? Eg.pcoff[1] : npc;
  const int woff1 = Eg.woff[1];
  const LB_GLOBAL uint8_t* aimg = gp(static_cast<const uint8_t*>(Eg.aimg));
  const float* cpart = Eg.cpart;
  const int nvg0 = Eg.nvg[0], nvg1 = Eg.nvg[1];
  const LB_GLOBAL uint8_t* ubase = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.udec));
  const LB_GLOBAL uint8_t* hb0 = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.p[0].h));
  const LB_GLOBAL uint8_t* hb1 = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(np > 1 ? Eg.p[1].h : Eg.p[0].h));
  void* yv = a.xs ? a.ys[e] : a.y0;
  LB_GLOBAL uint16_t* y = gp(reinterpret_cast<uint16_t*>(yv)) + (int64_t)a.t0 * m;
  const int T = a.T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mr = lane & 15, gr = lane >> 4;
  LB_GLOBAL uint16_t* sink = gp(a.sink) + ((int64_t)blockIdx.x * kWaves + wave) * 128 + (lane & 15) * 8;
  const int nmine = qa + wave < qb ? (qb - qa - wave + kWaves - 1) / kWaves : 0;   // quads of this wave
  const int nb = (nmine + kQW - 1) / kQW;                                          // its batches
  auto quad = [&](int jj) __attribute__((always_inline)) { return qa + wave + kWaves * jj; };
  auto valid = [&](int b, int j) __attribute__((always_inline)) { return b * kQW + j < nmine; };

  // correction sums C_p per token (V stage partials over its column groups)
  float cval[2][TB][2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int t = tb * 8 + 2 * gr + q;
        float sum = 0.f;
        if (p < np && t < T && t < TM)
          for (int g = 0; g < (p ? nvg1 : nvg0); ++g) sum += gp(cpart)[(p * kMaxGroups + g) * 16 + t];
        cval[p][tb][q] = sum;
      }
  constexpr int NA = NPC > 0 ? NPC : 1;
  v8i A[NA][TB];
  int sc[NA][TB];
  auto load_img = [&](int u, v8i* Au, int* su) __attribute__((always_inline)) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) load_a(aimg + (int64_t)(u * TB + tb) * kABytes, mr, gr, Au[tb], su[tb]);
  };

  // issue cursor: batch ib; unit iu (-1: the batch's row-scale step); quad ij
  int ib = 0, iu = -1, ij = 0;
  const LB_GLOBAL uint8_t* last = ubase + lane * 16;
  auto issue = [&](int slot) __attribute__((always_inline)) {
    if (ib < nb) {
      if (iu < 0) {
        // row scales: lane l -> quad (l / 16) % kQW of the batch, path (l / 8) % 2, rows 8 (l % 8) .. + 7
        const int jj = min(ib * kQW + (lane >> 4) % kQW, nmine - 1);
        last = ((lane >> 3) & 1 ? hb1 : hb0) + (int64_t)quad(jj) * 128 + (lane & 7) * 16;
        iu = 0;
      } else {
        const int w0 = iu < npc0 ? 4 * iu : woff1 + 4 * (iu - npc0);
        last = ubase + ((int64_t)quad(ib * kQW + ij) * uw + w0) * 256 + lane * 16;
        if (++ij == kQW || ib * kQW + ij >= nmine) {
          ij = 0;
          if (++iu == npc) {
            iu = -1;
            ++ib;
          }
        }
      }
    }
    dma16(last, ring + slot * 1024);
  };

  // prologue: the first kUDepth - 1 steps, then the operands; one wait covers all
#pragma unroll
  for (int k = 0; k < kUDepth - 1; ++k) issue(k);
  if (NPC > 0) {
#pragma unroll
    for (int u = 0; u < NA; ++u) load_img(u, A[u], sc[u]);
  }
  vm_wait<0>();

  v4f acc[kQW][4][TB];
  float part[kQW][4][TB][2];
  uint32_t hraw[kQW][4];                           // (h0 | h1 << 16) of row mr of each row tile
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kQW; ++j)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[j][rt][tb] = v4f{0.f, 0.f, 0.f, 0.f};
  };
  // part (+)= h_p (D_hi + D_lo + C_p); lane (mr, gr) holds MFMA rows 4 gr .. 4 gr + 3
  // = (hi, lo) of tokens tb * 8 + 2 gr + {0, 1}, column mr = output row
  auto fold = [&](int p, bool first) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kQW; ++j)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float h = f16f((uint16_t)(p ? hraw[j][rt] >> 16 : hraw[j][rt] & 0xffff));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const float v = h * ((acc[j][rt][tb][2 * qq] + acc[j][rt][tb][2 * qq + 1]) + cval[p][tb][qq]);
            part[j][rt][tb][qq] = first ? v : part[j][rt][tb][qq] + v;
          }
      }
  };

  // consumer: waits for step s's slot (see above) and returns it
  int s = 0, since_store = kUDepth;
  auto next_step = [&]() __attribute__((always_inline)) {
    lds_reads_wait();                              // the slot reloaded next was read last step
    issue((s + kUDepth - 1) % kUDepth);
    if (since_store < kUDepth - 2) vm_wait<kUDepth - 2 + kStores>();
    else vm_wait<kUDepth - 2>();
    ++since_store;
    const uint8_t* slot = ring + (s % kUDepth) * 1024;
    ++s;
    return slot;
  };
  auto unit = [&](int b, int u, const v8i* Au, const int* su) __attribute__((always_inline)) {
    if (u == npc0 && u > 0) {                      // path 1 starts: fold path 0
      fold(0, true);
      zero_acc();
    }
#pragma unroll
    for (int j = 0; j < kQW; ++j) {
      if (valid(b, j)) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(next_step() + lane * 16);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const v8i B = expand_signs(w[rt]);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[j][rt][tb] = mfma(Au[tb], B, acc[j][rt][tb], su[tb]);
        }
      }
    }
  };
  for (int b = 0; b < nb; ++b) {
    {  // the batch's row scales: [quad j][path][64 rows] fp16 in the slot
      const uint16_t* hs = reinterpret_cast<const uint16_t*>(next_step());
#pragma unroll
      for (int j = 0; j < kQW; ++j)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          hraw[j][rt] = (uint32_t)hs[(j * 2) * 64 + rt * 16 + mr] | ((uint32_t)hs[(j * 2 + 1) * 64 + rt * 16 + mr] << 16);
    }
    zero_acc();
    if (NPC > 0) {
#pragma unroll
      for (int u = 0; u < NA; ++u) unit(b, u, A[u], sc[u]);
    } else {
      for (int u = 0; u < npc; ++u) {
        load_img(u, A[0], sc[0]);
        vm_wait<0>();                              // (keeps the count exact; the slow path)
        unit(b, u, A[0], sc[0]);
      }
    }
    if (npc0 < npc) fold(1, false);
    else fold(0, true);
    // y: lane (mr, gr) holds tokens tb * 8 + 2 gr + {0, 1} of output row mr of each row
    // tile; every store is issued (kStores of them), lanes without an output hit the sink
#pragma unroll
    for (int j = 0; j < kQW; ++j)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int i = (4 * quad(b * kQW + j) + rt) * 16 + mr;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int qq = 0; qq < kQQ; ++qq) {
            const int t = tb * 8 + 2 * gr + qq;
            const bool ok = valid(b, j) && i < m && t < T;
            LB_GLOBAL uint16_t* dst = ok ? y + (uint32_t)(t * m + i) : sink + (gr & 3) * 2 + qq;
            *dst = bf16_bits(part[j][rt][tb][qq]);
          }
      }
    since_store = 0;
  }
  vm_wait<0>();                                    // no direct-to-LDS load may still be in flight
}

template <int TM>
__global__ void __launch_bounds__(kThreads, 2) k_decode_u(DecArgs a) {
  constexpr int TB = (TM + 7) / 8;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const UItem it = a.uitems[blockIdx.x];
  uint8_t* ring = lds + (threadIdx.x >> 6) * (kUDepth * 1024);
  int e = (int)it.entry, qa = (int)it.quad0, left = (int)it.count;
  while (left > 0 && e < a.nentries) {
    const DecEntry& Eg = a.entries[e];
    const int nq = (Eg.nrt + 3) / 4;
    const int qb = min(nq, qa + left);
    const int npc = Eg.npc;
    if (TB == 1) {
      switch (npc) {
        case 1: u_segment<TM, 1>(a, Eg, e, qa, qb, ring); break;
        case 2: u_segment<TM, 2>(a, Eg, e, qa, qb, ring); break;
        case 3: u_segment<TM, 3>(a, Eg, e, qa, qb, ring); break;
        case 4: u_segment<TM, 4>(a, Eg, e, qa, qb, ring); break;
        case 5: u_segment<TM, 5>(a, Eg, e, qa, qb, ring); break;
        case 6: u_segment<TM, 6>(a, Eg, e, qa, qb, ring); break;
        case 7: u_segment<TM, 7>(a, Eg, e, qa, qb, ring); break;
        case 8: u_segment<TM, 8>(a, Eg, e, qa, qb, ring); break;
        default: u_segment<TM, 0>(a, Eg, e, qa, qb, ring); break;
      }
    } else {
      switch (npc) {
        case 1: u_segment<TM, 1>(a, Eg, e, qa, qb, ring); break;
        case 2: u_segment<TM, 2>(a, Eg, e, qa, qb, ring); break;
        case 3: u_segment<TM, 3>(a, Eg, e, qa, qb, ring); break;
        case 4: u_segment<TM, 4>(a, Eg, e, qa, qb, ring); break;
        default: u_segment<TM, 0>(a, Eg, e, qa, qb, ring); break;
      }
    }
    left -= qb - qa;
    qa = 0;
    ++e;
  }
}

size_t decode_lds_bytes(int T) {
  const int tb = (decode_bucket(T) + 7) / 8;
  return (size_t)kWaves * tb * kABytes + (size_t)decode_ct_max(T) * tb * 256 * 4 + (16 + 16 * 32) * 4;
}

}  // namespace

hipError_t launch_decode_v(const DecArgs& a, int nitems, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  const int tm = decode_bucket(a.T);
  const size_t lds = decode_lds_bytes(a.T);
  switch (tm) {
    case 1: hipLaunchKernelGGL(k_decode_v<1>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL(k_decode_v<2>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL(k_decode_v<4>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    case 8: hipLaunchKernelGGL(k_decode_v<8>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    default: hipLaunchKernelGGL(k_decode_v<16>, dim3(nitems), dim3(kThreads), lds, st, a); break;
  }
  return hipGetLastError();
}

size_t decode_u_lds_bytes(const int* npc, int count, int T) {
  (void)npc;
  (void)count;
  (void)T;
  return (size_t)kWaves * kUDepth * 1024;
}

int decode_u_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus * kUSlotsPerCU;
}

hipError_t launch_decode_u(const DecArgs& a, int nitems, size_t lds, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  switch (decode_bucket(a.T)) {
    case 1: hipLaunchKernelGGL(k_decode_u<1>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    case 2: hipLaunchKernelGGL(k_decode_u<2>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    case 4: hipLaunchKernelGGL(k_decode_u<4>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    case 8: hipLaunchKernelGGL(k_decode_u<8>, dim3(nitems), dim3(kThreads), lds, st, a); break;
    default: hipLaunchKernelGGL(k_decode_u<16>, dim3(nitems), dim3(kThreads), lds, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace lb

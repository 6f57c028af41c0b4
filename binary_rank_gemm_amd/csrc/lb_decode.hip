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

#include <type_traits>

namespace lb {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;

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
  *reinterpret_cast<U16*>(ab + (mhi * 4 + L.gdst) * 32 + L.edst) = (uint16_t)hi;
  *reinterpret_cast<U16*>(ab + (mlo * 4 + L.gdst) * 32 + L.edst) = (uint16_t)lo;
  if (L.sub == 0) {
    ab[2048 + mhi * 4 + L.kb] = (uint8_t)(E + 127);
    ab[2048 + mlo * 4 + L.kb] = (uint8_t)(E + 127 - 4);
  }
  // quantised value of t (A / class factor), summed over the three {0, beta} classes
  return ldexpf((h0 + h1) + (l0 + l1) * 0.0625f, E) * L.finv;
}

// Reads lane (mr, gr)'s A operand and scale from an A image (LDS or global).
template <class Ptr>
__device__ inline void load_a(Ptr ab, int mr, int gr, int rows, v8i& a, int& sc) {
  const int mc = min(mr, rows - 1);   // rows >= 1; the load is unconditional, the value is selected
  using V8 = typename std::conditional<std::is_same<Ptr, const uint8_t*>::value || std::is_same<Ptr, uint8_t*>::value,
                                      const v8i, const LB_GLOBAL v8i>::type;
  const v8i v = *reinterpret_cast<V8*>(ab + (mc * 4 + gr) * 32);
  const int s = ab[2048 + mc * 4 + gr];
  const bool ok = mr < rows;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = ok ? v[i] : 0;
  sc = ok ? s : 127;
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
    for (int tb = 0; tb < TB; ++tb) load_a(abuf + tb * kABytes, mr, gr, 2 * min(8, T - tb * 8), A[tb], sc[tb]);
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
// The item's fp8 A operand images (written by the V stage) are staged in LDS;
// each wave owns every 4th row tile of the item and walks them in groups of 4
// (acc[4][path][token block]).  When all images fit (npc * TB <= kUImgMax)
// they are staged once and the next group's sign words and row scales are in
// flight while the current group multiplies; otherwise every group runs the
// images in passes.
constexpr int kUImgMax = 8;

template <int TM>
struct UCtx {
  static constexpr int TB = (TM + 7) / 8;
  int np, nrt, npc, m, uw, pcoff1, woff[2], W[2];
  const uint32_t* udec;
  const uint16_t* h[2];
  int T, rt0, nmine, nunits, mr, gr, lane;
  float cval[2][TB][2];
  LB_GLOBAL uint16_t* y;

  // word offset (inside a row tile's block) and lane validity of unit u
  __device__ void unit(int u, int& off, bool& ok, int& p, int& tb) const {
    const int pc = u / TB;
    tb = u % TB;
    p = (np > 1 && pc >= pcoff1) ? 1 : 0;
    const int w4 = 4 * (pc - (p ? pcoff1 : 0));
    off = ((p ? woff[1] : woff[0]) + w4) * 16;
    ok = w4 + gr < (p ? W[1] : W[0]);
  }
  __device__ void load_words(int grp, int u0, int nu, uint32_t (*w)[kUImgMax], uint32_t (*hv)[2]) const {
    const LB_GLOBAL uint32_t* ud = gp(udec) + lane;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rt = min(rt0 + 4 * (4 * grp + k), nrt - 1);
      const LB_GLOBAL uint32_t* blk = ud + (int64_t)rt * uw * 16;
#pragma unroll
      for (int q = 0; q < kUImgMax; ++q) {
        int off, p, tb;
        bool ok;
        unit(u0 + min(q, nu - 1), off, ok, p, tb);
        w[k][q] = blk[off];
      }
      const int i = min(rt * 16 + mr, m - 1);
      hv[k][0] = gp(h[0])[i];
      hv[k][1] = gp(h[np > 1 ? 1 : 0])[i];
    }
  }
  __device__ void multiply(int grp, int u0, int nu, const uint32_t (*w)[kUImgMax], const uint8_t* imgs,
                           v4f (*acc)[2][TB]) const {
#pragma unroll
    for (int q = 0; q < kUImgMax; ++q) {
      if (q < nu) {
        int off, p, tb;
        bool ok;
        unit(u0 + q, off, ok, p, tb);
        v8i A;
        int sc;
        load_a(imgs + q * kABytes, mr, gr, 2 * min(8, T - tb * 8), A, sc);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (4 * grp + k < nmine) {
            const v8i B = expand_signs(ok ? w[k][q] : 0u);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
              for (int tbb = 0; tbb < TB; ++tbb)
                if (pp == p && tbb == tb) acc[k][pp][tbb] = mfma(A, B, acc[k][pp][tbb], sc);
          }
        }
      }
    }
  }
  // y = sum_p h_p (D_hi + D_lo + C_p) for the group's row tiles
  __device__ void epilogue(int grp, const uint32_t (*hv)[2], v4f (*acc)[2][TB]) const {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rt = rt0 + 4 * (4 * grp + k);
      const int i = rt * 16 + mr;
      if (4 * grp + k < nmine && i < m) {
        const float h0 = f16f((uint16_t)hv[k][0]);
        const float h1 = np > 1 ? f16f((uint16_t)hv[k][1]) : 0.f;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int t = tb * 8 + 2 * gr + q;
            if (t < T) {
              float v = h0 * ((acc[k][0][tb][2 * q] + acc[k][0][tb][2 * q + 1]) + cval[0][tb][q]);
              if (np > 1) v += h1 * ((acc[k][1][tb][2 * q] + acc[k][1][tb][2 * q + 1]) + cval[1][tb][q]);
              y[(int64_t)t * m + i] = f32_to_bf16_rne(v);
            }
          }
      }
    }
  }
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline void stage_images(uint8_t* lds, const uint8_t* aimg, int u0, int nu) {
  const LB_GLOBAL u32x4* src = reinterpret_cast<const LB_GLOBAL u32x4*>(gp(aimg) + (int64_t)u0 * kABytes);
  u32x4* dst = reinterpret_cast<u32x4*>(lds);
  for (int i = threadIdx.x; i < nu * (kABytes / 16); i += kThreads) dst[i] = src[i];
}

template <int TM>
__device__ void u_item(const DecArgs& a, const DecEntry& Eg, void* yv, int rg, uint8_t* lds) {
  using Ctx = UCtx<TM>;
  constexpr int TB = Ctx::TB;
  Ctx c;
  c.np = Eg.np; c.nrt = Eg.nrt; c.npc = Eg.npc; c.m = Eg.m; c.uw = Eg.uw; c.pcoff1 = Eg.pcoff[1];
  c.woff[0] = Eg.woff[0]; c.woff[1] = Eg.woff[1]; c.W[0] = Eg.p[0].W; c.W[1] = Eg.p[1].W;
  c.udec = Eg.udec; c.h[0] = Eg.p[0].h; c.h[1] = Eg.p[1].h;
  const uint8_t* aimg = Eg.aimg;
  const float* cpart = Eg.cpart;
  const int nvg0 = Eg.nvg[0], nvg1 = Eg.nvg[1];
  const int tid = threadIdx.x, wave = tid >> 6;
  c.lane = tid & 63; c.mr = c.lane & 15; c.gr = c.lane >> 4;
  c.T = a.T;
  c.nunits = c.npc * TB;
  c.y = gp(reinterpret_cast<uint16_t*>(yv)) + (int64_t)a.t0 * c.m;
  c.rt0 = rg * kDecodeRowTilesPerItem + wave;
  c.nmine = c.rt0 < c.nrt ? min(kDecodeRowTilesPerItem / kWaves, (c.nrt - c.rt0 + kWaves - 1) / kWaves) : 0;
  const int ngroups = (c.nmine + 3) / 4;
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int t = tb * 8 + 2 * c.gr + q;
        float s = 0.f;
        if (p < c.np && t < c.T && t < TM)
          for (int g = 0; g < (p ? nvg1 : nvg0); ++g) s += gp(cpart)[(p * kMaxGroups + g) * 16 + t];
        c.cval[p][tb][q] = s;
      }

  if (c.nunits <= kUImgMax) {
    stage_images(lds, aimg, 0, c.nunits);
    __syncthreads();
    uint32_t wcur[4][kUImgMax], wnxt[4][kUImgMax], hcur[4][2], hnxt[4][2];
    if (ngroups > 0) c.load_words(0, 0, c.nunits, wcur, hcur);
    for (int grp = 0; grp < ngroups; ++grp) {
      if (grp + 1 < ngroups) c.load_words(grp + 1, 0, c.nunits, wnxt, hnxt);
      v4f acc[4][2][TB];
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[k][p][tb] = v4f{0.f, 0.f, 0.f, 0.f};
      c.multiply(grp, 0, c.nunits, wcur, lds, acc);
      c.epilogue(grp, hcur, acc);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int q = 0; q < kUImgMax; ++q) wcur[k][q] = wnxt[k][q];
        hcur[k][0] = hnxt[k][0];
        hcur[k][1] = hnxt[k][1];
      }
    }
    return;
  }
  // general path: every group runs the operand images in passes (all waves
  // take part in every pass because the staging is shared)
  constexpr int kMaxGroupsPerWave = kDecodeRowTilesPerItem / kWaves / 4;
  for (int grp = 0; grp < kMaxGroupsPerWave; ++grp) {
    v4f acc[4][2][TB];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[k][p][tb] = v4f{0.f, 0.f, 0.f, 0.f};
    uint32_t w[4][kUImgMax], hv[4][2];
    for (int u0 = 0; u0 < c.nunits; u0 += kUImgMax) {
      const int nu = min(kUImgMax, c.nunits - u0);
      __syncthreads();
      stage_images(lds, aimg, u0, nu);
      __syncthreads();
      if (grp < ngroups) {
        c.load_words(grp, u0, nu, w, hv);
        c.multiply(grp, u0, nu, w, lds, acc);
      }
    }
    if (grp < ngroups) c.epilogue(grp, hv, acc);
  }
}

// One workgroup per U item (kDecodeRowTilesPerItem row tiles of 16 output rows).
template <int TM>
__global__ void __launch_bounds__(kThreads, 2) k_decode_u(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const WorkItem wi = a.items[blockIdx.x];
  void* y = a.xs ? a.ys[wi.entry] : a.y0;
  u_item<TM>(a, a.entries[wi.entry], y, wi.group, lds);
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

hipError_t launch_decode_u(const DecArgs& a, int nitems, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  const size_t lds = (size_t)kUImgMax * kABytes;
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

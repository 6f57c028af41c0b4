// Fused decode forward (few tokens, bf16 I/O) over a list of linears.
//
// Computes, for every entry and path p, the factorised order of the paper
// notes ("LittleBit: Ultra Low-Bit Quantization via Latent Factorization",
// section "Key design"): t = x o g_p, z_p = t V_p, z'_p = z_p o l_p, and then
// y = sum_p (z'_p U_p^T) o h_p (section "Residual compensation" for the sum).
//
// One persistent launch runs a queue of work items:
//   V item (entry, path, column group): z'_p for up to 16 column tiles of 16
//     latents, reducing over all d_in rows; the four waves split the rows and
//     combine their partial sums in LDS in a fixed order (deterministic).
//   U item (entry, 256 output rows): waits until every V item of its entry
//     has published z', then produces y for its rows, both paths.
// All V items precede all U items in the queue, so a waiting U item only ever
// waits for items already held by running workgroups.
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

namespace lb {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kABytes = 2048 + 64;   // one A operand image: 16 rows x 4 groups x 32 B + scales
constexpr int kUnitsPerPass = 8;     // U-stage A images resident in LDS at once

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

__device__ inline void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

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
// token slot tt into the A image `ab`; returns the lane's contribution to C.
__device__ inline float convert_pair(const ConvLane& L, float t0, float t1, int tt, uint8_t* ab) {
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
  *reinterpret_cast<uint16_t*>(ab + (mhi * 4 + L.gdst) * 32 + L.edst) = (uint16_t)hi;
  *reinterpret_cast<uint16_t*>(ab + (mlo * 4 + L.gdst) * 32 + L.edst) = (uint16_t)lo;
  if (L.sub == 0) {
    ab[2048 + mhi * 4 + L.kb] = (uint8_t)(E + 127);
    ab[2048 + mlo * 4 + L.kb] = (uint8_t)(E + 127 - 4);
  }
  // quantised value of t (A / class factor), summed over the three {0, beta} classes
  return ldexpf((h0 + h1) + (l0 + l1) * 0.0625f, E) * L.finv;
}

// Reads lane (mr, gr)'s A operand and scale from an A image.
__device__ inline void load_a(const uint8_t* ab, int mr, int gr, int rows, v8i& a, int& sc) {
  if (mr < rows) {
    a = *reinterpret_cast<const v8i*>(ab + (mr * 4 + gr) * 32);
    sc = ab[2048 + mr * 4 + gr];
  } else {
    for (int i = 0; i < 8; ++i) a[i] = 0;
    sc = 127;
  }
}

__device__ inline bool spin_until(const unsigned int* flag, unsigned int want, int limit, Control* ctl) {
  for (int it = 0; it < limit; ++it) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(&ctl->err, 1u);
  return false;
}

// ---------------------------------------------------------------------------
// V stage
// ---------------------------------------------------------------------------
template <int TB>
__device__ void v_item(const DecArgs& a, const DecEntry& E, unsigned int e_idx, const void* xv, int p, int grp,
                       unsigned int gen, uint8_t* lds) {
  constexpr int CTM = TB == 1 ? 16 : 8;
  const PathDev& P = E.p[p];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mr = lane & 15, gr = lane >> 4;
  const int cti = E.vct[p];
  const int ct0 = grp * cti;
  const int nct = min(cti, P.nct - ct0);
  const int T = a.T, n = E.n;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(xv) + (int64_t)a.t0 * n;

  uint8_t* abuf = lds + wave * TB * kABytes;
  float* red = reinterpret_cast<float*>(lds + kWaves * TB * kABytes);   // [CTM*TB][16][16]
  float* cred = red + CTM * TB * 256;                                   // [16]

  ConvLane L(lane);
  v4f acc[CTM][TB];
#pragma unroll
  for (int c = 0; c < CTM; ++c)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[c][tb] = v4f{0.f, 0.f, 0.f, 0.f};
  float cpart[TB * 8];
#pragma unroll
  for (int t = 0; t < TB * 8; ++t) cpart[t] = 0.f;

  for (int kc = wave; kc < E.nkc; kc += kWaves) {
    uint32_t w[CTM];
    const uint32_t* vp = P.vdec + ((int64_t)kc * P.nct + ct0) * 64 + lane;
#pragma unroll
    for (int c = 0; c < CTM; ++c) w[c] = c < nct ? vp[c * 64] : 0u;

    const int k0 = kc * kChunk + L.kloc;
    const float g0 = k0 < n ? f16f(P.g[k0]) * L.fcls : 0.f;
    const float g1 = k0 + 1 < n ? f16f(P.g[k0 + 1]) * L.fcls : 0.f;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      uint8_t* ab = abuf + tb * kABytes;
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = tb * 8 + tt;
        if (t < T) {
          const float x0 = k0 < n ? bf16f(x[(int64_t)t * n + k0]) : 0.f;
          const float x1 = k0 + 1 < n ? bf16f(x[(int64_t)t * n + k0 + 1]) : 0.f;
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
        const v8i B = expand_signs(w[c]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[c][tb] = mfma(A[tb], B, acc[c][tb], sc[tb]);
      }
    }
    wave_lds_fence();
  }

  // fixed-order combine across waves: wave 0 stores, waves 1..3 add in turn
  float cw[TB * 8];
#pragma unroll
  for (int t = 0; t < TB * 8; ++t) cw[t] = wave_sum(cpart[t]);
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
        for (int t = 0; t < TB * 8; ++t) cred[t] = (wv == 0 ? 0.f : cred[t]) + cw[t];
      }
    }
    __syncthreads();
  }
  // z' = (D_hi + D_lo + C) o l for the group's columns
  const int total = nct * 16 * T;
  for (int idx = tid; idx < total; idx += kThreads) {
    const int c = idx / (16 * T);
    const int rem = idx - c * 16 * T;
    const int t = rem / 16, col = rem % 16;
    const int j = 16 * (ct0 + c) + col;
    if (j < P.r) {
      const int tb = t / 8, tt = t % 8;
      const float* base = red + (c * TB + tb) * 256;
      const float z = (base[(2 * tt) * 16 + col] + base[(2 * tt + 1) * 16 + col]) + cred[t];
      E.zbuf[((int64_t)p * T + t) * E.rpad + j] = z * f16f(P.l[j]);
    }
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    unsigned int prev = atomicAdd(&a.counters[e_idx], 1u);
    if (prev + 1 == (unsigned int)E.nv) {
      __hip_atomic_store(&a.counters[e_idx], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
      __hip_atomic_store(&a.ready[e_idx], gen + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// U stage
// ---------------------------------------------------------------------------
template <int TB>
__device__ void u_item(const DecArgs& a, const DecEntry& E, unsigned int e_idx, void* yv, int rg, unsigned int gen,
                       uint8_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mr = lane & 15, gr = lane >> 4;
  const int T = a.T, m = E.m;
  __shared__ int s_ok;
  if (tid == 0) {
    bool ok = spin_until(&a.ready[e_idx], gen + 1u, a.spin_limit, a.ctl);
    __threadfence();
    s_ok = ok;
  }
  __syncthreads();
  if (!s_ok) return;

  uint8_t* aimg = lds;                                                    // [kUnitsPerPass][kABytes]
  float* cu = reinterpret_cast<float*>(lds + kUnitsPerPass * kABytes);   // [2][16] C per path, token
  float* cw = cu + 32;                                                    // [kWaves][2][16]
  ConvLane L(lane);

  int nchunk[2] = {0, 0};
  for (int p = 0; p < E.np; ++p) nchunk[p] = (E.p[p].r + kChunk - 1) / kChunk;
  const int nunits = (nchunk[0] + nchunk[1]) * TB;

  v4f acc[4][2][TB];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[k][p][tb] = v4f{0.f, 0.f, 0.f, 0.f};
  float cpart[2][TB * 8];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int t = 0; t < TB * 8; ++t) cpart[p][t] = 0.f;

  for (int u0 = 0; u0 < nunits; u0 += kUnitsPerPass) {
    const int npass = min(kUnitsPerPass, nunits - u0);
    // convert this pass's units: unit u -> (p, chunk c, token block tb)
    for (int k = wave; k < npass; k += kWaves) {
      const int u = u0 + k;
      const int tbu = u % TB, pc = u / TB;
      const int p = pc < nchunk[0] ? 0 : 1, c = pc < nchunk[0] ? pc : pc - nchunk[0];
      const PathDev& P = E.p[p];
      uint8_t* ab = aimg + k * kABytes;
      const int j0 = c * kChunk + L.kloc;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (tb == tbu) {
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const int t = tb * 8 + tt;
            if (t < T) {
              const float* z = E.zbuf + ((int64_t)p * T + t) * E.rpad;
              const float z0 = j0 < P.r ? z[j0] * L.fcls : 0.f;
              const float z1 = j0 + 1 < P.r ? z[j0 + 1] * L.fcls : 0.f;
              const float cc = convert_pair(L, z0, z1, tt, ab);
              cpart[0][t] += p == 0 ? cc : 0.f;
              cpart[1][t] += p == 0 ? 0.f : cc;
            }
          }
        }
      }
    }
    __syncthreads();
    // MFMAs over this pass for each of the wave's row tiles
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rt = rg * kDecodeRowTilesPerItem + wave + kWaves * k;
      if (rt < E.nrt) {
        for (int q = 0; q < npass; ++q) {
          const int u = u0 + q;
          const int tb = u % TB, pc = u / TB;
          const int p = pc < nchunk[0] ? 0 : 1, c = pc < nchunk[0] ? pc : pc - nchunk[0];
          const int wi = 4 * c + gr;
          const uint32_t w = wi < E.p[p].W ? E.udec[((int64_t)rt * E.uw + E.woff[p] + wi) * 16 + mr] : 0u;
          v8i A;
          int sc;
          load_a(aimg + q * kABytes, mr, gr, 2 * min(8, T - tb * 8), A, sc);
          const v8i B = expand_signs(w);
#pragma unroll
          for (int tb2 = 0; tb2 < TB; ++tb2)
            if (tb2 == tb) {
              if (p == 0) acc[k][0][tb2] = mfma(A, B, acc[k][0][tb2], sc);
              else acc[k][1][tb2] = mfma(A, B, acc[k][1][tb2], sc);
            }
        }
      }
    }
    __syncthreads();
  }
  // C per (path, token): wave sums, then fixed-order sum over waves
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int t = 0; t < TB * 8; ++t) {
      float s = wave_sum(cpart[p][t]);
      if (lane == 0) cw[(wave * 2 + p) * 16 + t] = s;
    }
  __syncthreads();
  if (tid < 32) {
    const int p = tid / 16, t = tid % 16;
    cu[p * 16 + t] = ((cw[(0 * 2 + p) * 16 + t] + cw[(1 * 2 + p) * 16 + t]) + cw[(2 * 2 + p) * 16 + t]) +
                     cw[(3 * 2 + p) * 16 + t];
  }
  __syncthreads();
  uint16_t* y = reinterpret_cast<uint16_t*>(yv) + (int64_t)a.t0 * m;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int rt = rg * kDecodeRowTilesPerItem + wave + kWaves * k;
    const int i = rt * 16 + mr;
    if (rt < E.nrt && i < m) {
      const float h0 = f16f(E.p[0].h[i]);
      const float h1 = E.np > 1 ? f16f(E.p[1].h[i]) : 0.f;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int t = tb * 8 + 2 * gr + q;
          if (t < T) {
            float v = h0 * ((acc[k][0][tb][2 * q] + acc[k][0][tb][2 * q + 1]) + cu[t]);
            if (E.np > 1) v += h1 * ((acc[k][1][tb][2 * q] + acc[k][1][tb][2 * q + 1]) + cu[16 + t]);
            y[(int64_t)t * m + i] = f32_to_bf16_rne(v);
          }
        }
    }
  }
}

template <int TB>
__global__ void __launch_bounds__(kThreads, 2) k_decode(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int s_item;
  __shared__ unsigned int s_gen;
  if (threadIdx.x == 0) s_gen = __hip_atomic_load(&a.ctl->gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) s_item = (int)atomicAdd(&a.ctl->ticket, 1u);
    __syncthreads();
    const int it = s_item;
    const unsigned int gen = s_gen;
    if (it >= a.nitems) break;
    const WorkItem wi = a.items[it];
    const DecEntry& E = a.entries[wi.entry];
    if (wi.kind_path & 0x8000u) {
      void* y = a.xs ? a.ys[wi.entry] : a.y0;
      u_item<TB>(a, E, wi.entry, y, wi.group, gen, lds);
    } else {
      const void* x = a.xs ? a.xs[wi.entry] : a.x0;
      v_item<TB>(a, E, wi.entry, x, wi.kind_path & 0x7fff, wi.group, gen, lds);
    }
  }
  // last workgroup out resets the queue and advances the generation
  if (threadIdx.x == 0) {
    __threadfence();
    unsigned int d = atomicAdd(&a.ctl->done, 1u);
    if (d + 1 == gridDim.x) {
      __hip_atomic_store(&a.ctl->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&a.ctl->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
      atomicAdd(&a.ctl->gen, 1u);
    }
  }
}

size_t decode_lds_bytes(int tb) {
  const size_t v = (size_t)kWaves * tb * kABytes + (size_t)decode_ct_max(tb) * tb * 256 * 4 + 16 * 4;
  const size_t u = (size_t)kUnitsPerPass * kABytes + (32 + kWaves * 32) * 4;
  return v > u ? v : u;
}

}  // namespace

int decode_grid_size(int tb) {
  static int cached[3] = {0, 0, 0};
  if (cached[tb]) return cached[tb];
  int dev = 0, cus = 256, per = 1;
  if (hipGetDevice(&dev) == hipSuccess) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
  }
  hipError_t e = tb == 1 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_decode<1>, kThreads, decode_lds_bytes(1))
                         : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_decode<2>, kThreads, decode_lds_bytes(2));
  if (e != hipSuccess || per < 1) per = 1;
  cached[tb] = cus * per;
  return cached[tb];
}

hipError_t launch_decode(const DecArgs& a, int tb, hipStream_t st) {
  const int grid = decode_grid_size(tb);
  if (tb == 1) hipLaunchKernelGGL(k_decode<1>, dim3(grid), dim3(kThreads), decode_lds_bytes(1), st, a);
  else hipLaunchKernelGGL(k_decode<2>, dim3(grid), dim3(kThreads), decode_lds_bytes(2), st, a);
  return hipGetLastError();
}

}  // namespace lb

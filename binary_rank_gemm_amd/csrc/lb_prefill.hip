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
// Workgroup tile 256 x 256 (4 waves of 128 x 128, 32x32x16 MFMA), K blocks of
// 64.  A goes global -> registers -> LDS (double buffered, rows padded to 72
// elements against bank conflicts); B goes from packed bits straight into
// registers.  Each GEMM is one launch over every tile of every entry, tiles
// of one (entry, row stripe) placed on one XCD so the stripe is read into one
// L2.
#include <algorithm>

#include "lb_prefill.h"
#include <hip/hip_fp16.h>

namespace lb {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LB_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ inline LB_GLOBAL T* gp(T* p) { return (LB_GLOBAL T*)p; }
template <class T>
__device__ inline const LB_GLOBAL T* gp(const T* p) { return (const LB_GLOBAL T*)p; }

constexpr int kThreads = 256;
constexpr int kLdsRow = kPreBK + 8;                      // padded A row (elements)
constexpr int kLdsA = kPreBM * kLdsRow * 2;              // bytes per A buffer
constexpr int kLdsG = 2 * kPreBK * 2;                    // bytes per |g| stage (2 paths)
constexpr size_t kPreLds = 2 * (size_t)kLdsA + 2 * kLdsG;

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

template <int MODE>
__global__ void __launch_bounds__(kThreads, 1) k_prefill(PreArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const PreItem it = a.items[blockIdx.x];
  if (it.entry < 0) return;
  const PreEntry& Eg = a.entries[it.entry];
  const PrefillLayer L = Eg.L;
  const int T = a.T;
  const bool first = it.entry == 0 && a.x0 != nullptr;
  const uint16_t* A;
  int lda, K, N, kbn;
  const uint32_t* Bw;
  uint16_t* C;
  int ldc;
  if (MODE == 1) {
    A = reinterpret_cast<const uint16_t*>(first ? a.x0 : Eg.x);
    lda = L.n; K = L.n; N = L.Rp; kbn = L.kb1; Bw = L.b1;
    C = Eg.z; ldc = L.Rp;
  } else {
    A = Eg.z;
    lda = L.Rp; K = L.Rp; N = L.m; kbn = L.kb2; Bw = L.b2;
    C = reinterpret_cast<uint16_t*>(first ? a.y0 : Eg.y); ldc = L.m;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = it.mt * kPreBM, n0 = it.nt * kPreBN;
  // this wave's B tile; past the last tile (N not a multiple of 256) the loads
  // are clamped and every column of the wave is discarded in the epilogue
  const int ntile = min((n0 + wn * kPreWN) / kPreWN, (MODE == 1 ? L.nt1 : L.nt2) - 1);
  const int l32 = lane & 31, kg = lane >> 5;
  const bool vec_ok = (lda & 7) == 0;
  const int nkb = (K + kPreBK - 1) / kPreBK;

  uint16_t* As = reinterpret_cast<uint16_t*>(lds);                 // [2][256][72]
  uint16_t* Gs = reinterpret_cast<uint16_t*>(lds + 2 * kLdsA);     // [2][2 paths][64]

  // ---- global -> register staging of one A block (8 x 16 B per thread) and |g|
  u32x4 areg[8];
  uint32_t greg = 0;
  auto load_a = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i;
      const int row = m0 + (c >> 3), k = kb * kPreBK + (c & 7) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < T) {
        const LB_GLOBAL uint16_t* src = gp(A) + (int64_t)row * lda + k;
        if (vec_ok && k + 8 <= K) {
          v = *reinterpret_cast<const LB_GLOBAL u32x4*>(src);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = k + q < K ? src[q] : 0u;
          v = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        }
      }
      areg[i] = v;
    }
    if (MODE == 1 && tid < 64) {   // |g| of both paths for this K block, as bf16 pairs
      const int p = tid >> 5, k2 = (tid & 31) * 2;
      greg = *reinterpret_cast<const LB_GLOBAL uint32_t*>(gp(L.gabs) + (int64_t)p * L.kb1 * kPreBK + kb * kPreBK + k2);
    }
  };
  auto store_a = [&](int buf) {
    uint16_t* dst = As + buf * (kPreBM * kLdsRow);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(dst + (c >> 3) * kLdsRow + (c & 7) * 8) = areg[i];
    }
    if (MODE == 1 && tid < 64) *reinterpret_cast<uint32_t*>(Gs + buf * 2 * kPreBK + tid * 2) = greg;
  };
  // ---- B words: one dword per K step, 4 steps per K block
  const LB_GLOBAL u32x4* bsrc = reinterpret_cast<const LB_GLOBAL u32x4*>(gp(Bw)) + (int64_t)ntile * kbn * 64 + lane;
  auto load_b = [&](int kb) { return bsrc[(int64_t)kb * 64]; };

  // ---- scales that do not change along K (GEMM2: |h| of this lane's columns)
  u32x4 h2[2];
  int bpath[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = n0 + wn * kPreWN + 32 * b;   // first column of block b
    bpath[b] = (MODE == 1 && L.np > 1 && col >= L.roff[1]) ? 1 : 0;
  }
  if (MODE == 2) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t h = gp(L.habs)[(int64_t)p * L.nt2 * kPreWN + ntile * kPreWN + 32 * b + l32];
        h2[p][b] = h | (h << 16);
      }
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  load_a(0);
  u32x4 bcur = load_b(0), bnxt = bcur;
  store_a(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) {
      load_a(kb + 1);
      bnxt = load_b(kb + 1);
    }
    const uint16_t* Ab = As + cur * (kPreBM * kLdsRow) + (wm * 128 + l32) * kLdsRow + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 af[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) af[mb] = *reinterpret_cast<const u32x4*>(Ab + mb * 32 * kLdsRow + ks * 16);
      const uint32_t d = bcur[ks];
      u32x4 s2[2];
      if (MODE == 1) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
          s2[p] = *reinterpret_cast<const u32x4*>(Gs + cur * 2 * kPreBK + p * kPreBK + ks * 16 + 8 * kg);
      }
      const int kpath = (MODE == 2 && L.np > 1 && kb * kPreBK + ks * 16 >= L.roff[1]) ? 1 : 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        u32x4 sc;
        if (MODE == 1) sc = bpath[b] ? s2[1] : s2[0];
        else {
          const uint32_t h = kpath ? h2[1][b] : h2[0][b];
          sc = u32x4{h, h, h, h};
        }
        const u32x4 bf = expand_b(d, b, sc);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][b] = mfma32(af[mb], bf, acc[mb][b]);
      }
    }
    if (kb + 1 < nkb) {
      store_a(cur ^ 1);
      bcur = bnxt;
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds D[8 (q/4) + 4 kg + q%4][l32] of each 32x32 block
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = n0 + wn * kPreWN + 32 * b + l32;
    if (col < N) {
      const float ls = MODE == 1 ? gp(L.lpad)[col] : 1.f;
      LB_GLOBAL uint16_t* cp = gp(C) + col;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = m0 + wm * 128 + mb * 32 + 8 * (q >> 2) + 4 * kg + (q & 3);
          if (row < T) cp[(int64_t)row * ldc] = f32_to_bf16_rne(acc[mb][b][q] * ls);
        }
    }
  }
}

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

// Tiles of one (entry, row stripe) go to one XCD (workgroup b runs on XCD b % 8),
// stripes balanced over the XCDs by tile count.
std::vector<PreItem> xcd_order(const std::vector<std::vector<PreItem>>& stripes) {
  constexpr int kXcd = 8;
  std::vector<int> order(stripes.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return stripes[a].size() > stripes[b].size(); });
  std::vector<std::vector<PreItem>> per(kXcd);
  for (int s : order) {
    int best = 0;
    for (int x = 1; x < kXcd; ++x)
      if (per[x].size() < per[best].size()) best = x;
    per[best].insert(per[best].end(), stripes[s].begin(), stripes[s].end());
  }
  size_t len = 0;
  for (auto& v : per) len = std::max(len, v.size());
  std::vector<PreItem> out(len * kXcd, PreItem{-1, 0, 0});
  for (int x = 0; x < kXcd; ++x)
    for (size_t i = 0; i < per[x].size(); ++i) out[i * kXcd + x] = per[x][i];
  return out;
}

}  // namespace

hipError_t prefill_prepare(PrefillPlan& P, const PrefillLayer* const* layers, int count, int T,
                           const void* const* xs, void* const* ys) {
  const int mts = (T + kPreBM - 1) / kPreBM;
  std::vector<std::vector<PreItem>> s1, s2;
  size_t zoff = 0;
  std::vector<size_t> zoffs(count);
  P.entries_h.assign(count, PreEntry{});
  for (int e = 0; e < count; ++e) {
    const PrefillLayer& L = *layers[e];
    P.entries_h[e].L = L;
    zoffs[e] = zoff;
    zoff += align256((size_t)T * L.Rp * 2);
    const int nt1 = (L.Rp + kPreBN - 1) / kPreBN, nt2 = (L.m + kPreBN - 1) / kPreBN;
    for (int mt = 0; mt < mts; ++mt) {
      std::vector<PreItem> a, b;
      for (int nt = 0; nt < nt1; ++nt) a.push_back(PreItem{e, mt, nt});
      for (int nt = 0; nt < nt2; ++nt) b.push_back(PreItem{e, mt, nt});
      s1.push_back(a);
      s2.push_back(b);
    }
  }
  std::vector<PreItem> i1 = xcd_order(s1), i2 = xcd_order(s2);
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
  for (int e = 0; e < count; ++e) {
    P.entries_h[e].z = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(P.zbuf) + zoffs[e]);
    P.entries_h[e].x = xs ? xs[e] : nullptr;
    P.entries_h[e].y = ys ? ys[e] : nullptr;
  }
  if (P.entries_d) (void)hipFree(P.entries_d);
  if (P.items_d) (void)hipFree(P.items_d);
  P.entries_d = nullptr;
  P.items_d = nullptr;
  hipError_t e = hipMalloc(&P.entries_d, count * sizeof(PreEntry));
  if (e == hipSuccess) e = hipMalloc(&P.items_d, (i1.size() + i2.size()) * sizeof(PreItem));
  if (e == hipSuccess) e = hipMemcpy(P.entries_d, P.entries_h.data(), count * sizeof(PreEntry), hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  std::vector<PreItem> all(i1);
  all.insert(all.end(), i2.begin(), i2.end());
  if ((e = hipMemcpy(P.items_d, all.data(), all.size() * sizeof(PreItem), hipMemcpyHostToDevice)) != hipSuccess) return e;
  P.n1 = (int)i1.size();
  P.n2 = (int)i2.size();
  P.T = T;
  P.count = count;
  return hipSuccess;
}

hipError_t prefill_run(PrefillPlan& P, const PrefillLayer* const* layers, int count, const void* const* xs,
                       void* const* ys, int T, hipStream_t st, bool single) {
  PreArgs a{};
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
  a.items = P.items_d;
  hipLaunchKernelGGL(k_prefill<1>, dim3(P.n1), dim3(kThreads), kPreLds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  a.items = P.items_d + P.n1;
  hipLaunchKernelGGL(k_prefill<2>, dim3(P.n2), dim3(kThreads), kPreLds, st, a);
  return hipGetLastError();
}

void prefill_plan_release(PrefillPlan& P) {
  if (P.entries_d) (void)hipFree(P.entries_d);
  if (P.items_d) (void)hipFree(P.items_d);
  if (P.zbuf) (void)hipFree(P.zbuf);
  P.entries_d = nullptr;
  P.items_d = nullptr;
  P.zbuf = nullptr;
  P.zbytes = 0;
  P.T = -1;
  P.count = 0;
  P.entries_h.clear();
}

}  // namespace lb

// fp32 forward of one linear with plain vector arithmetic (the fp32-I/O path
// for few tokens; it also serves bf16 x with bf16 or fp32 y).  fp32 I/O with
// many tokens goes to the tiled form in lb_f32gemm.hip.
//
// It follows the factorised order of the paper notes ("LittleBit", section
// "Key design"): per path t = x o g, z = t V, z' = z o l, then
// y = sum_p (z'_p U_p^T) o h_p.  Signs are applied by selecting +t or -t from
// the canonical packed bits.  Sums are blocked (64-term partial sums, then a
// fixed-order combine across waves) so fp32 rounding stays far below 1e-5 of
// the output's rms at d_in up to 2^20.
#include "lb_internal.h"
#include <hip/hip_fp16.h>

namespace lb {

namespace {

__device__ inline float ld_act(const void* x, int64_t idx, int x_fp32) {
  if (x_fp32) return reinterpret_cast<const float*>(x)[idx];
  uint32_t b = (uint32_t)reinterpret_cast<const uint16_t*>(x)[idx] << 16;
  return __uint_as_float(b);
}

__device__ inline float f16(const uint16_t* p, int64_t i) { return __half2float(__ushort_as_half(p[i])); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct ExactArgs {
  PathDev p[2];
  const void* x;
  void* y;
  float* zbuf;
  int np, m, n, T, rpad, x_fp32, y_fp32, t0, splits;
};

// grid (ceil(r_max/64), np, tokens x splits), block 256: lane -> latent
// column j, wave -> row phase; split s sums rows [n s / S, n (s + 1) / S)
// (S > 1 only when tokens are few: more workgroups for the same work).
// Writes the split's sum of (x o g) V for column j; l is applied when the
// splits are added, in split order, by k_exact_y.
__global__ void __launch_bounds__(256) k_exact_z(ExactArgs a) {
  const int p = blockIdx.y, t = a.t0 + (int)blockIdx.z / a.splits, sp = (int)blockIdx.z % a.splits;
  const PathDev P = a.p[p];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int k0 = (int)((int64_t)a.n * sp / a.splits), k1 = (int)((int64_t)a.n * (sp + 1) / a.splits);
  __shared__ float part[4][64];
  float acc = 0.f;
  if (j < P.r) {
    float blk = 0.f;
    int cnt = 0;
    const int64_t xo = (int64_t)t * a.n;
    for (int k = k0 + wave; k < k1; k += 4) {
      float tv = ld_act(a.x, xo + k, a.x_fp32) * f16(P.g, k);
      uint32_t bit = (P.v_can[(int64_t)k * P.W + (j >> 5)] >> (j & 31)) & 1u;
      blk += bit ? -tv : tv;
      if (++cnt == 64) { acc += blk; blk = 0.f; cnt = 0; }
    }
    acc += blk;
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && j < P.r) {
    const float z = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
    a.zbuf[(((int64_t)sp * a.np + p) * a.T + t) * a.rpad + j] = z;
  }
}

// grid (ceil(m/256), T), block 256: thread -> output row i.
__global__ void __launch_bounds__(256) k_exact_y(ExactArgs a) {
  const int t = a.t0 + (int)blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  extern __shared__ float zs[];  // [np][rpad]
  for (int p = 0; p < a.np; ++p)
    for (int j = threadIdx.x; j < a.p[p].r; j += 256) {
      float z = 0.f;
      for (int sp = 0; sp < a.splits; ++sp) z += a.zbuf[(((int64_t)sp * a.np + p) * a.T + t) * a.rpad + j];
      zs[p * a.rpad + j] = z * f16(a.p[p].l, j);
    }
  __syncthreads();
  if (i >= a.m) return;
  float y = 0.f;
  for (int p = 0; p < a.np; ++p) {
    const PathDev P = a.p[p];
    const float* z = zs + p * a.rpad;
    float s = 0.f;
    for (int w = 0; w < P.W; ++w) {
      uint32_t bits = P.u_can[i * P.W + w];
      float blk = 0.f;
      const int jend = min(32, P.r - 32 * w);
      for (int b = 0; b < jend; ++b) {
        float zv = z[32 * w + b];
        blk += ((bits >> b) & 1u) ? -zv : zv;
      }
      s += blk;
    }
    y += s * f16(P.h, i);
  }
  const int64_t yo = (int64_t)t * a.m + i;
  if (a.y_fp32) reinterpret_cast<float*>(a.y)[yo] = y;
  else reinterpret_cast<uint16_t*>(a.y)[yo] = f32_to_bf16_rne(y);
}

}  // namespace

hipError_t launch_exact(const PathDev* p, int np, int m, int n, const void* x, void* y, int T,
                        int x_fp32, int y_fp32, float* zbuf, hipStream_t st) {
  if (exact_uses_gemm(T, x_fp32, y_fp32))
    return launch_f32_gemm(p, np, m, n, reinterpret_cast<const float*>(x), reinterpret_cast<float*>(y), T, zbuf, st);
  int rpad = 0;
  for (int i = 0; i < np; ++i) rpad = rpad > p[i].r ? rpad : p[i].r;
  rpad = (rpad + 15) / 16 * 16;
  ExactArgs a{};
  for (int i = 0; i < np; ++i) a.p[i] = p[i];
  a.x = x; a.y = y; a.zbuf = zbuf; a.np = np; a.m = m; a.n = n; a.T = T; a.rpad = rpad; a.x_fp32 = x_fp32;
  a.y_fp32 = y_fp32;
  int rmax = 0;
  for (int i = 0; i < np; ++i) rmax = rmax > p[i].r ? rmax : p[i].r;
  a.splits = exact_splits(rmax, np, T, n);
  const int kMaxY = 65535;  // grid y/z extent limit: tokens go in slices
  const int kMaxZ = kMaxY / a.splits;
  for (int t0 = 0; t0 < T; t0 += kMaxZ) {
    a.t0 = t0;
    int tn = T - t0 < kMaxZ ? T - t0 : kMaxZ;
    hipLaunchKernelGGL(k_exact_z, dim3((rmax + 63) / 64, np, tn * a.splits), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  size_t shmem = (size_t)np * rpad * sizeof(float);
  for (int t0 = 0; t0 < T; t0 += kMaxY) {
    a.t0 = t0;
    int tn = T - t0 < kMaxY ? T - t0 : kMaxY;
    hipLaunchKernelGGL(k_exact_y, dim3((m + 255) / 256, tn), dim3(256), shmem, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lb

// fp32 forward of one linear for many tokens: the factorised order of the
// paper notes ("LittleBit: Ultra Low-Bit Quantization via Latent
// Factorization", section "Key design": element-wise scales around binary
// matrix products; section "Residual compensation": a sum of two paths) as two
// tiled contractions on the fp32 matrix cores (v_mfma_f32_32x32x2_f32):
//
//   GEMM1, per path p:  Z'_p[T][rpad_p] = (x . B1_p) o l_p,   B1_p[k][j] = s(V_p[k][j]) g_p[k]
//   GEMM2:              y[T][m] = sum_p Z'_p . B2_p,           B2_p[j][i] = s(U_p[i][j]) h_p[i]
//
// s(.) = -1 where the sign bit is set.  A B element is the fp32 value of the
// fp16 scale with its sign bit flipped where the sign factor is -1: exact, so
// the only roundings are those of the fp32 sums.  Sums are blocked: each
// 32-deep K block is accumulated from zero on the matrix cores and then added
// to the running total, which keeps the error of a 28672-long sum far below
// 1e-5 of the output's rms.  rpad_p = r_p rounded up to 32; Z' columns past r_p
// are zero (l is taken as zero there).
//
// Workgroup tile 128 tokens x 128 columns, four waves of 64 x 64 (2 x 2 blocks
// of 32 x 32), K blocks of 32 staged in LDS, double buffered: the x (or Z')
// block transposed to [k][row] so a fragment read is 32 consecutive floats,
// and the block's sign words (with g, or h for the wave's columns).
#include "lb_internal.h"
#include <hip/hip_fp16.h>

namespace lb {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kTM = 128, kTN = 128, kKB = 32, kThreads = 256;

struct F32Args {
  PathDev p[2];
  const float* x;   // [T][n]
  float* y;         // [T][m]
  float* z;         // per path: [T][rpad_p] at z + zoff[p]
  int64_t zoff[2];
  int rpad[2];
  int np, m, n, T;
};

__device__ inline float f16f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// LDS of one K block: A^T [kKB][kTM] floats, sign words, and the K rows' g
// (GEMM1) -- 16.6 KB
struct Stage {
  float a[kKB][kTM];
  uint32_t w[kTN];         // GEMM1: [k][4] words (row k, 32-column word c); GEMM2: one word per output row
  float g[kKB];            // GEMM1: g of each K row
};

// MODE 1: GEMM1 of path blockIdx.z; MODE 2: GEMM2 (both paths' latents as K)
template <int MODE>
__global__ void __launch_bounds__(kThreads, 2) k_f32_gemm(F32Args a) {
  __shared__ Stage st[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int m0 = blockIdx.x * kTM, n0 = blockIdx.y * kTN;
  const int p1 = MODE == 1 ? (int)blockIdx.z : 0;
  const int N = MODE == 1 ? a.rpad[p1] : a.m;
  if (n0 >= N) return;                                   // (GEMM1: the other path has more column tiles)
  // K segments: GEMM1 one (k over n), GEMM2 one per path (k over its padded latents)
  const int nseg = MODE == 1 ? 1 : a.np;
  int nkb[2];
  for (int s = 0; s < 2; ++s) nkb[s] = s < nseg ? (MODE == 1 ? (a.n + kKB - 1) / kKB : a.rpad[s] / kKB) : 0;
  const int nk = nkb[0] + nkb[1];

  // loader roles: A rows (2 threads a row, 16 floats each); sign words
  const int arow = tid >> 1, akh = (tid & 1) * 16;
  const int t_row = m0 + arow;
  float areg[16];
  uint32_t wreg = 0;
  float greg = 0.f;
  auto load = [&](int kb) {
    const int seg = kb < nkb[0] ? 0 : 1, kl = seg ? kb - nkb[0] : kb;
    const int k0 = kl * kKB;
    if (MODE == 1) {
      const PathDev& P = a.p[p1];
      const bool rv = t_row < a.T;
      const float* src = a.x + (int64_t)(rv ? t_row : 0) * a.n + k0 + akh;
      if (rv && k0 + akh + 16 <= a.n && (a.n & 3) == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f4v v = *reinterpret_cast<const f4v*>(src + 4 * q);
          areg[4 * q] = v[0]; areg[4 * q + 1] = v[1]; areg[4 * q + 2] = v[2]; areg[4 * q + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) areg[q] = (rv && k0 + akh + q < a.n) ? src[q] : 0.f;
      }
      if (tid < kTN) {
        const int k = k0 + (tid >> 2), c = (n0 >> 5) + (tid & 3);
        wreg = (k < a.n && c < P.W) ? P.v_can[(int64_t)k * P.W + c] : 0u;
      } else if (tid < kTN + kKB) {
        const int k = k0 + tid - kTN;
        greg = k < a.n ? f16f(P.g[k]) : 0.f;
      }
    } else {
      const PathDev& P = a.p[seg];
      const int rp = a.rpad[seg];
      const bool rv = t_row < a.T;
      const float* src = a.z + a.zoff[seg] + (int64_t)(rv ? t_row : 0) * rp + k0 + akh;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f4v v = rv ? *reinterpret_cast<const f4v*>(src + 4 * q) : f4v{0.f, 0.f, 0.f, 0.f};
        areg[4 * q] = v[0]; areg[4 * q + 1] = v[1]; areg[4 * q + 2] = v[2]; areg[4 * q + 3] = v[3];
      }
      if (tid < kTN) {
        const int i = n0 + tid, c = k0 >> 5;
        wreg = (i < a.m && c < P.W) ? P.u_can[(int64_t)i * P.W + c] : 0u;
      }
    }
  };
  auto store = [&](int buf) {
    Stage& S = st[buf];
#pragma unroll
    for (int q = 0; q < 16; ++q) S.a[akh + q][arow] = areg[q];
    if (tid < kTN) S.w[tid] = wreg;
    else if (MODE == 1 && tid < kTN + kKB) S.g[tid - kTN] = greg;
  };

  // GEMM2: h of the wave's two 32-column blocks, for the current path
  float hcol[2] = {0.f, 0.f};
  auto load_h = [&](int seg) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int i = n0 + wn * 64 + 32 * cb + l32;
      hcol[cb] = i < a.m ? f16f(a.p[seg].h[i]) : 0.f;
    }
  };
  if (MODE == 2) load_h(0);

  v16f tot[2][2], blk[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) tot[i][j][q] = 0.f;

  load(0);
  store(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    if (kb + 1 < nk) load(kb + 1);                      // in flight during this block's products
    if (MODE == 2 && kb == nkb[0]) load_h(1);
    const Stage& S = st[kb & 1];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) blk[i][j][q] = 0.f;
#pragma unroll 4
    for (int s = 0; s < kKB / 2; ++s) {
      const int k = 2 * s + kh;
      float av[2], bv[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) av[mb] = S.a[k][wm * 64 + 32 * mb + l32];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        uint32_t bit, mag;
        if (MODE == 1) {
          bit = (S.w[k * 4 + wn * 2 + cb] >> l32) & 1u;
          mag = __float_as_uint(S.g[k]);
        } else {
          bit = (S.w[wn * 64 + 32 * cb + l32] >> k) & 1u;
          mag = __float_as_uint(hcol[cb]);
        }
        bv[cb] = __uint_as_float(mag ^ (bit << 31));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) blk[mb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[mb], bv[cb], blk[mb][cb], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) tot[i][j] += blk[i][j];
    if (kb + 1 < nk) store((kb + 1) & 1);                // the other buffer: last read before the previous barrier
    __syncthreads();
  }

  // epilogue: lane (l32, kh), element q of block (mb, cb) is row
  // 8 (q / 4) + 4 kh + (q % 4) and column l32 of the block
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = n0 + wn * 64 + 32 * cb + l32;
    if (col >= N) continue;
    float ls = 1.f;
    if (MODE == 1) ls = col < a.p[p1].r ? f16f(a.p[p1].l[col]) : 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int t = m0 + wm * 64 + 32 * mb + 8 * (q >> 2) + 4 * kh + (q & 3);
        if (t >= a.T) continue;
        if (MODE == 1) a.z[a.zoff[p1] + (int64_t)t * a.rpad[p1] + col] = tot[mb][cb][q] * ls;
        else a.y[(int64_t)t * a.m + col] = tot[mb][cb][q];
      }
  }
}

}  // namespace

size_t f32_gemm_scratch_floats(const PathDev* p, int np, int64_t T) {
  size_t f = 0;
  for (int i = 0; i < np; ++i) f += (size_t)T * (size_t)((p[i].r + 31) / 32 * 32);
  return f;
}

hipError_t launch_f32_gemm(const PathDev* p, int np, int m, int n, const float* x, float* y, int T, float* zbuf,
                           hipStream_t st) {
  F32Args a{};
  int tiles_n1 = 0;
  int64_t off = 0;
  for (int i = 0; i < np; ++i) {
    a.p[i] = p[i];
    a.rpad[i] = (p[i].r + 31) / 32 * 32;
    a.zoff[i] = off;
    off += (int64_t)T * a.rpad[i];
    tiles_n1 = std::max(tiles_n1, (a.rpad[i] + kTN - 1) / kTN);
  }
  a.x = x;
  a.y = y;
  a.z = zbuf;
  a.np = np;
  a.m = m;
  a.n = n;
  a.T = T;
  const unsigned mt = (unsigned)((T + kTM - 1) / kTM);
  hipLaunchKernelGGL(k_f32_gemm<1>, dim3(mt, tiles_n1, np), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_f32_gemm<2>, dim3(mt, (m + kTN - 1) / kTN, 1), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace lb

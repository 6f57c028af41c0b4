// Dual-SVID initialisation of a LittleBit layer from a dense weight
// ("LittleBit: Ultra Low-Bit Quantization via Latent Factorization", paper
// notes, sections "Key design / Dual-SVID initialisation" and "Residual
// compensation"): per path, a truncated SVD of what is left of W gives
// factors U', V' (singular values split evenly); the signs of U', V' are the
// binary factors; a rank-1 SVD of |U'| gives the row scale h and one latent
// factor, a rank-1 SVD of |V'| the column scale g and the other; their
// product is the latent scale l.  The residual path starts from W minus the
// primary path as stored (fp16 scales).
//
// The SVDs are rocSOLVER's partial SVD (gesvdx, fp64); the layout work is
// small HIP kernels; the residual update is one rocBLAS dgemm.  This runs once
// per layer when a model is compressed, not in the forward pass.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>
#include <rocsolver/rocsolver.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "lb_internal.h"

namespace lb {
namespace {

constexpr int kT = 256;

inline unsigned blocks(int64_t n) { return (unsigned)((n + kT - 1) / kT); }

// W row-major [m][n] fp32 -> A column-major m x n fp64
__global__ void k_to_colmajor(const float* W, int64_t m, int64_t n, double* A) {
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= m * n) return;
  const int64_t i = t % m, j = t / m;   // consecutive threads: consecutive rows of one column
  A[t] = (double)W[i * n + j];
}

// F[i + j rows] = X[i + j rows] * sqrt(s[j])  (left factor, column-major)
__global__ void k_scale_left(const double* X, int64_t rows, int r, const double* s, double* F) {
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= rows * r) return;
  F[t] = X[t] * sqrt(s[t / rows]);
}

// F[k + j n] = Vt[j + k r] * sqrt(s[j])  (right factor from the rows of V^T)
__global__ void k_scale_right(const double* Vt, int64_t n, int r, const double* s, double* F) {
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= n * r) return;
  const int64_t k = t % n, j = t / n;
  F[t] = Vt[j + k * r] * sqrt(s[j]);
}

__global__ void k_abs(const double* X, int64_t count, double* Y) {
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t < count) Y[t] = fabs(X[t]);
}

// Packed signs of F (column-major rows x r): bit b of word w of row i is set
// iff F[i + (32 w + b) rows] < 0 (sign(0) = +1); padding bits zero.
__global__ void k_pack_from(const double* F, int64_t rows, int r, uint32_t* out) {
  const int W = (r + 31) / 32;
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= rows * W) return;
  const int64_t i = t / W;
  const int w = (int)(t % W);
  uint32_t v = 0;
  for (int b = 0; b < 32; ++b) {
    const int j = 32 * w + b;
    if (j < r && F[i + (int64_t)j * rows] < 0.0) v |= 1u << b;
  }
  out[t] = v;
}

// out[i + j rows] = rs[i] * sign(F[i + j rows]) * (cs ? cs[j] : 1)
__global__ void k_signed(const double* F, int64_t rows, int r, const double* rs, const double* cs, double* out) {
  const int64_t t = (int64_t)blockIdx.x * kT + threadIdx.x;
  if (t >= rows * r) return;
  const int64_t i = t % rows, j = t / rows;
  const double sg = F[t] < 0.0 ? -1.0 : 1.0;
  out[t] = rs[i] * sg * (cs ? cs[j] : 1.0);
}

// IEEE half from double, rounded to nearest even (overflow to infinity).
// With a = f 2^e (f in [1/2, 1)), the half's quantum is 2^(e - 11) for
// normals and 2^-24 below them; k = a / quantum rounded to an integer is then
// the bit pattern's magnitude part directly for the smallest binade and the
// subnormals, and (biased exponent << 10) + k - 1024 above (k = 2048, a carry
// into the next binade, lands on the right pattern by the same formula).
uint16_t f64_to_f16(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  const double a = std::fabs(x);
  if (std::isnan(a)) return sign | 0x7e00;
  if (a == 0.0) return sign;
  int e;
  (void)std::frexp(a, &e);
  const int qexp = std::max(e - 11, -24);
  const double k = std::nearbyint(std::ldexp(a, -qexp));   // exact scaling, then nearest even
  double pat = qexp == -24 ? k : (double)((e - 1 + 15) << 10) + (k - 1024.0);
  if (pat >= 0x7c00) pat = 0x7c00;
  return sign | (uint16_t)pat;
}

double f16_to_f64(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1024.0 + m, e - 25);
  return (h & 0x8000) ? -v : v;
}

template <class T>
struct DevT {
  T* p = nullptr;
  ~DevT() {
    if (p) (void)hipFree(p);
  }
  hipError_t alloc(size_t count) { return hipMalloc(&p, std::max<size_t>(count, 1) * sizeof(T)); }
};
using Dev = DevT<double>;
using DevI = DevT<rocblas_int>;

#define LB_ROC(expr)                                                   \
  do {                                                                 \
    const rocblas_status s_ = (expr);                                  \
    if (s_ != rocblas_status_success) {                                \
      status = s_;                                                     \
      return hipErrorUnknown;                                          \
    }                                                                  \
  } while (0)
#define LB_HIPR(expr)                         \
  do {                                        \
    const hipError_t e_ = (expr);             \
    if (e_ != hipSuccess) return e_;          \
  } while (0)

// top singular pair of X (rows x cols, column-major, destroyed): a (rows),
// b (cols), sigma; signs chosen so that sum(a) + sum(b) >= 0
hipError_t rank1(rocblas_handle H, double* X, int64_t rows, int cols, std::vector<double>& a, std::vector<double>& b,
                 double& sigma, rocblas_status& status, hipStream_t st) {
  Dev S, U, Vt;
  DevI nsv, info, ifail;
  LB_HIPR(S.alloc(std::min<int64_t>(rows, cols)));
  LB_HIPR(U.alloc(rows));
  LB_HIPR(Vt.alloc(cols));
  LB_HIPR(nsv.alloc(1));
  LB_HIPR(info.alloc(1));
  LB_HIPR(ifail.alloc(std::min<int64_t>(rows, cols)));
  const rocblas_status rs = rocsolver_dgesvdx(H, rocblas_svect_singular, rocblas_svect_singular, rocblas_srange_index,
                                              (rocblas_int)rows, cols, X, (rocblas_int)rows, 0.0, 0.0, 1, 1, nsv.p, S.p,
                                              U.p, (rocblas_int)rows, Vt.p, 1, ifail.p, info.p);
  rocblas_int inf = 0;
  hipError_t e = hipSuccess;
  if (rs == rocblas_status_success) e = hipMemcpyAsync(&inf, info.p, sizeof(inf), hipMemcpyDeviceToHost, st);
  a.resize(rows);
  b.resize(cols);
  if (rs == rocblas_status_success && e == hipSuccess) e = hipMemcpyAsync(&sigma, S.p, sizeof(double), hipMemcpyDeviceToHost, st);
  if (rs == rocblas_status_success && e == hipSuccess) e = hipMemcpyAsync(a.data(), U.p, rows * sizeof(double), hipMemcpyDeviceToHost, st);
  if (rs == rocblas_status_success && e == hipSuccess) e = hipMemcpyAsync(b.data(), Vt.p, cols * sizeof(double), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (rs != rocblas_status_success) {
    status = rs;
    return hipErrorUnknown;
  }
  if (e != hipSuccess) return e;
  if (inf != 0) return hipErrorUnknown;
  double sum = 0;
  for (double v : a) sum += v;
  for (double v : b) sum += v;
  const double root = std::sqrt(sigma);
  const double sg = sum < 0 ? -root : root;
  for (double& v : a) v *= sg;
  for (double& v : b) v *= sg;
  return hipSuccess;
}

}  // namespace

hipError_t dual_svid_init(const float* W, int64_t m, int64_t n, const int64_t* ranks, int np, const InitPathOut* out,
                          hipStream_t st, int* rocstatus) {
  rocblas_status status = rocblas_status_success;
  *rocstatus = 0;
  rocblas_handle H = nullptr;
  if (rocblas_create_handle(&H) != rocblas_status_success) return hipErrorUnknown;
  struct HandleGuard {
    rocblas_handle h;
    ~HandleGuard() { rocblas_destroy_handle(h); }
  } guard{H};
  auto run = [&]() -> hipError_t {
    LB_ROC(rocblas_set_stream(H, st));
    const int64_t mn = m * n;
    Dev A, R;                                     // W, and what is left of it (column-major)
    LB_HIPR(A.alloc(mn));
    LB_HIPR(R.alloc(mn));
    hipLaunchKernelGGL(k_to_colmajor, dim3(blocks(mn)), dim3(kT), 0, st, W, m, n, A.p);
    LB_HIPR(hipGetLastError());
    for (int p = 0; p < np; ++p) {
      const int r = (int)ranks[p];
      // truncated SVD of the rest: the top r singular triplets
      LB_HIPR(hipMemcpyAsync(R.p, A.p, mn * sizeof(double), hipMemcpyDeviceToDevice, st));
      Dev S, U, Vt, Up, Vp, T1, T2;
      LB_HIPR(S.alloc(std::min(m, n)));
      LB_HIPR(U.alloc(m * r));
      LB_HIPR(Vt.alloc((int64_t)r * n));
      LB_HIPR(Up.alloc(m * r));
      LB_HIPR(Vp.alloc(n * r));
      LB_HIPR(T1.alloc(m * r));
      LB_HIPR(T2.alloc(n * r));
      DevI nsv, info, ifail;
      LB_HIPR(nsv.alloc(1));
      LB_HIPR(info.alloc(1));
      LB_HIPR(ifail.alloc(std::min(m, n)));
      const rocblas_status rs =
          rocsolver_dgesvdx(H, rocblas_svect_singular, rocblas_svect_singular, rocblas_srange_index, (rocblas_int)m,
                            (rocblas_int)n, R.p, (rocblas_int)m, 0.0, 0.0, 1, r, nsv.p, S.p, U.p, (rocblas_int)m, Vt.p, r,
                            ifail.p, info.p);
      rocblas_int inf = 0;
      hipError_t e = rs == rocblas_status_success ? hipMemcpyAsync(&inf, info.p, sizeof(inf), hipMemcpyDeviceToHost, st)
                                                  : hipSuccess;
      if (e == hipSuccess) e = hipStreamSynchronize(st);
      if (rs != rocblas_status_success) {
        status = rs;
        return hipErrorUnknown;
      }
      LB_HIPR(e);
      if (inf != 0) return hipErrorUnknown;
      // U' = U diag(sqrt s), V' = V diag(sqrt s)
      hipLaunchKernelGGL(k_scale_left, dim3(blocks(m * r)), dim3(kT), 0, st, U.p, m, r, S.p, Up.p);
      hipLaunchKernelGGL(k_scale_right, dim3(blocks(n * r)), dim3(kT), 0, st, Vt.p, n, r, S.p, Vp.p);
      // signs
      hipLaunchKernelGGL(k_pack_from, dim3(blocks(m * ((r + 31) / 32))), dim3(kT), 0, st, Up.p, m, r, out[p].u_packed);
      hipLaunchKernelGGL(k_pack_from, dim3(blocks(n * ((r + 31) / 32))), dim3(kT), 0, st, Vp.p, n, r, out[p].v_packed);
      LB_HIPR(hipGetLastError());
      // rank-1 fits of the magnitudes
      hipLaunchKernelGGL(k_abs, dim3(blocks(m * r)), dim3(kT), 0, st, Up.p, m * r, T1.p);
      hipLaunchKernelGGL(k_abs, dim3(blocks(n * r)), dim3(kT), 0, st, Vp.p, n * r, T2.p);
      LB_HIPR(hipGetLastError());
      std::vector<double> h, lu, g, lv;
      double s1 = 0, s2 = 0;
      LB_HIPR(rank1(H, T1.p, m, r, h, lu, s1, status, st));
      LB_HIPR(rank1(H, T2.p, n, r, g, lv, s2, status, st));
      // fp16 scales as stored, and their exact values for the residual
      std::vector<uint16_t> hb(m), gb(n), lb_(r);
      std::vector<double> hq(m), gq(n), lq(r);
      for (int64_t i = 0; i < m; ++i) hq[i] = f16_to_f64(hb[i] = f64_to_f16(h[i]));
      for (int64_t k = 0; k < n; ++k) gq[k] = f16_to_f64(gb[k] = f64_to_f16(g[k]));
      for (int j = 0; j < r; ++j) lq[j] = f16_to_f64(lb_[j] = f64_to_f16(lu[j] * lv[j]));
      LB_HIPR(hipMemcpyAsync(out[p].h, hb.data(), m * 2, hipMemcpyHostToDevice, st));
      LB_HIPR(hipMemcpyAsync(out[p].g, gb.data(), n * 2, hipMemcpyHostToDevice, st));
      LB_HIPR(hipMemcpyAsync(out[p].l, lb_.data(), (size_t)r * 2, hipMemcpyHostToDevice, st));
      if (p + 1 < np) {
        // A -= (h o U_sign o l) (g o V_sign)^T with the stored scales
        Dev dh, dg, dl;
        LB_HIPR(dh.alloc(m));
        LB_HIPR(dg.alloc(n));
        LB_HIPR(dl.alloc(r));
        LB_HIPR(hipMemcpyAsync(dh.p, hq.data(), m * sizeof(double), hipMemcpyHostToDevice, st));
        LB_HIPR(hipMemcpyAsync(dg.p, gq.data(), n * sizeof(double), hipMemcpyHostToDevice, st));
        LB_HIPR(hipMemcpyAsync(dl.p, lq.data(), r * sizeof(double), hipMemcpyHostToDevice, st));
        hipLaunchKernelGGL(k_signed, dim3(blocks(m * r)), dim3(kT), 0, st, Up.p, m, r, dh.p, dl.p, T1.p);
        hipLaunchKernelGGL(k_signed, dim3(blocks(n * r)), dim3(kT), 0, st, Vp.p, n, r, dg.p, nullptr, T2.p);
        LB_HIPR(hipGetLastError());
        const double alpha = -1.0, beta = 1.0;
        LB_ROC(rocblas_dgemm(H, rocblas_operation_none, rocblas_operation_transpose, (rocblas_int)m, (rocblas_int)n, r,
                             &alpha, T1.p, (rocblas_int)m, T2.p, (rocblas_int)n, &beta, A.p, (rocblas_int)m));
        LB_HIPR(hipStreamSynchronize(st));      // the host vectors above go out of scope
      } else {
        LB_HIPR(hipStreamSynchronize(st));
      }
    }
    return hipSuccess;
  };
  const hipError_t e = run();
  *rocstatus = (int)status;
  return e;
}

}  // namespace lb

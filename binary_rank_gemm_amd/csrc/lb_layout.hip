// Sign packing, unpacking and the one-time re-layout of packed factors into the
// decode kernel's tile order.  All of this runs at layer build time.
#include "lb_internal.h"

namespace lb {

namespace {

constexpr int kThreads = 256;

inline int blocks_for(int64_t n) { return (int)((n + kThreads - 1) / kThreads); }

__global__ void k_validate(const int8_t* __restrict__ s, int64_t count, int* bad) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int local = 0;
  for (; i < count; i += stride) {
    int8_t v = s[i];
    local |= (v != 1 && v != -1);
  }
  if (local) atomicOr(bad, 1);
}

// One thread per output word: bit b of word w of row i <=> signs[i][32 w + b] == -1.
__global__ void k_pack(const int8_t* __restrict__ s, int64_t rows, int64_t rank, int64_t W,
                       uint32_t* __restrict__ out) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * W) return;
  int64_t i = idx / W, w = idx % W;
  uint32_t word = 0;
  for (int b = 0; b < 32; ++b) {
    int64_t j = 32 * w + b;
    if (j < rank && s[i * rank + j] == -1) word |= 1u << b;
  }
  out[idx] = word;
}

__global__ void k_unpack(const uint32_t* __restrict__ words, int64_t rows, int64_t rank, int64_t W,
                         int8_t* __restrict__ out) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * rank) return;
  int64_t i = idx / rank, j = idx % rank;
  uint32_t bit = (words[i * W + j / 32] >> (j % 32)) & 1u;
  out[idx] = bit ? -1 : 1;
}

// Decode V layout: one thread per output dword (kc, ct, lane).
__global__ void k_retile_v(const uint32_t* __restrict__ vcan, int n, int r, int W, int nkc, int nct,
                           uint32_t* __restrict__ vdec) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)nkc * nct * 64;
  if (idx >= total) return;
  int lane = (int)(idx % 64);
  int ct = (int)((idx / 64) % nct);
  int kc = (int)(idx / (64 * (int64_t)nct));
  int j = 16 * ct + (lane & 15);
  int g = lane >> 4;
  uint32_t word = 0;
  if (j < r) {
    for (int e = 0; e < 32; ++e) {
      int64_t k = (int64_t)kChunk * kc + 32 * g + e;
      if (k < n) {
        uint32_t bit = (vcan[k * W + j / 32] >> (j % 32)) & 1u;
        word |= bit << fp4_bit_of_elem(e);
      }
    }
  }
  vdec[idx] = word;
}

// Decode U layout (UGeom): one thread per uint32 of every quad's blocks.
// Thread (quad, unit u, lane l = 16 w + row, rt) writes word 4 u' + w of output
// row 64 quad + 16 rt + row of the unit's path (u' = unit inside the path),
// bit-permuted; words past the path's rank and rows past m are zero.  Half
// units hold words 0 and 1 only.
__global__ void k_u_layout(const uint32_t* __restrict__ u0, const uint32_t* __restrict__ u1, int m, int W0, int W1,
                           UGeom g, uint8_t* __restrict__ udec) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_quad = (int64_t)g.nu * 256;   // threads per quad (64 lanes x 4 row tiles per unit)
  if (idx >= (int64_t)g.nq * per_quad) return;
  const int q = (int)(idx / per_quad);
  const int rem = (int)(idx % per_quad);
  const int u = rem / 256, l = (rem % 256) / 4, rt = rem % 4;
  const int p = u < g.nu0 ? 0 : 1;
  const int up = p ? u - g.nu0 : u;
  const bool half = p ? (g.half1 && u == g.nu - 1) : (g.half0 && u == g.nu0 - 1);
  if (half && l >= 32) return;
  const int w = l / 16, row = l % 16;
  const int word = 4 * up + w;
  const int W = p ? W1 : W0;
  const uint32_t* uc = p ? u1 : u0;
  const int64_t i = (int64_t)64 * q + 16 * rt + row;
  uint32_t out = 0;
  if (i < m && word < W) {
    const uint32_t in = uc[i * W + word];
    for (int e = 0; e < 32; ++e) out |= ((in >> e) & 1u) << fp4_bit_of_elem(e);
  }
  const int uoff = p ? g.uoff1 + 1024 * up : 1024 * up;
  *reinterpret_cast<uint32_t*>(udec + (int64_t)q * g.qbytes + uoff + (l * 4 + rt) * 4) = out;
}

// Row scales per quad: hq[quad][path][64] = h_path[64 quad + i] (zero past m
// and for a missing second path).
__global__ void k_h_layout(const uint16_t* __restrict__ h0, const uint16_t* __restrict__ h1, int m, int nq,
                           uint16_t* __restrict__ hq) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)nq * 128) return;
  const int q = (int)(idx / 128), p = (int)((idx / 64) % 2), i = (int)(idx % 64);
  const int64_t row = (int64_t)64 * q + i;
  const uint16_t* h = p ? h1 : h0;
  hq[idx] = (h && row < m) ? h[row] : (uint16_t)0;
}

}  // namespace

hipError_t launch_validate_signs(const int8_t* s, int64_t count, int* bad, hipStream_t st) {
  int blocks = blocks_for(count);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_validate, dim3(blocks), dim3(kThreads), 0, st, s, count, bad);
  return hipGetLastError();
}

hipError_t launch_pack_signs(const int8_t* s, int64_t rows, int64_t rank, uint32_t* out, hipStream_t st) {
  int64_t W = (rank + 31) / 32;
  hipLaunchKernelGGL(k_pack, dim3(blocks_for(rows * W)), dim3(kThreads), 0, st, s, rows, rank, W, out);
  return hipGetLastError();
}

hipError_t launch_unpack_signs(const uint32_t* w, int64_t rows, int64_t rank, int8_t* out, hipStream_t st) {
  int64_t W = (rank + 31) / 32;
  hipLaunchKernelGGL(k_unpack, dim3(blocks_for(rows * rank)), dim3(kThreads), 0, st, w, rows, rank, W, out);
  return hipGetLastError();
}

hipError_t launch_retile_v_decode(const uint32_t* vcan, int n, int r, uint32_t* vdec, hipStream_t st) {
  int W = (r + 31) / 32, nkc = (n + kChunk - 1) / kChunk, nct = (r + kTile - 1) / kTile;
  int64_t total = (int64_t)nkc * nct * 64;
  hipLaunchKernelGGL(k_retile_v, dim3(blocks_for(total)), dim3(kThreads), 0, st, vcan, n, r, W, nkc, nct, vdec);
  return hipGetLastError();
}

hipError_t launch_decode_u_layout(const uint32_t* ucan0, const uint32_t* ucan1, int m, const int* W, const UGeom& g,
                                  uint8_t* udec, hipStream_t st) {
  const int64_t total = (int64_t)g.nq * g.nu * 256;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_u_layout, dim3(blocks_for(total)), dim3(kThreads), 0, st, ucan0, ucan1, m, W[0], W[1], g, udec);
  return hipGetLastError();
}

hipError_t launch_decode_h_layout(const uint16_t* h0, const uint16_t* h1, int m, int nq, uint16_t* hq,
                                  hipStream_t st) {
  const int64_t total = (int64_t)nq * 128;
  hipLaunchKernelGGL(k_h_layout, dim3(blocks_for(total)), dim3(kThreads), 0, st, h0, h1, m, nq, hq);
  return hipGetLastError();
}

}  // namespace lb

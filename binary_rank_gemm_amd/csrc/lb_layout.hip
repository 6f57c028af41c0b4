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

// Decode U layout for one path: row tiles of 16 rows in quads, word-major inside
// a quad: element (quad, woff + w, row, rt % 4) = permuted canonical word of row
// 16 rt + row.  One (quad, 4 consecutive words) block is 1 KB: the 16 rows x 4
// words x 4 row tiles one MFMA step of the decode U stage consumes.
__global__ void k_retile_u(const uint32_t* __restrict__ ucan, int m, int W, int uw, int woff, int nrt,
                           uint32_t* __restrict__ udec) {
  int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t total = (int64_t)nrt * W * 16;
  if (idx >= total) return;
  int row = (int)(idx % 16);
  int w = (int)((idx / 16) % W);
  int rt = (int)(idx / (16 * (int64_t)W));
  int64_t i = (int64_t)16 * rt + row;
  uint32_t out = 0;
  if (i < m) {
    uint32_t in = ucan[i * W + w];
    for (int e = 0; e < 32; ++e) out |= ((in >> e) & 1u) << fp4_bit_of_elem(e);
  }
  udec[(((int64_t)(rt >> 2) * uw + woff + w) * 16 + row) * 4 + (rt & 3)] = out;
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

hipError_t launch_retile_u_decode(const uint32_t* ucan, int m, int r, int W, int uw, int woff,
                                  uint32_t* udec, hipStream_t st) {
  (void)r;
  int nrt = (m + kTile - 1) / kTile;
  int64_t total = (int64_t)nrt * W * 16;
  hipLaunchKernelGGL(k_retile_u, dim3(blocks_for(total)), dim3(kThreads), 0, st, ucan, m, W, uw, woff, nrt, udec);
  return hipGetLastError();
}

}  // namespace lb

// Fused decode forward (few tokens, bf16 I/O) over a list of linears.
//
// Computes, for every entry and path p, the factorised order of the paper
// notes ("LittleBit: Ultra Low-Bit Quantization via Latent Factorization",
// section "Key design"): t = x o g_p, z_p = t V_p, z'_p = z_p o l_p, and then
// y = sum_p (z'_p U_p^T) o h_p (section "Residual compensation" for the sum).
//
// Three launches per step, each over many small, evenly sized work items (one
// workgroup each, handed out by the hardware dispatcher, several resident per
// CU so that one item's start-up overlaps the others' streaming):
//   V kernel, item (entry, path, column tiles, range of 128-row chunks): the
//     four waves split the chunks, stream the sign words through per-wave rings
//     of direct-to-LDS loads, and leave the item's partial sums of z_p (and of
//     the correction term below) in a partial slot, combined across the waves
//     in a fixed order.
//   mid kernel, item (entry, path): sums the partial slots in a fixed order,
//     forms z'_p and writes it as the U stage's fp8 A operands plus the U
//     stage's correction sums.
//   U kernel, item (entry, run of quads of 64 output rows): each wave streams
//     its quads' sign words through its ring against the A operands held in
//     registers, and writes y for its rows, both paths.
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
//
// Ring bookkeeping: every ring step is exactly one direct-to-LDS load issued
// kRing - 1 steps ahead (past the end of the work a wave loads again bytes the
// cache holds), and vector-memory operations complete in issue order,
// so "at most N operations outstanding" tells when a slot has landed.  Sign
// words and row scales, read exactly once, go through the non-temporal cache
// policy in launches of up to 8 tokens.  The U kernel's output
// stores sit at fixed places in its step pattern and its waits allow for them.
#include "lb_internal.h"
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>
#include <utility>

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
// Launch-constant tables (work items, entries, pointer arrays) are read as
// constant memory, so uniform reads of them become scalar loads instead of
// vector loads queued behind the streaming traffic.
#define LB_CONST __attribute__((address_space(4)))
template <class T>
__device__ inline const LB_CONST T* cp(const T* p) { return (const LB_CONST T*)p; }
// copy of a constant-memory struct (word by word: copy constructors take generic references)
template <class T>
__device__ inline T cld(const LB_CONST T* p) {
  static_assert(sizeof(T) % 4 == 0, "word-sized struct");
  T v;
  const LB_CONST int* src = (const LB_CONST int*)p;
  int* dst = reinterpret_cast<int*>(&v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) dst[i] = src[i];
  return v;
}

// Loads of data another workgroup wrote earlier in the same launch (HL = true,
// the persistent chained kernel, whose workgroups all run on one XCD): group-
// scope loads, which miss in the compute unit's vector cache and read the
// XCD's L2, where the writer's stores have landed.  Other launches (HL =
// false) read plainly: a kernel boundary makes the data visible.
template <bool HL, class T>
__device__ inline T ld_h(const LB_GLOBAL T* p) {
  if constexpr (HL) return __hip_atomic_load(const_cast<LB_GLOBAL T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else return *p;
}
// cache policy of direct-to-LDS loads of such data (x): group scope when HL
template <bool HL>
constexpr int kHandAux = HL ? 1 : 0;

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ inline float f16f(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// float -> bf16 bits, round to nearest even (the hardware conversion)
__device__ inline uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <int N>
__device__ inline float ror16(float v) {  // rotate within a row of 16 lanes (DPP row_ror)
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
// Largest of a row of 16 lanes' values, all non-negative: for non-negative
// floats the order of their bit patterns is the order of the values, so an
// unsigned integer max (identity 0, which the rotate's fill value already is)
// becomes one DPP max per step, where fmaxf takes four instructions.
template <int N>
__device__ inline uint32_t ror16u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xF, 0xF, false);
}
__device__ inline float row16_max_nonneg(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, ror16u<8>(u));
  u = max(u, ror16u<4>(u));
  u = max(u, ror16u<2>(u));
  u = max(u, ror16u<1>(u));
  return __uint_as_float(u);
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

// 1.0 in every fp4 nibble, held in a register (made once per stream):
// three-operand instructions take no literal here, so with the constant as
// an immediate the sign class of expand_signs costs an and plus an or, with
// it in a register one v_and_or.
__device__ inline uint32_t fp4_ones() {
  uint32_t one = 0x22222222u;
  __asm__("" : "+v"(one));
  return one;
}

// fp4 B operand from one packed word (bit layout of fp4_bit_of_elem); one =
// fp4_ones().
__device__ inline v8i expand_signs(uint32_t w, uint32_t one) {
  v8i b;
  b[0] = (int)((w & 0x88888888u) | one);           // +-1
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
// An image of AR rows (AR = 2: the hi and lo rows of one token): row r is
// stored at r mod AR, so a lane of a row past AR reads a stored row (MFMA rows
// are independent; those rows of the result are never read).  AR = 16 is the
// full image above, with its scale bytes at 2048.
template <int AR>
__host__ __device__ inline int img_off_r(int row, int g, int e) {
  return (e >> 4) * (AR * 64) + ((row & (AR - 1)) * 4 + g) * 16 + (e & 15);
}
template <int AR>
__host__ __device__ inline constexpr int img_scales(int row, int g) { return AR * 128 + (row & (AR - 1)) * 4 + g; }
template <int AR>
__host__ __device__ inline constexpr int img_bytes() { return (AR * 132 + 15) / 16 * 16; }
static_assert(img_bytes<16>() == kABytes, "the full image is kABytes");

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

typedef short short2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Converts this lane's two values (already multiplied by the class factor) of
// token slot tt into the A image `ab` at the lane's K position; the 16 lanes of
// a DPP row hold one 32-element block.  Returns the lane's contribution to C.
template <int AR = 16, class Ptr>
__device__ inline float convert_pair(const ConvLane& L, float t0, float t1, int tt, Ptr ab) {
  float mx = row16_max_nonneg(fmaxf(fabsf(t0), fabsf(t1)));
  int ex;
  frexpf(mx, &ex);
  int E = ex - 8;                       // max / 2^E in [128, 256)
  E = E < -122 ? -122 : (E > 127 ? 127 : E);
  // the scaled conversions divide by their scale going to fp8 and multiply by
  // it coming back (powers of two: exact), so H = hi 2^E, L = lo 2^(E - 4)
  const float sc = __builtin_bit_cast(float, (E + 127) << 23), sl = __builtin_bit_cast(float, (E + 123) << 23);
  const short2v zero2 = {0, 0};
  const int hi = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero2, t0, t1, sc, false)) & 0xffff;
  const float2v H = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, sc, false);
  const int lo = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(zero2, t0 - H[0], t1 - H[1], sl, false)) & 0xffff;
  const float2v Lq = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, sl, false);
  const int mhi = 2 * tt, mlo = 2 * tt + 1;
  using U16 = typename std::conditional<std::is_same<Ptr, uint8_t*>::value, uint16_t, LB_GLOBAL uint16_t>::type;
  *reinterpret_cast<U16*>(ab + img_off_r<AR>(mhi, L.gdst, L.edst)) = (uint16_t)hi;
  *reinterpret_cast<U16*>(ab + img_off_r<AR>(mlo, L.gdst, L.edst)) = (uint16_t)lo;
  if (std::is_same<Ptr, uint8_t*>::value || L.sub == 0) {
    // into LDS every lane of the row writes its block's scale bytes (the same
    // value to the same byte): no branch, so the conversions of successive
    // tokens stay in one block that the compiler can interleave
    ab[img_scales<AR>(mhi, L.kb)] = (uint8_t)(E + 127);
    ab[img_scales<AR>(mlo, L.kb)] = (uint8_t)(E + 127 - 4);
  }
  // quantised value of t (A / class factor), summed over the three {0, beta} classes
  return ((H[0] + H[1]) + (Lq[0] + Lq[1])) * L.finv;
}

// Reads lane (mr, gr)'s A operand and scale from an A image (LDS or global).
// Rows past the real tokens hold stale values: MFMA rows are independent and
// those rows of the result are never read.
template <bool HL = false, int AR = 16, class Ptr>
__device__ inline void load_a(Ptr ab, int mr, int gr, v8i& a, int& sc) {
  constexpr bool kLds = std::is_same<Ptr, const uint8_t*>::value || std::is_same<Ptr, uint8_t*>::value;
  if constexpr (HL && !kLds) {
    // hand-over loads of 8 bytes (the widest such load)
    const LB_GLOBAL uint64_t* lo = reinterpret_cast<const LB_GLOBAL uint64_t*>(ab + img_off(mr, gr, 0));
    const LB_GLOBAL uint64_t* hi = reinterpret_cast<const LB_GLOBAL uint64_t*>(ab + img_off(mr, gr, 16));
    const uint64_t w0 = ld_h<true>(lo), w1 = ld_h<true>(lo + 1), w2 = ld_h<true>(hi), w3 = ld_h<true>(hi + 1);
    a = v8i{(int)w0, (int)(w0 >> 32), (int)w1, (int)(w1 >> 32), (int)w2, (int)(w2 >> 32), (int)w3, (int)(w3 >> 32)};
    sc = ld_h<true>(ab + 2048 + mr * 4 + gr);
  } else {
    using V4 = typename std::conditional<kLds, const v4i, const LB_GLOBAL v4i>::type;
    const v4i lo = *reinterpret_cast<V4*>(ab + img_off_r<AR>(mr, gr, 0));
    const v4i hi = *reinterpret_cast<V4*>(ab + img_off_r<AR>(mr, gr, 16));
    a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    sc = ab[img_scales<AR>(mr, gr)];
  }
}



// ---------------------------------------------------------------------------
// Ring of direct-to-LDS loads (one per wave)
// ---------------------------------------------------------------------------
constexpr int kRing = 10;                  // 1 KB slots per wave
constexpr int kRingBytes = kRing * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_block + 16 l.
template <int AUX = 0>
__device__ inline void dma16(const LB_GLOBAL void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)lds_block, 16, 0, AUX);
}
// The same with the non-temporal cache policy (NT), for data a step reads
// exactly once (the sign words and row scales): measured on MI355X, a ring of
// such loads streams 7.05 TB/s against 6.24 TB/s with the default policy.
// Launches of up to 8 tokens, which stream, take it (the Llama-2-70B stack at
// one token: 195.5 -> 183.5 us); at 16 tokens, where the stages are bound by
// their arithmetic, it measured 3 % slower, so they keep the default.
constexpr int kNtAux = 2;
template <int TM>
__device__ inline void dma16_once(const LB_GLOBAL void* src, void* lds_block) {
  __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)lds_block, 16, 0, TM <= 8 ? kNtAux : 0);
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
// Waits for this wave's outstanding LDS accesses.
__device__ inline void lds_wait() {
  constexpr int imm = 15 | (7 << 4) | (0 << 8) | (3 << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  asm volatile("" ::: "memory");
}

template <class F, int... I>
__device__ __attribute__((always_inline)) inline void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, i>) for i = 0 .. N-1, in order
template <int N, class F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// V stage
// ---------------------------------------------------------------------------
// TM: token-count bucket of the launch (1, 2, 4, 8 or 16): per-token state is
// sized by TM, MFMA token blocks of 8 by TB.
template <int TM>
struct VShape {
  static constexpr int TB = (TM + 7) / 8;
  static constexpr int CT = decode_v_tiles(TM);   // most column tiles of an item
  static constexpr int SMAX = (CT + 3) / 4;       // sign steps per chunk (4 tiles each)
  static constexpr int XS = (TM + 4) / 4;         // steps per chunk holding g and TM rows of x (256 B each)
  // rows of a wave's A image: at one and two tokens only their hi and lo rows
  // (272 and 528 bytes instead of 2112)
  static constexpr int AR = TM <= 2 ? 2 * TM : 16;
  static constexpr int AB = img_bytes<AR>();
  // ring slots per wave: 9 at one token, where four workgroups then fit a CU
  // (37 KB of LDS and at most 128 VGPRs each), 11 at two (the LDS the smaller
  // image leaves) and at eight (three workgroups of 53 KB), else kRing (at 4
  // tokens 11 or 12 measured no faster, at 16 tokens 14 slower)
  static constexpr int RING = TM == 1 ? 9 : TM == 2 || TM == 8 ? 11 : kRing;
  static constexpr int RINGB = RING * 1024;
  static constexpr int WPC = TM == 1 ? 4 : TM >= 16 ? 2 : 3;   // workgroups per CU
  static constexpr size_t lds = (size_t)kWaves * RINGB + (size_t)kWaves * TB * AB;
  static_assert(WPC * lds <= 160 * 1024, "workgroups per CU fit its LDS");
};

// Partial sums of one wave's chunks: acc (z_p before the correction term) and
// cpart (the correction term per token).  Fast form: every read goes through
// the wave's ring (x rows of n % 8 == 0 elements).  The chunks go in groups of
// G (two at one token, so that one 1 KB step carries both chunks' g and x
// rows), each group being its x/g steps followed by each chunk's sign steps.
template <int TM, bool HL>
__device__ __attribute__((always_inline)) inline void v_stream(const DecArgs& a, const VItem& it, int n, int nct,
                                                              const LB_GLOBAL uint8_t* xb, const LB_GLOBAL uint8_t* gdec,
                                                              const LB_GLOBAL uint8_t* vdec, int ca, int cb, uint8_t* ring,
                                                              uint8_t* abuf, v4f (&acc)[VShape<TM>::CT][VShape<TM>::TB],
                                                              float (&cpart)[TM]) {
  using S = VShape<TM>;
  constexpr int TB = S::TB, XS = S::XS;
  constexpr int G = TM == 1 ? 2 : 1;           // chunks per group
  const int lane = threadIdx.x & 63, mr = lane & 15, gr = lane >> 4;
  const int T = a.T, ntl = it.ntiles, ss = (ntl + 3) / 4;
  // issue cursor: group of chunks [ic, ic + ng), step ik of the group (XS x/g
  // steps, then chunk ic + jc's sign step js)
  int ic = ca, ik = 0, jc = 0, js = 0;
  int ng = min(G, cb - ca);
  const LB_GLOBAL uint8_t* last = gdec;
  bool last_signs = false;                     // the step streams sign words (read once)
  auto issue = [&](int slot) __attribute__((always_inline)) {
    if (ic < cb) {
      last_signs = ik >= XS;
      if (ik < XS) {
        if constexpr (G == 2) {
          // lane l: 16 bytes (elements 8 (l % 16) .. + 7) of g (l / 16 even) or x (odd) of chunk ic + l / 32
          const int c = ic + min(lane >> 5, ng - 1);
          const int e0 = c * kChunk + 8 * (lane & 15);
          last = (lane >> 4) & 1 ? xb + (int64_t)min(e0, n - 8) * 2 : gdec + (int64_t)e0 * 2;
        } else {
          // lane l: row 4 ik + l / 16 of the step (0: g, 1 + t: token t), elements 8 (l % 16) .. + 7
          const int rho = 4 * ik + (lane >> 4);
          const int e0 = ic * kChunk + 8 * (lane & 15);
          if (rho == 0) {
            last = gdec + (int64_t)e0 * 2;
          } else {
            const int t = min(rho - 1, T - 1);
            last = xb + ((int64_t)t * n + min(e0, n - 8)) * 2;
          }
        }
        ++ik;
      } else {
        // lane l: 16 bytes of column tile 4 js + l / 16 of the item (its last tile past the item's tiles)
        const int tile = it.tile0 + min(4 * js + (lane >> 4), ntl - 1);
        last = vdec + ((int64_t)(ic + jc) * nct + tile) * 256 + (lane & 15) * 16;
        if (++js == ss) {
          js = 0;
          if (++jc == ng) {
            ic += ng;
            ng = min(G, cb - ic);
            ik = 0;
            jc = 0;
          }
        }
      }
    } else if constexpr (TM <= 8) {
      // past the end of the work: a load that keeps the one-load-per-step
      // count, from bytes the cache holds (g at the wave's first chunk), not
      // the last, non-temporal, sign step again (which would go to memory)
      last = gdec + (int64_t)ca * kChunk * 2 + (lane & 15) * 16;
      last_signs = false;
    }
    if (last_signs) dma16_once<TM>(last, ring + slot * 1024);
    else dma16<kHandAux<HL>>(last, ring + slot * 1024);
  };
  constexpr int R = S::RING;
#pragma unroll
  for (int k = 0; k < R - 1; ++k) issue(k);
  int s = 0;
  auto next_step = [&]() __attribute__((always_inline)) {
    lds_wait();                                // the slot reloaded next was read last step
    issue((s + R - 1) % R);
    vm_wait<R - 1>();
    const uint8_t* slot = ring + (s % R) * 1024;
    ++s;
    return slot;
  };
  const ConvLane L(lane);
  const uint32_t one = fp4_ones();
  for (int c0 = ca; c0 < cb; c0 += G) {
    const int ngc = min(G, cb - c0);
    // this lane's elements kloc, kloc + 1 (= 2 lane, 2 lane + 1) of g and of each token row, per chunk
    uint32_t gpair[G], xpair[G][TM];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      gpair[g] = 0;
#pragma unroll
      for (int t = 0; t < TM; ++t) xpair[g][t] = 0;
    }
#pragma unroll
    for (int j = 0; j < XS; ++j) {
      const uint8_t* slot = next_step();
      if constexpr (G == 2) {
        gpair[0] = *reinterpret_cast<const uint32_t*>(slot + 4 * lane);
        xpair[0][0] = *reinterpret_cast<const uint32_t*>(slot + 256 + 4 * lane);
        gpair[1] = *reinterpret_cast<const uint32_t*>(slot + 512 + 4 * lane);
        xpair[1][0] = *reinterpret_cast<const uint32_t*>(slot + 768 + 4 * lane);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rho = 4 * j + q;
          if (rho == 0) gpair[0] = *reinterpret_cast<const uint32_t*>(slot + 4 * lane);
          else if (rho - 1 < TM) xpair[0][rho - 1] = *reinterpret_cast<const uint32_t*>(slot + q * 256 + 4 * lane);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g < ngc) {
        const int k0 = (c0 + g) * kChunk + L.kloc;
        const bool v0 = k0 < n, v1 = k0 + 1 < n;
        const float g0 = f16f((uint16_t)(gpair[g] & 0xffff)) * L.fcls, g1 = f16f((uint16_t)(gpair[g] >> 16)) * L.fcls;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const int t = tb * 8 + tt;
            // up to 8 tokens every token slot of the bucket: the ring holds
            // the last token's row again for slots past T, whose MFMA rows are
            // never read, and without a test per token the conversions form
            // one block the compiler interleaves (at 16 tokens that takes more
            // registers than two workgroups per CU leave: it keeps the test)
            if (t < TM && (TM <= 8 || t < T)) {
              const float x0 = bf16f((uint16_t)(xpair[g][t] & 0xffff)), x1 = bf16f((uint16_t)(xpair[g][t] >> 16));
              cpart[t] += convert_pair<S::AR>(L, v0 ? x0 * g0 : 0.f, v1 ? x1 * g1 : 0.f, tt, abuf + tb * S::AB);
            }
          }
        }
        wave_lds_fence();
        v8i A[TB];
        int sc[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) load_a<false, S::AR>(abuf + tb * S::AB, mr, gr, A[tb], sc[tb]);
        wave_lds_fence();
#pragma unroll
        for (int j = 0; j < S::SMAX; ++j) {
          if (j < ss) {
            const uint8_t* slot = next_step();
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = *reinterpret_cast<const uint32_t*>(slot + i * 256 + 4 * lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (4 * j + i < S::CT && 4 * j + i < ntl) {
                const v8i B = expand_signs(w[i], one);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) acc[4 * j + i][tb] = mfma(A[tb], B, acc[4 * j + i][tb], sc[tb]);
              }
            }
          }
        }
      }
    }
  }
  vm_wait<0>();                                // no direct-to-LDS load may still be in flight
}

// The same partial sums with plain loads (x rows that 16-byte loads cannot
// read: n % 8 != 0).  Slow, and only for odd shapes.
template <int TM>
__device__ __attribute__((always_inline)) inline void v_plain(const DecArgs& a, const VItem& it, int n, int nct,
                                                             const LB_GLOBAL uint8_t* xb, const LB_GLOBAL uint8_t* gdec,
                                                             const LB_GLOBAL uint8_t* vdec, int ca, int cb, uint8_t* abuf,
                                                             v4f (&acc)[VShape<TM>::CT][VShape<TM>::TB],
                                                             float (&cpart)[TM]) {
  using S = VShape<TM>;
  constexpr int TB = S::TB;
  const int lane = threadIdx.x & 63, mr = lane & 15, gr = lane >> 4;
  const int T = a.T, ntl = it.ntiles;
  const ConvLane L(lane);
  const LB_GLOBAL uint16_t* x = reinterpret_cast<const LB_GLOBAL uint16_t*>(xb);
  const LB_GLOBAL uint16_t* g = reinterpret_cast<const LB_GLOBAL uint16_t*>(gdec);
  const uint32_t one = fp4_ones();
  for (int c = ca; c < cb; ++c) {
    const int k0 = c * kChunk + L.kloc;
    const bool v0 = k0 < n, v1 = k0 + 1 < n;
    const float g0 = f16f(g[k0]) * L.fcls, g1 = f16f(g[k0 + 1]) * L.fcls;   // g is padded to whole chunks
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int t = tb * 8 + tt;
        if (t < TM && t < T) {
          const float x0 = v0 ? bf16f(x[(int64_t)t * n + k0]) : 0.f;
          const float x1 = v1 ? bf16f(x[(int64_t)t * n + k0 + 1]) : 0.f;
          cpart[t] += convert_pair<S::AR>(L, x0 * g0, x1 * g1, tt, abuf + tb * S::AB);
        }
      }
    }
    wave_lds_fence();
    v8i A[TB];
    int sc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) load_a<false, S::AR>(abuf + tb * S::AB, mr, gr, A[tb], sc[tb]);
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < S::CT; ++i) {
      if (i < ntl) {
        const uint32_t w = *reinterpret_cast<const LB_GLOBAL uint32_t*>(vdec + ((int64_t)c * nct + it.tile0 + i) * 256 +
                                                                       lane * 4);
        const v8i B = expand_signs(w, one);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[i][tb] = mfma(A[tb], B, acc[i][tb], sc[tb]);
      }
    }
  }
}

// One V work item on this workgroup (lds: VShape<TM>::lds bytes).  HL: x is
// read with hand-over loads (only entries with xdirect).
template <int TM, bool HL>
__device__ __attribute__((always_inline)) inline void v_item(const DecArgs& a, const VItem& it, uint8_t* lds) {
  using S = VShape<TM>;
  constexpr int TB = S::TB, CT = S::CT;
  const LB_CONST DecEntry& Eg = cp(a.entries)[it.entry];
  const int tid = threadIdx.x, lane = tid & 63, mr = lane & 15, gr = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = it.path;
  // snapshot of the entry
  const int n = Eg.n, nct = Eg.p[p].nct, xdirect = Eg.xdirect;
  const LB_GLOBAL uint8_t* vdec = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.p[p].vdec));
  const LB_GLOBAL uint8_t* gdec = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.gdec[p]));
  const void* xv = a.xs ? cp(a.xs)[it.entry] : a.x0;
  const LB_GLOBAL uint8_t* xb = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(xv)) + (int64_t)a.t0 * n * 2;
  uint8_t* ring = lds + wave * S::RINGB;
  uint8_t* abuf = lds + kWaves * S::RINGB + wave * TB * S::AB;
  // this wave's chunks: a contiguous quarter of the item's, the quarters as
  // even as whole groups of chunks allow (groups of two at one token)
  constexpr int GV = TM == 1 ? 2 : 1;
  const int ngrp = (it.c1 - it.c0 + GV - 1) / GV;
  const int ca = min(it.c0 + GV * (wave * ngrp / kWaves), it.c1);
  const int cb = min(it.c0 + GV * ((wave + 1) * ngrp / kWaves), it.c1);

  v4f acc[CT][TB];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[c][tb] = v4f{0.f, 0.f, 0.f, 0.f};
  float cpart[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) cpart[t] = 0.f;
  if (ca < cb) {
    if (HL || xdirect) v_stream<TM, HL>(a, it, n, nct, xb, gdec, vdec, ca, cb, ring, abuf, acc, cpart);
    else v_plain<TM>(a, it, n, nct, xb, gdec, vdec, ca, cb, abuf, acc, cpart);
  }

  // fixed-order combine across waves in the (now idle) ring memory
  float cw_[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) cw_[t] = wave_sum(cpart[t]);
  const int ntl = it.ntiles;
  LB_GLOBAL float* slot = gp(a.part) + (int64_t)it.slot * decode_slot_floats(TM);
  // lane (mr, gr) holds MFMA rows 4 gr .. 4 gr + 3 = (hi, lo) of tokens
  // tb * 8 + 2 gr + {0, 1}, column mr
  auto wave_part = [&](float* dst, bool add) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      if (c < ntl) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const int t = tb * 8 + 2 * gr + qq;
            if (t < TM) {
              float* d = dst + (c * TM + t) * 16 + mr;
              const float v = acc[c][tb][2 * qq] + acc[c][tb][2 * qq + 1];
              *d = add ? *d + v : v;
            }
          }
      }
    }
  };
  __syncthreads();
  if constexpr (kWaves * (CT * TM * 16 + TM) * 4 <= S::RINGB * kWaves) {
    // each wave writes its own copy, then every thread adds the four in wave order
    float* red = reinterpret_cast<float*>(lds);    // [wave][tile][token][16]
    float* cred = red + kWaves * CT * TM * 16;     // [wave][token]
    wave_part(red + wave * CT * TM * 16, false);
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < TM; ++t) cred[wave * TM + t] = cw_[t];
    }
    __syncthreads();
    for (int i = tid; i < ntl * TM * 16; i += kThreads)
      slot[i] = ((red[i] + red[CT * TM * 16 + i]) + red[2 * CT * TM * 16 + i]) + red[3 * CT * TM * 16 + i];
    if (tid < TM) slot[CT * TM * 16 + tid] = ((cred[tid] + cred[TM + tid]) + cred[2 * TM + tid]) + cred[3 * TM + tid];
    return;
  } else {
    // wave 0 stores, waves 1..3 add in turn
    float* red = reinterpret_cast<float*>(lds);    // [tile][token][16]
    float* cred = red + CT * TM * 16;              // [token]
    for (int wv = 0; wv < kWaves; ++wv) {
      if (wave == wv) {
        wave_part(red, wv != 0);
        if (lane == 0) {
#pragma unroll
          for (int t = 0; t < TM; ++t) cred[t] = (wv == 0 ? 0.f : cred[t]) + cw_[t];
        }
      }
      __syncthreads();
    }
    for (int i = tid; i < ntl * TM * 16; i += kThreads) slot[i] = red[i];
    if (tid < TM) slot[CT * TM * 16 + tid] = cred[tid];
  }
}

template <int TM>
__global__ void __launch_bounds__(kThreads, VShape<TM>::WPC) k_decode_v(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  v_item<TM, false>(a, cld(cp(a.vitems) + blockIdx.x), lds);
}

// ---------------------------------------------------------------------------
// mid stage
// ---------------------------------------------------------------------------
// z' = (sum of the partial sums + correction) o l for one path of one entry,
// written as the U stage's A operands: each 16-lane row takes one (token,
// 32-latent block), lane sub holding latents 2 sub and 2 sub + 1 of it.  Every
// block of the path's units is written (zeros past the rank).
// Floats of LDS the mid step uses (per-block correction sums).
constexpr int kMidLdsFloats = kDecodeMaxTokens * 4 * (LB_MAX_RANK / kChunk);

// One mid work item on this workgroup (cblk: kMidLdsFloats floats of LDS).
// HL: the partial sums are read with hand-over loads.
template <int TM, bool HL>
__device__ __attribute__((always_inline)) inline void mid_item(const DecArgs& a, const MItem& it, float* cblk) {
  constexpr int TB = (TM + 7) / 8, CT = decode_v_tiles(TM), SF = decode_slot_floats(TM);
  const LB_CONST DecEntry& E = cp(a.entries)[it.entry];
  const int p = it.path, r = E.p[p].r, T = a.T;
  const LB_GLOBAL uint16_t* lsc = gp(E.p[p].l);
  const LB_GLOBAL float* part = gp(a.part);
  const int ufirst = p ? E.ug.nu0 : 0;
  const int nblk = 4 * ((r + kChunk - 1) / kChunk);
  // 16-lane rows of the workgroup (16 in the chained kernel's 256 threads;
  // the mid launch has 32 at 4 and 8 tokens and 64 at 16: with one memory
  // round trip per position a row takes, more rows mean fewer round trips in
  // a row)
  const int tid = threadIdx.x, row = tid >> 4, sub = tid & 15, nrows = (int)(blockDim.x >> 4);
  for (int u = row; u < T * nblk; u += nrows) {
    const int t = u / nblk, blk = u % nblk, tb = t / 8, tt = t % 8;
    const int jj = 32 * blk + 2 * sub;             // latents jj, jj + 1
    const ConvLane LK(((jj % kChunk) / 32) * 16 + sub);
    // the partial sums of both latents over the splits, added in split order;
    // the loads of up to kB splits go out together (the two latents share a
    // column tile, hence a partial slot and its correction sum).  The mid
    // launch takes 8 (more registers would lower its occupancy: 32 measured
    // 7.8 against 4.9 us on the Llama-2-70B stack); the chained kernel, whose
    // mid steps sit on the critical path one at a time, takes 32
    constexpr int kB = HL ? 32 : 8;
    const int tile = jj / 16, col = jj % 16, g = tile / it.gtiles, tl = tile - g * it.gtiles;
    const bool in[2] = {jj < r, jj + 1 < r};
    const LB_GLOBAL float* sp = part + (int64_t)(it.slot0 + g * it.nsplit) * SF;
    const int off = (tl * TM + t) * 16 + col;
    float d[2] = {0.f, 0.f}, c = 0.f;
    for (int s0 = 0; s0 < it.nsplit; s0 += kB) {
      float dv[2][kB], cv[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (in[0] && s0 + i < it.nsplit) {
          const LB_GLOBAL float* q = sp + (int64_t)(s0 + i) * SF;
          dv[0][i] = ld_h<HL>(q + off);
          if (in[1]) dv[1][i] = ld_h<HL>(q + off + 1);
          cv[i] = ld_h<HL>(q + CT * TM * 16 + t);
        }
#pragma unroll
      for (int i = 0; i < kB; ++i)
        if (in[0] && s0 + i < it.nsplit) {
          d[0] += dv[0][i];
          if (in[1]) d[1] += dv[1][i];
          c += cv[i];
        }
    }
    float v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) v[q] = in[q] ? (d[q] + c) * f16f(lsc[jj + q]) * LK.fcls : 0.f;
    uint8_t* ab = E.aimg + ((int64_t)(ufirst + jj / kChunk) * TB + tb) * kABytes;
    const float cc = row16_sum(convert_pair(LK, v[0], v[1], tt, gp(ab)));
    if (sub == 0) cblk[u] = cc;
  }
  __syncthreads();
  if (tid < T) {
    float s = 0.f;
    for (int blk = 0; blk < nblk; ++blk) s += cblk[tid * nblk + blk];
    gp(E.cval)[p * 16 + tid] = s;
  }
}

// Threads of a mid workgroup: 256 up to 2 tokens (a path's positions fit
// 16 rows), 512 at 4 and 8 tokens (1024 left half the rows of the small k
// and v paths idle: 8 tokens measured 0.6 % faster), 1024 at 16.
template <int TM>
constexpr int mid_threads() { return TM >= 16 ? 1024 : TM >= 4 ? 512 : kThreads; }

template <int TM>
__global__ void __launch_bounds__(mid_threads<TM>()) k_decode_mid(DecArgs a) {
  __shared__ float cblk[kMidLdsFloats];
  mid_item<TM, false>(a, cld(cp(a.mitems) + blockIdx.x), cblk);
}

// ---------------------------------------------------------------------------
// U stage
// ---------------------------------------------------------------------------
// Outputs are staged in LDS for all of a wave's quads and stored after its
// stream has drained: a store inside the stream would hold up the in-order
// completion count of every load behind it for the store's own latency.
template <int TM>
struct UShape {
  static constexpr int TB = (TM + 7) / 8;
  static constexpr int KQQ = TM == 1 ? 1 : 2;          // token slots per lane and block
  static constexpr int KST = TM > 8 ? 2 : 1;           // output stores per quad (8 tokens x 64 rows each)
  static constexpr int NMAX = TB == 1 ? 8 : 6;         // most units with operands held in registers
  static constexpr int QW = decode_u_qw_max(TM);       // most quads per wave
  static constexpr int STG = QW * TM * 128;            // staging bytes per wave
  static constexpr size_t lds = (size_t)kWaves * (kRingBytes + STG);
};

// Per-lane state shared by both U forms.
template <int TM>
struct UCtx {
  static constexpr int TB = UShape<TM>::TB;
  int m, T, np, nu0, yf32;
  LB_GLOBAL uint16_t* y;                           // bf16 y at this launch's first token
  LB_GLOBAL float* yf;                             // the same as fp32 (yf32)
  float cv[2][TB][2];                              // U correction sums of the lane's tokens
};

// part (+)= h (D_hi + D_lo + C_p); lane (mr, gr) holds MFMA rows 4 gr .. 4 gr + 3
// = (hi, lo) of tokens tb * 8 + 2 gr + {0, 1}, column mr = output row
template <int TB>
__device__ __attribute__((always_inline)) inline void u_fold(const v4f (&acc)[4][TB], const float (&h)[4],
                                                            const float (&cv)[TB][2], float (&part)[4][TB][2],
                                                            bool first) {
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const float v = h[rt] * ((acc[rt][tb][2 * qq] + acc[rt][tb][2 * qq + 1]) + cv[tb][qq]);
        part[rt][tb][qq] = first ? v : part[rt][tb][qq] + v;
      }
}

// Element-wise stores of one quad (any m), then a wait for all of them.
template <int TM>
__device__ __attribute__((always_inline)) inline void u_store_plain(const UCtx<TM>& C, int q,
                                                                   const float (&part)[4][UShape<TM>::TB][2]) {
  const int lane = threadIdx.x & 63, mr = lane & 15, gr = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tb = 0; tb < UShape<TM>::TB; ++tb)
#pragma unroll
      for (int qq = 0; qq < UShape<TM>::KQQ; ++qq) {
        const int t = tb * 8 + 2 * gr + qq, i = 64 * q + 16 * rt + mr;
        if (t < C.T && i < C.m) {
          if (C.yf32) C.yf[(int64_t)t * C.m + i] = part[rt][tb][qq];
          else C.y[(int64_t)t * C.m + i] = bf16_bits(part[rt][tb][qq]);
        }
      }
  vm_wait<0>();
}

// One quad's outputs into the wave's staging area: [token][64 rows] bf16,
// or fp32 (twice the bytes per quad) when y is fp32.
template <int TM>
__device__ __attribute__((always_inline)) inline void u_stage(const float (&part)[4][UShape<TM>::TB][2], uint8_t* stq,
                                                             int yf32) {
  const int lane = threadIdx.x & 63, mr = lane & 15, gr = lane >> 4;
  uint16_t* s16 = reinterpret_cast<uint16_t*>(stq);
  float* s32 = reinterpret_cast<float*>(stq);
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int tb = 0; tb < UShape<TM>::TB; ++tb)
#pragma unroll
      for (int qq = 0; qq < UShape<TM>::KQQ; ++qq) {
        const int t = tb * 8 + 2 * gr + qq;
        if (t < TM) {
          if (yf32) s32[t * 64 + rt * 16 + mr] = part[rt][tb][qq];
          else s16[t * 64 + rt * 16 + mr] = bf16_bits(part[rt][tb][qq]);
        }
      }
}

// Staged quads [qa, qa + nst) to y: KST stores of 16 bytes per lane and quad
// (lane l: token 8 k + l / 8, rows 8 (l % 8) .. + 7).  Lanes past the last
// token repeat its store (same address, same value).
template <int TM>
__device__ __attribute__((always_inline)) inline void u_flush(const UCtx<TM>& C, int qa, int nst, const uint8_t* stg) {
  const int lane = threadIdx.x & 63;
  wave_lds_fence();
  if (C.yf32) {
    // fp32: 256 bytes per token and quad, lane l: token 4 k + l / 16, rows 4 (l % 16) .. + 3
    for (int j = 0; j < nst; ++j) {
#pragma unroll
      for (int k = 0; k < (TM + 3) / 4; ++k) {
        const int t = min(4 * k + (lane >> 4), C.T - 1);
        const u32x4 v = *reinterpret_cast<const u32x4*>(stg + (j * TM + t) * 256 + (lane & 15) * 16);
        *reinterpret_cast<LB_GLOBAL u32x4*>(C.yf + (int64_t)t * C.m + 64 * (qa + j) + (lane & 15) * 4) = v;
      }
    }
    return;
  }
  for (int j = 0; j < nst; ++j) {
#pragma unroll
    for (int k = 0; k < UShape<TM>::KST; ++k) {
      const int t = min(8 * k + (lane >> 3), C.T - 1);
      const u32x4 v = *reinterpret_cast<const u32x4*>(stg + (j * TM + t) * 128 + (lane & 7) * 16);
      *reinterpret_cast<LB_GLOBAL u32x4*>(C.y + (int64_t)t * C.m + 64 * (qa + j) + (lane & 7) * 8) = v;
    }
  }
}

// Fast form: NPC units, operands in registers, every read through the ring.
// Steps per quad: the row scales, then one per unit.
template <int TM, int NPC, bool HL>
__device__ __attribute__((always_inline)) inline void u_stream(const DecArgs& a, const LB_CONST DecEntry& Eg, UCtx<TM>& C,
                                                              int qa, int qb, uint8_t* ring, uint8_t* stg) {
  using S = UShape<TM>;
  constexpr int TB = S::TB, P = NPC + 1;
  const int lane = threadIdx.x & 63, mr = lane & 15, gr = lane >> 4;
  const UGeom g = cld(&Eg.ug);
  const LB_GLOBAL uint8_t* udec = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.udec));
  const LB_GLOBAL uint8_t* hq = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.hq));
  const LB_GLOBAL uint8_t* aimg = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(static_cast<const uint8_t*>(Eg.aimg)));
  // byte offset of each step inside a quad's data (this lane's 16 bytes)
  int uoff[NPC];
#pragma unroll
  for (int u = 0; u < NPC; ++u) {
    const bool half = (u == g.nu0 - 1 && g.half0) || (u == g.nu - 1 && g.half1);
    uoff[u] = (u < g.nu0 ? 1024 * u : g.uoff1 + 1024 * (u - g.nu0)) + (half ? (lane & 31) : lane) * 16;
  }
  const int hoff = (lane & 15) * 16;
  // step k of the wave's sequence (k = (quad - qa) * P + i) lands in slot k % kRing
  auto issue_at = [&](int quad, int i, int slot) __attribute__((always_inline)) {
    if (quad >= qb) {
      // past the end: a load that keeps the one-load-per-step count; with the
      // non-temporal policy from bytes the cache holds (the wave's first
      // quad's row scales), else the last quad again
      if constexpr (TM <= 8) {
        dma16(hq + (int64_t)qa * 256 + hoff, ring + slot * 1024);
        return;
      }
      quad = qb - 1;
    }
    const LB_GLOBAL uint8_t* src = i == 0 ? hq + (int64_t)quad * 256 + hoff : udec + (int64_t)quad * g.qbytes + uoff[i > 0 ? i - 1 : 0];
    dma16_once<TM>(src, ring + slot * 1024);
  };
  // operands first (rows past 2 T are never read: skip their loads), then the
  // ring's first steps, then a wait for the operands alone (loads complete in
  // issue order), which leaves the ring's loads in flight
  v8i A[NPC][TB];
  int sc[NPC][TB];
#pragma unroll
  for (int u = 0; u < NPC; ++u)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      if (mr < 2 * C.T) load_a<HL>(aimg + (int64_t)(u * TB + tb) * kABytes, mr, gr, A[u][tb], sc[u][tb]);
      else {
        A[u][tb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        sc[u][tb] = 127;
      }
    }
#pragma unroll
  for (int k = 0; k < kRing - 1; ++k) issue_at(qa + k / P, k % P, k);
  vm_wait<kRing - 1>();

  // quads whose 64 rows are whole (and 16-byte aligned in y) are staged
  // (as many as the staging area holds: half as many when y is fp32)
  const int nst = (C.m & 7) == 0 ? min(max(0, min(qb, C.m / 64) - qa), C.yf32 ? S::QW / 2 : S::QW) : 0;
  const uint32_t one = fp4_ones();
  int s = 0;
  for (int q = qa; q < qb; ++q) {
    v4f acc[4][TB];
    float h[2][4];
    float part[4][TB][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = v4f{0.f, 0.f, 0.f, 0.f};
    static_for<P>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      lds_wait();                                  // the slot reloaded next was read last step
      issue_at(q + (i + kRing - 1) / P, (i + kRing - 1) % P, (s + kRing - 1) % kRing);
      vm_wait<kRing - 1>();
      const uint8_t* slot = ring + (s % kRing) * 1024;
      ++s;
      if constexpr (i == 0) {
        const uint16_t* hs = reinterpret_cast<const uint16_t*>(slot);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          h[0][rt] = f16f(hs[rt * 16 + mr]);
          h[1][rt] = f16f(hs[64 + rt * 16 + mr]);
        }
      } else {
        constexpr int u = i - 1;
        const u32x4 w = *reinterpret_cast<const u32x4*>(slot + lane * 16);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const v8i B = expand_signs(w[rt], one);
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = mfma(A[u][tb], B, acc[rt][tb], sc[u][tb]);
        }
        if (u == C.nu0 - 1 && u < NPC - 1) {       // path 0 ends before the last unit: fold it
          u_fold<TB>(acc, h[0], C.cv[0], part, true);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = v4f{0.f, 0.f, 0.f, 0.f};
        }
      }
    });
    if (C.np > 1) u_fold<TB>(acc, h[1], C.cv[1], part, false);
    else u_fold<TB>(acc, h[0], C.cv[0], part, true);
    if (q - qa < nst) u_stage<TM>(part, stg + (q - qa) * TM * (C.yf32 ? 256 : 128), C.yf32);
    else u_store_plain<TM>(C, q, part);
  }
  vm_wait<0>();                                    // no direct-to-LDS load may still be in flight
  u_flush<TM>(C, qa, nst, stg);
}

// Plain form (more units than the fast form holds): plain loads, one unit at a time.
template <int TM>
__device__ __attribute__((always_inline)) inline void u_plain(const DecArgs& a, const LB_CONST DecEntry& Eg, UCtx<TM>& C,
                                                             int qa, int qb) {
  using S = UShape<TM>;
  constexpr int TB = S::TB;
  const int lane = threadIdx.x & 63, mr = lane & 15, gr = lane >> 4;
  const UGeom g = cld(&Eg.ug);
  const LB_GLOBAL uint8_t* udec = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(Eg.udec));
  const LB_GLOBAL uint16_t* hq = gp(Eg.hq);
  const LB_GLOBAL uint8_t* aimg = reinterpret_cast<const LB_GLOBAL uint8_t*>(gp(static_cast<const uint8_t*>(Eg.aimg)));
  for (int q = qa; q < qb; ++q) {
    v4f acc[4][TB];
    float h[2][4];
    float part[4][TB][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      h[0][rt] = f16f(hq[(int64_t)q * 128 + rt * 16 + mr]);
      h[1][rt] = f16f(hq[(int64_t)q * 128 + 64 + rt * 16 + mr]);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (int u = 0; u < g.nu; ++u) {
      const bool half = (u == g.nu0 - 1 && g.half0) || (u == g.nu - 1 && g.half1);
      const int off = (u < g.nu0 ? 1024 * u : g.uoff1 + 1024 * (u - g.nu0)) + (half ? (lane & 31) : lane) * 16;
      const u32x4 w = *reinterpret_cast<const LB_GLOBAL u32x4*>(udec + (int64_t)q * g.qbytes + off);
      const uint32_t one = fp4_ones();
      v8i A[TB];
      int sc[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) load_a(aimg + (int64_t)(u * TB + tb) * kABytes, mr, gr, A[tb], sc[tb]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const v8i B = expand_signs(w[rt], one);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = mfma(A[tb], B, acc[rt][tb], sc[tb]);
      }
      if (u == g.nu0 - 1 && u < g.nu - 1) {
        u_fold<TB>(acc, h[0], C.cv[0], part, true);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[rt][tb] = v4f{0.f, 0.f, 0.f, 0.f};
      }
    }
    if (C.np > 1) u_fold<TB>(acc, h[1], C.cv[1], part, false);
    else u_fold<TB>(acc, h[0], C.cv[0], part, true);
    u_store_plain<TM>(C, q, part);
  }
}

// YF: y is fp32 (a separate instantiation, so the bf16 kernel carries none of it)
// One U work item on this workgroup (lds: UShape<TM>::lds bytes).  HL: the
// persistent chained kernel's form: A operands and correction sums read with
// hand-over loads, and only entries whose units fit the fast form (the plain
// form is left out).
template <int TM, bool YF, bool HL, int NMX = UShape<TM>::NMAX>
__device__ __attribute__((always_inline)) inline void u_item(const DecArgs& a, const UItem& it, uint8_t* lds) {
  using S = UShape<TM>;
  constexpr int TB = S::TB;
  const LB_CONST DecEntry& Eg = cp(a.entries)[it.entry];
  const int lane = threadIdx.x & 63, gr = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qa = min(it.q0 + wave * it.qw, it.q0 + it.nq), qb = min(qa + it.qw, it.q0 + it.nq);
  if (qa >= qb) return;                            // no barrier below: idle waves may leave
  UCtx<TM> C;
  C.m = Eg.m;
  C.T = a.T;
  C.np = Eg.np;
  C.nu0 = Eg.ug.nu0;
  void* yv = a.xs ? cp(a.ys)[it.entry] : a.y0;
  C.yf32 = YF;
  C.y = gp(reinterpret_cast<uint16_t*>(yv)) + (int64_t)a.t0 * C.m;
  C.yf = gp(reinterpret_cast<float*>(yv)) + (int64_t)a.t0 * C.m;
  const LB_GLOBAL float* cval = gp(Eg.cval);
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int t = tb * 8 + 2 * gr + qq;
        C.cv[p][tb][qq] = (p < C.np && t < C.T && t < TM) ? ld_h<HL>(cval + p * 16 + t) : 0.f;
      }
  uint8_t* ring = lds + wave * kRingBytes;
  uint8_t* stg = lds + kWaves * kRingBytes + wave * S::STG;
  const int nu = Eg.ug.nu;
  static_for<NMX>([&](auto I) __attribute__((always_inline)) {
    constexpr int k = decltype(I)::value + 1;
    if (nu == k) u_stream<TM, k, HL>(a, Eg, C, qa, qb, ring, stg);
  });
  if constexpr (!HL) {
    if (nu > NMX) u_plain<TM>(a, Eg, C, qa, qb);
  }
}

template <int TM, bool YF>
__global__ void __launch_bounds__(kThreads, TM >= 16 ? 2 : 3) k_decode_u(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u_item<TM, YF, false>(a, cld(cp(a.uitems) + blockIdx.x), lds);
}

// The second U launch of a 16-token decode: entries of 7 or 8 units, in the
// fast form with one workgroup per CU (their operands need the registers two
// workgroups would share); four waves of nine 1 KB loads in flight per CU still
// keep the stream going.
template <int TM, bool YF>
__global__ void __launch_bounds__(kThreads, 1) k_decode_u_wide(DecArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  u_item<TM, YF, false, kDecodeWideUnits>(a, cld(cp(a.uitems) + blockIdx.x), lds);
}

// ---------------------------------------------------------------------------
// Persistent chained decode
// ---------------------------------------------------------------------------
// A chained stack (entries reading earlier entries' outputs) runs level after
// level, and at batch 1 each level is a few hundred KB to a few MB of sign
// words: its time is the latency of its three dependent stages, not
// bandwidth.  This kernel runs every level in one launch, on the compute
// units of ONE XCD, so that the data one workgroup hands to another (partial
// sums, A operands, correction sums, y as the next level's x) stays in that
// XCD's L2: plain stores, and hand-over loads that miss in the compute unit's
// vector cache and hit the L2 (ld_h, kHandAux), at L2 latency instead of a
// trip to memory and a kernel boundary.  One XCD streams about 1.3 TB/s,
// enough for levels of this size.  The counters are device-scope atomics
// (performed where all XCDs see them), polled with device-scope loads.  Per
// level: a V phase, in which the last V item to finish for an (entry, path)
// runs that pair's mid step, then a U phase, each followed by a barrier of
// the participating workgroups.  Work items (planned for the participants),
// buffers and arithmetic are those of the kernels above, so the results are
// the same bits as launches per level.
//
// The launch is cooperative over the whole GPU (all workgroups resident), a
// multiple of 8 workgroups; the dispatcher hands workgroups to the 8 XCDs in
// turn (from wherever the previous dispatch stopped), so each XCD holds an
// eighth of them.  The participants are the workgroups that find themselves
// on XCD 0 (hardware register XCC_ID); they take ranks from a ticket counter
// (which workgroup runs which item does not change any result), and the
// others leave at once.  A participant whose ticket is past the expected
// count sets the abort flag.  Counters only grow: a launch reads the epoch
// (launches of this plan so far) and aims at epoch-scaled targets, and rank 0
// advances the epoch after the last barrier.

constexpr int kChainXcds = 8;

__device__ inline unsigned xcc_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}
__device__ inline uint64_t dev_add(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint64_t dev_load(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Longest wait at one barrier: 1 s of the 100 MHz constant clock.
constexpr uint64_t kChainTimeoutTicks = 100000000ull;

// Waits (thread 0) until *w reaches `target` or the abort flag is set; sets
// the flag itself after kChainTimeoutTicks.  Returns false on abort.
__device__ inline bool chain_wait(uint64_t* sync, uint64_t* w, uint64_t target) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 1; dev_load(w) < target; ++i) {
    if ((i & 15) == 0) {
      if (dev_load(sync + kChainAbort)) return false;
      if (__builtin_amdgcn_s_memrealtime() - t0 > kChainTimeoutTicks) {
        dev_add(sync + kChainAbort, 1);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Barrier number `target` of the P participants (counted over all launches
// of the plan): every wave first waits for its own stores (in the L2 once
// complete), then thread 0 adds to the barrier counter and waits for
// P x target (+ extra, which only a test of the abort path sets: no
// workgroup ever makes that arrival, so the wait times out).  Returns false
// when the launch was aborted (every participant then leaves).
__device__ inline bool chain_barrier(uint64_t* sync, uint64_t target, uint64_t P, uint64_t extra, int* flag) {
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    dev_add(sync + kChainBar, 1);
    *flag = chain_wait(sync, sync + kChainBar, target * P + extra);
  }
  __syncthreads();
  return *flag != 0;
}

template <int TM>
__global__ void __launch_bounds__(kThreads, TM >= 16 ? 1 : 2) k_decode_chain(ChainArgs c) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int flag, rank_s;
  __shared__ uint64_t epoch_s;
  const int tid = threadIdx.x;
  if (xcc_id() != 0) return;
  const uint64_t P = gridDim.x / kChainXcds;
  uint64_t* sync = c.sync;
  if (tid == 0) {
    const uint64_t epoch = dev_load(sync + kChainEpoch);
    const uint64_t rank = dev_add(sync + kChainTicket, 1) - epoch * P;
    flag = 1;
    if (rank >= P) {                               // more workgroups on XCD 0 than an eighth
      dev_add(sync + kChainAbort, 1);
      flag = 0;
    }
    if (dev_load(sync + kChainAbort)) flag = 0;    // an aborted plan runs no more
    epoch_s = epoch;
    rank_s = (int)rank;
  }
  __syncthreads();
  if (!flag) return;
  const uint64_t epoch = epoch_s;
  const int rank = rank_s;
  uint64_t bar = epoch * 2 * (uint64_t)c.nlev;
  for (int lev = 0; lev < c.nlev; ++lev) {
    const ChainLevel L = cld(cp(c.levels) + lev);
    for (int i = rank; i < L.nv; i += (int)P) {
      const VItem it = cld(cp(L.a.vitems) + i);
      v_item<TM, true>(L.a, it, lds);
      vm_wait<0>();                                // this wave's partial sums are in the L2
      __syncthreads();
      if (tid == 0) {
        const MItem mi = cld(cp(L.a.mitems) + it.mid);
        const uint64_t need = (uint64_t)mi.ngroups * (uint64_t)mi.nsplit;
        const uint64_t old = dev_add(sync + kChainCnt + kChainCntStride * (L.moff + it.mid), 1);
        flag = old + 1 == (epoch + 1) * need;      // the last V item of its (entry, path)
      }
      __syncthreads();
      if (flag) mid_item<TM, true>(L.a, cld(cp(L.a.mitems) + it.mid), reinterpret_cast<float*>(lds));
      __syncthreads();                             // LDS is the next item's
    }
    if (!chain_barrier(sync, ++bar, P, lev == 0 ? (uint64_t)c.stall : 0, &flag)) return;
    for (int i = rank; i < L.nu; i += (int)P) {
      u_item<TM, false, true>(L.a, cld(cp(L.a.uitems) + i), lds);
      __syncthreads();
    }
    if (!chain_barrier(sync, ++bar, P, 0, &flag)) return;
  }
  if (rank == 0 && tid == 0) __hip_atomic_store(sync + kChainEpoch, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int TM>
constexpr size_t chain_lds() {
  constexpr size_t v = VShape<TM>::lds, u = UShape<TM>::lds, m = (size_t)kMidLdsFloats * 4;
  return v > u ? (v > m ? v : m) : (u > m ? u : m);
}

template <int TM>
int chain_grid_of(int device) {
  int coop = 0, cus = 0, per = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, device) != hipSuccess || !coop) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_decode_chain<TM>, kThreads, chain_lds<TM>()) != hipSuccess)
    return 0;
  const int grid = per * cus;
  return grid % kChainXcds == 0 ? grid : 0;        // an equal share per XCD
}

template <int TM>
hipError_t launch_chain(const ChainArgs& c, int grid, hipStream_t st) {
  ChainArgs arg = c;
  void* args[] = {&arg};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_decode_chain<TM>), dim3(grid), dim3(kThreads),
                                    args, (unsigned)chain_lds<TM>(), st);
}

}  // namespace

hipError_t launch_decode_v(const DecArgs& a, int nitems, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  switch (a.bucket) {
    case 1: hipLaunchKernelGGL(k_decode_v<1>, dim3(nitems), dim3(kThreads), VShape<1>::lds, st, a); break;
    case 2: hipLaunchKernelGGL(k_decode_v<2>, dim3(nitems), dim3(kThreads), VShape<2>::lds, st, a); break;
    case 4: hipLaunchKernelGGL(k_decode_v<4>, dim3(nitems), dim3(kThreads), VShape<4>::lds, st, a); break;
    case 8: hipLaunchKernelGGL(k_decode_v<8>, dim3(nitems), dim3(kThreads), VShape<8>::lds, st, a); break;
    default: hipLaunchKernelGGL(k_decode_v<16>, dim3(nitems), dim3(kThreads), VShape<16>::lds, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_decode_mid(const DecArgs& a, int nitems, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  switch (a.bucket) {
    case 1: hipLaunchKernelGGL(k_decode_mid<1>, dim3(nitems), dim3(mid_threads<1>()), 0, st, a); break;
    case 2: hipLaunchKernelGGL(k_decode_mid<2>, dim3(nitems), dim3(mid_threads<2>()), 0, st, a); break;
    case 4: hipLaunchKernelGGL(k_decode_mid<4>, dim3(nitems), dim3(mid_threads<4>()), 0, st, a); break;
    case 8: hipLaunchKernelGGL(k_decode_mid<8>, dim3(nitems), dim3(mid_threads<8>()), 0, st, a); break;
    default: hipLaunchKernelGGL(k_decode_mid<16>, dim3(nitems), dim3(mid_threads<16>()), 0, st, a); break;
  }
  return hipGetLastError();
}

template <bool YF>
static void launch_u(const DecArgs& a, int nitems, hipStream_t st) {
  switch (a.bucket) {
    case 1: hipLaunchKernelGGL((k_decode_u<1, YF>), dim3(nitems), dim3(kThreads), UShape<1>::lds, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_u<2, YF>), dim3(nitems), dim3(kThreads), UShape<2>::lds, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_u<4, YF>), dim3(nitems), dim3(kThreads), UShape<4>::lds, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_u<8, YF>), dim3(nitems), dim3(kThreads), UShape<8>::lds, st, a); break;
    default: hipLaunchKernelGGL((k_decode_u<16, YF>), dim3(nitems), dim3(kThreads), UShape<16>::lds, st, a); break;
  }
}

hipError_t launch_decode_u_wide(const DecArgs& a, int nitems, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  if (a.bucket != 16) return hipErrorInvalidValue;
  if (a.yf32) hipLaunchKernelGGL((k_decode_u_wide<16, true>), dim3(nitems), dim3(kThreads), UShape<16>::lds, st, a);
  else hipLaunchKernelGGL((k_decode_u_wide<16, false>), dim3(nitems), dim3(kThreads), UShape<16>::lds, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_u(const DecArgs& a, int nitems, hipStream_t st) {
  if (nitems <= 0) return hipSuccess;
  if (a.yf32) launch_u<true>(a, nitems, st);
  else launch_u<false>(a, nitems, st);
  return hipGetLastError();
}

}  // namespace lb

namespace lb {

static_assert(UShape<16>::NMAX == decode_u_fast_units(16) && UShape<8>::NMAX == decode_u_fast_units(8),
              "the planner's count of fast-form units");

bool decode_chain_takes(const DecEntry& e, int bucket) {
  return e.xdirect != 0 && e.ug.nu <= decode_u_fast_units(bucket);
}

int decode_chain_grid(int bucket, int device) {
  switch (bucket) {
    case 1: return chain_grid_of<1>(device);
    case 2: return chain_grid_of<2>(device);
    case 4: return chain_grid_of<4>(device);
    case 8: return chain_grid_of<8>(device);
    default: return chain_grid_of<16>(device);
  }
}

int decode_chain_participants(int grid) { return grid / kChainXcds; }

hipError_t launch_decode_chain(const ChainArgs& c, int bucket, int grid, hipStream_t st) {
  if (grid <= 0 || c.nlev <= 0) return hipErrorInvalidValue;
  switch (bucket) {
    case 1: return launch_chain<1>(c, grid, st);
    case 2: return launch_chain<2>(c, grid, st);
    case 4: return launch_chain<4>(c, grid, st);
    case 8: return launch_chain<8>(c, grid, st);
    default: return launch_chain<16>(c, grid, st);
  }
}

}  // namespace lb

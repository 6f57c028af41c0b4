// Host side of the C ABI declared in include/littlebit.h: validation, device
// memory ownership, layer build, regime dispatch, stacks and HIP graphs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "lb_internal.h"
#include "lb_prefill.h"
#include "littlebit_probe.h"

using namespace lb;

namespace {

thread_local std::string g_last_error;

lb_status fail(lb_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lb_status hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? LB_ERR_OUT_OF_MEMORY : LB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr)                                     \
  do {                                                    \
    hipError_t e_ = (expr);                               \
    if (e_ != hipSuccess) return hip_fail(e_, #expr);     \
  } while (0)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t words_per_row(int64_t r) { return r <= 0 ? 0 : (r + 31) / 32; }
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// One device allocation carved into 256-byte aligned pieces.
struct Arena {
  char* base = nullptr;
  size_t size = 0;
  size_t used = 0;
  void* take(size_t bytes) {
    void* p = base + used;
    used += align256(bytes);
    return p;
  }
};

// Device scratch that grows on demand (callers synchronise before reuse).
struct Scratch {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipError_t ensure(size_t want) {
    if (want <= bytes) return hipSuccess;
    if (ptr) {
      hipError_t e = hipFree(ptr);
      if (e != hipSuccess) return e;
      ptr = nullptr;
      bytes = 0;
    }
    hipError_t e = hipMalloc(&ptr, want);
    if (e == hipSuccess) bytes = want;
    return e;
  }
  void release() {
    if (ptr) (void)hipFree(ptr);
    ptr = nullptr;
    bytes = 0;
  }
};

}  // namespace

// ---------------------------------------------------------------------------
// objects
// ---------------------------------------------------------------------------

// Decode launch plan: entries and the three kernels' per-workgroup item lists
// for a given token count.  Owned by a linear (single forwards) or a stack.
struct DecodePlan {
  int T = -1;             // tokens per launch this plan was built for
  int count = 0;
  std::vector<DecEntry> entries_h;
  DecEntry* entries_d = nullptr;
  VItem* vitems_d = nullptr;      // V items, largest first
  MItem* mitems_d = nullptr;      // mid items, one per (entry, path)
  UItem* uitems_d = nullptr;      // U items, largest first; the last nuw of them for the wide U launch
  int nv = 0, nm = 0, nu = 0, nuw = 0;
  Scratch part;                   // V-stage partial slots
  Scratch work;                   // U-stage A operands and correction sums of every entry
  void release() {
    if (entries_d) (void)hipFree(entries_d);
    if (vitems_d) (void)hipFree(vitems_d);
    if (mitems_d) (void)hipFree(mitems_d);
    if (uitems_d) (void)hipFree(uitems_d);
    entries_d = nullptr;
    vitems_d = nullptr;
    mitems_d = nullptr;
    uitems_d = nullptr;
    part.release();
    work.release();
    T = -1;
    count = 0;
  }
};

struct lb_linear_s {
  int device = 0;
  int64_t m = 0, n = 0;
  int np = 0;
  int64_t r[2] = {0, 0};
  Arena arena;
  PathDev paths[2] = {};
  uint16_t* gdec[2] = {nullptr, nullptr};   // g zero-padded to whole 128-row chunks
  uint8_t* udec = nullptr;                  // decode U layout
  uint16_t* hq = nullptr;                   // decode row scales per quad
  UGeom ug = {};
  PrefillLayer pre = {};
  // single-forward state
  Scratch zexact;
  DecodePlan plan;
  PrefillPlan pplan;
  hipStream_t last_stream = nullptr;
  // no-allocation forward: the decode tables of this linear for every token
  // bucket, built at create against the fixed per-device scratch
  struct NoAllocDecode {
    bool ok = false;                 // the bucket's scratch fits kNoAllocScratchBytes
    int nv = 0, nm = 0, nu = 0, nuw = 0;
    size_t entries_off = 0, v_off = 0, m_off = 0, u_off = 0;   // bytes into na_tables
  };
  NoAllocDecode na[5];               // token buckets 1, 2, 4, 8, 16
  void* na_scratch = nullptr;        // this device's scratch array
  uint8_t* na_tables = nullptr;      // device copy of na_host
  std::vector<uint8_t> na_host;      // host image of the tables (source of the create-time copy)
};

// The decode layouts (V and U sign words) of every linear of a stack copied
// into one allocation, in stack order, so the decode kernels stream a single
// contiguous region instead of hundreds of per-linear arenas.
struct DecodeImage {
  Scratch buf;
  std::vector<const uint8_t*> udec;
  std::vector<const uint16_t*> hq;
  std::vector<std::array<const uint32_t*, 2>> vdec;
};

// Entries of a stack that run together: a level of mutually independent
// entries (all of them when no entry reads or writes another's output).
struct StackGroup {
  std::vector<int> idx;                     // entries of the stack, in order
  std::vector<lb_linear> lins;
  std::vector<const PrefillLayer*> pre;
  DecodeImage view;                         // the stack image's layouts of these entries (buf unused)
  DecodePlan plan;
  PrefillPlan pplan;
  const void** xs_d = nullptr;              // device copies of the entries' pointers
  void** ys_d = nullptr;
  std::vector<const void*> xs_h;
  std::vector<void*> ys_h;
  void release() {
    if (xs_d) (void)hipFree(xs_d);
    if (ys_d) (void)hipFree(ys_d);
    xs_d = nullptr;
    ys_d = nullptr;
    plan.release();
    prefill_plan_release(pplan);
  }
};

struct lb_stack_s {
  int device = 0;
  std::vector<lb_linear> linears;
  DecodeImage dimg;
  std::vector<StackGroup> groups;           // decode / prefill launch groups, run in order
  Scratch zexact;
  std::vector<const void*> xs_h;            // the caller's pointers of the current plans
  std::vector<void*> ys_h;
  // captured graph and what it was captured for
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipStream_t cap_stream = nullptr;
  int64_t g_tokens = -1;
  int g_io = -1, g_regime = -1;
  hipStream_t last_stream = nullptr;
  // AUTO's regime for the last (tokens, io) it was asked about
  int64_t auto_tokens = -1;
  int auto_io = -1;
  lb_regime auto_rg = LB_REGIME_DECODE;
  // persistent chained decode (lb_stack_set_persistent): all levels of a
  // chained decode in one cooperative launch of k_decode_chain
  int chain_enable = 0;                     // lb_stack_set_persistent's mode (0: level launches)
  int chain_active = 0;                     // the current plans run it
  int chain_grid = 0, chain_bucket = 0, chain_nlev = 0;
  int chain_stall = 0;                      // LITTLEBIT_CHAIN_STALL at planning (abort-path tests)
  ChainLevel* chain_levels_d = nullptr;     // per level: its decode tables and buffers
  std::vector<DecodePlan> chain_plans;      // per level, planned for the kernel's participants
  Scratch chain_sync;                       // epoch, abort flag, barrier and mid counters
  void chain_release() {
    if (chain_levels_d) (void)hipFree(chain_levels_d);
    chain_levels_d = nullptr;
    for (DecodePlan& P : chain_plans) P.release();
    chain_plans.clear();
    chain_active = 0;
    chain_grid = chain_bucket = chain_nlev = chain_stall = 0;
  }
};

namespace {

void linear_free(lb_linear L) {
  if (!L) return;
  if (L->arena.base) (void)hipFree(L->arena.base);
  if (L->na_tables) (void)hipFree(L->na_tables);
  L->zexact.release();
  L->plan.release();
  prefill_plan_release(L->pplan);
  delete L;
}

// ---------------------------------------------------------------------------
// decode plans
// ---------------------------------------------------------------------------

// Items sorted largest first (stable): the order the hardware dispatches them.
template <class Item>
std::vector<Item> largest_first(const std::vector<std::pair<double, Item>>& items) {
  std::vector<int> order(items.size());
  for (size_t i = 0; i < items.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return items[a].first > items[b].first; });
  std::vector<Item> out;
  for (int i : order) out.push_back(items[i].second);
  return out;
}

template <class Item>
hipError_t upload(Item** dst, const std::vector<Item>& v) {
  if (*dst) {
    hipError_t e = hipFree(*dst);
    if (e != hipSuccess) return e;
    *dst = nullptr;
  }
  hipError_t e = hipMalloc(dst, std::max<size_t>(v.size(), 1) * sizeof(Item));
  if (e == hipSuccess && !v.empty()) e = hipMemcpy(*dst, v.data(), v.size() * sizeof(Item), hipMemcpyHostToDevice);
  return e;
}

// Host side of a decode plan for `count` linears at `T` tokens per launch:
// the kernels' tables and the scratch they need.
//   V items: each path's column tiles in groups of at most decode_v_tiles, each
//     group's 128-row chunks cut into ranges of about decode_v_item_bytes of sign
//     words (at least 4 chunks, one per wave, where the path has them).
//   mid items: one per (entry, path).
//   U items: runs of 4 qw quads, qw quads per wave, about kDecodeUItemBytes.
// The entries' aimg / cval pointers are left null: they point into the work
// buffer, wherever the caller places it (img_off / cv_off bytes into it).
struct DecodeHostPlan {
  std::vector<DecEntry> entries;
  std::vector<VItem> vitems;        // largest first
  std::vector<MItem> mitems;
  std::vector<UItem> uitems;        // largest first, then the wide U launch's items largest first
  int nuw = 0;                      // items of the wide U launch (decode_u_wide), at the end
  std::vector<size_t> img_off, cv_off;
  size_t part_bytes = 0;            // V-stage partial slots
  size_t work_bytes = 0;            // U-stage operands and correction sums
};

void plan_decode_host(DecodeHostPlan& H, const lb_linear* L, int count, int T, const DecodeImage* img,
                      int item_slots = 0) {
  const int bucket = decode_bucket(T), tb = (bucket + 7) / 8, ct_max = decode_v_tiles(bucket);
  H.entries.assign(count, DecEntry{});
  H.img_off.assign(count, 0);
  H.cv_off.assign(count, 0);
  std::vector<std::pair<double, VItem>> vl;
  std::vector<std::pair<double, UItem>> ul, ulw;
  H.mitems.clear();
  size_t work_bytes = 0;
  int slots = 0;
  // Item sizes: about 192 KB of sign words per item when the launch has
  // plenty of work; a launch with less is cut into about one item per
  // workgroup slot of the GPU (CUs x workgroups per CU), so that it runs as
  // one wave of items and its latency is that of one item (8 KB at least:
  // against 16 KB, 2 % off the Llama-2-70B linears chained in model order).
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, L[0]->device) != hipSuccess || cus <= 0)
    cus = 256;
  const double slots_per_launch = item_slots > 0 ? (double)item_slots : (double)cus * (bucket >= 16 ? 2 : 3);
  double vtotal = 0, utotal = 0;
  for (int e = 0; e < count; ++e) {
    const int nkc = (int)((L[e]->n + kChunk - 1) / kChunk);
    for (int p = 0; p < L[e]->np; ++p) vtotal += (double)nkc * L[e]->paths[p].nct * 256.0;
    utotal += (double)L[e]->ug.nq * (L[e]->ug.qbytes + 256.0);
  }
  constexpr double kMinItemBytes = 8 * 1024;
  const double vtarget =
      std::min<double>(decode_v_item_bytes(bucket), std::max(kMinItemBytes, vtotal / slots_per_launch));
  const double utarget = std::min<double>(kDecodeUItemBytes, std::max(kMinItemBytes, utotal / slots_per_launch));
  for (int e = 0; e < count; ++e) {
    const lb_linear l = L[e];
    DecEntry& E = H.entries[e];
    E.m = (int)l->m;
    E.n = (int)l->n;
    E.np = l->np;
    E.nkc = (int)((l->n + kChunk - 1) / kChunk);
    E.xdirect = (l->n % 8) == 0;
    E.ug = l->ug;
    E.udec = img ? img->udec[e] : l->udec;
    E.hq = img ? img->hq[e] : l->hq;
    for (int p = 0; p < l->np; ++p) {
      E.p[p] = l->paths[p];
      if (img) E.p[p].vdec = img->vdec[e][p];
      E.gdec[p] = l->gdec[p];
      const int nct = l->paths[p].nct;
      const int groups = (nct + ct_max - 1) / ct_max;
      const int gt = (nct + groups - 1) / groups;
      const double chunk_bytes = gt * 256.0;
      const int max_split = std::max(1, E.nkc / kWavesPerGroup);
      const int nsplit = std::max(1, std::min(max_split, (int)std::lround(E.nkc * chunk_bytes / vtarget)));
      H.mitems.push_back(MItem{e, p, slots, groups, nsplit, gt, 0, 0});
      for (int g = 0; g < groups; ++g) {
        const int tile0 = g * gt, nt = std::min(gt, nct - tile0);
        for (int sp = 0; sp < nsplit; ++sp) {
          const int c0 = (int)((int64_t)E.nkc * sp / nsplit), c1 = (int)((int64_t)E.nkc * (sp + 1) / nsplit);
          // time of the item: its waves' 1 KB ring steps (x / g steps of each
          // group of chunks, then each chunk's sign steps), per wave
          const int ch = c1 - c0, grp = bucket == 1 ? (ch + 1) / 2 : ch;
          const double cost = ((double)grp * ((bucket + 4) / 4) + (double)ch * ((nt + 3) / 4)) / kWavesPerGroup;
          vl.push_back({cost, VItem{e, p, tile0, nt, c0, c1, slots + g * nsplit + sp, (int)H.mitems.size() - 1}});
        }
      }
      slots += groups * nsplit;
    }
    H.img_off[e] = work_bytes;
    work_bytes += align256((size_t)E.ug.nu * tb * kABytes);
    H.cv_off[e] = work_bytes;
    work_bytes += align256(2 * 16 * sizeof(float));
    const double qbytes = E.ug.qbytes + 256.0;
    const int qw = std::max(1, std::min(decode_u_qw_max(bucket),
                                        (int)std::lround(utarget / (kWavesPerGroup * qbytes))));
    for (int q0 = 0; q0 < E.ug.nq; q0 += kWavesPerGroup * qw) {
      const int nq = std::min(kWavesPerGroup * qw, E.ug.nq - q0);
      // a short run (small entries, the last run) is spread over all four waves
      (decode_u_wide(bucket, E.ug.nu) ? ulw : ul)
          .push_back({nq * qbytes, UItem{e, q0, nq, (nq + kWavesPerGroup - 1) / kWavesPerGroup}});
    }
  }
  H.work_bytes = work_bytes + kDmaPad;
  H.part_bytes = std::max<size_t>((size_t)slots * decode_slot_floats(bucket) * sizeof(float), 256);
  H.vitems = largest_first(vl);
  H.uitems = largest_first(ul);
  const std::vector<UItem> wide = largest_first(ulw);
  H.uitems.insert(H.uitems.end(), wide.begin(), wide.end());
  H.nuw = (int)wide.size();
}

// Builds (or reuses) the decode plan for `count` linears at `T` tokens per
// launch: the host plan, its scratch buffers and its tables on the device.
// slots: work-item slots the launch has (0: every workgroup slot of the GPU).
lb_status build_decode_plan(DecodePlan& P, const lb_linear* L, int count, int T, const DecodeImage* img = nullptr,
                            int slots = 0) {
  if (P.T == T && P.count == count) return LB_OK;
  // the buffers and tables below are freed and reallocated: until every step
  // has succeeded the plan must not look valid for any token count
  P.T = -1;
  P.count = 0;
  DecodeHostPlan H;
  plan_decode_host(H, L, count, T, img, slots);
  HIP_TRY(P.work.ensure(H.work_bytes));
  HIP_TRY(P.part.ensure(H.part_bytes));
  for (int e = 0; e < count; ++e) {
    H.entries[e].aimg = reinterpret_cast<uint8_t*>(P.work.ptr) + H.img_off[e];
    H.entries[e].cval = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(P.work.ptr) + H.cv_off[e]);
  }
  P.entries_h = H.entries;
  HIP_TRY(upload(&P.entries_d, P.entries_h));
  HIP_TRY(upload(&P.vitems_d, H.vitems));
  HIP_TRY(upload(&P.mitems_d, H.mitems));
  HIP_TRY(upload(&P.uitems_d, H.uitems));
  P.nv = (int)H.vitems.size();
  P.nm = (int)H.mitems.size();
  P.nu = (int)H.uitems.size();
  P.nuw = H.nuw;
  P.T = T;
  P.count = count;
  return LB_OK;
}

// Device tables of one decode plan and its partial-slot buffer.
struct DecodeTables {
  const DecEntry* entries;
  const VItem* vitems;
  const MItem* mitems;
  const UItem* uitems;
  int nv, nm, nu, nuw;     // nuw: the last U items, for the wide U launch
  float* part;
};

// Launches the three decode kernels over token slices of at most
// kDecodeMaxTokens, on tables built for Tplan = min(kDecodeMaxTokens, tokens)
// tokens (a shorter last slice runs the same kernels on fewer tokens).
hipError_t launch_decode_slices(const DecodeTables& D, const void* const* xs_d, void* const* ys_d, const void* x0,
                                void* y0, int64_t tokens, int yf32, hipStream_t st) {
  const int Tplan = (int)std::min<int64_t>(kDecodeMaxTokens, tokens);
  for (int64_t t0 = 0; t0 < tokens; t0 += kDecodeMaxTokens) {
    DecArgs a{};
    a.entries = D.entries;
    a.xs = xs_d;
    a.ys = ys_d;
    a.x0 = x0;
    a.y0 = y0;
    a.T = (int)std::min<int64_t>(kDecodeMaxTokens, tokens - t0);
    a.t0 = (int)t0;
    a.bucket = decode_bucket(Tplan);
    a.yf32 = yf32;
    a.vitems = D.vitems;
    a.mitems = D.mitems;
    a.uitems = D.uitems;
    a.part = D.part;
    hipError_t e = launch_decode_v(a, D.nv, st);
    if (e == hipSuccess) e = launch_decode_mid(a, D.nm, st);
    if (e == hipSuccess) e = launch_decode_u(a, D.nu - D.nuw, st);
    if (e == hipSuccess && D.nuw > 0) {
      a.uitems = D.uitems + (D.nu - D.nuw);
      e = launch_decode_u_wide(a, D.nuw, st);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Launches the three decode kernels over token slices of at most
// kDecodeMaxTokens.  Every slice of one forward runs on one plan, built for
// the first slice's token count (a shorter last slice runs the same kernels
// on fewer tokens), so a ragged token count never rebuilds the plan.
lb_status run_decode(DecodePlan& P, const lb_linear* L, int count, const void* const* xs_d, void* const* ys_d,
                     const void* x0, void* y0, int64_t tokens, int yf32, hipStream_t st,
                     const DecodeImage* img = nullptr) {
  const int Tplan = (int)std::min<int64_t>(kDecodeMaxTokens, tokens);
  if (P.T != Tplan && P.T != -1) HIP_TRY(hipStreamSynchronize(st));  // the plan is rewritten below
  lb_status s = build_decode_plan(P, L, count, Tplan, img);
  if (s != LB_OK) return s;
  const DecodeTables D{P.entries_d, P.vitems_d, P.mitems_d, P.uitems_d, P.nv, P.nm, P.nu, P.nuw,
                       reinterpret_cast<float*>(P.part.ptr)};
  HIP_TRY(launch_decode_slices(D, xs_d, ys_d, x0, y0, tokens, yf32, st));
  return LB_OK;
}

// index of a token bucket (1, 2, 4, 8, 16) in lb_linear_s::na
inline int bucket_index(int bucket) { return bucket <= 1 ? 0 : bucket <= 2 ? 1 : bucket <= 4 ? 2 : bucket <= 8 ? 3 : 4; }

// The no-allocation forward's tables of a linear (see lb_linear_s::na): for
// every token bucket, the single-linear decode plan that lb_linear_forward_ex
// builds (so both run the same work items), its work buffer placed after the
// partial slots in this device's scratch array; a bucket whose scratch would
// not fit is marked unavailable.  One device allocation and one copy, on
// `st`, from a host image the linear keeps.
hipError_t build_noalloc_tables(lb_linear L, hipStream_t st) {
  hipError_t e = noalloc_scratch(L->device, &L->na_scratch);
  if (e != hipSuccess) return e;
  std::vector<uint8_t>& img = L->na_host;
  img.clear();
  auto put = [&](const void* src, size_t bytes) {
    const size_t off = align256(img.size());
    img.resize(off + std::max<size_t>(bytes, 1));
    if (bytes) std::memcpy(img.data() + off, src, bytes);
    return off;
  };
  static constexpr int kBuckets[5] = {1, 2, 4, 8, 16};
  for (int b = 0; b < 5; ++b) {
    DecodeHostPlan H;
    lb_linear one[1] = {L};
    plan_decode_host(H, one, 1, kBuckets[b], nullptr);
    const size_t work_off = align256(H.part_bytes);
    lb_linear_s::NoAllocDecode& N = L->na[b];
    N.ok = work_off + H.work_bytes <= kNoAllocScratchBytes;
    if (!N.ok) continue;
    uint8_t* work = reinterpret_cast<uint8_t*>(L->na_scratch) + work_off;
    H.entries[0].aimg = work + H.img_off[0];
    H.entries[0].cval = reinterpret_cast<float*>(work + H.cv_off[0]);
    N.entries_off = put(H.entries.data(), sizeof(DecEntry));
    N.v_off = put(H.vitems.data(), H.vitems.size() * sizeof(VItem));
    N.m_off = put(H.mitems.data(), H.mitems.size() * sizeof(MItem));
    N.u_off = put(H.uitems.data(), H.uitems.size() * sizeof(UItem));
    N.nv = (int)H.vitems.size();
    N.nm = (int)H.mitems.size();
    N.nu = (int)H.uitems.size();
    N.nuw = H.nuw;
  }
  if (img.empty()) return hipSuccess;
  img.resize(align256(img.size()));
  e = hipMalloc(&L->na_tables, img.size());
  if (e == hipSuccess) e = hipMemcpyAsync(L->na_tables, img.data(), img.size(), hipMemcpyHostToDevice, st);
  return e;
}

// The integer a caller passed for an enum parameter.  A C caller may pass any
// int; in C++ reading an enum object that holds a value outside its
// enumerators' range is undefined, so the ABI reads the bytes and checks them
// before any value is used as the enum.
template <class E>
inline int enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enums of the ABI are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

lb_status check_io(int64_t tokens, const lb_dtype& io_arg, const lb_regime& regime_arg) {
  if (tokens <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "tokens must be positive (got %lld)", (long long)tokens);
  if (tokens > LB_MAX_TOKENS) return fail(LB_ERR_UNSUPPORTED, "tokens %lld exceeds %d", (long long)tokens, LB_MAX_TOKENS);
  const int io = enum_bits(io_arg), regime = enum_bits(regime_arg);
  if (io != LB_BF16 && io != LB_FP32 && io != LB_BF16_FP32)
    return fail(LB_ERR_INVALID_ARGUMENT, "io must be LB_BF16, LB_FP32 or LB_BF16_FP32 (got %d)", io);
  if (regime < LB_REGIME_AUTO || regime > LB_REGIME_PREFILL)
    return fail(LB_ERR_INVALID_ARGUMENT, "unknown regime %d", regime);
  if (io == LB_FP32 && (regime == LB_REGIME_DECODE || regime == LB_REGIME_PREFILL))
    return fail(LB_ERR_UNSUPPORTED, "the decode and prefill kernels read bf16 x; fp32 x runs the exact kernels");
  return LB_OK;
}

// element types of x and y
inline int x_is_fp32(lb_dtype io) { return io == LB_FP32 ? 1 : 0; }
inline int y_is_fp32(lb_dtype io) { return io == LB_BF16 ? 0 : 1; }

// Estimated time (µs) of the decode kernels on `count` linears at T tokens.
// Per launch sequence of up to 16 tokens: the V stage's and the U stage's
// sign bytes at rates measured on whole Llama-shaped stacks at 16 tokens on
// MI355X (V 0.72 µs/MB; U 0.34 µs/MB where a quad's 128-latent units fit the
// U kernel's registers, 0.62 µs/MB where they do not; sequences of 8 tokens
// or fewer 0.6 of that), at least 6 µs (one work item's latency), plus 12 µs
// for the three launches.
double decode_cost_us(const lb_linear* L, int count, int64_t T) {
  const int bucket = decode_bucket((int)std::min<int64_t>(T, kDecodeMaxTokens));
  const int nmax = decode_u_fast_units(bucket);   // units a U wave keeps in registers
  double us = 0;
  for (int e = 0; e < count; ++e) {
    double vb = 0, ub = 0;
    for (int p = 0; p < L[e]->np; ++p) {
      vb += (double)L[e]->n * L[e]->r[p] / 8;
      ub += (double)L[e]->m * L[e]->r[p] / 8;
    }
    us += vb * 0.72e-6 + ub * (L[e]->ug.nu <= nmax ? 0.34e-6 : 0.62e-6);
  }
  const int64_t launches = (T + kDecodeMaxTokens - 1) / kDecodeMaxTokens;
  return (double)launches * (std::max(us * (bucket <= 8 ? 0.6 : 1.0), 6.0) + 12.0);
}

// Estimated time (µs) of the prefill GEMMs on `count` linears at T tokens:
// the larger of the throughput estimate and the longest single tile (0.5 µs
// per K block of both GEMMs), plus 8 µs for the launches.  Throughput, fitted
// to the benchmark stacks (Llama-2-70B, Llama-2-13B, Llama-3-8B) at 8 to 256
// tokens: a whole 64-row stripe costs 1.54 ns per (256-column tile, 64-deep K
// block), 7.4 ns per tile and 57 µs; one with at most 32 tokens 0.72 of the
// K-block term; a 128-row stripe 1.36 + 0.125 whole 64-row stripes per 32-row
// block it computes, a 256-row stripe 1.6 + 0.3 per block.
double prefill_cost_us(const lb_linear* L, int count, int64_t T) {
  double tk = 0, tn = 0, longest = 0, blocks1 = 0;
  const int bm = prefill_rows_per_tile((int)T), mts = (int)((T + bm - 1) / bm);
  for (int e = 0; e < count; ++e)
    blocks1 += (double)mts * ((L[e]->pre.Rp + kPreBN - 1) / kPreBN) * L[e]->pre.kb1;
  bool cut = false;
  for (int e = 0; e < count; ++e) {
    const PrefillLayer& P = L[e]->pre;
    const double t1 = (P.Rp + kPreBN - 1) / kPreBN, t2 = (P.m + kPreBN - 1) / kPreBN;
    tk += t1 * P.kb1 + t2 * P.kb2;
    tn += t1 + t2;
    const int nks = prefill_k_parts(P.kb1, (int)T, blocks1);   // GEMM1 K parts (the longest tile's blocks)
    cut = cut || nks > 1;
    longest = std::max(longest, 0.5 * ((P.kb1 + nks - 1) / nks + P.kb2));
  }
  const double whole = tk * 1.54e-3 + tn * 7.4e-3 + 57.0, small = tk * 1.54e-3 * 0.72 + tn * 7.4e-3 + 57.0;
  double us = cut ? 6.0 : 0.0;                         // the launch adding the K parts
  for (int64_t m0 = 0; m0 < T; m0 += bm) {
    const int live = (int)std::min<int64_t>(bm, T - m0);
    // blocks computed: all of the tile unless the stripe skips empty ones
    const int blocks = live <= bm - 32 ? (live + 31) / 32 : bm / 32;
    if (bm == 64) us += live <= 32 ? small : whole;
    else if (bm == 128) us += whole * (1.36 + 0.125 * blocks);
    else us += whole * (1.6 + 0.3 * blocks);
  }
  return std::max(us, longest) + 8.0;
}

// AUTO: fp32 x runs the exact path; bf16 x runs whichever of the decode and
// prefill kernels the two estimates above make faster for these linears.
lb_regime pick_regime(const lb_linear* L, int count, int64_t tokens, lb_dtype io, lb_regime regime) {
  if (regime != LB_REGIME_AUTO) return regime;
  if (io == LB_FP32) return LB_REGIME_EXACT;
  if (tokens > 4 * kPreSmallMaxTokens) return LB_REGIME_PREFILL;
  return decode_cost_us(L, count, tokens) <= prefill_cost_us(L, count, tokens) ? LB_REGIME_DECODE : LB_REGIME_PREFILL;
}

int current_device() {
  int d = 0;
  (void)hipGetDevice(&d);
  return d;
}

}  // namespace

// ---------------------------------------------------------------------------
// ABI
// ---------------------------------------------------------------------------
extern "C" {

const char* lb_status_string(lb_status s_arg) {
  switch (enum_bits(s_arg)) {
    case LB_OK: return "ok";
    case LB_ERR_INVALID_ARGUMENT: return "invalid argument";
    case LB_ERR_INVALID_SIGN: return "sign value outside {-1, +1}";
    case LB_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case LB_ERR_UNSUPPORTED: return "unsupported size";
    case LB_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LB_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* lb_last_error(void) { return g_last_error.c_str(); }

int64_t lb_packed_words_per_row(int64_t rank) { return words_per_row(rank); }

int64_t lb_rank_for_bpw(int64_t d_out, int64_t d_in, int64_t bpw_num, int64_t bpw_den) {
  if (d_out <= 0 || d_in <= 0 || bpw_num <= 0 || bpw_den <= 0) return -1;
  // round(num * m * n / (2 den (m + n))), ties up: floor((2 A + B) / (2 B))
  const __int128 A = (__int128)bpw_num * d_out * d_in;
  const __int128 B = (__int128)2 * bpw_den * (d_out + d_in);
  return (int64_t)((2 * A + B) / (2 * B));
}

lb_status lb_pack_signs_host(const int8_t* signs, int64_t rows, int64_t rank, uint32_t* packed) {
  if (!signs || !packed) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer");
  if (rows <= 0 || rank <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "rows and rank must be positive");
  const int64_t W = words_per_row(rank);
  for (int64_t i = 0; i < rows * rank; ++i)
    if (signs[i] != 1 && signs[i] != -1)
      return fail(LB_ERR_INVALID_SIGN, "value %d at row %lld, column %lld", (int)signs[i], (long long)(i / rank),
                  (long long)(i % rank));
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t w = 0; w < W; ++w) {
      uint32_t word = 0;
      for (int b = 0; b < 32; ++b) {
        const int64_t j = 32 * w + b;
        if (j < rank && signs[i * rank + j] == -1) word |= 1u << b;
      }
      packed[i * W + w] = word;
    }
  return LB_OK;
}

lb_status lb_pack_signs(const int8_t* signs, int64_t rows, int64_t rank, uint32_t* packed, void* stream) {
  if (!signs || !packed) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer");
  if (rows <= 0 || rank <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "rows and rank must be positive");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int* flag = nullptr;
  HIP_TRY(hipMalloc(&flag, sizeof(int)));
  int bad = 0;
  hipError_t e = hipMemsetAsync(flag, 0, sizeof(int), st);
  if (e == hipSuccess) e = launch_validate_signs(signs, rows * rank, flag, st);
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess && !bad) e = launch_pack_signs(signs, rows, rank, packed, st);
  (void)hipFree(flag);
  if (e != hipSuccess) return hip_fail(e, "lb_pack_signs");
  if (bad) return fail(LB_ERR_INVALID_SIGN, "a sign value is not -1 or +1");
  return LB_OK;
}

lb_status lb_init_dual_svid(const float* W, int64_t d_out, int64_t d_in, const lb_path_init* paths, int32_t n_paths,
                            void* stream) {
  if (!W || !paths) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer");
  if (n_paths != 1 && n_paths != 2) return fail(LB_ERR_INVALID_ARGUMENT, "n_paths must be 1 or 2 (got %d)", n_paths);
  if (d_out <= 0 || d_in <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "d_out and d_in must be positive");
  if (d_out > LB_MAX_DIM || d_in > LB_MAX_DIM) return fail(LB_ERR_UNSUPPORTED, "dimension exceeds %d", LB_MAX_DIM);
  int64_t ranks[2] = {0, 0};
  InitPathOut out[2] = {};
  for (int p = 0; p < n_paths; ++p) {
    const lb_path_init& P = paths[p];
    if (P.rank < 1 || P.rank > std::min<int64_t>(std::min(d_out, d_in), LB_MAX_RANK))
      return fail(LB_ERR_INVALID_ARGUMENT, "path %d: rank must be in 1..min(d_out, d_in, %d)", p, LB_MAX_RANK);
    if (!P.u_packed || !P.v_packed || !P.h || !P.g || !P.l)
      return fail(LB_ERR_INVALID_ARGUMENT, "path %d: null output pointer", p);
    ranks[p] = P.rank;
    out[p] = InitPathOut{P.u_packed, P.v_packed, P.h, P.g, P.l};
  }
  int rocstatus = 0;
  const hipError_t e = dual_svid_init(W, d_out, d_in, ranks, n_paths, out, reinterpret_cast<hipStream_t>(stream),
                                      &rocstatus);
  if (e != hipSuccess) {
    if (rocstatus) return fail(LB_ERR_HIP, "lb_init_dual_svid: rocBLAS/rocSOLVER status %d", rocstatus);
    return hip_fail(e, "lb_init_dual_svid");
  }
  return LB_OK;
}

lb_status lb_probe_stream_read(const void* buf, int64_t bytes, void* stream) {
  if (!buf) return fail(LB_ERR_INVALID_ARGUMENT, "null buffer");
  if (bytes <= 0 || bytes % 16) return fail(LB_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16");
  if (!aligned16(buf)) return fail(LB_ERR_ALIGNMENT, "buffer not 16-byte aligned");
  HIP_TRY(launch_probe_stream_read(buf, bytes, reinterpret_cast<hipStream_t>(stream)));
  return LB_OK;
}

lb_status lb_unpack_signs(const uint32_t* packed, int64_t rows, int64_t rank, int8_t* signs, void* stream) {
  if (!signs || !packed) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer");
  if (rows <= 0 || rank <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "rows and rank must be positive");
  HIP_TRY(launch_unpack_signs(packed, rows, rank, signs, reinterpret_cast<hipStream_t>(stream)));
  return LB_OK;
}

lb_status lb_linear_create(int64_t d_out, int64_t d_in, const lb_path* paths, int32_t n_paths, void* stream,
                           lb_linear* out) {
  if (!out) return fail(LB_ERR_INVALID_ARGUMENT, "out is null");
  if (!paths) return fail(LB_ERR_INVALID_ARGUMENT, "paths is null");
  if (n_paths != 1 && n_paths != 2) return fail(LB_ERR_INVALID_ARGUMENT, "n_paths must be 1 or 2 (got %d)", n_paths);
  if (d_out <= 0 || d_in <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "d_out and d_in must be positive");
  if (d_out > LB_MAX_DIM || d_in > LB_MAX_DIM) return fail(LB_ERR_UNSUPPORTED, "dimension exceeds %d", LB_MAX_DIM);
  for (int p = 0; p < n_paths; ++p) {
    const lb_path& P = paths[p];
    if (P.rank <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "path %d: rank must be positive", p);
    if (P.rank > LB_MAX_RANK) return fail(LB_ERR_UNSUPPORTED, "path %d: rank exceeds %d", p, LB_MAX_RANK);
    if (!P.u_packed || !P.v_packed || !P.h || !P.g || !P.l)
      return fail(LB_ERR_INVALID_ARGUMENT, "path %d: null pointer", p);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  lb_linear L = new (std::nothrow) lb_linear_s();
  if (!L) return fail(LB_ERR_OUT_OF_MEMORY, "host allocation failed");
  L->device = current_device();
  L->m = d_out;
  L->n = d_in;
  L->np = n_paths;
  // sizes of every piece
  const int nkc = (int)((d_in + kChunk - 1) / kChunk);
  size_t total = 0;
  size_t pre_bytes = prefill_layer_bytes(d_out, d_in, paths, n_paths);
  for (int p = 0; p < n_paths; ++p) {
    const int64_t r = paths[p].rank, W = words_per_row(r), nct = (r + kTile - 1) / kTile;
    L->r[p] = r;
    total += align256(d_out * W * 4) + align256(d_in * W * 4);                  // canonical
    total += align256((d_out + d_in + r) * 2);                                   // fp16 scales
    total += align256((size_t)nkc * nct * 64 * 4 + kDmaPad);                    // decode V
    total += align256((size_t)nkc * kChunk * 2);                                 // decode g
  }
  L->ug = u_geom(d_out, L->r, n_paths);
  total += align256(decode_u_bytes(L->ug)) + align256(decode_h_bytes(L->ug));   // decode U, row scales
  total += pre_bytes;
  hipError_t e = hipMalloc(&L->arena.base, total);
  if (e != hipSuccess) {
    delete L;
    return hip_fail(e, "hipMalloc(layer)");
  }
  L->arena.size = total;
  auto bail = [&](hipError_t err, const char* what) {
    linear_free(L);
    return hip_fail(err, what);
  };
  L->udec = reinterpret_cast<uint8_t*>(L->arena.take(decode_u_bytes(L->ug)));
  L->hq = reinterpret_cast<uint16_t*>(L->arena.take(decode_h_bytes(L->ug)));
  // the DMA slack after both is never used by a result, but keep it defined
  if ((e = hipMemsetAsync(L->udec, 0, decode_u_bytes(L->ug), st)) != hipSuccess) return bail(e, "clear U");
  if ((e = hipMemsetAsync(L->hq, 0, decode_h_bytes(L->ug), st)) != hipSuccess) return bail(e, "clear h");
  for (int p = 0; p < n_paths; ++p) {
    const lb_path& S = paths[p];
    const int64_t r = S.rank, W = words_per_row(r);
    PathDev& D = L->paths[p];
    D.r = (int)r;
    D.W = (int)W;
    D.nct = (int)((r + kTile - 1) / kTile);
    uint32_t* ucan = reinterpret_cast<uint32_t*>(L->arena.take(d_out * W * 4));
    uint32_t* vcan = reinterpret_cast<uint32_t*>(L->arena.take(d_in * W * 4));
    uint16_t* sc = reinterpret_cast<uint16_t*>(L->arena.take((d_out + d_in + r) * 2));
    uint32_t* vdec = reinterpret_cast<uint32_t*>(L->arena.take((size_t)nkc * D.nct * 64 * 4 + kDmaPad));
    L->gdec[p] = reinterpret_cast<uint16_t*>(L->arena.take((size_t)nkc * kChunk * 2));
    D.u_can = ucan;
    D.v_can = vcan;
    D.h = sc;
    D.g = sc + d_out;
    D.l = sc + d_out + d_in;
    D.vdec = vdec;
    if ((e = hipMemcpyAsync(ucan, S.u_packed, d_out * W * 4, hipMemcpyDefault, st)) != hipSuccess) return bail(e, "copy U");
    if ((e = hipMemcpyAsync(vcan, S.v_packed, d_in * W * 4, hipMemcpyDefault, st)) != hipSuccess) return bail(e, "copy V");
    if ((e = hipMemcpyAsync(sc, S.h, d_out * 2, hipMemcpyDefault, st)) != hipSuccess) return bail(e, "copy h");
    if ((e = hipMemcpyAsync(sc + d_out, S.g, d_in * 2, hipMemcpyDefault, st)) != hipSuccess) return bail(e, "copy g");
    if ((e = hipMemcpyAsync(sc + d_out + d_in, S.l, r * 2, hipMemcpyDefault, st)) != hipSuccess) return bail(e, "copy l");
    if ((e = launch_retile_v_decode(vcan, (int)d_in, (int)r, vdec, st)) != hipSuccess) return bail(e, "retile V");
    if ((e = hipMemsetAsync(L->gdec[p], 0, (size_t)nkc * kChunk * 2, st)) != hipSuccess) return bail(e, "clear g");
    if ((e = hipMemcpyAsync(L->gdec[p], D.g, d_in * 2, hipMemcpyDeviceToDevice, st)) != hipSuccess)
      return bail(e, "copy g");
  }
  {
    const int W[2] = {L->paths[0].W, n_paths > 1 ? L->paths[1].W : 0};
    if ((e = launch_decode_u_layout(L->paths[0].u_can, n_paths > 1 ? L->paths[1].u_can : nullptr, (int)d_out, W, L->ug,
                                    L->udec, st)) != hipSuccess)
      return bail(e, "retile U");
    if ((e = launch_decode_h_layout(L->paths[0].h, n_paths > 1 ? L->paths[1].h : nullptr, (int)d_out, L->ug.nq, L->hq,
                                    st)) != hipSuccess)
      return bail(e, "row scales");
  }
  if ((e = prefill_layer_build(L->pre, L->arena.take(pre_bytes), pre_bytes, d_out, d_in, L->paths, n_paths, st)) !=
      hipSuccess)
    return bail(e, "prefill layout");
  if ((e = build_noalloc_tables(L, st)) != hipSuccess) return bail(e, "no-allocation forward tables");
  *out = L;
  return LB_OK;
}

lb_status lb_auto_regime(const lb_linear* linears, int32_t count, int64_t tokens, lb_dtype io, lb_regime* out) {
  if (!linears || !out) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer");
  if (count < 1) return fail(LB_ERR_INVALID_ARGUMENT, "count must be positive");
  for (int i = 0; i < count; ++i)
    if (!linears[i]) return fail(LB_ERR_INVALID_ARGUMENT, "linear %d is null", i);
  lb_status s = check_io(tokens, io, LB_REGIME_AUTO);
  if (s != LB_OK) return s;
  *out = pick_regime(linears, count, tokens, io, LB_REGIME_AUTO);
  return LB_OK;
}

lb_status lb_linear_info(lb_linear L, int64_t* d_out, int64_t* d_in, int32_t* n_paths, int64_t* ranks,
                         int64_t* device_bytes) {
  if (!L) return fail(LB_ERR_INVALID_ARGUMENT, "null linear");
  if (d_out) *d_out = L->m;
  if (d_in) *d_in = L->n;
  if (n_paths) *n_paths = L->np;
  if (ranks)
    for (int p = 0; p < L->np; ++p) ranks[p] = L->r[p];
  if (device_bytes) *device_bytes = (int64_t)L->arena.size;
  return LB_OK;
}

lb_status lb_linear_forward_ex(lb_linear L, const void* x, void* y, int64_t tokens, lb_dtype io, lb_regime regime,
                               void* stream) {
  if (!L) return fail(LB_ERR_INVALID_ARGUMENT, "null linear");
  if (!x || !y) return fail(LB_ERR_INVALID_ARGUMENT, "null x or y");
  lb_status s = check_io(tokens, io, regime);
  if (s != LB_OK) return s;
  if (!aligned16(x) || !aligned16(y)) return fail(LB_ERR_ALIGNMENT, "x and y must be 16-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const lb_regime rg = pick_regime(&L, 1, tokens, io, regime);
  // scratch and plans are rebuilt on the host: order them after the previous call's work
  if (L->last_stream != st && L->last_stream) HIP_TRY(hipStreamSynchronize(L->last_stream));
  L->last_stream = st;
  if (rg == LB_REGIME_EXACT) {
    const size_t want =
        std::max<size_t>(exact_scratch_floats(L->paths, L->np, tokens, (int)L->n, x_is_fp32(io), y_is_fp32(io)), 64) *
        sizeof(float);
    if (want > L->zexact.bytes) {
      HIP_TRY(hipStreamSynchronize(st));
      HIP_TRY(L->zexact.ensure(want));
    }
    HIP_TRY(launch_exact(L->paths, L->np, (int)L->m, (int)L->n, x, y, (int)tokens, x_is_fp32(io), y_is_fp32(io),
                         reinterpret_cast<float*>(L->zexact.ptr), st));
    return LB_OK;
  }
  if (rg == LB_REGIME_DECODE) {
    const int T = (int)std::min<int64_t>(tokens, kDecodeMaxTokens);
    if (L->plan.T != T) HIP_TRY(hipStreamSynchronize(st));
    lb_linear one[1] = {L};
    return run_decode(L->plan, one, 1, nullptr, nullptr, x, y, tokens, y_is_fp32(io), st);
  }
  if (!prefill_available()) return fail(LB_ERR_UNSUPPORTED, "the prefill kernels are not available in this library");
  const PrefillLayer* one[1] = {&L->pre};
  const void* xs[1] = {x};
  void* ys[1] = {y};
  HIP_TRY(prefill_run(L->pplan, one, 1, xs, ys, (int)tokens, y_is_fp32(io), st, /*single=*/true));
  return LB_OK;
}

lb_status lb_linear_forward(lb_linear L, const void* x, void* y, int64_t tokens, lb_dtype io, void* stream) {
  return lb_linear_forward_ex(L, x, y, tokens, io, LB_REGIME_AUTO, stream);
}

lb_status lb_linear_forward_noalloc(lb_linear L, const void* x, void* y, int64_t tokens, lb_dtype io, void* stream) {
  if (!L) return fail(LB_ERR_INVALID_ARGUMENT, "null linear");
  if (!x || !y) return fail(LB_ERR_INVALID_ARGUMENT, "null x or y");
  lb_status s = check_io(tokens, io, LB_REGIME_AUTO);
  if (s != LB_OK) return s;
  if (!aligned16(x) || !aligned16(y)) return fail(LB_ERR_ALIGNMENT, "x and y must be 16-byte aligned");
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != L->device)
    return fail(LB_ERR_INVALID_ARGUMENT, "the linear lives on device %d but device %d is current", L->device, dev);
  if (!L->na_scratch || !L->na_tables) return fail(LB_ERR_UNSUPPORTED, "no scratch was set up for this linear");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (io == LB_FP32) {
    const size_t need = exact_scratch_floats(L->paths, L->np, tokens, (int)L->n, 1, 1) * sizeof(float);
    if (need > kNoAllocScratchBytes)
      return fail(LB_ERR_UNSUPPORTED, "%lld fp32 tokens need %zu bytes of scratch; the no-allocation forward has %zu",
                  (long long)tokens, need, kNoAllocScratchBytes);
    HIP_TRY(launch_exact(L->paths, L->np, (int)L->m, (int)L->n, x, y, (int)tokens, 1, 1,
                         reinterpret_cast<float*>(L->na_scratch), st));
    return LB_OK;
  }
  const int Tplan = (int)std::min<int64_t>(kDecodeMaxTokens, tokens);
  const lb_linear_s::NoAllocDecode& N = L->na[bucket_index(decode_bucket(Tplan))];
  if (!N.ok)
    return fail(LB_ERR_UNSUPPORTED, "the decode scratch of this %lld x %lld linear exceeds the %zu bytes of the "
                "no-allocation forward", (long long)L->m, (long long)L->n, kNoAllocScratchBytes);
  const DecodeTables D{reinterpret_cast<const DecEntry*>(L->na_tables + N.entries_off),
                       reinterpret_cast<const VItem*>(L->na_tables + N.v_off),
                       reinterpret_cast<const MItem*>(L->na_tables + N.m_off),
                       reinterpret_cast<const UItem*>(L->na_tables + N.u_off), N.nv, N.nm, N.nu, N.nuw,
                       reinterpret_cast<float*>(L->na_scratch)};
  HIP_TRY(launch_decode_slices(D, nullptr, nullptr, x, y, tokens, y_is_fp32(io), st));
  return LB_OK;
}

lb_status lb_linear_destroy(lb_linear L) {
  linear_free(L);
  return LB_OK;
}

}  // extern "C"

namespace {

// Copies the decode layouts of the stack's linears into one allocation (see
// DecodeImage); the linears' own copies stay in place for single forwards.
hipError_t build_decode_image(DecodeImage& D, const std::vector<lb_linear>& lins) {
  size_t total = 0;
  std::vector<size_t> off;
  for (lb_linear L : lins) {
    const int nkc = (int)((L->n + kChunk - 1) / kChunk);
    for (int p = 0; p < L->np; ++p) {
      off.push_back(total);
      total += align256((size_t)nkc * L->paths[p].nct * 64 * 4 + kDmaPad);
    }
    off.push_back(total);
    total += align256(decode_u_bytes(L->ug));
    off.push_back(total);
    total += align256(decode_h_bytes(L->ug));
  }
  // the linears' layouts were written on their creation streams
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = D.buf.ensure(std::max<size_t>(total, 256));
  if (e != hipSuccess) return e;
  uint8_t* base = reinterpret_cast<uint8_t*>(D.buf.ptr);
  size_t k = 0;
  for (lb_linear L : lins) {
    const int nkc = (int)((L->n + kChunk - 1) / kChunk);
    std::array<const uint32_t*, 2> v = {nullptr, nullptr};
    for (int p = 0; p < L->np; ++p) {
      const size_t bytes = (size_t)nkc * L->paths[p].nct * 64 * 4 + kDmaPad;
      if ((e = hipMemcpy(base + off[k], L->paths[p].vdec, bytes, hipMemcpyDeviceToDevice)) != hipSuccess) return e;
      v[p] = reinterpret_cast<const uint32_t*>(base + off[k++]);
    }
    if ((e = hipMemcpy(base + off[k], L->udec, decode_u_bytes(L->ug), hipMemcpyDeviceToDevice)) != hipSuccess) return e;
    D.udec.push_back(base + off[k++]);
    if ((e = hipMemcpy(base + off[k], L->hq, decode_h_bytes(L->ug), hipMemcpyDeviceToDevice)) != hipSuccess) return e;
    D.hq.push_back(reinterpret_cast<const uint16_t*>(base + off[k++]));
    D.vdec.push_back(v);
  }
  return hipSuccess;
}

}  // namespace

extern "C" {

lb_status lb_stack_create(const lb_linear* linears, int32_t count, lb_stack* out) {
  if (!out || !linears) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer");
  if (count <= 0) return fail(LB_ERR_INVALID_ARGUMENT, "count must be positive");
  if (count > LB_MAX_STACK) return fail(LB_ERR_UNSUPPORTED, "count exceeds %d", LB_MAX_STACK);
  for (int i = 0; i < count; ++i) {
    if (!linears[i]) return fail(LB_ERR_INVALID_ARGUMENT, "linear %d is null", i);
    if (linears[i]->device != linears[0]->device) return fail(LB_ERR_INVALID_ARGUMENT, "linears on different devices");
  }
  lb_stack S = new (std::nothrow) lb_stack_s();
  if (!S) return fail(LB_ERR_OUT_OF_MEMORY, "host allocation failed");
  S->device = linears[0]->device;
  S->linears.assign(linears, linears + count);
  hipError_t e = hipStreamCreateWithFlags(&S->cap_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = build_decode_image(S->dimg, S->linears);
  if (e != hipSuccess) {
    lb_stack_destroy(S);
    return hip_fail(e, "lb_stack_create");
  }
  *out = S;
  return LB_OK;
}

}  // extern "C"

namespace {

// Enqueues the stack's kernels on `st`; `capture`: into a graph being
// captured (level launches only).
lb_status stack_launch(lb_stack S, lb_regime rg, int64_t tokens, lb_dtype io, hipStream_t st, bool capture) {
  const int count = (int)S->linears.size();
  if (rg == LB_REGIME_DECODE && S->chain_active) {
    if (S->chain_enable == 1 && !capture) {
      const ChainArgs c{S->chain_levels_d, reinterpret_cast<uint64_t*>(S->chain_sync.ptr), S->chain_nlev,
                        S->chain_stall};
      HIP_TRY(launch_decode_chain(c, S->chain_bucket, S->chain_grid, st));
      return LB_OK;
    }
    // the same plans as launches per level (a graph, or mode 2): the same bits
    for (size_t g = 0; g < S->groups.size(); ++g) {
      StackGroup& G = S->groups[g];
      lb_status s = run_decode(S->chain_plans[g], G.lins.data(), (int)G.lins.size(), G.xs_d, G.ys_d, nullptr, nullptr,
                               tokens, y_is_fp32(io), st, &G.view);
      if (s != LB_OK) return s;
    }
    return LB_OK;
  }
  if (rg == LB_REGIME_DECODE) {
    for (StackGroup& G : S->groups) {
      lb_status s = run_decode(G.plan, G.lins.data(), (int)G.lins.size(), G.xs_d, G.ys_d, nullptr, nullptr, tokens,
                               y_is_fp32(io), st, &G.view);
      if (s != LB_OK) return s;
    }
    return LB_OK;
  }
  if (rg == LB_REGIME_PREFILL) {
    for (StackGroup& G : S->groups)
      HIP_TRY(prefill_run(G.pplan, G.pre.data(), (int)G.lins.size(), G.xs_h.data(), G.ys_h.data(), (int)tokens,
                          y_is_fp32(io), st, false));
    return LB_OK;
  }
  // exact: one pair of kernels per linear, sharing one z' scratch laid out per entry
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    lb_linear L = S->linears[i];
    HIP_TRY(launch_exact(L->paths, L->np, (int)L->m, (int)L->n, S->xs_h[i], S->ys_h[i], (int)tokens, x_is_fp32(io),
                         y_is_fp32(io), reinterpret_cast<float*>(S->zexact.ptr) + off, st));
    off += exact_scratch_floats(L->paths, L->np, tokens, (int)L->n, x_is_fp32(io), y_is_fp32(io));
  }
  return LB_OK;
}

// Levels of the stack's entries: entry j runs after every earlier entry i
// whose output it reads (y_i overlaps x_j), whose output it also writes
// (y_i overlaps y_j) or whose input it overwrites (y_j overlaps x_i);
// level[j] = 1 + the highest such level[i], 0 if none.  An entry whose y
// overlaps its own x is refused (-1 in bad).
std::vector<int> stack_levels(const std::vector<lb_linear>& lins, const std::vector<const void*>& xs,
                              const std::vector<void*>& ys, int64_t tokens, lb_dtype io, int* bad) {
  const int count = (int)lins.size();
  *bad = -1;
  const uint64_t xes = x_is_fp32(io) ? 4 : 2, yes = y_is_fp32(io) ? 4 : 2;   // element bytes of x, y
  auto range = [&](const void* p, int64_t cols, uint64_t es) {
    const uint64_t a = reinterpret_cast<uintptr_t>(p);
    return std::make_pair(a, a + (uint64_t)tokens * (uint64_t)cols * es);
  };
  auto overlap = [](std::pair<uint64_t, uint64_t> u, std::pair<uint64_t, uint64_t> v) {
    return u.first < v.second && v.first < u.second;
  };
  std::vector<int> level(count, 0);
  for (int j = 0; j < count; ++j) {
    const auto xj = range(xs[j], lins[j]->n, xes), yj = range(ys[j], lins[j]->m, yes);
    if (overlap(xj, yj) && *bad < 0) *bad = j;
    for (int i = 0; i < j; ++i) {
      const auto xi = range(xs[i], lins[i]->n, xes), yi = range(ys[i], lins[i]->m, yes);
      if (overlap(yi, xj) || overlap(yi, yj) || overlap(yj, xi)) level[j] = std::max(level[j], level[i] + 1);
    }
  }
  return level;
}

// Splits the stack into launch groups by level (one group when the entries
// are independent) and copies each group's pointers to the device.
lb_status stack_groups(lb_stack S, int64_t tokens, lb_dtype io) {
  const int count = (int)S->linears.size();
  int bad = -1;
  const std::vector<int> level = stack_levels(S->linears, S->xs_h, S->ys_h, tokens, io, &bad);
  if (bad >= 0) return fail(LB_ERR_INVALID_ARGUMENT, "entry %d: y overlaps its own x", bad);
  const int nlev = 1 + *std::max_element(level.begin(), level.end());
  for (StackGroup& G : S->groups) G.release();
  S->groups.clear();
  S->groups.resize(nlev);
  for (int i = 0; i < count; ++i) S->groups[level[i]].idx.push_back(i);
  for (StackGroup& G : S->groups) {
    const int n = (int)G.idx.size();
    for (int i : G.idx) {
      G.lins.push_back(S->linears[i]);
      G.pre.push_back(&S->linears[i]->pre);
      G.view.udec.push_back(S->dimg.udec[i]);
      G.view.hq.push_back(S->dimg.hq[i]);
      G.view.vdec.push_back(S->dimg.vdec[i]);
      G.xs_h.push_back(S->xs_h[i]);
      G.ys_h.push_back(S->ys_h[i]);
    }
    HIP_TRY(hipMalloc(&G.xs_d, n * sizeof(void*)));
    HIP_TRY(hipMalloc(&G.ys_d, n * sizeof(void*)));
    HIP_TRY(hipMemcpy(G.xs_d, G.xs_h.data(), n * sizeof(void*), hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(G.ys_d, G.ys_h.data(), n * sizeof(void*), hipMemcpyHostToDevice));
  }
  return LB_OK;
}

// The persistent chained decode for the stack's levels, when it can run
// them: more than one level, one launch of at most kDecodeMaxTokens tokens,
// bf16 y, every entry in the kernel's fast forms, and a device that can
// launch all of its workgroups at once.  Otherwise the levels run as launches
// (chain_active stays 0).  Direct launches use it; a captured graph holds
// the level launches (both give the same bits).
lb_status chain_prepare(lb_stack S, int64_t tokens, lb_dtype io, hipStream_t st) {
  S->chain_release();
  if (!S->chain_enable || S->groups.size() < 2 || tokens > kDecodeMaxTokens || y_is_fp32(io)) return LB_OK;
  const int bucket = decode_bucket((int)tokens);
  for (const StackGroup& G : S->groups)
    for (const DecEntry& e : G.plan.entries_h)
      if (!decode_chain_takes(e, bucket)) return LB_OK;
  const int grid = decode_chain_grid(bucket, S->device);
  if (grid <= 0) return LB_OK;
  const int slots = decode_chain_participants(grid);
  S->chain_plans.resize(S->groups.size());
  std::vector<ChainLevel> lv;
  int moff = 0;
  for (size_t g = 0; g < S->groups.size(); ++g) {
    StackGroup& G = S->groups[g];
    DecodePlan& P = S->chain_plans[g];
    lb_status s = build_decode_plan(P, G.lins.data(), (int)G.lins.size(), (int)tokens, &G.view, slots);
    if (s != LB_OK) return s;
    ChainLevel c{};
    c.a.entries = P.entries_d;
    c.a.xs = G.xs_d;
    c.a.ys = G.ys_d;
    c.a.vitems = P.vitems_d;
    c.a.mitems = P.mitems_d;
    c.a.uitems = P.uitems_d;
    c.a.part = reinterpret_cast<float*>(P.part.ptr);
    c.a.T = (int)tokens;
    c.a.t0 = 0;
    c.a.bucket = bucket;
    c.a.yf32 = 0;
    c.nv = P.nv;
    c.nm = P.nm;
    c.nu = P.nu;
    c.moff = moff;
    moff += P.nm;
    lv.push_back(c);
  }
  HIP_TRY(upload(&S->chain_levels_d, lv));
  // counters start at zero for a new plan (stream-ordered before its first launch)
  HIP_TRY(S->chain_sync.ensure(chain_sync_bytes(moff)));
  HIP_TRY(hipMemsetAsync(S->chain_sync.ptr, 0, chain_sync_bytes(moff), st));
  S->chain_grid = grid;
  S->chain_bucket = bucket;
  S->chain_nlev = (int)lv.size();
  const char* stall = std::getenv("LITTLEBIT_CHAIN_STALL");
  S->chain_stall = stall && std::strcmp(stall, "1") == 0 ? 1 : 0;
  S->chain_active = 1;
  return LB_OK;
}

// Prepares everything a launch sequence needs outside of any graph capture.
lb_status stack_prepare(lb_stack S, lb_regime rg, int64_t tokens, lb_dtype io, hipStream_t st) {
  S->chain_release();
  if (rg == LB_REGIME_DECODE) {
    lb_status s = stack_groups(S, tokens, io);
    if (s != LB_OK) return s;
    const int T = (int)std::min<int64_t>(tokens, kDecodeMaxTokens);
    for (StackGroup& G : S->groups) {
      s = build_decode_plan(G.plan, G.lins.data(), (int)G.lins.size(), T, &G.view);
      if (s != LB_OK) return s;
    }
    s = chain_prepare(S, tokens, io, st);
    if (s != LB_OK) return s;
    // (a ragged last slice of a long decode uses another plan shape: those
    // runs launch directly and rebuild the plan per slice)
  } else if (rg == LB_REGIME_PREFILL) {
    if (!prefill_available()) return fail(LB_ERR_UNSUPPORTED, "the prefill kernels are not available in this library");
    lb_status s = stack_groups(S, tokens, io);
    if (s != LB_OK) return s;
    for (StackGroup& G : S->groups)
      HIP_TRY(prefill_prepare(G.pplan, G.pre.data(), (int)G.lins.size(), (int)tokens, G.xs_h.data(), G.ys_h.data()));
  } else {
    size_t want = 0;
    for (lb_linear L : S->linears)
      want += exact_scratch_floats(L->paths, L->np, tokens, (int)L->n, x_is_fp32(io), y_is_fp32(io));
    HIP_TRY(S->zexact.ensure(std::max<size_t>(want, 1) * sizeof(float)));
  }
  return LB_OK;
}

}  // namespace

extern "C" {

lb_status lb_stack_forward_ex(lb_stack S, const void* const* xs, void* const* ys, int64_t tokens, lb_dtype io,
                              lb_regime regime, int32_t use_graph, void* stream) {
  if (!S) return fail(LB_ERR_INVALID_ARGUMENT, "null stack");
  if (!xs || !ys) return fail(LB_ERR_INVALID_ARGUMENT, "null pointer array");
  lb_status s = check_io(tokens, io, regime);
  if (s != LB_OK) return s;
  const int count = (int)S->linears.size();
  for (int i = 0; i < count; ++i) {
    if (!xs[i] || !ys[i]) return fail(LB_ERR_INVALID_ARGUMENT, "entry %d: null x or y", i);
    if (!aligned16(xs[i]) || !aligned16(ys[i])) return fail(LB_ERR_ALIGNMENT, "entry %d: pointer not 16-byte aligned", i);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // AUTO's choice for these linears, kept per (tokens, io)
  if (regime == LB_REGIME_AUTO && (S->auto_tokens != tokens || S->auto_io != (int)io)) {
    S->auto_rg = pick_regime(S->linears.data(), count, tokens, io, LB_REGIME_AUTO);
    S->auto_tokens = tokens;
    S->auto_io = (int)io;
  }
  const lb_regime rg = regime == LB_REGIME_AUTO ? S->auto_rg : regime;
  const bool same_ptrs = S->xs_h.size() == (size_t)count && std::equal(xs, xs + count, S->xs_h.begin()) &&
                         std::equal(ys, ys + count, S->ys_h.begin());
  const bool same = same_ptrs && S->g_tokens == tokens && S->g_io == (int)io && S->g_regime == (int)rg;
  if (!same) {
    // everything below rewrites memory earlier launches read: wait for them
    if (S->last_stream) HIP_TRY(hipStreamSynchronize(S->last_stream));
    HIP_TRY(hipStreamSynchronize(st));
    // The old plans and graph go first, and the stack records what it was
    // prepared for only once the new plans exist: a failed call (an entry
    // whose y overlaps its own x, an allocation failure) leaves a stack that
    // matches no pointers, so a retry is checked again instead of replaying
    // launches that write into the previous call's buffers.
    S->g_tokens = -1;
    S->g_io = -1;
    S->g_regime = -1;
    if (S->exec) (void)hipGraphExecDestroy(S->exec);
    if (S->graph) (void)hipGraphDestroy(S->graph);
    S->exec = nullptr;
    S->graph = nullptr;
    for (StackGroup& G : S->groups) G.release();
    S->groups.clear();
    S->xs_h.assign(xs, xs + count);
    S->ys_h.assign(ys, ys + count);
    s = stack_prepare(S, rg, tokens, io, st);
    if (s != LB_OK) {
      S->chain_release();
      for (StackGroup& G : S->groups) G.release();
      S->groups.clear();
      S->xs_h.clear();
      S->ys_h.clear();
      return s;
    }
    S->g_tokens = tokens;
    S->g_io = (int)io;
    S->g_regime = (int)rg;
  }
  S->last_stream = st;
  const bool ragged_decode = rg == LB_REGIME_DECODE && tokens > kDecodeMaxTokens && tokens % kDecodeMaxTokens;
  if (!use_graph || ragged_decode) return stack_launch(S, rg, tokens, io, st, false);
  if (!S->exec) {
    HIP_TRY(hipStreamBeginCapture(S->cap_stream, hipStreamCaptureModeThreadLocal));
    lb_status ls = stack_launch(S, rg, tokens, io, S->cap_stream, true);
    hipGraph_t g = nullptr;
    hipError_t ce = hipStreamEndCapture(S->cap_stream, &g);
    if (ls != LB_OK) {
      if (g) (void)hipGraphDestroy(g);
      return ls;
    }
    if (ce != hipSuccess) return hip_fail(ce, "hipStreamEndCapture");
    S->graph = g;
    HIP_TRY(hipGraphInstantiate(&S->exec, S->graph, nullptr, nullptr, 0));
  }
  HIP_TRY(hipGraphLaunch(S->exec, st));
  return LB_OK;
}

lb_status lb_stack_forward(lb_stack S, const void* const* xs, void* const* ys, int64_t tokens, lb_dtype io,
                           void* stream) {
  // a graph only where launches are many (exact: two per linear); for the
  // decode and prefill kernels a graph replay costs more than it saves
  return lb_stack_forward_ex(S, xs, ys, tokens, io, LB_REGIME_AUTO, enum_bits(io) == LB_FP32 ? 1 : 0, stream);
}

lb_status lb_stack_set_persistent(lb_stack S, int32_t enable) {
  if (!S) return fail(LB_ERR_INVALID_ARGUMENT, "null stack");
  if (enable < 0 || enable > 2) return fail(LB_ERR_INVALID_ARGUMENT, "enable must be 0, 1 or 2");
  if (S->chain_enable != enable) {
    S->chain_enable = enable;
    S->g_tokens = -1;                       // the next forward plans again
  }
  return LB_OK;
}

lb_status lb_stack_persistent_status(lb_stack S, int32_t* active, int32_t* aborted) {
  if (!S) return fail(LB_ERR_INVALID_ARGUMENT, "null stack");
  if (active) *active = S->chain_active;
  if (aborted) {
    *aborted = 0;
    if (S->chain_sync.ptr) {
      int dev = 0;
      HIP_TRY(hipGetDevice(&dev));
      if (dev != S->device) HIP_TRY(hipSetDevice(S->device));
      uint64_t flag = 0;
      hipError_t e = S->last_stream ? hipStreamSynchronize(S->last_stream) : hipSuccess;
      if (e == hipSuccess) e = hipMemcpy(&flag, reinterpret_cast<uint64_t*>(S->chain_sync.ptr) + kChainAbort, 8,
                                         hipMemcpyDeviceToHost);
      if (dev != S->device) (void)hipSetDevice(dev);
      if (e != hipSuccess) return hip_fail(e, "reading the persistent kernel's abort flag");
      *aborted = flag != 0;
    }
  }
  return LB_OK;
}

lb_status lb_stack_destroy(lb_stack S) {
  if (!S) return LB_OK;
  if (S->exec) (void)hipGraphExecDestroy(S->exec);
  if (S->graph) (void)hipGraphDestroy(S->graph);
  if (S->cap_stream) (void)hipStreamDestroy(S->cap_stream);
  S->chain_release();
  S->chain_sync.release();
  for (StackGroup& G : S->groups) G.release();
  S->zexact.release();
  S->dimg.buf.release();
  delete S;
  return LB_OK;
}

}  // extern "C"

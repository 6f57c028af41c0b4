/*
 * littlebit.h -- C ABI of the MI355X (gfx950) LittleBit factorised-linear library.
 *
 * The layer (paper notes "LittleBit: Ultra Low-Bit Quantization via Latent
 * Factorization", section "Key design / multi-scale compensation" for one path
 * and section "Residual compensation" for the sum of two paths):
 *
 *     W = sum_{p < n_paths} diag(h_p) * U_p * diag(l_p) * V_p^T * diag(g_p)
 *     y = x * W^T
 *
 * U_p in {-1,+1}^{d_out x r_p} and V_p in {-1,+1}^{d_in x r_p} are the sign
 * factors, h_p (length d_out), g_p (length d_in) and l_p (length r_p) the row,
 * column and latent scales, stored as IEEE fp16.  The same section says the
 * inference forward is a sequence of element-wise products and binary matrix
 * products that never forms W; every forward entry point here follows that
 * order (x o g -> V -> o l -> U -> o h) and never materialises W.
 *
 * Conventions common to every call
 * --------------------------------
 * - Shapes: d_out = m rows of W (length of h), d_in = n columns (length of g).
 *   x is [tokens][d_in], y is [tokens][d_out], both row-major and contiguous.
 *   y is overwritten, never accumulated into.
 * - Canonical packed signs (the interchange format of this ABI): a factor
 *   S in {-1,+1}^{rows x r} packs row by row into W = ceil(r/32) uint32 words
 *   per row; bit (j mod 32) of word i*W + j/32 is 1 iff S[i][j] == -1.  Bits
 *   at positions j >= r are zero.
 * - Pointers marked "device" are HIP device pointers on the device that is
 *   current when the call is made; "host" pointers are ordinary CPU memory.
 *   Every pointer passed to a forward call must be 16-byte aligned.
 * - stream is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *   that take a stream are asynchronous on it unless stated otherwise.
 * - Errors: every call returns lb_status.  No C++ exception crosses the ABI.
 *   On any error the call's outputs are left untouched and lb_last_error()
 *   returns a description (thread-local).  HIP failures return LB_ERR_HIP
 *   with the HIP error text.  Faults inside kernels surface at the caller's
 *   next synchronisation, as with any asynchronous stream API.
 */
#ifndef LITTLEBIT_H
#define LITTLEBIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LB_OK = 0,
  LB_ERR_INVALID_ARGUMENT = 1, /* null pointer, non-positive size, bad enum  */
  LB_ERR_INVALID_SIGN = 2,     /* an unpacked sign value outside {-1, +1}     */
  LB_ERR_ALIGNMENT = 3,        /* a forward pointer is not 16-byte aligned    */
  LB_ERR_UNSUPPORTED = 4,      /* a size beyond the documented limits         */
  LB_ERR_OUT_OF_MEMORY = 5,    /* device allocation failed                    */
  LB_ERR_HIP = 6               /* a HIP runtime call failed                   */
} lb_status;

/* Element types of x and y.  LB_BF16_FP32 reads bf16 x and writes fp32 y:
 * the kernels' fp32 results are stored without the final rounding to bf16
 * (for callers that keep an fp32 residual stream). */
typedef enum { LB_BF16 = 0, LB_FP32 = 1, LB_BF16_FP32 = 2 } lb_dtype;

/* Which kernels run a forward.  AUTO picks by tokens and dtype:
 *   fp32 I/O -> EXACT (fp32 arithmetic end to end: vector kernels for fewer
 *               than 16 tokens, fp32 matrix-core contractions from 16 on);
 *   bf16 x (y bf16 or fp32) -> DECODE (fused fp8 x fp4 MFMA passes of up to
 *               16 tokens) or PREFILL (bf16 MFMA GEMMs in 64-row tiles up to
 *               128 tokens, 256-row tiles above), whichever the library's
 *               cost estimate for these linears at this token count makes
 *               faster (sign bytes streamed per 16-token pass against GEMM
 *               tiles and K blocks per row stripe, at rates measured on
 *               MI355X).  On the Llama-shaped stacks DECODE wins up to 16
 *               tokens (0.1-0.55 bits per weight) and up to 32 on a
 *               0.1-bit-per-weight Llama-2-70B stack.
 * Forcing a regime is for tests and measurements; every regime accepts every
 * token count.  DECODE and PREFILL require bf16 x (LB_BF16 or LB_BF16_FP32). */
typedef enum { LB_REGIME_AUTO = 0, LB_REGIME_EXACT = 1, LB_REGIME_DECODE = 2,
               LB_REGIME_PREFILL = 3 } lb_regime;

/* Limits (LB_ERR_UNSUPPORTED beyond them). */
#define LB_MAX_DIM    (1 << 20)   /* d_in, d_out                */
#define LB_MAX_RANK   4096        /* r_p                        */
#define LB_MAX_TOKENS (1 << 20)   /* tokens per forward         */
#define LB_MAX_STACK  65536       /* linears in one stack       */

typedef struct lb_linear_s* lb_linear; /* opaque, immutable after create */
typedef struct lb_stack_s* lb_stack;   /* opaque                         */

/* One path: diag(h) * U * diag(l) * V^T * diag(g).  All pointers are device
 * pointers; they are only read during lb_linear_create. */
typedef struct {
  int64_t rank;              /* r_p >= 1                                     */
  const uint32_t* u_packed;  /* [d_out][ceil(r/32)] canonical packed U signs */
  const uint32_t* v_packed;  /* [d_in ][ceil(r/32)] canonical packed V signs */
  const uint16_t* h;         /* [d_out] fp16 bit patterns, row scale         */
  const uint16_t* g;         /* [d_in ] fp16 bit patterns, column scale      */
  const uint16_t* l;         /* [rank ] fp16 bit patterns, latent scale      */
} lb_path;

/* ceil(rank / 32): uint32 words per row of a canonical packed factor
 * (0 for rank <= 0). */
int64_t lb_packed_words_per_row(int64_t rank);

/* Per-path rank for a sign-bit budget of bpw_num/bpw_den bits per weight:
 * round(BPW * d_out * d_in / (2 * (d_out + d_in))) in exact integer
 * arithmetic, ties rounded up.  Two paths of this rank store 2 r (m + n) sign
 * bits for m n weights (bits-per-weight accounting: paper notes "LittleBit",
 * sections "Overall framework" and "Residual compensation"; the aibk.xyz
 * article's advice on how bpp is counted).  Scale bits are not counted.
 * Returns -1 for non-positive arguments. */
int64_t lb_rank_for_bpw(int64_t d_out, int64_t d_in, int64_t bpw_num, int64_t bpw_den);

/* Pack an int8 sign matrix [rows][rank] (values -1 / +1, host memory) into
 * canonical words [rows][ceil(rank/32)] (host memory).  Synchronous.
 * LB_ERR_INVALID_SIGN if any value is not -1 or +1 (packed untouched). */
lb_status lb_pack_signs_host(const int8_t* signs, int64_t rows, int64_t rank, uint32_t* packed);

/* Device version of lb_pack_signs_host: signs and packed are device
 * pointers.  Validates every value first and returns LB_ERR_INVALID_SIGN
 * without writing packed if any is not +-1.  Synchronises `stream` (it reads
 * the validation result back). */
lb_status lb_pack_signs(const int8_t* signs, int64_t rows, int64_t rank, uint32_t* packed, void* stream);

/* Inverse of lb_pack_signs (test aid): device packed -> device int8 +-1.
 * Padding bits are ignored.  Asynchronous on stream. */
lb_status lb_unpack_signs(const uint32_t* packed, int64_t rows, int64_t rank, int8_t* signs, void* stream);

/* Build a linear from n_paths (1 or 2) paths.  The library COPIES the packed
 * signs and scales into memory it owns (re-laid out for its kernels) using
 * `stream`; the caller's buffers may be freed once `stream` has synchronised.
 * The linear is bound to the current device.  Returns LB_ERR_INVALID_ARGUMENT
 * for null pointers, d_out/d_in/rank <= 0 or n_paths not in {1, 2}. */
lb_status lb_linear_create(int64_t d_out, int64_t d_in, const lb_path* paths, int32_t n_paths,
                           void* stream, lb_linear* out);

/* y = x W^T for `tokens` rows, W the sum over the paths of
 * diag(h) U diag(l) V^T diag(g) ("LittleBit: Ultra Low-Bit Quantization via
 * Latent Factorization" paper notes, section "Key design" for one path and
 * section "Residual compensation" for the sum), computed in the factored
 * order the same section gives (element-wise scales around two binary matrix
 * products; W is never formed).  x and y are device pointers (element types
 * per `io`), borrowed until the stream work completes.  Runs the kernels of
 * LB_REGIME_AUTO.  Concurrent forwards of the same linear must be ordered on
 * one stream (they share the linear's scratch memory). */
lb_status lb_linear_forward(lb_linear L, const void* x, void* y, int64_t tokens, lb_dtype io, void* stream);

/* As lb_linear_forward with an explicit regime. */
lb_status lb_linear_forward_ex(lb_linear L, const void* x, void* y, int64_t tokens, lb_dtype io,
                               lb_regime regime, void* stream);

/* Forward for callers that cannot allocate device memory during the call
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  It runs the kernels lb_linear_forward_ex runs with an explicit
 * regime and gives the same results bit for bit: bf16 x (io LB_BF16 or
 * LB_BF16_FP32) -> LB_REGIME_DECODE, any token count, in launches of up to 16
 * tokens; fp32 I/O (LB_FP32) -> LB_REGIME_EXACT.  It calls no allocator:
 * its work buffers live in one fixed scratch array of 8 MiB per GPU (a device
 * global of this library, which each GPU it runs on holds until the process
 * ends), and the kernels' work-item tables were built by lb_linear_create.
 * Errors: as lb_linear_forward, plus LB_ERR_UNSUPPORTED when the call would
 * need more than the 8 MiB (the decode partial sums of very long rows or
 * large ranks; the exact path's latent sums of many fp32 tokens: splits x
 * n_paths x tokens x rank rounded to 16, 4 bytes each), and
 * LB_ERR_INVALID_ARGUMENT when the current device is not the linear's.
 * Every such call on one GPU shares that GPU's scratch: calls that overlap
 * in time on one GPU (on different streams, or from different threads
 * without ordering) race and give undefined results; calls ordered on one
 * stream are safe.  Nothing in the scratch must start at zero: each call
 * writes every value it reads back. */
lb_status lb_linear_forward_noalloc(lb_linear L, const void* x, void* y, int64_t tokens, lb_dtype io,
                                    void* stream);

/* The regime LB_REGIME_AUTO runs for these `count` linears (one linear, or
 * the linears of a stack, in which case every entry runs that regime) at
 * `tokens` tokens and element types `io`, into *out.  Host only: no device
 * work.  LB_ERR_INVALID_ARGUMENT for null pointers, count < 1, tokens < 1 or
 * an unknown io. */
lb_status lb_auto_regime(const lb_linear* linears, int32_t count, int64_t tokens, lb_dtype io, lb_regime* out);

/* Shape of a linear; any output pointer may be NULL.  ranks receives n_paths
 * values; device_bytes is the library-owned device memory of the linear. */
lb_status lb_linear_info(lb_linear L, int64_t* d_out, int64_t* d_in, int32_t* n_paths,
                         int64_t* ranks, int64_t* device_bytes);

/* Frees the linear's device memory.  Does not synchronise: the caller must
 * make sure no queued work still uses it.  NULL is accepted. */
lb_status lb_linear_destroy(lb_linear L);

/* A stack is an ordered list of linears run together by lb_stack_forward.
 * It borrows the linears, which must outlive it.  All linears must live on
 * the same device. */
lb_status lb_stack_create(const lb_linear* linears, int32_t count, lb_stack* out);

/* Runs every linear i of the stack, in order: ys[i] = xs[i] W_i^T, `tokens`
 * rows each (xs and ys are host arrays of `count` device pointers), each
 * W_i the layer of lb_linear_forward -- e.g. the seven linears of every
 * transformer layer of the models the paper notes evaluate (experiments
 * section: Llama-2 7B / 13B / 70B, Llama-3 8B).  Entries
 * may be chained through their buffers: when ys[i] overlaps xs[j] or ys[j] of
 * a later entry j, or ys[j] overlaps xs[i], entry j runs after entry i (so a
 * model's linears can be listed in their real order, each reading an earlier
 * one's output).  The stack is split into levels of mutually independent
 * entries; each level's entries run together (one launch per stage), levels
 * one after another.  An entry's y must not overlap its own x
 * (LB_ERR_INVALID_ARGUMENT).  The decode and prefill kernels go directly onto
 * `stream`; the exact fp32 kernels (two launches per linear) are captured once
 * into a HIP graph and replayed.  Plans and graphs are rebuilt when the
 * pointers, tokens, io or regime change.  Calls on one stack must be ordered
 * on one stream (they share the stack's scratch memory and graph). */
lb_status lb_stack_forward(lb_stack S, const void* const* xs, void* const* ys, int64_t tokens,
                           lb_dtype io, void* stream);

/* As lb_stack_forward with an explicit regime and graph use (use_graph = 1
 * captures the launches of any regime into a HIP graph and replays it;
 * use_graph = 0 launches the same kernels directly). */
lb_status lb_stack_forward_ex(lb_stack S, const void* const* xs, void* const* ys, int64_t tokens,
                              lb_dtype io, lb_regime regime, int32_t use_graph, void* stream);

/* Persistent chained decode.  A stack whose entries are chained (levels, see
 * lb_stack_forward), run in the decode regime with at most 16 tokens and
 * bf16 y, whose entries all have d_in a multiple of 8 and
 * ceil(r_1/128) + ceil(r_2/128) <= 8 (<= 6 above 8 tokens; e.g. ranks up to
 * 512 per path), runs all of its levels in ONE launch when enable = 1 and
 * the device supports cooperative launches, instead of three launches per
 * level.  It is meant for a model's linears run in their real order at batch
 * 1, where each level is a few hundred KB to a few MB of signs and its time
 * is latency, not bandwidth; measured on MI355X it is slower than the level
 * launches (about 21 against 17 us per level of a Llama-2-70B-shaped stack),
 * so the default is enable = 0 (paper notes "LittleBit:
 * Ultra Low-Bit Quantization via Latent Factorization", section "Key
 * design": the layer's factorised order, which every form follows).  The
 * kernel works on the compute units of one XCD, so that the data its stages
 * hand to each other stays in that XCD's L2 cache; per level a V phase
 * (partial latent sums; the last V work item of each (entry, path) forms that
 * pair's z' = z o l) and a U phase, each followed by a barrier of those
 * workgroups.  Its work items are planned for those workgroups, so its sums
 * are grouped differently from the level launches of enable = 0 (both within
 * the same tolerance of the exact result).  enable = 2 runs the persistent
 * kernel's plans as launches per level, with the same bits as enable = 1 (a
 * reference for tests); a captured graph (lb_stack_forward_ex with
 * use_graph = 1) does the same when enable is 1 or 2.  enable = 0 plans and
 * launches per level as any stack.  Any other value ->
 * LB_ERR_INVALID_ARGUMENT.  The change applies from the next forward (which
 * plans again). */
lb_status lb_stack_set_persistent(lb_stack S, int32_t enable);

/* Whether the stack's current plan runs the persistent chained kernel's plans
 * (*active, 0 or 1; host only), and whether a launch of that kernel gave up
 * (*aborted, 0 or 1): a barrier that waits longer than one second (a
 * workgroup that never arrives), or a participating workgroup that finds
 * itself on another XCD than the dispatch order puts it on, makes every
 * participant leave; the outputs of that launch are then not written in
 * full, those of every later launch of the plan not at all (its workgroups
 * leave at once), and the flag stays set until the stack plans
 * again.  Reading *aborted synchronises the stream of the stack's last
 * forward.  Either pointer may be NULL.  To test this path, the environment
 * variable LITTLEBIT_CHAIN_STALL=1 at planning makes the first barrier of
 * every launch wait for one arrival more than take part, so each launch times
 * out after one second and aborts; plan again without it (set enable to 0,
 * then back) for normal launches. */
lb_status lb_stack_persistent_status(lb_stack S, int32_t* active, int32_t* aborted);

/* Frees the stack (not its linears).  Does not synchronise.  NULL accepted. */
lb_status lb_stack_destroy(lb_stack S);

/* Static text for a status code. */
const char* lb_status_string(lb_status s);

/* Thread-local description of this thread's last failure ("" if none). */
const char* lb_last_error(void);

/* One path's outputs of lb_init_dual_svid: caller-owned device buffers in the
 * form lb_linear_create reads (lb_path). */
typedef struct {
  int64_t   rank;          /* r_p, 1 <= r_p <= min(d_out, d_in, LB_MAX_RANK)        */
  uint32_t* u_packed;      /* device, [d_out][ceil(r/32)] words, canonical packing  */
  uint32_t* v_packed;      /* device, [d_in ][ceil(r/32)] words                     */
  uint16_t* h;             /* device, fp16 bits, [d_out]                            */
  uint16_t* g;             /* device, fp16 bits, [d_in]                             */
  uint16_t* l;             /* device, fp16 bits, [rank]                             */
} lb_path_init;

/* Dual-SVID initialisation ("LittleBit: Ultra Low-Bit Quantization via Latent
 * Factorization", paper notes, sections "Key design / Dual-SVID
 * initialisation" and "Residual compensation") of an n_paths-path layer from a
 * dense weight W (device, fp32, row-major [d_out][d_in]).  Path p starts from
 * what the earlier stored paths leave of W: a truncated rank-r_p SVD gives
 * U', V' (singular values split evenly); U_sign = sign(U'), V_sign = sign(V')
 * (sign(0) = +1); the top singular pair of |U'| gives h and one latent factor,
 * that of |V'| gives g and the other, and l is their product.  Scales are
 * rounded to fp16 (nearest even), and the next path starts from W minus the
 * paths as stored.  fp64 arithmetic (rocSOLVER's partial SVD, rocBLAS);
 * allocates working memory of about 2 d_out d_in doubles; returns after the
 * work on `stream` has completed.  Errors: null pointers, n_paths not 1 or 2,
 * or a rank outside 1..min(d_out, d_in, LB_MAX_RANK) -> LB_ERR_INVALID_ARGUMENT;
 * solver or HIP failures -> LB_ERR_HIP (outputs then undefined). */
lb_status lb_init_dual_svid(const float* W, int64_t d_out, int64_t d_in, const lb_path_init* paths,
                            int32_t n_paths, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LITTLEBIT_H */
